// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace qsg {

// Q8_0 activation quantisation.  Writes the canonical 34-byte blocks to
// `canon` (may be NULL) and/or the library's internal wdata layout
// (codes int8 [rows][k], scales f32 [rows][k/32], bias -8*sum(q) int32
// [rows][k/32]; all NULL to skip).
hipError_t launch_quantize_q8_0(const float* x, int64_t nrows, int64_t k, uint8_t* canon,
                                int8_t* wq, float* wd, int32_t* wb, hipStream_t s);

hipError_t launch_quantize_q4_0(const float* x, int64_t nrows, int64_t k, uint8_t* y,
                                hipStream_t s);

// INIT for the skinny MFMA kernels: the internal wdata (wq, wd, wb as above)
// and the same codes and scales in that kernel's operand order (sq, ss) over
// `rows` x `phases` * 8 blocks, zero past nrows and k; `rows8` selects the
// layout of the 8-row kernel (16-row tiles otherwise).
hipError_t launch_quantize_q8_0_skinny(const float* x, int64_t nrows, int64_t k, int8_t* wq,
                                       float* wd, int32_t* wb, uint8_t* sq, float* ss,
                                       int64_t rows, int64_t phases, bool rows8, hipStream_t s);

struct Q4Args {
  const uint8_t* w;      // Q4_0 src0
  const int8_t* aq;      // wdata codes
  const float* ad;       // wdata scales
  const int32_t* ab;     // wdata -8*sum(q)
  const uint8_t* sq;     // skinny kernel: codes in operand order (NULL otherwise)
  const float* ss;       // skinny kernel: d_a in operand order (16-row tiles: binary16
                         // bits, 8 blocks in 16 bytes per row and phase; 8-row: fp32)
  int sk_phases;         // skinny kernel: phases of 8 blocks per row
  int sq_bytes, ss_bytes; // skinny kernel: sizes of those two ranges
  float* dst;
  float* part;           // split-K partials [split][M][N]
  int M, N, K;
  int32_t* dots;         // debug block dots (NULL in production)
  int n0, n1;
};

// Weight matrices that share src1, concatenated along N for the narrow
// kernel: global row r of the group belongs to matrix i with
// row0[i] <= r < row0[i+1] and is row r - row0[i] of w[i]; its outputs go to
// column r - row0[i] of dst[i] ([M][N_i]).
constexpr int kMaxGroup = 8;
struct Q4Mats {
  const uint8_t* w[kMaxGroup];
  float* dst[kMaxGroup];
  int row0[kMaxGroup + 1];
  int count;
};

// x != NULL selects the fused kernel: src1 (f32) is quantized to Q8_0 in LDS
// by every workgroup (p.fuse must be set); x == NULL reads the wdata in a.
// a.N is the total row count of mats; a.w / a.dst are unused here.
hipError_t launch_q4_narrow(const Plan& p, const Q4Args& a, const Q4Mats& mats, const float* x,
                            hipStream_t s);
// Skinny MFMA kernel on repacked weights (repack.hip); reads the operand-
// order wdata of 16-row tiles (INIT must have run).
hipError_t launch_q4r_skinny(const Plan& p, const Q4Args& a, hipStream_t s);
// Weight repack: Q4_0 [N][K/32] blocks <-> the repacked layout.
hipError_t launch_repack_q4_0(const uint8_t* src, uint8_t* dst, int64_t N, int64_t K,
                              hipStream_t s);
hipError_t launch_unpack_q4_0(const uint8_t* src, uint8_t* dst, int64_t N, int64_t K,
                              hipStream_t s);
// Wide kernel (INIT must have run): int8 MFMA; plain or repacked weights
// (p.type).
hipError_t launch_q4_wide_i8(const Plan& p, const Q4Args& a, hipStream_t s);
// Skinny MFMA kernel: reads the wdata in a (INIT must have run), writes
// a.dst.  16-row workgroups when K % 64 == 0 and src0 is 4-byte aligned
// (q4_skinny_ok); otherwise the 32-row kernel with LDS-staged chunks.
bool q4_skinny_ok(int K, const void* w);
hipError_t launch_q4_skinny(const Plan& p, const Q4Args& a, hipStream_t s);
hipError_t launch_q4_mma(const Plan& p, const Q4Args& a, hipStream_t s);

hipError_t launch_f_narrow(const Plan& p, int type, const void* w, const float* x, float* dst,
                           int M, int N, int K, hipStream_t s);
// src1 is converted to binary16 into ws + p.off_ah ([M][K]) first, with a
// power of two per row (exponents at ws + p.off_rexp) undone on dst.
hipError_t launch_f16_wide(const Plan& p, const uint16_t* w, const float* x, float* dst, int M,
                           int N, int K, void* ws, hipStream_t s);
// Skinny F16 / F32 MFMA kernel (one launch, no workspace); needs f_mma_ok():
// src0 and src1 16-byte aligned, K a multiple of 8 (F16) or 4 (F32), K <=
// kFMmaMaxK.
bool f_mma_ok(int type, const void* w, const float* x, int64_t K);
hipError_t launch_f_mma(const Plan& p, int type, const void* w, const float* x, float* dst, int M,
                        int N, int K, hipStream_t s);
hipError_t launch_zero(float* dst, int64_t n, hipStream_t s);
// dst[i] = sum over z = 0..split-1, in that order, of part[z * n + i].
hipError_t launch_splitk_reduce(const float* part, float* dst, int64_t n, int split, hipStream_t s);

}  // namespace qsg
