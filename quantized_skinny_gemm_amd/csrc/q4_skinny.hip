// Skinny Q4_0 x Q8_0 product on the 16 x 16 int8 matrix cores, for batches
// of a few src1 rows (2 < M <= 32 per pass).
//
// dst[m][n] = sum_b f32(d_w[n][b]) * f32(d_a[m][b]) * S_b[m][n],
// S_b = sum_j (q4 - 8) * q8 (int32).
//
// With a few src1 rows the product is still bound by reading each weight
// once (arXiv 2407.07304, section 2.2; DeepSpeed-Inference notes, III.A),
// but per weight byte it does M times the dot-product work of the M = 1
// kernel, so the block dots go to the matrix cores:
// v_mfma_i32_16x16x32_i8 has K = 32, one Q4_0 / Q8_0 block, so every MFMA
// output is one block dot and takes one scale pair.
//
//   * A workgroup owns 16 weight rows (the MFMA's rows); its W waves split
//     their K range (each a contiguous run of block pairs), so that a large
//     grid of small, equal shares keeps every CU's loads in flight, and add
//     their partial tiles in LDS at the end in a fixed order (DeepSpeed-
//     Inference notes, III.C: partial sums reduced on chip).
//   * A wave walks its run in phases of 4 block pairs.  A phase's 16 rows x
//     4 pairs x 36 bytes are loaded one unit (a row's block pair) per lane,
//     consecutive lanes on consecutive bytes of a row: loading the MFMA
//     operands straight from memory would give each instruction 16 partly
//     used rows and reads far slower.  The units are reordered through a
//     small LDS patch private to the wave (no workgroup barrier), and the
//     next phase's loads are in flight while one phase is computed.
//   * Lane (row i = l % 16, group g = l / 16) of the A operand takes code
//     bytes 4g .. 4g+3 of its row's block: their low nibbles are elements
//     4g .. 4g+3, their high nibbles elements 16+4g .. 19+4g, and the B
//     operand (the Q8_0 codes of src1 row l % 16) holds the same elements.
//     Nibbles become signed bytes 16 * (q - 8) with a shift and two masked
//     xors ((q ^ 8) << 4 read as a signed byte is 16 (q - 8)), so the MFMA
//     ends at 16 S_b exactly and no bias term is needed; every output is
//     multiplied by 1/16 once, when it is stored (exact: a power of two, and
//     the scaled partial sums round exactly as the unscaled ones would).
//   * Output lane l holds src1 row l % 16 and weight rows 4 (l / 16) + r.
//     The scale of each output, d_w[row] * d_a[col], comes from a second
//     MFMA (an outer product on the fp16 matrix cores: both scales are
//     binary16 values, so each product is exact in fp32), already in the
//     result layout; the epilogue per output and block is a convert and an
//     fma: acc += f32(16 S_b) * (d_w * d_a).
//   * M <= 8 (k_q4_skinny8): v_mfma_i32_16x16x64_i8 takes two blocks at once,
//     its 16 columns being 8 src1 rows x the pair's two blocks (the B operand
//     of column (m, e) is zero outside block e), which halves the MFMAs, the
//     scale products and the epilogue per block, and reads no padding rows.
#include "device.h"
#include "kernels.h"
#include "../../include/mm.h"

namespace qsg {

namespace {

constexpr int kPH = kSkinnyPairs;        // block pairs per phase (16 rows x 4 = 64 units)
constexpr int kRP = kPH * 36 + 4;        // LDS row pitch: 37 dwords, odd, so rows spread the banks

// LDS of one wave: its patch of RT x 16 weight rows (kQ8: 68-byte units,
// row pitch 69 dwords).
template <int RT, bool kQ8 = false>
struct WaveLds {
  static constexpr int kUnit = kQ8 ? 17 : 9;             // dwords per block pair
  static constexpr int kPitch = kQ8 ? kPH * 68 + 4 : kRP;
  static constexpr int kBytes = RT * 16 * kPitch;
};

template <int MP, int RT, bool kQ8 = false>
struct Phase {
  uint32_t w[RT][kQ8 ? 17 : 9];  // this lane's units: one row's block pair per row tile
  v4i act[MP][kPH];           // B operands of pair j: blocks 2j and 2j+1
  v4i da[MP];                 // d_a (binary16) of the phase's 8 blocks, lanes 0-15
};

__device__ __forceinline__ uint32_t gload32(const void* p) {
  return *(const __attribute__((address_space(1))) uint32_t*)p;
}
typedef float v4f __attribute__((ext_vector_type(4)));

// Activation loads go through a buffer resource over the operand-order
// wdata: a lane whose offset is at or past the end of the range reads zeros
// and sends no request, which is how lanes of rows past M (and, in the
// 8-row kernel, lanes that hold no activation) skip their loads without a
// branch.
constexpr int kSkip = 0x7FFFFFF0;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wdata_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ v4i bload128(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// One phase's loads: this lane's weight units (row lane / 4 of each row
// tile, pair lane % 4, clamped to the row's last pair) and, per m tile, the
// activations in operand order as INIT laid them out (4 KB of codes per
// tile and phase, lane l of pair j at 1024 j + 16 l; then the 16 rows' 8
// scales).  Lanes of rows past M load nothing (zeros), and only lanes 0-15
// load scales: the scale MFMA reads its B operand from k = 0 alone, so the
// other lanes' zeros keep it a plain outer product.  Blocks past K hold
// zeros in the wdata.
template <int MP, int RT, bool kQ8>
__device__ __forceinline__ void load_phase(Phase<MP, RT, kQ8>& P, const Q4Args& a,
                                           const uint8_t* const (&wrow)[RT], int j0, int pairs,
                                           int ty) {
  constexpr int UW = WaveLds<RT, kQ8>::kUnit;
  const int lane = threadIdx.x & 63;
  int pc = j0 + (lane & 3);
  pc = pc < pairs ? pc : pairs - 1;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const uint8_t* wp = wrow[rt] + 4 * UW * (int64_t)pc;
#pragma unroll
    for (int i = 0; i < UW; ++i) P.w[rt][i] = gload32(wp + 4 * i);
  }
  const int f = j0 / kPH;
  const __amdgpu_buffer_rsrc_t rq = wdata_rsrc(a.sq, a.sq_bytes);
  const __amdgpu_buffer_rsrc_t rs = wdata_rsrc(a.ss, a.ss_bytes);
#pragma unroll
  for (int t = 0; t < MP; ++t) {
    const int tp = (ty * MP + t) * a.sk_phases + f;
    const bool rv = (lane & 15) < a.M - (ty * MP + t) * 16;
    const int qo = rv ? tp * 4096 + 16 * lane : kSkip;
#pragma unroll
    for (int j = 0; j < kPH; ++j) P.act[t][j] = bload128(rq, rv ? qo + 1024 * j : kSkip);
    const bool sv = rv && lane < 16;
    P.da[t] = bload128(rs, sv ? (tp * 16 + lane) * 16 : kSkip);
  }
}

// Signed bytes 16 (q - 8) of the low and high nibbles of four code bytes.
__device__ __forceinline__ long nibbles_x16(uint32_t q) {
  const uint32_t lo = ((q << 4) ^ 0x80808080u) & 0xF0F0F0F0u;
  const uint32_t hi = (q ^ 0x88888888u) & 0xF0F0F0F0u;
  return (long)(((uint64_t)hi << 32) | lo);
}

// The 16 x 16 tile of scale products d_w[row] * d_a[col] in the layout of
// the MFMA results: an outer product on the fp16 matrix cores
// (v_mfma_f32_16x16x16_f16; lane l supplies k = 4 (l / 16) .. +3 of row or
// column l % 16, and only k = 4 (l / 16) is set here), in place of four
// multiplies per lane and of a trip through LDS to bring each lane the
// weight scales of its rows.  Both scales are binary16 values held widened
// in fp32: narrowing them back is exact, each product is exact in fp32 and
// the sum over k adds zeros.  Every lane passes its row's weight scale
// (finite), and only the lanes of one k group a non-zero activation scale.
// (Keeping them in fp32 until here costs a convert each, but keeps each
// scale in one register: operands built from the bits need a zero register
// beside every scale, which cost the 32-row kernel a wave per SIMD.)
__device__ __forceinline__ v4f scale_tile(float dw_row, float da_col) {
  const v4h A = {(_Float16)dw_row, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
  const v4h B = {(_Float16)da_col, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
  return __builtin_amdgcn_mfma_f32_16x16x16f16(A, B, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
}

// The same outer product for block kb of a phase from binary16 bits as
// loaded: the B operand is the dword pair of d_a (lanes 0-15) that holds
// blocks 4 (kb / 4) .. +3 at k = 0..3, and the A operand carries the weight
// scale at k = kb % 4 alone (x: the scale's bits already in the low half for
// an even block, the high half for an odd one), so one pair of loaded
// registers serves four blocks and a block's operands cost one mask.
__device__ __forceinline__ v4f scale_tile_k4(uint32_t x, int kb, const v4i& da) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i a = (kb & 2) ? v2i{0, (int)x} : v2i{(int)x, 0};
  const v2i b = (kb & 4) ? v2i{da.z, da.w} : v2i{da.x, da.y};
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4h, a), __builtin_bit_cast(v4h, b),
                                              v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
}

template <int MP, int RT, bool kDump, bool kQ8>
__device__ __forceinline__ void compute_phase(const Phase<MP, RT, kQ8>& P, float (&acc)[RT][MP][4],
                                              uint8_t* stage, int j0, int j1, int n0, int m0,
                                              const Q4Args& a) {
  constexpr int UW = WaveLds<RT, kQ8>::kUnit, RP = WaveLds<RT, kQ8>::kPitch;
  const int lane = threadIdx.x & 63;
  const int i16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    // this lane's unit -> row 16 rt + lane / 4, pair lane % 4 of the patch
    uint32_t* d = reinterpret_cast<uint32_t*>(stage + (16 * rt + (lane >> 2)) * RP + 4 * UW * (lane & 3));
#pragma unroll
    for (int i = 0; i < UW; ++i) d[i] = P.w[rt][i];
  }
  // LDS operations of one wave complete in order: the reads below see the
  // writes above, and the next phase's writes come after these reads.
  const int nb = a.K / 32;
#pragma unroll
  for (int jj = 0; jj < kPH; ++jj) {
    const int pair = j0 + jj;
    const bool live = pair < j1;                   // for the dump (uniform over the wave)
    long A[RT][2];
    uint32_t dw[RT][2];     // binary16 bits of d_w, row 16 rt + i16: low half (even
                            // block), high half (odd block)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const uint32_t* u = reinterpret_cast<const uint32_t*>(stage + (16 * rt + i16) * RP) + UW * jj;
      if constexpr (kQ8) {
        // elements 4g .. 4g+3 and 16+4g .. 19+4g of each block: code dwords g
        // and 4 + g (even block: bytes from 2, shifted by 16 bits; odd block:
        // dword aligned from dword 9); the MFMA yields S_b
        auto c0 = [&](int q) { return (uint64_t)__builtin_amdgcn_alignbit(u[q + 1], u[q], 16); };
        A[rt][0] = (long)(c0(g) | (c0(4 + g) << 32));
        A[rt][1] = (long)((uint64_t)u[9 + g] | ((uint64_t)u[13 + g] << 32));
        dw[rt][0] = u[0] & 0xFFFFu;
        dw[rt][1] = u[8] & 0xFFFF0000u;
      } else {
        A[rt][0] = nibbles_x16(__builtin_amdgcn_alignbit(u[g + 1], u[g], 16));   // even block
        A[rt][1] = nibbles_x16(u[5 + g]);                                       // odd block
        dw[rt][0] = u[0] & 0xFFFFu;
        dw[rt][1] = u[4] & 0xFFFF0000u;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kb = 2 * jj + h;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int t = 0; t < MP; ++t) {
          const v4i& ac = P.act[t][jj];
          const long B = h ? (long)(((uint64_t)(uint32_t)ac.w << 32) | (uint32_t)ac.z)
                           : (long)(((uint64_t)(uint32_t)ac.y << 32) | (uint32_t)ac.x);
          const v4i D = __builtin_amdgcn_mfma_i32_16x16x32_i8(A[rt][h], B, v4i{0, 0, 0, 0}, 0, 0, 0);
          const v4f sc = scale_tile_k4(dw[rt][h], kb, P.da[t]);   // d_w * d_a
          acc[rt][t][0] = fmaf((float)D.x, sc.x, acc[rt][t][0]);
          acc[rt][t][1] = fmaf((float)D.y, sc.y, acc[rt][t][1]);
          acc[rt][t][2] = fmaf((float)D.z, sc.z, acc[rt][t][2]);
          acc[rt][t][3] = fmaf((float)D.w, sc.w, acc[rt][t][3]);
          if (kDump && live) {
            const int m = m0 + 16 * t + i16;
            const int b = 2 * pair + h;
            const int Dv[4] = {D.x, D.y, D.z, D.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int n = n0 + 16 * rt + 4 * g + r;
              if (m < a.M && n >= a.n0 && n < a.n1)
                a.dots[((int64_t)m * (a.n1 - a.n0) + (n - a.n0)) * nb + b] = kQ8 ? Dv[r] : Dv[r] / 16;
            }
          }
        }
      }
    }
  }
}

// Workgroup: RT x 16 weight rows; its W waves split K into runs of pp block
// pairs (a multiple of the phase).
template <int MP, int RT, int W, bool kDump, bool kQ8>
__global__ __launch_bounds__(64 * W)
void k_q4_skinny(Q4Args a, int pp) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nb = a.K / 32, pairs = nb / 2;
  const int64_t rb = (int64_t)nb * (kQ8 ? 34 : 18);
  const int n0 = blockIdx.x * 16 * RT, ty = blockIdx.y, m0 = ty * 16 * MP;
  // this wave's block pairs [j0w, j1w)
  const int j0w = wave * pp < pairs ? wave * pp : pairs;
  const int j1w = j0w + pp < pairs ? j0w + pp : pairs;
  const int nph = (j1w - j0w + kPH - 1) / kPH;
  uint8_t* stage = smem + wave * WaveLds<RT, kQ8>::kBytes;
  const uint8_t* wrow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int nrow = n0 + 16 * rt + (lane >> 2);
    nrow = nrow < a.N ? nrow : a.N - 1;
    wrow[rt] = a.w + nrow * rb;
  }

  float acc[RT][MP][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < MP; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[rt][t][r] = 0.0f;

  // Two register sets; every load in the loop is unconditional, and the
  // last one or two phases are computed after it.
  // (The scheduling barriers keep the loads of one set from being hoisted
  // above the computation of the other, which would hold three sets.)
  Phase<MP, RT, kQ8> P0, P1;
  if (nph > 0) load_phase<MP, RT, kQ8>(P0, a, wrow, j0w, pairs, ty);
  int f = 0;
  for (; f + 2 < nph; f += 2) {
    load_phase<MP, RT, kQ8>(P1, a, wrow, j0w + (f + 1) * kPH, pairs, ty);
    __builtin_amdgcn_sched_barrier(0);
    compute_phase<MP, RT, kDump, kQ8>(P0, acc, stage, j0w + f * kPH, j1w, n0, m0, a);
    __builtin_amdgcn_sched_barrier(0);
    load_phase<MP, RT, kQ8>(P0, a, wrow, j0w + (f + 2) * kPH, pairs, ty);
    __builtin_amdgcn_sched_barrier(0);
    compute_phase<MP, RT, kDump, kQ8>(P1, acc, stage, j0w + (f + 1) * kPH, j1w, n0, m0, a);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (f + 1 < nph) {
    load_phase<MP, RT, kQ8>(P1, a, wrow, j0w + (f + 1) * kPH, pairs, ty);
    __builtin_amdgcn_sched_barrier(0);
    compute_phase<MP, RT, kDump, kQ8>(P0, acc, stage, j0w + f * kPH, j1w, n0, m0, a);
    compute_phase<MP, RT, kDump, kQ8>(P1, acc, stage, j0w + (f + 1) * kPH, j1w, n0, m0, a);
  } else if (f < nph) {
    compute_phase<MP, RT, kDump, kQ8>(P0, acc, stage, j0w + f * kPH, j1w, n0, m0, a);
  }

  // ---- add the W waves' partial tiles in a fixed order (LDS reused)
  constexpr int NT = RT * MP;                      // 16 x 16 tiles per wave
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < MP; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[((wave * NT + rt * MP + t) * 4 + r) * 64 + lane] = acc[rt][t][r];
  __syncthreads();
  for (int idx = threadIdx.x; idx < NT * 256; idx += 64 * W) {
    const int tt = idx >> 8, r = (idx >> 6) & 3, l = idx & 63;
    const int rt = tt / MP, t = tt - rt * MP;
    float s = 0.0f;
    for (int w2 = 0; w2 < W; ++w2) s += red[((w2 * NT + tt) * 4 + r) * 64 + l];
    const int m = m0 + 16 * t + (l & 15);
    const int n = n0 + 16 * rt + 4 * (l >> 4) + r;
    if (m < a.M && n < a.N) a.dst[(int64_t)m * a.N + n] = kQ8 ? s : s * 0.0625f;   // 16 S_b
  }
}

template <int MP, int RT, int W, bool kQ8>
hipError_t launch_wq(const Plan& p, const Q4Args& a, int pp, hipStream_t s) {
  const dim3 grid((unsigned)p.tiles_n, (unsigned)p.tiles_m, 1u);
  const size_t stage = (size_t)W * WaveLds<RT, kQ8>::kBytes;
  const size_t red = (size_t)W * RT * MP * 4 * 64 * 4;
  const size_t lds = stage > red ? stage : red;
  if (a.dots) hipLaunchKernelGGL((k_q4_skinny<MP, RT, W, true, kQ8>), grid, dim3(64 * W), lds, s, a, pp);
  else hipLaunchKernelGGL((k_q4_skinny<MP, RT, W, false, kQ8>), grid, dim3(64 * W), lds, s, a, pp);
  return hipGetLastError();
}

template <int MP, int RT, int W>
hipError_t launch_w(const Plan& p, const Q4Args& a, int pp, hipStream_t s) {
  return p.type == MM_TYPE_Q8_0 ? launch_wq<MP, RT, W, true>(p, a, pp, s)
                                : launch_wq<MP, RT, W, false>(p, a, pp, s);
}

template <int MP, int RT>
hipError_t launch_mp(const Plan& p, const Q4Args& a, hipStream_t s) {
  const int pp = (int)p.kchunk;                     // block pairs per wave
  if (!a.sq || pp % kPH) return hipErrorInvalidValue;
  if (p.waves == 4) return launch_w<MP, RT, 4>(p, a, pp, s);
  if (p.waves == 8) return launch_w<MP, RT, 8>(p, a, pp, s);
  if constexpr (MP == 1) {
    if (p.waves == 16) return launch_w<MP, RT, 16>(p, a, pp, s);
  }
  return hipErrorInvalidValue;
}


// ---- M <= 8: two blocks per MFMA.  v_mfma_i32_16x16x64_i8 contracts 64
// elements; the 16 columns are 8 src1 rows x the pair's two blocks, and the
// B operand of column (m, e) is zero outside block e, so output (n, (m, e))
// is the block dot of block e alone.  Lane (row i, group g) of A holds half
// g & 1 of block g >> 1 of its row.
//
// kQ8: Q8_0 weights.  A unit (block pair) is 68 bytes, 17 dwords: block 0's
// scale in the low half of dword 0 and its codes from byte 2 (dwords shifted
// by 16 bits), block 1's scale in the high half of dword 8 and its codes
// dword-aligned from dword 9.  The codes are the A operand as stored (the
// MFMA gives S_b, not 16 S_b), so its outputs take no factor 1/16.
template <bool kQ8>
struct Unit8 {
  static constexpr int kDwords = kQ8 ? 17 : 9;          // dwords per block pair
  static constexpr int kPitch = kPH * 4 * kDwords + 4;  // LDS row pitch (odd dword count)
  static constexpr int kBytes = 16 * kPitch;            // one wave's patch
};

template <bool kQ8>
struct Phase8 {
  uint32_t w[Unit8<kQ8>::kDwords];
  v4i act[kPH];
  v4i da;                     // d_a (fp32 bits) of pair j's block, this column (lanes of group e)
};

template <bool kQ8>
__device__ __forceinline__ void load_phase8(Phase8<kQ8>& P, const Q4Args& a, const uint8_t* wrow,
                                            int j0, int pairs, int ty) {
  constexpr int UW = Unit8<kQ8>::kDwords;
  const int lane = threadIdx.x & 63;
  int pc = j0 + (lane & 3);
  pc = pc < pairs ? pc : pairs - 1;
  const uint8_t* wp = wrow + 4 * UW * (int64_t)pc;
#pragma unroll
  for (int i = 0; i < UW; ++i) P.w[i] = gload32(wp + 4 * i);
  const __amdgpu_buffer_rsrc_t rq = wdata_rsrc(a.sq, a.sq_bytes);
  const __amdgpu_buffer_rsrc_t rs = wdata_rsrc(a.ss, a.ss_bytes);
  const int tp = ty * a.sk_phases + j0 / kPH;
  const int c = lane & 15, g = lane >> 4, e = c >> 3;
  const bool mv = (c & 7) < a.M - ty * 8;
  const bool rv = mv && (g >> 1) == e;
  const int qo = tp * 2048 + 16 * (2 * c + (g & 1));
#pragma unroll
  for (int j = 0; j < kPH; ++j) P.act[j] = bload128(rq, rv ? qo + 512 * j : kSkip);
  P.da = bload128(rs, (mv && g == e) ? (tp * 16 + c) * 16 : kSkip);
}

template <bool kDump, bool kQ8>
__device__ __forceinline__ void compute_phase8(const Phase8<kQ8>& P, float (&acc)[4], uint8_t* stage,
                                               int j0, int j1, int n0, int m0, const Q4Args& a) {
  constexpr int UW = Unit8<kQ8>::kDwords, RP = Unit8<kQ8>::kPitch;
  const int lane = threadIdx.x & 63;
  const int i16 = lane & 15, g = lane >> 4;
  {
    uint32_t* d = reinterpret_cast<uint32_t*>(stage + (lane >> 2) * RP + 4 * UW * (lane & 3));
#pragma unroll
    for (int i = 0; i < UW; ++i) d[i] = P.w[i];
  }
  // Code dwords of this lane's half block: block 0's codes start 2 bytes into
  // the unit (a funnel shift by 16 of dwords b .. b+2), block 1's are dword
  // aligned (shift 0, so dword b+2 -- for g = 3 the row's pad dword after the
  // last pair -- is read but not used).
  // Q4_0: code bytes 8s .. 8s + 7 of block g >> 1 (s = g & 1), whose low and
  // high nibbles are elements 8s .. 8s+7 and 16+8s .. 23+8s.  Q8_0: code
  // dwords 2s, 4+2s, 2s+1, 5+2s of that block (dword q holds elements 4q ..
  // 4q+3), the same element order as the activation operand.
  const int b = kQ8 ? ((g >> 1) ? 9 : 0) : (g < 2 ? 2 * g : 2 * g + 1);
  const int sh = kQ8 ? ((g >> 1) ? 0 : 16) : (g < 2 ? 16 : 0);
  const int s2 = 2 * (g & 1);
  // Weight scale of block g & 1 (Q4_0 unit bytes 0-1 or 18-19; Q8_0 bytes
  // 0-1 or 34-35): the scale MFMA's k = 4 g, where the B operand of column
  // (m, e) holds d_a for g = e only; for g = 2, 3 the B operand is zero
  // there, any finite value works.
  const int ds = kQ8 ? ((g & 1) ? 8 : 0) : ((g & 1) ? 4 : 0), dsh = (g & 1) * 16;
  const int nb = a.K / 32;
#pragma unroll
  for (int jj = 0; jj < kPH; ++jj) {
    const uint32_t* u = reinterpret_cast<const uint32_t*>(stage + i16 * RP) + UW * jj;
    v4i A;
    float dw;
    if constexpr (kQ8) {
      // code dword q of the block: dwords b + q, b + q + 1 shifted by sh (for
      // block 1, q = 7, the second is the next unit's first dword or the
      // row's pad: unused, the shift is 0)
      auto cd = [&](int q) { return (int)__builtin_amdgcn_alignbit(u[b + q + 1], u[b + q], sh); };
      A = v4i{cd(s2), cd(4 + s2), cd(s2 + 1), cd(5 + s2)};
      dw = f16_bits_to_f32((u[ds] >> dsh) & 0xFFFFu);
    } else {
      const uint32_t x0 = u[b], x1 = u[b + 1], x2 = u[b + 2];
      const long A0 = nibbles_x16(__builtin_amdgcn_alignbit(x1, x0, sh));
      const long A1 = nibbles_x16(__builtin_amdgcn_alignbit(x2, x1, sh));
      A = v4i{(int)(uint32_t)A0, (int)(uint32_t)((uint64_t)A0 >> 32),
              (int)(uint32_t)A1, (int)(uint32_t)((uint64_t)A1 >> 32)};
      dw = f16_bits_to_f32((u[ds] >> dsh) & 0xFFFFu);
    }
    const v4i D = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, P.act[jj], v4i{0, 0, 0, 0}, 0, 0, 0);
    const v4f sc = scale_tile(dw, __int_as_float(P.da[jj]));
    acc[0] = fmaf((float)D.x, sc.x, acc[0]);
    acc[1] = fmaf((float)D.y, sc.y, acc[1]);
    acc[2] = fmaf((float)D.z, sc.z, acc[2]);
    acc[3] = fmaf((float)D.w, sc.w, acc[3]);
    if (kDump && j0 + jj < j1) {
      const int m = m0 + (i16 & 7);
      const int bk = 2 * (j0 + jj) + (i16 >> 3);
      const int Dv[4] = {D.x, D.y, D.z, D.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + 4 * g + r;
        if (m < a.M && n >= a.n0 && n < a.n1)
          a.dots[((int64_t)m * (a.n1 - a.n0) + (n - a.n0)) * nb + bk] = kQ8 ? Dv[r] : Dv[r] / 16;
      }
    }
  }
}

template <int W, bool kDump, bool kQ8>
__global__ __launch_bounds__(64 * W)
void k_q4_skinny8(Q4Args a, int pp) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nb = a.K / 32, pairs = nb / 2;
  const int64_t rb = (int64_t)nb * (kQ8 ? 34 : 18);
  const int n0 = blockIdx.x * 16, ty = blockIdx.y, m0 = ty * 8;
  const int j0w = wave * pp < pairs ? wave * pp : pairs;
  const int j1w = j0w + pp < pairs ? j0w + pp : pairs;
  const int nph = (j1w - j0w + kPH - 1) / kPH;
  uint8_t* stage = smem + wave * Unit8<kQ8>::kBytes;
  int nrow = n0 + (lane >> 2);
  nrow = nrow < a.N ? nrow : a.N - 1;
  const uint8_t* wrow = a.w + nrow * rb;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  Phase8<kQ8> P0, P1;
  if (nph > 0) load_phase8(P0, a, wrow, j0w, pairs, ty);
  int f = 0;
  for (; f + 2 < nph; f += 2) {
    load_phase8(P1, a, wrow, j0w + (f + 1) * kPH, pairs, ty);
    __builtin_amdgcn_sched_barrier(0);
    compute_phase8<kDump, kQ8>(P0, acc, stage, j0w + f * kPH, j1w, n0, m0, a);
    __builtin_amdgcn_sched_barrier(0);
    load_phase8(P0, a, wrow, j0w + (f + 2) * kPH, pairs, ty);
    __builtin_amdgcn_sched_barrier(0);
    compute_phase8<kDump, kQ8>(P1, acc, stage, j0w + (f + 1) * kPH, j1w, n0, m0, a);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (f + 1 < nph) {
    load_phase8(P1, a, wrow, j0w + (f + 1) * kPH, pairs, ty);
    __builtin_amdgcn_sched_barrier(0);
    compute_phase8<kDump, kQ8>(P0, acc, stage, j0w + f * kPH, j1w, n0, m0, a);
    compute_phase8<kDump, kQ8>(P1, acc, stage, j0w + (f + 1) * kPH, j1w, n0, m0, a);
  } else if (f < nph) {
    compute_phase8<kDump, kQ8>(P0, acc, stage, j0w + f * kPH, j1w, n0, m0, a);
  }
  // the W waves' partial tiles, then the two block halves of each column,
  // added in a fixed order
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = acc[r];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 128; idx += 64 * W) {
    const int r = idx & 3, m = (idx >> 2) & 7, gq = idx >> 5;
    const int l = 16 * gq + m;
    float s = 0.0f;
    for (int w2 = 0; w2 < W; ++w2) s += red[(w2 * 4 + r) * 64 + l] + red[(w2 * 4 + r) * 64 + l + 8];
    const int n = n0 + 4 * gq + r;
    if (m0 + m < a.M && n < a.N) a.dst[(int64_t)(m0 + m) * a.N + n] = kQ8 ? s : s * 0.0625f;
  }
}

template <int W, bool kQ8>
hipError_t launch_w8(const Plan& p, const Q4Args& a, int pp, hipStream_t s) {
  const dim3 grid((unsigned)p.tiles_n, (unsigned)p.tiles_m, 1u);
  const size_t stage = (size_t)W * Unit8<kQ8>::kBytes;
  const size_t red = (size_t)W * 4 * 64 * 4;
  const size_t lds = stage > red ? stage : red;
  if (a.dots) hipLaunchKernelGGL((k_q4_skinny8<W, true, kQ8>), grid, dim3(64 * W), lds, s, a, pp);
  else hipLaunchKernelGGL((k_q4_skinny8<W, false, kQ8>), grid, dim3(64 * W), lds, s, a, pp);
  return hipGetLastError();
}

template <bool kQ8>
hipError_t launch_8q(const Plan& p, const Q4Args& a, int pp, hipStream_t s) {
  if (p.waves == 4) return launch_w8<4, kQ8>(p, a, pp, s);
  if (p.waves == 8) return launch_w8<8, kQ8>(p, a, pp, s);
  if (p.waves == 16) return launch_w8<16, kQ8>(p, a, pp, s);
  return hipErrorInvalidValue;
}

hipError_t launch_8(const Plan& p, const Q4Args& a, hipStream_t s) {
  const int pp = (int)p.kchunk;
  if (!a.sq || pp % kPH) return hipErrorInvalidValue;
  return p.type == MM_TYPE_Q8_0 ? launch_8q<true>(p, a, pp, s) : launch_8q<false>(p, a, pp, s);
}

// ---- Repacked weights (Q4_0R, repack.hip): per 16-row tile and phase of 8
// blocks one 2304-byte chunk whose 16-byte lane pieces are already this
// kernel's A operands (lane i + 16 g: code bytes 4 g .. 4 g + 3 of row i, for
// 4 blocks per piece) followed by the rows' scales.  A phase is two 16-byte
// loads of codes and one of scales per lane and row tile: no LDS patch, no
// funnel shifts.  Blocks past K are zero padding in both the weights and the
// operand-order wdata, so every wave runs whole phases.
template <int MP, int RT>
struct PhaseR {
  v4i w[RT][2];               // code dwords of blocks 0..3 and 4..7 of this lane's row
  v4i sc[RT];                 // the row's 8 scales (binary16)
  v4i act[MP][kPH];
  v4i da[MP];                 // d_a (binary16) of the phase's 8 blocks, lanes 0-15
};

template <int MP, int RT>
__device__ __forceinline__ void load_phase_r(PhaseR<MP, RT>& P, const Q4Args& a,
                                             const uint8_t* const (&tbase)[RT], int f, int ty) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const uint8_t* c = tbase[rt] + (int64_t)f * kQ4RChunk;
    P.w[rt][0] = *(const __attribute__((address_space(1))) v4i*)(c + 16 * lane);
    P.w[rt][1] = *(const __attribute__((address_space(1))) v4i*)(c + 1024 + 16 * lane);
    P.sc[rt] = *(const __attribute__((address_space(1))) v4i*)(c + 2048 + 16 * (lane & 15));
  }
  const __amdgpu_buffer_rsrc_t rq = wdata_rsrc(a.sq, a.sq_bytes);
  const __amdgpu_buffer_rsrc_t rs = wdata_rsrc(a.ss, a.ss_bytes);
#pragma unroll
  for (int t = 0; t < MP; ++t) {
    const int tp = (ty * MP + t) * a.sk_phases + f;
    const bool rv = (lane & 15) < a.M - (ty * MP + t) * 16;
    const int qo = rv ? tp * 4096 + 16 * lane : kSkip;
#pragma unroll
    for (int j = 0; j < kPH; ++j) P.act[t][j] = bload128(rq, rv ? qo + 1024 * j : kSkip);
    const bool sv = rv && lane < 16;
    P.da[t] = bload128(rs, sv ? (tp * 16 + lane) * 16 : kSkip);
  }
}

template <int MP, int RT, bool kDump>
__device__ __forceinline__ void compute_phase_r(const PhaseR<MP, RT>& P, float (&acc)[RT][MP][4],
                                                int f, int n0, int m0, const Q4Args& a) {
  const int lane = threadIdx.x & 63;
  const int i16 = lane & 15, g = lane >> 4;
  const int nb = a.K / 32;
#pragma unroll
  for (int kb = 0; kb < 2 * kPH; ++kb) {
    const int b = 8 * f + kb;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const long A = nibbles_x16((uint32_t)P.w[rt][kb >> 2][kb & 3]);
      const uint32_t sw = (uint32_t)P.sc[rt][kb >> 1];
      const uint32_t dw = (kb & 1) ? sw & 0xFFFF0000u : sw & 0xFFFFu;
#pragma unroll
      for (int t = 0; t < MP; ++t) {
        const v4i& ac = P.act[t][kb >> 1];
        const long B = (kb & 1) ? (long)(((uint64_t)(uint32_t)ac.w << 32) | (uint32_t)ac.z)
                                : (long)(((uint64_t)(uint32_t)ac.y << 32) | (uint32_t)ac.x);
        const v4i D = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, v4i{0, 0, 0, 0}, 0, 0, 0);
        const v4f sc = scale_tile_k4(dw, kb, P.da[t]);
        acc[rt][t][0] = fmaf((float)D.x, sc.x, acc[rt][t][0]);
        acc[rt][t][1] = fmaf((float)D.y, sc.y, acc[rt][t][1]);
        acc[rt][t][2] = fmaf((float)D.z, sc.z, acc[rt][t][2]);
        acc[rt][t][3] = fmaf((float)D.w, sc.w, acc[rt][t][3]);
        if (kDump && b < nb) {
          const int m = m0 + 16 * t + i16;
          const int Dv[4] = {D.x, D.y, D.z, D.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int n = n0 + 16 * rt + 4 * g + r;
            if (m < a.M && n >= a.n0 && n < a.n1)
              a.dots[((int64_t)m * (a.n1 - a.n0) + (n - a.n0)) * nb + b] = Dv[r] / 16;
          }
        }
      }
    }
  }
}

// Workgroup: RT x 16 weight rows; its W waves split the phases into runs of
// pp phases and add their partial tiles in LDS at the end in a fixed order.
template <int MP, int RT, int W, bool kDump>
__global__ __launch_bounds__(64 * W)
void k_q4r_skinny(Q4Args a, int pp) {
  __shared__ float red[W * RT * MP * 4 * 64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nb = a.K / 32, phases = (nb + 7) / 8, tiles = (a.N + 15) / 16;
  const int n0 = blockIdx.x * 16 * RT, ty = blockIdx.y, m0 = ty * 16 * MP;
  const int f0 = wave * pp < phases ? wave * pp : phases;
  const int f1 = f0 + pp < phases ? f0 + pp : phases;
  const uint8_t* tbase[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int tt = blockIdx.x * RT + rt;
    tt = tt < tiles ? tt : tiles - 1;                // a missing tile's outputs are dropped
    tbase[rt] = a.w + (int64_t)tt * phases * kQ4RChunk;
  }

  float acc[RT][MP][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < MP; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[rt][t][r] = 0.0f;

  // Two register sets, the next phase's loads in flight while one is
  // computed.
  PhaseR<MP, RT> P0, P1;
  const int nph = f1 - f0;
  if (nph > 0) load_phase_r<MP, RT>(P0, a, tbase, f0, ty);
  int f = 0;
  for (; f + 2 < nph; f += 2) {
    load_phase_r<MP, RT>(P1, a, tbase, f0 + f + 1, ty);
    __builtin_amdgcn_sched_barrier(0);
    compute_phase_r<MP, RT, kDump>(P0, acc, f0 + f, n0, m0, a);
    __builtin_amdgcn_sched_barrier(0);
    load_phase_r<MP, RT>(P0, a, tbase, f0 + f + 2, ty);
    __builtin_amdgcn_sched_barrier(0);
    compute_phase_r<MP, RT, kDump>(P1, acc, f0 + f + 1, n0, m0, a);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (f + 1 < nph) {
    load_phase_r<MP, RT>(P1, a, tbase, f0 + f + 1, ty);
    __builtin_amdgcn_sched_barrier(0);
    compute_phase_r<MP, RT, kDump>(P0, acc, f0 + f, n0, m0, a);
    compute_phase_r<MP, RT, kDump>(P1, acc, f0 + f + 1, n0, m0, a);
  } else if (f < nph) {
    compute_phase_r<MP, RT, kDump>(P0, acc, f0 + f, n0, m0, a);
  }

  constexpr int NT = RT * MP;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < MP; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[((wave * NT + rt * MP + t) * 4 + r) * 64 + lane] = acc[rt][t][r];
  __syncthreads();
  for (int idx = threadIdx.x; idx < NT * 256; idx += 64 * W) {
    const int tt = idx >> 8, r = (idx >> 6) & 3, l = idx & 63;
    const int rt = tt / MP, t = tt - rt * MP;
    float s = 0.0f;
    for (int w2 = 0; w2 < W; ++w2) s += red[((w2 * NT + tt) * 4 + r) * 64 + l];
    const int m = m0 + 16 * t + (l & 15);
    const int n = n0 + 16 * rt + 4 * (l >> 4) + r;
    if (m < a.M && n < a.N) a.dst[(int64_t)m * a.N + n] = s * 0.0625f;   // 16 S_b
  }
}

template <int MP, int RT, int W>
hipError_t launch_r(const Plan& p, const Q4Args& a, hipStream_t s) {
  const dim3 grid((unsigned)p.tiles_n, (unsigned)p.tiles_m, 1u);
  const int pp = (int)p.kchunk;                     // phases per wave
  if (a.dots) hipLaunchKernelGGL((k_q4r_skinny<MP, RT, W, true>), grid, dim3(64 * W), 0, s, a, pp);
  else hipLaunchKernelGGL((k_q4r_skinny<MP, RT, W, false>), grid, dim3(64 * W), 0, s, a, pp);
  return hipGetLastError();
}

template <int MP, int RT>
hipError_t launch_r_mp(const Plan& p, const Q4Args& a, hipStream_t s) {
  if (p.waves == 4) return launch_r<MP, RT, 4>(p, a, s);
  if (p.waves == 8) return launch_r<MP, RT, 8>(p, a, s);
  if constexpr (MP == 1 && RT == 1) {
    if (p.waves == 16) return launch_r<MP, RT, 16>(p, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool q4_skinny_ok(int K, const void* w) {
  return K % 64 == 0 && (uintptr_t)w % 4 == 0;
}

hipError_t launch_q4_skinny(const Plan& p, const Q4Args& a, hipStream_t s) {
  if (p.split != 1 || !q4_skinny_ok(a.K, a.w)) return hipErrorInvalidValue;
  if (p.mt == 8 && p.rpw == 16) return launch_8(p, a, s);
  if (p.type == MM_TYPE_Q8_0 && p.rpw != 16) return hipErrorInvalidValue;
  if (p.mt == 16 && p.rpw == 16) return launch_mp<1, 1>(p, a, s);
  if (p.mt == 32 && p.rpw == 16) return launch_mp<2, 1>(p, a, s);
  if (p.mt == 16 && p.rpw == 32) return launch_mp<1, 2>(p, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_q4r_skinny(const Plan& p, const Q4Args& a, hipStream_t s) {
  if (p.split != 1 || !a.sq) return hipErrorInvalidValue;
  if (p.mt == 16 && p.rpw == 16) return launch_r_mp<1, 1>(p, a, s);
  if (p.mt == 32 && p.rpw == 16) return launch_r_mp<2, 1>(p, a, s);
  if (p.mt == 16 && p.rpw == 32) return launch_r_mp<1, 2>(p, a, s);
  return hipErrorInvalidValue;
}

}  // namespace qsg
