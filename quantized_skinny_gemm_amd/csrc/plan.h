// Host-only dispatch plan and argument validation (no HIP calls).
//
// The plan is a pure function of (type, M, N, K, variant): the workspace
// size a caller is told to allocate and the kernels the entry point launches
// always agree.  Tile and split choices follow two observations from the
// pages: a narrow-M kernel that streams each weight once beats tiled kernels
// for small M but loses quickly past its threshold (smallbard "Generer a
// plusieurs", "La courbe, une premiere fois"), and a product whose output
// tiles are too few to fill the device is split along the common dimension
// with the partial sums added afterwards (same section; DeepSpeed-Inference
// notes, SBI-GeMM tiling strategy).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace qsg {

constexpr int kQK = 32;            // values per Q4_0 / Q8_0 block
constexpr int kQ4Bytes = 18;       // bytes per Q4_0 block
constexpr int kQ8Bytes = 34;       // bytes per Q8_0 block
constexpr int kQ4RChunk = 2304;    // repacked Q4_0: bytes per 16-row tile and phase of 8 blocks
constexpr int kCUs = 256;          // MI355X compute units
constexpr int kWideI8KB = 4;       // Q4_0 blocks per LDS stage, int8 wide kernel
constexpr int kNarrowQ4MaxM = 8;   // largest M the Q4_0 narrow kernel takes in one pass
constexpr int kNarrowFMaxM = 16;   // largest M the f16/f32 narrow kernel takes in one pass
constexpr int kFuseMaxM = 2;       // narrow Q4_0 passes of at most this many rows fuse INIT
constexpr int kNarrowMaxLds = 65536; // LDS bytes the narrow kernel may stage activations in
constexpr int kNarrowMaxGrid = 768;  // narrow workgroups along N (3 per CU)
constexpr int kMmaMaxM = 32;       // largest M the skinny MFMA kernel takes by default
constexpr int kSkinnyPairs = 4;    // skinny kernel: block pairs per wave phase
constexpr int64_t kFMmaMaxK = 1 << 23;  // skinny F kernel: 32-bit buffer offsets over 32 rows
constexpr int64_t kMaxGridY = 65535; // documented limit of a grid's y dimension (workgroups)
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;  // mm_mul_mat_q4_0_f32_noalloc's array
constexpr int kMmaWaves = 8;       // waves per workgroup of the skinny kernel for unaligned
                                   // weights or K % 64 != 0 (32 rows per workgroup)

enum KernelKind {
  KK_NONE = 0,      // nothing to do (M == 0 or N == 0)
  KK_ZERO = 1,      // K == 0: dst = 0
  KK_Q4_NARROW = 2,
  KK_Q4_WIDE = 3,
  KK_F_NARROW = 4,  // f16 or f32 src0
  KK_F16_WIDE = 5,
  KK_Q4_MMA = 6,    // skinny Q4_0 on int8 MFMA (16 weight rows per workgroup)
  KK_Q4R_SKINNY = 9, // skinny Q4_0 on repacked weights (int8 MFMA, operands loaded as stored)
  KK_F_MMA = 8,     // skinny F16 / F32 on the 16x16 MFMA (16 weight rows per workgroup,
                    // passes of 16 src1 rows, waves split K)
};

struct Plan {
  int type = 0;
  int kind = KK_NONE;
  int variant = 0;          // 1 narrow, 2 wide (Q4_0: int8; F16: fp16), 3 skinny MFMA
  // narrow kernels
  int mt = 1;               // src1 rows per pass (compile-time tile)
  int rpw = 1;              // src0 rows per wave (skinny MFMA: per workgroup)
  int waves = 4;            // waves per workgroup (skinny MFMA: they split K)
  // wide kernels
  int bm = 0, bn = 0, waves_m = 0, waves_n = 0;   // (skinny F MFMA kernel: bn = steps per sub-slice)
  // grid
  int64_t tiles_m = 1;      // wide: output tile rows; narrow: passes over M
  int64_t tiles_n = 1;      // output tile columns (narrow: row groups of waves*rpw src0 rows)
  int64_t grid_n = 1;       // narrow: workgroups along N (each walks tiles_n / grid_n row groups)
  int split = 1;            // split-K factor
  bool fuse = false;        // narrow Q4_0: quantize src1 inside the product kernel
  int fuse_rpw = 2, fuse_waves = 8;  // fused kernel: rows per wave and waves per workgroup
  int64_t fuse_grid = 0;    // fused kernel: workgroups along N
  int kslices = 1;          // narrow F kernel: waves of a workgroup splitting K over the same rows
  int64_t kchunk = 0;       // K per split (Q4 narrow: units; Q4 wide / skinny: blocks;
                            // skinny F: MFMA steps per wave)
  // workspace layout (bytes)
  size_t off_aq = 0, off_ad = 0, off_ab = 0, off_part = 0;
  size_t off_ah = 0;        // wide F16 kernel: src1 as binary16 [M][K]
  size_t off_rexp = 0;      // wide F16 kernel: int32 [M] power-of-two exponent per src1 row
  size_t off_sq = 0, off_ss = 0;   // skinny MFMA kernel: its operand-order codes and scales
                                   // (0: not written)
  int64_t sk_rows = 0;      // skinny layout: src1 rows padded to 16-row tiles
  int64_t sk_phases = 0;    // skinny layout: phases of 8 blocks (K padded to 256)
  size_t ws_bytes = 0;
};

// The measured dispatch table (dispatch_table.cpp): the variant listed for
// (type, N, K) at this M, or 0 when the table has none (or no table was
// found).  The file is read once per process.
int dispatch_table_variant(int type, int64_t M, int64_t N, int64_t K);
// Experiment overrides from the environment, read once per process with the
// table; -1 when unset.  MM_NARROW_MAX_M: Q4_0 products with M up to this
// value take the narrow kernel and larger ones never do (0: never).
// MM_SPLIT_K: the K split of the narrow and wide kernels (clamped to what
// the shape allows).
int env_narrow_max_m();
int env_split_k();
// Logs a dispatch decision on stderr when MM_VERBOSE is set.
void dispatch_log(int type, int64_t M, int64_t N, int64_t K, int variant, bool from_table);

// Builds the plan; returns 0 (MM_OK) or a negative mm_status.  variant 0
// takes the table's choice for the shape if it lists one, else the built-in
// rules.
// allow_split = false keeps K whole (used when several matrices share one
// launch: their outputs are written directly, never as split partials).
int make_plan(int type, int64_t M, int64_t N, int64_t K, int variant, Plan* p,
              bool allow_split = true);

// Which operands a call takes: the whole product, or one of the two stages
// of the quantized product (INIT: src1 -> wdata; COMPUTE: src0 x wdata -> dst).
enum Stage { STAGE_ALL = 0, STAGE_INIT = 1, STAGE_COMPUTE = 2 };

// Argument checks of mm_mul_mat_* / mm_q4_0_init / mm_q4_0_compute /
// mm_debug_mul_mat; no HIP calls.
// check_ws = false skips the workspace checks (the no-allocation entry
// point supplies its own array).
int validate_mul_mat(int type, const void* src0, const void* src1, const void* dst,
                     int64_t M, int64_t N, int64_t K, const void* ws, size_t ws_bytes,
                     const Plan& p, int stage = STAGE_ALL, bool check_ws = true);

// Argument checks of mm_quantize_q4_0 / mm_quantize_q8_0; no HIP calls.
int validate_quantize(int out_type, const void* x, const void* y, int64_t nrows, int64_t k);

int64_t row_bytes(int type, int64_t K);

// Bytes of N x K Q4_0 weights in the repacked layout (repack.hip): tiles of
// 16 rows x phases of 8 blocks, padded; -1 for an invalid shape.
int64_t repacked_bytes(int64_t N, int64_t K);

}  // namespace qsg
