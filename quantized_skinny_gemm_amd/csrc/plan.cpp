// Host-only dispatch plan, workspace layout and argument validation.
#include "plan.h"

#include <stdint.h>

#include "../../include/mm.h"

namespace qsg {

namespace {

constexpr int64_t kMaxDim = 0x7fffffff;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

int narrow_mt(int64_t M, int cap) {
  int mt = 1;
  while (mt < M && mt < cap) mt <<= 1;
  return mt;
}

}  // namespace

int64_t row_bytes(int type, int64_t K) {
  if (K < 0) return -1;
  switch (type) {
    case MM_TYPE_F32: return 4 * K;
    case MM_TYPE_F16: return 2 * K;
    case MM_TYPE_Q4_0: return (K % kQK) ? -1 : K / kQK * kQ4Bytes;
    case MM_TYPE_Q8_0: return (K % kQK) ? -1 : K / kQK * kQ8Bytes;
    case MM_TYPE_Q4_0R: return -1;                 // tiled, not row-major (repacked_bytes)
    default: return -1;
  }
}

int64_t repacked_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0 || K % kQK || N > kMaxDim || K > kMaxDim) return -1;
  return ceil_div(N, 16) * ceil_div(K / kQK, 8) * kQ4RChunk;
}

int make_plan(int type, int64_t M, int64_t N, int64_t K, int variant, Plan* p, bool allow_split) {
  *p = Plan();
  p->type = type;
  if (type != MM_TYPE_F32 && type != MM_TYPE_F16 && type != MM_TYPE_Q4_0 &&
      type != MM_TYPE_Q4_0R && type != MM_TYPE_Q8_0)
    return MM_ERR_ARG;
  if (variant < 0 || variant > 3) return MM_ERR_ARG;
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return MM_ERR_SHAPE;
  const bool q8 = type == MM_TYPE_Q8_0;
  if ((type == MM_TYPE_Q4_0 || type == MM_TYPE_Q4_0R || q8) && (K % kQK)) return MM_ERR_SHAPE;
  if (type == MM_TYPE_Q4_0R && variant == 1) return MM_ERR_ARG;   // no narrow kernel for it
  // Q8_0 weights: the skinny kernel takes block pairs (K / 32 even)
  if (q8 && variant == 3 && (K / kQK) % 2) return MM_ERR_ARG;
  if (M == 0 || N == 0) { p->kind = KK_NONE; return MM_OK; }
  if (K == 0) { p->kind = KK_ZERO; return MM_OK; }
  // The narrow and skinny kernels put src1 row tiles in the grid's y
  // dimension (at most kMaxGridY workgroups): products of more rows keep to
  // the built-in rules, which give the block types the wide kernel there
  // (a one-dimensional grid); the F16 / F32 launchers run such grids as
  // several launches over consecutive row ranges.
  if (variant == 0 && M <= kMaxGridY) {
    int tv = dispatch_table_variant(type, M, N, K);
    const int nm = env_narrow_max_m();
    if (nm >= 0 && type == MM_TYPE_Q4_0)             // experiment override
      tv = M <= nm ? 1 : (tv > 1 ? tv : (M <= kMmaMaxM ? 3 : 2));
    dispatch_log(type, M, N, K, tv, tv != 0);
    variant = tv;
  }

  if (type == MM_TYPE_Q4_0 || type == MM_TYPE_Q4_0R || q8) {
    const bool rep = type == MM_TYPE_Q4_0R;
    const int64_t nb = K / kQK;
    // M <= 2: the fused narrow kernel; up to kMmaMaxM: the skinny MFMA
    // kernel; beyond: the tiled wide kernel.  Repacked weights: the skinny
    // kernel from M = 1.  Q8_0 weights: the fused kernel (block pairs, so K
    // a multiple of 64, and src1 staged whole in LDS) for M <= 2 or when
    // forced (passes of two src1 rows), the wide kernel otherwise.
    const bool q8_fusable = q8 && nb % 2 == 0 && 2 * nb * 40 <= kNarrowMaxLds;
    const bool mma = q8 ? nb % 2 == 0 && (variant == 3 || (variant == 0 && M > kFuseMaxM && M <= kMmaMaxM))
                        : variant == 3 || (variant == 0 && (rep || M > kFuseMaxM) && M <= kMmaMaxM);
    const bool narrow = q8 ? q8_fusable && (variant == 1 || (variant == 0 && M <= kFuseMaxM))
                           : !mma && (variant == 1 || (variant == 0 && M <= kNarrowQ4MaxM));
    if (q8 && variant == 1 && !narrow) return MM_ERR_ARG;
    if ((mma || narrow) && M > kMaxGridY) return MM_ERR_SHAPE;   // forced on too many rows
    // wdata: codes, scales, bias; the codes and scales are followed by 256
    // spare bytes (the skinny kernel's last phase may read up to 7 blocks past
    // the end, and drops them)
    size_t off = 0;
    p->off_aq = off; off = align_up(off + (size_t)M * (size_t)K + 256, 256);
    p->off_ad = off; off = align_up(off + (size_t)M * (size_t)nb * 4 + 256, 256);
    p->off_ab = off; off = align_up(off + (size_t)M * (size_t)nb * 4, 256);
    if (mma && rep) {
      // one 16-row tile per workgroup; its waves split the phases of 8 blocks
      // among themselves (whole phases: the weights and the operand-order
      // wdata are zero past K); passes of 16 or 32 src1 rows.
      p->kind = KK_Q4R_SKINNY;
      p->variant = 3;
      p->mt = M <= 16 ? 16 : 32;
      p->rpw = 16;
      p->tiles_m = ceil_div(M, p->mt);
      p->tiles_n = ceil_div(N, p->rpw);
      p->split = 1;
      const int64_t phases = ceil_div(nb, 2 * kSkinnyPairs);
      const int wmax = p->mt == 16 ? 16 : 8;
      const int64_t wtarget = (p->mt == 32 ? 8 : 16) * (int64_t)kCUs;
      const int64_t tiles = p->tiles_m * p->tiles_n;
      int w = 4;
      while (w < wmax && tiles * w < wtarget && phases >= 2 * w) w *= 2;
      p->waves = w;
      p->kchunk = ceil_div(phases, w);                 // phases per wave
      const int64_t sk_rows = p->tiles_m * p->mt;
      if (sk_rows * phases * 256 > ((int64_t)1 << 30)) return MM_ERR_SHAPE;
      p->sk_rows = sk_rows;
      p->sk_phases = phases;
      p->off_sq = off; off = align_up(off + (size_t)sk_rows * phases * 256, 256);
      p->off_ss = off; off = align_up(off + (size_t)sk_rows * phases * 32, 256);
    } else if (mma) {
      // 16-row workgroups whose waves split K among themselves (no split
      // across workgroups, so no partial sums in the workspace); passes of
      // 8 src1 rows (two blocks per MFMA), 16 or 32.
      p->kind = KK_Q4_MMA;
      p->variant = 3;
      p->mt = M <= 8 ? 8 : M <= 16 ? 16 : 32;
      // 16 weight rows per workgroup (and per wave).  (32, two MFMA row
      // tiles sharing each activation load, measured no faster at 14336 rows
      // and slower at 4096: half the workgroups.)
      p->rpw = 16;
      p->tiles_m = ceil_div(M, p->mt);
      p->tiles_n = ceil_div(N, p->rpw);
      p->split = 1;
      // Waves per workgroup: enough workgroups x waves for about 16 waves
      // per CU (8 with 32-row passes, whose waves hold twice the
      // activations), each wave keeping at least one phase of block pairs;
      // at most 16 waves with 8-row passes, 8 otherwise (measured, us per
      // call: M = 32, 14336 x 4096 with 4 waves instead of 8, 27.6 -> 23.9;
      // M = 16, 4096 x 14336 with 8 instead of 16, 17.6 -> 17.1; fewer waves
      // at M = 8 / 16 on 14336 x 4096, or more anywhere, are slower).
      const int wmax = p->mt <= 8 ? 16 : 8;
      const int64_t wtarget = (p->mt == 32 ? 8 : 16) * (int64_t)kCUs;
      const int64_t tiles = p->tiles_m * p->tiles_n;
      int w = 4;
      while (w < wmax && tiles * w < wtarget && nb / 2 >= 2 * w * kSkinnyPairs) w *= 2;
      p->waves = w;
      // block pairs per wave: whole phases, so that every wave's phases
      // start on a phase of the operand-order wdata
      const int64_t pairs = nb / 2;
      p->kchunk = ceil_div(ceil_div(pairs, w), kSkinnyPairs) * kSkinnyPairs;
      // INIT also writes the codes and scales in the kernel's operand order:
      // per tile and phase of 8 blocks, mt x 256 bytes of codes and 16 x 8
      // (8-row tiles: 16 x 4) scales; padding rows and blocks are zero.  The
      // kernels address these ranges with 32-bit offsets: past 1 GiB of codes
      // the layout is not written and the product takes the fallback kernel.
      const int64_t sk_rows = p->tiles_m * p->mt, sk_phases = ceil_div(nb, 2 * kSkinnyPairs);
      if (sk_rows * sk_phases * 256 <= ((int64_t)1 << 30)) {
        p->sk_rows = sk_rows;
        p->sk_phases = sk_phases;
        p->off_sq = off; off = align_up(off + (size_t)sk_rows * sk_phases * 256, 256);
        p->off_ss = off; off = align_up(off + (size_t)sk_rows * sk_phases * 32, 256);
      }
    } else if (narrow) {
      p->kind = KK_Q4_NARROW;
      p->variant = 1;
      p->mt = narrow_mt(M, kNarrowQ4MaxM);
      p->rpw = p->mt <= 2 ? 2 : 4;
      // M = 1 with many rows: one weight row per wave (twice the row groups;
      // decode step: q,k,v grouped 8.6 -> 8.2 us, gate,up grouped 12.7 ->
      // 11.4 us); up to 8192 rows two rows per wave stay as fast or faster.
      if (p->mt == 1 && N > 8192) p->rpw = 1;
      p->waves = p->mt <= 2 ? 8 : 4;
      p->tiles_m = ceil_div(M, p->mt);
      p->tiles_n = ceil_div(N, p->waves * p->rpw);
      // K units of the narrow kernel are block pairs (blocks when K/32 is odd).
      const int64_t units = (nb % 2 == 0) ? nb / 2 : nb;
      // Split K when there are fewer than 4 waves per CU.
      const int64_t waves = p->tiles_m * p->tiles_n * p->waves;
      int64_t split = 1;
      if (allow_split && waves < 4 * kCUs) {
        const int64_t max_split = units / 64;        // keep every lane busy
        split = ceil_div(4 * kCUs, waves);
        if (split > max_split) split = max_split;
        if (split > 16) split = 16;
        if (split < 1) split = 1;
      }
      if (allow_split && env_split_k() > 0) {         // experiment override
        const int64_t max_split = units / 64 > 1 ? units / 64 : 1;
        split = env_split_k() < max_split ? env_split_k() : max_split;
      }
      p->kchunk = ceil_div(units, split);
      p->split = (int)ceil_div(units, p->kchunk);
      // At most kNarrowMaxGrid workgroups along N, each walking an equal
      // number of row groups (the activation slice is staged once per
      // workgroup, so fewer, longer-lived workgroups re-read it less).
      p->grid_n = p->tiles_n < kNarrowMaxGrid ? p->tiles_n : kNarrowMaxGrid;
      // Fuse the INIT stage (src1 -> Q8_0 in LDS, 40 bytes per block and row)
      // when the pass is small: every workgroup re-quantizes its src1 slice,
      // which costs about M / (0.56 * rows per wave) of the weight traffic in
      // L2 reads, and saves a launch and the wdata round trip.
      const int64_t kblocks = (nb % 2 == 0) ? 2 * p->kchunk : p->kchunk;
      p->fuse = p->mt <= kFuseMaxM && (int64_t)p->mt * kblocks * 40 <= kNarrowMaxLds;
      // The fused kernel's own geometry (same arithmetic per row): as the
      // narrow plan, except at M = 1 with at most 8192 rows, where it also
      // takes one row per wave: with 8 waves per workgroup (twice the row
      // groups; us per call: 2048 x 4096 4.25 -> 3.61, 8192 x 4096 7.00 ->
      // 6.88, 4096 x 4096 unchanged), and for K > 8192 with 16 (the same 16
      // rows per group, twice the waves per CU in flight: decode step, down
      // projection 4096 x 11008, 8.19 -> 7.61).
      p->fuse_rpw = p->rpw;
      p->fuse_waves = p->waves;
      if (p->fuse && p->mt == 1 && N <= 8192) { p->fuse_rpw = 1; p->fuse_waves = K > 8192 ? 16 : 8; }
      // M = 2: only the long-K case pays (4096 x 11008: 11.0 -> 9.8 us; one
      // row per wave elsewhere is slower, 4096 x 4096 5.2 -> 5.4)
      if (p->fuse && p->mt == 2 && N <= 8192 && K > 8192) { p->fuse_rpw = 1; p->fuse_waves = 16; }
      if (q8) {
        // Q8_0 weights: the fused kernel only, in passes of at most two src1
        // rows, K whole (every workgroup stages all of src1)
        p->mt = narrow_mt(M, kFuseMaxM);
        p->tiles_m = ceil_div(M, p->mt);
        p->kchunk = units;
        p->split = 1;
        p->fuse = true;
        p->fuse_rpw = p->mt == 1 ? 1 : 2;
        p->fuse_waves = K > 8192 ? 16 : 8;
        if (p->mt == 2 && K > 8192) p->fuse_rpw = 1;
      }
      {
        const int64_t groups = ceil_div(N, (int64_t)p->fuse_rpw * p->fuse_waves);
        p->fuse_grid = groups < kNarrowMaxGrid ? groups : kNarrowMaxGrid;
      }
    } else {
      p->kind = KK_Q4_WIDE;
      p->variant = 2;
      // Output tile by M.  The 128 x 128 tile does about three times the
      // MFMA work per staged byte of a 128 x 64 one, so a grid that cannot
      // fill the device splits K (below) rather than shrinking the tile.
      // Measured tile choices (us):  up to M = 64 with few weight rows
      // (N <= 8192, so K is split at least 4 ways) a 64 x 128 tile, whose
      // waves hold two MFMA tiles each, beats 64 x 64 (4096 x 14336, M = 64:
      // 34.7 against 43.7), with many rows it does not; from M = 65 to 128 it
      // is the reverse: with many rows two 64-row tiles sharing each weight
      // tile through L2 beat one 128 x 128 tile (14336 x 4096, M = 128: 51.7
      // against 57.6; M = 100: 47.9 against 55.2), with few rows they lose
      // (4096 x 14336: 56.3 against 52.7).  Tiles with 8 or 16 waves were
      // slower everywhere.
      const bool many_rows = N > 8192;
      if (M <= 32) { p->bm = 32; p->bn = 64; p->waves_m = 1; p->waves_n = 2; }
      else if (M <= 64 && !many_rows) { p->bm = 64; p->bn = 128; p->waves_m = 2; p->waves_n = 2; }
      else if (M <= 64) { p->bm = 64; p->bn = 64; p->waves_m = 2; p->waves_n = 2; }
      else if (M <= 128 && many_rows) { p->bm = 64; p->bn = 128; p->waves_m = 2; p->waves_n = 2; }
      else { p->bm = 128; p->bn = 128; p->waves_m = 2; p->waves_n = 2; }
      // Q8_0 weights stage twice the bytes per pair: the 128 x 128 tile
      // would hold more than 256 VGPRs (one wave per SIMD); 128 x 64 keeps two
      if (q8 && p->bm == 128 && p->bn == 128) p->bn = 64;
      p->tiles_m = ceil_div(M, p->bm);
      p->tiles_n = ceil_div(N, p->bn);
      const int64_t tiles = p->tiles_m * p->tiles_n;
      const int64_t stages = ceil_div(nb, kWideI8KB);
      // Fewer tiles than CUs: split K for about two workgroups per CU, at
      // least 4 stages per split (us per call, against one workgroup per CU
      // and 2 stages: M = 512, 4096 x 4096 58.7 -> 49.5; M = 128, 4096 x 14336
      // 54.2 -> 47.3-48.8; M = 256, 4096 x 4096 39.2 -> 34.5; M = 40,
      // 11008 x 4096 33.9 -> 31.8; M = 64, 14336 x 4096 35.4 -> 36.3).  With
      // enough tiles it does not pay (M = 512, 14336 x 4096, split 2: 127 ->
      // 142).
      int64_t split = 1;
      if (allow_split && tiles < kCUs) {
        split = ceil_div(2 * kCUs, tiles);
        const int64_t max_split = stages / 4;          // >= 4 stages per split
        if (split > max_split) split = max_split;
        if (split > 16) split = 16;
        if (split < 1) split = 1;
      }
      if (allow_split && env_split_k() > 0)            // experiment override
        split = env_split_k() < stages ? env_split_k() : stages;
      p->kchunk = ceil_div(stages, split) * kWideI8KB;   // blocks per split
      p->split = (int)ceil_div(nb, p->kchunk);
    }
    if (p->split > 1) {
      p->off_part = off; off = align_up(off + (size_t)p->split * (size_t)M * (size_t)N * 4, 256);
    }
    p->ws_bytes = off;
    return MM_OK;
  }

  // F16 / F32: M = 1 the narrow kernel; from 2 rows the skinny MFMA kernel
  // (passes of 16 rows), for F16 only up to the limit below, beyond which
  // the wide kernel takes it.
  if (variant == 2 && type != MM_TYPE_F16) return MM_ERR_ARG;
  const bool f16 = type == MM_TYPE_F16;
  // F16 from 17 rows: the wide kernel, except up to 64 rows with at most
  // 8192 weight rows, where its 64 x 64 tiles give too few workgroups and
  // passes of the skinny kernel are faster (4096 x 4096: M = 32 17.8 against
  // 39.6 us, M = 64 33.1 against 39.9; 14336 rows favour the wide kernel).
  const bool wide = f16 && (variant == 2 || (variant == 0 && M > kNarrowFMaxM && (M > 64 || N > 8192)));
  const bool fmma = !wide && (variant == 3 || (variant == 0 && M >= 2));
  if (fmma) {
    p->kind = KK_F_MMA;
    p->variant = 3;
    p->mt = 16;
    // One workgroup per 16 weight rows (32 when src1 takes several 16-row
    // passes, which then share each src1 load between two row tiles) and
    // pass; its waves split K into runs of whole MFMA steps (32 k for F16,
    // 16 k for F32) and add their partial tiles in LDS, so no K slice goes
    // through the workspace.  8 waves of two-step sub-slices, 4 with 32-row
    // workgroups (us per call, against the best of 4 / 8 / 16 waves and
    // 2 / 4 steps: F32 4096 x 4096 M = 4 14.6, M = 16 18.9; 11008 x 4096
    // M = 4 38.8, M = 16 52.3; F16 11008 x 4096 M = 4 26.2; F16 4096 x 4096
    // M = 4 10.7 against 10.6, M = 16 14.7 against 14.0; M = 32 / 64 with
    // 32-row workgroups: F16 17.8 / 33.1 against 24.6 / 45.6 with 16 rows).
    const int rt = M > 16 ? 2 : 1;
    p->rpw = 16 * rt;                                  // weight rows per workgroup
    p->tiles_m = ceil_div(M, 16);
    p->tiles_n = ceil_div(N, p->rpw);
    const int64_t step = f16 ? 32 : 16;
    const int64_t steps = ceil_div(K, step);
    p->bn = 2;                                         // steps per sub-slice
    int w = rt == 1 ? 8 : 4;
    while (w > 1 && steps < 2 * p->bn * w) w /= 2;     // every wave at least one sub-slice pair
    if (w < 4) w = 4;
    p->waves = w;
    // steps per wave: a whole number of sub-slice pairs (the kernel's two
    // register sets)
    p->kchunk = ceil_div(ceil_div(steps, w), 2 * p->bn) * 2 * p->bn;
    p->split = 1;
    p->ws_bytes = 0;
    return MM_OK;
  }
  if (!wide) {
    p->kind = KK_F_NARROW;
    p->variant = 1;
    p->mt = narrow_mt(M, kNarrowFMaxM);
    p->rpw = p->mt >= 8 ? 2 : 4;
    // M = 1: one weight row per wave (four times the workgroups, each wave's
    // loads of several chunks in flight) except for F16 with many rows,
    // where four rows per wave stay faster (measured: F32 4096 x 4096
    // 18.6 -> 14.1 us, 11008 x 4096 42.6 -> 33.9; F16 4096 x 4096 9.6 -> 8.2;
    // F16 11008 x 4096 19.0 with four rows against 20.1)
    if (p->mt == 1 && (type == MM_TYPE_F32 || N <= 8192)) p->rpw = 1;
    p->tiles_m = ceil_div(M, p->mt);
    // K slices: when the row groups alone give fewer than about four waves
    // per SIMD, the waves of a workgroup split K over the same rows (each
    // slice keeping at least one 64-chunk round per lane).  Measured (us per
    // call, F16 M = 2): 4096 x 4096 10.7 -> 8.5, 4096 x 11008 25.4 -> 21.4;
    // with more than 8192 rows (four rows per wave) it is slower (11008 x
    // 4096, M = 1: 18.7 -> 21.1), so those keep one slice.
    p->kslices = 1;
    const int64_t groups = ceil_div(N, p->rpw);
    while (N <= 8192 && p->kslices < 4 && groups * p->kslices < 16 * kCUs &&
           K >= (int64_t)1024 * p->kslices)
      p->kslices *= 2;
    p->tiles_n = ceil_div(N, (4 / p->kslices) * p->rpw);
  } else {
    p->kind = KK_F16_WIDE;
    p->variant = 2;
    p->bm = 128; p->bn = 128; p->waves_m = 2; p->waves_n = 2;
    p->tiles_m = ceil_div(M, p->bm);
    p->tiles_n = ceil_div(N, p->bn);
    if (p->tiles_m * p->tiles_n < kCUs) {
      p->bm = 64; p->bn = 64;
      p->tiles_m = ceil_div(M, p->bm);
      p->tiles_n = ceil_div(N, p->bn);
    }
    // At most one tile per two CUs: split K (slices of whole k stages, at
    // least four stages each) for about two workgroups per CU, the partial
    // tiles added by the split-K reduce (us per call, M = 4 / 64 / 128:
    // 4096 x 4096 25.9 / 28.1 / 29.1 -> 17.9 / 22.1 / 24.9; 4096 x 14336
    // 77.2 / 81.0 / 81.8 -> 37.6 / 43.6 / 55.8).  With 172 or 224 tiles
    // (11008 / 14336 rows) the reduce costs more than it gains (14336 x 4096,
    // M = 64: 35.3 -> 41.7).
    const int64_t ks = p->bm == 128 ? 64 : 128;       // k per stage
    const int64_t stages = ceil_div(K, ks);
    const int64_t tiles = p->tiles_m * p->tiles_n;
    int64_t split = 1;
    if (allow_split && 2 * tiles <= kCUs) {
      split = ceil_div(2 * kCUs, tiles);
      if (split > stages / 4) split = stages / 4;
      if (split > 8) split = 8;
      if (split < 1) split = 1;
    }
    if (allow_split && env_split_k() > 0)              // experiment override
      split = env_split_k() < stages ? env_split_k() : stages;
    p->kchunk = ceil_div(stages, split) * ks;
    p->split = (int)ceil_div(K, p->kchunk);
    if (p->split < 1) p->split = 1;
    // src1 as binary16 [M][K], converted once (not per tile and stage), and
    // its power-of-two exponent per row; then the split partials
    p->off_ah = 0;
    p->off_rexp = align_up((size_t)M * (size_t)K * 2, 256);
    size_t off = align_up(p->off_rexp + (size_t)M * 4, 256);
    if (p->split > 1) {
      p->off_part = off;
      off = align_up(off + (size_t)p->split * (size_t)M * (size_t)N * 4, 256);
    }
    p->ws_bytes = off;
    return MM_OK;
  }
  p->ws_bytes = 0;
  return MM_OK;
}

int validate_mul_mat(int type, const void* src0, const void* src1, const void* dst,
                     int64_t M, int64_t N, int64_t K, const void* ws, size_t ws_bytes,
                     const Plan& p, int stage, bool check_ws) {
  if (p.kind == KK_NONE) return MM_OK;
  const bool need_src0 = stage != STAGE_INIT && K > 0;
  const bool need_src1 = stage != STAGE_COMPUTE && K > 0;
  const bool need_dst = stage != STAGE_INIT;
  if (need_dst && !dst) return MM_ERR_NULL;
  if ((need_src0 && !src0) || (need_src1 && !src1)) return MM_ERR_NULL;
  if (!need_src0) src0 = nullptr;
  if (!need_src1) src1 = nullptr;
  if (!need_dst) dst = nullptr;
  const uintptr_t s0 = (uintptr_t)src0, s1 = (uintptr_t)src1, d = (uintptr_t)dst;
  if (d % 4) return MM_ERR_ALIGN;
  if (type == MM_TYPE_Q4_0) {
    if (s0 % 2 || s1 % 16) return MM_ERR_ALIGN;
  } else if (type == MM_TYPE_Q8_0) {
    if (s0 % 4 || s1 % 16) return MM_ERR_ALIGN;
  } else if (type == MM_TYPE_Q4_0R) {
    if (s0 % 16 || s1 % 16) return MM_ERR_ALIGN;
  } else if (type == MM_TYPE_F16) {
    if (s0 % 2 || s1 % 4) return MM_ERR_ALIGN;
  } else {
    if (s0 % 4 || s1 % 4) return MM_ERR_ALIGN;
  }
  if (!check_ws) ws = nullptr;
  if (check_ws && p.ws_bytes > 0) {
    if (!ws || ws_bytes < p.ws_bytes) return MM_ERR_WORKSPACE;
    if ((uintptr_t)ws % 256) return MM_ERR_ALIGN;
  }
  const size_t dst_bytes = dst ? (size_t)M * (size_t)N * 4 : 0;
  const size_t s0_bytes = !src0 ? 0
                          : type == MM_TYPE_Q4_0R ? (size_t)repacked_bytes(N, K)
                                                  : (size_t)N * (size_t)row_bytes(type, K);
  const size_t s1_bytes = src1 ? (size_t)M * (size_t)K * 4 : 0;
  if (overlaps(dst, dst_bytes, src0, s0_bytes) || overlaps(dst, dst_bytes, src1, s1_bytes))
    return MM_ERR_ALIAS;
  if (ws && p.ws_bytes > 0 &&
      (overlaps(ws, p.ws_bytes, dst, dst_bytes) || overlaps(ws, p.ws_bytes, src0, s0_bytes) ||
       overlaps(ws, p.ws_bytes, src1, s1_bytes)))
    return MM_ERR_ALIAS;
  return MM_OK;
}

int validate_quantize(int out_type, const void* x, const void* y, int64_t nrows, int64_t k) {
  if (nrows < 0 || k < 0 || nrows > kMaxDim || k > kMaxDim) return MM_ERR_SHAPE;
  if (k % kQK) return MM_ERR_SHAPE;
  if (nrows == 0 || k == 0) return MM_OK;
  if (!x || !y) return MM_ERR_NULL;
  if ((uintptr_t)x % 16 || (uintptr_t)y % 2) return MM_ERR_ALIGN;
  const size_t xb = (size_t)nrows * (size_t)k * 4;
  const size_t yb = (size_t)nrows * (size_t)row_bytes(out_type, k);
  if (overlaps(x, xb, y, yb)) return MM_ERR_ALIAS;
  return MM_OK;
}

}  // namespace qsg
