// Narrow-M Q4_0 x Q8_0 product for gfx950 (M <= 8 per pass).
//
// dst[m][n] = sum_b f32(d_w[n][b]) * f32(d_a[m][b]) * S_b[m][n],
// S_b = sum_j (q4 - 8) * q8 (int32).
//
// At decode shapes the product is bound by reading the weights (arXiv
// 2407.07304, section 2.2: the next-token phase is GEMV-like and memory
// bound; DeepSpeed-Inference notes, III.A: small batches are limited by the
// bandwidth of reading the weights, and by the fixed cost of every kernel
// launch).  smallbard "Generer a plusieurs" shows a narrow kernel that
// re-reads each weight per pack of 8 rows; here each weight byte is read
// exactly once for all M rows of the pass:
//
//   * a wave owns R consecutive weight rows; lane l walks the row's 36-byte
//     block pairs l, l+64, ... (a pair is 4-byte aligned when K/32 is even,
//     so it loads as dwordx4 + dwordx4 + dword), and the next pair's loads
//     are issued before the current pair is computed;
//   * nibbles are unpacked in registers; each block costs 8 v_dot4 per
//     activation row, seeded with -8 * sum(q8) so that the unsigned nibbles
//     give the signed block dot;
//   * the fp32 accumulators are reduced over the 64 lanes with DPP row
//     operations in a fixed order (DeepSpeed-Inference notes, III.C: reduce
//     each output's partials in registers within one wave);
//   * the activations of the workgroup's K slice are staged in LDS; for
//     small M the INIT stage is fused in: every workgroup quantizes the src1
//     rows (and K range) it needs into LDS with the same Q8_0 routine as the
//     stand-alone quantizer, so one launch does the whole product;
//   * when the grid would not fill the device, K is split across workgroups
//     and a second kernel adds the partial sums in a fixed order (smallbard,
//     "La courbe, une premiere fois": cut the common dimension into slices
//     and add the partial sums afterwards).
#include "device.h"
#include "kernels.h"
#include "../../include/mm.h"

namespace qsg {

namespace {

// Where a kernel reads the Q8_0 activation codes, scales and -8*sum(q).
struct ActView {
  const int8_t* q;      // codes of row 0, block boff
  const float* d;       // scale of row 0, block boff
  const int32_t* bias;  // -8 * sum(q) of row 0, block boff
  int64_t qpitch;       // bytes between rows of codes
  int64_t dpitch;       // entries between rows of scales / bias
  int boff;             // first block held
  int rows;             // valid rows (>= 1)
  bool swz;             // codes in LDS, chunks swizzled (act_chunk); rows of
                        // whole block pairs only
};

// Byte offset of 16-byte code chunk h (0, 1) of block bl within a row of
// activation codes in LDS.  A lane reads its K unit (two blocks, 64 bytes)
// at a 64-byte stride from its neighbours; with the chunks in place every
// 16-byte read of a wave would land four lanes on the same banks.  The
// chunk's slot within its 64-byte unit is therefore XORed with bits 1-4 of
// the unit index, which puts any 8 or 16 consecutive units' reads of one
// chunk on distinct banks (32- or 64-bank LDS).  Writers and readers both go
// through this function; code in global memory is not swizzled, and neither
// are rows of an odd number of blocks (a last, unpaired block would be moved
// into the next row's first).
__device__ __forceinline__ int act_chunk(int bl, int h, bool swz) {
  const int x = swz ? (((bl >> 2) ^ (bl >> 4)) & 3) << 4 : 0;
  return (bl * 32 + 16 * h) ^ x;
}

// kMask: lanes with !valid hold a clamped (valid) unit whose contribution
// is dropped; they still compute, so every loaded register is consumed on
// every path.
template <int MT, int R, bool kDump, bool kMask>
__device__ __forceinline__ void block_mac(const uint32_t (&q)[R][4], const float (&dw)[R], int b,
                                          bool valid, const ActView& av, float (&acc)[R][MT],
                                          int nw, int m0, int nb, const Q4Args& a) {
  uint32_t lo[R][4], hi[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[r][j] = q[r][j] & 0x0F0F0F0Fu;          // elements 4j .. 4j+3
      hi[r][j] = (q[r][j] >> 4) & 0x0F0F0F0Fu;   // elements 16+4j .. 16+4j+3
    }
  }
  const int bl = b - av.boff;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int mm = m < av.rows ? m : av.rows - 1;
    const int8_t* ar = av.q + mm * av.qpitch;
    const v4i a0 = *reinterpret_cast<const v4i*>(ar + act_chunk(bl, 0, av.swz));
    const v4i a1 = *reinterpret_cast<const v4i*>(ar + act_chunk(bl, 1, av.swz));
    const float da = av.d[mm * av.dpitch + bl];
    const int bias = av.bias[mm * av.dpitch + bl];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int s = bias;
      s = __builtin_amdgcn_sdot4((int)lo[r][0], a0.x, s, false);
      s = __builtin_amdgcn_sdot4((int)lo[r][1], a0.y, s, false);
      s = __builtin_amdgcn_sdot4((int)lo[r][2], a0.z, s, false);
      s = __builtin_amdgcn_sdot4((int)lo[r][3], a0.w, s, false);
      s = __builtin_amdgcn_sdot4((int)hi[r][0], a1.x, s, false);
      s = __builtin_amdgcn_sdot4((int)hi[r][1], a1.y, s, false);
      s = __builtin_amdgcn_sdot4((int)hi[r][2], a1.z, s, false);
      s = __builtin_amdgcn_sdot4((int)hi[r][3], a1.w, s, false);
      const float sc = dw[r] * da;
      // s * 0 is a zero, so a dropped lane leaves its sum unchanged
      acc[r][m] = fmaf((float)s, kMask ? (valid ? sc : 0.0f) : sc, acc[r][m]);
      if (kDump) {
        const int n = nw + r;
        if ((!kMask || valid) && m0 + m < a.M && n >= a.n0 && n < a.n1)
          a.dots[((int64_t)(m0 + m) * (a.n1 - a.n0) + (n - a.n0)) * nb + b] = s;
      }
    }
  }
}

// Loads one K unit (a 36-byte block pair, or one 18-byte block as 16-bit
// words) of each of the wave's rows.
template <int R, bool kPairs>
__device__ __forceinline__ void load_unit(uint32_t (&wv)[R][9], const uint8_t* const (&rowp)[R],
                                          int64_t u) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    // weights live in global memory: say so, so the loads are global_load
    // (a flat load would also count against the LDS wait counter)
    if (kPairs) {
      const __attribute__((address_space(1))) uint32_t* p =
          (const __attribute__((address_space(1))) uint32_t*)(rowp[r] + 36 * u);
#pragma unroll
      for (int i = 0; i < 9; ++i) wv[r][i] = p[i];
    } else {
      const __attribute__((address_space(1))) uint16_t* p =
          (const __attribute__((address_space(1))) uint16_t*)(rowp[r] + 18 * u);
#pragma unroll
      for (int i = 0; i < 9; ++i) wv[r][i] = p[i];
    }
  }
}

template <int MT, int R, bool kPairs, bool kDump, bool kMask>
__device__ __forceinline__ void unit_mac(const uint32_t (&wv)[R][9], int64_t u, bool valid,
                                         const ActView& av, float (&acc)[R][MT], int nw, int m0,
                                         int nb, const Q4Args& a) {
  if (kPairs) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t q[R][4];
      float dw[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (half == 0) {
          dw[r] = f16_bits_to_f32(wv[r][0]);
#pragma unroll
          for (int j = 0; j < 4; ++j) q[r][j] = __builtin_amdgcn_alignbit(wv[r][j + 1], wv[r][j], 16);
        } else {
          dw[r] = f16_bits_to_f32(wv[r][4] >> 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) q[r][j] = wv[r][5 + j];
        }
      }
      block_mac<MT, R, kDump, kMask>(q, dw, (int)(2 * u + half), valid, av, acc, nw, m0, nb, a);
    }
  } else {
    uint32_t q[R][4];
    float dw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      dw[r] = f16_bits_to_f32(wv[r][0]);
#pragma unroll
      for (int j = 0; j < 4; ++j) q[r][j] = wv[r][1 + 2 * j] | (wv[r][2 + 2 * j] << 16);
    }
    block_mac<MT, R, kDump, kMask>(q, dw, (int)u, valid, av, acc, nw, m0, nb, a);
  }
}

// Q8_0 weights (the fused kernel only): a K unit is a pair of 34-byte
// blocks, 68 bytes, 4-byte aligned when K/32 is even; block 0's scale is
// bytes 0-1 and its codes start at byte 2 (dwords shifted by 16 bits),
// block 1's scale is the high half of dword 8 and its codes are dwords 9-16.
// The codes are signed bytes, so each block dot is 8 v_dot4 from zero.
template <int R>
__device__ __forceinline__ void load_unit8(uint32_t (&wv)[R][17], const uint8_t* const (&rowp)[R],
                                           int64_t u) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const __attribute__((address_space(1))) uint32_t* p =
        (const __attribute__((address_space(1))) uint32_t*)(rowp[r] + 68 * u);
#pragma unroll
    for (int i = 0; i < 17; ++i) wv[r][i] = p[i];
  }
}

template <int MT, int R>
__device__ __forceinline__ void unit_mac8(const uint32_t (&wv)[R][17], int64_t u,
                                          const ActView& av, float (&acc)[R][MT]) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint32_t q[R][8];
    float dw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      dw[r] = f16_bits_to_f32(half == 0 ? wv[r][0] : wv[r][8] >> 16);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        q[r][j] = half == 0 ? __builtin_amdgcn_alignbit(wv[r][j + 1], wv[r][j], 16) : wv[r][9 + j];
    }
    const int bl = (int)(2 * u + half) - av.boff;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int mm = m < av.rows ? m : av.rows - 1;
      const int8_t* ar = av.q + mm * av.qpitch;
      const v4i a0 = *reinterpret_cast<const v4i*>(ar + act_chunk(bl, 0, av.swz));
      const v4i a1 = *reinterpret_cast<const v4i*>(ar + act_chunk(bl, 1, av.swz));
      const float da = av.d[mm * av.dpitch + bl];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        int s = 0;
        s = __builtin_amdgcn_sdot4((int)q[r][0], a0.x, s, false);
        s = __builtin_amdgcn_sdot4((int)q[r][1], a0.y, s, false);
        s = __builtin_amdgcn_sdot4((int)q[r][2], a0.z, s, false);
        s = __builtin_amdgcn_sdot4((int)q[r][3], a0.w, s, false);
        s = __builtin_amdgcn_sdot4((int)q[r][4], a1.x, s, false);
        s = __builtin_amdgcn_sdot4((int)q[r][5], a1.y, s, false);
        s = __builtin_amdgcn_sdot4((int)q[r][6], a1.z, s, false);
        s = __builtin_amdgcn_sdot4((int)q[r][7], a1.w, s, false);
        acc[r][m] = fmaf((float)s, dw[r] * da, acc[r][m]);
      }
    }
  }
}

// Staging of the activation slice into LDS, in batches of kBatch rounds of
// NT threads.  load_*: issue the global loads of one batch (unconditional,
// on clamped addresses); store_*: consume them into LDS.
struct Slice {
  int total, kbmax, nbs, rows, m0, b0, K, nb;
};

// Splits a staging block index into (row m < MT, block bl < kbmax) without a
// division (MT is small).
template <int MT>
__device__ __forceinline__ void split_blk(int blk, int kbmax, int& m, int& bl) {
  m = 0;
#pragma unroll
  for (int j = 1; j < MT; ++j) m += blk >= j * kbmax ? 1 : 0;
  bl = blk - m * kbmax;
}

// Quantize staging: two lanes per block (items i = 2*block + half), each
// holding 16 values.
template <int NT, int kBatch, int MT>
__device__ __forceinline__ void quant_load(const Slice& sl, const float* __restrict__ x, int it0,
                                           int rounds, float (&v)[kBatch][16],
                                           bool (&ok)[kBatch]) {
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int i = (it0 + j) * NT + (int)threadIdx.x;
    const int blk = i >> 1, h = i & 1;
    int m, bl;
    split_blk<MT>(blk, sl.kbmax, m, bl);
    ok[j] = it0 + j < rounds && i < sl.total && bl < sl.nbs && m < sl.rows;
    const int64_t off = ok[j] ? (int64_t)(sl.m0 + m) * sl.K + (int64_t)(sl.b0 + bl) * 32 + 16 * h
                              : (int64_t)sl.m0 * sl.K + (int64_t)sl.b0 * 32 + 16 * h;
    const float4* p = reinterpret_cast<const float4*>(x + off);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = p[q];
      v[j][4 * q] = f.x; v[j][4 * q + 1] = f.y; v[j][4 * q + 2] = f.z; v[j][4 * q + 3] = f.w;
    }
  }
}

template <int NT, int kBatch, int MT, bool kSwz>
__device__ __forceinline__ void quant_store(const Slice& sl, int it0, int rounds,
                                            float (&v)[kBatch][16], const bool (&ok)[kBatch],
                                            int8_t* sq, float* sd, int32_t* sb) {
  // Every round of the batch is computed, also past the last one (on zeros,
  // nothing stored): a loaded register left unread on some path would make
  // the compiler wait for the loads in flight wherever it is next written.
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int i = (it0 + j) * NT + (int)threadIdx.x;
    const int blk = i >> 1, h = i & 1;
    int m, bl;
    split_blk<MT>(blk, sl.kbmax, m, bl);
    if (!ok[j]) {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[j][e] = 0.0f;
    }
    uint32_t packed[4], dbits;
    int sum;
    q8_0_pair(v[j], packed, dbits, sum);
    if (ok[j]) {
      *reinterpret_cast<uint4*>(sq + (int64_t)m * sl.kbmax * 32 + act_chunk(bl, h, kSwz)) =
          make_uint4(packed[0], packed[1], packed[2], packed[3]);
      if (h == 0) {
        sd[m * sl.kbmax + bl] = f16_bits_to_f32(dbits);
        sb[m * sl.kbmax + bl] = -8 * sum;
      }
    }
  }
}

// Q8_0 of one 32-value block held by a quad of adjacent lanes (lane q of
// the quad: values 8q .. 8q+7): the same operation sequence as q8_0_pair
// (amax over the block, d = amax / 127 correctly rounded, id = 1 / d, codes
// rounded half away from zero, their integer sum), so the bytes are the
// same; the maximum and the sum are exact whatever the grouping of lanes.
__device__ __forceinline__ void q8_0_quad(const float (&v)[8], uint32_t (&packed)[2],
                                          uint32_t& dbits, int& sum) {
#pragma clang fp contract(off)
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, dpp_f<0xB1>(amax));             // lane ^ 1
  amax = fmaxf(amax, dpp_f<0x4E>(amax));             // lane ^ 2
  const float d = amax / 127.0f;
  const float id = d != 0.0f ? 1.0f / d : 0.0f;
  int s = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) w |= (uint32_t)(round_half_away(v[4 * j + e] * id) & 0xff) << (8 * e);
    packed[j] = w;
    s = __builtin_amdgcn_sdot4((int)w, 0x01010101, s, false);
  }
  s += dpp_i<0xB1>(s);
  s += dpp_i<0x4E>(s);
  sum = s;
  dbits = f32_to_f16_bits(d);
}

// Quantize staging with four lanes per block (items i = 4 * block + q,
// each holding 8 values): twice the lanes of quant_load / quant_store at
// half the work each, for the fused kernel's one-round prologue.
template <int NT, int kBatch, int MT>
__device__ __forceinline__ void quad_load(const Slice& sl, const float* __restrict__ x, int it0,
                                          int rounds, float (&v)[kBatch][8], bool (&ok)[kBatch]) {
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int i = (it0 + j) * NT + (int)threadIdx.x;
    const int blk = i >> 2, q = i & 3;
    int m, bl;
    split_blk<MT>(blk, sl.kbmax, m, bl);
    ok[j] = it0 + j < rounds && i < sl.total && bl < sl.nbs && m < sl.rows;
    const int64_t off = ok[j] ? (int64_t)(sl.m0 + m) * sl.K + (int64_t)(sl.b0 + bl) * 32 + 8 * q
                              : (int64_t)sl.m0 * sl.K + (int64_t)sl.b0 * 32 + 8 * q;
    const float4* p = reinterpret_cast<const float4*>(x + off);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 f = p[h];
      v[j][4 * h] = f.x; v[j][4 * h + 1] = f.y; v[j][4 * h + 2] = f.z; v[j][4 * h + 3] = f.w;
    }
  }
}

template <int NT, int kBatch, int MT, bool kSwz>
__device__ __forceinline__ void quad_store(const Slice& sl, int it0, int rounds,
                                           float (&v)[kBatch][8], const bool (&ok)[kBatch],
                                           int8_t* sq, float* sd, int32_t* sb) {
  // every round computed, also past the last one (see quant_store)
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int i = (it0 + j) * NT + (int)threadIdx.x;
    const int blk = i >> 2, q = i & 3;
    int m, bl;
    split_blk<MT>(blk, sl.kbmax, m, bl);
    if (!ok[j]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = 0.0f;
    }
    uint32_t packed[2], dbits;
    int sum;
    q8_0_quad(v[j], packed, dbits, sum);
    if (ok[j]) {
      // values 8q .. 8q+7: bytes 8 (q & 1) .. of code chunk q >> 1
      *reinterpret_cast<uint2*>(sq + (int64_t)m * sl.kbmax * 32 + act_chunk(bl, q >> 1, kSwz) + 8 * (q & 1)) =
          make_uint2(packed[0], packed[1]);
      if (q == 0) {
        sd[m * sl.kbmax + bl] = f16_bits_to_f32(dbits);
        sb[m * sl.kbmax + bl] = -8 * sum;
      }
    }
  }
}

template <int NT, int kBatch, int MT>
__device__ __forceinline__ void copy_load(const Slice& sl, const Q4Args& a, int it0, int rounds,
                                          v4i (&c)[kBatch], float (&d)[kBatch], int (&bi)[kBatch],
                                          bool (&ok)[kBatch]) {
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int i = (it0 + j) * NT + (int)threadIdx.x;
    int m, bl;
    split_blk<MT>(i >> 1, sl.kbmax, m, bl);
    const int cc = 2 * bl + (i & 1);
    ok[j] = it0 + j < rounds && i < sl.total && bl < sl.nbs && m < sl.rows;
    const int64_t row = ok[j] ? sl.m0 + m : sl.m0;
    const int64_t blk = ok[j] ? sl.b0 + bl : sl.b0;
    const int half = ok[j] ? (cc & 1) : 0;
    c[j] = *reinterpret_cast<const v4i*>(a.aq + row * sl.K + blk * 32 + half * 16);
    d[j] = a.ad[row * sl.nb + blk];
    bi[j] = a.ab[row * sl.nb + blk];
  }
}

template <int NT, int kBatch, int MT, bool kSwz>
__device__ __forceinline__ void copy_store(const Slice& sl, int it0, const v4i (&c)[kBatch],
                                           const float (&d)[kBatch], const int (&bi)[kBatch],
                                           const bool (&ok)[kBatch], int8_t* sq, float* sd,
                                           int32_t* sb) {
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int i = (it0 + j) * NT + (int)threadIdx.x;
    int m, bl;
    split_blk<MT>(i >> 1, sl.kbmax, m, bl);
    const int cc = 2 * bl + (i & 1);
    if (ok[j]) {
      *reinterpret_cast<v4i*>(sq + (int64_t)m * sl.kbmax * 32 + act_chunk(bl, cc & 1, kSwz)) = c[j];
      if ((cc & 1) == 0) {
        sd[m * sl.kbmax + bl] = d[j];
        sb[m * sl.kbmax + bl] = bi[j];
      }
    }
  }
}

// Where the activations come from.  kActGlobal: the Q8_0 wdata in global
// memory, read at use.  kActCopy: the wdata K-slice copied into LDS first.
// kActQuant: src1 (f32) quantized into LDS by the workgroup itself (INIT
// fused).  In both LDS forms the slice's loads are issued before the first
// weight loads: vmcnt retires in order, so consuming the activations never
// waits on weights still streaming in from HBM, and the barrier is LDS-only.
enum { kActGlobal = 0, kActCopy = 1, kActQuant = 2 };

__device__ __forceinline__ int mat_of(const Q4Mats& mats, int n) {
  int i = 0;
#pragma unroll
  for (int j = 1; j < kMaxGroup; ++j)
    if (j < mats.count && n >= mats.row0[j]) i = j;
  return i;
}

// Row pointers of the wave's R rows in row group g (rows past the end are
// clamped to the last row; their results are never stored).
template <int R, int RPG>
__device__ __forceinline__ void rows_of(const Q4Mats& mats, int g, int wave, int N, int64_t rb,
                                        const uint8_t* (&rp)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int n = g * RPG + wave * R + r;
    n = n < N ? n : N - 1;
    const int i = mat_of(mats, n);
    rp[r] = mats.w[i] + (int64_t)(n - mats.row0[i]) * rb;
  }
}

// kBatch: activation-slice loads in flight per thread (sized to the slice).
// Small-M variants with short K slices ask for 6 waves per SIMD (at most 80
// VGPRs; the second launch-bounds argument is waves per execution unit
// here), so that all workgroups are resident at once; longer K slices
// (larger kBatch) hold more staging registers.
//
// Work layout: rows are taken in groups of WAVES * R (R per wave); a grid of
// at most a few workgroups per CU walks the groups g = blockIdx.x,
// blockIdx.x + gridDim.x, ... after staging the activations once, so the
// activation slice is read (and, fused, quantized) once per workgroup rather
// than once per row group.  Each wave runs a flat sequence of (group, K unit)
// steps and loads the next step's weights before computing the current one.
template <int MT, int R, int WAVES, bool kPairs, bool kDump, int kAct, int kBatch>
__global__ __launch_bounds__(64 * WAVES, MT > 2 ? 1 : kAct == kActQuant ? (kBatch <= 1 ? 4 : 4) : (kBatch <= 4 ? 6 : 1))
void k_q4_narrow(Q4Args a, Q4Mats mats, const float* __restrict__ x, int64_t kchunk, int split) {
  constexpr int NT = 64 * WAVES;
  constexpr int RPG = WAVES * R;                     // rows per group
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  const int lane = threadIdx.x & 63;
  // uniform within the wave: row and matrix lookups run on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int M = a.M, N = a.N, K = a.K;
  const int nb = K / 32;
  const int64_t rb = (int64_t)nb * 18;
  const int m0 = blockIdx.y * MT;
  const int z = blockIdx.z;
  const int ngroups = (N + RPG - 1) / RPG;
  constexpr int kBPU = kPairs ? 2 : 1;               // blocks per K unit
  const int64_t units = kPairs ? nb / 2 : nb;
  const int64_t u0 = (int64_t)z * kchunk;
  const int64_t u1 = (u0 + kchunk < units) ? u0 + kchunk : units;
  const int SU = (int)((u1 - u0 + 63) / 64);         // steps per row group
  int g = blockIdx.x;
  if (g >= ngroups || SU <= 0) return;               // uniform over the workgroup
  const int kbmax = (int)(kchunk * kBPU);            // LDS capacity in blocks per row
  const int b0 = (int)(u0 * kBPU);
  const int nbs = (int)((u1 * kBPU < nb ? u1 * kBPU : nb) - b0);

  ActView av;
  av.rows = (M - m0 < MT) ? M - m0 : MT;
  int8_t* sq = smem;
  float* sd = reinterpret_cast<float*>(smem + (int64_t)MT * kbmax * 32);
  int32_t* sb = reinterpret_cast<int32_t*>(sd + MT * kbmax);

  const uint8_t* rp[R];
  rows_of<R, RPG>(mats, g, wave, N, rb, rp);
  uint32_t wv[R][9];
  // Loads below are unconditional, on clamped (always valid) addresses, with
  // the values masked afterwards: straight-line code lets the compiler wait
  // for exactly the loads a value needs instead of for every load in flight.
  const int64_t ufirst = u0 + lane < u1 ? u0 + lane : u0;
  Slice sl;
  sl.kbmax = kbmax; sl.nbs = nbs; sl.rows = av.rows; sl.m0 = m0; sl.b0 = b0; sl.K = K; sl.nb = nb;
  if (kAct == kActQuant) {
    sl.total = MT * kbmax * 2;                       // 2 lanes per block
    const int rounds = (sl.total + NT - 1) / NT;
    {
      float v[kBatch][16];
      bool ok[kBatch];
      quant_load<NT, kBatch, MT>(sl, x, 0, rounds, v, ok);
      load_unit<R, kPairs>(wv, rp, ufirst);          // after the slice's loads
      quant_store<NT, kBatch, MT, kPairs>(sl, 0, rounds, v, ok, sq, sd, sb);
    }
    for (int it0 = kBatch; it0 < rounds; it0 += kBatch) {
      float v[kBatch][16];
      bool ok[kBatch];
      quant_load<NT, kBatch, MT>(sl, x, it0, rounds, v, ok);
      quant_store<NT, kBatch, MT, kPairs>(sl, it0, rounds, v, ok, sq, sd, sb);
    }
    lds_barrier();
  } else if (kAct == kActCopy) {
    // 16-byte code chunks; the thread holding a block's first chunk also
    // stores its scale and bias.
    sl.total = MT * kbmax * 2;
    const int rounds = (sl.total + NT - 1) / NT;
    {
      v4i c[kBatch];
      float d[kBatch];
      int bi[kBatch];
      bool ok[kBatch];
      copy_load<NT, kBatch, MT>(sl, a, 0, rounds, c, d, bi, ok);
      load_unit<R, kPairs>(wv, rp, ufirst);          // after the slice's loads
      copy_store<NT, kBatch, MT, kPairs>(sl, 0, c, d, bi, ok, sq, sd, sb);
    }
    for (int it0 = kBatch; it0 < rounds; it0 += kBatch) {
      v4i c[kBatch];
      float d[kBatch];
      int bi[kBatch];
      bool ok[kBatch];
      copy_load<NT, kBatch, MT>(sl, a, it0, rounds, c, d, bi, ok);
      copy_store<NT, kBatch, MT, kPairs>(sl, it0, c, d, bi, ok, sq, sd, sb);
    }
    lds_barrier();
  } else {
    load_unit<R, kPairs>(wv, rp, ufirst);
  }

  if (kAct == kActGlobal) {
    av.q = a.aq + (int64_t)m0 * K;
    av.d = a.ad + (int64_t)m0 * nb;
    av.bias = a.ab + (int64_t)m0 * nb;
    av.qpitch = K; av.dpitch = nb; av.boff = 0; av.swz = false;
  } else {
    av.q = sq; av.d = sd; av.bias = sb;
    av.qpitch = (int64_t)kbmax * 32; av.dpitch = kbmax; av.boff = b0; av.swz = kPairs;
  }

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  // One step of the wave's (group, K unit) sequence: issue the loads of the
  // next step into `nxt`, then compute the current step from `cur`.  The
  // loop below alternates two register buffers, so a step's loads stay in
  // flight while the previous step is computed (no register copy waits for
  // them).  Returns false after the wave's last step.
  int i = 0;                                         // K step within the group
  auto step = [&](const uint32_t (&cur)[R][9], uint32_t (&nxt)[R][9]) -> bool {
    int in = i + 1, gn = g;
    if (in == SU) { in = 0; gn = g + (int)gridDim.x; }
    const bool more = gn < ngroups;
    const uint8_t* rpn[R];
    if (gn != g) {
      rows_of<R, RPG>(mats, more ? gn : g, wave, N, rb, rpn);
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) rpn[r] = rp[r];
    }
    // past the wave's last step this reloads a valid unit
    int64_t un = u0 + lane + 64 * (int64_t)in;
    un = un < u1 ? un : u0;
    load_unit<R, kPairs>(nxt, rpn, un);
    // keep the scheduler from hoisting the current step's first uses (which
    // wait for its loads) above the next step's loads
    __builtin_amdgcn_sched_barrier(0);

    // the current step's unit, clamped as its loads were
    const int64_t u = u0 + lane + 64 * (int64_t)i;
    const bool valid = u < u1;
    const int64_t uc = valid ? u : u0;
    const int nw = g * RPG + wave * R;
    if (u0 + 64 * (int64_t)(i + 1) <= u1)              // every lane valid (uniform)
      unit_mac<MT, R, kPairs, kDump, false>(cur, uc, true, av, acc, nw, m0, nb, a);
    else
      unit_mac<MT, R, kPairs, kDump, true>(cur, uc, valid, av, acc, nw, m0, nb, a);

    if (i == SU - 1) {
      // Reduce each accumulator over the wave; lane r*MT+m stores (m, row nw+r).
      float mine = 0.0f;
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float v = wave_sum_dpp(acc[r][m]);
          if (lane == r * MT + m) mine = v;
          acc[r][m] = 0.0f;
        }
      const int r = lane / MT, m = lane % MT;
      const int n = nw + r;
      if (split == 1) {
        // Output row of each of the R rows: the matrix lookups use the
        // wave-uniform row index (scalar loads of the kernel arguments), and
        // each lane then picks its own row's pointer.  A lane-indexed lookup
        // would read the argument block with vector loads, whose wait would
        // also wait for the weight loads already in flight.
        float* out = nullptr;
        int ldo = 0;
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          const int nr = nw + rr < N ? nw + rr : N - 1;
          const int mi = mat_of(mats, nr);
          float* pr = mats.dst[mi] + (nr - mats.row0[mi]);
          const int nir = mats.row0[mi + 1] - mats.row0[mi];
          if (r == rr) { out = pr; ldo = nir; }
        }
        if (lane < R * MT && m0 + m < M && n < N) out[(int64_t)(m0 + m) * ldo] = mine;
      } else if (lane < R * MT && m0 + m < M && n < N) {
        a.part[((int64_t)z * M + m0 + m) * N + n] = mine;
      }
    }
    if (!more && in == 0) return false;
    g = gn;
    i = in;
#pragma unroll
    for (int r = 0; r < R; ++r) rp[r] = rpn[r];
    return true;
  };
  uint32_t wv2[R][9];
  for (;;) {
    if (!step(wv, wv2)) break;
    if (!step(wv2, wv)) break;
  }
}

// Fused small-M kernel (MT <= 2 rows of src1, K/32 even, 4-byte aligned
// weights, no K split): the common decode case, kept as lean as possible.
// Each workgroup quantizes src1 into LDS once, then walks row groups
// g = blockIdx.x, blockIdx.x + G, ...; wave w of the group owns R rows
// rows RPG g + R w .. RPG g + R w + R - 1, and lane l the K units (block
// pairs) l, l + 64, ...  The steps (group, K unit range) of a wave form one
// flat sequence whose next step's weights are loaded before the current one
// is computed.
//
// Arguments: everything a wave needs before its first weight load (src1,
// up to three weight matrices with their first rows, N, K, M and the grid
// size G) comes first, in 14 dwords that the launch preloads into scalar
// registers, so no wave waits on a memory round trip for its kernel
// arguments before it can issue a load.  A row n belongs to matrix 0 below
// r1, to matrix 1 below r2 and to matrix 2 beyond (r1 = r2 = N for a single
// matrix).  Groups of more than three matrices (kMany) look their rows up
// in the descriptor instead; the outputs always come from it (their
// addresses are needed only at the end).
struct FusedOut {
  const uint8_t* w[kMaxGroup];
  float* dst[kMaxGroup];
  int row0[kMaxGroup + 1];
  int count;
};

// Matrix of row n in a group of more than three (descriptor lookup).
__device__ __forceinline__ int fused_mat(const FusedOut& fo, int n) {
  int i = 0;
#pragma unroll
  for (int j = 1; j < kMaxGroup; ++j)
    if (j < fo.count && n >= fo.row0[j]) i = j;
  return i;
}

// kQuad: src1 quantized with four lanes per block (quad_load / quad_store)
// when that takes one round of the workgroup's threads, else with two.
template <int MT, int NR, int R, int WAVES, bool kMany, bool kQ8, bool kQuad>
__global__ __launch_bounds__(64 * WAVES)
void k_q4_fused(const float* __restrict__ x, const uint8_t* w0, const uint8_t* w1,
                const uint8_t* w2, int N, int K, int r1, int r2, int M, int G, FusedOut fo) {
  constexpr int NT = 64 * WAVES, RPG = WAVES * R;
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nb = K / 32;
  const int units = nb / 2;
  const int64_t rb = (int64_t)nb * (kQ8 ? 34 : 18);
  constexpr int UW = kQ8 ? 17 : 9;                   // dwords per K unit (block pair)
  const int SU = (units + 63) / 64;                  // steps per row group
  const int m0 = blockIdx.y * MT;
  const int rows = M - m0 < MT ? M - m0 : MT;
  const int ngroups = (N + RPG - 1) / RPG;
  const int mygroups = (int)blockIdx.x < ngroups ? (ngroups - 1 - (int)blockIdx.x) / G + 1 : 0;
  const int S = mygroups * SU;
  if (S == 0) return;                                // uniform over the workgroup
  int8_t* sq = smem;
  float* sd = reinterpret_cast<float*>(smem + (int64_t)MT * nb * 32);
  int32_t* sb = reinterpret_cast<int32_t*>(sd + MT * nb);
  // output bases, read from the descriptor now (constant offsets) so that
  // their loads are long complete when the first result is stored
  float* const d0 = fo.dst[0];
  float* const d1 = fo.dst[1];
  float* const d2 = fo.dst[2];

  // weight row pointer of the wave's row r in group g (rows past N clamped)
  auto rowptr = [&](int g, int r) -> const uint8_t* {
    int n = g * RPG + wave * R + r;
    n = n < N ? n : N - 1;
    if (kMany) {
      const int i = fused_mat(fo, n);
      return fo.w[i] + (int64_t)(n - fo.row0[i]) * rb;
    }
    if (n < r1) return w0 + (int64_t)n * rb;
    if (n < r2) return w1 + (int64_t)(n - r1) * rb;
    return w2 + (int64_t)(n - r2) * rb;
  };

  // activation loads first (vmcnt retires in order), then the first weights
  Slice sl;
  sl.kbmax = nb; sl.nbs = nb; sl.rows = rows; sl.m0 = m0; sl.b0 = 0; sl.K = K; sl.nb = nb;
  constexpr int LPB = kQuad ? 4 : 2;                 // lanes per src1 block
  sl.total = MT * nb * LPB;
  const int rounds = (sl.total + NT - 1) / NT;
  float v[NR][32 / LPB];
  bool ok[NR];
  auto stage_load = [&](int it0) {
    if constexpr (kQuad) quad_load<NT, NR, MT>(sl, x, it0, rounds, v, ok);
    else quant_load<NT, NR, MT>(sl, x, it0, rounds, v, ok);
  };
  auto stage_store = [&](int it0) {
    if constexpr (kQuad) quad_store<NT, NR, MT, true>(sl, it0, rounds, v, ok, sq, sd, sb);
    else quant_store<NT, NR, MT, true>(sl, it0, rounds, v, ok, sq, sd, sb);
  };
  stage_load(0);
  int g = blockIdx.x, i = 0;                         // current step: group g, K step i
  uint32_t wv[R][UW];
  {
    const uint8_t* rp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rp[r] = rowptr(g, r);
    const int u = lane < units ? lane : 0;
    if constexpr (kQ8) load_unit8<R>(wv, rp, u);
    else load_unit<R, true>(wv, rp, u);
  }
  // the first weights are in flight before src1 is waited for
  __builtin_amdgcn_sched_barrier(0);
  stage_store(0);
  for (int it0 = NR; it0 < rounds; it0 += NR) {
    stage_load(it0);
    stage_store(it0);
  }
  if (!kMany) asm volatile("" ::"s"(d0), "s"(d1), "s"(d2));
  lds_barrier();

  ActView av;
  av.q = sq; av.d = sd; av.bias = sb;
  av.qpitch = (int64_t)nb * 32; av.dpitch = nb; av.boff = 0; av.rows = rows; av.swz = true;
  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  for (int s = 0; s < S; ++s) {
    // next step (the last step reloads itself: valid, and never computed)
    int in = i + 1, gn = g;
    if (in == SU) { in = 0; gn = g + G; }
    if (s + 1 == S) { in = i; gn = g; }
    uint32_t cur[R][UW];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < UW; ++j) cur[r][j] = wv[r][j];
    {
      const uint8_t* rp[R];
#pragma unroll
      for (int r = 0; r < R; ++r) rp[r] = rowptr(gn, r);
      int un = lane + 64 * in;
      un = un < units ? un : 0;
      if constexpr (kQ8) load_unit8<R>(wv, rp, un);
      else load_unit<R, true>(wv, rp, un);
    }
    const int u = lane + 64 * i;
    const int nw = g * RPG + wave * R;
    if (u < units) {
      if constexpr (kQ8) unit_mac8<MT, R>(cur, u, av, acc);
      else unit_mac<MT, R, true, false, false>(cur, u, true, av, acc, nw, m0, nb, Q4Args{});
    }
    if (i == SU - 1) {
      float mine = 0.0f;
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float t = wave_sum_dpp(acc[r][m]);
          if (lane == r * MT + m) mine = t;
          acc[r][m] = 0.0f;
        }
      // output pointers of the wave's rows (wave-uniform lookups)
      float* out[R];
      int ldo[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int nr = nw + r < N ? nw + r : N - 1;
        if (kMany) {
          const int mi = fused_mat(fo, nr);
          out[r] = fo.dst[mi] + (nr - fo.row0[mi]);
          ldo[r] = fo.row0[mi + 1] - fo.row0[mi];
        } else if (nr < r1) {
          out[r] = d0 + nr;
          ldo[r] = r1;
        } else if (nr < r2) {
          out[r] = d1 + (nr - r1);
          ldo[r] = r2 - r1;
        } else {
          out[r] = d2 + (nr - r2);
          ldo[r] = N - r2;
        }
      }
      const int r = lane / MT, m = lane % MT;
      float* o = out[0];
      int ld = ldo[0];
#pragma unroll
      for (int rr = 1; rr < R; ++rr)
        if (r == rr) { o = out[rr]; ld = ldo[rr]; }
      if (lane < R * MT && m < rows && nw + r < N) o[(int64_t)(m0 + m) * ld] = mine;
    }
    g = gn;
    i = in;
  }
}

template <int MT, int R, int WAVES, bool kPairs, bool kDump, int kBatch>
void launch_5(const dim3& grid, size_t lds, int act, const Q4Args& a, const Q4Mats& mats,
              const float* x, int64_t kchunk, int split, hipStream_t s) {
  const dim3 block(64 * WAVES);
  if constexpr (kBatch <= 2) {
    if (act == kActQuant) {
      hipLaunchKernelGGL((k_q4_narrow<MT, R, WAVES, kPairs, kDump, kActQuant, kBatch>), grid, block, lds, s, a, mats, x, kchunk, split);
      return;
    }
  }
  hipLaunchKernelGGL((k_q4_narrow<MT, R, WAVES, kPairs, kDump, kActCopy, kBatch>), grid, block, lds, s, a, mats, x, kchunk, split);
}

template <int MT, int R, int WAVES, bool kPairs, bool kDump>
void launch_4(const dim3& grid, size_t lds, int act, int rounds, const Q4Args& a,
              const Q4Mats& mats, const float* x, int64_t kchunk, int split, hipStream_t s) {
  if (act == kActGlobal) {
    hipLaunchKernelGGL((k_q4_narrow<MT, R, WAVES, kPairs, kDump, kActGlobal, 1>), grid, dim3(64 * WAVES), 0, s, a, mats, x, kchunk, split);
    return;
  }
  // quantize items hold 16 floats each: at most 2 in flight per thread
  if (rounds <= 1) launch_5<MT, R, WAVES, kPairs, kDump, 1>(grid, lds, act, a, mats, x, kchunk, split, s);
  else if (rounds <= 2 || act == kActQuant) launch_5<MT, R, WAVES, kPairs, kDump, 2>(grid, lds, act, a, mats, x, kchunk, split, s);
  else if (rounds <= 4) launch_5<MT, R, WAVES, kPairs, kDump, 4>(grid, lds, act, a, mats, x, kchunk, split, s);
  else launch_5<MT, R, WAVES, kPairs, kDump, 8>(grid, lds, act, a, mats, x, kchunk, split, s);
}

template <int MT, int R, int WAVES>
hipError_t launch_mt(const Plan& p, const Q4Args& a, const Q4Mats& mats, const float* x, bool pairs,
                     hipStream_t s) {
  const dim3 grid((unsigned)p.grid_n, (unsigned)p.tiles_m, (unsigned)p.split);
  const int bpu = pairs ? 2 : 1;
  const size_t lds = (size_t)MT * (size_t)(p.kchunk * bpu) * 40;
  const int act = x ? kActQuant : (lds <= (size_t)kNarrowMaxLds ? kActCopy : kActGlobal);
  // staging rounds per thread: 2 lane items per block (quantize or copy)
  const int64_t items = (int64_t)MT * p.kchunk * bpu * 2;
  const int rounds = (int)((items + 64 * WAVES - 1) / (64 * WAVES));
  const bool dump = a.dots != nullptr;
  if (pairs) {
    if (dump) launch_4<MT, R, WAVES, true, true>(grid, lds, act, rounds, a, mats, x, p.kchunk, p.split, s);
    else launch_4<MT, R, WAVES, true, false>(grid, lds, act, rounds, a, mats, x, p.kchunk, p.split, s);
  } else {
    if (dump) launch_4<MT, R, WAVES, false, true>(grid, lds, act, rounds, a, mats, x, p.kchunk, p.split, s);
    else launch_4<MT, R, WAVES, false, false>(grid, lds, act, rounds, a, mats, x, p.kchunk, p.split, s);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q4_narrow(const Plan& p, const Q4Args& a, const Q4Mats& mats, const float* x,
                            hipStream_t s) {
  const int nb = a.K / 32;
  bool aligned = true;
  for (int i = 0; i < mats.count; ++i) aligned = aligned && ((uintptr_t)mats.w[i] % 4 == 0);
  const bool pairs = (nb % 2 == 0) && aligned;
  // The plan counts K units as pairs exactly when K/32 is even; with a
  // 2-byte-aligned src0 the kernel walks single blocks instead, so the chunk
  // (in units) doubles and the split count is unchanged.
  Plan q = p;
  if (!pairs && nb % 2 == 0) q.kchunk = p.kchunk * 2;
  // Q8_0 weights have the fused kernel only (the plan and the validation
  // guarantee its conditions; a dump of block dots takes the wide kernel)
  if (p.type == MM_TYPE_Q8_0 && !(x && pairs && p.split == 1 && a.dots == nullptr && p.fuse))
    return hipErrorInvalidValue;
  if (x && pairs && p.split == 1 && a.dots == nullptr && p.fuse) {
    const dim3 grid((unsigned)p.fuse_grid, (unsigned)p.tiles_m, 1u);
    const size_t lds = (size_t)p.mt * nb * 40;
    const int nt = 64 * p.fuse_waves;
    // four lanes per src1 block when they fit one round of the threads
    // (K = 4096: q,k,v 7.5 -> 7.1 us, gate,up 10.6 -> 10.3; with two rounds,
    // as the down projection's 344 blocks would take, two lanes are faster)
    const bool quad = (int64_t)p.mt * nb * 4 <= nt;
    const int rounds = (int)(((int64_t)p.mt * nb * 2 + nt - 1) / nt);
    FusedOut fo;
    for (int i = 0; i < kMaxGroup; ++i) {
      fo.w[i] = i < mats.count ? mats.w[i] : nullptr;
      fo.dst[i] = i < mats.count ? mats.dst[i] : nullptr;
    }
    for (int i = 0; i <= kMaxGroup; ++i) fo.row0[i] = mats.row0[i < mats.count ? i : mats.count];
    fo.count = mats.count;
    const bool many = mats.count > 3;
    const uint8_t* w1 = mats.count > 1 ? mats.w[1] : mats.w[0];
    const uint8_t* w2 = mats.count > 2 ? mats.w[2] : w1;
    const int r1 = mats.count > 1 ? mats.row0[1] : a.N;
    const int r2 = mats.count > 2 ? mats.row0[2] : a.N;
    const int G = p.fuse_grid;
    const bool q8 = p.type == MM_TYPE_Q8_0;
#define QSG_FUSED_K(MT_, NR_, R_, W_, MANY_, QUAD_)                                                \
    do {                                                                                           \
      if (q8)                                                                                      \
        hipLaunchKernelGGL((k_q4_fused<MT_, NR_, R_, W_, MANY_, true, QUAD_>), grid, dim3(nt), lds, \
                           s, x, mats.w[0], w1, w2, a.N, a.K, r1, r2, a.M, G, fo);                 \
      else                                                                                         \
        hipLaunchKernelGGL((k_q4_fused<MT_, NR_, R_, W_, MANY_, false, QUAD_>), grid, dim3(nt), lds, \
                           s, x, mats.w[0], w1, w2, a.N, a.K, r1, r2, a.M, G, fo);                 \
    } while (0)
#define QSG_FUSED_GO(MT_, NR_, R_, W_, QUAD_)                                                      \
    do {                                                                                           \
      if (many) QSG_FUSED_K(MT_, NR_, R_, W_, true, QUAD_);                                        \
      else QSG_FUSED_K(MT_, NR_, R_, W_, false, QUAD_);                                            \
    } while (0)
#define QSG_FUSED(MT_, R_, W_)                                                                     \
    if (p.mt == MT_ && p.fuse_rpw == R_ && p.fuse_waves == W_) {                                   \
      if (quad) QSG_FUSED_GO(MT_, 1, R_, W_, true);                                                \
      else if (rounds <= 1) QSG_FUSED_GO(MT_, 1, R_, W_, false);                                   \
      else QSG_FUSED_GO(MT_, 2, R_, W_, false);                                                    \
      return hipGetLastError();                                                                    \
    }
    QSG_FUSED(1, 2, 8)
    QSG_FUSED(1, 1, 8)
    QSG_FUSED(1, 1, 16)
    QSG_FUSED(2, 2, 8)
    QSG_FUSED(2, 1, 16)
#undef QSG_FUSED
#undef QSG_FUSED_GO
#undef QSG_FUSED_K
    return hipErrorInvalidValue;
  }
  // rows per wave and waves per workgroup must match make_plan()
  if (p.mt == 1 && p.rpw == 1 && p.waves == 8) return launch_mt<1, 1, 8>(q, a, mats, x, pairs, s);
  if (p.mt == 1 && p.rpw == 2 && p.waves == 8) return launch_mt<1, 2, 8>(q, a, mats, x, pairs, s);
  if (p.mt == 2 && p.rpw == 2 && p.waves == 8) return launch_mt<2, 2, 8>(q, a, mats, x, pairs, s);
  if (p.mt == 4 && p.rpw == 4 && p.waves == 4) return launch_mt<4, 4, 4>(q, a, mats, x, pairs, s);
  if (p.mt == 8 && p.rpw == 4 && p.waves == 4) return launch_mt<8, 4, 4>(q, a, mats, x, pairs, s);
  return hipErrorInvalidValue;
}

}  // namespace qsg
