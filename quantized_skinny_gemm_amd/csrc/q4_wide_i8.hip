// Wide-M Q4_0 x Q8_0 product for gfx950 on int8 MFMA (every M past the skinny
// kernel, M > 32).
//
// Past the narrow kernel's threshold the product is a dense contraction (the
// first-token / prefill regime, arXiv 2407.07304 section 2.2), so it runs on
// v_mfma_i32_32x32x32_i8: K = 32 is exactly one Q4_0/Q8_0 block, hence one
// (d_w, d_a) pair per MFMA output and the int32 block dot S_b comes out of
// the matrix core unchanged.  The weights are dequantized to int8 codes in
// LDS, not to floats (llama.cpp PR 1632, "Parallel de-quantizing": turning
// the weights into floats ahead of the product can cost as much as the
// product itself at these M).
//
// Per workgroup: an output tile BM x BN (32 x 64, 64 x 64, 64 x 128 or
// 128 x 128, four waves); per stage, KB = 4 blocks (128 k):
//   * weight rows are loaded as 36-byte block pairs (4-byte aligned when K/32
//     is even), the nibbles unpacked to signed int8 (q - 8) and the scales to
//     fp32, both into LDS;
//   * the Q8_0 activation codes (wdata) and scales are copied into LDS;
//   * each wave runs WM x WN MFMAs per block and applies the fp32 scale
//     epilogue acc += f32(S_b) * (d_a * d_w), the scale products coming
//     from a second (fp16) MFMA as an outer product, off the vector ALU;
// and, when the tiles cannot fill the device, K is split across workgroups
// whose partial tiles a second kernel adds in fixed order (smallbard
// "Generer a plusieurs", "La courbe, une premiere fois"; DeepSpeed-Inference
// notes, III.C SBI-GeMM: a second kernel reduces across the input-dim tiles).
#include "device.h"
#include "kernels.h"
#include "../../include/mm.h"

namespace qsg {

namespace {

constexpr int KB = kWideI8KB;        // blocks per stage
constexpr int PITCH = KB * 32 + 8;   // bytes per LDS row of codes (pad against bank conflicts)

__device__ __forceinline__ uint32_t nib_lo_signed(uint32_t q) {
  // per byte: (q & 15) - 8 as int8: add 0x78 (no carry out of a byte), flip bit 7
  return ((q & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
}
__device__ __forceinline__ uint32_t nib_hi_signed(uint32_t q) {
  return (((q >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
}

// Writes one decoded block (binary16 scale bits + 32 signed codes) into LDS.
__device__ __forceinline__ void put_block(int8_t* sB, uint16_t* sBd, int bn, int r, int bb,
                                          uint32_t d, const uint32_t (&q)[4]) {
  uint2* p = reinterpret_cast<uint2*>(sB + r * PITCH + bb * 32);
  p[0] = make_uint2(nib_lo_signed(q[0]), nib_lo_signed(q[1]));   // elements 0..7
  p[1] = make_uint2(nib_lo_signed(q[2]), nib_lo_signed(q[3]));   // elements 8..15
  p[2] = make_uint2(nib_hi_signed(q[0]), nib_hi_signed(q[1]));   // elements 16..23
  p[3] = make_uint2(nib_hi_signed(q[2]), nib_hi_signed(q[3]));   // elements 24..31
  sBd[bb * bn + r] = (uint16_t)d;
}

// Writes one Q8_0 block (binary16 scale bits + its 32 int8 codes as stored).
__device__ __forceinline__ void put_block8(int8_t* sB, uint16_t* sBd, int bn, int r, int bb,
                                           uint32_t d, const uint32_t (&q)[8]) {
  uint2* p = reinterpret_cast<uint2*>(sB + r * PITCH + bb * 32);
#pragma unroll
  for (int j = 0; j < 4; ++j) p[j] = make_uint2(q[2 * j], q[2 * j + 1]);
  sBd[bb * bn + r] = (uint16_t)d;
}

__device__ __forceinline__ v4i lds_operand(const int8_t* row, int bb, int h) {
  // lane half h supplies elements 8h..8h+7 and 16+8h..16+8h+7 of the block;
  // the A and B operands use the same assignment, so the MFMA's k-sum runs
  // over all 32 elements of the block.
  const uint2 x = *reinterpret_cast<const uint2*>(row + bb * 32 + 8 * h);
  const uint2 y = *reinterpret_cast<const uint2*>(row + bb * 32 + 16 + 8 * h);
  v4i v;
  v.x = (int)x.x; v.y = (int)x.y; v.z = (int)y.x; v.w = (int)y.y;
  return v;
}

// Operand of the 32 x 32 x 8 fp16 MFMA that forms the outer product of two
// scale vectors: element k = 0 of lane l < 32 is the scale of row (or
// column) l, every other element zero, so the MFMA's result is
// d_a[row] * d_w[col] in the layout of the int32 block dots.  The scales are
// staged as their binary16 bits; their product is exact in fp32.  (K = 8
// takes two registers per operand where K = 16 takes four, at the same
// issue cost: fewer zero registers to refill per block.)
__device__ __forceinline__ v4h scale_operand(uint32_t bits, int h) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i v = {h == 0 ? (int)bits : 0, 0};
  return __builtin_bit_cast(v4h, v);
}

// kRep: the weights are in the repacked layout (repack.hip): a stage of
// KB = 4 blocks is half a phase of each 16-row tile, 1 KB of codes (each
// lane piece: code bytes 4 g .. 4 g + 3 of one row for the 4 blocks) and the
// rows' scales, staged with one 16-byte load per piece.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool kPairs, bool kDump, bool kRep = false,
          bool kQ8 = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void k_q4_wide(Q4Args a, int tiles_m,
                                                                   int tiles_n, int kchunk,
                                                                   int split) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int WM = WTM / 32, WN = WTN / 32;
  static_assert(WM >= 1 && WN >= 1, "wave tile must be a multiple of 32x32");
  __shared__ __attribute__((aligned(16))) int8_t sA[BM * PITCH];
  __shared__ __attribute__((aligned(16))) int8_t sB[BN * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sAd[KB * BM];
  __shared__ __attribute__((aligned(16))) uint16_t sBd[KB * BN];

  const int M = a.M, N = a.N, K = a.K;
  const int nb = K / 32;
  const int64_t rb = (int64_t)nb * (kQ8 ? 34 : 18);
  const int tiles = tiles_m * tiles_n;
  const int t = xcd_remap(blockIdx.x, tiles * split);
  const int z = t / tiles;
  const int tt = t % tiles;
  const int tm = tt % tiles_m, tn = tt / tiles_m;     // m fastest: same weight tile adjacent
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb0 = z * kchunk;
  const int kb1 = (kb0 + kchunk < nb) ? kb0 + kchunk : nb;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int h = lane >> 5, l32 = lane & 31;

  float acc[WM][WN][16];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Register prefetch: the next stage's global loads are issued before the
  // current stage is computed.  Loads are unconditional, with addresses
  // clamped into the matrices; what lies outside the tile or the K range is
  // masked when the registers are written to LDS (codes 8 and zero scales for
  // weights, zero codes and scales for activations).
  static_assert(!kRep || (KB == 4 && BN % 16 == 0), "repacked stages are half a phase of whole tiles");
  constexpr int WI = kRep ? (BN * 4 + NT - 1) / NT
                   : kPairs ? (BN * (KB / 2) + NT - 1) / NT : (BN * KB + NT - 1) / NT;
  constexpr int AI = (BM * KB * 2 + NT - 1) / NT;
  constexpr int SI = (BM * KB + NT - 1) / NT;
  uint32_t wreg[WI][kQ8 ? 17 : kRep ? 6 : 9];
  const int rtiles = (N + 15) / 16, rphases = (nb + 7) / 8;
  v4i areg[AI];
  float sreg[SI];
  auto load_stage = [&](int kb) {
#pragma unroll
    for (int u = 0; u < WI; ++u) {
      const int i = tid + u * NT;
      if (kRep) {
        // piece (tile tq, lane l) of this half phase, and lane l's row scales
        const int ii = i < BN * 4 ? i : 0;
        const int tq = ii >> 6, l = ii & 63;
        int tile = n0 / 16 + tq;
        tile = tile < rtiles ? tile : rtiles - 1;
        const __attribute__((address_space(1))) uint8_t* c =
            (const __attribute__((address_space(1))) uint8_t*)(a.w + ((int64_t)tile * rphases + kb / 8) * kQ4RChunk);
        const v4i q = *(const __attribute__((address_space(1))) v4i*)(c + ((kb / 4) & 1) * 1024 + 16 * l);
        typedef int v2i __attribute__((ext_vector_type(2)));
        const v2i d = *(const __attribute__((address_space(1))) v2i*)(c + 2048 + 16 * (l & 15) + ((kb / 4) & 1) * 8);
        wreg[u][0] = (uint32_t)q.x; wreg[u][1] = (uint32_t)q.y;
        wreg[u][2] = (uint32_t)q.z; wreg[u][3] = (uint32_t)q.w;
        wreg[u][4] = (uint32_t)d.x; wreg[u][5] = (uint32_t)d.y;
      } else if (kPairs) {
        // a block pair: 36 bytes (Q4_0) or 68 (Q8_0), 4-byte aligned
        constexpr int UW = kQ8 ? 17 : 9;
        const int r = (i / (KB / 2)) % BN, pp = i % (KB / 2);
        const int n = n0 + r < N ? n0 + r : N - 1;
        const int b = kb + 2 * pp < kb1 ? kb + 2 * pp : kb0;
        const __attribute__((address_space(1))) uint32_t* p =
            (const __attribute__((address_space(1))) uint32_t*)(a.w + (int64_t)n * rb + (int64_t)b * (kQ8 ? 34 : 18));
#pragma unroll
        for (int j = 0; j < UW; ++j) wreg[u][j] = p[j];
      } else {
        // one block as 16-bit words: 18 bytes (Q4_0) or 34 (Q8_0)
        constexpr int UH = kQ8 ? 17 : 9;
        const int r = (i / KB) % BN, bb = i % KB;
        const int n = n0 + r < N ? n0 + r : N - 1;
        const int b = kb + bb < kb1 ? kb + bb : kb0;
        const __attribute__((address_space(1))) uint16_t* p =
            (const __attribute__((address_space(1))) uint16_t*)(a.w + (int64_t)n * rb + (int64_t)b * (kQ8 ? 34 : 18));
#pragma unroll
        for (int j = 0; j < UH; ++j) wreg[u][j] = p[j];
      }
    }
#pragma unroll
    for (int u = 0; u < AI; ++u) {
      const int i = tid + u * NT;
      const int r = (i / (KB * 2)) % BM, c = i % (KB * 2);
      const int m = m0 + r < M ? m0 + r : M - 1;
      // codes of block kb + c/2, half c%2; out of range: block kb0 (valid)
      const int64_t off = kb + c / 2 < kb1 ? (int64_t)kb * 32 + c * 16 : (int64_t)kb0 * 32 + (c & 1) * 16;
      areg[u] = *(const __attribute__((address_space(1))) v4i*)(a.aq + (int64_t)m * K + off);
    }
#pragma unroll
    for (int u = 0; u < SI; ++u) {
      const int i = tid + u * NT;
      const int r = i % BM, bb = (i / BM) % KB;
      const int m = m0 + r < M ? m0 + r : M - 1;
      const int b = kb + bb < kb1 ? kb + bb : kb0;
      sreg[u] = *(const __attribute__((address_space(1))) float*)(a.ad + (int64_t)m * nb + b);
    }
  };
  auto store_stage = [&](int kb) {
#pragma unroll
    for (int u = 0; u < WI; ++u) {
      const int i = tid + u * NT;
      if (kRep) {
        if (i >= BN * 4) continue;
        const int tq = i >> 6, l = i & 63;
        const int r = 16 * tq + (l & 15), g = l >> 4;
        const bool okr = n0 + r < N;
        // codes: finite for every row and block (padding is q = 8); a
        // block outside the tile or the K range gets a zero scale
#pragma unroll
        for (int bb = 0; bb < KB; ++bb) {
          *reinterpret_cast<uint32_t*>(sB + r * PITCH + bb * 32 + 4 * g) = nib_lo_signed(wreg[u][bb]);
          *reinterpret_cast<uint32_t*>(sB + r * PITCH + bb * 32 + 16 + 4 * g) = nib_hi_signed(wreg[u][bb]);
        }
        if (g == 0) {
#pragma unroll
          for (int bb = 0; bb < KB; ++bb) {
            const uint32_t dw = wreg[u][4 + (bb >> 1)];
            sBd[bb * BN + r] = (okr && kb + bb < kb1) ? (uint16_t)((bb & 1) ? dw >> 16 : dw) : (uint16_t)0;
          }
        }
      } else if (kPairs && kQ8) {
        // Q8_0 pair: block 0 = bytes 0-33 (scale, then codes from byte 2:
        // dwords shifted by 16 bits), block 1 = bytes 34-67 (scale in the high
        // half of dword 8, codes dword aligned from dword 9); codes are the
        // int8 operands as stored (0 outside the tile or the K range)
        if (i >= BN * (KB / 2)) continue;
        const int r = i / (KB / 2), pp = i % (KB / 2);
        const int b = kb + 2 * pp;
        const bool ok0 = n0 + r < N && b < kb1, ok1 = ok0 && b + 1 < kb1;
        uint32_t q0[8], q1[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          q0[j] = ok0 ? __builtin_amdgcn_alignbit(wreg[u][j + 1], wreg[u][j], 16) : 0u;
          q1[j] = ok1 ? wreg[u][9 + j] : 0u;
        }
        put_block8(sB, sBd, BN, r, 2 * pp, ok0 ? wreg[u][0] & 0xFFFFu : 0u, q0);
        put_block8(sB, sBd, BN, r, 2 * pp + 1, ok1 ? wreg[u][8] >> 16 : 0u, q1);
      } else if (kQ8) {
        if (i >= BN * KB) continue;
        const int r = i / KB, bb = i % KB;
        const bool ok = n0 + r < N && kb + bb < kb1;
        uint32_t q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = ok ? (wreg[u][1 + 2 * j] | (wreg[u][2 + 2 * j] << 16)) : 0u;
        put_block8(sB, sBd, BN, r, bb, ok ? wreg[u][0] : 0u, q);
      } else if (kPairs) {
        if (i >= BN * (KB / 2)) continue;
        const int r = i / (KB / 2), pp = i % (KB / 2);
        const int b = kb + 2 * pp;
        const bool ok0 = n0 + r < N && b < kb1, ok1 = ok0 && b + 1 < kb1;
        uint32_t q0[4], q1[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          q0[j] = ok0 ? __builtin_amdgcn_alignbit(wreg[u][j + 1], wreg[u][j], 16) : 0x88888888u;
          q1[j] = ok1 ? wreg[u][5 + j] : 0x88888888u;
        }
        const uint32_t d0 = ok0 ? wreg[u][0] & 0xFFFFu : 0u;
        const uint32_t d1 = ok1 ? wreg[u][4] >> 16 : 0u;
        put_block(sB, sBd, BN, r, 2 * pp, d0, q0);
        put_block(sB, sBd, BN, r, 2 * pp + 1, d1, q1);
      } else {
        if (i >= BN * KB) continue;
        const int r = i / KB, bb = i % KB;
        const bool ok = n0 + r < N && kb + bb < kb1;
        uint32_t q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) q[j] = ok ? (wreg[u][1 + 2 * j] | (wreg[u][2 + 2 * j] << 16)) : 0x88888888u;
        put_block(sB, sBd, BN, r, bb, ok ? wreg[u][0] & 0xFFFFu : 0u, q);
      }
    }
#pragma unroll
    for (int u = 0; u < AI; ++u) {
      const int i = tid + u * NT;
      if (i >= BM * KB * 2) continue;
      const int r = i / (KB * 2), c = i % (KB * 2);
      const bool ok = m0 + r < M && kb + c / 2 < kb1;
      uint2* p = reinterpret_cast<uint2*>(sA + r * PITCH + c * 16);
      p[0] = make_uint2(ok ? (uint32_t)areg[u].x : 0u, ok ? (uint32_t)areg[u].y : 0u);
      p[1] = make_uint2(ok ? (uint32_t)areg[u].z : 0u, ok ? (uint32_t)areg[u].w : 0u);
    }
#pragma unroll
    for (int u = 0; u < SI; ++u) {
      const int i = tid + u * NT;
      if (i >= BM * KB) continue;
      const int r = i % BM, bb = i / BM;
      // the wdata keeps d_a widened to fp32: back to its binary16 bits (exact)
      sAd[bb * BM + r] = (m0 + r < M && kb + bb < kb1) ? (uint16_t)f32_to_f16_bits(sreg[u]) : (uint16_t)0;
    }
  };

  load_stage(kb0);
  for (int kb = kb0; kb < kb1; kb += KB) {
    __syncthreads();                                // the last stage's MFMAs are done
    store_stage(kb);
    __syncthreads();
    if (kb + KB < kb1) load_stage(kb + KB);         // uniform over the workgroup
    // ---- MFMA over the stage's blocks
    const int nblk = (kb1 - kb < KB) ? kb1 - kb : KB;
    for (int bb = 0; bb < nblk; ++bb) {
      v4i A[WM], B[WN];
      v4h Ad[WM], Bd[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        A[i] = lds_operand(sA + (wm * WTM + 32 * i + l32) * PITCH, bb, h);
        Ad[i] = scale_operand(sAd[bb * BM + wm * WTM + 32 * i + l32], h);
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        B[j] = lds_operand(sB + (wn * WTN + 32 * j + l32) * PITCH, bb, h);
        Bd[j] = scale_operand(sBd[bb * BN + wn * WTN + 32 * j + l32], h);
      }
#pragma unroll
      for (int i = 0; i < WM; ++i) {
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const v16i zero = {};
          const v16i c = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[i], B[j], zero, 0, 0, 0);
          // d_a[row] * d_w[col] for every output of the tile, in the MFMA
          // result layout (output row of register r: 8*(r/4) + 4*h + (r%4))
          const v16f sc = __builtin_amdgcn_mfma_f32_32x32x8f16(Ad[i], Bd[j], v16f{}, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf((float)c[r], sc[r], acc[i][j][r]);
          if (kDump) {
            const int n = n0 + wn * WTN + 32 * j + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int m = m0 + wm * WTM + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
              if (m < M && n >= a.n0 && n < a.n1)
                a.dots[((int64_t)m * (a.n1 - a.n0) + (n - a.n0)) * nb + kb + bb] = c[r];
            }
          }
        }
      }
    }
  }

  // ---- store (or split-K partials)
  float* out = split == 1 ? a.dst : a.part + (int64_t)z * M * N;
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int n = n0 + wn * WTN + 32 * j + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * WTM + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
        if (m < M && n < N) out[(int64_t)m * N + n] = acc[i][j][r];
      }
    }
}

template <int BM, int BN, int WMS, int WNS>
hipError_t launch_cfg(const Plan& p, const Q4Args& a, bool pairs, hipStream_t s) {
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n * p.split));
  const dim3 block(64 * WMS * WNS);
  const int tm = (int)p.tiles_m, tn = (int)p.tiles_n, kc = (int)p.kchunk, sp = p.split;
  const bool dump = a.dots != nullptr;
  if (p.type == MM_TYPE_Q4_0R) {
    if (dump) hipLaunchKernelGGL((k_q4_wide<BM, BN, WMS, WNS, false, true, true>), grid, block, 0, s, a, tm, tn, kc, sp);
    else hipLaunchKernelGGL((k_q4_wide<BM, BN, WMS, WNS, false, false, true>), grid, block, 0, s, a, tm, tn, kc, sp);
  } else if (p.type == MM_TYPE_Q8_0) {
    if (pairs) {
      if (dump) hipLaunchKernelGGL((k_q4_wide<BM, BN, WMS, WNS, true, true, false, true>), grid, block, 0, s, a, tm, tn, kc, sp);
      else hipLaunchKernelGGL((k_q4_wide<BM, BN, WMS, WNS, true, false, false, true>), grid, block, 0, s, a, tm, tn, kc, sp);
    } else {
      if (dump) hipLaunchKernelGGL((k_q4_wide<BM, BN, WMS, WNS, false, true, false, true>), grid, block, 0, s, a, tm, tn, kc, sp);
      else hipLaunchKernelGGL((k_q4_wide<BM, BN, WMS, WNS, false, false, false, true>), grid, block, 0, s, a, tm, tn, kc, sp);
    }
  } else if (pairs) {
    if (dump) hipLaunchKernelGGL((k_q4_wide<BM, BN, WMS, WNS, true, true>), grid, block, 0, s, a, tm, tn, kc, sp);
    else hipLaunchKernelGGL((k_q4_wide<BM, BN, WMS, WNS, true, false>), grid, block, 0, s, a, tm, tn, kc, sp);
  } else {
    if (dump) hipLaunchKernelGGL((k_q4_wide<BM, BN, WMS, WNS, false, true>), grid, block, 0, s, a, tm, tn, kc, sp);
    else hipLaunchKernelGGL((k_q4_wide<BM, BN, WMS, WNS, false, false>), grid, block, 0, s, a, tm, tn, kc, sp);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q4_wide_i8(const Plan& p, const Q4Args& a, hipStream_t s) {
  const bool pairs = ((a.K / 32) % 2 == 0) && ((uintptr_t)a.w % 4 == 0);
  if (p.bm == 32 && p.bn == 64) return launch_cfg<32, 64, 1, 2>(p, a, pairs, s);
  if (p.bm == 64 && p.bn == 64) return launch_cfg<64, 64, 2, 2>(p, a, pairs, s);
  if (p.bm == 64 && p.bn == 128) return launch_cfg<64, 128, 2, 2>(p, a, pairs, s);
  if (p.bm == 128 && p.bn == 64) return launch_cfg<128, 64, 2, 2>(p, a, pairs, s);
  if (p.bm == 128 && p.bn == 128) return launch_cfg<128, 128, 2, 2>(p, a, pairs, s);
  return hipErrorInvalidValue;
}

}  // namespace qsg
