// Narrow-M Q4_0 x Q8_0 product for gfx950 (M <= 8 per pass).
//
// dst[m][n] = sum_b f32(d_w[n][b]) * f32(d_a[m][b]) * S_b[m][n],
// S_b = sum_j (q4 - 8) * q8 (int32).
//
// At decode shapes the product is bound by reading the weights (arXiv
// 2407.07304, section 2.2: the next-token phase is GEMV-like and memory
// bound; DeepSpeed-Inference notes, III.A: small batches are limited by the
// bandwidth of reading the weights).  smallbard "Generer a plusieurs" shows
// a narrow kernel that re-reads each weight per pack of 8 rows; here each
// weight byte is read exactly once for all M rows of the pass:
//
//   * a wave owns R consecutive weight rows; lane l walks the row's 36-byte
//     block pairs l, l+64, ... (a pair is 4-byte aligned when K/32 is even,
//     so it loads as dwordx4 + dwordx4 + dword);
//   * nibbles are unpacked in registers; each block costs 8 v_dot4 per
//     activation row, seeded with -8 * sum(q8) so that the unsigned nibbles
//     give the signed block dot;
//   * the fp32 accumulators are reduced over the 64 lanes with a fixed
//     butterfly (DeepSpeed-Inference notes, III.C: reduce each output's
//     partials in registers within one wave);
//   * when the grid would not fill the device, K is split across workgroups
//     and the last workgroup of each tile adds the partial sums in a fixed
//     order (smallbard, "La courbe, une premiere fois": cut the common
//     dimension into slices and add the partial sums afterwards).
#include "device.h"
#include "kernels.h"

namespace qsg {

namespace {

template <int MT, int R, bool kDump>
__device__ __forceinline__ void block_mac(const uint32_t (&q)[R][4], const float (&dw)[R],
                                          int b, int nb, int K, const int8_t* __restrict__ aq,
                                          const float* __restrict__ ad,
                                          const int32_t* __restrict__ ab, int m0, int M,
                                          float (&acc)[R][MT], int nw, int32_t* __restrict__ dots,
                                          int n0d, int n1d) {
  uint32_t lo[R][4], hi[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[r][j] = q[r][j] & 0x0F0F0F0Fu;          // elements 4j .. 4j+3
      hi[r][j] = (q[r][j] >> 4) & 0x0F0F0F0Fu;   // elements 16+4j .. 16+4j+3
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int mm = (m0 + m < M) ? m0 + m : M - 1;
    const v4i* ap = reinterpret_cast<const v4i*>(aq + (int64_t)mm * K + (int64_t)b * 32);
    const v4i a0 = ap[0], a1 = ap[1];
    const float da = ad[(int64_t)mm * nb + b];
    const int bias = ab[(int64_t)mm * nb + b];
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
      acc[r][m] = fmaf((float)s, dw[r] * da, acc[r][m]);
      if (kDump) {
        const int n = nw + r;
        if (m0 + m < M && n >= n0d && n < n1d)
          dots[((int64_t)(m0 + m) * (n1d - n0d) + (n - n0d)) * nb + b] = s;
      }
    }
  }
}

template <int MT, int R, bool kPairs, bool kDump>
__global__ __launch_bounds__(256) void k_q4_narrow(Q4Args a, int64_t kchunk, int split) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int M = a.M, N = a.N, K = a.K;
  const int nb = K / 32;
  const int64_t rb = (int64_t)nb * 18;
  const int m0 = blockIdx.y * MT;
  const int z = blockIdx.z;
  const int nw = (blockIdx.x * 4 + wave) * R;

  const uint8_t* rowp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = (nw + r < N) ? nw + r : N - 1;
    rowp[r] = a.w + (int64_t)n * rb;
  }
  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  const int64_t units = kPairs ? nb / 2 : nb;
  const int64_t u0 = (int64_t)z * kchunk;
  const int64_t u1 = (u0 + kchunk < units) ? u0 + kchunk : units;

  for (int64_t u = u0 + lane; u < u1; u += 64) {
    if (kPairs) {
      uint32_t wv[R][9];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(rowp[r] + 36 * u);
#pragma unroll
        for (int i = 0; i < 9; ++i) wv[r][i] = p[i];
      }
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
        block_mac<MT, R, kDump>(q, dw, (int)(2 * u + half), nb, K, a.aq, a.ad, a.ab, m0, M, acc,
                                nw, a.dots, a.n0, a.n1);
      }
    } else {
      uint32_t q[R][4];
      float dw[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(rowp[r] + 18 * u);
        uint32_t hw[9];
#pragma unroll
        for (int i = 0; i < 9; ++i) hw[i] = p[i];
        dw[r] = f16_bits_to_f32(hw[0]);
#pragma unroll
        for (int j = 0; j < 4; ++j) q[r][j] = hw[1 + 2 * j] | (hw[2 + 2 * j] << 16);
      }
      block_mac<MT, R, kDump>(q, dw, (int)u, nb, K, a.aq, a.ad, a.ab, m0, M, acc, nw, a.dots,
                              a.n0, a.n1);
    }
  }

  // Reduce each accumulator over the wave; lane r*MT+m stores output (m, nw+r).
  float mine = 0.0f;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float v = wave_sum(acc[r][m]);
      if (lane == r * MT + m) mine = v;
    }
  const int r = lane / MT, m = lane % MT;
  const bool owner = lane < R * MT && m0 + m < M && nw + r < N;
  if (split == 1) {
    if (owner) a.dst[(int64_t)(m0 + m) * N + nw + r] = mine;
    return;
  }
  if (owner) a.part[((int64_t)z * M + m0 + m) * N + nw + r] = mine;
  const int tile = blockIdx.y * gridDim.x + blockIdx.x;
  if (splitk_arrive(a.tick + tile, split))
    splitk_reduce_tile(a.part, a.dst, M, N, m0, MT, blockIdx.x * 4 * R, 4 * R, split);
}

template <int MT, int R>
hipError_t launch_mt(const Plan& p, const Q4Args& a, bool pairs, hipStream_t s) {
  const dim3 grid((unsigned)p.tiles_n, (unsigned)p.tiles_m, (unsigned)p.split);
  const dim3 block(256);
  const bool dump = a.dots != nullptr;
  if (pairs) {
    if (dump) hipLaunchKernelGGL((k_q4_narrow<MT, R, true, true>), grid, block, 0, s, a, p.kchunk, p.split);
    else hipLaunchKernelGGL((k_q4_narrow<MT, R, true, false>), grid, block, 0, s, a, p.kchunk, p.split);
  } else {
    if (dump) hipLaunchKernelGGL((k_q4_narrow<MT, R, false, true>), grid, block, 0, s, a, p.kchunk, p.split);
    else hipLaunchKernelGGL((k_q4_narrow<MT, R, false, false>), grid, block, 0, s, a, p.kchunk, p.split);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q4_narrow(const Plan& p, const Q4Args& a, hipStream_t s) {
  const int nb = a.K / 32;
  const bool pairs = (nb % 2 == 0) && ((uintptr_t)a.w % 4 == 0);
  // The plan counts K units as pairs exactly when K/32 is even; the generic
  // path (single blocks) is only taken with an odd K/32 or a 2-byte-aligned
  // src0, in which case the plan's units are blocks or the split is 1.
  Plan q = p;
  if (!pairs && nb % 2 == 0) {
    // units become blocks: rescale the chunk (split count unchanged)
    q.kchunk = p.kchunk * 2;
  }
  switch (p.mt) {
    case 1: return launch_mt<1, 2>(q, a, pairs, s);
    case 2: return launch_mt<2, 2>(q, a, pairs, s);
    case 4: return launch_mt<4, 4>(q, a, pairs, s);
    case 8: return launch_mt<8, 4>(q, a, pairs, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qsg
