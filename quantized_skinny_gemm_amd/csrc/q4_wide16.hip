// Wide-M Q4_0 x Q8_0 product for gfx950 on fp16 MFMA with exact block dots
// (an alternative to the int8 wide kernel, reached through the debug variant 4:
// the int8 kernel, which prefetches its stages, is faster at the measured M).
//
// Past the skinny kernels' range the product is a dense contraction (the
// first-token / prefill regime, arXiv 2407.07304 section 2.2).  Every block
// needs its own scale pair, so per output element and block the vector ALU
// must apply acc += S_b * (d_a * d_w): that epilogue, not the matrix core,
// bounds this kernel.  To keep it at two operations (multiply, fma) the
// block dot S_b comes out of the matrix core already in fp32, exactly:
//
//   * v_mfma_f32_32x32x16_f16, two per block (K = 32).  The A operand is the
//     Q8_0 codes as binary16 (written by INIT; integers |q| <= 127, exact).
//     The B operand is 1024 + q for each unsigned nibble q: the binary16 bit
//     pattern 0x6400 | q, built from the nibbles with a byte permute and one
//     and-or, never converted.  Products are integers below 2^17 and every
//     partial sum an integer below 2^24, so the fp32 accumulation is exact.
//   * The accumulator starts from -1032 * sum(q8) = 129 * (-8 * sum(q8)) of
//     the activation block, which removes both the 1024 offset and the -8 of
//     the Q4_0 code: the MFMA result is S_b = sum (q4 - 8) * q8 exactly.
//   * The weights are dequantized to nothing at all ahead of the product
//     (llama.cpp PR 1632, "Parallel de-quantizing": turning them into floats
//     first can cost as much as the product): the raw 18-byte blocks are
//     staged in LDS and each lane builds its operand in registers.
//
// Per workgroup: an output tile BM x BN (waves WM_ x WN_, each a multiple
// of 32 x 32).  K goes in stages of KBS blocks: the binary16 activation
// codes, the raw weight blocks and the activation scales and offsets of a
// stage are staged in LDS; the next stage's global loads are issued into
// registers before the current stage is computed, so they have a whole
// stage of matrix work to arrive.  K is split across workgroups when the
// tiles cannot fill the device; a second kernel adds the partials in a
// fixed order (smallbard "Generer a plusieurs", "La courbe, une premiere
// fois"; DeepSpeed-Inference notes, III.C SBI-GeMM).
#include "device.h"
#include "kernels.h"

namespace qsg {

namespace {

constexpr int KBS = kWide16KB;         // blocks per stage (even: whole block pairs)

template <int BM, int BN>
struct StageLds {
  static constexpr int kPA = KBS * 32 + 8;              // halves per activation row (padded)
  static constexpr int kPB = KBS * 18 + 4;              // bytes per weight row (odd dword count)
  static constexpr int kA = 0;                          // binary16 [BM][kPA]
  static constexpr int kB = BM * kPA * 2;               // raw weights [BN][kPB]
  static constexpr int kD = kB + BN * kPB;              // d_a f32 [KBS][BM]
  static constexpr int kC = kD + KBS * BM * 4;          // accumulator start f32 [KBS][BM]
  static constexpr int kBytes = kC + KBS * BM * 4;
};

// binary16 operands from 4 code bytes: 1024 + low nibble of bytes 0..3, as
// two dwords of two halves each.
__device__ __forceinline__ void nib_halves(uint32_t u, uint32_t& h01, uint32_t& h23) {
  h01 = (__builtin_amdgcn_perm(0u, u, 0x0c010c00u) & 0x000f000fu) | 0x64006400u;
  h23 = (__builtin_amdgcn_perm(0u, u, 0x0c030c02u) & 0x000f000fu) | 0x64006400u;
}

// Global -> register -> LDS copy of one stage.  Loads are unconditional
// (clamped addresses); what lies outside the tile or the K range is stored
// as zeros (zero codes, zero scale: no contribution).
template <int BM, int BN, int NT, bool kPairs>
struct Stager {
  using L = StageLds<BM, BN>;
  static constexpr int kAP = BM * KBS * 4;               // 16-byte activation pieces
  static constexpr int kAPT = (kAP + NT - 1) / NT;
  static constexpr int kBW = kPairs ? KBS * 9 / 2 : KBS * 9;   // pieces per weight row
  static constexpr int kBP = BN * kBW;
  static constexpr int kBPT = (kBP + NT - 1) / NT;
  static constexpr int kSP = KBS * BM;                   // scale items
  static constexpr int kSPT = (kSP + NT - 1) / NT;
  v4i av[kAPT];
  uint32_t bv[kBPT];
  float dv[kSPT];
  int32_t cv[kSPT];

  // stage starting at block kb, of which nlive blocks lie in the range
  __device__ __forceinline__ void load(const Q4Args& a, int64_t rb, int m0, int n0, int kb,
                                       int nlive) {
    const int t = threadIdx.x;
    const int M = a.M, N = a.N, K = a.K, nb = K / 32;
#pragma unroll
    for (int k = 0; k < kAPT; ++k) {
      int p = t + k * NT;
      p = p < kAP ? p : 0;
      const int r = p / (KBS * 4), c = p - r * (KBS * 4);   // 8 halves per piece
      const int m = m0 + r < M ? m0 + r : M - 1;
      const int blk = c >> 2;
      const int kk = (blk < nlive ? kb * 32 + 8 * c : kb * 32);
      const __attribute__((address_space(1))) v4i* src =
          (const __attribute__((address_space(1))) v4i*)(a.ah + (int64_t)m * K + kk);
      av[k] = *src;
    }
#pragma unroll
    for (int k = 0; k < kBPT; ++k) {
      int p = t + k * NT;
      p = p < kBP ? p : 0;
      const int r = p / kBW, c = p - r * kBW;
      const int n = n0 + r < N ? n0 + r : N - 1;
      if (kPairs) {
        const int cc = c < 9 * nlive / 2 ? c : 0;       // dwords past the range: reload a valid one
        const __attribute__((address_space(1))) uint32_t* src =
            (const __attribute__((address_space(1))) uint32_t*)(a.w + (int64_t)n * rb + (int64_t)kb * 18 + 4 * cc);
        bv[k] = *src;
      } else {
        const int cc = c < 9 * nlive ? c : 0;
        const __attribute__((address_space(1))) uint16_t* src =
            (const __attribute__((address_space(1))) uint16_t*)(a.w + (int64_t)n * rb + (int64_t)kb * 18 + 2 * cc);
        bv[k] = *src;
      }
    }
#pragma unroll
    for (int k = 0; k < kSPT; ++k) {
      int i = t + k * NT;
      i = i < kSP ? i : 0;
      const int r = i % BM, bl = i / BM;
      const int m = m0 + r < M ? m0 + r : 0;
      const int b = bl < nlive ? kb + bl : kb;
      const __attribute__((address_space(1))) float* pd =
          (const __attribute__((address_space(1))) float*)(a.ad + (int64_t)m * nb + b);
      const __attribute__((address_space(1))) int32_t* pb =
          (const __attribute__((address_space(1))) int32_t*)(a.ab + (int64_t)m * nb + b);
      dv[k] = *pd;
      cv[k] = *pb;
    }
  }

  __device__ __forceinline__ void store(uint8_t* buf, int m0, int M, int n0, int N,
                                        int nlive) const {
    const int t = threadIdx.x;
    _Float16* sa = reinterpret_cast<_Float16*>(buf + L::kA);
    uint8_t* sbw = buf + L::kB;
    float* sd = reinterpret_cast<float*>(buf + L::kD);
    float* sc = reinterpret_cast<float*>(buf + L::kC);
#pragma unroll
    for (int k = 0; k < kAPT; ++k) {
      const int p = t + k * NT;
      if (p < kAP) {
        const int r = p / (KBS * 4), c = p - r * (KBS * 4);
        const bool ok = m0 + r < M && (c >> 2) < nlive;
        const v4i v = ok ? av[k] : v4i{0, 0, 0, 0};
        *reinterpret_cast<v4i*>(sa + r * L::kPA + 8 * c) = v;
      }
    }
#pragma unroll
    for (int k = 0; k < kBPT; ++k) {
      const int p = t + k * NT;
      if (p < kBP) {
        const int r = p / kBW, c = p - r * kBW;
        if (kPairs) {
          const bool ok = n0 + r < N && c < 9 * nlive / 2;
          *reinterpret_cast<uint32_t*>(sbw + r * L::kPB + 4 * c) = ok ? bv[k] : 0u;
        } else {
          const bool ok = n0 + r < N && c < 9 * nlive;
          *reinterpret_cast<uint16_t*>(sbw + r * L::kPB + 2 * c) = ok ? (uint16_t)bv[k] : (uint16_t)0;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kSPT; ++k) {
      const int i = t + k * NT;
      if (i < kSP) {
        const int r = i % BM, bl = i / BM;
        const bool ok = m0 + r < M && bl < nlive;
        sd[bl * BM + r] = ok ? dv[k] : 0.0f;
        // 129 * (-8 * sum q8) = -1032 * sum q8: an integer below 2^23, exact
        sc[bl * BM + r] = ok ? (float)(129 * cv[k]) : 0.0f;
      }
    }
  }
};

// Stages past the range (pairs mode with an odd block count per split never
// happens: splits are whole pairs), a dropped block has zero codes and a zero
// scale in LDS, hence S_b = 0 and no contribution.
template <int BM, int BN, int WM_, int WN_, bool kPairs, bool kDump>
__global__ __launch_bounds__(64 * WM_ * WN_, 2)
void k_q4_wide(Q4Args a, int tiles_m, int tiles_n, int kchunk, int split) {
  constexpr int NT = 64 * WM_ * WN_;
  constexpr int WTM = BM / WM_, WTN = BN / WN_;
  constexpr int TM = WTM / 32, TN = WTN / 32;          // 32 x 32 tiles per wave
  static_assert(TM >= 1 && TN >= 1, "wave tile must be a multiple of 32x32");
  using L = StageLds<BM, BN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int M = a.M, N = a.N, K = a.K;
  const int nb = K / 32;
  const int64_t rb = (int64_t)nb * 18;
  const int tiles = tiles_m * tiles_n;
  const int tt0 = xcd_remap(blockIdx.x, tiles * split);
  const int z = tt0 / tiles;
  const int tt = tt0 - z * tiles;
  const int tm = tt % tiles_m, tn = tt / tiles_m;      // m fastest: same weight tile adjacent
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb0 = z * kchunk;
  const int kb1 = (kb0 + kchunk < nb) ? kb0 + kchunk : nb;
  const int nst = (kb1 - kb0 + KBS - 1) / KBS;
  auto live_of = [&](int s) { const int r = kb1 - (kb0 + s * KBS); return r < KBS ? r : KBS; };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave / WN_, wn = wave % WN_;
  const int h = lane >> 5, l32 = lane & 31;

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16f{};

  const _Float16* sa = reinterpret_cast<const _Float16*>(smem + L::kA);
  const uint8_t* sbw = smem + L::kB;
  const float* sd = reinterpret_cast<const float*>(smem + L::kD);
  const float* sc = reinterpret_cast<const float*>(smem + L::kC);

  Stager<BM, BN, NT, kPairs> st;
  if (nst > 0) {
    st.load(a, rb, m0, n0, kb0, live_of(0));
    st.store(smem, m0, M, n0, N, live_of(0));
  }
  __syncthreads();

  for (int s = 0; s < nst; ++s) {
    // the next stage's loads go out before this stage's matrix work
    if (s + 1 < nst) st.load(a, rb, m0, n0, kb0 + (s + 1) * KBS, live_of(s + 1));

#pragma unroll 2
    for (int blk = 0; blk < KBS; ++blk) {
      // B operands of the wave's column tiles: this lane's weight row, code
      // bytes 8h .. 8h+7 of the block (low nibbles: k = 8h..8h+7, high
      // nibbles: k = 16+8h..16+8h+7)
      v8h B0[TN], B1[TN];
      float dw[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint32_t* row = reinterpret_cast<const uint32_t*>(
            sbw + (wn * WTN + 32 * j + l32) * L::kPB + (blk >> 1) * 36);
        uint32_t u0, u1, dbits;
        if ((blk & 1) == 0) {
          const uint32_t x0 = row[2 * h], x1 = row[2 * h + 1], x2 = row[2 * h + 2];
          u0 = __builtin_amdgcn_alignbit(x1, x0, 16);
          u1 = __builtin_amdgcn_alignbit(x2, x1, 16);
          dbits = row[0] & 0xffffu;
        } else {
          u0 = row[5 + 2 * h];
          u1 = row[6 + 2 * h];
          dbits = row[4] >> 16;
        }
        dw[j] = f16_bits_to_f32(dbits);
        uint32_t lo[4], hi[4];
        nib_halves(u0, lo[0], lo[1]);
        nib_halves(u1, lo[2], lo[3]);
        nib_halves(u0 >> 4, hi[0], hi[1]);
        nib_halves(u1 >> 4, hi[2], hi[3]);
        B0[j] = __builtin_bit_cast(v8h, v4i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]});
        B1[j] = __builtin_bit_cast(v8h, v4i{(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]});
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int mr = wm * WTM + 32 * i;              // first row of the 32 x 32 tile
        const v8h A0 = *reinterpret_cast<const v8h*>(sa + (mr + l32) * L::kPA + blk * 32 + 8 * h);
        const v8h A1 = *reinterpret_cast<const v8h*>(sa + (mr + l32) * L::kPA + blk * 32 + 16 + 8 * h);
        // accumulator start and d_a of this lane's 16 output rows
        v16f c;
        float da[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 cv4 = *reinterpret_cast<const float4*>(sc + blk * BM + mr + 8 * g + 4 * h);
          const float4 dv4 = *reinterpret_cast<const float4*>(sd + blk * BM + mr + 8 * g + 4 * h);
          c[4 * g + 0] = cv4.x; c[4 * g + 1] = cv4.y; c[4 * g + 2] = cv4.z; c[4 * g + 3] = cv4.w;
          da[4 * g + 0] = dv4.x; da[4 * g + 1] = dv4.y; da[4 * g + 2] = dv4.z; da[4 * g + 3] = dv4.w;
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          v16f d = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0, B0[j], c, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1, B1[j], d, 0, 0, 0);
          // d = S_b exactly; dropped blocks and rows have d_a = 0
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(d[r], da[r] * dw[j], acc[i][j][r]);
          if constexpr (kDump) {
            const int b = kb0 + s * KBS + blk;
            const int n = n0 + wn * WTN + 32 * j + l32;
            if (blk < live_of(s)) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int m = m0 + mr + 8 * (r / 4) + 4 * h + (r % 4);
                if (m < M && n >= a.n0 && n < a.n1)
                  a.dots[((int64_t)m * (a.n1 - a.n0) + (n - a.n0)) * nb + b] = (int32_t)d[r];
              }
            }
          }
        }
      }
    }
    if (s + 1 < nst) {
      __syncthreads();                                 // every wave is done with this stage
      st.store(smem, m0, M, n0, N, live_of(s + 1));
      __syncthreads();
    }
  }

  // ---- store (or split-K partials)
  float* out = split == 1 ? a.dst : a.part + (int64_t)z * M * N;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
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
  const size_t lds = (size_t)StageLds<BM, BN>::kBytes;
  const int tm = (int)p.tiles_m, tn = (int)p.tiles_n, kc = (int)p.kchunk, sp = p.split;
  const bool dump = a.dots != nullptr;
  if (pairs) {
    if (dump) hipLaunchKernelGGL((k_q4_wide<BM, BN, WMS, WNS, true, true>), grid, block, lds, s, a, tm, tn, kc, sp);
    else hipLaunchKernelGGL((k_q4_wide<BM, BN, WMS, WNS, true, false>), grid, block, lds, s, a, tm, tn, kc, sp);
  } else {
    if (dump) hipLaunchKernelGGL((k_q4_wide<BM, BN, WMS, WNS, false, true>), grid, block, lds, s, a, tm, tn, kc, sp);
    else hipLaunchKernelGGL((k_q4_wide<BM, BN, WMS, WNS, false, false>), grid, block, lds, s, a, tm, tn, kc, sp);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q4_wide16(const Plan& p, const Q4Args& a, hipStream_t s) {
  if (!a.ah) return hipErrorInvalidValue;
  // pairs: whole block pairs per split and 4-byte aligned rows
  const bool pairs = ((a.K / 32) % 2 == 0) && (p.kchunk % 2 == 0) && ((uintptr_t)a.w % 4 == 0);
  if (p.bm == 32 && p.bn == 64) return launch_cfg<32, 64, 1, 2>(p, a, pairs, s);
  if (p.bm == 64 && p.bn == 64) return launch_cfg<64, 64, 2, 2>(p, a, pairs, s);
  return hipErrorInvalidValue;
}

}  // namespace qsg
