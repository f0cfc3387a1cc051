// mul_mat_f32 and mul_mat_f16_f32 for gfx950 (llama.cpp PR 1632 "mulmat
// tune", Introduction: the two unquantized MUL_MAT kinds).
//
// Narrow (VALU) kernel: each weight row is streamed once with 16-byte loads
// and widened to fp32 in registers; src1 stays fp32; fp32 FMA accumulation;
// 64-lane butterfly reduction.  At M = 1 a wave owns one weight row and
// issues the loads of several 16-byte chunks per lane before their FMAs
// (four rows per wave for F16 beyond 8192 rows).  Rows of src1 beyond 16
// are handled by further passes (grid.y).
//
// Skinny MFMA kernel (F16 at 2 <= M <= 16, F32 at M >= 2; rows 16-byte
// aligned): passes of 16 src1 rows on the 16 x 16 matrix cores.  Each wave
// owns 16 weight rows of a K slice and loads their 16-byte pieces straight
// into MFMA operand order (no unpacking, no per-block epilogue: the weights
// are the B operand as stored); the workgroup's src1 slice is staged in LDS
// per sub-slice (128-512 k) and read by its 4 or 8 waves (both chosen in the
// plan by type and row count).  F16 uses v_mfma_f32_16x16x32_f16 with src1
// split into two binary16 terms hi + lo (their sum carries about 22 bits of
// the f32 value; each f16 x f16 product is exact in fp32), F32 uses
// v_mfma_f32_16x16x4_f32 on the values as they are.  K slices beyond one
// go to split-K partials added by the fixed-order reduce kernel.
//
// Wide f16 kernel (M > 16): a dense contraction on v_mfma_f32_32x32x16_f16
// with src1 rounded to binary16 while staging into LDS and fp32 accumulation.
// bf16 is avoided: the pages note that at small sizes converting operands to
// bf16 costs more than it gains (smallbard "Generer a plusieurs"), and its
// 8-bit mantissa would also sit too close to the 1e-3 accuracy bound.
#include "device.h"
#include "kernels.h"
#include "../../include/mm.h"

namespace qsg {

namespace {

template <typename WT>
struct WLoad;

template <>
struct WLoad<uint16_t> {   // binary16 weights: 8 values per 16-byte load
  static __device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = f16_bits_to_f32(w[i]);
      v[2 * i + 1] = f16_bits_to_f32(w[i] >> 16);
    }
  }
  static __device__ __forceinline__ float load1(const uint16_t* p) { return f16_bits_to_f32(*p); }
};

template <>
struct WLoad<float> {
  static __device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
};

template <typename WT, int MT, int R, bool kVec>
__global__ __launch_bounds__(256) void k_f_narrow(const WT* __restrict__ w,
                                                  const float* __restrict__ x,
                                                  float* __restrict__ dst, int M, int N, int K) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = blockIdx.y * MT;
  const int nw = (blockIdx.x * 4 + wave) * R;
  const WT* rowp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rowp[r] = w + (int64_t)((nw + r < N) ? nw + r : N - 1) * K;
  const float* xp[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) xp[m] = x + (int64_t)((m0 + m < M) ? m0 + m : M - 1) * K;
  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  int kdone = 0;
  if (kVec) {
    // U chunks per lane per step, all loads of a step issued before its
    // FMAs: one row per wave keeps few bytes in flight per step otherwise
    constexpr int U = R == 1 ? (sizeof(WT) == 2 ? 4 : 2) : 1;
    const int nchunks = K / 8;
    int c = lane;
    for (; c + 64 * (U - 1) < nchunks; c += 64 * U) {
      float wv[U][R][8];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r) WLoad<WT>::load8(rowp[r] + 8 * (c + 64 * u), wv[u][r]);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float4 xa = reinterpret_cast<const float4*>(xp[m] + 8 * (c + 64 * u))[0];
          const float4 xb = reinterpret_cast<const float4*>(xp[m] + 8 * (c + 64 * u))[1];
          const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][m] = fmaf(wv[u][r][e], xv[e], acc[r][m]);
        }
    }
    for (; c < nchunks; c += 64) {
      float wv[R][8];
#pragma unroll
      for (int r = 0; r < R; ++r) WLoad<WT>::load8(rowp[r] + 8 * c, wv[r]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float4 xa = reinterpret_cast<const float4*>(xp[m] + 8 * c)[0];
        const float4 xb = reinterpret_cast<const float4*>(xp[m] + 8 * c)[1];
        const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][m] = fmaf(wv[r][e], xv[e], acc[r][m]);
      }
    }
    kdone = nchunks * 8;
  }
  for (int k = kdone + lane; k < K; k += 64) {
    float wv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wv[r] = WLoad<WT>::load1(rowp[r] + k);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float xv = xp[m][k];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r][m] = fmaf(wv[r], xv, acc[r][m]);
    }
  }

  float mine = 0.0f;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float v = wave_sum(acc[r][m]);
      if (lane == r * MT + m) mine = v;
    }
  const int r = lane / MT, m = lane % MT;
  if (lane < R * MT && m0 + m < M && nw + r < N) dst[(int64_t)(m0 + m) * N + nw + r] = mine;
}

template <typename WT, int MT, int R>
hipError_t launch_f_mt(const Plan& p, const WT* w, const float* x, float* dst, int M, int N,
                       int K, bool vec, hipStream_t s) {
  const dim3 grid((unsigned)p.tiles_n, (unsigned)p.tiles_m);
  if (vec) hipLaunchKernelGGL((k_f_narrow<WT, MT, R, true>), grid, dim3(256), 0, s, w, x, dst, M, N, K);
  else hipLaunchKernelGGL((k_f_narrow<WT, MT, R, false>), grid, dim3(256), 0, s, w, x, dst, M, N, K);
  return hipGetLastError();
}

template <typename WT>
hipError_t launch_f_typed(const Plan& p, const WT* w, const float* x, float* dst, int M, int N,
                          int K, hipStream_t s) {
  const bool vec = (K % 8 == 0) && ((uintptr_t)w % 16 == 0) && ((uintptr_t)x % 16 == 0);
  switch (p.mt) {
    case 1: return p.rpw == 1 ? launch_f_mt<WT, 1, 1>(p, w, x, dst, M, N, K, vec, s)
                              : launch_f_mt<WT, 1, 4>(p, w, x, dst, M, N, K, vec, s);
    case 2: return launch_f_mt<WT, 2, 4>(p, w, x, dst, M, N, K, vec, s);
    case 4: return launch_f_mt<WT, 4, 4>(p, w, x, dst, M, N, K, vec, s);
    case 8: return launch_f_mt<WT, 8, 2>(p, w, x, dst, M, N, K, vec, s);
    case 16: return launch_f_mt<WT, 16, 2>(p, w, x, dst, M, N, K, vec, s);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------ skinny MFMA (F16, F32)
typedef float v4f __attribute__((ext_vector_type(4)));

template <bool kF16, int SUB_>
struct FmCfg {
  static constexpr int kSub = SUB_;                             // k per LDS sub-slice
  static constexpr int kStep = kF16 ? 32 : 16;                  // k per MFMA step
  static constexpr int kSteps = kSub / kStep;
  static constexpr int kPitch = kSub + (kF16 ? 8 : 4);          // LDS row pitch (elements)
  static constexpr int kLds = kF16 ? 2 * 16 * kPitch * 2 : 16 * kPitch * 4;
};

// Lane (l16, kq) of wave w: B operand column = weight row n0 + 16 w + l16; in
// step s of a sub-slice starting at k0 it holds k = k0 + kStep s + 8 kq ..
// +7 (F16) or k0 + kStep s + 4 kq .. +3 (F32: one element per 16x16x4 MFMA,
// the same k in the A operand).  Output: rows m0 + 4 kq .. +3, column n.
template <bool kF16, bool kVecX, int W, int SUB_>
__global__ __launch_bounds__(64 * W, 2)
void k_f_mma(const void* __restrict__ wv_, const float* __restrict__ x, float* __restrict__ out,
             int M, int N, int K, int krange) {
  typedef FmCfg<kF16, SUB_> C;
  constexpr int SUB = C::kSub, XP = C::kPitch, ST = C::kStep, NSTEP = C::kSteps, NT = 64 * W;
  __shared__ __attribute__((aligned(16))) uint8_t xs[C::kLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, kq = lane >> 4;
  const int m0 = blockIdx.y * 16, z = blockIdx.z;
  const int n = blockIdx.x * (16 * W) + 16 * wave + l16;
  const int nr = n < N ? n : N - 1;
  const int kbeg = z * krange;
  const int kend = kbeg + krange < K ? kbeg + krange : K;
  const uint8_t* wrow = reinterpret_cast<const uint8_t*>(wv_) + (int64_t)nr * K * (kF16 ? 2 : 4);
  float* o = out + (int64_t)z * M * N;               // the slice's partial (dst when one slice)
  const int kl = kF16 ? 8 * kq : 4 * kq;             // this lane's k offset within a step
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};

  constexpr int IT = 16 * SUB / 4 / NT;               // src1 float4 items per thread
  static_assert(IT * NT == 16 * SUB / 4, "src1 items must fill the threads");
  for (int k0 = kbeg; k0 < kend; k0 += SUB) {
    // src1 rows m0 .. m0+15, k0 .. k0+SUB-1 first (their wait then leaves
    // the weights in flight), clamped into range and zeroed past M and kend
    // (kend % 4 == 0: an item is wholly in or out)
    float4 xv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = tid + NT * it;
      const int r = i / (SUB / 4), c = i % (SUB / 4);
      const int m = m0 + r < M ? m0 + r : M - 1, k = k0 + 4 * c < kend ? k0 + 4 * c : kbeg;
      const float* px = x + (int64_t)m * K + k;
      if (kVecX) {
        xv[it] = *reinterpret_cast<const float4*>(px);
      } else {
        xv[it] = make_float4(px[0], px[1], px[2], px[3]);
      }
    }
    // this lane's 16 weight pieces of the sub-slice (past kend: clamped,
    // then zeroed)
    v4i wp[NSTEP];
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      const int k = k0 + ST * s + kl;
      const int kc = k < kend ? k : 0;
      wp[s] = *(const __attribute__((address_space(1))) v4i*)(wrow + (int64_t)kc * (kF16 ? 2 : 4));
    }
    __syncthreads();                                 // the last sub-slice's LDS reads are done
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = tid + NT * it;
      const int r = i / (SUB / 4), c = i % (SUB / 4);
      const bool ok = m0 + r < M && k0 + 4 * c < kend;
      const float v[4] = {ok ? xv[it].x : 0.0f, ok ? xv[it].y : 0.0f, ok ? xv[it].z : 0.0f,
                          ok ? xv[it].w : 0.0f};
      if constexpr (kF16) {
        _Float16* xh = reinterpret_cast<_Float16*>(xs);
        _Float16* xl = xh + 16 * XP;
        v4h hi, lo;
        hi.x = (_Float16)v[0]; hi.y = (_Float16)v[1]; hi.z = (_Float16)v[2]; hi.w = (_Float16)v[3];
        lo.x = (_Float16)(v[0] - (float)hi.x); lo.y = (_Float16)(v[1] - (float)hi.y);
        lo.z = (_Float16)(v[2] - (float)hi.z); lo.w = (_Float16)(v[3] - (float)hi.w);
        *reinterpret_cast<v4h*>(xh + r * XP + 4 * c) = hi;
        *reinterpret_cast<v4h*>(xl + r * XP + 4 * c) = lo;
      } else {
        float* xf = reinterpret_cast<float*>(xs);
        *reinterpret_cast<float4*>(xf + r * XP + 4 * c) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      const bool in = k0 + ST * s + kl < kend;
      v4i b = wp[s];
      b.x = in ? b.x : 0; b.y = in ? b.y : 0; b.z = in ? b.z : 0; b.w = in ? b.w : 0;
      if constexpr (kF16) {
        const _Float16* xh = reinterpret_cast<const _Float16*>(xs);
        const _Float16* xl = xh + 16 * XP;
        const v8h bh = __builtin_bit_cast(v8h, b);
        const v8h ah = *reinterpret_cast<const v8h*>(xh + l16 * XP + ST * s + kl);
        const v8h al = *reinterpret_cast<const v8h*>(xl + l16 * XP + ST * s + kl);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, acc, 0, 0, 0);
      } else {
        const float* xf = reinterpret_cast<const float*>(xs);
        const float4 a4 = *reinterpret_cast<const float4*>(xf + l16 * XP + ST * s + kl);
        // whole-vector bit cast (a bit cast of one element lvalue of an
        // ext_vector reads element 0 with this compiler)
        const v4f bf = __builtin_bit_cast(v4f, b);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.x, bf[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.y, bf[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.z, bf[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.w, bf[3], acc, 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + 4 * kq + r;
    if (m < M && n < N) o[(int64_t)m * N + n] = acc[r];
  }
}

// ------------------------------------------------------------ wide f16

// src1 -> binary16 (round to nearest even), [M][K] as given; the wide
// kernel's A operand.  Four values per thread when src1 is 16-byte aligned
// and the count a multiple of four.
template <bool kVec>
__global__ __launch_bounds__(256) void k_f32_to_f16(const float* __restrict__ x,
                                                    uint16_t* __restrict__ y, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  if (kVec) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; 4 * i < n; i += stride) {
      const float4 f = reinterpret_cast<const float4*>(x)[i];
      v4h hv;
      hv.x = (_Float16)f.x; hv.y = (_Float16)f.y; hv.z = (_Float16)f.z; hv.w = (_Float16)f.w;
      reinterpret_cast<v4h*>(y)[i] = hv;
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
      y[i] = (uint16_t)f32_to_f16_bits(x[i]);
  }
}

// KS: k per LDS stage.  128 x 128 tiles take 64 (more would cost the
// prefetch registers two waves per SIMD need), 64 x 64 tiles 128 (half the
// barriers per MFMA: M = 512, 4096 x 4096 61.4 -> 45.6 us; M = 64,
// 14336 x 4096 61.6 -> 45.0 us; 128 x 128 at 14336 / 128256 rows gains
// nothing from it).
template <int BM, int BN, bool kVec, int KS>
__global__ __launch_bounds__(256) void k_f16_wide(const uint16_t* __restrict__ w,
                                                  const uint16_t* __restrict__ xh,
                                                  float* __restrict__ dst, int M, int N, int K,
                                                  int tiles_m, int tiles_n) {
  constexpr int HP = KS + 8;         // halves per LDS row (pad)
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int WM = WTM / 32, WN = WTN / 32;
  __shared__ __attribute__((aligned(16))) _Float16 sA[BM * HP];
  __shared__ __attribute__((aligned(16))) _Float16 sB[BN * HP];
  const int tiles = tiles_m * tiles_n;
  const int t = xcd_remap(blockIdx.x, tiles);
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / 2, wn = wave % 2;
  const int h = lane >> 5, l32 = lane & 31;

  v16f acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = v16f{};

  // Register prefetch: the next stage's pieces of 8 halves of src1 (binary16,
  // converted beforehand) and src0 are loaded before the current stage's
  // MFMAs; loads are unconditional with clamped addresses, and what lies
  // outside the matrices is zeroed when the registers go to LDS.
  constexpr int XI = BM * (KS / 8) / 256, WI = BN * (KS / 8) / 256;
  static_assert(XI * 256 == BM * (KS / 8) && WI * 256 == BN * (KS / 8), "whole items per thread");
  uint4 xr[XI], wr[WI];
  auto load8 = [&](const uint16_t* base, int row, int k) -> uint4 {
    if (kVec) {
      const int kk = k < K ? k : 0;                  // K % 8 == 0: k < K means k + 8 <= K
      const v4i v = *(const __attribute__((address_space(1))) v4i*)(base + (int64_t)row * K + kk);
      return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
    }
    uint32_t hw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) hw[e] = base[(int64_t)row * K + (k + e < K ? k + e : 0)];
    return make_uint4(hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16), hw[4] | (hw[5] << 16),
                      hw[6] | (hw[7] << 16));
  };
  auto mask8 = [&](uint4 v, bool okrow, int k) -> uint4 {
    if (kVec) {
      const bool ok = okrow && k < K;
      return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
    }
    uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = (okrow && k + 2 * e < K) ? (d[e] & 0xffffu) : 0u;
      const uint32_t hi = (okrow && k + 2 * e + 1 < K) ? (d[e] >> 16) : 0u;
      d[e] = lo | (hi << 16);
    }
    return make_uint4(d[0], d[1], d[2], d[3]);
  };
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < XI; ++u) {
      const int i = tid + 256 * u;
      const int r = i / (KS / 8), c = i % (KS / 8);
      xr[u] = load8(xh, m0 + r < M ? m0 + r : M - 1, k0 + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < WI; ++u) {
      const int i = tid + 256 * u;
      const int r = i / (KS / 8), c = i % (KS / 8);
      wr[u] = load8(w, n0 + r < N ? n0 + r : N - 1, k0 + 8 * c);
    }
  };
  auto store = [&](int k0) {
#pragma unroll
    for (int u = 0; u < XI; ++u) {
      const int i = tid + 256 * u;
      const int r = i / (KS / 8), c = i % (KS / 8);
      *reinterpret_cast<uint4*>(sA + r * HP + 8 * c) = mask8(xr[u], m0 + r < M, k0 + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < WI; ++u) {
      const int i = tid + 256 * u;
      const int r = i / (KS / 8), c = i % (KS / 8);
      *reinterpret_cast<uint4*>(sB + r * HP + 8 * c) = mask8(wr[u], n0 + r < N, k0 + 8 * c);
    }
  };

  load(0);
  for (int k0 = 0; k0 < K; k0 += KS) {
    __syncthreads();                                 // the last stage's MFMAs are done
    store(k0);
    __syncthreads();
    if (k0 + KS < K) load(k0 + KS);                  // uniform over the workgroup
#pragma unroll
    for (int s = 0; s < KS / 16; ++s) {
      v8h A[WM], B[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i)
        A[i] = *reinterpret_cast<const v8h*>(sA + (wm * WTM + 32 * i + l32) * HP + 16 * s + 8 * h);
#pragma unroll
      for (int j = 0; j < WN; ++j)
        B[j] = *reinterpret_cast<const v8h*>(sB + (wn * WTN + 32 * j + l32) * HP + 16 * s + 8 * h);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int n = n0 + wn * WTN + 32 * j + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * WTM + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
        if (m < M && n < N) dst[(int64_t)m * N + n] = acc[i][j][r];
      }
    }
}

__global__ void k_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part,
                                                      float* __restrict__ dst, int64_t n,
                                                      int split) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float s = 0.0f;
    for (int z = 0; z < split; ++z) s += part[(int64_t)z * n + i];
    dst[i] = s;
  }
}

}  // namespace

hipError_t launch_splitk_reduce(const float* part, float* dst, int64_t n, int split,
                                hipStream_t s) {
  int64_t grid = (n + 255) / 256;
  if (grid > 2048) grid = 2048;
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)grid), dim3(256), 0, s, part, dst, n, split);
  return hipGetLastError();
}

hipError_t launch_f_narrow(const Plan& p, int type, const void* w, const float* x, float* dst,
                           int M, int N, int K, hipStream_t s) {
  if (type == MM_TYPE_F16)
    return launch_f_typed<uint16_t>(p, (const uint16_t*)w, x, dst, M, N, K, s);
  return launch_f_typed<float>(p, (const float*)w, x, dst, M, N, K, s);
}

hipError_t launch_f16_wide(const Plan& p, const uint16_t* w, const float* x, float* dst, int M,
                           int N, int K, void* ws, hipStream_t s) {
  // src1 -> binary16 into the workspace, then the tiled product
  uint16_t* xh = reinterpret_cast<uint16_t*>((uint8_t*)ws + p.off_ah);
  const int64_t n = (int64_t)M * K;
  const bool cvec = (uintptr_t)x % 16 == 0 && n % 4 == 0;
  int64_t cgrid = ((cvec ? n / 4 : n) + 255) / 256;
  if (cgrid > 4096) cgrid = 4096;
  if (cvec) hipLaunchKernelGGL((k_f32_to_f16<true>), dim3((unsigned)cgrid), dim3(256), 0, s, x, xh, n);
  else hipLaunchKernelGGL((k_f32_to_f16<false>), dim3((unsigned)cgrid), dim3(256), 0, s, x, xh, n);
  const bool vec = (K % 8 == 0) && ((uintptr_t)w % 16 == 0);    // xh is 256-byte aligned
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
  const int tm = (int)p.tiles_m, tn = (int)p.tiles_n;
  if (p.bm == 128) {
    if (vec) hipLaunchKernelGGL((k_f16_wide<128, 128, true, 64>), grid, dim3(256), 0, s, w, xh, dst, M, N, K, tm, tn);
    else hipLaunchKernelGGL((k_f16_wide<128, 128, false, 64>), grid, dim3(256), 0, s, w, xh, dst, M, N, K, tm, tn);
  } else {
    if (vec) hipLaunchKernelGGL((k_f16_wide<64, 64, true, 128>), grid, dim3(256), 0, s, w, xh, dst, M, N, K, tm, tn);
    else hipLaunchKernelGGL((k_f16_wide<64, 64, false, 128>), grid, dim3(256), 0, s, w, xh, dst, M, N, K, tm, tn);
  }
  return hipGetLastError();
}

bool f_mma_aligned(int type, const void* w, int K) {
  return (uintptr_t)w % 16 == 0 && K % (type == MM_TYPE_F16 ? 8 : 4) == 0;
}

template <bool kF16, int W, int SUB>
hipError_t launch_f_mma_cfg(const Plan& p, const void* w, const float* x, float* out, int M, int N,
                            int K, hipStream_t s) {
  const dim3 grid((unsigned)p.tiles_n, (unsigned)p.tiles_m, (unsigned)p.split);
  const int kr = (int)p.kchunk;
  if ((uintptr_t)x % 16 == 0)
    hipLaunchKernelGGL((k_f_mma<kF16, true, W, SUB>), grid, dim3(64 * W), 0, s, w, x, out, M, N, K, kr);
  else
    hipLaunchKernelGGL((k_f_mma<kF16, false, W, SUB>), grid, dim3(64 * W), 0, s, w, x, out, M, N, K, kr);
  return hipGetLastError();
}

hipError_t launch_f_mma(const Plan& p, int type, const void* w, const float* x, float* out, int M,
                        int N, int K, hipStream_t s) {
  // (waves, k per sub-slice) as the plan chose them
  if (type == MM_TYPE_F16) {
    if (p.waves == 8 && p.bn == 512) return launch_f_mma_cfg<true, 8, 512>(p, w, x, out, M, N, K, s);
    if (p.waves == 8 && p.bn == 256) return launch_f_mma_cfg<true, 8, 256>(p, w, x, out, M, N, K, s);
  } else {
    if (p.waves == 4 && p.bn == 128) return launch_f_mma_cfg<false, 4, 128>(p, w, x, out, M, N, K, s);
    if (p.waves == 8 && p.bn == 128) return launch_f_mma_cfg<false, 8, 128>(p, w, x, out, M, N, K, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_zero(float* dst, int64_t n, hipStream_t s) {
  int64_t grid = (n + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)grid), dim3(256), 0, s, dst, n);
  return hipGetLastError();
}

}  // namespace qsg
