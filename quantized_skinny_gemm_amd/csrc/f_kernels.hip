// mul_mat_f32 and mul_mat_f16_f32 for gfx950 (llama.cpp PR 1632 "mulmat
// tune", Introduction: the two unquantized MUL_MAT kinds).
//
// Narrow (VALU) kernel: each weight row is streamed once with 16-byte loads
// and widened to fp32 in registers; src1 stays fp32; fp32 FMA accumulation;
// 64-lane butterfly reduction.  At M = 1 a wave owns one weight row and
// issues the loads of several 16-byte chunks per lane before their FMAs
// (four rows per wave for F16 beyond 8192 rows).  With few rows the waves of
// a workgroup split K over the same rows and add their partial sums in LDS
// in slice order.  Rows of src1 beyond 16 are handled by further passes
// (grid.y).
//
// Skinny MFMA kernel (F16 at 2 <= M <= 16 and, with at most 8192 weight
// rows, up to 64; F32 from M = 2; operands 16-byte aligned): one workgroup
// per 16 weight rows and pass of 16 src1 rows, its waves splitting K and
// adding their partial tiles in LDS at the end, so one launch does the whole
// product.  The products run on v_mfma_f32_16x16x4_f32: F16 weights are
// widened to fp32 in registers (exact) and src1 is used as given, so every
// product is an exact fp32 product and no magnitude of src1 is lost to a
// narrower format.  (Rounding src1 to binary16 for the fp16 matrix
// instruction saves about 5% of a call at M = 2-8 and nothing at 16-32:
// this kernel is not bound by its matrix instructions.)
//
// Wide f16 kernel (M beyond that): a dense contraction on
// v_mfma_f32_32x32x16_f16; src1 is rounded to binary16 once per call after a
// power-of-two scale per row (undone on the outputs), fp32 accumulation.
// bf16 is avoided: the pages note that at small sizes converting operands to
// bf16 costs more than it gains (smallbard "Generer a plusieurs"), and its
// 8-bit mantissa would also sit too close to the 1e-3 accuracy bound.
#include <type_traits>

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

// Narrow kernel: 4 waves per workgroup, R weight rows and MT src1 rows per
// wave, each lane 8 values of K per load.  With KS > 1 the waves form 4 / KS
// row groups of KS waves that split K into contiguous slices over the same
// rows (more waves in flight when the rows alone give too few) and add their
// partial results in LDS in slice order.
template <typename WT, int MT, int R, bool kVec, int KS>
__global__ __launch_bounds__(256) void k_f_narrow(const WT* __restrict__ w,
                                                  const float* __restrict__ x,
                                                  float* __restrict__ dst, int M, int N, int K) {
  static_assert(KS == 1 || KS == 2 || KS == 4, "K slices per row group");
  constexpr int GPW = 4 / KS;                        // row groups per workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave / KS, ks = wave % KS;
  const int m0 = blockIdx.y * MT;
  const int nw = (blockIdx.x * GPW + grp) * R;
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
    // this wave's chunks [cs, ce): slices of whole 64-chunk rounds
    const int per = ((nchunks + 64 * KS - 1) / (64 * KS)) * 64;
    const int cs = ks * per < nchunks ? ks * per : nchunks;
    const int ce = cs + per < nchunks ? cs + per : nchunks;
    int c = cs + lane;
    for (; c + 64 * (U - 1) < ce; c += 64 * U) {
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
    for (; c < ce; c += 64) {
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
  // the values past the last whole chunk (all of K without kVec): slice 0
  for (int k = kdone + lane; ks == 0 && k < K; k += 64) {
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
  if constexpr (KS > 1) {
    __shared__ float part[4][R * MT];
    if (ks > 0 && lane < R * MT) part[wave][lane] = mine;
    __syncthreads();
    if (ks > 0) return;
#pragma unroll
    for (int j = 1; j < KS; ++j)
      if (lane < R * MT) mine += part[wave + j][lane];
  }
  const int r = lane / MT, m = lane % MT;
  if (lane < R * MT && m0 + m < M && nw + r < N) dst[(int64_t)(m0 + m) * N + nw + r] = mine;
}

template <typename WT, int MT, int R>
hipError_t launch_f_mt(const Plan& p, const WT* w, const float* x, float* dst, int M, int N,
                       int K, bool vec, hipStream_t s) {
  // K slices only on the vector path (the scalar path is one wave's)
  const int ks = vec ? p.kslices : 1;
  if (ks != 1 && ks != 2 && ks != 4) return hipErrorInvalidValue;
  const int64_t rows_per_wg = (int64_t)(4 / ks) * R;
  // src1 passes of MT rows go in the grid's y dimension: more than
  // kMaxGridY of them run as launches over consecutive row ranges
  const int64_t rows = kMaxGridY * MT;
  for (int64_t r0 = 0; r0 < M; r0 += rows) {
    const int mc = (int)(M - r0 < rows ? M - r0 : rows);
    const float* xc = x + r0 * K;
    float* dc = dst + r0 * N;
    const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg), (unsigned)((mc + MT - 1) / MT));
    if (!vec)
      hipLaunchKernelGGL((k_f_narrow<WT, MT, R, false, 1>), grid, dim3(256), 0, s, w, xc, dc, mc, N, K);
    else if (ks == 4)
      hipLaunchKernelGGL((k_f_narrow<WT, MT, R, true, 4>), grid, dim3(256), 0, s, w, xc, dc, mc, N, K);
    else if (ks == 2)
      hipLaunchKernelGGL((k_f_narrow<WT, MT, R, true, 2>), grid, dim3(256), 0, s, w, xc, dc, mc, N, K);
    else
      hipLaunchKernelGGL((k_f_narrow<WT, MT, R, true, 1>), grid, dim3(256), 0, s, w, xc, dc, mc, N, K);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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

// Buffer resources: a lane whose byte offset lies at or past the end of the
// range reads zeros and sends no request, which is how lanes of weight rows
// past N, of src1 rows past M, of k past K and of steps past the wave's K run
// skip their loads without a branch.
constexpr int kSkip = 0x7FFFFFF0;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t f_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ v4i f_bload(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// One workgroup per RT x 16 weight rows and pass of 16 src1 rows (grid.y);
// its W waves split K into runs of `spw` steps and add their partial tiles in
// LDS at the end, in wave order (DeepSpeed-Inference notes, III.C: partial
// sums reduced on chip rather than by another kernel).  A step is 32 k (F16)
// or 16 k (F32): one 16-byte weight piece per lane and row tile.  Lane
// (l16, kq) holds weight rows n0 + 16 i + l16 (i < RT) and src1 row m0 + l16
// at k = step * STEP + P * kq .. + P - 1 (P = 8 for F16, 4 for F32).  The
// products run on v_mfma_f32_16x16x4_f32, element j of every lane's piece in
// MFMA j: the weights (binary16 widened to fp32, exact) are the A operand,
// src1 as it is the B operand, shared by the RT row tiles; every product is
// an exact fp32 product of the given values, so no magnitude of src1 is
// lost to a narrower format.  Output lane (l16, kq) of tile i holds
// dst[m0 + l16][n0 + 16 i + 4 kq + r].
template <bool kF16, int W, int S, int RT>
__global__ __launch_bounds__(64 * W) void k_f_skinny(const void* __restrict__ w_,
                                                     const float* __restrict__ x,
                                                     float* __restrict__ dst, int M, int N, int K,
                                                     int spw) {
  constexpr int ES = kF16 ? 2 : 4;                 // bytes per weight
  constexpr int P = kF16 ? 8 : 4;                  // k per lane and step
  constexpr int STEP = 4 * P;                      // k per step
  constexpr int XL = P / 4;                        // 16-byte src1 loads per lane and step
  __shared__ v4f red[W][RT][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, kq = lane >> 4;
  const int n0 = blockIdx.x * (16 * RT), m0 = blockIdx.y * 16;
  const int nrows = N - n0 < 16 * RT ? N - n0 : 16 * RT;
  const int mrows = M - m0 < 16 ? M - m0 : 16;
  const __amdgpu_buffer_rsrc_t rw =
      f_rsrc(reinterpret_cast<const uint8_t*>(w_) + (int64_t)n0 * K * ES, nrows * K * ES);
  const __amdgpu_buffer_rsrc_t rx = f_rsrc(x + (int64_t)m0 * K, mrows * K * 4);
  const bool xok = l16 < mrows;
  const int nsteps = (K + STEP - 1) / STEP;
  const int s0 = wave * spw;
  const int s1 = s0 + spw < nsteps ? s0 + spw : nsteps;

  auto load = [&](v4i (&wv)[S][RT], v4i (&xv)[S][XL], int s) {
#pragma unroll
    for (int t = 0; t < S; ++t) {
      const int k = (s + t) * STEP + P * kq;
      const bool in = s + t < s1 && k < K;           // K % P == 0: a piece is whole
#pragma unroll
      for (int i = 0; i < RT; ++i)
        wv[t][i] = f_bload(rw, in && 16 * i + l16 < nrows ? ((16 * i + l16) * K + k) * ES : kSkip);
#pragma unroll
      for (int h = 0; h < XL; ++h)
        xv[t][h] = f_bload(rx, in && xok ? (l16 * K + k + 4 * h) * 4 : kSkip);
    }
  };

  v4f acc[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](const v4i (&wv)[S][RT], const v4i (&xv)[S][XL]) {
#pragma unroll
    for (int t = 0; t < S; ++t) {
      float b[P];
#pragma unroll
      for (int h = 0; h < XL; ++h) {
        const v4f f = __builtin_bit_cast(v4f, xv[t][h]);
        b[4 * h] = f.x; b[4 * h + 1] = f.y; b[4 * h + 2] = f.z; b[4 * h + 3] = f.w;
      }
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        float a[P];
        if constexpr (kF16) {
          const uint32_t u[4] = {(uint32_t)wv[t][i].x, (uint32_t)wv[t][i].y, (uint32_t)wv[t][i].z,
                                 (uint32_t)wv[t][i].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            a[2 * j] = f16_bits_to_f32(u[j]);
            a[2 * j + 1] = f16_bits_to_f32(u[j] >> 16);
          }
        } else {
          const v4f f = __builtin_bit_cast(v4f, wv[t][i]);
          a[0] = f.x; a[1] = f.y; a[2] = f.z; a[3] = f.w;
        }
#pragma unroll
        for (int j = 0; j < P; ++j)
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc[i], 0, 0, 0);
      }
    }
  };

  // two register sets: the next sub-slice's loads are in flight while one
  // is computed.  The loads are issued unconditionally (past the run they
  // send no request): a load under a branch would make the compiler wait
  // for it before the current sub-slice's MFMAs.  (The plan makes every run
  // a whole number of sub-slice pairs; past K the pair computes zeros.)
  v4i w0[S][RT], w1[S][RT], x0[S][XL], x1[S][XL];
  load(w0, x0, s0);
  for (int s = s0; s < s1; s += 2 * S) {
    load(w1, x1, s + S);
    __builtin_amdgcn_sched_barrier(0);               // keep the loads ahead of the MFMAs
    compute(w0, x0);
    load(w0, x0, s + 2 * S);
    __builtin_amdgcn_sched_barrier(0);
    compute(w1, x1);
  }

#pragma unroll
  for (int i = 0; i < RT; ++i) red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave >= RT) return;
  // wave i adds row tile i's partial tiles in wave order
  const int i = wave;
  v4f v = red[0][i][lane];
#pragma unroll
  for (int u = 1; u < W; ++u) v += red[u][i][lane];
  const int m = m0 + l16, n = n0 + 16 * i + 4 * kq;
  if (m >= M) return;
  float* o = dst + (int64_t)m * N + n;
  if (n + 3 < N && ((uintptr_t)o & 15) == 0) {
    *reinterpret_cast<v4f*>(o) = v;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) o[r] = v[r];
  }
}

// ------------------------------------------------------------ wide f16

// src1 -> binary16 with one power of two per row: row m is scaled by 2^e[m]
// so that its largest magnitude lies in [2^14, 2^15), then rounded to
// binary16 (nearest even); the product kernel scales its outputs back by
// 2^-e[m] (exact).  Without the scale, rows below about 1e-5 would fall on
// binary16's subnormal grid and rows past 65504 would overflow.  One
// workgroup per row; four values per load when the row is 16-byte aligned.
template <bool kVec>
__global__ __launch_bounds__(256) void k_f32_to_f16_rows(const float* __restrict__ x,
                                                         uint16_t* __restrict__ y,
                                                         int* __restrict__ rexp, int K) {
  __shared__ float wmax[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float* xr = x + (int64_t)m * K;
  uint16_t* yr = y + (int64_t)m * K;
  float amax = 0.0f;
  if (kVec) {
    for (int i = tid; 4 * i < K; i += 256) {
      const float4 f = reinterpret_cast<const float4*>(xr)[i];
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
    }
  } else {
    for (int i = tid; i < K; i += 256) amax = fmaxf(amax, fabsf(xr[i]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int e = 15 - __builtin_amdgcn_frexp_expf(amax);
  if (tid == 0) rexp[m] = e;
  if (kVec) {
    for (int i = tid; 4 * i < K; i += 256) {
      const float4 f = reinterpret_cast<const float4*>(xr)[i];
      v4h hv;
      hv.x = (_Float16)__builtin_amdgcn_ldexpf(f.x, e);
      hv.y = (_Float16)__builtin_amdgcn_ldexpf(f.y, e);
      hv.z = (_Float16)__builtin_amdgcn_ldexpf(f.z, e);
      hv.w = (_Float16)__builtin_amdgcn_ldexpf(f.w, e);
      reinterpret_cast<v4h*>(yr)[i] = hv;
    }
  } else {
    for (int i = tid; i < K; i += 256) yr[i] = (uint16_t)f32_to_f16_bits(__builtin_amdgcn_ldexpf(xr[i], e));
  }
}

// KS: k per LDS stage.  128 x 128 tiles take 64 (more would cost the
// prefetch registers two waves per SIMD need), 64 x 64 tiles 128 (half the
// barriers per MFMA: M = 512, 4096 x 4096 61.4 -> 45.6 us; M = 64,
// 14336 x 4096 61.6 -> 45.0 us; 128 x 128 at 14336 / 128256 rows gains
// nothing from it).
// NS: stages whose global loads are in flight in registers.  The 64 x 64
// tile serves grids of about one workgroup per CU or fewer, where nothing
// else hides a stage's load latency: with NS = 3 the loads of stage k + 3
// are issued when stage k goes to LDS (us per call, M = 64: 4096 x 4096
// 42.4 -> 27.9, 14336 x 4096 47.4 -> 35.6, 4096 x 14336 134.0 -> 81.3; the
// same within 3% from two workgroups per CU up).  The 128 x 128 tile keeps
// NS = 1: its second set would take it to 190 VGPRs, two waves per SIMD,
// and it is slower where its grids fill the device (128256 x 4096, M = 512:
// 708 -> 779-789 us with NS = 2).
template <int BM, int BN, bool kVec, int KS, int NS>
__global__ __launch_bounds__(256) void k_f16_wide(const uint16_t* __restrict__ w,
                                                  const uint16_t* __restrict__ xh,
                                                  const int* __restrict__ rexp,
                                                  float* __restrict__ dst, int M, int N, int K,
                                                  int tiles_m, int tiles_n, int kchunk) {
  constexpr int HP = KS + 8;         // halves per LDS row (pad)
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int WM = WTM / 32, WN = WTN / 32;
  __shared__ __attribute__((aligned(16))) _Float16 sA[BM * HP];
  __shared__ __attribute__((aligned(16))) _Float16 sB[BN * HP];
  const int tiles = tiles_m * tiles_n;
  const int t = xcd_remap(blockIdx.x, tiles);
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  // K range of this workgroup (blockIdx.y of a K split; kchunk a multiple of KS)
  const int kb = (int)blockIdx.y * kchunk;
  const int ke = kb + kchunk < K ? kb + kchunk : K;
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
  uint4 xr[NS][XI], wr[NS][WI];
  auto load8 = [&](const uint16_t* base, int row, int k) -> uint4 {
    if (kVec) {
      const int kk = k < ke ? k : kb;                // K % 8 == 0: k < ke means k + 8 <= ke
      const v4i v = *(const __attribute__((address_space(1))) v4i*)(base + (int64_t)row * K + kk);
      return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
    }
    uint32_t hw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) hw[e] = base[(int64_t)row * K + (k + e < ke ? k + e : kb)];
    return make_uint4(hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16), hw[4] | (hw[5] << 16),
                      hw[6] | (hw[7] << 16));
  };
  auto mask8 = [&](uint4 v, bool okrow, int k) -> uint4 {
    if (kVec) {
      const bool ok = okrow && k < ke;
      return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
    }
    uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = (okrow && k + 2 * e < ke) ? (d[e] & 0xffffu) : 0u;
      const uint32_t hi = (okrow && k + 2 * e + 1 < ke) ? (d[e] >> 16) : 0u;
      d[e] = lo | (hi << 16);
    }
    return make_uint4(d[0], d[1], d[2], d[3]);
  };
  // register set S (a std::integral_constant: registers are not indexed at
  // run time)
  auto load = [&](auto set, int k0) {
    constexpr int S = decltype(set)::value;
#pragma unroll
    for (int u = 0; u < XI; ++u) {
      const int i = tid + 256 * u;
      const int r = i / (KS / 8), c = i % (KS / 8);
      xr[S][u] = load8(xh, m0 + r < M ? m0 + r : M - 1, k0 + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < WI; ++u) {
      const int i = tid + 256 * u;
      const int r = i / (KS / 8), c = i % (KS / 8);
      wr[S][u] = load8(w, n0 + r < N ? n0 + r : N - 1, k0 + 8 * c);
    }
  };
  auto store = [&](auto set, int k0) {
    constexpr int S = decltype(set)::value;
#pragma unroll
    for (int u = 0; u < XI; ++u) {
      const int i = tid + 256 * u;
      const int r = i / (KS / 8), c = i % (KS / 8);
      *reinterpret_cast<uint4*>(sA + r * HP + 8 * c) = mask8(xr[S][u], m0 + r < M, k0 + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < WI; ++u) {
      const int i = tid + 256 * u;
      const int r = i / (KS / 8), c = i % (KS / 8);
      *reinterpret_cast<uint4*>(sB + r * HP + 8 * c) = mask8(wr[S][u], n0 + r < N, k0 + 8 * c);
    }
  };
  auto compute = [&]() {
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
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  static_assert(NS >= 1 && NS <= 3, "one to three register sets");

  if constexpr (NS == 1) {
    load(I0{}, kb);
    for (int k0 = kb; k0 < ke; k0 += KS) {
      __syncthreads();                               // the last stage's MFMAs are done
      store(I0{}, k0);
      __syncthreads();
      if (k0 + KS < ke) load(I0{}, k0 + KS);         // uniform over the workgroup
      compute();
    }
  } else {
    // Stage k comes from set k % NS, whose loads for stage k + NS are issued
    // once stage k is in LDS.  Loads are unconditional (addresses past K are
    // clamped, the data unused) and kept in issue order by scheduling
    // barriers: the same loads are in flight on every path, so the wait
    // before a stage's store leaves the other sets' loads in flight.
    load(I0{}, kb);
    __builtin_amdgcn_sched_barrier(0);
    load(I1{}, kb + KS);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NS > 2) {
      load(I2{}, kb + 2 * KS);
      __builtin_amdgcn_sched_barrier(0);
    }
    auto step = [&](auto set, int kk) {
      const bool live = kk < ke;                     // uniform
      if (live) {
        __syncthreads();                             // the last stage's MFMAs are done
        store(set, kk);
        __syncthreads();
      }
      load(set, kk + NS * KS);
      __builtin_amdgcn_sched_barrier(0);
      if (live) compute();
    };
    for (int k0 = kb; k0 < ke; k0 += NS * KS) {
      step(I0{}, k0);
      step(I1{}, k0 + KS);
      if constexpr (NS > 2) step(I2{}, k0 + 2 * KS);
    }
  }
  // with a K split: this slice's partial tile (scaled back, exact), added by
  // the split-K reduce
  float* const out = dst + (int64_t)blockIdx.y * M * N;
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int n = n0 + wn * WTN + 32 * j + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * WTM + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
        if (m < M && n < N) out[(int64_t)m * N + n] = __builtin_amdgcn_ldexpf(acc[i][j][r], -rexp[m]);
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
  // src1 -> binary16 (a power of two per row) into the workspace, then the
  // tiled product
  uint16_t* xh = reinterpret_cast<uint16_t*>((uint8_t*)ws + p.off_ah);
  int* rexp = reinterpret_cast<int*>((uint8_t*)ws + p.off_rexp);
  const bool cvec = (uintptr_t)x % 16 == 0 && K % 4 == 0;
  if (cvec) hipLaunchKernelGGL((k_f32_to_f16_rows<true>), dim3((unsigned)M), dim3(256), 0, s, x, xh, rexp, K);
  else hipLaunchKernelGGL((k_f32_to_f16_rows<false>), dim3((unsigned)M), dim3(256), 0, s, x, xh, rexp, K);
  const bool vec = (K % 8 == 0) && ((uintptr_t)w % 16 == 0);    // xh is 256-byte aligned
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n), (unsigned)p.split);
  const int tm = (int)p.tiles_m, tn = (int)p.tiles_n, kc = (int)p.kchunk;
  float* out = p.split > 1 ? reinterpret_cast<float*>((uint8_t*)ws + p.off_part) : dst;
  if (p.bm == 128) {
    if (vec) hipLaunchKernelGGL((k_f16_wide<128, 128, true, 64, 1>), grid, dim3(256), 0, s, w, xh, rexp, out, M, N, K, tm, tn, kc);
    else hipLaunchKernelGGL((k_f16_wide<128, 128, false, 64, 1>), grid, dim3(256), 0, s, w, xh, rexp, out, M, N, K, tm, tn, kc);
  } else {
    if (vec) hipLaunchKernelGGL((k_f16_wide<64, 64, true, 128, 3>), grid, dim3(256), 0, s, w, xh, rexp, out, M, N, K, tm, tn, kc);
    else hipLaunchKernelGGL((k_f16_wide<64, 64, false, 128, 1>), grid, dim3(256), 0, s, w, xh, rexp, out, M, N, K, tm, tn, kc);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && p.split > 1) e = launch_splitk_reduce(out, dst, (int64_t)M * N, p.split, s);
  return e;
}

bool f_mma_ok(int type, const void* w, const float* x, int64_t K) {
  // 16-byte pieces of both operands; 32-bit buffer offsets over 16 rows
  return (uintptr_t)w % 16 == 0 && (uintptr_t)x % 16 == 0 &&
         K % (type == MM_TYPE_F16 ? 8 : 4) == 0 && K <= kFMmaMaxK;
}

template <bool kF16, int W, int S, int RT>
hipError_t launch_f_mma_cfg(const Plan& p, const void* w, const float* x, float* dst, int M, int N,
                            int K, hipStream_t s) {
  // 16-row src1 passes in the grid's y dimension, at most kMaxGridY per launch
  const int64_t rows = kMaxGridY * 16;
  for (int64_t r0 = 0; r0 < M; r0 += rows) {
    const int mc = (int)(M - r0 < rows ? M - r0 : rows);
    const dim3 grid((unsigned)p.tiles_n, (unsigned)((mc + 15) / 16));
    hipLaunchKernelGGL((k_f_skinny<kF16, W, S, RT>), grid, dim3(64 * W), 0, s, w, x + r0 * K,
                       dst + r0 * N, mc, N, K, (int)p.kchunk);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_f_mma(const Plan& p, int type, const void* w, const float* x, float* dst, int M,
                        int N, int K, hipStream_t s) {
  // (waves, steps per sub-slice, row tiles) as the plan chose them
  const bool f16 = type == MM_TYPE_F16;
#define QSG_FCFG(W_, S_, RT_)                                                                \
  if (p.waves == W_ && p.bn == S_ && p.rpw == 16 * RT_)                                      \
    return f16 ? launch_f_mma_cfg<true, W_, S_, RT_>(p, w, x, dst, M, N, K, s)               \
               : launch_f_mma_cfg<false, W_, S_, RT_>(p, w, x, dst, M, N, K, s);
  QSG_FCFG(4, 2, 1) QSG_FCFG(8, 2, 1) QSG_FCFG(4, 2, 2)
#undef QSG_FCFG
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
