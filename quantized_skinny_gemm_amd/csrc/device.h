// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
}

// fp32 -> binary16 bits, round to nearest even (v_cvt_f16_f32 under the
// default rounding mode), subnormals kept.
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Sum over the 64 lanes of a wave; every lane receives the total.  The
// butterfly order is fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Dispatch places workgroup i on XCD i % 8.  Give each XCD a contiguous run
// of tile ids, so tiles that share an operand tile share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  const int per = total / 8, rem = total % 8;
  const int x = id % 8, k = id / 8;
  return x * per + (x < rem ? x : rem) + k;
}

// Split-K completion: every workgroup of a tile calls this after storing its
// partial sums.  The workgroup that arrives last (by an atomic ticket) gets
// `true` and then adds the partials in a fixed order.  Release/acquire
// fences at device scope make the other workgroups' partials visible.
__device__ __forceinline__ bool splitk_arrive(uint32_t* ticket, int split) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(ticket, 1u);
    s_last = (prev == (uint32_t)(split - 1)) ? 1 : 0;
    if (s_last) *ticket = 0u;
  }
  __syncthreads();
  const bool last = s_last != 0;
  if (last) __threadfence();
  return last;
}

// Adds the split partials of one output tile [m0, m0+bm) x [n0, n0+bn) in
// split order 0..split-1 and stores the sums into dst.
__device__ __forceinline__ void splitk_reduce_tile(const float* __restrict__ part,
                                                   float* __restrict__ dst, int M, int N,
                                                   int m0, int bm, int n0, int bn, int split) {
  const int total = bm * bn;
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const int m = m0 + i / bn, n = n0 + i % bn;
    if (m >= M || n >= N) continue;
    float s = 0.0f;
    for (int z = 0; z < split; ++z)
      s += part[((int64_t)z * M + m) * N + n];
    dst[(int64_t)m * N + n] = s;
  }
}

}  // namespace qsg
