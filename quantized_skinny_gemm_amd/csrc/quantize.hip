// Q8_0 (activation, INIT / wdata) and Q4_0 (weight) quantisation for gfx950.
//
// The INIT stage that prepares src1 for the quantized MUL_MAT: llama.cpp PR
// 1632 "mulmat tune", Introduction (mul_mat_q_f32 has an INIT stage before
// COMPUTE); Arm China NUMA article, MulMat operator section (src1 is
// quantized into wdata, then dst = src0 * wdata).
//
// Layout of the work: one 8-lane group per 32-value block, each lane owning
// four consecutive values (one 16-byte load).  The block's absmax is reduced
// across the 8 lanes with xor shuffles.  Codes follow the fp32 op sequence:
// one correctly rounded reciprocal per block, one fp32 product per value,
// (Q4_0) one fp32 add of 8.5 -- with FP contraction disabled so that no
// multiply-add is fused -- then floor/clamp (Q4_0) or round half away from
// zero (Q8_0); only the stored scale is rounded to fp16 (nearest even).
#include "device.h"
#include "kernels.h"

namespace qsg {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void load4(const float* __restrict__ p, float& a, float& b, float& c,
                                      float& d) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  a = v.x; b = v.y; c = v.z; d = v.w;
}

__device__ __forceinline__ void store_u16(uint8_t* p, uint32_t v) {
  *reinterpret_cast<uint16_t*>(p) = (uint16_t)v;
}

__global__ __launch_bounds__(kThreads) void k_quantize_q8_0(
    const float* __restrict__ x, int64_t nblocks, uint8_t* __restrict__ canon,
    int8_t* __restrict__ wq, float* __restrict__ wd, int32_t* __restrict__ wb,
    uint32_t* __restrict__ zero, int64_t zero_words) {
#pragma clang fp contract(off)
  const int64_t gtid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (int64_t i = gtid; i < zero_words; i += (int64_t)gridDim.x * kThreads) zero[i] = 0u;

  const int64_t blk = gtid >> 3;
  const int g = threadIdx.x & 7;
  const bool active = blk < nblocks;
  float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
  if (active) load4(x + blk * 32 + g * 4, v0, v1, v2, v3);

  float amax = fmaxf(fmaxf(fabsf(v0), fabsf(v1)), fmaxf(fabsf(v2), fabsf(v3)));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 8));

  const float d = amax / 127.0f;                    // correctly rounded fp32 division
  const float id = d != 0.0f ? 1.0f / d : 0.0f;     // one correctly rounded reciprocal
  const int q0 = (int)roundf(v0 * id);              // round half away from zero
  const int q1 = (int)roundf(v1 * id);
  const int q2 = (int)roundf(v2 * id);
  const int q3 = (int)roundf(v3 * id);
  const uint32_t packed = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) |
                          ((uint32_t)(q2 & 0xff) << 16) | ((uint32_t)(q3 & 0xff) << 24);
  int sum = q0 + q1 + q2 + q3;
  sum += __shfl_xor(sum, 1, 8);
  sum += __shfl_xor(sum, 2, 8);
  sum += __shfl_xor(sum, 4, 8);
  if (!active) return;

  const uint32_t dbits = f32_to_f16_bits(d);
  if (canon) {
    uint8_t* b = canon + blk * 34;
    if (g == 0) store_u16(b, dbits);
    store_u16(b + 2 + 4 * g, packed & 0xffffu);
    store_u16(b + 4 + 4 * g, packed >> 16);
  }
  if (wq) {
    reinterpret_cast<uint32_t*>(wq + blk * 32)[g] = packed;
    if (g == 0) {
      wd[blk] = f16_bits_to_f32(dbits);
      wb[blk] = -8 * sum;
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_quantize_q4_0(const float* __restrict__ x,
                                                            int64_t nblocks,
                                                            uint8_t* __restrict__ y) {
#pragma clang fp contract(off)
  const int64_t gtid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t blk = gtid >> 3;
  const int g = threadIdx.x & 7;
  const bool active = blk < nblocks;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (active) load4(x + blk * 32 + g * 4, v[0], v[1], v[2], v[3]);

  // First element (lowest index) with the strictly largest |x|.
  float ba = fabsf(v[0]), bm = v[0];
  int bi = 4 * g;
#pragma unroll
  for (int j = 1; j < 4; ++j) {
    if (fabsf(v[j]) > ba) { ba = fabsf(v[j]); bm = v[j]; bi = 4 * g + j; }
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    const float oa = __shfl_xor(ba, o, 8);
    const float om = __shfl_xor(bm, o, 8);
    const int oi = __shfl_xor(bi, o, 8);
    if (oa > ba || (oa == ba && oi < bi)) { ba = oa; bm = om; bi = oi; }
  }
  const float mx = ba > 0.0f ? bm : 0.0f;           // the scan starts from +0
  const float d = mx * -0.125f;                     // == mx / -8, correctly rounded
  const float id = d != 0.0f ? 1.0f / d : 0.0f;
  uint32_t packed = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float t = v[j] * id + 8.5f;               // two roundings: contraction is off
    int q = (int)floorf(t);
    q = q < 0 ? 0 : (q > 15 ? 15 : q);
    packed |= (uint32_t)q << (8 * j);
  }
  // Lanes 0-3 hold elements 0-15, lanes 4-7 elements 16-31: byte i of the
  // block is element i (low nibble) | element i+16 (high nibble).
  const uint32_t other = (uint32_t)__shfl_xor((int)packed, 4, 8);
  if (!active || g >= 4) return;
  const uint32_t bytes = packed | (other << 4);
  uint8_t* b = y + blk * 18;
  if (g == 0) store_u16(b, f32_to_f16_bits(d));
  store_u16(b + 2 + 4 * g, bytes & 0xffffu);
  store_u16(b + 4 + 4 * g, bytes >> 16);
}

int64_t grid_for(int64_t nblocks) { return (nblocks * 8 + kThreads - 1) / kThreads; }

}  // namespace

hipError_t launch_quantize_q8_0(const float* x, int64_t nrows, int64_t k, uint8_t* canon,
                                int8_t* wq, float* wd, int32_t* wb, uint32_t* zero,
                                int64_t zero_words, hipStream_t s) {
  const int64_t nblocks = nrows * (k / 32);
  int64_t grid = grid_for(nblocks);
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(k_quantize_q8_0, dim3((unsigned)grid), dim3(kThreads), 0, s, x, nblocks,
                     canon, wq, wd, wb, zero, zero_words);
  return hipGetLastError();
}

hipError_t launch_quantize_q4_0(const float* x, int64_t nrows, int64_t k, uint8_t* y,
                                hipStream_t s) {
  const int64_t nblocks = nrows * (k / 32);
  const int64_t grid = grid_for(nblocks);
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(k_quantize_q4_0, dim3((unsigned)grid), dim3(kThreads), 0, s, x, nblocks, y);
  return hipGetLastError();
}

}  // namespace qsg
