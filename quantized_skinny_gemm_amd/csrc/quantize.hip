// Q8_0 (activation, INIT / wdata) and Q4_0 (weight) quantisation for gfx950.
//
// The INIT stage that prepares src1 for the quantized MUL_MAT: llama.cpp PR
// 1632 "mulmat tune", Introduction (mul_mat_q_f32 has an INIT stage before
// COMPUTE); Arm China NUMA article, MulMat operator section (src1 is
// quantized into wdata, then dst = src0 * wdata).
//
// Layout of the work: Q8_0 uses a pair of lanes per 32-value block (16
// values, four 16-byte loads each); Q4_0 an 8-lane group per block (four
// values each).  The block's absmax is reduced across the lanes of the group.  Codes follow the fp32 op sequence:
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
    int8_t* __restrict__ wq, float* __restrict__ wd, int32_t* __restrict__ wb) {
  // two lanes per block, 16 values (64 bytes) each
  const int64_t gtid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t blk = gtid >> 1;
  const int h = threadIdx.x & 1;
  const bool active = blk < nblocks;
  float v[16];
  const float4* p = reinterpret_cast<const float4*>(x + (active ? blk : 0) * 32 + 16 * h);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 f = p[i];
    v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
  }
  uint32_t packed[4], dbits;
  int sum;
  q8_0_pair(v, packed, dbits, sum);
  if (!active) return;

  if (canon) {
    uint8_t* b = canon + blk * 34;
    if (h == 0) store_u16(b, dbits);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      store_u16(b + 2 + 16 * h + 4 * j, packed[j] & 0xffffu);
      store_u16(b + 4 + 16 * h + 4 * j, packed[j] >> 16);
    }
  }
  if (wq) {
    *reinterpret_cast<uint4*>(wq + blk * 32 + 16 * h) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    if (h == 0) {
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

// INIT of the skinny MFMA kernels: the plain wdata of the real blocks, and
// over the padded domain (rows x phases * 8 blocks; zeros past the real ones)
// the codes and scales in that kernel's operand order.  16-row tiles: row
// m = 16 t + i, block b = 8 f + 2 j + e: the 4 code bytes 4g .. 4g+3 (lane
// h = 0) or 16+4g .. 19+4g (h = 1) go to byte 8e + 4h of the 16 bytes that
// lane 16g + i of the MFMA loads for pair j of phase f of tile t.  8-row
// tiles (rows8): see below.
__global__ __launch_bounds__(kThreads) void k_quantize_q8_0_skinny(
    const float* __restrict__ x, int M, int K, int phases, int64_t nblocks,
    int8_t* __restrict__ wq, float* __restrict__ wd, int32_t* __restrict__ wb,
    uint8_t* __restrict__ sq, float* __restrict__ ss, bool rows8) {
  const int64_t gtid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t blk = gtid >> 1;                    // over the padded domain
  const int h = threadIdx.x & 1;
  const int nbp = 8 * phases, nb = K / 32;
  const int m = (int)(blk / nbp), b = (int)(blk % nbp);
  const bool active = blk < nblocks;
  const bool real = active && m < M && b < nb;
  float v[16];
  if (real) {
    const float4* p = reinterpret_cast<const float4*>(x + (int64_t)m * K + 32 * b + 16 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = p[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.0f;
  }
  uint32_t packed[4], dbits;
  int sum;
  q8_0_pair(v, packed, dbits, sum);
  if (!active) return;
  if (real) {
    const int64_t pb = (int64_t)m * nb + b;
    *reinterpret_cast<uint4*>(wq + pb * 32 + 16 * h) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    if (h == 0) {
      wd[pb] = f16_bits_to_f32(dbits);
      wb[pb] = -8 * sum;
    }
  }
  if (rows8) {
    // 8-row tiles: row m = 8 t + i, block b = 8 f + 2 j + e is column
    // c = 8 e + i of pair j's 16 x 16 x 64 MFMA; the lane of column c in
    // group 2 e + s loads slot 2 c + s (16 bytes) of the pair's 512: elements
    // 8s .. 8s+3, 16+8s .. 19+8s, 8s+4 .. 8s+7, 20+8s .. 23+8s, i.e. this
    // thread's code dword qd (elements 16 h + 4 qd ..) goes to slot
    // 2 c + qd / 2, dword 2 (qd % 2) + h.  Scales: d_a at (c, j).
    const int t = m >> 3, i = m & 7;
    const int f = b >> 3, kb = b & 7, j = kb >> 1, e = kb & 1;
    const int c = 8 * e + i;
    uint8_t* base = sq + (((int64_t)t * phases + f) * 4 + j) * 512;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
      *reinterpret_cast<uint32_t*>(base + 16 * (2 * c + (qd >> 1)) + 4 * (2 * (qd & 1) + h)) = packed[qd];
    if (h == 0) ss[(((int64_t)t * phases + f) * 16 + c) * 4 + j] = f16_bits_to_f32(dbits);
    return;
  }
  const int t = m >> 4, i = m & 15;
  const int f = b >> 3, kb = b & 7, j = kb >> 1, e = kb & 1;
  uint8_t* base = sq + (((int64_t)t * phases + f) * 4 + j) * 1024 + 8 * e + 4 * h;
#pragma unroll
  for (int g = 0; g < 4; ++g) *reinterpret_cast<uint32_t*>(base + 16 * (16 * g + i)) = packed[g];
  // d_a as binary16 bits, the 8 blocks of the phase in 16 bytes per row (the
  // kernel's fp16 scale product takes them as loaded: dword q = blocks 2q,
  // 2q + 1)
  if (h == 0)
    reinterpret_cast<uint16_t*>(ss)[(((int64_t)t * phases + f) * 16 + i) * 8 + kb] = (uint16_t)dbits;
}

int64_t grid_for(int64_t nblocks, int lanes) { return (nblocks * lanes + kThreads - 1) / kThreads; }

}  // namespace

hipError_t launch_quantize_q8_0(const float* x, int64_t nrows, int64_t k, uint8_t* canon,
                                int8_t* wq, float* wd, int32_t* wb, hipStream_t s) {
  const int64_t nblocks = nrows * (k / 32);
  const int64_t grid = grid_for(nblocks, 2);
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(k_quantize_q8_0, dim3((unsigned)grid), dim3(kThreads), 0, s, x, nblocks,
                     canon, wq, wd, wb);
  return hipGetLastError();
}

hipError_t launch_quantize_q4_0(const float* x, int64_t nrows, int64_t k, uint8_t* y,
                                hipStream_t s) {
  const int64_t nblocks = nrows * (k / 32);
  const int64_t grid = grid_for(nblocks, 8);
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(k_quantize_q4_0, dim3((unsigned)grid), dim3(kThreads), 0, s, x, nblocks, y);
  return hipGetLastError();
}

hipError_t launch_quantize_q8_0_skinny(const float* x, int64_t nrows, int64_t k, int8_t* wq,
                                       float* wd, int32_t* wb, uint8_t* sq, float* ss,
                                       int64_t rows, int64_t phases, bool rows8, hipStream_t s) {
  const int64_t nblocks = rows * phases * 8;
  const int64_t grid = grid_for(nblocks, 2);
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(k_quantize_q8_0_skinny, dim3((unsigned)grid), dim3(kThreads), 0, s, x,
                     (int)nrows, (int)k, (int)phases, nblocks, wq, wd, wb, sq, ss, rows8);
  return hipGetLastError();
}

}  // namespace qsg
