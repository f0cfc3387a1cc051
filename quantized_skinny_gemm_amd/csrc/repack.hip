// Q4_0 weight repack at load time (DeepSpeed-Inference notes, III.C SBI-GeMM
// item 3: lay the weights out once, at initialisation, so that the product
// kernels read whole cache lines in the order they consume them).
//
// Repacked layout ("Q4_0R"): the same 18 bytes per 32-value block, grouped
// per tile of 16 weight rows and phase of 8 blocks into one 2304-byte chunk,
// chunks ordered tile-major ([ceil(N/16)][ceil(K/256)]):
//   bytes    0 .. 2047  codes: [half hh][lane l][dword j], 16 bytes per lane:
//                       lane l = i + 16 g holds, for blocks 4 hh + j
//                       (j = 0..3), code bytes 4 g .. 4 g + 3 of row i of the
//                       tile (low nibbles: elements 4 g .. 4 g + 3, high
//                       nibbles: elements 16 + 4 g .. 19 + 4 g).  This is the
//                       A-operand order of v_mfma_i32_16x16x32_i8 for one
//                       block per MFMA: a lane's operand is one dword.
//   bytes 2048 .. 2303  scales: [row i][block b] binary16 d, 16 bytes per row.
// Rows past N and blocks past K/32 are padding: codes 0x88 (q = 8, i.e. the
// value 0) and scale 0, so they add nothing to a product.
#include "device.h"
#include "kernels.h"

namespace qsg {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ size_t chunk_base(int64_t t, int64_t f, int64_t phases) {
  return (size_t)(t * phases + f) * kQ4RChunk;
}

// One thread per (tile, phase, row, block): reads the block (18 bytes,
// 2-byte aligned) or writes padding, scatters its 4 code dwords and scale.
__global__ __launch_bounds__(kThreads) void k_repack_q4_0(const uint8_t* __restrict__ src,
                                                          uint8_t* __restrict__ dst, int64_t N,
                                                          int64_t nb, int64_t tiles,
                                                          int64_t phases) {
  const int64_t total = tiles * phases * 128;
  for (int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * kThreads) {
    const int b = (int)(id & 7), i = (int)((id >> 3) & 15);
    const int64_t tf = id >> 7;
    const int64_t f = tf % phases, t = tf / phases;
    const int64_t row = 16 * t + i, blk = 8 * f + b;
    uint32_t w[4];
    uint32_t d = 0;
    if (row < N && blk < nb) {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(src + (row * nb + blk) * 18);
      d = p[0];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = (uint32_t)p[1 + 2 * j] | ((uint32_t)p[2 + 2 * j] << 16);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = 0x88888888u;
    }
    uint8_t* c = dst + chunk_base(t, f, phases);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<uint32_t*>(c + (b >> 2) * 1024 + (i + 16 * g) * 16 + (b & 3) * 4) = w[g];
    *reinterpret_cast<uint16_t*>(c + 2048 + i * 16 + b * 2) = (uint16_t)d;
  }
}

// The inverse for the rows and blocks that exist.
__global__ __launch_bounds__(kThreads) void k_unpack_q4_0(const uint8_t* __restrict__ src,
                                                          uint8_t* __restrict__ dst, int64_t N,
                                                          int64_t nb, int64_t phases) {
  const int64_t total = N * nb;
  for (int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * kThreads) {
    const int64_t row = id / nb, blk = id % nb;
    const int64_t t = row / 16, f = blk / 8;
    const int i = (int)(row % 16), b = (int)(blk % 8);
    const uint8_t* c = src + chunk_base(t, f, phases);
    uint16_t* p = reinterpret_cast<uint16_t*>(dst + id * 18);
    p[0] = *reinterpret_cast<const uint16_t*>(c + 2048 + i * 16 + b * 2);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t w =
          *reinterpret_cast<const uint32_t*>(c + (b >> 2) * 1024 + (i + 16 * g) * 16 + (b & 3) * 4);
      p[1 + 2 * g] = (uint16_t)(w & 0xffffu);
      p[2 + 2 * g] = (uint16_t)(w >> 16);
    }
  }
}

int64_t grid_of(int64_t items) {
  int64_t g = (items + kThreads - 1) / kThreads;
  return g > 8192 ? 8192 : g;
}

}  // namespace

hipError_t launch_repack_q4_0(const uint8_t* src, uint8_t* dst, int64_t N, int64_t K,
                              hipStream_t s) {
  const int64_t nb = K / 32, tiles = (N + 15) / 16, phases = (nb + 7) / 8;
  const int64_t g = grid_of(tiles * phases * 128);
  if (g < 1) return hipSuccess;
  hipLaunchKernelGGL(k_repack_q4_0, dim3((unsigned)g), dim3(kThreads), 0, s, src, dst, N, nb,
                     tiles, phases);
  return hipGetLastError();
}

hipError_t launch_unpack_q4_0(const uint8_t* src, uint8_t* dst, int64_t N, int64_t K,
                              hipStream_t s) {
  const int64_t nb = K / 32, phases = (nb + 7) / 8;
  const int64_t g = grid_of(N * nb);
  if (g < 1) return hipSuccess;
  hipLaunchKernelGGL(k_unpack_q4_0, dim3((unsigned)g), dim3(kThreads), 0, s, src, dst, N, nb,
                     phases);
  return hipGetLastError();
}

}  // namespace qsg
