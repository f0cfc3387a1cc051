// Plain streaming read of device buffers, for bench.py only (not part of the
// MUL_MAT library): the HBM read ceiling that the decode step's product
// kernels are compared with.  One launch reads a group of buffers (the same
// grouping as the step's launches: q,k,v / o / gate,up / down) with 16-byte
// loads, four in flight per thread, and folds every loaded word into a value
// that is stored only if it equals a constant no input produces in practice,
// so that no load can be removed.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kMaxBufs = 8;

struct Bufs {
  const uint4* p[kMaxBufs];
  int64_t n16[kMaxBufs];   // 16-byte units per buffer
  int count;
};

__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(256) void k_stream_read(Bufs b, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (int i = 0; i < b.count; ++i) {
    const uint4* __restrict__ p = b.p[i];
    const int64_t n = b.n16[i];
    int64_t j = t;
    for (; j + 3 * stride < n; j += 4 * stride) {
      const uint4 a = p[j], c = p[j + stride], d = p[j + 2 * stride], e = p[j + 3 * stride];
      acc ^= fold(a) ^ fold(c) ^ fold(d) ^ fold(e);
    }
    for (; j < n; j += stride) acc ^= fold(p[j]);
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

// Reads `count` (1..8) device buffers of bytes[i] bytes (multiples of 16,
// 16-byte aligned) in one launch of `grid` workgroups on `stream`; sink: a
// device buffer of at least grid words.  Returns 0, or -1 on bad arguments,
// or the HIP error code of the launch.
extern "C" int qsg_bench_stream_read(const void* const* ptrs, const int64_t* bytes, int count,
                                     void* sink, int grid, void* stream) {
  if (count < 1 || count > kMaxBufs || grid < 1 || !ptrs || !bytes || !sink) return -1;
  Bufs b;
  for (int i = 0; i < kMaxBufs; ++i) { b.p[i] = nullptr; b.n16[i] = 0; }
  for (int i = 0; i < count; ++i) {
    if (!ptrs[i] || bytes[i] < 0 || bytes[i] % 16 || (uintptr_t)ptrs[i] % 16) return -1;
    b.p[i] = reinterpret_cast<const uint4*>(ptrs[i]);
    b.n16[i] = bytes[i] / 16;
  }
  b.count = count;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, b,
                     reinterpret_cast<uint32_t*>(sink));
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}
