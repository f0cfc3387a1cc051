// extern "C" entry points declared in include/mm.h.
//
// Each entry point validates its arguments on the host (plan.cpp) before any
// HIP call, checks once per device that it runs on gfx950, then enqueues the
// kernels on the caller's stream without synchronising.
#include <hip/hip_runtime.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/mm.h"
#include "kernels.h"
#include "plan.h"

using namespace qsg;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MM_ERR_DEVICE;
  int state = g_device_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MM_ERR_HIP;
    state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_device_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? MM_OK : MM_ERR_DEVICE;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MM_OK : MM_ERR_HIP; }

// Workspace of mm_mul_mat_q4_0_f32_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address on the current
// GPU comes from hipGetSymbolAddress, looked up once per device (with that
// device current) and kept in g_scratch_ptr; only that pointer is ever
// passed to a kernel.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call on each device), or NULL with *st set on failure.
void* scratch_ptr(int* st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) { *st = MM_ERR_HIP; return nullptr; }
  if (dev < 0 || dev >= kMaxDevices) { *st = MM_ERR_DEVICE; return nullptr; }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      *st = MM_ERR_HIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *st = MM_OK;
  return g_scratch_ptr[dev];
}

Q4Args q4_args(const Plan& p, const void* src0, float* dst, int32_t* dots, int64_t M,
               int64_t N, int64_t K, int64_t n0, int64_t n1, void* ws) {
  uint8_t* base = (uint8_t*)ws;
  Q4Args a;
  a.w = (const uint8_t*)src0;
  a.aq = (const int8_t*)(base + p.off_aq);
  a.ad = (const float*)(base + p.off_ad);
  a.ab = (const int32_t*)(base + p.off_ab);
  a.sq = p.off_sq ? (const uint8_t*)(base + p.off_sq) : nullptr;
  a.ss = p.off_ss ? (const float*)(base + p.off_ss) : nullptr;
  a.sk_phases = (int)p.sk_phases;
  a.sq_bytes = (int)(p.sk_rows * p.sk_phases * 256);
  a.ss_bytes = (int)(p.sk_rows * p.sk_phases * 32);
  a.dst = dst;
  a.part = p.split > 1 ? (float*)(base + p.off_part) : nullptr;
  a.M = (int)M; a.N = (int)N; a.K = (int)K;
  a.dots = dots; a.n0 = (int)n0; a.n1 = (int)n1;
  return a;
}

// INIT: src1 -> Q8_0 wdata in the workspace.
int q4_init(const Plan& p, const float* src1, int64_t M, int64_t K, void* ws, hipStream_t s) {
  uint8_t* base = (uint8_t*)ws;
  if (p.off_sq)
    return hip_status(launch_quantize_q8_0_skinny(
        src1, M, K, (int8_t*)(base + p.off_aq), (float*)(base + p.off_ad),
        (int32_t*)(base + p.off_ab), base + p.off_sq, (float*)(base + p.off_ss), p.sk_rows,
        p.sk_phases, p.mt == 8, s));
  return hip_status(launch_quantize_q8_0(src1, M, K, nullptr, (int8_t*)(base + p.off_aq),
                                         (float*)(base + p.off_ad), (int32_t*)(base + p.off_ab), s));
}

Q4Mats single_mat(const void* src0, float* dst, int64_t N) {
  Q4Mats m;
  for (int i = 0; i < kMaxGroup; ++i) { m.w[i] = nullptr; m.dst[i] = nullptr; }
  for (int i = 0; i <= kMaxGroup; ++i) m.row0[i] = (int)N;
  m.w[0] = (const uint8_t*)src0;
  m.dst[0] = dst;
  m.row0[0] = 0;
  m.count = 1;
  return m;
}

// The product kernel (x != NULL: INIT fused), then the split-K reduction.
int q4_product(const Plan& p, const Q4Args& a, const float* x, hipStream_t s) {
  // Q8_0 weights have no staged-chunk fallback for the skinny plan
  if (p.type == MM_TYPE_Q8_0 && p.kind == KK_Q4_MMA && !(a.sq && q4_skinny_ok(a.K, a.w)))
    return MM_ERR_ARG;
  hipError_t e = p.kind == KK_Q4_NARROW    ? launch_q4_narrow(p, a, single_mat(a.w, a.dst, a.N), x, s)
                 : p.kind == KK_Q4_MMA     ? (a.sq && q4_skinny_ok(a.K, a.w) ? launch_q4_skinny(p, a, s)
                                                                       : launch_q4_mma(p, a, s))
                 : p.kind == KK_Q4R_SKINNY ? launch_q4r_skinny(p, a, s)
                                           : launch_q4_wide_i8(p, a, s);
  if (e == hipSuccess && p.split > 1)
    e = launch_splitk_reduce(a.part, a.dst, (int64_t)a.M * a.N, p.split, s);
  return hip_status(e);
}

int run_q4_0(const Plan& p, const void* src0, const float* src1, float* dst, int32_t* dots,
             int64_t M, int64_t N, int64_t K, int64_t n0, int64_t n1, void* ws, hipStream_t s) {
  const Q4Args a = q4_args(p, src0, dst, dots, M, N, K, n0, n1, ws);
  if (p.kind == KK_Q4_NARROW && p.fuse) return q4_product(p, a, src1, s);
  const int st = q4_init(p, src1, M, K, ws, s);
  if (st != MM_OK) return st;
  return q4_product(p, a, nullptr, s);
}

// Skinny F16 / F32 product: the MFMA kernel, one launch; operands that it
// cannot take (not 16-byte aligned, K off its step) take the narrow kernel's
// plan for the same shape instead.
int run_f_mma(const Plan& p, int type, const void* src0, const float* src1, float* dst,
              int64_t M, int64_t N, int64_t K, hipStream_t s) {
  if (!f_mma_ok(type, src0, src1, K)) {
    Plan q;
    const int st = make_plan(type, M, N, K, 1, &q);
    if (st != MM_OK) return st;
    return hip_status(launch_f_narrow(q, type, src0, src1, dst, (int)M, (int)N, (int)K, s));
  }
  return hip_status(launch_f_mma(p, type, src0, src1, dst, (int)M, (int)N, (int)K, s));
}

int mul_mat(int type, const void* src0, const float* src1, float* dst, int32_t* dots,
            int64_t M, int64_t N, int64_t K, int64_t n0, int64_t n1, int variant, void* ws,
            size_t ws_bytes, void* stream) {
  Plan p;
  int st = make_plan(type, M, N, K, variant, &p);
  if (st != MM_OK) return st;
  st = validate_mul_mat(type, src0, src1, dst, M, N, K, ws, ws_bytes, p);
  if (st != MM_OK) return st;
  if (p.kind == KK_NONE) return MM_OK;
  st = check_device();
  if (st != MM_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  switch (p.kind) {
    case KK_ZERO: return hip_status(launch_zero(dst, M * N, s));
    case KK_Q4_NARROW:
    case KK_Q4_MMA:
    case KK_Q4R_SKINNY:
    case KK_Q4_WIDE: return run_q4_0(p, src0, src1, dst, dots, M, N, K, n0, n1, ws, s);
    case KK_F_NARROW:
      return hip_status(launch_f_narrow(p, type, src0, src1, dst, (int)M, (int)N, (int)K, s));
    case KK_F_MMA: return run_f_mma(p, type, src0, src1, dst, M, N, K, s);
    case KK_F16_WIDE:
      return hip_status(launch_f16_wide(p, (const uint16_t*)src0, src1, dst, (int)M, (int)N,
                                        (int)K, ws, s));
    default: return MM_ERR_ARG;
  }
}

int quantize(int out_type, const float* x, void* y, int64_t nrows, int64_t k, void* stream) {
  int st = validate_quantize(out_type, x, y, nrows, k);
  if (st != MM_OK) return st;
  if (nrows == 0 || k == 0) return MM_OK;
  st = check_device();
  if (st != MM_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (out_type == MM_TYPE_Q4_0) return hip_status(launch_quantize_q4_0(x, nrows, k, (uint8_t*)y, s));
  return hip_status(launch_quantize_q8_0(x, nrows, k, (uint8_t*)y, nullptr, nullptr, nullptr, s));
}

// Q4_0 <-> repacked Q4_0: plain rows are 2-byte aligned, the repacked
// buffer 16-byte aligned; the two must not overlap.
int repack(const void* src, void* dst, int64_t N, int64_t K, bool to_repacked, void* stream) {
  const int64_t rb = repacked_bytes(N, K);
  if (rb < 0) return MM_ERR_SHAPE;
  if (N == 0 || K == 0) return MM_OK;
  if (!src || !dst) return MM_ERR_NULL;
  const void* plain = to_repacked ? src : dst;
  const void* packed = to_repacked ? dst : src;
  if ((uintptr_t)plain % 2 || (uintptr_t)packed % 16) return MM_ERR_ALIGN;
  const uintptr_t p0 = (uintptr_t)plain, p1 = (uintptr_t)packed;
  const size_t pb = (size_t)N * (size_t)row_bytes(MM_TYPE_Q4_0, K);
  if (p0 < p1 + (size_t)rb && p1 < p0 + pb) return MM_ERR_ALIAS;
  const int st = check_device();
  if (st != MM_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  return hip_status(to_repacked
                        ? launch_repack_q4_0((const uint8_t*)src, (uint8_t*)dst, N, K, s)
                        : launch_unpack_q4_0((const uint8_t*)src, (uint8_t*)dst, N, K, s));
}

}  // namespace

// Status codes travel as int inside the library; the C entry points return
// them as the header's enum.
inline mm_status as_status(int st) { return static_cast<mm_status>(st); }

extern "C" {

mm_status mm_quantize_q4_0(const float* x, void* y, int64_t nrows, int64_t k, void* stream) {
  return as_status(quantize(MM_TYPE_Q4_0, x, y, nrows, k, stream));
}

mm_status mm_quantize_q8_0(const float* x, void* y, int64_t nrows, int64_t k, void* stream) {
  return as_status(quantize(MM_TYPE_Q8_0, x, y, nrows, k, stream));
}

mm_status mm_mul_mat_q4_0_f32(const void* src0, const float* src1, float* dst,
                              int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                              void* stream) {
  return as_status(
      mul_mat(MM_TYPE_Q4_0, src0, src1, dst, nullptr, M, N, K, 0, 0, 0, ws, ws_bytes, stream));
}

mm_status mm_mul_mat_q4_0_f32_noalloc(const void* src0, const float* src1, float* dst, int64_t M,
                                      int64_t N, int64_t K, void* stream) {
  // the plan first: a shape whose workspace does not fit the array is
  // rejected before any HIP call
  Plan p;
  int st = make_plan(MM_TYPE_Q4_0, M, N, K, 0, &p);
  if (st != MM_OK) return as_status(st);
  if (p.ws_bytes > kNoAllocScratchBytes) return MM_ERR_WORKSPACE;
  if (p.kind == KK_NONE) return MM_OK;
  st = validate_mul_mat(MM_TYPE_Q4_0, src0, src1, dst, M, N, K, nullptr, 0, p, STAGE_ALL,
                        /*check_ws=*/false);
  if (st != MM_OK) return as_status(st);
  st = check_device();
  if (st != MM_OK) return as_status(st);
  void* ws = scratch_ptr(&st);
  if (!ws) return as_status(st);
  return as_status(mul_mat(MM_TYPE_Q4_0, src0, src1, dst, nullptr, M, N, K, 0, 0, 0, ws,
                 kNoAllocScratchBytes, stream));
}

mm_status mm_mul_mat_q8_0_f32(const void* src0, const float* src1, float* dst,
                              int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                              void* stream) {
  return as_status(
      mul_mat(MM_TYPE_Q8_0, src0, src1, dst, nullptr, M, N, K, 0, 0, 0, ws, ws_bytes, stream));
}

mm_status mm_mul_mat_q4_0r_f32(const void* src0r, const float* src1, float* dst,
                               int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                               void* stream) {
  return as_status(
      mul_mat(MM_TYPE_Q4_0R, src0r, src1, dst, nullptr, M, N, K, 0, 0, 0, ws, ws_bytes, stream));
}

int64_t mm_repacked_q4_0_bytes(int64_t N, int64_t K) { return repacked_bytes(N, K); }

mm_status mm_repack_q4_0(const void* src0, void* dst, int64_t N, int64_t K, void* stream) {
  return as_status(repack(src0, dst, N, K, /*to_repacked=*/true, stream));
}

mm_status mm_unpack_q4_0(const void* src0r, void* dst, int64_t N, int64_t K, void* stream) {
  return as_status(repack(src0r, dst, N, K, /*to_repacked=*/false, stream));
}

mm_status mm_mul_mat_f16_f32(const uint16_t* src0, const float* src1, float* dst, int64_t M,
                             int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream) {
  return as_status(
      mul_mat(MM_TYPE_F16, src0, src1, dst, nullptr, M, N, K, 0, 0, 0, ws, ws_bytes, stream));
}

mm_status mm_mul_mat_f32(const float* src0, const float* src1, float* dst,
                         int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                         void* stream) {
  return as_status(
      mul_mat(MM_TYPE_F32, src0, src1, dst, nullptr, M, N, K, 0, 0, 0, ws, ws_bytes, stream));
}

mm_status mm_q4_0_init(const float* src1, void* ws, int64_t M, int64_t N, int64_t K,
                       size_t ws_bytes, void* stream) {
  Plan p;
  int st = make_plan(MM_TYPE_Q4_0, M, N, K, 0, &p);
  if (st != MM_OK) return as_status(st);
  st = validate_mul_mat(MM_TYPE_Q4_0, nullptr, src1, nullptr, M, N, K, ws, ws_bytes, p, STAGE_INIT);
  if (st != MM_OK) return as_status(st);
  if (p.kind == KK_NONE || p.kind == KK_ZERO) return MM_OK;
  st = check_device();
  if (st != MM_OK) return as_status(st);
  return as_status(q4_init(p, src1, M, K, ws, (hipStream_t)stream));
}

mm_status mm_q4_0_compute(const void* src0, float* dst, int64_t M, int64_t N, int64_t K,
                          const void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int st = make_plan(MM_TYPE_Q4_0, M, N, K, 0, &p);
  if (st != MM_OK) return as_status(st);
  st = validate_mul_mat(MM_TYPE_Q4_0, src0, nullptr, dst, M, N, K, ws, ws_bytes, p, STAGE_COMPUTE);
  if (st != MM_OK) return as_status(st);
  if (p.kind == KK_NONE) return MM_OK;
  st = check_device();
  if (st != MM_OK) return as_status(st);
  hipStream_t s = (hipStream_t)stream;
  if (p.kind == KK_ZERO) return as_status(hip_status(launch_zero(dst, M * N, s)));
  return as_status(
      q4_product(p, q4_args(p, src0, dst, nullptr, M, N, K, 0, 0, (void*)ws), nullptr, s));
}

namespace {

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Plan of a grouped product: narrow -> one launch over the concatenated rows
// (no split); wide -> one plan per matrix, sharing the wdata at the front of
// the workspace.  Returns the workspace size through *ws.
int group_plan(int count, const int64_t* Ns, int64_t M, int64_t K, Plan* whole, int64_t* ntot,
               size_t* ws) {
  if (count < 1 || count > kMaxGroup) return MM_ERR_ARG;
  if (!Ns) return MM_ERR_NULL;
  int64_t tot = 0;
  for (int i = 0; i < count; ++i) {
    if (Ns[i] < 0) return MM_ERR_SHAPE;
    tot += Ns[i];
  }
  if (tot > 0x7fffffff) return MM_ERR_SHAPE;
  *ntot = tot;
  int st = make_plan(MM_TYPE_Q4_0, M, tot, K, 0, whole, /*allow_split=*/false);
  if (st != MM_OK) return st;
  size_t need = whole->ws_bytes;
  if (whole->kind == KK_Q4_WIDE || whole->kind == KK_Q4_MMA) {
    // every member takes the group's kernel (one INIT writes the wdata
    // layout of that kernel for all of them)
    for (int i = 0; i < count; ++i) {
      Plan pi;
      st = make_plan(MM_TYPE_Q4_0, M, Ns[i], K, whole->variant, &pi);
      if (st != MM_OK) return st;
      if (pi.ws_bytes > need) need = pi.ws_bytes;
    }
  }
  *ws = need;
  return MM_OK;
}

}  // namespace

size_t mm_mul_mat_q4_0_group_workspace_size(int count, const int64_t* Ns, int64_t M, int64_t K) {
  Plan p;
  int64_t tot;
  size_t ws = 0;
  if (group_plan(count, Ns, M, K, &p, &tot, &ws) != MM_OK) return 0;
  return ws;
}

mm_status mm_mul_mat_q4_0_f32_group(int count, const void* const* src0s, float* const* dsts,
                                    const int64_t* Ns, const float* src1, int64_t M, int64_t K,
                                    void* ws, size_t ws_bytes, void* stream) {
  Plan whole;
  int64_t ntot = 0;
  size_t need = 0;
  int st = group_plan(count, Ns, M, K, &whole, &ntot, &need);
  if (st != MM_OK) return as_status(st);
  if (!src0s || !dsts) return MM_ERR_NULL;
  if (M == 0 || ntot == 0) return MM_OK;
  // each product on its own, then the group as a whole
  const int64_t rbytes = row_bytes(MM_TYPE_Q4_0, K);
  for (int i = 0; i < count; ++i) {
    if (Ns[i] == 0) continue;
    Plan pi = whole;
    pi.ws_bytes = need;
    st = validate_mul_mat(MM_TYPE_Q4_0, src0s[i], src1, dsts[i], M, Ns[i], K, ws, ws_bytes, pi);
    if (st != MM_OK) return as_status(st);
    for (int j = 0; j < count; ++j) {
      if (j == i || Ns[j] == 0) continue;
      if (ranges_overlap(dsts[i], (size_t)M * Ns[i] * 4, dsts[j], (size_t)M * Ns[j] * 4) ||
          (K > 0 && ranges_overlap(dsts[i], (size_t)M * Ns[i] * 4, src0s[j], (size_t)Ns[j] * rbytes)))
        return MM_ERR_ALIAS;
    }
  }
  st = check_device();
  if (st != MM_OK) return as_status(st);
  hipStream_t s = (hipStream_t)stream;
  if (K == 0) {
    for (int i = 0; i < count; ++i) {
      if (Ns[i] == 0) continue;
      st = hip_status(launch_zero(dsts[i], M * Ns[i], s));
      if (st != MM_OK) return as_status(st);
    }
    return MM_OK;
  }
  if (whole.kind == KK_Q4_NARROW) {
    Q4Mats mats;
    int row = 0, c = 0;
    for (int i = 0; i < kMaxGroup; ++i) { mats.w[i] = nullptr; mats.dst[i] = nullptr; }
    for (int i = 0; i < count; ++i) {
      if (Ns[i] == 0) continue;
      mats.w[c] = (const uint8_t*)src0s[i];
      mats.dst[c] = dsts[i];
      mats.row0[c] = row;
      row += (int)Ns[i];
      ++c;
    }
    for (int i = c; i <= kMaxGroup; ++i) mats.row0[i] = row;
    mats.count = c;
    const Q4Args a = q4_args(whole, mats.w[0], mats.dst[0], nullptr, M, ntot, K, 0, 0, ws);
    if (!whole.fuse) {
      st = q4_init(whole, src1, M, K, ws, s);
      if (st != MM_OK) return as_status(st);
    }
    return as_status(hip_status(launch_q4_narrow(whole, a, mats, whole.fuse ? src1 : nullptr, s)));
  }
  // wide and skinny MFMA: one INIT, then one product per matrix (same wdata
  // layout at the front of every per-matrix plan)
  st = q4_init(whole, src1, M, K, ws, s);
  if (st != MM_OK) return as_status(st);
  for (int i = 0; i < count; ++i) {
    if (Ns[i] == 0) continue;
    Plan pi;
    make_plan(MM_TYPE_Q4_0, M, Ns[i], K, whole.variant, &pi);
    st = q4_product(pi, q4_args(pi, src0s[i], dsts[i], nullptr, M, Ns[i], K, 0, 0, ws), nullptr, s);
    if (st != MM_OK) return as_status(st);
  }
  return MM_OK;
}

size_t mm_mul_mat_workspace_size(int type, int64_t M, int64_t N, int64_t K) {
  Plan p;
  if (make_plan(type, M, N, K, 0, &p) != MM_OK) return 0;
  return p.ws_bytes;
}

size_t mm_debug_workspace_size(int type, int64_t M, int64_t N, int64_t K, int variant) {
  Plan p;
  if (make_plan(type, M, N, K, variant, &p) != MM_OK) return 0;
  return p.ws_bytes;
}

int64_t mm_row_bytes(int type, int64_t K) { return row_bytes(type, K); }

mm_status mm_dispatch(int type, int64_t M, int64_t N, int64_t K, int* out) {
  Plan p;
  const int st = make_plan(type, M, N, K, 0, &p);
  if (st != MM_OK) return as_status(st);
  if (out) {
    out[0] = p.variant;
    out[1] = p.split;
    const bool tiled = p.variant == 2;
    out[2] = tiled ? p.bm : p.mt;
    out[3] = tiled ? p.bn : p.variant == 3 ? p.waves : p.kind == KK_Q4_NARROW && p.fuse ? p.fuse_rpw : p.rpw;
    const bool q4 = p.type == MM_TYPE_Q4_0 || p.type == MM_TYPE_Q4_0R || p.type == MM_TYPE_Q8_0;
    // INIT (quantized kinds, unless fused), the src1 pre-pass of the wide
    // F16 kernel, the product, the split-K reduce
    const int init = (q4 && !(p.kind == KK_Q4_NARROW && p.fuse)) ? 1 : 0;
    const int pre = p.kind == KK_F16_WIDE ? 1 : 0;
    out[4] = init + pre + 1 + (p.split > 1 ? 1 : 0);
  }
  return MM_OK;
}

mm_status mm_debug_mul_mat(int type, const void* src0, const float* src1, float* dst, int32_t* dots,
                           int64_t M, int64_t N, int64_t K, int64_t n0, int64_t n1, int variant,
                           void* ws, size_t ws_bytes, void* stream) {
  if (variant < 0 || variant > 3) return MM_ERR_ARG;
  if (n0 < 0 || n1 < n0 || n1 > N) return MM_ERR_SHAPE;
  if ((type != MM_TYPE_Q4_0 && type != MM_TYPE_Q4_0R && type != MM_TYPE_Q8_0) || n1 == n0)
    dots = nullptr;
  else if (!dots) return MM_ERR_NULL;
  if (type == MM_TYPE_Q8_0 && dots) {
    // Q8_0 weights: only the wide kernel writes block dots
    Plan p;
    const int st = make_plan(type, M, N, K, variant, &p);
    if (st != MM_OK) return as_status(st);
    if (p.kind == KK_Q4_NARROW) return MM_ERR_ARG;
  }
  return as_status(
      mul_mat(type, src0, src1, dst, dots, M, N, K, n0, n1, variant, ws, ws_bytes, stream));
}

const char* mm_status_string(int status) {
  switch (status) {
    case MM_OK: return "ok";
    case MM_ERR_NULL: return "a required pointer is NULL";
    case MM_ERR_SHAPE: return "invalid shape (negative size, K not a multiple of 32 for a block type, or too large)";
    case MM_ERR_ALIGN: return "pointer not aligned as required";
    case MM_ERR_WORKSPACE:
      return "workspace missing or smaller than mm_mul_mat_workspace_size() (for "
             "mm_mul_mat_q4_0_f32_noalloc: the shape needs more than its fixed 64 MiB array)";
    case MM_ERR_ALIAS: return "output or workspace overlaps another operand";
    case MM_ERR_DEVICE: return "current device is not gfx950 (MI355X)";
    case MM_ERR_HIP: return "HIP runtime error";
    case MM_ERR_ARG: return "unknown type or variant";
    default: return "unknown status";
  }
}

}  // extern "C"
