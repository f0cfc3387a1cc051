// Skinny Q4_0 x Q8_0 product on int8 MFMA for small batches (2 < M <= 32
// per pass).
//
// dst[m][n] = sum_b f32(d_w[n][b]) * f32(d_a[m][b]) * S_b[m][n],
// S_b = sum_j (q4 - 8) * q8 (int32).
//
// With a few src1 rows the product is still bound by reading the weights
// once (arXiv 2407.07304, section 2.2; DeepSpeed-Inference notes, III.A),
// but per weight byte it does M times the dot-product work of the M = 1
// kernel, more than the vector ALU keeps up with from M of about 8 on.  The
// int32 block dots therefore go to the matrix cores: v_mfma_i32_32x32x32_i8
// has K = 32, exactly one Q4_0 / Q8_0 block, so each MFMA output is one block
// dot S_b and takes one scale pair.
//
//   * A workgroup owns 32 weight rows (the MFMA's N).  It walks their K range
//     in chunks of 32 blocks: the chunk's 32 x 576 bytes are read with
//     coalesced loads (consecutive lanes, consecutive bytes of a row) and
//     written to LDS, double buffered, with the next chunks' loads in flight
//     while the current one is computed.  (Loading the MFMA operands straight
//     from HBM would put every lane of an instruction in a different row:
//     many more memory requests per byte.)
//   * Each of the W waves takes 4 blocks of the chunk.  Lane l feeds weight
//     row l % 32 and the half h = l / 32 of every block: elements
//     16h .. 16h+15, i.e. the low (h = 0) or high (h = 1) nibbles of the
//     block's 16 code bytes.  The A operand (Q8_0 codes of src1 row l % 32 of
//     the pass, read from the wdata) uses the same element split, so the
//     MFMA sums over the block's 32 elements.
//   * The nibbles stay unsigned (0..15); the MFMA accumulator starts from
//     -8 * sum(q8) of the activation block, so it ends at the signed block
//     dot S_b exactly.
//   * Epilogue per output and block: acc += f32(S_b) * (d_a * d_w), with d_a
//     and the bias of the chunk's blocks staged in LDS beside its weights.
//   * The waves' partial tiles are added in LDS at the end in a fixed order
//     (DeepSpeed-Inference notes, III.C: partial sums reduced on chip); when
//     the 32-row tiles cannot fill the device, K is also split across
//     workgroups and a second kernel adds those partials in a fixed order.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace qsg {

namespace {

constexpr int CB = 32;                  // blocks per LDS chunk
constexpr int ROWB = CB * 18;           // bytes of one row's chunk (576)
constexpr int PITCH = ROWB + 4;         // LDS row pitch: an odd dword count spreads the banks
constexpr int WBUF = 32 * PITCH;        // weights of one chunk (32 rows)

// One LDS chunk buffer: the weights, then d_a and the bias -8*sum(q8) of the
// chunk's blocks for the pass's MT src1 rows as [block][row].
template <int MT>
struct ChunkLds {
  static constexpr int kScaleOff = WBUF;                   // float [CB][MT]
  static constexpr int kBiasOff = WBUF + CB * MT * 4;      // int32 [CB][MT]
  static constexpr int kBytes = WBUF + CB * MT * 8;
  static constexpr int kTotal = 2 * kBytes + 16;           // two buffers + a sink
};

// Global -> register -> LDS copy of one chunk: the workgroup's 32 weight
// rows in pieces of G bytes (16 when rows and chunk starts are 16-byte
// aligned, 4 when they are 4-byte aligned, else 2), and the chunk's
// activation scales and biases.  Thread t copies row t / 16, pieces
// t % 16 + 16k: sixteen consecutive lanes read consecutive bytes of a row,
// and every address is one per-thread base plus a constant.  Loads are
// unconditional (clamped); pieces past the chunk go to a sink.
template <int MT, int G, int NT>
struct Copier {
  static_assert(NT == 512, "32 rows x 16 threads");
  static constexpr int kPerRow = ROWB / G;                  // pieces per row of a chunk
  static constexpr int kPPT = (kPerRow + 15) / 16;          // pieces per thread
  static constexpr int kSPT = (CB * MT + NT - 1) / NT;      // scale items per thread
  typedef typename std::conditional<G == 16, v4i,
                                    typename std::conditional<G == 4, uint32_t, uint16_t>::type>::type T;
  T v[kPPT];
  float d[kSPT];
  int32_t bi[kSPT];

  __device__ __forceinline__ void load(const Q4Args& a, int64_t rb, int n0, int m0, int bstart,
                                       int nbc) {
    const int t = threadIdx.x;
    const int r = t >> 4, cl = t & 15;
    const int valid = nbc * 18 / G;
    const int n = n0 + r < a.N ? n0 + r : a.N - 1;
    const uint8_t* base = a.w + (int64_t)n * rb + (int64_t)bstart * 18;
#pragma unroll
    for (int k = 0; k < kPPT; ++k) {
      const int c = cl + 16 * k;
      const int cc = c < valid ? c : 0;
      const __attribute__((address_space(1))) T* p =
          (const __attribute__((address_space(1))) T*)(base + cc * G);
      v[k] = *p;
    }
    // item k: src1 row t / CB + k * (NT / CB) (rows past MT idle), block
    // t % CB of the chunk
    const int nbt = a.K / 32;
    const int bl = t % CB;
    const int b = bl < nbc ? bstart + bl : bstart;
#pragma unroll
    for (int k = 0; k < kSPT; ++k) {
      const int m = t / CB + k * (NT / CB);
      const int row = m < MT && m0 + m < a.M ? m0 + m : 0;
      const __attribute__((address_space(1))) float* pd =
          (const __attribute__((address_space(1))) float*)(a.ad + (int64_t)row * nbt + b);
      const __attribute__((address_space(1))) int32_t* pb =
          (const __attribute__((address_space(1))) int32_t*)(a.ab + (int64_t)row * nbt + b);
      d[k] = *pd;
      bi[k] = *pb;
    }
  }
  __device__ __forceinline__ void store(uint8_t* buf, uint8_t* sink, int m0, int M, int nbc) const {
    const int t = threadIdx.x;
    const int r = t >> 4, cl = t & 15;
    const int valid = nbc * 18 / G;
    uint8_t* base = buf + r * PITCH;
#pragma unroll
    for (int k = 0; k < kPPT; ++k) {
      const int c = cl + 16 * k;
      uint8_t* dst = c < valid ? base + c * G : sink;
      if constexpr (G == 16) {
        uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);   // PITCH keeps 4-byte alignment
        d32[0] = (uint32_t)v[k].x; d32[1] = (uint32_t)v[k].y;
        d32[2] = (uint32_t)v[k].z; d32[3] = (uint32_t)v[k].w;
      } else {
        *reinterpret_cast<T*>(dst) = v[k];
      }
    }
    float* sd = reinterpret_cast<float*>(buf + ChunkLds<MT>::kScaleOff);
    int32_t* sb = reinterpret_cast<int32_t*>(buf + ChunkLds<MT>::kBiasOff);
    const int bl = t % CB;
#pragma unroll
    for (int k = 0; k < kSPT; ++k) {
      const int m = t / CB + k * (NT / CB);
      if (m < MT) {
        const bool ok = m0 + m < M;                   // rows past M: zero scale and bias
        sd[bl * MT + m] = ok ? d[k] : 0.0f;
        sb[bl * MT + m] = ok ? bi[k] : 0;
      }
    }
  }
};

// Activation codes (this lane's src1 row and half) of 4 blocks b .. b+3,
// each clamped to blast; unconditional loads, inactive lanes masked to 0.
__device__ __forceinline__ void load_a(v4i (&av)[4], const int8_t* arow, int b, int blast,
                                       bool active) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int bi = b + i < blast ? b + i : blast;
    const __attribute__((address_space(1))) v4i* p =
        (const __attribute__((address_space(1))) v4i*)(arow + 32 * (int64_t)bi);
    const v4i v = *p;
    av[i].x = active ? v.x : 0;
    av[i].y = active ? v.y : 0;
    av[i].z = active ? v.z : 0;
    av[i].w = active ? v.w : 0;
  }
}

// Block j of this lane's row in an LDS chunk: fp16 scale bits and the 16
// code bytes as 4 dwords (5 dword reads: the block starts 4-byte aligned for
// even j and 2 bytes past an aligned dword for odd j).
template <int kOdd>
__device__ __forceinline__ void lds_block(const uint8_t* row, int j, uint32_t& dbits,
                                          uint32_t (&q)[4]) {
  constexpr int odd = kOdd;
  const uint32_t* p = reinterpret_cast<const uint32_t*>(row + 18 * j - 2 * odd);
  uint32_t d[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) d[k] = p[k];
  if constexpr (odd) {
    dbits = d[0] >> 16;
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = d[1 + k];
  } else {
    dbits = d[0] & 0xffffu;
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = __builtin_amdgcn_alignbit(d[k + 1], d[k], 16);
  }
}

// One workgroup per CU (the second launch-bounds argument is waves per
// execution unit here): the two chunks in flight, the activation codes of the
// next chunk and the accumulators need more than the 128 VGPRs of two.
template <int MT, int W, int G, bool kDump>
__global__ __launch_bounds__(64 * W, 2)
void k_q4_mma(Q4Args a, int kchunk, int split) {
  static_assert(CB == 4 * W, "each wave takes 4 blocks of a chunk");
  constexpr int NG = MT / 8;                 // accumulator groups of 4 rows that hold src1 rows
  constexpr int NT = 64 * W;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int h = lane >> 5, l32 = lane & 31;
  const int M = a.M, N = a.N, K = a.K;
  const int nb = K / 32;
  const int64_t rb = (int64_t)nb * 18;
  const int n0 = blockIdx.x * 32, m0 = blockIdx.y * MT, z = blockIdx.z;
  // the workgroup's blocks [b0, b1) in chunks of CB
  const int b0 = z * kchunk;
  const int b1 = b0 + kchunk < nb ? b0 + kchunk : nb;
  const int nbr = b1 - b0;
  const int nch = (nbr + CB - 1) / CB;
  auto chunk_blocks = [&](int c) { const int r = nbr - c * CB; return r < CB ? r : CB; };

  constexpr int BUFB = ChunkLds<MT>::kBytes;
  uint8_t* sink = smem + 2 * BUFB;

  const bool aact = l32 < MT && m0 + l32 < M;
  const int8_t* arow = a.aq + (int64_t)(aact ? m0 + l32 : 0) * K + 16 * h;
  const int jw = 4 * wave;                   // this wave's first block in a chunk
  auto next_c = [&](int c) { return c < nch ? c : 0; };

  // chunks 0 and 1 in flight, then the activation codes of chunk 0
  Copier<MT, G, NT> cpa, cpb;
  cpa.load(a, rb, n0, m0, b0, chunk_blocks(0));
  cpb.load(a, rb, n0, m0, b0 + next_c(1) * CB, chunk_blocks(next_c(1)));
  v4i a0[4], a1[4];
  load_a(a0, arow, b0 + jw, b1 - 1, aact);
  cpa.store(smem, sink, m0, M, chunk_blocks(0));
  lds_barrier();

  float acc[NG * 4];
#pragma unroll
  for (int r = 0; r < NG * 4; ++r) acc[r] = 0.0f;

  // Blocks jw .. jw+3 of chunk c from LDS buffer `buf`; a block past the
  // range has its contribution dropped (zero scale: f32(S) * 0 adds a zero).
  auto compute = [&](const uint8_t* buf, const v4i (&ca)[4], int c) {
    const int nbc = chunk_blocks(c);
    const uint8_t* row = buf + l32 * PITCH;
    const float* sd = reinterpret_cast<const float*>(buf + ChunkLds<MT>::kScaleOff);
    const int32_t* sb = reinterpret_cast<const int32_t*>(buf + ChunkLds<MT>::kBiasOff);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = jw + jj;
      const bool live = j < nbc;                      // uniform over the wave
      const int jr = live ? j : (jj & 1);             // same parity: same code path
      uint32_t dbits, q[4];
      if (jj & 1) lds_block<1>(row, jr, dbits, q);
      else lds_block<0>(row, jr, dbits, q);
      // unsigned nibbles of this lane's half: low (h = 0) or high (h = 1)
      const int sh = 4 * h;
      v4i bop;
      bop.x = (int)((q[0] >> sh) & 0x0F0F0F0Fu);
      bop.y = (int)((q[1] >> sh) & 0x0F0F0F0Fu);
      bop.z = (int)((q[2] >> sh) & 0x0F0F0F0Fu);
      bop.w = (int)((q[3] >> sh) & 0x0F0F0F0Fu);
      const float dw = live ? f16_bits_to_f32(dbits) : 0.0f;
      const int bl = jr;                              // block within the chunk
      v16i cc = {};
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const v4i bi = *reinterpret_cast<const v4i*>(sb + bl * MT + 8 * g + 4 * h);
        cc[4 * g + 0] = bi.x; cc[4 * g + 1] = bi.y; cc[4 * g + 2] = bi.z; cc[4 * g + 3] = bi.w;
      }
      const v16i dd = __builtin_amdgcn_mfma_i32_32x32x32_i8(ca[jj], bop, cc, 0, 0, 0);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float4 da = *reinterpret_cast<const float4*>(sd + bl * MT + 8 * g + 4 * h);
        acc[4 * g + 0] = fmaf((float)dd[4 * g + 0], da.x * dw, acc[4 * g + 0]);
        acc[4 * g + 1] = fmaf((float)dd[4 * g + 1], da.y * dw, acc[4 * g + 1]);
        acc[4 * g + 2] = fmaf((float)dd[4 * g + 2], da.z * dw, acc[4 * g + 2]);
        acc[4 * g + 3] = fmaf((float)dd[4 * g + 3], da.w * dw, acc[4 * g + 3]);
      }
      if (kDump && live) {
        const int n = n0 + l32;
        const int b = b0 + c * CB + j;
#pragma unroll
        for (int r = 0; r < NG * 4; ++r) {
          const int m = m0 + 8 * (r / 4) + 4 * h + (r % 4);
          if (m < M && n >= a.n0 && n < a.n1)
            a.dots[((int64_t)m * (a.n1 - a.n0) + (n - a.n0)) * nb + b] = dd[r];
        }
      }
      // one block's MFMA in flight at a time: its 16 result registers are
      // then reused by the next block (the registers hold the loads in
      // flight instead)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Chunk c: load chunk c+2 into the register set just written to LDS and
  // the next chunk's activation codes, compute chunk c, write chunk c+1 to
  // the other LDS buffer (read by every wave two chunks ago, before the last
  // barrier), barrier.  Past the end the loads repeat chunk 0 (valid, never
  // used).
  for (int c = 0; c < nch; c += 2) {
    cpa.load(a, rb, n0, m0, b0 + next_c(c + 2) * CB, chunk_blocks(next_c(c + 2)));
    load_a(a1, arow, b0 + next_c(c + 1) * CB + jw, b1 - 1, aact);
    compute(smem, a0, c);
    if (c + 1 >= nch) break;
    cpb.store(smem + BUFB, sink, m0, M, chunk_blocks(c + 1));
    lds_barrier();
    cpb.load(a, rb, n0, m0, b0 + next_c(c + 3) * CB, chunk_blocks(next_c(c + 3)));
    load_a(a0, arow, b0 + next_c(c + 2) * CB + jw, b1 - 1, aact);
    compute(smem + BUFB, a1, c + 1);
    if (c + 2 >= nch) break;
    cpa.store(smem, sink, m0, M, chunk_blocks(c + 2));
    lds_barrier();
  }

  // ---- add the W waves' partial tiles in a fixed order (LDS reused)
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int r = 0; r < NG * 4; ++r) red[((int64_t)wave * NG * 4 + r) * 64 + lane] = acc[r];
  __syncthreads();
  const int n = n0 + l32;
  float* out = split == 1 ? a.dst : a.part + (int64_t)z * M * N;
  for (int r = wave; r < NG * 4; r += W) {
    float t = 0.0f;
    for (int w2 = 0; w2 < W; ++w2) t += red[((int64_t)w2 * NG * 4 + r) * 64 + lane];
    const int m = m0 + 8 * (r / 4) + 4 * h + (r % 4);
    if (m < M && n < N) out[(int64_t)m * N + n] = t;
  }
}

template <int MT, int W, int G>
hipError_t launch_g(const Plan& p, const Q4Args& a, hipStream_t s) {
  const dim3 grid((unsigned)p.tiles_n, (unsigned)p.tiles_m, (unsigned)p.split);
  const dim3 block(64 * W);
  const size_t stage = (size_t)ChunkLds<MT>::kTotal;
  const size_t red = (size_t)W * (MT / 2) * 64 * 4;
  const size_t lds = stage > red ? stage : red;
  const int kc = (int)p.kchunk;
  if (a.dots) hipLaunchKernelGGL((k_q4_mma<MT, W, G, true>), grid, block, lds, s, a, kc, p.split);
  else hipLaunchKernelGGL((k_q4_mma<MT, W, G, false>), grid, block, lds, s, a, kc, p.split);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(const Plan& p, const Q4Args& a, hipStream_t s) {
  // 16-byte pieces need 16-byte aligned rows (K/32 a multiple of 8, src0
  // 16-byte aligned) and chunk starts (the per-split range is a multiple of
  // 8 blocks); 4-byte pieces need K/32 even and src0 4-byte aligned
  const int nb = a.K / 32;
  if (nb % 8 == 0 && p.kchunk % 8 == 0 && (uintptr_t)a.w % 16 == 0)
    return launch_g<MT, kMmaWaves, 16>(p, a, s);
  if (nb % 2 == 0 && p.kchunk % 2 == 0 && (uintptr_t)a.w % 4 == 0)
    return launch_g<MT, kMmaWaves, 4>(p, a, s);
  return launch_g<MT, kMmaWaves, 2>(p, a, s);
}

}  // namespace

hipError_t launch_q4_mma(const Plan& p, const Q4Args& a, hipStream_t s) {
  // 32 weight rows per workgroup, the whole K range (the plan splits none)
  if (p.split != 1) return hipErrorInvalidValue;
  Plan q = p;
  const int nb = a.K / 32;
  q.tiles_n = (a.N + 31) / 32;
  q.kchunk = (nb + 7) / 8 * 8;
  if (q.mt == 8) return launch_mt<8>(q, a, s);
  if (q.mt == 16) return launch_mt<16>(q, a, s);
  if (q.mt == 32) return launch_mt<32>(q, a, s);
  return hipErrorInvalidValue;
}

}  // namespace qsg
