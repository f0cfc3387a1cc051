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

// Sum over the 64 lanes of a wave with DPP row operations (no LDS traffic);
// the total lands in lane 63 and is returned to every lane through
// v_readlane.  Order: pairs, quads, half rows, rows (quad_perm / mirrors),
// then row 0+1 and 2+3 (row_bcast15), then all (row_bcast31) -- fixed, so
// the result is deterministic.
// Lane permutations within rows of 16 lanes (DPP); every source lane valid.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, false));
}
template <int kCtrl>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xf, 0xf, false);
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, kRowMask, 0xf, false);
  return v + __builtin_bit_cast(float, moved);
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = dpp_add<0xB1, 0xf>(v);    // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xf>(v);    // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xf>(v);   // row_half_mirror
  v = dpp_add<0x140, 0xf>(v);   // row_mirror: every lane holds its row's sum
  v = dpp_add<0x142, 0xa>(v);   // row_bcast15 into rows 1 and 3
  v = dpp_add<0x143, 0xc>(v);   // row_bcast31 into rows 2 and 3: lane 63 = total
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Round half away from zero of an fp32 value with |v| < 2^31, as
// trunc(fl32(v + copysign(0.5 - 2^-25, v))) (v_cvt_i32_f32 truncates).
// Equal to roundf for every float32 |v| <= 130 (checked exhaustively: the
// only values where adding 0.5 itself would round up across an integer lie
// just below 0.5, and the slightly smaller addend keeps them below 1).
__device__ __forceinline__ int round_half_away(float v) {
#pragma clang fp contract(off)
  const float c = __builtin_bit_cast(float, 0x3effffffu);   // 0.5 - 2^-25
  return (int)(v + __builtin_copysignf(c, v));
}

// Q8_0 of one 32-value block held by a pair of adjacent lanes (even lane:
// values 0..15, odd lane: values 16..31): amax over the block, d = amax/127
// (correctly rounded), id = 1/d (correctly rounded; 0 when d == 0), q = round
// half away from zero of fl32(x * id).  Returns this lane's 16 codes packed
// little endian, the fp16 bits of d and the block's code sum (both lanes).
// Both lanes of the pair must execute this together.
__device__ __forceinline__ void q8_0_pair(const float (&v)[16], uint32_t (&packed)[4],
                                          uint32_t& dbits, int& sum) {
#pragma clang fp contract(off)
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, dpp_f<0xB1>(amax));             // the other lane of the pair
  const float d = amax / 127.0f;
  const float id = d != 0.0f ? 1.0f / d : 0.0f;
  int s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) w |= (uint32_t)(round_half_away(v[4 * j + e] * id) & 0xff) << (8 * e);
    packed[j] = w;
    s = __builtin_amdgcn_sdot4((int)w, 0x01010101, s, false);   // sum of the 4 signed codes
  }
  s += dpp_i<0xB1>(s);
  sum = s;
  dbits = f32_to_f16_bits(d);
}

// Dispatch places workgroup i on XCD i % 8.  Give each XCD a contiguous run
// of tile ids, so tiles that share an operand tile share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  const int per = total / 8, rem = total % 8;
  const int x = id % 8, k = id / 8;
  return x * per + (x < rem ? x : rem) + k;
}

// Barrier for LDS data only: waits for this wave's LDS writes, not for its
// outstanding global loads (which may still be streaming weights in).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace qsg
