// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace qsg {

// Q8_0 activation quantisation.  Writes the canonical 34-byte blocks to
// `canon` (may be NULL) and/or the library's internal wdata layout
// (codes int8 [rows][k], scales f32 [rows][k/32], bias -8*sum(q) int32
// [rows][k/32]; all NULL to skip).  Also zeroes `zero_words` 32-bit words at
// `zero` (split-K tickets) in the same launch.
hipError_t launch_quantize_q8_0(const float* x, int64_t nrows, int64_t k, uint8_t* canon,
                                int8_t* wq, float* wd, int32_t* wb, uint32_t* zero,
                                int64_t zero_words, hipStream_t s);

hipError_t launch_quantize_q4_0(const float* x, int64_t nrows, int64_t k, uint8_t* y,
                                hipStream_t s);

struct Q4Args {
  const uint8_t* w;      // Q4_0 src0
  const int8_t* aq;      // wdata codes
  const float* ad;       // wdata scales
  const int32_t* ab;     // wdata -8*sum(q)
  float* dst;
  float* part;           // split-K partials [split][M][N]
  uint32_t* tick;        // split-K tickets, one per output tile
  int M, N, K;
  int32_t* dots;         // debug block dots (NULL in production)
  int n0, n1;
};

hipError_t launch_q4_narrow(const Plan& p, const Q4Args& a, hipStream_t s);
hipError_t launch_q4_wide(const Plan& p, const Q4Args& a, hipStream_t s);

hipError_t launch_f_narrow(const Plan& p, int type, const void* w, const float* x, float* dst,
                           int M, int N, int K, hipStream_t s);
hipError_t launch_f16_wide(const Plan& p, const uint16_t* w, const float* x, float* dst,
                           int M, int N, int K, hipStream_t s);
hipError_t launch_zero(float* dst, int64_t n, hipStream_t s);

}  // namespace qsg
