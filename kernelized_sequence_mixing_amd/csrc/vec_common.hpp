// fp32 vector-ALU helpers shared by the non-causal, decode and feature-map
// kernels: typed loads/stores with the dtype chosen at run time (these paths
// are bound by memory or latency, not by the cost of a uniform branch), and
// the feature map of one row staged in LDS.
#pragma once

#include "common.hpp"
#include "plan.hpp"

namespace la {

__device__ __forceinline__ float ld_elem(const void* base, long long i, int dtype) {
  return dtype == LA_BF16 ? to_f32(static_cast<const bf16*>(base)[i]) : static_cast<const float*>(base)[i];
}

__device__ __forceinline__ void st_elem(void* base, long long i, int dtype, float v) {
  if (dtype == LA_BF16)
    static_cast<bf16*>(base)[i] = (bf16)v;
  else
    static_cast<float*>(base)[i] = v;
}

// Feature map of `rows` rows staged in LDS: x [rows][DK] (fp32) -> phi [rows][R].
// `valid(t)` rows only; others get phi = 0. Called by all threads of the block
// (nthreads), followed by a barrier by the caller.
//   elu+1: phi = elu(x) + 1 elementwise (R == DK).
//   FAVOR: phi_m = exp(w_m . x - |x|^2/2) / sqrt(R), w_m read from omega (global).
template <int R, int DK, int FMAP>
__device__ __forceinline__ void phi_rows(const float* sx, float* sphi, const float* shalf, int rows, int nvalid,
                                         const void* omega, int odt, int tid, int nthreads) {
  for (int idx = tid; idx < rows * R; idx += nthreads) {
    const int t = idx / R, m = idx % R;
    float v = 0.f;
    if (t < nvalid) {
      if constexpr (FMAP == 0) {
        v = elu1(sx[t * DK + m]);
      } else {
        float acc = 0.f;
        for (int d = 0; d < DK; ++d) acc += ld_elem(omega, (long long)m * DK + d, odt) * sx[t * DK + d];
        v = __expf(acc - shalf[t]) * rsqrtf(float(R));
      }
    }
    sphi[t * R + m] = v;
  }
}

// |x|^2 / 2 per staged row (FAVOR only); one thread per row.
template <int DK>
__device__ __forceinline__ void half_sq_rows(const float* sx, float* shalf, int rows, int tid, int nthreads) {
  for (int t = tid; t < rows; t += nthreads) {
    float s = 0.f;
    for (int d = 0; d < DK; ++d) s += sx[t * DK + d] * sx[t * DK + d];
    shalf[t] = 0.5f * s;
  }
}

}  // namespace la
