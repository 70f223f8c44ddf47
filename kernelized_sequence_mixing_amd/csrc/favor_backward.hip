// The FAVOR+ pieces of the backward pass ("Choosing the Feature Map phi",
// "Linear Attention Mechanisms" (dileepadev.github.io): positive random
// features phi(x)_m = exp(w_m . x - |x|^2/2) / sqrt(r)).
//
// la_backward runs FAVOR+ in three steps: the features of the queries and
// keys are materialised as bf16 [rows][r] (favor_features), the chunked
// backward kernels run on them as precomputed features (normalised read-out,
// phi' = 1), which gives dphi for every query and key, and favor_vjp takes
// those back through the feature map:
//   d phi_m / dx = phi_m (w_m - x)  =>  dx = sum_m u_m w_m - x sum_m u_m,  u_m = dphi_m phi_m.
#include "vec_common.hpp"

namespace la {

// phi of `rows` rows of X (in_dt) as bf16 [rows][R]: 64 rows per workgroup,
// 16 at a time staged in LDS, fp32 arithmetic, one rounding.
template <int R, int DK>
__global__ __launch_bounds__(256) void favor_features_kernel(const void* __restrict__ X, int in_dt, long long rows,
                                                             const void* __restrict__ omega,
                                                             bf16* __restrict__ out) {
  constexpr int TR = 16;
  __shared__ float sx[TR * DK];
  __shared__ float sphi[TR * R];
  __shared__ float shalf[TR];
  const int tid = threadIdx.x;
  const long long r_begin = (long long)blockIdx.x * 64;
  for (int sub = 0; sub < 64; sub += TR) {
    const long long row0 = r_begin + sub;
    if (row0 >= rows) break;
    const int nv = int(min((long long)TR, rows - row0));
    __syncthreads();
    for (int idx = tid; idx < TR * DK; idx += 256) {
      const int t = idx / DK;
      sx[idx] = t < nv ? ld_elem(X, (row0 + t) * DK + idx % DK, in_dt) : 0.f;
    }
    __syncthreads();
    half_sq_rows<DK>(sx, shalf, TR, tid, 256);
    __syncthreads();
    phi_rows<R, DK, 1>(sx, sphi, shalf, TR, nv, omega, in_dt, tid, 256);
    __syncthreads();
    for (int idx = tid; idx < nv * R; idx += 256) out[(row0 + idx / R) * R + idx % R] = (bf16)sphi[idx];
  }
}

// dX [rows][DK] (out_dt) from dphi and phi (bf16 [rows][R]) and X:
// dx_d = sum_m u_m w_md - x_d sum_m u_m with u_m = dphi_m phi_m (fp32). omega
// sits in LDS as fp32; 16 rows per pass, each thread four outputs, each a dot
// over the R features.
template <int R, int DK>
__global__ __launch_bounds__(256) void favor_vjp_kernel(const bf16* __restrict__ dphi, const bf16* __restrict__ phi,
                                                        const void* __restrict__ X, int in_dt, long long rows,
                                                        const void* __restrict__ omega, void* __restrict__ dX,
                                                        int out_dt) {
  constexpr int TR = 16;
  extern __shared__ __attribute__((aligned(16))) float vjp_sm[];
  float* som = vjp_sm;           // [R][DK]
  float* su = som + R * DK;      // [TR][R]
  float* ssum = su + TR * R;     // [TR]
  const int tid = threadIdx.x;
  for (int idx = tid; idx < R * DK; idx += 256) som[idx] = ld_elem(omega, idx, in_dt);
  const long long r_begin = (long long)blockIdx.x * 64;
  for (int sub = 0; sub < 64; sub += TR) {
    const long long row0 = r_begin + sub;
    if (row0 >= rows) break;
    const int nv = int(min((long long)TR, rows - row0));
    __syncthreads();
    for (int idx = tid; idx < TR * R; idx += 256) {
      const int t = idx / R;
      su[idx] = t < nv ? to_f32(dphi[(row0 + t) * R + idx % R]) * to_f32(phi[(row0 + t) * R + idx % R]) : 0.f;
    }
    __syncthreads();
    if (tid < TR) {
      float sacc = 0.f;
      for (int m = 0; m < R; ++m) sacc += su[tid * R + m];  // fixed order
      ssum[tid] = sacc;
    }
    __syncthreads();
    for (int idx = tid; idx < nv * DK; idx += 256) {
      const int t = idx / DK, d = idx % DK;
      float acc = 0.f;
      for (int m = 0; m < R; ++m) acc += su[t * R + m] * som[m * DK + d];
      const float x = ld_elem(X, (row0 + t) * DK + d, in_dt);
      st_elem(dX, (row0 + t) * DK + d, out_dt, acc - x * ssum[t]);
    }
  }
}

template <int R, int DK>
static la_status run_favor_features(const void* X, int in_dt, long long rows, const void* omega, void* out,
                                    hipStream_t st) {
  const long long blocks = (rows + 63) / 64;
  LA_LAUNCH((favor_features_kernel<R, DK>), dim3(unsigned(blocks)), dim3(256), 0, st, X, in_dt, rows, omega,
            static_cast<bf16*>(out));
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

template <int R, int DK>
static la_status run_favor_vjp(const void* dphi, const void* phi, const void* X, int in_dt, long long rows,
                               const void* omega, void* dX, int out_dt, hipStream_t st) {
  const long long blocks = (rows + 63) / 64;
  constexpr int lds = (R * DK + 16 * R + 16) * 4;
  auto k = favor_vjp_kernel<R, DK>;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, lds) !=
      hipSuccess)
    return LA_ERR_HIP;
  LA_LAUNCH(k, dim3(unsigned(blocks)), dim3(256), lds, st, static_cast<const bf16*>(dphi),
            static_cast<const bf16*>(phi), X, in_dt, rows, omega, dX, out_dt);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

// Built: r in {64, 128} (the backward kernels' feature widths), d_k in {32, 64, 128}.
#define LA_FAVOR_BWD_DISPATCH(FN, ...)                        \
  switch (r * 1000 + dk) {                                    \
    case 64032: return FN<64, 32>(__VA_ARGS__);               \
    case 64064: return FN<64, 64>(__VA_ARGS__);               \
    case 64128: return FN<64, 128>(__VA_ARGS__);              \
    case 128032: return FN<128, 32>(__VA_ARGS__);             \
    case 128064: return FN<128, 64>(__VA_ARGS__);             \
    case 128128: return FN<128, 128>(__VA_ARGS__);            \
  }                                                           \
  return LA_ERR_UNSUPPORTED;

la_status launch_favor_features(const void* X, int in_dt, long long rows, int dk, int r, const void* omega, void* out,
                                hipStream_t st) {
  LA_FAVOR_BWD_DISPATCH(run_favor_features, X, in_dt, rows, omega, out, st)
}

la_status launch_favor_vjp(const void* dphi, const void* phi, const void* X, int in_dt, long long rows, int dk, int r,
                           const void* omega, void* dX, int out_dt, hipStream_t st) {
  LA_FAVOR_BWD_DISPATCH(run_favor_vjp, dphi, phi, X, in_dt, rows, omega, dX, out_dt, st)
}

}  // namespace la
