// The feature map alone, fp32 out ("Choosing the Feature Map phi",
// "Linear Attention Mechanisms" (dileepadev.github.io)):
//   elu+1:  phi(x) = elu(x) + 1 elementwise;
//   FAVOR+: phi(x)_m = exp(w_m . x - |x|^2 / 2) / sqrt(r).
// 64 rows per workgroup, staged in LDS.
#include "vec_common.hpp"

namespace la {

template <int R, int DK, int FMAP>
__global__ __launch_bounds__(256) void feature_map_kernel(const void* __restrict__ X, int in_dt, long long rows,
                                                          const void* __restrict__ omega, float* __restrict__ out) {
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
    if constexpr (FMAP == 1) {
      half_sq_rows<DK>(sx, shalf, TR, tid, 256);
      __syncthreads();
    }
    phi_rows<R, DK, FMAP>(sx, sphi, shalf, TR, nv, omega, in_dt, tid, 256);
    __syncthreads();
    for (int idx = tid; idx < nv * R; idx += 256) out[(row0 + idx / R) * R + idx % R] = sphi[idx];
  }
}

template <int R, int DK, int FMAP>
static la_status run_fmap(const FmapPlan& p) {
  const long long blocks = (p.rows + 63) / 64;
  LA_LAUNCH((feature_map_kernel<R, DK, FMAP>), dim3(unsigned(blocks)), dim3(256), 0, p.stream, p.X,
                     p.in_dtype, p.rows, p.omega, p.out);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

template <int R>
static la_status fm_favor_by_dk(const FmapPlan& p) {
  switch (p.dk) {
    case 32: return run_fmap<R, 32, 1>(p);
    case 64: return run_fmap<R, 64, 1>(p);
    case 128: return run_fmap<R, 128, 1>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

la_status launch_feature_map(const FmapPlan& p) {
  if (p.fmap == LA_FMAP_ELU1) {
    switch (p.dk) {
      case 32: return run_fmap<32, 32, 0>(p);
      case 64: return run_fmap<64, 64, 0>(p);
      case 128: return run_fmap<128, 128, 0>(p);
    }
    return LA_ERR_UNSUPPORTED;
  }
  switch (p.r) {
    case 32: return fm_favor_by_dk<32>(p);
    case 64: return fm_favor_by_dk<64>(p);
    case 128: return fm_favor_by_dk<128>(p);
    case 256: return fm_favor_by_dk<256>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

}  // namespace la
