// Non-causal kernelized linear attention in fp32 on the vector ALUs:
//   S = sum_j phi(k_j) v_j^T,  z = sum_j phi(k_j),  o_i = phi(q_i)^T S / (phi(q_i)^T z + eps)
// ("The linear attention trick: drop or approximate the softmax",
// "Linear Attention Mechanisms" (sadullah.online): the sums are formed once and
// reused by every query, never building the n x n matrix).
//
// Pass 1 (grid: splits x heads): each workgroup sums phi(k_j) v_j^T over its
// slice of the sequence in 32-token tiles. Pass 2 (grid: 64-token blocks x
// heads): adds the slices' partial sums in a fixed order, then reads out.
#include "noncausal.hpp"

namespace la {

template <int R, int E, int DK, int FMAP>
__global__ __launch_bounds__(256) void nc_readout(const void* __restrict__ Q, const void* __restrict__ omega,
                                                  int in_dt, int out_dt, int n, int splits, float eps,
                                                  const float* __restrict__ wsS, const float* __restrict__ wsz,
                                                  void* __restrict__ out, float* __restrict__ S_final,
                                                  float* __restrict__ z_final) {
  constexpr int TQ = 16;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* sS = reinterpret_cast<float*>(smem);  // [R][E]
  float* sz = sS + R * E;                       // [R]
  float* sx = sz + R;                           // [TQ][DK]
  float* sphi = sx + TQ * DK;                   // [TQ][R]
  float* shalf = sphi + TQ * R;                 // [TQ]
  const int tid = threadIdx.x;
  const long long bh = blockIdx.y;
  for (int idx = tid; idx < R * E; idx += 256) {
    float a = 0.f;
    for (int sp = 0; sp < splits; ++sp) a += wsS[(bh * splits + sp) * R * E + idx];
    sS[idx] = a;
    if (S_final != nullptr && blockIdx.x == 0) S_final[bh * R * E + idx] = a;
  }
  if (tid < R) {
    float a = 0.f;
    for (int sp = 0; sp < splits; ++sp) a += wsz[(bh * splits + sp) * R + tid];
    sz[tid] = a;
    if (z_final != nullptr && blockIdx.x == 0) z_final[bh * R + tid] = a;
  }
  const int b_begin = blockIdx.x * 64, b_end = min(n, b_begin + 64);
  for (int t0 = b_begin; t0 < b_end; t0 += TQ) {
    const int nv = min(TQ, b_end - t0);
    __syncthreads();
    for (int idx = tid; idx < TQ * DK; idx += 256) {
      const int t = idx / DK;
      sx[idx] = t < nv ? ld_elem(Q, (bh * n + t0 + t) * DK + idx % DK, in_dt) : 0.f;
    }
    __syncthreads();
    if constexpr (FMAP == 1) {
      half_sq_rows<DK>(sx, shalf, TQ, tid, 256);
      __syncthreads();
    }
    phi_rows<R, DK, FMAP>(sx, sphi, shalf, TQ, nv, omega, in_dt, tid, 256);
    __syncthreads();
    for (int idx = tid; idx < TQ * E; idx += 256) {
      const int t = idx / E, e = idx % E;
      if (t >= nv) continue;
      float num = 0.f, den = 0.f;
      for (int r = 0; r < R; ++r) {
        const float p = sphi[t * R + r];
        num += p * sS[r * E + e];
        den += p * sz[r];
      }
      st_elem(out, (bh * n + t0 + t) * E + e, out_dt, num / (den + eps));
    }
  }
}

template <int R, int E, int DK, int FMAP>
static la_status run_nc(const FwdPlan& p) {
  const unsigned BH = unsigned(p.B) * unsigned(p.H);
  LA_LAUNCH((nc_partial<R, E, DK, FMAP>), dim3(p.splits, BH), dim3(256), 0, p.stream, p.K, p.V, p.omega,
                     p.in_dtype, p.n, p.split_len, p.splits, p.ws_S, p.ws_z);
  if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
  constexpr int lds = (R * E + R + 16 * DK + 16 * R + 16) * 4;
  auto k2 = nc_readout<R, E, DK, FMAP>;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k2), hipFuncAttributeMaxDynamicSharedMemorySize, lds) !=
      hipSuccess)
    return LA_ERR_HIP;
  LA_LAUNCH(k2, dim3((p.n + 63) / 64, BH), dim3(256), lds, p.stream, p.Q, p.omega, p.in_dtype,
                     p.out_dtype, p.n, p.splits, p.eps, p.ws_S, p.ws_z, p.out, p.S_final, p.z_final);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

template <int R, int DK, int FMAP>
static la_status nc_by_dv(const FwdPlan& p) {
  switch (p.dv) {
    case 32: return run_nc<R, 32, DK, FMAP>(p);
    case 64: return run_nc<R, 64, DK, FMAP>(p);
    case 128:
      if constexpr (R * 128 <= 16384) return run_nc<R, 128, DK, FMAP>(p);
      break;
  }
  return LA_ERR_UNSUPPORTED;
}

template <int R>
static la_status nc_favor_by_dk(const FwdPlan& p) {
  switch (p.dk) {
    case 32: return nc_by_dv<R, 32, 1>(p);
    case 64: return nc_by_dv<R, 64, 1>(p);
    case 128: return nc_by_dv<R, 128, 1>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

la_status launch_noncausal(const FwdPlan& p) {
  if (p.fmap == LA_FMAP_ELU1) {
    switch (p.dk) {
      case 32: return nc_by_dv<32, 32, 0>(p);
      case 64: return nc_by_dv<64, 64, 0>(p);
      case 128: return nc_by_dv<128, 128, 0>(p);
    }
    return LA_ERR_UNSUPPORTED;
  }
  switch (p.r) {
    case 32: return nc_favor_by_dk<32>(p);
    case 64: return nc_favor_by_dk<64>(p);
    case 128: return nc_favor_by_dk<128>(p);
    case 256: return nc_favor_by_dk<256>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

}  // namespace la
