// Gradients of the non-causal form in fp32 on the vector ALUs. With the sums
// S = sum_j phi(k_j) v_j^T and z = sum_j phi(k_j) of "The linear attention
// trick" ("Linear Attention Mechanisms", sadullah.online) and an incoming
// gradient dO:
//   den_i = phi(q_i).z + eps,  o_i = phi(q_i)^T S / den_i,
//   g_i = dO_i / den_i,  h_i = -(dO_i . o_i) / den_i,
//   dphi(q_i) = S g_i + z h_i,
//   G = sum_i phi(q_i) g_i^T,  hq = sum_i phi(q_i) h_i,
//   dphi(k_j) = G v_j + hq,  dv_j = G^T phi(k_j),
// then elu+1's derivative (1 above zero, exp(x) = phi below). Like the forward,
// nothing n x n is formed: pass 1 is the forward's partial-sum kernel, pass 2
// (per split of the sequence) reduces S, z in a fixed order, writes dQ and
// the split's partial G, hq; pass 3 reduces those and writes dK, dV.
#include "noncausal.hpp"

namespace la {

namespace {

constexpr int kTB = 16;  // tokens per tile

// The sum over `splits` partial [R][E] blocks (and [R] vectors) of this head
// into LDS, in split order.
template <int R, int E>
__device__ __forceinline__ void reduce_partials(const float* __restrict__ wM, const float* __restrict__ wv,
                                                long long bh, int splits, float* sM, float* sv, int tid) {
  for (int idx = tid; idx < R * E; idx += 256) {
    float a = 0.f;
    for (int sp = 0; sp < splits; ++sp) a += wM[(bh * splits + sp) * R * E + idx];
    sM[idx] = a;
  }
  if (tid < R) {
    float a = 0.f;
    for (int sp = 0; sp < splits; ++sp) a += wv[(bh * splits + sp) * R + tid];
    sv[tid] = a;
  }
}

// Pass 2: dQ for this split's tokens, and the split's partial G, hq.
template <int R, int E, int DK>
__global__ __launch_bounds__(256) void ncb_query(const void* __restrict__ Q, const void* __restrict__ dO, int dt,
                                                 int n, int split_len, int splits, float eps,
                                                 const float* __restrict__ wsS, const float* __restrict__ wsz,
                                                 float* __restrict__ wsG, float* __restrict__ wsh,
                                                 void* __restrict__ dQ) {
  static_assert(R == DK, "elementwise feature map");
  constexpr int PER = (R * E) / 256;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* sS = reinterpret_cast<float*>(smem);  // [R][E]
  float* sz = sS + R * E;                       // [R]
  float* sx = sz + R;                           // [kTB][DK] q
  float* sphi = sx + kTB * DK;                  // [kTB][R]
  float* sdo = sphi + kTB * R;                  // [kTB][E] dO, then g
  float* so = sdo + kTB * E;                    // [kTB][E] o
  float* sden = so + kTB * E;                   // [kTB]
  float* sh = sden + kTB;                       // [kTB]
  const int tid = threadIdx.x;
  const long long bh = blockIdx.y;
  reduce_partials<R, E>(wsS, wsz, bh, splits, sS, sz, tid);
  float gacc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) gacc[j] = 0.f;
  float hacc = 0.f;
  const int t_begin = blockIdx.x * split_len, t_end = min(n, t_begin + split_len);
  for (int t0 = t_begin; t0 < t_end; t0 += kTB) {
    const int nv = min(kTB, t_end - t0);
    __syncthreads();
    for (int idx = tid; idx < kTB * DK; idx += 256) {
      const int t = idx / DK;
      sx[idx] = t < nv ? ld_elem(Q, (bh * n + t0 + t) * DK + idx % DK, dt) : 0.f;
    }
    for (int idx = tid; idx < kTB * E; idx += 256) {
      const int t = idx / E;
      sdo[idx] = t < nv ? ld_elem(dO, (bh * n + t0 + t) * E + idx % E, dt) : 0.f;
    }
    __syncthreads();
    phi_rows<R, DK, 0>(sx, sphi, nullptr, kTB, nv, nullptr, dt, tid, 256);
    __syncthreads();
    // den and o
    for (int idx = tid; idx < kTB * E; idx += 256) {
      const int t = idx / E, e = idx % E;
      float num = 0.f, den = 0.f;
      for (int r = 0; r < R; ++r) {
        const float p = sphi[t * R + r];
        num += p * sS[r * E + e];
        den += p * sz[r];
      }
      den += eps;
      const bool ok = t < nv;  // rows past the end: o = 0, den = 1 (their dO is 0)
      so[idx] = ok ? num / den : 0.f;
      if (e == 0) sden[t] = ok ? den : 1.f;
    }
    __syncthreads();
    // h = -(dO . o) / den, then g = dO / den in place (rows past the end: dO = 0)
    if (tid < kTB) {
      float d = 0.f;
      for (int e = 0; e < E; ++e) d += sdo[tid * E + e] * so[tid * E + e];
      sh[tid] = -d / sden[tid];
    }
    __syncthreads();
    for (int idx = tid; idx < kTB * E; idx += 256) sdo[idx] = sdo[idx] / sden[idx / E];
    __syncthreads();
    // dphi(q) = S g + z h, times phi'(q)
    for (int idx = tid; idx < kTB * R; idx += 256) {
      const int t = idx / R, r = idx % R;
      if (t >= nv) continue;
      float a = sz[r] * sh[t];
      for (int e = 0; e < E; ++e) a += sS[r * E + e] * sdo[t * E + e];
      st_elem(dQ, (bh * n + t0 + t) * DK + r, dt, a * fminf(sphi[t * R + r], 1.f));
    }
    // the split's G += phi(q) g^T and hq += phi(q) h (rows past the end have phi = 0)
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = tid + 256 * j, r = idx / E, e = idx % E;
      float a = gacc[j];
      for (int t = 0; t < kTB; ++t) a += sphi[t * R + r] * sdo[t * E + e];
      gacc[j] = a;
    }
    if (tid < R)
      for (int t = 0; t < kTB; ++t) hacc += sphi[t * R + tid] * sh[t];
  }
  const long long slot = bh * splits + blockIdx.x;
#pragma unroll
  for (int j = 0; j < PER; ++j) wsG[slot * R * E + tid + 256 * j] = gacc[j];
  if (tid < R) wsh[slot * R + tid] = hacc;
}

// Pass 3: dK and dV for this split's tokens from the reduced G, hq.
template <int R, int E, int DK>
__global__ __launch_bounds__(256) void ncb_key(const void* __restrict__ K, const void* __restrict__ V, int dt, int n,
                                               int split_len, int splits, const float* __restrict__ wsG,
                                               const float* __restrict__ wsh, void* __restrict__ dK,
                                               void* __restrict__ dV) {
  static_assert(R == DK, "elementwise feature map");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* sG = reinterpret_cast<float*>(smem);  // [R][E]
  float* shq = sG + R * E;                      // [R]
  float* sx = shq + R;                          // [kTB][DK] k
  float* sphi = sx + kTB * DK;                  // [kTB][R]
  float* sv = sphi + kTB * R;                   // [kTB][E]
  const int tid = threadIdx.x;
  const long long bh = blockIdx.y;
  reduce_partials<R, E>(wsG, wsh, bh, splits, sG, shq, tid);
  const int t_begin = blockIdx.x * split_len, t_end = min(n, t_begin + split_len);
  for (int t0 = t_begin; t0 < t_end; t0 += kTB) {
    const int nv = min(kTB, t_end - t0);
    __syncthreads();
    for (int idx = tid; idx < kTB * DK; idx += 256) {
      const int t = idx / DK;
      sx[idx] = t < nv ? ld_elem(K, (bh * n + t0 + t) * DK + idx % DK, dt) : 0.f;
    }
    for (int idx = tid; idx < kTB * E; idx += 256) {
      const int t = idx / E;
      sv[idx] = t < nv ? ld_elem(V, (bh * n + t0 + t) * E + idx % E, dt) : 0.f;
    }
    __syncthreads();
    phi_rows<R, DK, 0>(sx, sphi, nullptr, kTB, nv, nullptr, dt, tid, 256);
    __syncthreads();
    for (int idx = tid; idx < kTB * R; idx += 256) {
      const int t = idx / R, r = idx % R;
      if (t >= nv) continue;
      float a = shq[r];
      for (int e = 0; e < E; ++e) a += sG[r * E + e] * sv[t * E + e];
      st_elem(dK, (bh * n + t0 + t) * DK + r, dt, a * fminf(sphi[t * R + r], 1.f));
    }
    for (int idx = tid; idx < kTB * E; idx += 256) {
      const int t = idx / E, e = idx % E;
      if (t >= nv) continue;
      float a = 0.f;
      for (int r = 0; r < R; ++r) a += sG[r * E + e] * sphi[t * R + r];
      st_elem(dV, (bh * n + t0 + t) * E + e, dt, a);
    }
  }
}

template <int R, int E>
la_status run_nc_backward(const BwdPlan& p) {
  const unsigned BH = unsigned(p.B) * unsigned(p.H);
  LA_LAUNCH((nc_partial<R, E, R, 0>), dim3(p.splits, BH), dim3(256), 0, p.stream, p.K, p.V, nullptr,
                     p.in_dtype, p.n, p.split_len, p.splits, p.ws_S, p.ws_z);
  if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
  constexpr int lds2 = (R * E + R + kTB * R + kTB * R + 2 * kTB * E + 2 * kTB) * 4;
  auto k2 = ncb_query<R, E, R>;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k2), hipFuncAttributeMaxDynamicSharedMemorySize, lds2) !=
      hipSuccess)
    return LA_ERR_HIP;
  LA_LAUNCH(k2, dim3(p.splits, BH), dim3(256), lds2, p.stream, p.Q, p.dO, p.in_dtype, p.n, p.split_len,
                     p.splits, p.eps, p.ws_S, p.ws_z, p.ws_R, p.ws_rh, p.dQ);
  if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
  constexpr int lds3 = (R * E + R + kTB * R + kTB * R + kTB * E) * 4;
  auto k3 = ncb_key<R, E, R>;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k3), hipFuncAttributeMaxDynamicSharedMemorySize, lds3) !=
      hipSuccess)
    return LA_ERR_HIP;
  LA_LAUNCH(k3, dim3(p.splits, BH), dim3(256), lds3, p.stream, p.K, p.V, p.in_dtype, p.n, p.split_len,
                     p.splits, p.ws_R, p.ws_rh, p.dK, p.dV);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

template <int R>
la_status nc_backward_by_dv(const BwdPlan& p) {
  switch (p.dv) {
    case 32: return run_nc_backward<R, 32>(p);
    case 64: return run_nc_backward<R, 64>(p);
    case 128:
      if constexpr (R * 128 <= 16384) return run_nc_backward<R, 128>(p);
      break;
  }
  return LA_ERR_UNSUPPORTED;
}

}  // namespace

la_status launch_noncausal_backward(const BwdPlan& p) {
  if (p.fmap != LA_FMAP_ELU1) return LA_ERR_UNSUPPORTED;
  switch (p.r) {
    case 32: return nc_backward_by_dv<32>(p);
    case 64: return nc_backward_by_dv<64>(p);
    case 128: return nc_backward_by_dv<128>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

}  // namespace la
