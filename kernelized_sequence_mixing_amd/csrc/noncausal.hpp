// Pass 1 of the non-causal form, shared by its forward and backward passes:
// each workgroup (grid: splits x heads) sums phi(k_j) v_j^T and phi(k_j) over
// its slice of the sequence in 32-token tiles, in fp32 on the vector ALUs, and
// writes the slice's partial S and z.
#pragma once

#include "vec_common.hpp"

namespace la {

constexpr int kNcTile = 32;

template <int R, int E, int DK, int FMAP>
__global__ __launch_bounds__(256) void nc_partial(const void* __restrict__ K, const void* __restrict__ V,
                                                  const void* __restrict__ omega, int in_dt, int n, int split_len,
                                                  int splits, float* __restrict__ wsS, float* __restrict__ wsz) {
  __shared__ float sx[kNcTile * DK];
  __shared__ float sphi[kNcTile * R];
  __shared__ float sv[kNcTile * E];
  __shared__ float shalf[kNcTile];
  constexpr int PER = (R * E) / 256;
  const int tid = threadIdx.x;
  const int sp = blockIdx.x;
  const long long bh = blockIdx.y;
  const int t_begin = sp * split_len, t_end = min(n, t_begin + split_len);
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  float zacc = 0.f;
  for (int t0 = t_begin; t0 < t_end; t0 += kNcTile) {
    const int nv = min(kNcTile, t_end - t0);
    for (int idx = tid; idx < kNcTile * DK; idx += 256) {
      const int t = idx / DK;
      sx[idx] = t < nv ? ld_elem(K, (bh * n + t0 + t) * DK + idx % DK, in_dt) : 0.f;
    }
    for (int idx = tid; idx < kNcTile * E; idx += 256) {
      const int t = idx / E;
      sv[idx] = t < nv ? ld_elem(V, (bh * n + t0 + t) * E + idx % E, in_dt) : 0.f;
    }
    __syncthreads();
    if constexpr (FMAP == 1) {
      half_sq_rows<DK>(sx, shalf, kNcTile, tid, 256);
      __syncthreads();
    }
    phi_rows<R, DK, FMAP>(sx, sphi, shalf, kNcTile, nv, omega, in_dt, tid, 256);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = tid + 256 * j, r = idx / E, e = idx % E;
      float a = acc[j];
      for (int t = 0; t < kNcTile; ++t) a += sphi[t * R + r] * sv[t * E + e];
      acc[j] = a;
    }
    if (tid < R)
      for (int t = 0; t < kNcTile; ++t) zacc += sphi[t * R + tid];
    __syncthreads();
  }
  const long long slot = bh * splits + sp;
#pragma unroll
  for (int j = 0; j < PER; ++j) wsS[slot * R * E + tid + 256 * j] = acc[j];
  if (tid < R) wsz[slot * R + tid] = zacc;
}

}  // namespace la
