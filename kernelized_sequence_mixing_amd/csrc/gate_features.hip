// The selective scalar gate in the backward pass. Its recurrence
// S_t = a_t S_{t-1} + phi(k_t) v_t^T is the diagonal gate with the same
// alpha_t on every feature (the dileepadev page, "Gating and Selective State
// Updates": A_t = a_t I), so the gradient passes of the diagonal gate serve
// it: the per-step input g [rows] is repeated over the r features, and the
// per-feature gradient of the repeated input is summed back over features
// (every alpha_tk is the same function of g_t).
#include "common.hpp"
#include "plan.hpp"

namespace la {
namespace {

// gx[row][f] = g[row]; one thread writes 8 features (16 bytes).
__global__ __launch_bounds__(256) void gate_repeat_kernel(const bf16* __restrict__ g, bf16* __restrict__ gx,
                                                          long long rows, int r) {
  const int per_row = r / 8;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * per_row) return;
  const bf16 v = g[i / per_row];
  bf16x8 o;
#pragma unroll
  for (int u = 0; u < 8; ++u) o[u] = v;
  *reinterpret_cast<bf16x8*>(gx + 8 * i) = o;
}

// dg[row] = sum_f dgx[row][f]: r / 8 lanes per row each add 8 features, then
// a butterfly over those lanes (a fixed order: deterministic).
template <int R>
__global__ __launch_bounds__(256) void gate_feature_sum_kernel(const bf16* __restrict__ dgx, bf16* __restrict__ dg,
                                                               long long rows) {
  constexpr int PER = R / 8;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = i / PER;
  float s = 0.f;
  if (row < rows) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(dgx + 8 * i);
#pragma unroll
    for (int u = 0; u < 8; ++u) s += to_f32(x[u]);
  }
#pragma unroll
  for (int m = 1; m < PER; m <<= 1) s += __shfl_xor(s, m);
  if (row < rows && (i % PER) == 0) dg[row] = (bf16)s;
}

}  // namespace

la_status launch_gate_repeat(const void* g, void* gx, long long rows, int r, hipStream_t stream) {
  if (r % 8 != 0 || r > 512) return LA_ERR_UNSUPPORTED;
  const long long threads = rows * (r / 8);
  if (threads == 0) return LA_OK;
  const long long blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return LA_ERR_UNSUPPORTED;
  LA_LAUNCH(gate_repeat_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, static_cast<const bf16*>(g),
                     static_cast<bf16*>(gx), rows, r);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status launch_gate_feature_sum(const void* dgx, void* dg, long long rows, int r, hipStream_t stream) {
  const long long threads = rows * (r / 8);
  if (threads == 0) return LA_OK;
  const long long blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return LA_ERR_UNSUPPORTED;
  const bf16* src = static_cast<const bf16*>(dgx);
  bf16* dst = static_cast<bf16*>(dg);
  if (r == 64)
    LA_LAUNCH(gate_feature_sum_kernel<64>, dim3(unsigned(blocks)), dim3(256), 0, stream, src, dst, rows);
  else if (r == 128)
    LA_LAUNCH(gate_feature_sum_kernel<128>, dim3(unsigned(blocks)), dim3(256), 0, stream, src, dst, rows);
  else
    return LA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // namespace la
