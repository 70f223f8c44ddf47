// Chaining of per-segment states across one head's sequence (fp32):
//   S_in(0) = S0 (or 0),  S_in(s+1) = Gamma_s S_in(s) + dS_s,
// the associativity of the prefix state (the recurrence S_t = G_t S_{t-1} +
// phi(k_t) v_t^T of "Recurrent Reformulation", "Linear Attention Mechanisms",
// dileepadev.github.io, applied one segment at a time). Slot s of the workspace
// holds dS_s on entry and S_in(s) on exit; z is chained the same way.
// Reverse mode (the backward pass's state over later tokens) chains from the
// last segment: R_in(P-1) = 0, R_in(s) = dR_{s+1} + Gamma_{s+1} R_in(s+1)
// (GLA: logG slot s + 1 holds segment s + 1's summed log-gate; slot 0 and
// dR_0 only feed a value that is never stored). With the outer-product gate,
// Gamma_s scales entry (f, e) of S by e^{logG[f] + logGv[e]} and z by e^{logG[f]}.
#include "chunked.hpp"

namespace la {

__global__ __launch_bounds__(256) void segment_scan_kernel(float* __restrict__ S, float* __restrict__ z,
                                                           const float* __restrict__ logG,
                                                           const float* __restrict__ logGv,
                                                           const float* __restrict__ S0,
                                                           const float* __restrict__ z0,
                                                           const float* __restrict__ gamma,
                                                           const int* __restrict__ slot, int nslot, int H, int P,
                                                           int R, int E, int seg_len, int gate, int reverse) {
  const long long bh = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int RE = R * E;
  if (idx >= RE + R) return;
  const bool is_z = idx >= RE;
  const int row = is_z ? idx - RE : idx / E;
  const int col = is_z ? 0 : idx % E;
  const bool per_input = gate == GT_GLA || gate == GT_SEL || gate == GT_OUTER;  // summed log-gates per segment
  const bool vside = gate == GT_OUTER && !is_z && logGv != nullptr;
  float* base = is_z ? z + bh * P * R + row : S + bh * P * RE + idx;
  const long long stride = is_z ? R : RE;
  float cur = 0.f;
  // the carried-in state of this (sequence, head): its slot's entry, if any
  long long st = bh;
  if (slot != nullptr) {
    const int sl = slot[bh / H];
    st = (sl >= 0 && sl < nslot) ? (long long)sl * H + bh % H : -1;
  }
  if (S0 != nullptr && !reverse && st >= 0) cur = is_z ? z0[st * R + row] : S0[st * RE + idx];
  float seg_decay = 1.f;
  if (gate == GT_DECAY) seg_decay = exp2f(float(seg_len) * log2f(gamma[bh % H]));
  // Batches of 8 segments: all loads of a batch are issued before the chain
  // that consumes them, so their latencies overlap.
  constexpr int BATCH = 8;
  for (int s0 = 0; s0 < P; s0 += BATCH) {
    float d[BATCH], G[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int s = min(s0 + j, P - 1);
      const int si = reverse ? P - 1 - s : s;
      d[j] = base[si * stride];
      G[j] = per_input ? logG[(bh * P + si) * R + row] : 0.f;
      if (vside) G[j] += logGv[(bh * P + si) * E + col];
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int s = s0 + j;
      if (s < P) {
        base[(reverse ? P - 1 - s : s) * stride] = cur;
        const float g = per_input ? __expf(G[j]) : seg_decay;
        cur = g * cur + d[j];
      }
    }
  }
}

la_status launch_segment_scan(const FwdPlan& p) {
  const int items = p.r * p.dv + p.r;
  dim3 grid((items + 255) / 256, unsigned(p.nseq) * unsigned(p.H));
  LA_LAUNCH(segment_scan_kernel, grid, dim3(256), 0, p.stream, p.ws_S, p.ws_z, p.ws_logG, p.ws_logGv, p.S0, p.z0,
                     p.gamma, p.slot, p.nslot, p.H, p.P, p.r, p.dv, p.seg_len, p.gate, 0);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status launch_segment_scan_reverse(const FwdPlan& p, float* S, float* z, const float* logG, const float* logGv) {
  const int items = p.r * p.dv + p.r;
  dim3 grid((items + 255) / 256, unsigned(p.nseq) * unsigned(p.H));
  LA_LAUNCH(segment_scan_kernel, grid, dim3(256), 0, p.stream, S, z, logG, logGv, nullptr, nullptr, p.gamma,
                     nullptr, 0, p.H, p.P, p.r, p.dv, p.seg_len, p.gate, 1);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // namespace la
