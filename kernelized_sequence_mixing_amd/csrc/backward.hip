// Launchers of the causal backward pass (backward.hpp) and its built shapes.
#include "backward.hpp"

namespace la {

template <class K>
static la_status launch_with_lds(K kernel, dim3 grid, int lds, hipStream_t st, const BwdArgs& b) {
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, lds) !=
      hipSuccess)
    return LA_ERR_HIP;
  LA_LAUNCH(kernel, grid, dim3(256), lds, st, b);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

// SG: the GLA passes with one gate input per token (the selective gate).
template <int R, int E, int GATE, int FMAP, bool SG = false>
static la_status run_backward(const BwdPlan& p) {
  static_assert(Waves<R, E>::NW == 4, "the backward kernels use four-wave workgroups");
  const unsigned BH = unsigned(p.B) * unsigned(p.H);
  BwdArgs b{};
  b.Q = static_cast<const bf16*>(p.Q);
  b.K = static_cast<const bf16*>(p.K);
  b.V = static_cast<const bf16*>(p.V);
  b.dO = static_cast<const bf16*>(p.dO);
  b.gamma = p.gamma;
  b.G = static_cast<bf16*>(p.ws_G);
  b.h = p.ws_h;
  b.R_ws = p.ws_R;
  b.rh_ws = p.ws_rh;
  b.dQ = static_cast<bf16*>(p.dQ);
  b.dK = static_cast<bf16*>(p.dK);
  b.dV = static_cast<bf16*>(p.dV);
  b.ldv = p.ldv > 0 ? p.ldv : E;
  b.accum = p.accum;
  b.H = p.H;
  b.n = p.n;
  b.P = p.P;
  b.seg_len = p.seg_len;
  b.eps = p.eps;
  if constexpr (kKeyGate<GATE>) {
    b.gl = static_cast<const bf16*>(p.g);
    b.inv_tau = 1.f / p.tau;
    b.dB = p.ws_dB;
    b.logG = p.ws_logG;
    b.dg = static_cast<bf16*>(p.dg);
  }
  if constexpr (GATE == GT_OUTER) {
    b.gvl = static_cast<const bf16*>(p.gv);
    b.Pw = p.ws_P;
    b.logGv = p.ws_logGv;
    b.dgv = static_cast<bf16*>(p.dgv);
  }
  la_status st;
  // forward state entering each segment: the forward's segment pass and scan
  if (p.P > 1) {
    CausalArgs a1{};
    a1.Q = b.Q;
    a1.K = b.K;
    a1.V = b.V;
    a1.ldv = b.ldv;
    a1.gamma = p.gamma;
    a1.H = p.H;
    a1.n = p.n;
    a1.P = p.P;
    a1.seg_len = p.seg_len;
    a1.eps = p.eps;
    a1.S_out = p.ws_S;
    a1.z_out = p.ws_z;
    a1.g = b.gl;
    a1.gv = b.gvl;
    a1.ldgv = b.ldv;
    a1.inv_tau = b.inv_tau;
    a1.logG_out = p.ws_logG;
    a1.logGv_out = p.ws_logGv;
    if ((st = launch_segment_pass<R, E, R, FMAP, GATE, SG, GATE == GT_GLA>(a1, p.P, BH, p.stream)) != LA_OK) return st;
    if ((st = launch_segment_scan(p)) != LA_OK) return st;
    b.S_in = p.ws_S;
    b.z_in = p.ws_z;
    b.in_head = (long long)p.P * R * E;
    b.in_seg = (long long)R * E;
  } else {
    b.S_in = p.S0;
    b.z_in = p.z0;
    b.in_head = (long long)R * E;
    b.in_seg = 0;
  }
  if ((st = launch_with_lds(bwd_pass_a<R, E, GATE, FMAP, SG>, dim3(p.P, BH), BwdALayout<R, E, GATE>::bytes, p.stream,
                            b)) != LA_OK)
    return st;
  if (p.P > 1) {
    if constexpr (kKeyGate<GATE>)
      st = launch_with_lds(bwd_rstate_gla<R, E, GATE, FMAP, SG>, dim3(p.P - 1, BH), BwdRGLayout<R, E, GATE>::bytes,
                           p.stream, b);
    else
      st = launch_with_lds(bwd_rstate<R, E, GATE, FMAP>, dim3(p.P - 1, BH), BwdRLayout<R, E, GATE>::bytes, p.stream,
                           b);
    if (st != LA_OK) return st;
    if ((st = launch_segment_scan_reverse(p, p.ws_R, p.ws_rh, kKeyGate<GATE> ? p.ws_logG : nullptr,
                                          GATE == GT_OUTER ? p.ws_logGv : nullptr)) != LA_OK)
      return st;
  }
  return launch_with_lds(bwd_pass_b<R, E, GATE, FMAP, SG>, dim3(p.P, BH), BwdBLayout<R, E, GATE>::bytes, p.stream, b);
}

template <int R, int E, int FMAP>
static la_status run_backward_gated(const BwdPlan& p) {
  switch (p.gate) {
    case LA_GATE_NONE: return run_backward<R, E, GT_NONE, FMAP>(p);
    case LA_GATE_DECAY: return run_backward<R, E, GT_DECAY, FMAP>(p);
    case LA_GATE_GLA:
      return p.g_scalar ? run_backward<R, E, GT_GLA, FMAP, true>(p) : run_backward<R, E, GT_GLA, FMAP, false>(p);
    case LA_GATE_OUTER: return run_backward<R, E, GT_OUTER, FMAP>(p);
    default: return LA_ERR_UNSUPPORTED;
  }
}

template <int R, int E>
static la_status run_backward_fmap(const BwdPlan& p) {
  switch (p.fmap) {
    case LA_FMAP_ELU1: return run_backward_gated<R, E, FM_ELU1>(p);
    case LA_FMAP_IDENTITY: return run_backward_gated<R, E, FM_IDENT>(p);
    case kFmapPrecomputed:  // FAVOR+'s materialised features: no gate or the RetNet decay
      if (p.gate == LA_GATE_NONE) return run_backward<R, E, GT_NONE, FM_PRE>(p);
      if (p.gate == LA_GATE_DECAY) return run_backward<R, E, GT_DECAY, FM_PRE>(p);
      return LA_ERR_UNSUPPORTED;
    default: return LA_ERR_UNSUPPORTED;
  }
}

// Built shapes: elu+1 or the state-space form with (d_k, d_v) in {(64, 64), (64, 128), (128, 64)}; no gate,
// RetNet decay, GLA or the outer-product gate. (128, 128) runs as two (128, 64) halves of the value
// columns (la_backward).
la_status launch_backward(const BwdPlan& p) {
  switch (p.r * 1000 + p.dv) {
    case 64064: return run_backward_fmap<64, 64>(p);
    case 64128: return run_backward_fmap<64, 128>(p);
    case 128064: return run_backward_fmap<128, 64>(p);
    default: return LA_ERR_UNSUPPORTED;
  }
}

}  // namespace la
