// Dispatch of the chunkwise causal kernels with an elementwise feature map
// (r = d_k) over the built (d_k, d_v, gate) set; one translation unit per
// feature map instantiates it.
#pragma once

#include "chunked.hpp"

namespace la {

template <int FMAP, int R, int E>
static la_status causal_by_gate(const FwdPlan& p) {
  switch (p.gate) {
    case GT_NONE: return run_causal<R, E, R, FMAP, GT_NONE>(p);
    case GT_DECAY: return run_causal<R, E, R, FMAP, GT_DECAY>(p);
    case GT_GLA: return run_causal<R, E, R, FMAP, GT_GLA>(p);
    case GT_SEL: return run_causal<R, E, R, FMAP, GT_SEL>(p);
    case GT_OUTER: return run_causal<R, E, R, FMAP, GT_OUTER>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

template <int FMAP, int R>
static la_status causal_by_dv(const FwdPlan& p) {
  switch (p.dv) {
    case 64: return causal_by_gate<FMAP, R, 64>(p);
    case 128: return causal_by_gate<FMAP, R, 128>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

template <int FMAP>
static la_status causal_by_dk(const FwdPlan& p) {
  switch (p.dk) {
    case 32: return causal_by_dv<FMAP, 32>(p);
    case 64: return causal_by_dv<FMAP, 64>(p);
    case 128: return causal_by_dv<FMAP, 128>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

}  // namespace la
