// elu+1 instances of the chunkwise causal kernels (r = d_k).
#include "chunked.hpp"

namespace la {

template <int R, int E>
static la_status by_gate(const FwdPlan& p) {
  switch (p.gate) {
    case GT_NONE: return run_causal<R, E, R, FM_ELU1, GT_NONE>(p);
    case GT_DECAY: return run_causal<R, E, R, FM_ELU1, GT_DECAY>(p);
    case GT_GLA: return run_causal<R, E, R, FM_ELU1, GT_GLA>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

template <int R>
static la_status by_dv(const FwdPlan& p) {
  switch (p.dv) {
    case 64: return by_gate<R, 64>(p);
    case 128: return by_gate<R, 128>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

la_status launch_causal_elu1(const FwdPlan& p) {
  switch (p.dk) {
    case 32: return by_dv<32>(p);
    case 64: return by_dv<64>(p);
    case 128: return by_dv<128>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

}  // namespace la
