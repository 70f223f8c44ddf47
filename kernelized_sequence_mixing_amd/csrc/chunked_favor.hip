// FAVOR+ instances of the chunkwise causal kernels (projection on the matrix cores,
// hi/lo bf16 operand pairs).
#include "chunked_favor.hpp"

namespace la {

template <int R, int E, int DK>
static la_status by_gate(const FwdPlan& p) {
  switch (p.gate) {
    case GT_NONE: return run_causal_favor<R, E, DK, GT_NONE>(p);
    case GT_DECAY: return run_causal_favor<R, E, DK, GT_DECAY>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

template <int R, int E>
static la_status by_dk(const FwdPlan& p) {
  switch (p.dk) {
    case 32: return by_gate<R, E, 32>(p);
    case 64: return by_gate<R, E, 64>(p);
    case 128: return by_gate<R, E, 128>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

template <int R>
static la_status by_dv(const FwdPlan& p) {
  switch (p.dv) {
    case 64: return by_dk<R, 64>(p);
    case 128:
      if constexpr (R * 128 <= 16384) return by_dk<R, 128>(p);
      break;
  }
  return LA_ERR_UNSUPPORTED;
}

la_status launch_causal_favor(const FwdPlan& p) {
  switch (p.r) {
    case 64: return by_dv<64>(p);
    case 128: return by_dv<128>(p);
    case 256: return by_dv<256>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

}  // namespace la
