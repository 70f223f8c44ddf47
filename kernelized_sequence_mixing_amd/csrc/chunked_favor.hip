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

template <int R, int GATE, int E>
static int favor_lds_dk(int dk) {
  using LY = FavorFwdLayout<R, E, GATE>;
  switch (dk) {
    case 32: return LY::template bytes_dk<32>;
    case 64: return LY::template bytes_dk<64>;
    case 128: return LY::template bytes_dk<128>;
  }
  return 0;
}

template <int R, int GATE>
static int favor_lds_gate(int dv, int dk) {
  if (dv == 64) return favor_lds_dk<R, GATE, 64>(dk);
  if (dv == 128 && R * 128 <= 16384) return favor_lds_dk<R, GATE, 128>(dk);
  return 0;
}

template <int R>
static int favor_lds(int dv, int dk, int gate) {
  return gate == GT_DECAY ? favor_lds_gate<R, GT_DECAY>(dv, dk) : favor_lds_gate<R, GT_NONE>(dv, dk);
}

template <int R, int GATE>
static int elu_lds_gate(int dv) {
  if (dv == 64) return FwdLayout<R, 64, GATE>::bytes;
  if (dv == 128) return FwdLayout<R, 128, GATE>::bytes;
  return 0;
}

template <int R>
static int elu_lds(int dv, int gate) {
  switch (gate) {
    case GT_NONE: return elu_lds_gate<R, GT_NONE>(dv);
    case GT_DECAY: return elu_lds_gate<R, GT_DECAY>(dv);
    case GT_GLA: return elu_lds_gate<R, GT_GLA>(dv);
    case GT_SEL: return elu_lds_gate<R, GT_SEL>(dv);
    case GT_OUTER: return elu_lds_gate<R, GT_OUTER>(dv);
  }
  return 0;
}

static_assert(GT_NONE == LA_GATE_NONE && GT_DECAY == LA_GATE_DECAY && GT_GLA == LA_GATE_GLA &&
                  GT_SEL == LA_GATE_SEL && GT_OUTER == LA_GATE_OUTER,
              "gate codes");

int causal_output_lds_bytes(int fmap, int r, int dv, int dk, int gate) {
  if (fmap == LA_FMAP_FAVOR) {
    switch (r) {
      case 64: return favor_lds<64>(dv, dk, gate);
      case 128: return favor_lds<128>(dv, dk, gate);
      case 256: return favor_lds<256>(dv, dk, gate);
    }
    return 0;
  }
  switch (r) {
    case 32: return elu_lds<32>(dv, gate);
    case 64: return elu_lds<64>(dv, gate);
    case 128: return elu_lds<128>(dv, gate);
  }
  return 0;
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
