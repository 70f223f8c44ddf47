// State-space instances of the chunkwise causal kernels: identity features
// (C = q, B = k enter as they are) and the unnormalised read-out
// y_t = C_t^T h_t ("State Space Models as Linear Attention", "Linear Attention
// Mechanisms" (dileepadev.github.io)), under every gate.
#include "chunked_launch.hpp"

namespace la {

la_status launch_causal_ssm(const FwdPlan& p) { return causal_by_dk<FM_IDENT>(p); }

}  // namespace la
