// elu+1 instances of the chunkwise causal kernels (r = d_k).
#include "chunked_launch.hpp"

namespace la {

la_status launch_causal_elu1(const FwdPlan& p) { return causal_by_dk<FM_ELU1>(p); }

}  // namespace la
