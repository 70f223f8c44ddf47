// la_forward_noalloc: la_forward with its scratch memory in a fixed device
// array of the library instead of a caller workspace, for callers that cannot
// allocate device memory (code under graph capture, serving loops, harnesses
// that forbid allocation).
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy for the life of the process. In host code its name is a
// host-side stand-in, not a device address, so the address is taken once per
// device with hipGetSymbolAddress (with that device current) and only that
// pointer is ever handed to a kernel. Calls that overlap on one GPU share the
// array and race; the kernels need no part of it cleared (every scratch value
// they read was written earlier in the same call).
#include <mutex>

#include "plan.hpp"

namespace la {
namespace {

__device__ __align__(256) char scratch[LA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's scratch array (looked up on first use).
la_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return LA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return LA_OK;
}

}  // namespace
}  // namespace la

extern "C" la_status la_forward_noalloc(const la_problem* p, const void* Q, const void* K, const void* V,
                                        const la_feature_map* fmap, int32_t causal, const la_gate* gate,
                                        const float* S0, const float* z0, float* S_final, float* z_final,
                                        void* out, void* stream) {
  size_t need = 0;
  la_status st = la_forward_workspace_size(p, fmap, causal, gate, &need);
  if (st != LA_OK) return st;
  if (need > LA_NOALLOC_SCRATCH_BYTES) return LA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && (st = la::scratch_of_current_device(&ws)) != LA_OK) return st;
  return la_forward(p, Q, K, V, fmap, causal, gate, S0, z0, S_final, z_final, out, need > 0 ? ws : nullptr, need,
                    stream);
}
