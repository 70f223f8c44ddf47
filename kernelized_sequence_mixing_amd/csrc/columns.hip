// Column padding for the causal form at d_v = 32: the chunk kernels tile the
// value columns in 64-wide blocks, so la_forward runs a 32-column problem on
// copies in its workspace whose rows are 64 wide (columns 32..63 zero) and
// copies the 32 real columns back. A zero value column adds nothing to the
// state or to the outputs of the others (the normaliser z does not involve V).
#include "plan.hpp"

namespace la {

// dst[row][c] = src[row][c] for c < cols, 0 for cols <= c < dst_ld; rows of
// src_ld and dst_ld elements of `esz` bytes (2 or 4). One thread per element
// of dst's first `width` columns.
__global__ __launch_bounds__(256) void copy_columns_kernel(const void* __restrict__ src, void* __restrict__ dst,
                                                           long long rows, int src_ld, int dst_ld, int cols, int width,
                                                           int esz) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * width) return;
  const long long row = idx / width;
  const int c = int(idx % width);
  if (esz == 2) {
    const uint16_t v = c < cols ? static_cast<const uint16_t*>(src)[row * src_ld + c] : uint16_t(0);
    static_cast<uint16_t*>(dst)[row * dst_ld + c] = v;
  } else {
    const uint32_t v = c < cols ? static_cast<const uint32_t*>(src)[row * src_ld + c] : 0u;
    static_cast<uint32_t*>(dst)[row * dst_ld + c] = v;
  }
}

la_status launch_copy_columns(const void* src, void* dst, long long rows, int src_ld, int dst_ld, int cols, int width,
                              int esz, hipStream_t st) {
  if (rows <= 0 || width <= 0) return LA_OK;
  const long long total = rows * width;
  LA_LAUNCH(copy_columns_kernel, dim3(unsigned((total + 255) / 256)), dim3(256), 0, st, src, dst, rows, src_ld,
            dst_ld, cols, width, esz);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // namespace la
