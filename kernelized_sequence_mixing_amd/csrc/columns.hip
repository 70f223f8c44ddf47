// Zero-padded copies for the causal form at the widths its chunk kernels do
// not tile: they work in 64-wide blocks of value columns and of FAVOR+
// features, so la_forward runs d_v = 32 (and FAVOR+ r = 32) on copies in its
// workspace that are 64 wide (the extra columns, feature rows of omega and
// state rows zero), then copies the real part back. A zero value column adds
// nothing to the state, z or the other columns; a FAVOR+ feature that the
// kernel masks to zero adds nothing to the scores, state, z or read-out.
#include "plan.hpp"

namespace la {

// dst[h][i][j] = src[h][i][j] for i < src_rows and j < src_cols, 0 elsewhere,
// over dst's [heads][dst_rows][dst_cols] (both contiguous; esz 2 or 4 bytes).
// Pads when dst is larger and crops when it is smaller. One thread per element of dst.
__global__ __launch_bounds__(256) void copy_block_kernel(const void* __restrict__ src, void* __restrict__ dst,
                                                         long long heads, int src_rows, int src_cols, int dst_rows,
                                                         int dst_cols, int esz) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long per = (long long)dst_rows * dst_cols;
  if (idx >= heads * per) return;
  const long long h = idx / per;
  const int i = int((idx % per) / dst_cols), j = int(idx % dst_cols);
  const bool in = i < src_rows && j < src_cols;
  const long long s = (h * src_rows + (in ? i : 0)) * src_cols + (in ? j : 0);
  if (esz == 2) {
    static_cast<uint16_t*>(dst)[idx] = in ? static_cast<const uint16_t*>(src)[s] : uint16_t(0);
  } else {
    static_cast<uint32_t*>(dst)[idx] = in ? static_cast<const uint32_t*>(src)[s] : 0u;
  }
}

la_status launch_copy_block(const void* src, void* dst, long long heads, int src_rows, int src_cols, int dst_rows,
                            int dst_cols, int esz, hipStream_t st) {
  const long long total = heads * dst_rows * (long long)dst_cols;
  if (total <= 0) return LA_OK;
  LA_LAUNCH(copy_block_kernel, dim3(unsigned((total + 255) / 256)), dim3(256), 0, st, src, dst, heads, src_rows,
            src_cols, dst_rows, dst_cols, esz);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // namespace la
