// The FAVOR+ pieces of the backward pass ("Choosing the Feature Map phi",
// "Linear Attention Mechanisms" (dileepadev.github.io): positive random
// features phi(x)_m = exp(w_m . x - |x|^2/2) / sqrt(r)).
//
// la_backward runs FAVOR+ in three steps: the features of the queries and
// keys are materialised as bf16 [rows][r] (favor_features), the chunked
// backward kernels run on them as precomputed features (normalised read-out,
// phi' = 1), which gives dphi for every query and key, and favor_vjp takes
// those back through the feature map:
//   d phi_m / dx = phi_m (w_m - x)  =>  dx = sum_m u_m w_m - x sum_m u_m,  u_m = dphi_m phi_m.
#include "vec_common.hpp"

namespace la {

// Both kernels are dense contractions with omega on the matrix cores: rows in
// blocks of 16 per wave (rows_per_wave of them per workgroup), each output
// tile a 16 x 16 fp32 accumulator taken as its transpose, so that a lane holds
// four consecutive columns of one row (lane c: row c of the block) and stores
// them with one 8-byte write.
constexpr int kFavorRowsPerWave = 64;  // four 16-row blocks per wave
constexpr int kFavorRowsPerBlock = 4 * kFavorRowsPerWave;

// The eight bf16 of X[row][k0 .. k0 + 7] (zeros past the last row).
__device__ __forceinline__ bf16x8 load_row8(const bf16* __restrict__ X, long long row, long long rows, int ld, int k0) {
  if (row >= rows) return bf16x8{};
  return *reinterpret_cast<const bf16x8*>(X + row * ld + k0);
}

// phi of the rows of X (bf16 [rows][DK]) as bf16 [rows][R]: acc = w_m . x on
// the matrix cores (exact bf16 products, fp32 sums), then
// phi_m = 2^(acc log2 e - (|x|^2/2 + ln(R)/2) log2 e), one rounding to bf16.
// omega [R][DK] is staged once per workgroup in LDS with padded rows.
template <int R, int DK>
__global__ __launch_bounds__(256) void favor_features_kernel(const bf16* __restrict__ X, long long rows,
                                                             const bf16* __restrict__ omega, bf16* __restrict__ out) {
  constexpr int KB = DK / 32, OLD = DK + 8;  // k-blocks; LDS row of omega in bf16 (16 bytes of padding)
  __shared__ __attribute__((aligned(16))) bf16 som[R * OLD];
  const int tid = threadIdx.x;
  for (int idx = tid; idx < R * DK / 8; idx += 256) {
    const int m = idx / (DK / 8), k8 = idx % (DK / 8);
    *reinterpret_cast<bf16x8*>(som + m * OLD + 8 * k8) = *reinterpret_cast<const bf16x8*>(omega + m * DK + 8 * k8);
  }
  __syncthreads();
  const int lane = lane_id(), c = lane & 15, g = lane >> 4;
  const long long base = (long long)blockIdx.x * kFavorRowsPerBlock + wave_id() * kFavorRowsPerWave;
  if (base >= rows) return;
  constexpr int NB = kFavorRowsPerWave / 16;
  bf16x8 xf[NB][KB];
  float shift2[NB];
  const float lnr_half = 0.5f * __logf(float(R));
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float sq = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      xf[b][kb] = load_row8(X, base + 16 * b + c, rows, DK, 32 * kb + 8 * g);
#pragma unroll
      for (int j = 0; j < 8; ++j) sq += float(xf[b][kb][j]) * float(xf[b][kb][j]);
    }
    shift2[b] = (0.5f * sum_over_groups(sq) + lnr_half) * 1.44269504f;
  }
#pragma unroll
  for (int mt = 0; mt < R / 16; ++mt) {
    bf16x8 of[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) of[kb] = *reinterpret_cast<const bf16x8*>(som + (16 * mt + c) * OLD + 32 * kb + 8 * g);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc = mfma16(of[kb], xf[b][kb], acc);  // [feature 4g+i][row c]
      const long long row = base + 16 * b + c;
      if (row < rows) {
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], 1.44269504f, -shift2[b]));
        *reinterpret_cast<bf16x4*>(out + row * R + 16 * mt + 4 * g) = pack4(f[0], f[1], f[2], f[3]);
      }
    }
  }
}

// dX (bf16 [rows][DK]) from dphi, phi (bf16 [rows][R]) and X:
//   dx_d = sum_m u_m w_md - x_d sum_m u_m,  u_m = dphi_m phi_m.
// u is exact in fp32 (a product of two bf16); it enters the matrix cores as
// hi + lo bf16 pairs, so the contraction keeps ~16 significant bits of it, and
// its row sum is taken in fp32 in a fixed order. omega^T [DK][R] sits in LDS
// with padded rows.
template <int R, int DK>
__global__ __launch_bounds__(256) void favor_vjp_kernel(const bf16* __restrict__ dphi, const bf16* __restrict__ phi,
                                                        const bf16* __restrict__ X, long long rows,
                                                        const bf16* __restrict__ omega, bf16* __restrict__ dX) {
  constexpr int KB = R / 32, TLD = R + 8;  // k-blocks over the features; LDS row of omega^T in bf16
  __shared__ __attribute__((aligned(16))) bf16 somt[DK * TLD];
  const int tid = threadIdx.x;
  for (int idx = tid; idx < R * DK; idx += 256) {
    const int m = idx / DK, d = idx % DK;
    somt[d * TLD + m] = omega[idx];
  }
  __syncthreads();
  const int lane = lane_id(), c = lane & 15, g = lane >> 4;
  const long long base = (long long)blockIdx.x * kFavorRowsPerBlock + wave_id() * kFavorRowsPerWave;
  if (base >= rows) return;
  for (int b = 0; b < kFavorRowsPerWave / 16; ++b) {
    const long long row = base + 16 * b + c;
    bf16x8 uh[KB], ul[KB];
    float su = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bf16x8 dp = load_row8(dphi, row, rows, R, 32 * kb + 8 * g);
      const bf16x8 ph = load_row8(phi, row, rows, R, 32 * kb + 8 * g);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float u = float(dp[j]) * float(ph[j]);
        su += u;
        uh[kb][j] = (bf16)u;
        ul[kb][j] = (bf16)(u - float(uh[kb][j]));
      }
    }
    su = sum_over_groups(su);
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 ot = *reinterpret_cast<const bf16x8*>(somt + (16 * dt + c) * TLD + 32 * kb + 8 * g);
        acc = mfma16(ot, uh[kb], acc);  // [column 4g+i][row c]
        acc = mfma16(ot, ul[kb], acc);
      }
      if (row < rows) {
        const bf16x4 x = *reinterpret_cast<const bf16x4*>(X + row * DK + 16 * dt + 4 * g);
        *reinterpret_cast<bf16x4*>(dX + row * DK + 16 * dt + 4 * g) =
            pack4(acc[0] - float(x[0]) * su, acc[1] - float(x[1]) * su, acc[2] - float(x[2]) * su,
                  acc[3] - float(x[3]) * su);
      }
    }
  }
}

template <int R, int DK>
static la_status run_favor_features(const void* X, long long rows, const void* omega, void* out, hipStream_t st) {
  const long long blocks = (rows + kFavorRowsPerBlock - 1) / kFavorRowsPerBlock;
  LA_LAUNCH((favor_features_kernel<R, DK>), dim3(unsigned(blocks)), dim3(256), 0, st, static_cast<const bf16*>(X),
            rows, static_cast<const bf16*>(omega), static_cast<bf16*>(out));
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

template <int R, int DK>
static la_status run_favor_vjp(const void* dphi, const void* phi, const void* X, long long rows, const void* omega,
                               void* dX, hipStream_t st) {
  const long long blocks = (rows + kFavorRowsPerBlock - 1) / kFavorRowsPerBlock;
  LA_LAUNCH((favor_vjp_kernel<R, DK>), dim3(unsigned(blocks)), dim3(256), 0, st, static_cast<const bf16*>(dphi),
            static_cast<const bf16*>(phi), static_cast<const bf16*>(X), rows, static_cast<const bf16*>(omega),
            static_cast<bf16*>(dX));
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

// Built: r in {64, 128} (the backward kernels' feature widths), d_k in {32, 64, 128}.
#define LA_FAVOR_BWD_DISPATCH(FN, ...)                        \
  switch (r * 1000 + dk) {                                    \
    case 64032: return FN<64, 32>(__VA_ARGS__);               \
    case 64064: return FN<64, 64>(__VA_ARGS__);               \
    case 64128: return FN<64, 128>(__VA_ARGS__);              \
    case 128032: return FN<128, 32>(__VA_ARGS__);             \
    case 128064: return FN<128, 64>(__VA_ARGS__);             \
    case 128128: return FN<128, 128>(__VA_ARGS__);            \
  }                                                           \
  return LA_ERR_UNSUPPORTED;

la_status launch_favor_features(const void* X, int in_dt, long long rows, int dk, int r, const void* omega, void* out,
                                hipStream_t st) {
  if (in_dt != LA_BF16) return LA_ERR_UNSUPPORTED;
  LA_FAVOR_BWD_DISPATCH(run_favor_features, X, rows, omega, out, st)
}

la_status launch_favor_vjp(const void* dphi, const void* phi, const void* X, int in_dt, long long rows, int dk, int r,
                           const void* omega, void* dX, int out_dt, hipStream_t st) {
  if (in_dt != LA_BF16 || out_dt != LA_BF16) return LA_ERR_UNSUPPORTED;
  LA_FAVOR_BWD_DISPATCH(run_favor_vjp, dphi, phi, X, rows, omega, dX, st)
}

}  // namespace la
