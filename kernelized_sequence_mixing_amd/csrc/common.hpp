// Device helpers for gfx950 (CDNA4): bf16 vectors, the 16x16x32 bf16 MFMA,
// wave64 cross-lane reductions and scans, and the two feature maps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }  // exact widening

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// float -> bf16 lowers to v_cvt_pk_bf16_f32: round to nearest even, NaN kept.
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ bf16x4 pack4(float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
  return v;
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Two floats rounded to bf16 and packed (a in the low half): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned pack2_bits(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
// The two halves of a packed bf16 pair, widened exactly to float.
__device__ __forceinline__ float lo_bf16_f32(unsigned p) { return __builtin_bit_cast(float, p << 16); }
__device__ __forceinline__ float hi_bf16_f32(unsigned p) { return __builtin_bit_cast(float, p & 0xffff0000u); }

// ---------------------------------------------------------------- matrix core

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16) on one wave.
// Lane l (g = l / 16, c = l % 16) supplies A[c][k] and B[k][c] for the eight
// k-slots it owns, and receives D[4 g + i][c], i = 0..3. The k-slot -> k
// assignment only has to agree between A and B, which lets callers build
// operands from any eight contraction indices per lane.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- wave64 lanes

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// The lane index, opaque to the optimizer. Addresses derived from it inside a
// loop body are rebuilt there (a few integer ops) instead of being hoisted out
// of the loop and kept live in registers for its whole duration; the mask
// restores the 0..63 range that lets constant offsets fold into instructions.
__device__ __forceinline__ int opaque_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane & 63;
}
// Wave index in a workgroup of NW waves. The mask gives the compiler its range
// (readfirstlane alone hides it), so LDS addresses built from it keep their
// constant parts in the instruction's offset field instead of in registers.
template <int NW = 4>
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & (NW - 1); }

// Sum over the four lanes {c, c+16, c+32, c+48} that share c = lane % 16.
__device__ __forceinline__ float sum_over_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, true));
}

// Inclusive prefix sum across the 64 lanes of a wave (lane t gets x_0 + ... + x_t).
// Hillis-Steele within each row of 16 lanes (row_shr 1, 2, 4, 8), then the row
// totals are carried with the row broadcasts of lane 15 (into rows 1, 3) and
// lane 31 (into rows 2, 3).
template <int CTRL, int ROW_MASK, int N>
__device__ __forceinline__ void scan_step(float (&x)[N]) {
  float t[N];
#pragma unroll
  for (int u = 0; u < N; ++u) t[u] = dpp_or_zero<CTRL, ROW_MASK>(x[u]);
#pragma unroll
  for (int u = 0; u < N; ++u) x[u] += t[u];
}

// N independent scans of wave_inclusive_scan, taken step by step across the
// N values, so that no DPP read of a register follows right after its write
// (a back-to-back chain needs wait states between the two).
template <int N>
__device__ __forceinline__ void wave_inclusive_scan_n(float (&x)[N]) {
  scan_step<0x111, 0xf>(x);
  scan_step<0x112, 0xf>(x);
  scan_step<0x114, 0xf>(x);
  scan_step<0x118, 0xf>(x);
  scan_step<0x142, 0xa>(x);
  scan_step<0x143, 0xc>(x);
}

__device__ __forceinline__ float wave_inclusive_scan(float x) {
  x += dpp_or_zero<0x111, 0xf>(x);
  x += dpp_or_zero<0x112, 0xf>(x);
  x += dpp_or_zero<0x114, 0xf>(x);
  x += dpp_or_zero<0x118, 0xf>(x);
  x += dpp_or_zero<0x142, 0xa>(x);
  x += dpp_or_zero<0x143, 0xc>(x);
  return x;
}

// ---------------------------------------------------------------- masking

// x if ok else +0, without a branch (a select around an expensive expression
// would otherwise be compiled as a divergent branch per element).
__device__ __forceinline__ float keep_if(bool ok, float x) {
  return __builtin_bit_cast(float, __builtin_bit_cast(unsigned, x) & (ok ? 0xffffffffu : 0u));
}

__device__ __forceinline__ bf16x8 keep_if(bool ok, bf16x8 x) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const unsigned m = ok ? 0xffffffffu : 0u;
  return __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, x) & m);
}

// ---------------------------------------------------------------- feature maps

// elu(x) + 1 = x + 1 for x > 0, exp(x) for x <= 0.
__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// log(alpha) of the GLA gate alpha = sigmoid(g)^(1/tau): -softplus(-g) / tau,
// with softplus(y) = max(y, 0) + log(1 + exp(-|y|)).
__device__ __forceinline__ float gla_log_alpha(float g, float inv_tau) {
  float y = -g;
  float sp = fmaxf(y, 0.f) + __logf(1.f + __expf(-fabsf(y)));
  return -sp * inv_tau;
}

// The same quantity in base 2, log2(alpha) = -softplus(-g) / (tau ln 2), with
// softplus / ln 2 = max(y, 0) + log2(1 + 2^-|y|) for y = -g log2(e): the chunk
// preludes scan it and exponentiate with the hardware's base-2 exp directly.
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.693147180559945309f;
__device__ __forceinline__ float gla_log2_alpha(float g, float inv_tau) {
  const float y = -g * kLog2e;
  const float sp2 = fmaxf(y, 0.f) + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(y)));
  return -sp2 * inv_tau;
}

}  // namespace la
