// Host-side description of one validated call, shared by the C ABI layer and
// the kernel launchers. Everything here is plain data; no HIP types leak into
// the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/linattn.h"

namespace la {

constexpr int kChunk = 64;          // tokens per chunk of the causal kernel (= wave64)
constexpr int kComputeUnits = 256;  // MI355X
constexpr int kLdsPerCU = 160 * 1024;
constexpr int kMaxGroupsPerCU = 2;  // measured: 2 beats 1 and 3 on the chunked passes (fewer segments, less state traffic)
constexpr int kNonCausalGroups = 512;
// la_forward_batch steps of at most this many tokens per sequence (no
// cu_seqlens) run the recurrent step kernel, each state read and written once
constexpr int kMaxStepTokens = 16;

// LDS bytes of the causal output-pass workgroup for this shape (0 if not built);
// pure host arithmetic over the kernels' own layout definitions.
int causal_output_lds_bytes(int fmap, int r, int dv, int dk, int gate);

struct FwdPlan {
  int B, H, n, dk, dv, r;
  int r_valid;  // FAVOR+ run on kernels wider than its map: the map's feature count (0 = r)
  int in_dtype, out_dtype;
  float eps;
  int fmap, gate, causal;
  int g_scalar;  // GLA passes with one gate input per token (the selective gate's backward)
  float tau;
  const void* Q;
  const void* K;
  const void* V;
  const void* g;
  const void* gv;  // value-side gate input (the outer-product gate only)
  const void* omega;
  const float* gamma;
  const float* S0;
  const float* z0;
  float* S_final;
  float* z_final;
  void* out;
  // causal segmentation: P segments of seg_len tokens (multiple of kChunk)
  int P, seg_len;
  // a batch of sequences (la_forward_batch): nseq sequences (= B without cu);
  // cu: device [nseq + 1] offsets along n (B == 1), slot: device [nseq] state
  // slots of S0 / S_final ([nslot][H][r][d_v]); both null for la_forward
  int nseq;
  const int* cu;
  const int* slot;
  int nslot;
  // non-causal split of the sequence into partial sums
  int splits, split_len;
  // workspace carve (device)
  float* ws_S;     // [BH][P or splits][r][dv]
  float* ws_z;     // [BH][P or splits][r]
  float* ws_logG;  // [BH][P][r]  (gates with an input)
  float* ws_logGv; // [BH][P][dv] (the outer-product gate's value side)
  hipStream_t stream;
};

// The backward pass of the causal form: the forward plan (segments, state
// workspace) plus the incoming gradient, the gradient outputs and the
// workspace of the reverse passes.
struct BwdPlan : FwdPlan {
  const void* dO;
  void* dQ;
  void* dK;
  void* dV;
  float* ws_R;   // [BH][P][r][dv]
  float* ws_rh;  // [BH][P][r]
  void* ws_G;    // [BH][n][dv] bf16
  float* ws_h;   // [BH][n]
  // GLA and outer-product gates
  void* dg;      // [BH][n][r] out_dtype
  float* ws_dB;  // [BH][ceil(n / 64) * 64][r] in the kernels' own order
  // outer-product gate: the gradient of gv, dO * o per token and column
  void* dgv;     // [BH][n][ldv] out_dtype
  float* ws_P;   // [BH][n][dv]
  // a value-column half of a wider V: elements between rows of V, dO, dV, gv
  // and dgv (0: dv), and whether dQ, dK, dg are added to (the second half) or stored
  int ldv, accum;
};

struct DecodePlan {
  int B, H, dk, dv, r;
  int in_dtype, out_dtype;
  float eps;
  int fmap, gate;
  float tau;
  float* S;
  float* z;
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* gv;  // value-side gate input (the outer-product gate only)
  const void* omega;
  const float* gamma;
  void* out;
  // state slots (la_forward_batch with a few tokens per sequence): state index
  // slot[b] H + h; flags 1 read, 2 write (la_decode_step: no slots, both)
  const int* slot;
  int nslot, flags;
  hipStream_t stream;
  int m;  // tokens per sequence (0 or 1: one step; at most kMaxStepTokens)
};

struct FmapPlan {
  int64_t rows;
  int dk, r, in_dtype, fmap;
  const void* X;
  const void* omega;
  float* out;
  hipStream_t stream;
};

// Softmax attention (the quadratic baseline): bf16 [B][H][n][d] in and out.
struct SoftmaxPlan {
  int B, H, n, d, causal;
  float scale;
  const void* Q;
  const void* K;
  const void* V;
  void* out;
  hipStream_t stream;
};

// Launch timing (la_timing_begin / la_timing_end): while a bracket is open on
// this host thread, every launch first records the next caller-owned event on
// its stream. Launches past the events supplied are counted, not recorded.
struct LaunchTimer {
  void* const* ev;
  int n;
  int used;
  bool failed;
};
extern thread_local LaunchTimer* t_launch_timer;
inline void mark_launch(hipStream_t s) {
  LaunchTimer* t = t_launch_timer;
  if (t == nullptr) return;
  if (t->used < t->n && hipEventRecord(static_cast<hipEvent_t>(t->ev[t->used]), s) != hipSuccess) t->failed = true;
  t->used++;
}
// Every kernel launch of the library goes through this.
#define LA_LAUNCH(kernel, grid, block, lds, stream, ...)          \
  do {                                                            \
    ::la::mark_launch(stream);                                    \
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__); \
  } while (0)

// Launchers (each returns LA_OK or LA_ERR_HIP / LA_ERR_UNSUPPORTED).
la_status launch_causal_elu1(const FwdPlan& p);
la_status launch_causal_ssm(const FwdPlan& p);
la_status launch_causal_favor(const FwdPlan& p);
la_status launch_segment_scan(const FwdPlan& p);
la_status launch_segment_scan_reverse(const FwdPlan& p, float* S, float* z, const float* logG,
                                      const float* logGv = nullptr);
la_status launch_backward(const BwdPlan& p);
la_status launch_noncausal_backward(const BwdPlan& p);  // ws_S, ws_z: partial S, z; ws_R, ws_rh: partial G, hq
la_status launch_noncausal(const FwdPlan& p);
// dst[h][i][j] = src[h][i][j] inside src's [src_rows][src_cols], 0 elsewhere in dst's [dst_rows][dst_cols]
// (heads of each, contiguous, esz bytes per element): zero-padded or cropped copies
la_status launch_copy_block(const void* src, void* dst, long long heads, int src_rows, int src_cols, int dst_rows,
                            int dst_cols, int esz, hipStream_t st);
la_status launch_decode(const DecodePlan& p);
la_status launch_feature_map(const FmapPlan& p);
la_status launch_softmax(const SoftmaxPlan& p);
// FAVOR+ backward: its features materialised (bf16 [rows][r]) and the
// gradient through the feature map, dX = sum_m dphi_m phi_m (w_m - x).
la_status launch_favor_features(const void* X, int in_dt, long long rows, int dk, int r, const void* omega, void* out,
                                hipStream_t st);
la_status launch_favor_vjp(const void* dphi, const void* phi, const void* X, int in_dt, long long rows, int dk, int r,
                           const void* omega, void* dX, int out_dt, hipStream_t st);
// BwdPlan::fmap value for features computed beforehand (not a public feature map).
constexpr int kFmapPrecomputed = 3;

}  // namespace la
