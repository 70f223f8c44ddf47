// C ABI of the library: argument validation (all of it before any HIP call),
// workspace sizing and segment planning (pure host arithmetic), and dispatch
// to the kernel launchers on the caller's stream.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "plan.hpp"

namespace la {

thread_local LaunchTimer* t_launch_timer = nullptr;

namespace {

thread_local LaunchTimer t_timer_slot;

constexpr size_t kAlign = 256;

typedef uint16_t bf16_bits;  // element type for pointer offsets into bf16 arrays

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t dtype_size(int dt) { return dt == LA_BF16 ? 2 : 4; }

bool valid_dtype(int dt) { return dt == LA_F32 || dt == LA_BF16; }

bool in_set(int x, std::initializer_list<int> s) {
  for (int v : s)
    if (x == v) return true;
  return false;
}

struct Range {
  uintptr_t lo, hi;
};

Range range_of(const void* p, size_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a, a + bytes};
}

bool overlaps(Range a, Range b) { return a.lo != 0 && b.lo != 0 && a.lo < b.hi && b.lo < a.hi; }

la_status check_problem(const la_problem* p) {
  if (p == nullptr) return LA_ERR_INVALID_ARG;
  if (p->B < 1 || p->H < 1 || p->n < 1 || p->d_k < 1 || p->d_v < 1) return LA_ERR_INVALID_ARG;
  if (!valid_dtype(p->in_dtype) || !valid_dtype(p->out_dtype)) return LA_ERR_INVALID_ARG;
  if (!(p->eps >= 0.f) || !isfinite(p->eps)) return LA_ERR_INVALID_ARG;
  if ((long long)p->B * p->H > 65535) return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

la_status check_fmap(const la_feature_map* f, int dk) {
  if (f == nullptr) return LA_ERR_INVALID_ARG;
  if (f->kind == LA_FMAP_ELU1 || f->kind == LA_FMAP_IDENTITY) {
    if (f->r != dk || f->omega != nullptr) return LA_ERR_INVALID_ARG;
  } else if (f->kind == LA_FMAP_FAVOR) {
    if (f->r < 1 || f->omega == nullptr) return LA_ERR_INVALID_ARG;
    if (!aligned16(f->omega)) return LA_ERR_INVALID_ARG;
  } else {
    return LA_ERR_INVALID_ARG;
  }
  return LA_OK;
}

// gate may be NULL (= NONE). `check_ptrs` is false for the size queries.
la_status check_gate(const la_gate* g, bool check_ptrs) {
  if (g == nullptr) return LA_OK;
  if (check_ptrs && g->gv != nullptr && g->kind != LA_GATE_OUTER) return LA_ERR_INVALID_ARG;
  if (g->kind == LA_GATE_NONE) return LA_OK;
  if (g->kind == LA_GATE_DECAY) {
    if (check_ptrs && (g->gamma == nullptr || !aligned16(g->gamma))) return LA_ERR_INVALID_ARG;
    return LA_OK;
  }
  if (g->kind == LA_GATE_GLA || g->kind == LA_GATE_SEL || g->kind == LA_GATE_OUTER) {
    if (!(g->tau > 0.f) || !isfinite(g->tau)) return LA_ERR_INVALID_ARG;
    if (check_ptrs && (g->g == nullptr || !aligned16(g->g))) return LA_ERR_INVALID_ARG;
    if (check_ptrs && g->kind == LA_GATE_OUTER && (g->gv == nullptr || !aligned16(g->gv))) return LA_ERR_INVALID_ARG;
    if (check_ptrs && g->kind != LA_GATE_OUTER && g->gv != nullptr) return LA_ERR_INVALID_ARG;
    return LA_OK;
  }
  return LA_ERR_INVALID_ARG;
}

int gate_kind(const la_gate* g) { return g == nullptr ? LA_GATE_NONE : g->kind; }

// Gates driven by a raw input g (GLA: one value per feature and token; the
// selective scalar gate: one per token), and that input's elements per token.
bool gate_has_input(int gk) { return gk == LA_GATE_GLA || gk == LA_GATE_SEL || gk == LA_GATE_OUTER; }
size_t gate_input_per_token(int gk, size_t r) {
  return (gk == LA_GATE_GLA || gk == LA_GATE_OUTER) ? r : (gk == LA_GATE_SEL ? 1 : 0);
}
// The outer-product gate's value-side input gv: d_v elements per token.
size_t gate_vinput_per_token(int gk, size_t dv) { return gk == LA_GATE_OUTER ? dv : 0; }
const void* gate_vinput(const la_gate* g) { return gate_kind(g) == LA_GATE_OUTER ? g->gv : nullptr; }

// The built set of (d_k, r, d_v) shapes; see the header.
bool shapes_built(const la_feature_map* f, int dk, int dv, bool causal) {
  (void)causal;  // causal d_v = 32 runs the 64-column kernels on padded copies (padded_dv)
  if (!in_set(dk, {32, 64, 128})) return false;
  if (!in_set(dv, {32, 64, 128})) return false;
  if (f->kind == LA_FMAP_FAVOR && !in_set(f->r, {32, 64, 128, 256})) return false;
  return (long long)f->r * dv <= 16384;
}

// Output-pass workgroups the GPU holds at once: every CU with as many as its
// LDS fits, at most kMaxGroupsPerCU.
long long resident_groups(int fmap, int r, int dv, int dk, int gate) {
  const int lds = causal_output_lds_bytes(fmap, r, dv, dk, gate);
  int per_cu = lds > 0 ? kLdsPerCU / lds : 1;
  if (per_cu < 1) per_cu = 1;
  if (per_cu > kMaxGroupsPerCU) per_cu = kMaxGroupsPerCU;
  // elu+1 with a 128 x 128 state: the fp32 state and its bf16 image alone take
  // a third of a lane's 512 registers, and the output pass runs one
  // workgroup per CU
  if (fmap != LA_FMAP_FAVOR && (long long)r * dv >= 128 * 128) per_cu = 1;
  return (long long)kComputeUnits * per_cu;
}

// Segments per head for the causal form: enough (head, segment) workgroups to
// fill the resident workgroup slots, each segment a whole number of chunks.
void plan_segments(int B, int H, int n, int fmap, int r, int dv, int dk, int gate, int* P, int* seg_len) {
  const int nchunks = (n + kChunk - 1) / kChunk;
  const long long BH = (long long)B * H;
  const long long target = resident_groups(fmap, r, dv, dk, gate);
  long long want = (target + BH - 1) / BH;
  if (want < 1) want = 1;
  if (want > nchunks) want = nchunks;
  const int seg_chunks = int((nchunks + want - 1) / want);
  *P = (nchunks + seg_chunks - 1) / seg_chunks;
  *seg_len = seg_chunks * kChunk;
}

// Segments for a ragged batch (la_forward_batch with cu_seqlens): the lengths
// live on the device, so the plan takes the total (at most total / 64 + nseq
// chunks over all sequences) and the longest: segments of equal length sized
// so that all sequences' segments give about one round of workgroups, and P
// segments cover the longest sequence. Sequences shorter than P segments
// leave the rest of their workgroups idle (they exit at once).
void plan_segments_ragged(int nseq, int H, int total, int max_len, int fmap, int r, int dv, int dk, int gate, int* P,
                          int* seg_len) {
  const long long target = resident_groups(fmap, r, dv, dk, gate);
  const long long chunks = ((long long)total + kChunk - 1) / kChunk + nseq;
  const int max_chunks = (max_len + kChunk - 1) / kChunk;
  long long seg_chunks = (chunks * H + target - 1) / target;
  if (seg_chunks < 1) seg_chunks = 1;
  if (seg_chunks > max_chunks) seg_chunks = max_chunks;
  *P = int((max_chunks + seg_chunks - 1) / seg_chunks);
  *seg_len = int(seg_chunks) * kChunk;
}

void plan_splits(int B, int H, int n, int* splits, int* split_len) {
  const int tiles = (n + 31) / 32;
  const long long BH = (long long)B * H;
  long long want = (kNonCausalGroups + BH - 1) / BH;
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  const int per = int((tiles + want - 1) / want);
  *split_len = per * 32;
  *splits = (n + *split_len - 1) / *split_len;
}

struct WsLayout {
  size_t S_off, z_off, logG_off, logGv_off, bytes;
  // causal d_v = 32 / FAVOR+ r = 32: zero-padded copies of V (and gv), the
  // output, omega, S0, z0, S_final and z_final
  size_t vpad_off = 0, gvpad_off = 0, opad_off = 0, ompad_off = 0, s0pad_off = 0, sfpad_off = 0, z0pad_off = 0,
         zfpad_off = 0;
};

// The causal chunk kernels tile the value columns and the FAVOR+ features 64
// wide: la_forward runs d_v = 32 and FAVOR+ r = 32 on zero-padded copies held
// in its workspace (columns.hip): V, gv and out with rows of kPadDv columns;
// omega with kPadR rows, the kernel masking features past r to zero; the
// states with rows and columns padded alike.
constexpr int kPadDv = 64, kPadR = 64;
bool padded_dv(int causal, int dv) { return causal != 0 && dv == 32; }
bool padded_r(int causal, const la_feature_map* f) { return causal != 0 && f->kind == LA_FMAP_FAVOR && f->r == 32; }

// Segment states (and GLA log-gates) of BH sequences cut into `pieces`.
WsLayout workspace_pieces(size_t BH, size_t pieces, size_t r, size_t dv, bool gla, bool outer = false) {
  WsLayout w{0, 0, 0, 0, 0};
  w.S_off = 0;
  w.z_off = round_up(BH * pieces * r * dv * 4, kAlign);
  w.logG_off = round_up(w.z_off + BH * pieces * r * 4, kAlign);
  w.logGv_off = w.bytes = gla ? round_up(w.logG_off + BH * pieces * r * 4, kAlign) : w.logG_off;
  if (gla && outer) w.bytes = round_up(w.logGv_off + BH * pieces * dv * 4, kAlign);
  return w;
}

WsLayout workspace_layout(const la_problem* p, const la_feature_map* f, int causal, int gate) {
  const size_t BH = (size_t)p->B * p->H;
  const bool pad_dv = padded_dv(causal, p->d_v), pad_r = padded_r(causal, f);
  const int dv = pad_dv ? kPadDv : p->d_v, rk = pad_r ? kPadR : f->r;
  WsLayout w{0, 0, 0, 0, 0};
  if (causal) {
    int P, L;
    plan_segments(p->B, p->H, p->n, f->kind, rk, dv, p->d_k, gate, &P, &L);
    if (P > 1) w = workspace_pieces(BH, (size_t)P, rk, dv, gate_has_input(gate), gate == LA_GATE_OUTER);
  } else {
    int sp, L;
    plan_splits(p->B, p->H, p->n, &sp, &L);
    w = workspace_pieces(BH, (size_t)sp, f->r, dv, false, false);
  }
  if (pad_dv || pad_r) {
    const size_t rows = BH * (size_t)p->n;
    size_t off = round_up(w.bytes, kAlign);
    auto take = [&](size_t& at, size_t bytes) {
      at = off;
      off = round_up(off + bytes, kAlign);
    };
    if (pad_dv) {
      take(w.vpad_off, rows * kPadDv * 2);  // bf16 (causal inputs and outputs are bf16)
      if (gate == LA_GATE_OUTER) take(w.gvpad_off, rows * kPadDv * 2);
      take(w.opad_off, rows * kPadDv * 2);
    }
    if (pad_r) take(w.ompad_off, (size_t)kPadR * p->d_k * 2);
    take(w.s0pad_off, BH * rk * dv * 4);
    take(w.sfpad_off, BH * rk * dv * 4);
    if (pad_r) {
      take(w.z0pad_off, BH * rk * 4);
      take(w.zfpad_off, BH * rk * 4);
    }
    w.bytes = off;
  }
  return w;
}

// The causal kernels of the plan's feature map.
la_status launch_causal(const FwdPlan& p) {
  switch (p.fmap) {
    case LA_FMAP_ELU1: return launch_causal_elu1(p);
    case LA_FMAP_IDENTITY: return launch_causal_ssm(p);
    case LA_FMAP_FAVOR: return launch_causal_favor(p);
  }
  return LA_ERR_UNSUPPORTED;
}

// Validation shared by la_forward and its size queries (no pointers inspected).
la_status check_forward_shape(const la_problem* p, const la_feature_map* f, int causal, const la_gate* g) {
  la_status st = check_problem(p);
  if (st != LA_OK) return st;
  if ((st = check_fmap(f, p->d_k)) != LA_OK) return st;
  if ((st = check_gate(g, false)) != LA_OK) return st;
  if (causal != 0 && causal != 1) return LA_ERR_INVALID_ARG;
  const int gk = gate_kind(g);
  if (!causal && gk != LA_GATE_NONE) return LA_ERR_INVALID_ARG;
  if (!shapes_built(f, p->d_k, p->d_v, causal != 0)) return LA_ERR_UNSUPPORTED;
  if (!causal && f->kind == LA_FMAP_IDENTITY) return LA_ERR_UNSUPPORTED;  // the state-space form is causal
  if (causal) {
    if (p->in_dtype != LA_BF16 || p->out_dtype != LA_BF16) return LA_ERR_UNSUPPORTED;
    if (f->kind == LA_FMAP_FAVOR && gate_has_input(gk)) return LA_ERR_UNSUPPORTED;
  }
  return LA_OK;
}

// The backward pass: causal elu+1 or identity features with any gate, or
// FAVOR+ without a gate input; bf16 in and out; (d_k, d_v) in {(64, 64),
// (64, 128), (128, 64), (128, 128)}.
la_status check_backward_shape(const la_problem* p, const la_feature_map* f, int causal, const la_gate* g) {
  la_status st = check_problem(p);
  if (st != LA_OK) return st;
  if ((st = check_fmap(f, p->d_k)) != LA_OK) return st;
  if ((st = check_gate(g, false)) != LA_OK) return st;
  if (causal != 0 && causal != 1) return LA_ERR_INVALID_ARG;
  const int gk = gate_kind(g);
  if (!causal && gk != LA_GATE_NONE) return LA_ERR_INVALID_ARG;
  if (!causal) {
    // the non-causal form: elu+1, fp32 vector-ALU kernels, gradients in the input dtype
    if (f->kind != LA_FMAP_ELU1 || p->in_dtype != p->out_dtype) return LA_ERR_UNSUPPORTED;
    return shapes_built(f, p->d_k, p->d_v, false) ? LA_OK : LA_ERR_UNSUPPORTED;
  }
  if (p->in_dtype != LA_BF16 || p->out_dtype != LA_BF16) return LA_ERR_UNSUPPORTED;
  if (f->kind == LA_FMAP_FAVOR) {
    // the chunked kernels on the materialised features (r wide), then back through the map
    if (gk != LA_GATE_NONE && gk != LA_GATE_DECAY) return LA_ERR_UNSUPPORTED;
    if (!in_set(p->d_k, {32, 64, 128})) return LA_ERR_UNSUPPORTED;
  } else if (f->kind != LA_FMAP_ELU1 && f->kind != LA_FMAP_IDENTITY) {
    return LA_ERR_UNSUPPORTED;
  }
  const int key = f->r * 1000 + p->d_v;
  if (key != 64064 && key != 64128 && key != 128064 && key != 128128) return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

// (r, d_v) = (128, 128) runs the (128, 64) kernels on the two halves of the
// value columns: every gradient is linear in g = dO / den and h = -(dO . o) /
// den, and both split into per-half sums (h = h_1 + h_2), so dQ, dK and dg are
// the sums of the halves' and dV their concatenation.
bool backward_in_halves(const la_problem* p, int r) { return r == 128 && p->d_v == 128; }

struct BwdWsLayout {
  size_t S_off, z_off, R_off, rh_off, G_off, h_off, dB_off, logG_off, Pw_off, logGv_off, s0h_off, fv_off, bytes;
  int P, L;
};

// Forward segment states, reverse segment states, g (bf16) and h per token;
// GLA adds dQ~ . Q~ per token and feature and the segments' summed log-gates
// (the selective scalar gate runs the GLA passes on its one input per token);
// the outer-product gate adds dO * o per token and value column (fp32) and
// the segments' summed value-side log-gates.
// The non-causal form: the splits' partial S, z (forward sums) and G, hq.
BwdWsLayout nc_bwd_workspace_layout(const la_problem* p, const la_feature_map* f) {
  BwdWsLayout w{};
  plan_splits(p->B, p->H, p->n, &w.P, &w.L);
  const size_t pieces = (size_t)p->B * p->H * w.P, r = (size_t)f->r, dv = (size_t)p->d_v;
  w.S_off = 0;
  w.z_off = round_up(pieces * r * dv * 4, kAlign);
  w.R_off = round_up(w.z_off + pieces * r * 4, kAlign);
  w.rh_off = round_up(w.R_off + pieces * r * dv * 4, kAlign);
  w.bytes = round_up(w.rh_off + pieces * r * 4, kAlign);
  return w;
}

BwdWsLayout bwd_workspace_layout(const la_problem* p_in, const la_feature_map* f, int gate, int causal = 1) {
  if (!causal) return nc_bwd_workspace_layout(p_in, f);
  la_problem half = *p_in;
  if (backward_in_halves(p_in, f->r)) half.d_v = p_in->d_v / 2;  // the halves run one after the other
  const la_problem* p = &half;
  BwdWsLayout w{};
  // the selective gate runs the GLA passes, on their segment plan
  plan_segments(p->B, p->H, p->n, f->kind, f->r, p->d_v, p->d_k, gate == LA_GATE_SEL ? LA_GATE_GLA : gate, &w.P,
                &w.L);
  const size_t BH = (size_t)p->B * p->H, r = (size_t)f->r, dv = (size_t)p->d_v, n = (size_t)p->n;
  const size_t states = BH * w.P * r * dv * 4, zs = BH * w.P * r * 4;
  w.S_off = 0;
  w.z_off = round_up(w.S_off + states, kAlign);
  w.R_off = round_up(w.z_off + zs, kAlign);
  w.rh_off = round_up(w.R_off + states, kAlign);
  w.G_off = round_up(w.rh_off + zs, kAlign);
  w.h_off = round_up(w.G_off + BH * n * dv * 2, kAlign);
  w.dB_off = round_up(w.h_off + BH * n * 4, kAlign);
  if (gate != LA_GATE_GLA && gate != LA_GATE_SEL && gate != LA_GATE_OUTER) {
    w.logG_off = w.Pw_off = w.logGv_off = w.bytes = w.dB_off;
  } else {
    const size_t n64 = (n + 63) / 64 * 64;  // dQ~ . Q~ is stored by whole chunks
    w.logG_off = round_up(w.dB_off + BH * n64 * r * 4, kAlign);
    w.Pw_off = w.logGv_off = w.bytes = round_up(w.logG_off + BH * w.P * r * 4, kAlign);
    if (gate == LA_GATE_OUTER) {
      w.logGv_off = round_up(w.Pw_off + BH * n * dv * 4, kAlign);
      w.bytes = round_up(w.logGv_off + BH * w.P * dv * 4, kAlign);
    }
  }
  // value-column halves: one half of a carried-in state at a time, dense
  w.s0h_off = w.bytes;
  if (backward_in_halves(p_in, f->r)) w.bytes = round_up(w.s0h_off + BH * r * dv * 4, kAlign);
  // FAVOR+: phi(Q), phi(K) and their gradients, bf16 [BH][n][r] each
  w.fv_off = w.bytes;
  if (f->kind == LA_FMAP_FAVOR) w.bytes = round_up(w.fv_off + 4 * BH * n * r * 2, kAlign);
  return w;
}

}  // namespace
}  // namespace la

using namespace la;

extern "C" {

int32_t la_abi_version(void) { return LA_ABI_VERSION; }

const char* la_status_str(int32_t s) {
  switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_INVALID_ARG: return "LA_ERR_INVALID_ARG";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE";
    case LA_ERR_ALIAS: return "LA_ERR_ALIAS";
    case LA_ERR_HIP: return "LA_ERR_HIP";
  }
  return "LA_ERR_UNKNOWN";
}

la_status la_forward_workspace_size(const la_problem* p, const la_feature_map* fmap, int32_t causal,
                                    const la_gate* gate, size_t* bytes) {
  if (bytes == nullptr) return LA_ERR_INVALID_ARG;
  la_status st = check_forward_shape(p, fmap, causal, gate);
  if (st != LA_OK) return st;
  *bytes = workspace_layout(p, fmap, causal, gate_kind(gate)).bytes;
  return LA_OK;
}

la_status la_forward_segments(const la_problem* p, const la_feature_map* fmap, int32_t causal,
                              const la_gate* gate, int32_t* segments, int32_t* segment_len) {
  if (segments == nullptr || segment_len == nullptr) return LA_ERR_INVALID_ARG;
  la_status st = check_forward_shape(p, fmap, causal, gate);
  if (st != LA_OK) return st;
  if (!causal) {
    *segments = 1;
    *segment_len = p->n;
    return LA_OK;
  }
  int P, L;
  // the plan of the kernels that run (64-wide copies for d_v = 32 and FAVOR+ r = 32)
  const int dv = padded_dv(causal, p->d_v) ? kPadDv : p->d_v, rk = padded_r(causal, fmap) ? kPadR : fmap->r;
  plan_segments(p->B, p->H, p->n, fmap->kind, rk, dv, p->d_k, gate_kind(gate), &P, &L);
  *segments = P;
  *segment_len = L;
  return LA_OK;
}

la_status la_forward(const la_problem* p, const void* Q, const void* K, const void* V,
                     const la_feature_map* fmap, int32_t causal, const la_gate* gate, const float* S0,
                     const float* z0, float* S_final, float* z_final, void* out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  la_status st = check_forward_shape(p, fmap, causal, gate);
  if (st != LA_OK) return st;
  if ((st = check_gate(gate, true)) != LA_OK) return st;
  const int gk = gate_kind(gate);
  if (Q == nullptr || K == nullptr || V == nullptr || out == nullptr) return LA_ERR_INVALID_ARG;
  if ((S0 == nullptr) != (z0 == nullptr)) return LA_ERR_INVALID_ARG;
  if ((S_final == nullptr) != (z_final == nullptr)) return LA_ERR_INVALID_ARG;
  if (!causal && S0 != nullptr) return LA_ERR_INVALID_ARG;
  for (const void* ptr : {Q, K, V, (const void*)out, (const void*)S0, (const void*)z0, (const void*)S_final,
                          (const void*)z_final})
    if (ptr != nullptr && !aligned16(ptr)) return LA_ERR_INVALID_ARG;

  const size_t BH = (size_t)p->B * p->H, n = (size_t)p->n, r = (size_t)fmap->r;
  const size_t isz = dtype_size(p->in_dtype);
  const Range rq = range_of(Q, BH * n * p->d_k * isz), rk = range_of(K, BH * n * p->d_k * isz),
              rv = range_of(V, BH * n * p->d_v * isz);
  const Range rg = range_of(gate_has_input(gk) ? gate->g : nullptr, BH * n * gate_input_per_token(gk, r) * isz);
  const Range rgv = range_of(gate_vinput(gate), BH * n * gate_vinput_per_token(gk, p->d_v) * isz);
  const Range rgam = range_of(gk == LA_GATE_DECAY ? gate->gamma : nullptr, (size_t)p->H * 4);
  const Range rom = range_of(fmap->kind == LA_FMAP_FAVOR ? fmap->omega : nullptr, r * p->d_k * isz);
  const Range rs0 = range_of(S0, BH * r * p->d_v * 4), rz0 = range_of(z0, BH * r * 4);
  const Range ro = range_of(out, BH * n * p->d_v * dtype_size(p->out_dtype));
  const Range rsf = range_of(S_final, BH * r * p->d_v * 4), rzf = range_of(z_final, BH * r * 4);
  const WsLayout wl = workspace_layout(p, fmap, causal, gk);
  const Range rws = range_of(wl.bytes ? workspace : nullptr, wl.bytes);
  for (Range o : {ro, rsf, rzf, rws}) {
    for (Range i : {rq, rk, rv, rg, rgv, rgam, rom, rs0, rz0})
      if (overlaps(o, i)) return LA_ERR_ALIAS;
  }
  if (overlaps(ro, rsf) || overlaps(ro, rzf) || overlaps(rsf, rzf) || overlaps(rws, ro) || overlaps(rws, rsf) ||
      overlaps(rws, rzf))
    return LA_ERR_ALIAS;
  if (wl.bytes > 0) {
    if (workspace == nullptr || workspace_bytes < wl.bytes) return LA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return LA_ERR_WORKSPACE;
  }

  FwdPlan plan{};
  plan.B = p->B;
  plan.H = p->H;
  plan.n = p->n;
  plan.dk = p->d_k;
  plan.dv = p->d_v;
  plan.r = fmap->r;
  plan.in_dtype = p->in_dtype;
  plan.out_dtype = p->out_dtype;
  plan.eps = p->eps;
  plan.fmap = fmap->kind;
  plan.gate = gk;
  plan.causal = causal;
  plan.tau = gate_has_input(gk) ? gate->tau : 1.f;
  plan.Q = Q;
  plan.K = K;
  plan.V = V;
  plan.g = gate_has_input(gk) ? gate->g : nullptr;
  plan.gv = gate_vinput(gate);
  plan.gamma = gk == LA_GATE_DECAY ? gate->gamma : nullptr;
  plan.omega = fmap->omega;
  plan.S0 = S0;
  plan.z0 = z0;
  plan.S_final = S_final;
  plan.z_final = z_final;
  plan.out = out;
  plan.nseq = p->B;
  plan.stream = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  // the segment states live at the workspace's start (the padded copies, if any, after them)
  const bool seg_ws = wl.S_off != wl.z_off;
  plan.ws_S = seg_ws ? reinterpret_cast<float*>(ws + wl.S_off) : nullptr;
  plan.ws_z = seg_ws ? reinterpret_cast<float*>(ws + wl.z_off) : nullptr;
  plan.ws_logG = (seg_ws && causal && gate_has_input(gk)) ? reinterpret_cast<float*>(ws + wl.logG_off) : nullptr;
  plan.ws_logGv = (seg_ws && causal && gk == LA_GATE_OUTER) ? reinterpret_cast<float*>(ws + wl.logGv_off) : nullptr;
  const bool pad_dv = padded_dv(causal, p->d_v), pad_r = padded_r(causal, fmap);
  if (pad_dv || pad_r) {
    // the 64-wide kernels on zero-padded copies, then the real part back
    const long long heads = (long long)BH;
    const int rr = int(r), dv = p->d_v, rk = pad_r ? kPadR : rr, dvk = pad_dv ? kPadDv : dv;
    const hipStream_t hs = plan.stream;
    plan.dv = dvk;
    plan.r = rk;
    plan.r_valid = pad_r ? rr : 0;
    if (pad_dv) {
      const int nn = p->n;
      if ((st = launch_copy_block(V, ws + wl.vpad_off, heads, nn, dv, nn, dvk, 2, hs)) != LA_OK) return st;
      plan.V = ws + wl.vpad_off;
      if (gk == LA_GATE_OUTER) {
        if ((st = launch_copy_block(plan.gv, ws + wl.gvpad_off, heads, nn, dv, nn, dvk, 2, hs)) != LA_OK) return st;
        plan.gv = ws + wl.gvpad_off;
      }
      plan.out = ws + wl.opad_off;
    }
    if (pad_r) {
      if ((st = launch_copy_block(fmap->omega, ws + wl.ompad_off, 1, rr, p->d_k, rk, p->d_k, 2, hs)) != LA_OK)
        return st;
      plan.omega = ws + wl.ompad_off;
    }
    if (S0 != nullptr) {
      if ((st = launch_copy_block(S0, ws + wl.s0pad_off, heads, rr, dv, rk, dvk, 4, hs)) != LA_OK) return st;
      plan.S0 = reinterpret_cast<const float*>(ws + wl.s0pad_off);
      if (pad_r) {
        if ((st = launch_copy_block(z0, ws + wl.z0pad_off, heads, 1, rr, 1, rk, 4, hs)) != LA_OK) return st;
        plan.z0 = reinterpret_cast<const float*>(ws + wl.z0pad_off);
      }
    }
    if (S_final != nullptr) {
      plan.S_final = reinterpret_cast<float*>(ws + wl.sfpad_off);
      if (pad_r) plan.z_final = reinterpret_cast<float*>(ws + wl.zfpad_off);
    }
    plan_segments(p->B, p->H, p->n, fmap->kind, rk, dvk, p->d_k, gk, &plan.P, &plan.seg_len);
    if ((st = launch_causal(plan)) != LA_OK) return st;
    if (pad_dv && (st = launch_copy_block(ws + wl.opad_off, out, heads, p->n, dvk, p->n, dv, 2, hs)) != LA_OK)
      return st;
    if (S_final != nullptr) {
      if ((st = launch_copy_block(ws + wl.sfpad_off, S_final, heads, rk, dvk, rr, dv, 4, hs)) != LA_OK) return st;
      if (pad_r && (st = launch_copy_block(ws + wl.zfpad_off, z_final, heads, 1, rk, 1, rr, 4, hs)) != LA_OK)
        return st;
    }
    return LA_OK;
  }
  if (causal) {
    plan_segments(p->B, p->H, p->n, fmap->kind, fmap->r, p->d_v, p->d_k, gk, &plan.P, &plan.seg_len);
    return launch_causal(plan);
  }
  plan_splits(p->B, p->H, p->n, &plan.splits, &plan.split_len);
  return launch_noncausal(plan);
}

// ---- serving batches

namespace {
// Validation of a batch description shared by la_forward_batch and its size
// query; *eff gets num_seqs sequences of max_seqlen tokens.
la_status check_batch(const la_problem* p, const la_batch* b, const la_feature_map* f, const la_gate* g,
                      la_problem* eff) {
  if (b == nullptr) return LA_ERR_INVALID_ARG;
  la_status st = check_forward_shape(p, f, 1, g);
  if (st != LA_OK) return st;
  if ((b->flags & ~(LA_SLOT_READ | LA_SLOT_WRITE)) != 0) return LA_ERR_INVALID_ARG;
  *eff = *p;
  if (b->cu_seqlens != nullptr) {
    if (p->B != 1 || b->num_seqs < 1 || b->max_seqlen < 1 || b->max_seqlen > p->n) return LA_ERR_INVALID_ARG;
    eff->B = b->num_seqs;
    eff->n = b->max_seqlen;
  } else if (b->num_seqs != p->B || b->max_seqlen != p->n) {
    return LA_ERR_INVALID_ARG;
  }
  if (b->flags != 0 && b->num_slots < 1) return LA_ERR_INVALID_ARG;
  // d_v = 32 only on short steps (the recurrent kernel); the chunk kernels'
  // padded copies are a la_forward workspace feature
  if ((p->d_v == 32 || (f->kind == LA_FMAP_FAVOR && f->r == 32)) &&
      !(b->cu_seqlens == nullptr && p->n <= kMaxStepTokens))
    return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

// Segment plan and workspace of a validated batch.
WsLayout batch_plan(const la_problem* p, const la_batch* b, const la_problem& eff, const la_feature_map* f, int gate,
                    int* P, int* seg_len) {
  if (b->cu_seqlens != nullptr)
    plan_segments_ragged(eff.B, p->H, p->n, eff.n, f->kind, f->r, p->d_v, p->d_k, gate, P, seg_len);
  else
    plan_segments(eff.B, p->H, eff.n, f->kind, f->r, p->d_v, p->d_k, gate, P, seg_len);
  if (*P <= 1) return WsLayout{0, 0, 0, 0, 0};
  return workspace_pieces((size_t)eff.B * p->H, (size_t)*P, f->r, p->d_v, gate_has_input(gate),
                          gate == LA_GATE_OUTER);
}
}  // namespace

la_status la_forward_batch_workspace_size(const la_problem* p, const la_batch* batch, const la_feature_map* fmap,
                                          const la_gate* gate, size_t* bytes) {
  if (bytes == nullptr) return LA_ERR_INVALID_ARG;
  la_problem eff;
  la_status st = check_batch(p, batch, fmap, gate, &eff);
  if (st != LA_OK) return st;
  int P, L;
  *bytes = batch_plan(p, batch, eff, fmap, gate_kind(gate), &P, &L).bytes;
  return LA_OK;
}

la_status la_forward_batch(const la_problem* p, const la_batch* batch, const void* Q, const void* K, const void* V,
                           const la_feature_map* fmap, const la_gate* gate, void* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  la_problem eff;
  la_status st = check_batch(p, batch, fmap, gate, &eff);
  if (st != LA_OK) return st;
  if ((st = check_gate(gate, true)) != LA_OK) return st;
  const int gk = gate_kind(gate);
  if (Q == nullptr || K == nullptr || V == nullptr || out == nullptr) return LA_ERR_INVALID_ARG;
  const bool slots = batch->flags != 0;
  if (slots && (batch->S == nullptr || batch->z == nullptr || batch->slot_ids == nullptr)) return LA_ERR_INVALID_ARG;
  for (const void* ptr : {Q, K, V, (const void*)out, (const void*)(slots ? batch->S : nullptr),
                          (const void*)(slots ? batch->z : nullptr)})
    if (ptr != nullptr && !aligned16(ptr)) return LA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(batch->cu_seqlens) & 3) != 0 ||
      (slots && (reinterpret_cast<uintptr_t>(batch->slot_ids) & 3) != 0))
    return LA_ERR_INVALID_ARG;

  const size_t BH = (size_t)p->B * p->H, n = (size_t)p->n, r = (size_t)fmap->r;
  const size_t isz = dtype_size(p->in_dtype);
  const Range rq = range_of(Q, BH * n * p->d_k * isz), rk = range_of(K, BH * n * p->d_k * isz),
              rv = range_of(V, BH * n * p->d_v * isz);
  const Range rg = range_of(gate_has_input(gk) ? gate->g : nullptr, BH * n * gate_input_per_token(gk, r) * isz);
  const Range rgv = range_of(gate_vinput(gate), BH * n * gate_vinput_per_token(gk, p->d_v) * isz);
  const Range rgam = range_of(gk == LA_GATE_DECAY ? gate->gamma : nullptr, (size_t)p->H * 4);
  const Range rom = range_of(fmap->kind == LA_FMAP_FAVOR ? fmap->omega : nullptr, r * p->d_k * isz);
  const Range rcu = range_of(batch->cu_seqlens, ((size_t)batch->num_seqs + 1) * 4);
  const Range rsl = range_of(slots ? batch->slot_ids : nullptr, (size_t)batch->num_seqs * 4);
  const size_t pool = slots ? (size_t)batch->num_slots * p->H : 0;
  const Range rS = range_of(slots ? batch->S : nullptr, pool * r * p->d_v * 4),
              rz = range_of(slots ? batch->z : nullptr, pool * r * 4);
  const Range ro = range_of(out, BH * n * p->d_v * dtype_size(p->out_dtype));
  int P, seg_len;
  const WsLayout wl = batch_plan(p, batch, eff, fmap, gk, &P, &seg_len);
  const Range rws = range_of(wl.bytes ? workspace : nullptr, wl.bytes);
  for (Range o : {ro, rS, rz, rws})
    for (Range i : {rq, rk, rv, rg, rgv, rgam, rom, rcu, rsl})
      if (overlaps(o, i)) return LA_ERR_ALIAS;
  if (overlaps(ro, rS) || overlaps(ro, rz) || overlaps(rS, rz) || overlaps(rws, ro) || overlaps(rws, rS) ||
      overlaps(rws, rz))
    return LA_ERR_ALIAS;
  if (wl.bytes > 0) {
    if (workspace == nullptr || workspace_bytes < wl.bytes) return LA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return LA_ERR_WORKSPACE;
  }

  FwdPlan plan{};
  plan.B = p->B;
  plan.H = p->H;
  plan.n = p->n;
  plan.dk = p->d_k;
  plan.dv = p->d_v;
  plan.r = fmap->r;
  plan.in_dtype = p->in_dtype;
  plan.out_dtype = p->out_dtype;
  plan.eps = p->eps;
  plan.fmap = fmap->kind;
  plan.gate = gk;
  plan.causal = 1;
  plan.tau = gate_has_input(gk) ? gate->tau : 1.f;
  plan.Q = Q;
  plan.K = K;
  plan.V = V;
  plan.g = gate_has_input(gk) ? gate->g : nullptr;
  plan.gv = gate_vinput(gate);
  plan.gamma = gk == LA_GATE_DECAY ? gate->gamma : nullptr;
  plan.omega = fmap->omega;
  plan.nseq = eff.B;
  plan.cu = batch->cu_seqlens;
  plan.slot = slots ? batch->slot_ids : nullptr;
  plan.nslot = slots ? batch->num_slots : 0;
  if (batch->flags & LA_SLOT_READ) {
    plan.S0 = batch->S;
    plan.z0 = batch->z;
  }
  if (batch->flags & LA_SLOT_WRITE) {
    plan.S_final = batch->S;
    plan.z_final = batch->z;
  }
  plan.out = out;
  plan.stream = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  plan.ws_S = wl.bytes ? reinterpret_cast<float*>(ws + wl.S_off) : nullptr;
  plan.ws_z = wl.bytes ? reinterpret_cast<float*>(ws + wl.z_off) : nullptr;
  plan.ws_logG = (wl.bytes && gate_has_input(gk)) ? reinterpret_cast<float*>(ws + wl.logG_off) : nullptr;
  plan.ws_logGv = (wl.bytes && gk == LA_GATE_OUTER) ? reinterpret_cast<float*>(ws + wl.logGv_off) : nullptr;
  plan.P = P;
  plan.seg_len = seg_len;
  if (batch->cu_seqlens == nullptr && p->n <= kMaxStepTokens) {
    // a few tokens per sequence: the recurrent step kernel streams each state
    // once and takes the tokens in order with the state in registers
    DecodePlan dp{};
    dp.m = p->n;
    dp.B = p->B;
    dp.H = p->H;
    dp.dk = p->d_k;
    dp.dv = p->d_v;
    dp.r = fmap->r;
    dp.in_dtype = p->in_dtype;
    dp.out_dtype = p->out_dtype;
    dp.eps = p->eps;
    dp.fmap = fmap->kind;
    dp.gate = gk;
    dp.tau = plan.tau;
    dp.S = batch->S;
    dp.z = batch->z;
    dp.q = Q;
    dp.k = K;
    dp.v = V;
    dp.g = plan.g;
    dp.gv = plan.gv;
    dp.gamma = plan.gamma;
    dp.omega = fmap->omega;
    dp.out = out;
    dp.slot = plan.slot;
    dp.nslot = plan.nslot;
    dp.flags = batch->flags;
    dp.stream = plan.stream;
    const la_status ds = launch_decode(dp);
    if (ds != LA_ERR_UNSUPPORTED) return ds;
  }
  return launch_causal(plan);
}

la_status la_decode_step(const la_problem* p, float* S, float* z, const void* q, const void* k, const void* v,
                         const la_feature_map* fmap, const la_gate* gate, void* out, void* stream) {
  la_status st = check_problem(p);
  if (st != LA_OK) return st;
  if (p->n != 1) return LA_ERR_INVALID_ARG;
  if ((st = check_fmap(fmap, p->d_k)) != LA_OK) return st;
  if ((st = check_gate(gate, true)) != LA_OK) return st;
  if (S == nullptr || z == nullptr || q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return LA_ERR_INVALID_ARG;
  for (const void* ptr : {(const void*)S, (const void*)z, q, k, v, (const void*)out})
    if (!aligned16(ptr)) return LA_ERR_INVALID_ARG;
  if (!shapes_built(fmap, p->d_k, p->d_v, false)) return LA_ERR_UNSUPPORTED;
  const int gk = gate_kind(gate);
  const size_t BH = (size_t)p->B * p->H, r = (size_t)fmap->r, isz = dtype_size(p->in_dtype);
  const Range rS = range_of(S, BH * r * p->d_v * 4), rz = range_of(z, BH * r * 4);
  const Range rq = range_of(q, BH * p->d_k * isz), rk = range_of(k, BH * p->d_k * isz),
              rv = range_of(v, BH * p->d_v * isz);
  const Range rg = range_of(gate_has_input(gk) ? gate->g : nullptr, BH * gate_input_per_token(gk, r) * isz);
  const Range rgv = range_of(gate_vinput(gate), BH * gate_vinput_per_token(gk, p->d_v) * isz);
  const Range rgam = range_of(gk == LA_GATE_DECAY ? gate->gamma : nullptr, (size_t)p->H * 4);
  const Range rom = range_of(fmap->kind == LA_FMAP_FAVOR ? fmap->omega : nullptr, r * p->d_k * isz);
  const Range ro = range_of(out, BH * p->d_v * dtype_size(p->out_dtype));
  for (Range o : {rS, rz, ro})
    for (Range i : {rq, rk, rv, rg, rgv, rgam, rom})
      if (overlaps(o, i)) return LA_ERR_ALIAS;
  if (overlaps(rS, rz) || overlaps(ro, rS) || overlaps(ro, rz)) return LA_ERR_ALIAS;

  DecodePlan plan{};
  plan.B = p->B;
  plan.H = p->H;
  plan.dk = p->d_k;
  plan.dv = p->d_v;
  plan.r = fmap->r;
  plan.in_dtype = p->in_dtype;
  plan.out_dtype = p->out_dtype;
  plan.eps = p->eps;
  plan.fmap = fmap->kind;
  plan.gate = gk;
  plan.tau = gate_has_input(gk) ? gate->tau : 1.f;
  plan.S = S;
  plan.z = z;
  plan.q = q;
  plan.k = k;
  plan.v = v;
  plan.g = gate_has_input(gk) ? gate->g : nullptr;
  plan.gv = gate_vinput(gate);
  plan.gamma = gk == LA_GATE_DECAY ? gate->gamma : nullptr;
  plan.omega = fmap->omega;
  plan.out = out;
  plan.flags = 3;
  plan.stream = static_cast<hipStream_t>(stream);
  return launch_decode(plan);
}

la_status la_backward_workspace_size(const la_problem* p, const la_feature_map* fmap, int32_t causal,
                                     const la_gate* gate, size_t* bytes) {
  if (bytes == nullptr) return LA_ERR_INVALID_ARG;
  la_status st = check_backward_shape(p, fmap, causal, gate);
  if (st != LA_OK) return st;
  *bytes = bwd_workspace_layout(p, fmap, gate_kind(gate), causal).bytes;
  return LA_OK;
}

la_status la_backward(const la_problem* p, const void* Q, const void* K, const void* V, const void* dO,
                      const la_feature_map* fmap, int32_t causal, const la_gate* gate, const float* S0,
                      const float* z0, void* dQ, void* dK, void* dV, void* dg, void* dgv, void* workspace,
                      size_t workspace_bytes, void* stream) {
  la_status st = check_backward_shape(p, fmap, causal, gate);
  if (st != LA_OK) return st;
  if ((st = check_gate(gate, true)) != LA_OK) return st;
  const int gk = gate_kind(gate);
  if (Q == nullptr || K == nullptr || V == nullptr || dO == nullptr || dQ == nullptr || dK == nullptr ||
      dV == nullptr)
    return LA_ERR_INVALID_ARG;
  const bool sel = gk == LA_GATE_SEL, outer = gk == LA_GATE_OUTER;
  if ((dg != nullptr) != (gk == LA_GATE_GLA || sel || outer)) return LA_ERR_INVALID_ARG;
  if ((dgv != nullptr) != outer) return LA_ERR_INVALID_ARG;
  if ((S0 == nullptr) != (z0 == nullptr)) return LA_ERR_INVALID_ARG;
  if (!causal && S0 != nullptr) return LA_ERR_INVALID_ARG;  // the non-causal form has no carried state
  for (const void* ptr : {Q, K, V, dO, (const void*)S0, (const void*)z0, (const void*)dQ, (const void*)dK,
                          (const void*)dV, (const void*)dg, (const void*)dgv})
    if (ptr != nullptr && !aligned16(ptr)) return LA_ERR_INVALID_ARG;
  const size_t BH = (size_t)p->B * p->H, n = (size_t)p->n, r = (size_t)fmap->r, isz = dtype_size(p->in_dtype);
  const size_t qk = BH * n * p->d_k * isz, vv = BH * n * p->d_v * isz, gg = BH * n * (sel ? 1 : r) * 2;
  const Range rq = range_of(Q, qk), rk = range_of(K, qk), rv = range_of(V, vv), rdo = range_of(dO, vv);
  const Range rgam = range_of(gk == LA_GATE_DECAY ? gate->gamma : nullptr, (size_t)p->H * 4);
  const Range rgl = range_of(gate_has_input(gk) ? gate->g : nullptr, gg);
  const Range rgv = range_of(outer ? gate->gv : nullptr, vv);
  const Range rs0 = range_of(S0, BH * r * p->d_v * 4), rz0 = range_of(z0, BH * r * 4);
  const Range rom = range_of(fmap->kind == LA_FMAP_FAVOR ? fmap->omega : nullptr, r * p->d_k * isz);
  const Range rdq = range_of(dQ, qk), rdk = range_of(dK, qk), rdv = range_of(dV, vv), rdg = range_of(dg, gg);
  const Range rdgv = range_of(dgv, vv);
  const BwdWsLayout wl = bwd_workspace_layout(p, fmap, gk, causal);
  const Range rws = range_of(workspace, wl.bytes);
  const Range outs[] = {rdq, rdk, rdv, rdg, rdgv, rws};
  for (Range o : outs)
    for (Range i : {rq, rk, rv, rdo, rgam, rgl, rgv, rs0, rz0, rom})
      if (overlaps(o, i)) return LA_ERR_ALIAS;
  for (size_t a = 0; a < 6; ++a)
    for (size_t c = a + 1; c < 6; ++c)
      if (overlaps(outs[a], outs[c])) return LA_ERR_ALIAS;
  if (workspace == nullptr || workspace_bytes < wl.bytes) return LA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return LA_ERR_WORKSPACE;

  BwdPlan plan{};
  plan.B = p->B;
  plan.H = p->H;
  plan.n = p->n;
  plan.dk = p->d_k;
  plan.dv = p->d_v;
  plan.r = fmap->r;
  plan.in_dtype = p->in_dtype;
  plan.out_dtype = p->out_dtype;
  plan.eps = p->eps;
  plan.fmap = fmap->kind;
  plan.gate = sel ? LA_GATE_GLA : gk;  // the selective gate: the GLA passes, its input broadcast over features
  plan.causal = 1;
  plan.Q = Q;
  plan.K = K;
  plan.V = V;
  plan.gamma = gk == LA_GATE_DECAY ? gate->gamma : nullptr;
  plan.g = gate_has_input(gk) ? gate->g : nullptr;
  plan.gv = outer ? gate->gv : nullptr;
  plan.tau = gate_has_input(gk) ? gate->tau : 1.f;
  plan.S0 = S0;
  plan.z0 = z0;
  plan.P = wl.P;
  plan.seg_len = wl.L;
  plan.nseq = p->B;
  plan.stream = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  plan.ws_S = reinterpret_cast<float*>(ws + wl.S_off);
  plan.ws_z = reinterpret_cast<float*>(ws + wl.z_off);
  plan.ws_R = reinterpret_cast<float*>(ws + wl.R_off);
  plan.ws_rh = reinterpret_cast<float*>(ws + wl.rh_off);
  plan.ws_G = ws + wl.G_off;
  plan.ws_h = reinterpret_cast<float*>(ws + wl.h_off);
  if (gk == LA_GATE_GLA || sel || outer) {
    plan.ws_dB = reinterpret_cast<float*>(ws + wl.dB_off);
    plan.ws_logG = reinterpret_cast<float*>(ws + wl.logG_off);
    plan.dg = dg;
    plan.g_scalar = sel ? 1 : 0;  // the selective gate: one input per token, dg summed over features in pass B
  }
  if (outer) {
    plan.ws_P = reinterpret_cast<float*>(ws + wl.Pw_off);
    plan.ws_logGv = reinterpret_cast<float*>(ws + wl.logGv_off);
    plan.dgv = dgv;
  }
  plan.dO = dO;
  plan.dQ = dQ;
  plan.dK = dK;
  plan.dV = dV;
  if (!causal) {  // splits of the sequence: wl.P of wl.L tokens
    plan.causal = 0;
    plan.splits = wl.P;
    plan.split_len = wl.L;
    return launch_noncausal_backward(plan);
  }
  // FAVOR+: the kernels run on the materialised features phi(Q), phi(K) and
  // write d phi, which favor_vjp takes back through the map into dQ, dK
  const bool favor = fmap->kind == LA_FMAP_FAVOR;
  bf16_bits* fv = reinterpret_cast<bf16_bits*>(ws + wl.fv_off);
  const size_t fsz = BH * n * r;
  if (favor) {
    if ((st = launch_favor_features(Q, p->in_dtype, (long long)(BH * n), p->d_k, fmap->r, fmap->omega, fv,
                                    plan.stream)) != LA_OK ||
        (st = launch_favor_features(K, p->in_dtype, (long long)(BH * n), p->d_k, fmap->r, fmap->omega, fv + fsz,
                                    plan.stream)) != LA_OK)
      return st;
    plan.Q = fv;
    plan.K = fv + fsz;
    plan.dQ = fv + 2 * fsz;
    plan.dK = fv + 3 * fsz;
    plan.fmap = kFmapPrecomputed;
    plan.dk = fmap->r;
  }
  if (backward_in_halves(p, fmap->r)) {
    const int half = p->d_v / 2;
    BwdPlan hp = plan;
    hp.dv = half;
    hp.ldv = p->d_v;
    float* s0h = reinterpret_cast<float*>(ws + wl.s0h_off);
    for (int k = 0; k < 2; ++k) {
      hp.V = static_cast<const bf16_bits*>(V) + k * half;
      hp.dO = static_cast<const bf16_bits*>(dO) + k * half;
      hp.dV = static_cast<bf16_bits*>(dV) + k * half;
      if (outer) {  // this half's value columns of gv and dgv (row stride d_v)
        hp.gv = static_cast<const bf16_bits*>(gate->gv) + k * half;
        hp.dgv = static_cast<bf16_bits*>(dgv) + k * half;
      }
      hp.accum = k;
      if (S0 != nullptr) {  // this half's columns of the carried-in state, dense ([BH][r][half]); z0 is shared
        if (hipMemcpy2DAsync(s0h, half * sizeof(float), S0 + k * half, p->d_v * sizeof(float), half * sizeof(float),
                             BH * r, hipMemcpyDeviceToDevice, plan.stream) != hipSuccess)
          return LA_ERR_HIP;
        hp.S0 = s0h;
      }
      if ((st = launch_backward(hp)) != LA_OK) return st;
    }
  } else if ((st = launch_backward(plan)) != LA_OK) {
    return st;
  }
  if (favor) {
    if ((st = launch_favor_vjp(fv + 2 * fsz, fv, Q, p->in_dtype, (long long)(BH * n), p->d_k, fmap->r, fmap->omega, dQ,
                               p->out_dtype, plan.stream)) != LA_OK)
      return st;
    return launch_favor_vjp(fv + 3 * fsz, fv + fsz, K, p->in_dtype, (long long)(BH * n), p->d_k, fmap->r, fmap->omega,
                            dK, p->out_dtype, plan.stream);
  }
  return LA_OK;
}

la_status la_softmax_attention(const la_problem* p, const void* Q, const void* K, const void* V, int32_t causal,
                               float scale, void* out, void* stream) {
  la_status st = check_problem(p);
  if (st != LA_OK) return st;
  if (causal != 0 && causal != 1) return LA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return LA_ERR_INVALID_ARG;
  if (Q == nullptr || K == nullptr || V == nullptr || out == nullptr) return LA_ERR_INVALID_ARG;
  for (const void* ptr : {Q, K, V, (const void*)out})
    if (!aligned16(ptr)) return LA_ERR_INVALID_ARG;
  if (p->in_dtype != LA_BF16 || p->out_dtype != LA_BF16) return LA_ERR_UNSUPPORTED;
  if (p->d_k != p->d_v || !in_set(p->d_k, {64, 128})) return LA_ERR_UNSUPPORTED;
  const size_t bytes = (size_t)p->B * p->H * p->n * p->d_k * 2;
  const Range ro = range_of(out, bytes);
  for (Range i : {range_of(Q, bytes), range_of(K, bytes), range_of(V, bytes)})
    if (overlaps(ro, i)) return LA_ERR_ALIAS;
  if ((long long)p->B * p->H * ((p->n + 127) / 128) > 0x7fffffffLL) return LA_ERR_UNSUPPORTED;
  SoftmaxPlan plan{p->B, p->H, p->n, p->d_k, causal, scale, Q, K, V, out, static_cast<hipStream_t>(stream)};
  return launch_softmax(plan);
}

la_status la_timing_begin(void* const* events, int32_t n_events) {
  if (n_events < 0 || (n_events > 0 && events == nullptr)) return LA_ERR_INVALID_ARG;
  if (t_launch_timer != nullptr) return LA_ERR_INVALID_ARG;  // brackets do not nest
  for (int32_t i = 0; i < n_events; ++i)
    if (events[i] == nullptr) return LA_ERR_INVALID_ARG;
  t_timer_slot = LaunchTimer{events, n_events, 0, false};
  t_launch_timer = &t_timer_slot;
  return LA_OK;
}

la_status la_timing_end(void* stream, int32_t* launches) {
  if (t_launch_timer == nullptr) return LA_ERR_INVALID_ARG;
  LaunchTimer* t = t_launch_timer;
  mark_launch(static_cast<hipStream_t>(stream));  // the end of the last launch
  t_launch_timer = nullptr;
  if (launches != nullptr) *launches = t->used - 1;
  return t->failed ? LA_ERR_HIP : LA_OK;
}

la_status la_feature_map_apply(const la_feature_map* fmap, int64_t rows, int32_t d_k, int32_t in_dtype,
                               const void* X, float* out, void* stream) {
  if (rows < 1 || d_k < 1 || !valid_dtype(in_dtype)) return LA_ERR_INVALID_ARG;
  la_status st = check_fmap(fmap, d_k);
  if (st != LA_OK) return st;
  if (X == nullptr || out == nullptr || !aligned16(X) || !aligned16(out)) return LA_ERR_INVALID_ARG;
  if (fmap->kind == LA_FMAP_IDENTITY) return LA_ERR_UNSUPPORTED;  // nothing to apply
  if (!in_set(d_k, {32, 64, 128})) return LA_ERR_UNSUPPORTED;
  if (fmap->kind == LA_FMAP_FAVOR && !in_set(fmap->r, {32, 64, 128, 256})) return LA_ERR_UNSUPPORTED;
  if ((rows + 63) / 64 > 0x7fffffffLL) return LA_ERR_UNSUPPORTED;
  const size_t isz = dtype_size(in_dtype);
  const Range rx = range_of(X, (size_t)rows * d_k * isz), ro = range_of(out, (size_t)rows * fmap->r * 4);
  const Range rom = range_of(fmap->kind == LA_FMAP_FAVOR ? fmap->omega : nullptr, (size_t)fmap->r * d_k * isz);
  if (overlaps(ro, rx) || overlaps(ro, rom)) return LA_ERR_ALIAS;
  FmapPlan plan{rows, d_k, fmap->r, in_dtype, fmap->kind, X, fmap->omega, out, static_cast<hipStream_t>(stream)};
  return launch_feature_map(plan);
}

}  // extern "C"
