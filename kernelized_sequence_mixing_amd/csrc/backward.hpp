// Backward pass of the chunkwise causal kernel (elu+1 features or the
// state-space form's identity features without a normaliser; no gate, the
// RetNet decay or the diagonal GLA gate), for training with the parallel form ("Recurrent
// Reformulation", "Linear Attention Mechanisms" (dileepadev.github.io): the
// layer is trained in parallel and served as an RNN).
//
// For a loss with dL/do_i = dO_i, write the forward output o_i = num_i / den_i
// with num_i = sum_{j<=i} w_ij v_j, den_i = sum_{j<=i} w_ij + eps,
// w_ij = phi(q_i).phi(k_j) gamma^(i-j). Then
//   g_i = dO_i / den_i,  h_i = -(dO_i . o_i) / den_i,  dW_ij = g_i . v_j + h_i,
//   dphi(q_i) = sum_{j<=i} dW_ij gamma^(i-j) phi(k_j)   (+ the carried state's share)
//   dphi(k_j) = sum_{i>=j} dW_ij gamma^(i-j) phi(q_i),  dv_j = sum_{i>=j} w_ij g_i,
// and dq = dphi(q) phi'(q), dk = dphi(k) phi'(k) with phi'(x) = min(phi(x), 1)
// for elu+1 (1 for x > 0, exp(x) = phi(x) below). The sums over j <= i run
// chunkwise exactly like the forward: intra-chunk masked products plus the
// forward state (S, z) entering the chunk. The sums over i >= j run the other
// way: intra-chunk products plus the reverse state R = sum_{later i}
// gamma^(..) phi(q_i) [g_i, h_i]^T entering the chunk from its end.
//
// Kernels (one workgroup of four waves per (head, segment), as the forward):
//   forward segment pass + scan  -> S, z entering each segment (forward code)
//   bwd_pass_a   chunks in order: recompute den, o; g, h (to the workspace);
//                dW; dq = (Phi_k^T dW^T + gamma^(t+1) (S^T g + z h))^T phi'(q)
//   bwd_rstate   each segment's own reverse state, rows read back to front
//   scan (reverse)                -> R entering each segment from its end
//   bwd_pass_b   chunks back to front: W, dW; dv = W^T g + Phi_k R'^T-part;
//                dk = (Phi_q^T dW + R [v; 1])^T phi'(k); then R <- gamma^L R + ...
// With the diagonal GLA gate ("Gating and Selective State Updates",
// dileepadev page) the chunk tiles hold Q~ = e^{b} phi(q), K~ = e^{-b} phi(k)
// as in the forward (b the chunk's inclusive summed log-gate per feature), the
// same passes give dQ~ and dK~, and the gate's gradient follows from
// dB = dQ~ . Q~ - dK~ . K~ (the gradient of the cumulative log-gate; the
// carried-in state, weighted by e^{B}, enters through dQ~) by a suffix sum
// over the sequence: pass B sums the segment's own tokens back to front and
// starts from d log alpha at the next segment's first token, which is the
// row-wise product of the forward and reverse states there (scaling the state
// that crosses a boundary is scaling every pair weight across it). The
// reverse state of a segment runs in natural row order (bwd_rstate_gla).
// All LDS tiles use the per-row chunk permutation of FeatTile.
#pragma once

#include "chunked.hpp"

namespace la {

struct BwdArgs {
  const bf16* Q;
  const bf16* K;
  const bf16* V;
  const bf16* dO;
  const float* gamma;
  const float* S_in;  // pass A: forward state entering each segment (nullable)
  const float* z_in;
  long long in_head, in_seg;  // S_in element strides between heads and segments
  bf16* G;                    // [B H n E] g_i (pass A writes, passes R / B read)
  float* h;                   // [B H n] h_i
  float* R_ws;                // [B H P R E] reverse state deltas (bwd_rstate), then R entering (scan)
  float* rh_ws;               // [B H P R]
  bf16* dQ;
  bf16* dK;
  bf16* dV;
  // GLA gate (per feature: alpha = sigmoid(g)^(1/tau))
  const bf16* gl;  // [B H n R] raw gate input
  float* dB;       // dQ~ . Q~ (pass A, read by pass B), in the order of dbq_at
  float* logG;     // [B H P R] summed log-gate of each segment (bwd_rstate_gla)
  bf16* dg;        // [B H n R]
  // outer-product gate (per value column: beta = sigmoid(gv)^(1/tau))
  const bf16* gvl;  // [B H n ldv] raw value-side gate input
  float* Pw;        // [B H n E] g * num (= dO * o) per token and column (pass A), read by pass B
  float* logGv;     // [B H P E] summed value-side log-gate of each segment
  bf16* dgv;        // [B H n ldv]
  int ldv;         // elements between rows of V, dO, dV, gv and dgv (a value-column half of a wider V)
  int accum;       // add dQ, dK, dg to what the arrays hold (the second value-column half)
  int H, n, P, seg_len;
  float eps, inv_tau;
};

// Four gradient entries stored as bf16, or added to the stored ones prev (the
// gradients are sums over value columns; a wide V runs in column halves).
__device__ __forceinline__ void store_grad4(bf16* p, const float (&x)[4], bool accum, bf16x4 prev) {
  float y[4] = {x[0], x[1], x[2], x[3]};
  if (accum) {
#pragma unroll
    for (int u = 0; u < 4; ++u) y[u] += to_f32(prev[u]);
  }
  *reinterpret_cast<bf16x4*>(p) = pack4(y[0], y[1], y[2], y[3]);
}

// The stored entries that the second value-column half adds to, loaded at the
// start of a chunk so that their latency hides behind the chunk's work (a load
// at the store would wait for every memory access in flight before it).
__device__ __forceinline__ bf16x4 load_prev4(const bf16* p, bool accum, bool valid) {
  return accum && valid ? *reinterpret_cast<const bf16x4*>(p) : bf16x4{};
}

// The (r, d_v) = (128, 64) kernels are the ones that run as the halves of a
// 128 x 128 state; only they hold the prefetched entries in registers.
template <int R, int E>
constexpr bool kHalfCols = R == 128 && E == 64;

// Index (floats) of the four features 16 ft + 4 g .. + 3 of token 16 it + c of
// chunk ch (chunks counted from the head's first token) in the GLA workspace of
// dQ~ . Q~: per head ceil(n / 64) chunks of R / 16 feature tiles of four token
// tiles, 16 bytes per lane (g, c), so the lanes that write it in pass A and the
// lanes that read it in pass B move 1 KB contiguous per instruction.
template <int R>
__device__ __forceinline__ long long dbq_at(long long bh, int n, int ch, int ft, int it, int lane) {
  const long long nch = (n + kChunk - 1) / kChunk;
  return ((((bh * nch + ch) * (R / 16) + ft) * 4 + it) * 64 + lane) * 4;
}

// One chunk of an E-wide bf16 array in the row-major layout of RawChunk with
// four waves: wave w holds tokens 16 w .. 16 w + 15, lane l token 16 w + l / 4
// and 8-column blocks l % 4 + 4 j.
template <int E>
struct RowsE {
  bf16x8 v[E / 32];
  __device__ __forceinline__ void load(const bf16* X, long long ld, long long tok0, int t0, int row_end, int lane,
                                       int w) {
    const long long row = tok0 + min(t0 + 16 * w + lane / 4, row_end - 1);
#pragma unroll
    for (int j = 0; j < E / 32; ++j) v[j] = *reinterpret_cast<const bf16x8*>(X + row * ld + 8 * (lane % 4 + 4 * j));
  }
  // into a FeatTile<E> tile; rows >= L are zero
  __device__ __forceinline__ void store(char* sm, int off, int L, int lane, int w) const {
    const int t = 16 * w + lane / 4;
#pragma unroll
    for (int j = 0; j < E / 32; ++j) lds<bf16x8>(sm, off + FeatTile<E>::at(t, lane % 4 + 4 * j)) = keep_if(t < L, v[j]);
  }
};

// bf16 image of a wave's state slab (rows all R, value columns [w E/4, (w+1) E/4))
// into an [R][E] tile (FeatTile<E> rows), for products that contract over E;
// with colscale_off >= 0 each column is first scaled by the fp32 factor there.
template <int R, int E, class SArr>
__device__ __forceinline__ void state_image(const SArr& S, char* sm, int off, int lane, int w,
                                            int colscale_off = -1, int lo_off = -1) {
  constexpr int NEB = E / 64;
  const int g4 = lane >> 4, c16 = lane & 15, ebase = w * (E / 4);
#pragma unroll
  for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) {
      const int e = ebase + 16 * eb + c16;
      const float cs = colscale_off >= 0 ? lds<float>(sm, colscale_off + 4 * e) : 1.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = S[rt][eb][i] * cs;
        const bf16 hi = (bf16)x;
        const int at = FeatTile<E>::at(16 * rt + 4 * g4 + i, e / 8, 2 * (e % 8));
        lds<bf16>(sm, off + at) = hi;
        // the residual x - hi as a second image (a hi + lo pair of the state)
        if (lo_off >= 0) lds<bf16>(sm, lo_off + at) = (bf16)(x - to_f32(hi));
      }
    }
}

// The state slab as the A operand of a product over the state rows (features):
// k-slot j of lane (g, c) is feature 32 p + 4 g + j (j < 4) or 32 p + 16 + 4 g +
// (j - 4), the order of the forward's inter-chunk product.
template <int R, int E, class SArr, class OArr>
__device__ __forceinline__ void state_operand(const SArr& S, OArr& op) {
#pragma unroll
  for (int p = 0; p < R / 32; ++p)
#pragma unroll
    for (int eb = 0; eb < E / 64; ++eb)
      op[p][eb] = cat8(pack4(S[2 * p][eb][0], S[2 * p][eb][1], S[2 * p][eb][2], S[2 * p][eb][3]),
                       pack4(S[2 * p + 1][eb][0], S[2 * p + 1][eb][1], S[2 * p + 1][eb][2], S[2 * p + 1][eb][3]));
}

// B operand of that product from a feature tile: row t, the same eight features.
template <int R>
__device__ __forceinline__ bf16x8 feature_pairs(char* sm, int off, int t, int p, int g4) {
  using FT = FeatTile<R>;
  return cat8(lds<bf16x4>(sm, off + FT::at(t, 4 * p + (g4 >> 1), 8 * (g4 & 1))),
              lds<bf16x4>(sm, off + FT::at(t, 4 * p + 2 + (g4 >> 1), 8 * (g4 & 1))));
}

// ---------------------------------------------------------------------------
// Pass A: g, h and dq, chunks in order from the forward state.
// ---------------------------------------------------------------------------
template <int R, int E, int GATE>
struct BwdALayout {
  static constexpr int FTB = FeatTile<R>::BYTES, VTB = FeatTile<E>::BYTES, ATB = FeatTile<kChunk>::BYTES;
  static constexpr int q_off = 0;                      // phi(q)
  static constexpr int k_off = q_off + FTB;            // phi(k)
  static constexpr int v_off = k_off + FTB;            // v
  static constexpr int g_off = v_off + VTB;            // dO, then g = dO / den
  static constexpr int kh_off = g_off + VTB;           // RetNet: gamma^(L-1-t) phi(k); outer: K^
  static constexpr int qd_off = kh_off + (GATE == GT_DECAY || GATE == GT_OUTER ? FTB : 0);  // e^{b} phi'(q)
  static constexpr int a_off = qd_off + (kKeyGate<GATE> ? FTB : 0);     // scores A, then dW
  static constexpr int sb_off = a_off + ATB;           // bf16 [R][E] image of S entering the chunk
  static constexpr int z_off = sb_off + R * 2 * E;     // [R] z entering the chunk
  static constexpr int rs_off = z_off + R * 4;         // [64] score row sums
  static constexpr int zd_off = rs_off + kChunk * 4;   // [64] phi(q) . z
  static constexpr int inv_off = zd_off + kChunk * 4;  // [64] 1 / den
  static constexpr int hp_off = inv_off + kChunk * 4;  // [4][64] partial g . o per wave
  static constexpr int gam_off = hp_off + 4 * kChunk * 4;
  // outer-product gate: e^{c} per token and value column (rows of E + 4),
  // e^{c_end} per column, the lo half of V~ = e^{-c} v (the v tile holds hi)
  static constexpr int ec_off = gam_off + R * 4;
  static constexpr int gamv_off = ec_off + (GATE == GT_OUTER ? kChunk * (E + 4) * 4 : 0);
  static constexpr int vl_off = gamv_off + (GATE == GT_OUTER ? E * 4 : 0);
  // the bf16 residuals of the key features (dq's product over keys) and of the
  // scores (the numerator of o; then of dW for dq), which enter those products
  // as hi + lo pairs
  static constexpr int klo_off = vl_off + (GATE == GT_OUTER ? VTB : 0);
  static constexpr int alo_off = klo_off + FTB;
  // GLA: the bf16 residual of the state image, so that dq's state product takes
  // S as a hi + lo pair (the largest of the remaining roundings in dq). With 64
  // features it has the v tile's shape and takes its place once the state
  // update has read v (SLO_V: the update moves ahead of dq), which keeps the
  // 64 x 64 layout within the LDS of two workgroups per CU; otherwise it has a
  // region of its own.
  static constexpr bool SLO = GATE == GT_GLA;
  static constexpr bool SLO_V = SLO && R == kChunk;
  static constexpr int sblo_off = SLO_V ? v_off : alo_off + ATB;
  static constexpr int bytes = alo_off + ATB + (SLO && !SLO_V ? R * 2 * E : 0);
};

// h_i = -g_i . o_i from the four waves' partial dot products (fixed order).
// h is taken against the bf16-rounded g that every product uses, so that
// g_i . v_j + h_i = g_i . (v_j - o_i) holds for the rounded g: the two terms
// cancel to a difference of the size of v_j - o_i, and an error in g that is
// the same for every key would otherwise survive that cancellation (measured
// on a CPU model of these rounding points: dq error 2.2% of the head's largest
// entry with h = -(dO . o) / den, 0.3% with this h, all else exact).
__device__ __forceinline__ float bwd_h(char* sm, int hp_off, int i) {
  const float s = ((lds<float>(sm, hp_off + 4 * i) + lds<float>(sm, hp_off + 256 + 4 * i)) +
                   lds<float>(sm, hp_off + 512 + 4 * i)) +
                  lds<float>(sm, hp_off + 768 + 4 * i);
  return -s;
}

// SG (GLA only): one gate input per token for every feature (the selective gate).
template <int R, int E, int GATE, int FMAP = FM_ELU1, bool SG = false>
__global__ __launch_bounds__(256) void bwd_pass_a(BwdArgs b) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  using LY = BwdALayout<R, E, GATE>;
  using FT = FeatTile<R>;
  using VT = FeatTile<E>;
  using AT = FeatTile<kChunk>;
  constexpr int NW = 4, NEB = E / 64, KP = R / 32, KE = E / 32, FPW = R / 64;
  static_assert(R * E < 128 * 128, "four-wave layout");
  const int lane = lane_id(), w = wave_id<NW>();
  const int g4 = lane >> 4, c16 = lane & 15;
  const int s = blockIdx.x;
  const long long bh = blockIdx.y;
  const int hd = int(bh % b.H);
  const int t_begin = s * b.seg_len;
  const int t_end = min(b.n, t_begin + b.seg_len);
  const long long tok0 = bh * b.n;
  const int ebase = w * (E / NW);
  float lg2gam = 0.f;
  if constexpr (GATE == GT_DECAY) lg2gam = log2f(b.gamma[hd]);
  CausalArgs ca{};
  ca.Q = b.Q;
  ca.K = b.K;
  ca.V = b.V;
  ca.ldv = b.ldv;
  ca.g = b.gl;
  ca.gv = b.gvl;
  ca.ldgv = b.ldv;
  ca.inv_tau = b.inv_tau;

  using Raw = RawChunk<R, E, R, FMAP, GATE, true, NW, SG>;
  const int nch = (t_end - t_begin + kChunk - 1) / kChunk;
  Raw raw;
  RowsE<E> rdo;
  raw.load(ca, tok0, t_begin, t_end, lane, w);
  rdo.load(b.dO, b.ldv, tok0, t_begin, t_end, lane, w);

  // ---- forward state entering the segment
  f32x4 S[R / 16][NEB];
  f32x4 Z[ZTiles<R, NW>::ZT];
  if (b.S_in != nullptr) {
    const float* Sp = b.S_in + bh * b.in_head + s * b.in_seg;
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[rt][eb][i] = Sp[(16 * rt + 4 * g4 + i) * E + ebase + 16 * eb + c16];
  } else {
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) S[rt][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  z_load<R, NW>(Z, b.S_in != nullptr ? b.z_in + (bh * b.in_head + s * b.in_seg) / E : nullptr, lane, w);
  z_store<R, NW>(Z, reinterpret_cast<float*>(sm + LY::z_off), lane, w);
  // the state-space read-out: h = 0 (the partial sums stay zero)
  if constexpr (FMAP == FM_IDENT) lds<float>(sm, LY::hp_off + 4 * threadIdx.x) = 0.f;

  for (int ci = 0; ci < nch; ++ci) {
    const int t0 = t_begin + ci * kChunk;
    const int L = min(kChunk, b.n - t0);
    constexpr bool PF = kHalfCols<R, E>;
    bf16x4 prevq[PF ? FPW : 1][4];
    if constexpr (PF) {
#pragma unroll
      for (int u = 0; u < FPW; ++u)
#pragma unroll
        for (int it = 0; it < 4; ++it)
          prevq[u][it] = load_prev4(b.dQ + (tok0 + t0 + 16 * it + c16) * R + 16 * (w * FPW + u) + 4 * g4,
                                    b.accum != 0, 16 * it + c16 < L);
    }
    // ---- prelude: features, values, dO, and the bf16 image of S
    chunk_prelude<R, E, R, FMAP, GATE, true, NW, true, (kKeyGate<GATE> ? kPreQD : 0) | kPreKLo>(
        raw, ca, L, lg2gam, sm, LY::q_off, LY::k_off, LY::kh_off, LY::v_off, LY::gam_off, 0, lane, w, LY::qd_off, 0, 0,
        LY::ec_off, LY::gamv_off, 0, LY::vl_off, LY::klo_off);
    rdo.store(sm, LY::g_off, L, lane, w);
    state_image<R, E>(S, sm, LY::sb_off, lane, w, -1, LY::SLO && !LY::SLO_V ? LY::sblo_off : -1);
    raw.load(ca, tok0, t0 + kChunk, t_end, lane, w);
    rdo.load(b.dO, b.ldv, tok0, t0 + kChunk, t_end, lane, w);
    lds_barrier();

    // ---- scores A (masked, RetNet-weighted) and their row sums; phi(q) . z
    // (the state-space read-out has no normaliser: g = dO, h = 0, and neither
    // the scores nor o are needed, except by the outer-product gate, whose
    // G~ and dO * o take the output's value-side factors; there 1 / den = 1)
    constexpr bool NEED_O = FMAP != FM_IDENT || GATE == GT_OUTER;
    if constexpr (NEED_O) {
      const int qw = w;
      const int q = 16 * qw + c16;
      bf16x8 qop[KP];
#pragma unroll
      for (int ks = 0; ks < KP; ++ks) qop[ks] = lds<bf16x8>(sm, LY::q_off + FT::at(q, 4 * ks + g4));
      float rs = 0.f;
      for (int c = 0; c <= qw; ++c) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KP; ++ks)
          acc = mfma16(lds<bf16x8>(sm, LY::k_off + FT::at(16 * c + c16, 4 * ks + g4)), qop[ks], acc);
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * c + 4 * g4 + i;
          v[i] = acc[i];
          if constexpr (GATE == GT_DECAY) v[i] *= exp2f(float(max(q - key, 0)) * lg2gam);
          if (key > q) v[i] = 0.f;  // select after the factor (gamma^-15 overflows for a small gamma)
        }
        // hi and lo bf16 parts; the row sum of exactly what the products read
        const unsigned p01 = pack2_bits(v[0], v[1]), p23 = pack2_bits(v[2], v[3]);
        const float h0 = lo_bf16_f32(p01), h1 = hi_bf16_f32(p01), h2 = lo_bf16_f32(p23), h3 = hi_bf16_f32(p23);
        const unsigned l01 = pack2_bits(v[0] - h0, v[1] - h1), l23 = pack2_bits(v[2] - h2, v[3] - h3);
        rs += ((h0 + lo_bf16_f32(l01)) + (h1 + hi_bf16_f32(l01))) + ((h2 + lo_bf16_f32(l23)) + (h3 + hi_bf16_f32(l23)));
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        const int ao = AT::at(q, 2 * c + (g4 >> 1), 8 * (g4 & 1));
        lds<u32x2>(sm, LY::a_off + ao) = u32x2{p01, p23};
        lds<u32x2>(sm, LY::alo_off + ao) = u32x2{l01, l23};
      }
      if ((qw & 1) == 0) {
        const int ao = AT::at(q, 2 * (qw + 1) + (g4 >> 1), 8 * (g4 & 1));
        lds<bf16x4>(sm, LY::a_off + ao) = bf16x4{};
        lds<bf16x4>(sm, LY::alo_off + ao) = bf16x4{};
      }
      rs = sum_over_groups(rs);
      float zd = 0.f;
#pragma unroll
      for (int ks = 0; ks < KP; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) zd += to_f32(qop[ks][j]) * lds<float>(sm, LY::z_off + 4 * (32 * ks + 8 * g4 + j));
      zd = sum_over_groups(zd);
      if constexpr (GATE == GT_DECAY) zd *= exp2f(float(q + 1) * lg2gam);
      if (g4 == 0) {
        lds<float>(sm, LY::rs_off + 4 * q) = rs;
        lds<float>(sm, LY::zd_off + 4 * q) = zd;
        lds<float>(sm, LY::inv_off + 4 * q) = FMAP == FM_IDENT ? 1.f : 1.f / (rs + zd + b.eps);
      }
    }
    lds_barrier();

    // ---- o (fp32, not stored), g = dO / den (bf16) and the wave's share of g . o.
    // The outer-product gate: the products give num e^{-c} (V~ = e^{-c} v as hi +
    // lo); the tile takes G~ = e^{c} g, and h uses G~ . (num e^{-c}) / den (the
    // same sum as g . o); dO * o goes to the workspace for the value-side gradient.
    if constexpr (NEED_O) {
      bf16x8 Sop[KP][NEB];
      state_operand<R, E>(S, Sop);
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const int q = 16 * qt + c16;
        bf16x8 qb[KP];
#pragma unroll
        for (int p = 0; p < KP; ++p) qb[p] = feature_pairs<R>(sm, LY::q_off, q, p, g4);
        const float inv_den = lds<float>(sm, LY::inv_off + 4 * q);
        float isc = 1.f;
        if constexpr (GATE == GT_DECAY) isc = exp2f(float(q + 1) * lg2gam);
        float hp = 0.f;
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb) {
          const int e = ebase + 16 * eb;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < KP; ++p) acc = mfma16(Sop[p][eb], qb[p], acc);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] *= isc;
#pragma unroll
          for (int p2 = 0; p2 <= qt / 2; ++p2) {
            const bf16x8 ab = lds<bf16x8>(sm, LY::a_off + AT::at(q, 4 * p2 + g4));
            const bf16x8 abl = lds<bf16x8>(sm, LY::alo_off + AT::at(q, 4 * p2 + g4));
            const bf16x8 vt = tr_feat<E, true>(sm, LY::v_off, 32 * p2, e, lane);
            acc = mfma16(vt, ab, acc);
            acc = mfma16(vt, abl, acc);
            if constexpr (GATE == GT_OUTER) acc = mfma16(tr_feat<E, true>(sm, LY::vl_off, 32 * p2, e, lane), ab, acc);
          }
          // acc[i] = num[q][e + 4 g + i] (outer: times e^{-c})
          const int go = LY::g_off + VT::at(q, (e + 4 * g4) / 8, 2 * ((e + 4 * g4) % 8));
          const bf16x4 dov = lds<bf16x4>(sm, go);
          float gsc[4] = {inv_den, inv_den, inv_den, inv_den};
          if constexpr (GATE == GT_OUTER) {
            const f32x4 ec = lds<f32x4>(sm, LY::ec_off + 4 * (q * (E + 4) + e + 4 * g4));
#pragma unroll
            for (int i = 0; i < 4; ++i) gsc[i] = inv_den * ec[i];
          }
          const bf16x4 gb = pack4(to_f32(dov[0]) * gsc[0], to_f32(dov[1]) * gsc[1], to_f32(dov[2]) * gsc[2],
                                  to_f32(dov[3]) * gsc[3]);
          if constexpr (GATE == GT_OUTER) {
            // g * num = G~ * (num e^{-c}) with the rounded G~ that pass B's dV
            // uses too, so the pairs inside a suffix cancel in dO * o - dV * v
            f32x4 pw;
#pragma unroll
            for (int i = 0; i < 4; ++i) pw[i] = to_f32(gb[i]) * acc[i];
            if (q < L) *reinterpret_cast<f32x4*>(b.Pw + (tok0 + t0 + q) * E + e + 4 * g4) = pw;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) hp += to_f32(gb[i]) * (acc[i] * inv_den);
          lds<bf16x4>(sm, go) = gb;
        }
        hp = sum_over_groups(hp);
        if (FMAP != FM_IDENT && g4 == 0) lds<float>(sm, LY::hp_off + 256 * w + 4 * q) = hp;
      }
    }
    lds_barrier();

    // ---- dW (masked, RetNet-weighted) over the score tile: dW^T tiles = V G^T, + h
    {
      const int it = w;
      const int i = 16 * it + c16;
      const float hi = bwd_h(sm, LY::hp_off, i);
      for (int jt = 0; jt <= it; ++jt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KE; ++ks) {
          const bf16x8 gb = lds<bf16x8>(sm, LY::g_off + VT::at(i, 4 * ks + g4));
          acc = mfma16(lds<bf16x8>(sm, LY::v_off + VT::at(16 * jt + c16, 4 * ks + g4)), gb, acc);
          // the outer-product gate: V~ as hi + lo (V~ = e^{-c} v is not exact in bf16)
          if constexpr (GATE == GT_OUTER)
            acc = mfma16(lds<bf16x8>(sm, LY::vl_off + VT::at(16 * jt + c16, 4 * ks + g4)), gb, acc);
        }
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = 16 * jt + 4 * g4 + u;
          v[u] = acc[u] + hi;
          if constexpr (GATE == GT_DECAY) v[u] *= exp2f(float(max(i - j, 0)) * lg2gam);
          if (j > i) v[u] = 0.f;
        }
        const int ao = AT::at(i, 2 * jt + (g4 >> 1), 8 * (g4 & 1));
        const bf16x4 dwh = pack4(v[0], v[1], v[2], v[3]);
        lds<bf16x4>(sm, LY::a_off + ao) = dwh;
        lds<bf16x4>(sm, LY::alo_off + ao) = pack4(v[0] - to_f32(dwh[0]), v[1] - to_f32(dwh[1]),
                                                  v[2] - to_f32(dwh[2]), v[3] - to_f32(dwh[3]));
      }
      if ((it & 1) == 0) {
        const int ao = AT::at(i, 2 * (it + 1) + (g4 >> 1), 8 * (g4 & 1));
        lds<bf16x4>(sm, LY::a_off + ao) = bf16x4{};
        lds<bf16x4>(sm, LY::alo_off + ao) = bf16x4{};
      }
    }
    lds_barrier();

    if constexpr (LY::SLO_V) {
      // the state's residual image replaces v: the residual of S entering the
      // chunk is kept in registers, the state moves past the chunk (its last
      // read of v), and the residual is written over v once every wave is done
      bf16 slo[R / 16][E / 64][4];
#pragma unroll
      for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
        for (int eb = 0; eb < E / 64; ++eb)
#pragma unroll
          for (int i = 0; i < 4; ++i) slo[rt][eb][i] = (bf16)(S[rt][eb][i] - to_f32((bf16)S[rt][eb][i]));
      state_update<R, E, GATE, NW, true, false, false, true>(S, Z, sm, LY::k_off, LY::v_off, LY::gam_off, 1.f, lane,
                                                             w, 0, 0, 0, LY::klo_off);
      lds_barrier();
#pragma unroll
      for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
        for (int eb = 0; eb < E / 64; ++eb) {
          const int e = ebase + 16 * eb + c16;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            lds<bf16>(sm, LY::sblo_off + FeatTile<E>::at(16 * rt + 4 * g4 + i, e / 8, 2 * (e % 8))) = slo[rt][eb][i];
        }
      lds_barrier();
    }

    // ---- dphi(q)^T = Phi_k^T dW^T + gamma^(t+1) (S G^T + z h^T); dq = dphi(q) phi'(q).
    // GLA and the outer-product gate: the tiles hold Q~ = e^{b} phi(q) and
    // K~ = e^{-b} phi(k) (and G~ for the outer gate), so this is
    // dQ~ (with the state terms unweighted); dq = dQ~ e^{b} phi'(q), and
    // dQ~ . Q~ goes to dB (the log-gates' gradient, completed by pass B).
#pragma unroll
    for (int u = 0; u < FPW; ++u) {
      const int ft = w * FPW + u;
      const int f0 = 16 * ft + 4 * g4;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int i = 16 * it + c16;
        // a1: K^T dW^T on the bf16 parts, which pass B's dK~ . K~ mirrors (dg
        // relies on the two cancelling pair by pair); a1c: the residual
        // products (K_lo dW + K dW_lo) that dq adds
        f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a1c = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p <= it / 2; ++p) {
          const bf16x8 dwb = lds<bf16x8>(sm, LY::a_off + AT::at(i, 4 * p + g4));
          const bf16x8 dwl = lds<bf16x8>(sm, LY::alo_off + AT::at(i, 4 * p + g4));
          const bf16x8 kt = tr_feat<R, true>(sm, LY::k_off, 32 * p, 16 * ft, lane);
          a1 = mfma16(kt, dwb, a1);
          a1c = mfma16(tr_feat<R, true>(sm, LY::klo_off, 32 * p, 16 * ft, lane), dwb, a1c);
          a1c = mfma16(kt, dwl, a1c);
        }
#pragma unroll
        for (int ks = 0; ks < KE; ++ks) {
          const bf16x8 gop = lds<bf16x8>(sm, LY::g_off + VT::at(i, 4 * ks + g4));
          a2 = mfma16(lds<bf16x8>(sm, LY::sb_off + VT::at(16 * ft + c16, 4 * ks + g4)), gop, a2);
          if constexpr (LY::SLO) a2 = mfma16(lds<bf16x8>(sm, LY::sblo_off + VT::at(16 * ft + c16, 4 * ks + g4)), gop, a2);
        }
        const float hi = bwd_h(sm, LY::hp_off, i);
        float sc = 1.f;
        if constexpr (GATE == GT_DECAY) sc = exp2f(float(i + 1) * lg2gam);
        const bf16x4 ph = lds<bf16x4>(sm, LY::q_off + FT::at(i, f0 / 8, 2 * (f0 % 8)));
        bf16x4 qd = ph;
        if constexpr (kKeyGate<GATE>) qd = lds<bf16x4>(sm, LY::qd_off + FT::at(i, f0 / 8, 2 * (f0 % 8)));
        float dq[4];
        f32x4 db;
#pragma unroll
        for (int u2 = 0; u2 < 4; ++u2) {
          const float dphi_b = a1[u2] + sc * (a2[u2] + lds<float>(sm, LY::z_off + 4 * (f0 + u2)) * hi);
          const float dphi = dphi_b + a1c[u2];
          if constexpr (kKeyGate<GATE>) {
            dq[u2] = dphi * to_f32(qd[u2]);
            db[u2] = dphi_b * to_f32(ph[u2]);
          } else {
            dq[u2] = dphi * phi_ew_deriv<FMAP>(to_f32(ph[u2]));
          }
        }
        if (i < L) {
          bf16* at = b.dQ + (tok0 + t0 + i) * R + f0;
          store_grad4(at, dq, b.accum != 0, PF ? prevq[PF ? u : 0][it] : load_prev4(at, b.accum != 0, true));
        }
        if constexpr (kKeyGate<GATE>)
          *reinterpret_cast<f32x4*>(b.dB + dbq_at<R>(bh, b.n, t0 / kChunk, ft, it, lane)) = db;
      }
    }

    // ---- g and h for the reverse passes
    {
      const int t = 16 * w + lane / 4;
      if (t < L) {
#pragma unroll
        for (int j = 0; j < E / 32; ++j)
          *reinterpret_cast<bf16x8*>(b.G + (tok0 + t0 + t) * E + 8 * (lane % 4 + 4 * j)) =
              lds<bf16x8>(sm, LY::g_off + VT::at(t, lane % 4 + 4 * j));
      }
      if (w == 0 && lane < L) b.h[tok0 + t0 + lane] = bwd_h(sm, LY::hp_off, lane);
    }
    lds_barrier();  // z, the S image and the tiles are read above; the update below rewrites z

    // ---- carry the forward state past this chunk (SLO_V: done above)
    if constexpr (!LY::SLO_V) {
      const float gsc = GATE == GT_DECAY ? exp2f(float(L) * lg2gam) : 1.f;
      // GLA: the gated keys K~ as a hi + lo pair (their bf16 rounding in the state
      // is the largest remaining term in dq)
      state_update<R, E, GATE, NW, true, false, false, GATE == GT_GLA>(
          S, Z, sm, GATE == GT_DECAY || GATE == GT_OUTER ? LY::kh_off : LY::k_off, LY::v_off, LY::gam_off, gsc, lane,
          w, 0, LY::gamv_off, LY::vl_off, LY::klo_off);
    }
    z_store<R, NW>(Z, reinterpret_cast<float*>(sm + LY::z_off), lane, w);
    lds_barrier();
  }
}

// ---------------------------------------------------------------------------
// Reverse state of each segment (segments 1 .. P-1):
//   dR_s = sum_{i in s} gamma^(i - start_s) phi(q_i) g_i^T,  dr_s = the same with h_i,
// chunks from the segment's end, rows of each chunk back to front, so that
// with t the row index of the reversed chunk, gamma^(i - chunk start) =
// gamma^(L-1-t): the weighting and update of the forward segment pass.
// ---------------------------------------------------------------------------
template <int R, int E, int GATE>
struct BwdRLayout {
  static constexpr int k_off = 0;  // gamma^(L-1-t) phi(q) (reversed rows)
  static constexpr int v_off = k_off + FeatTile<R>::BYTES;  // g (reversed rows)
  static constexpr int hw_off = v_off + FeatTile<E>::BYTES;  // [64] h (reversed rows)
  static constexpr int gam_off = hw_off + kChunk * 4;
  static constexpr int logg_off = gam_off + R * 4;
  static constexpr int bytes = logg_off + R * 4;
};

template <int R, int E, int GATE, int FMAP = FM_ELU1>
__global__ __launch_bounds__(256) void bwd_rstate(BwdArgs b) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  using LY = BwdRLayout<R, E, GATE>;
  constexpr int NW = 4, NEB = E / 64;
  const int lane = lane_id(), w = wave_id<NW>();
  const int g4 = lane >> 4, c16 = lane & 15;
  const int s = blockIdx.x + 1;
  const long long bh = blockIdx.y;
  const int hd = int(bh % b.H);
  const int t_begin = s * b.seg_len;
  const int t_end = min(b.n, t_begin + b.seg_len);
  const long long tok0 = bh * b.n;
  const int ebase = w * (E / NW);
  float lg2gam = 0.f;
  if constexpr (GATE == GT_DECAY) lg2gam = log2f(b.gamma[hd]);
  CausalArgs ca{};

  f32x4 Rs[R / 16][NEB];
#pragma unroll
  for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) Rs[rt][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 Rz[ZTiles<R, NW>::ZT];
  z_load<R, NW>(Rz, nullptr, lane, w);

  using Raw = RawChunk<R, E, R, FMAP, GATE, false, NW>;
  // reversed chunk u0: row t holds token t_end - 1 - (u0 + t) (clamped into the segment)
  auto load_rev = [&](Raw& rw, float& hv, int u0) {
    const int tt = t_end - 1 - (u0 + 16 * w + lane / 4);
    const long long row = tok0 + max(tt, t_begin);
#pragma unroll
    for (int j = 0; j < R / 32; ++j) rw.k[j] = *reinterpret_cast<const bf16x8*>(b.Q + row * R + 8 * (lane % 4 + 4 * j));
#pragma unroll
    for (int j = 0; j < E / 32; ++j) rw.v[j] = *reinterpret_cast<const bf16x8*>(b.G + row * E + 8 * (lane % 4 + 4 * j));
    hv = b.h[row];
  };
  const int seg = t_end - t_begin;
  Raw raw;
  float hv;
  load_rev(raw, hv, 0);
  for (int u0 = 0; u0 < seg; u0 += kChunk) {
    const int L = min(kChunk, seg - u0);
    chunk_prelude<R, E, R, FMAP, GATE, false, NW, true>(raw, ca, L, lg2gam, sm, 0, LY::k_off, 0, LY::v_off,
                                                           LY::gam_off, LY::logg_off, lane, w);
    {
      const int t = 16 * w + lane / 4;
      if ((lane & 3) == 0) lds<float>(sm, LY::hw_off + 4 * t) = t < L ? hv : 0.f;
    }
    load_rev(raw, hv, u0 + kChunk);
    lds_barrier();
    const float gsc = GATE == GT_DECAY ? exp2f(float(L) * lg2gam) : 1.f;
    state_update<R, E, GATE, NW, true, true>(Rs, Rz, sm, LY::k_off, LY::v_off, LY::gam_off, gsc, lane, w,
                                             LY::hw_off);
    lds_barrier();
  }
  const long long slot = bh * b.P + s;
  float* Ro = b.R_ws + slot * R * E;
#pragma unroll
  for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i) Ro[(16 * rt + 4 * g4 + i) * E + ebase + 16 * eb + c16] = Rs[rt][eb][i];
  z_store<R, NW>(Rz, b.rh_ws + slot * R, lane, w);
}

// ---------------------------------------------------------------------------
// Pass B: dk and dv, chunks from the segment's end, from the reverse state R
// entering each chunk from its end.
// ---------------------------------------------------------------------------
template <int R, int E, int GATE>
struct BwdBLayout {
  static constexpr int FTB = FeatTile<R>::BYTES, VTB = FeatTile<E>::BYTES, ATB = FeatTile<kChunk>::BYTES;
  static constexpr int q_off = 0;                      // phi(q)
  static constexpr int k_off = q_off + FTB;            // phi(k)
  static constexpr int v_off = k_off + FTB;            // v
  static constexpr int g_off = v_off + VTB;            // g
  static constexpr int qw_off = g_off + VTB;           // RetNet: gamma^t phi(q)
  static constexpr int kd_off = qw_off + (GATE == GT_DECAY ? FTB : 0);  // GLA, outer: e^{-b} phi'(k)
  static constexpr int gr_off = kd_off + (kKeyGate<GATE> ? FTB : 0);    // GLA, outer: the raw gate input g
  static constexpr int w_off = gr_off + (kKeyGate<GATE> ? FTB : 0);     // W^T [key][query]
  static constexpr int dw_off = w_off + ATB;           // dW^T [key][query]
  static constexpr int rb_off = dw_off + ATB;          // bf16 [R][E] image of R entering the chunk
  static constexpr int rh_off = rb_off + R * 2 * E;    // [R] r_h entering the chunk
  static constexpr int hw_off = rh_off + R * 4;        // [64] h
  static constexpr int gam_off = hw_off + kChunk * 4;  // GLA: e^{chunk's summed log-gate}
  // GLA, outer: [4][R] the waves' partial products of the states at the next segment's start
  static constexpr int cpart_off = gam_off + R * 4;
  // GLA with one gate input per token: [4][64] the waves' sums of dg over their features
  static constexpr int dgs_off = cpart_off + (kKeyGate<GATE> ? 4 * R * 4 : 0);
  // outer: e^{c} per token and value column (rows of E + 4), e^{c_end} per column
  static constexpr int ec_off = dgs_off + (GATE == GT_GLA ? 4 * kChunk * 4 : 0);
  static constexpr int gamv_off = ec_off + (GATE == GT_OUTER ? kChunk * (E + 4) * 4 : 0);
  // outer: the bf16 residual of W^T (dv's product, so that dO * o - dv * v
  // cancels within a token's own pairs as pass A forms it)
  static constexpr int wlo_off = gamv_off + (GATE == GT_OUTER ? E * 4 : 0);
  static constexpr int vl_off = wlo_off + (GATE == GT_OUTER ? ATB : 0);  // outer: the lo half of V~
  // the bf16 residuals of the query features and of dW^T, for dk's product over
  // queries: not for the outer-product gate, whose tiles fill the LDS, nor where
  // they would halve the workgroups a CU holds (two fit in 80 KB each)
  static constexpr int base_end = vl_off + (GATE == GT_OUTER ? VTB : 0);
  static constexpr int kTwoPerCu = 80 * 1024;
  static constexpr bool DK_SPLIT =
      GATE != GT_OUTER && (base_end + FTB + ATB <= kTwoPerCu || base_end > kTwoPerCu);
  static constexpr int qlo_off = base_end;
  static constexpr int dwlo_off = qlo_off + (DK_SPLIT ? FTB : 0);
  static constexpr int bytes = dwlo_off + (DK_SPLIT ? ATB : 0);
};

// Inclusive prefix sum across each row of 16 lanes (lane c gets x_0 + ... + x_c
// of its row).
__device__ __forceinline__ float row_inclusive_scan(float x) {
  x += dpp_or_zero<0x111, 0xf>(x);
  x += dpp_or_zero<0x112, 0xf>(x);
  x += dpp_or_zero<0x114, 0xf>(x);
  x += dpp_or_zero<0x118, 0xf>(x);
  return x;
}

// SG (GLA only): one gate input per token for every feature; dg [B H n] is its
// gradient summed over features.
template <int R, int E, int GATE, int FMAP = FM_ELU1, bool SG = false>
__global__ __launch_bounds__(256) void bwd_pass_b(BwdArgs b) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  using LY = BwdBLayout<R, E, GATE>;
  using FT = FeatTile<R>;
  using VT = FeatTile<E>;
  using AT = FeatTile<kChunk>;
  constexpr int NW = 4, NEB = E / 64, KP = R / 32, KE = E / 32, FPW = R / 64;
  static_assert(R * E < 128 * 128, "four-wave layout");
  const int lane = lane_id(), w = wave_id<NW>();
  const int g4 = lane >> 4, c16 = lane & 15;
  const int s = blockIdx.x;
  const long long bh = blockIdx.y;
  const int hd = int(bh % b.H);
  const int t_begin = s * b.seg_len;
  const int t_end = min(b.n, t_begin + b.seg_len);
  const long long tok0 = bh * b.n;
  const int ebase = w * (E / NW);
  float lg2gam = 0.f;
  if constexpr (GATE == GT_DECAY) lg2gam = log2f(b.gamma[hd]);
  CausalArgs ca{};
  ca.Q = b.Q;
  ca.K = b.K;
  ca.V = b.V;
  ca.ldv = b.ldv;
  ca.g = b.gl;
  ca.gv = b.gvl;
  ca.ldgv = b.ldv;
  ca.inv_tau = b.inv_tau;
  // the chunk's tiles: plain features (RetNet weights are applied per product)
  // or, with the GLA and outer-product gates, Q~ and K~ as in the forward (and
  // V~ = e^{-c} v, its bf16 hi part, for the outer gate)
  constexpr int PG = kKeyGate<GATE> ? GATE : GT_NONE;
  constexpr bool OUT = GATE == GT_OUTER;

  // ---- reverse state entering the segment from its end
  f32x4 Rs[R / 16][NEB];
  f32x4 Rz[ZTiles<R, NW>::ZT];
  const bool has_in = b.P > 1;
  {
    const long long slot = bh * b.P + s;
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Rs[rt][eb][i] = has_in ? b.R_ws[slot * R * E + (16 * rt + 4 * g4 + i) * E + ebase + 16 * eb + c16] : 0.f;
    z_load<R, NW>(Rz, has_in ? b.rh_ws + slot * R : nullptr, lane, w);
  }
  // GLA: d log alpha at the next segment's first token t1 is
  // sum_e S(t1)[f][e] R(t1)[f][e] + z(t1)[f] r_h(t1)[f], S(t1) the forward
  // state entering that segment and R(t1) the reverse state entering this one
  // from its end: the waves' partial sums over their value columns here, the
  // z share in the first chunk. The outer-product gate's d log beta there is
  // sum_f S(t1)[f][e] R(t1)[f][e] (z has no value-side factor): a column sum
  // over the wave's own slab.
  const bool later = s + 1 < b.P;
  float cvt[NEB];  // outer: d log beta at t1 for column ebase + 16 eb + c16
  if constexpr (kKeyGate<GATE>) {
    const float* Sn = later ? b.S_in + bh * b.in_head + (long long)(s + 1) * b.in_seg : nullptr;
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) cvt[eb] = 0.f;
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = 16 * rt + 4 * g4 + i;
        float acc = 0.f;
        if (later) {
#pragma unroll
          for (int eb = 0; eb < NEB; ++eb) {
            const float pr = Rs[rt][eb][i] * Sn[f * E + ebase + 16 * eb + c16];
            acc += pr;
            if constexpr (OUT) cvt[eb] += pr;
          }
        }
        acc += __shfl_xor(acc, 1);
        acc += __shfl_xor(acc, 2);
        acc += __shfl_xor(acc, 4);
        acc += __shfl_xor(acc, 8);
        if (c16 == 0) lds<float>(sm, LY::cpart_off + 4 * (w * R + f)) = acc;
      }
    if constexpr (OUT) {
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) {
        cvt[eb] += __shfl_xor(cvt[eb], 16);
        cvt[eb] += __shfl_xor(cvt[eb], 32);
      }
    }
  }
  // outer: d log beta entering from the later tokens, for the columns
  // e + 4 g + u this lane holds in the dV products below
  float carryv[OUT ? NEB : 1][4];
  if constexpr (OUT) {
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
      for (int u = 0; u < 4; ++u) carryv[eb][u] = __shfl(cvt[eb], 4 * g4 + u);
  }

  const int nslot = w < 2 ? 3 : 2;
  int sqi[3], skj[3];
  score_tiles(w, sqi, skj);
  float carry[FPW][4];  // GLA: d log alpha at the end of the chunk, for this lane's features

  using Raw = RawChunk<R, E, R, FMAP, PG, true, NW, SG>;
  const int nch = (t_end - t_begin + kChunk - 1) / kChunk;
  Raw raw;
  RowsE<E> rg;
  float hv = 0.f;
  auto load = [&](int ci) {
    const int t0 = t_begin + ci * kChunk;
    raw.load(ca, tok0, t0, t_end, lane, w);
    rg.load(b.G, E, tok0, t0, t_end, lane, w);
    hv = b.h[tok0 + min(t0 + lane, t_end - 1)];
  };
  load(nch - 1);
  for (int ci = nch - 1; ci >= 0; --ci) {
    const int t0 = t_begin + ci * kChunk;
    const int L = min(kChunk, b.n - t0);
    constexpr bool PF = kHalfCols<R, E>;
    constexpr bool DGF = kKeyGate<GATE> && !SG;  // dg per feature
    bf16x4 prevk[PF ? FPW : 1][4], prevg[PF && DGF ? FPW : 1][4];
    bf16 prevgs = bf16(0.f);
    if constexpr (PF) {
#pragma unroll
      for (int u = 0; u < FPW; ++u)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const long long at = (tok0 + t0 + 16 * jt + c16) * R + 16 * (w * FPW + u) + 4 * g4;
          prevk[u][jt] = load_prev4(b.dK + at, b.accum != 0, 16 * jt + c16 < L);
          if constexpr (DGF) prevg[u][jt] = load_prev4(b.dg + at, b.accum != 0, 16 * jt + c16 < L);
        }
      if constexpr (SG) {
        if (b.accum != 0 && w == 0 && lane < L) prevgs = b.dg[tok0 + t0 + lane];
      }
    }
    // ---- prelude
    chunk_prelude<R, E, R, FMAP, PG, true, NW, true,
                  (kKeyGate<GATE> ? (kPreKD | (OUT ? kPreNoKH : 0)) : 0) | (LY::DK_SPLIT ? kPreQLo : 0)>(
        raw, ca, L, 0.f, sm, LY::q_off, LY::k_off, 0, LY::v_off, LY::gam_off, 0, lane, w, 0, LY::kd_off, 0,
        LY::ec_off, LY::gamv_off, 0, LY::vl_off, 0, LY::qlo_off);
    if constexpr (GATE == GT_DECAY) {
      // gamma^t phi(q) for the reverse-state update
      const int t = 16 * w + lane / 4;
      const float wt = exp2f(float(t) * lg2gam);
#pragma unroll
      for (int j = 0; j < R / 32; ++j) {
        float f[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) f[u] = phi_ew<FMAP>(to_f32(raw.q[j][u])) * wt;
        lds<bf16x8>(sm, LY::qw_off + FT::at(t, lane % 4 + 4 * j)) =
            keep_if(t < L, cat8(pack4(f[0], f[1], f[2], f[3]), pack4(f[4], f[5], f[6], f[7])));
      }
    }
    if constexpr (kKeyGate<GATE>) {
      // the raw gate of this lane's token and the wave's features, for dg
#pragma unroll
      for (int jg = 0; jg < R / 32; ++jg) {
        bf16x8 gp;
        if constexpr (SG) {
#pragma unroll
          for (int u = 0; u < 8; ++u) gp[u] = raw.gs;
        } else {
          gp = raw.g[jg];
        }
        lds<bf16x8>(sm, LY::gr_off + FT::at(lane, (w * (R / 4) + 8 * jg) / 8)) = gp;
      }
    }
    rg.store(sm, LY::g_off, L, lane, w);
    if (w == 0) lds<float>(sm, LY::hw_off + 4 * lane) = lane < L ? hv : 0.f;
    // (outer: R scaled by e^{c_end} per column, for the dK~ product with V~)
    state_image<R, E>(Rs, sm, LY::rb_off, lane, w, OUT ? LY::gamv_off : -1);
    z_store<R, NW>(Rz, reinterpret_cast<float*>(sm + LY::rh_off), lane, w);
    if (ci > 0) load(ci - 1);
    lds_barrier();

    // ---- W^T and dW^T tiles [key j][query i], i >= j, dealt 3, 3, 2, 2 over the waves
#pragma unroll
    for (int sl = 0; sl < 3; ++sl) {
      if (sl < nslot) {
        const int it = sqi[sl], jt = skj[sl];
        const int j = 16 * jt + c16;
        f32x4 aw = {0.f, 0.f, 0.f, 0.f}, ad = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KP; ++ks)
          aw = mfma16(lds<bf16x8>(sm, LY::q_off + FT::at(16 * it + c16, 4 * ks + g4)),
                      lds<bf16x8>(sm, LY::k_off + FT::at(j, 4 * ks + g4)), aw);
#pragma unroll
        for (int ks = 0; ks < KE; ++ks) {
          const bf16x8 gb = lds<bf16x8>(sm, LY::g_off + VT::at(16 * it + c16, 4 * ks + g4));
          ad = mfma16(gb, lds<bf16x8>(sm, LY::v_off + VT::at(j, 4 * ks + g4)), ad);
          // the outer-product gate: V~ as hi + lo, as pass A forms dW
          if constexpr (OUT) ad = mfma16(gb, lds<bf16x8>(sm, LY::vl_off + VT::at(j, 4 * ks + g4)), ad);
        }
        // aw[u] = phi(q_i) . phi(k_j), ad[u] = g_i . v_j with i = 16 it + 4 g + u
        float vw[4], vd[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = 16 * it + 4 * g4 + u;
          const bool ok = i >= j;
          float dec = 1.f;
          if constexpr (GATE == GT_DECAY) dec = exp2f(float(max(i - j, 0)) * lg2gam);
          vw[u] = ok ? aw[u] * dec : 0.f;
          vd[u] = ok ? (ad[u] + lds<float>(sm, LY::hw_off + 4 * i)) * dec : 0.f;
        }
        const int o = AT::at(j, 2 * it + (g4 >> 1), 8 * (g4 & 1));
        const bf16x4 wh = pack4(vw[0], vw[1], vw[2], vw[3]);
        lds<bf16x4>(sm, LY::w_off + o) = wh;
        if constexpr (OUT)
          lds<bf16x4>(sm, LY::wlo_off + o) = pack4(vw[0] - to_f32(wh[0]), vw[1] - to_f32(wh[1]),
                                                   vw[2] - to_f32(wh[2]), vw[3] - to_f32(wh[3]));
        const bf16x4 dh = pack4(vd[0], vd[1], vd[2], vd[3]);
        lds<bf16x4>(sm, LY::dw_off + o) = dh;
        if constexpr (LY::DK_SPLIT)
          lds<bf16x4>(sm, LY::dwlo_off + o) = pack4(vd[0] - to_f32(dh[0]), vd[1] - to_f32(dh[1]),
                                                    vd[2] - to_f32(dh[2]), vd[3] - to_f32(dh[3]));
      }
    }
    // tiles below the diagonal read by the products over 32 queries: (key 1, query 0) and (3, 2)
    if (w >= 2) {
      const int o = AT::at(16 * (2 * w - 3) + c16, 2 * (2 * w - 4) + (g4 >> 1), 8 * (g4 & 1));
      lds<bf16x4>(sm, LY::w_off + o) = bf16x4{};
      if constexpr (OUT) lds<bf16x4>(sm, LY::wlo_off + o) = bf16x4{};
      lds<bf16x4>(sm, LY::dw_off + o) = bf16x4{};
      if constexpr (LY::DK_SPLIT) lds<bf16x4>(sm, LY::dwlo_off + o) = bf16x4{};
    }
    lds_barrier();

    // ---- dv^T = G^T W (intra) + gamma^(L-t) R'^T phi(k)^T (inter): the wave's value columns.
    // GLA: a key's share of the state reaches the chunk's end scaled by
    // Gamma = e^{chunk's summed log-gate} per feature, so the inter term is
    // (Gamma R)^T K~^T. The outer-product gate: dv = e^{-c} ((Gamma R Gamma_v)^T K~^T
    // + G~^T W), and the value-side log-gate's gradient dC = dO * o - dv * v,
    // summed over the later tokens of each column (key tiles back to front),
    // gives dgv = d log beta sigmoid(-gv) / tau.
    {
      bf16x8 Rop[KP][NEB];
      if constexpr (kKeyGate<GATE>) {
        float gc[NEB];
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb) gc[eb] = OUT ? lds<float>(sm, LY::gamv_off + 4 * (ebase + 16 * eb + c16)) : 1.f;
        f32x4 Rg[R / 16][NEB];
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gm = lds<float>(sm, LY::gam_off + 4 * (16 * rt + 4 * g4 + i));
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb) Rg[rt][eb][i] = OUT ? Rs[rt][eb][i] * (gm * gc[eb]) : Rs[rt][eb][i] * gm;
          }
        state_operand<R, E>(Rg, Rop);
      } else {
        state_operand<R, E>(Rs, Rop);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int jt = OUT ? 3 - jj : jj;
        const int j = 16 * jt + c16;
        bf16x8 kb[KP];
#pragma unroll
        for (int p = 0; p < KP; ++p) kb[p] = feature_pairs<R>(sm, LY::k_off, j, p, g4);
        float sc = 1.f;
        if constexpr (GATE == GT_DECAY) sc = exp2f(float(max(L - j, 0)) * lg2gam);
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb) {
          const int e = ebase + 16 * eb;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < KP; ++p) acc = mfma16(Rop[p][eb], kb[p], acc);
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[u] *= sc;
#pragma unroll
          for (int p = jt / 2; p < 2; ++p) {
            const bf16x8 gt = tr_feat<E, true>(sm, LY::g_off, 32 * p, e, lane);
            acc = mfma16(gt, lds<bf16x8>(sm, LY::w_off + AT::at(j, 4 * p + g4)), acc);
            if constexpr (OUT) acc = mfma16(gt, lds<bf16x8>(sm, LY::wlo_off + AT::at(j, 4 * p + g4)), acc);
          }
          if constexpr (OUT) {
            const f32x4 ec = lds<f32x4>(sm, LY::ec_off + 4 * (j * (E + 4) + e + 4 * g4));
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[u] *= __builtin_amdgcn_rcpf(ec[u]);
            // rows past the chunk read the segment's last row (in bounds) and are masked
            const long long row = tok0 + min(t0 + j, t_end - 1);
            const f32x4 pw = *reinterpret_cast<const f32x4*>(b.Pw + row * E + e + 4 * g4);
            const bf16x4 vr = *reinterpret_cast<const bf16x4*>(b.V + row * b.ldv + e + 4 * g4);
            const bf16x4 gvr = *reinterpret_cast<const bf16x4*>(b.gvl + row * b.ldv + e + 4 * g4);
            float o[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float x = j < L ? pw[u] - acc[u] * to_f32(vr[u]) : 0.f;
              const float pre = row_inclusive_scan(x);
              const float tot = __shfl(pre, (lane & 48) | 15);
              o[u] = (carryv[eb][u] + ((tot - pre) + x)) * b.inv_tau *
                     __builtin_amdgcn_rcpf(1.f + __expf(to_f32(gvr[u])));
              carryv[eb][u] += tot;
            }
            if (j < L)
              *reinterpret_cast<bf16x4*>(b.dgv + (tok0 + t0 + j) * b.ldv + e + 4 * g4) = pack4(o[0], o[1], o[2], o[3]);
          }
          if (j < L)
            *reinterpret_cast<bf16x4*>(b.dV + (tok0 + t0 + j) * b.ldv + e + 4 * g4) =
                pack4(acc[0], acc[1], acc[2], acc[3]);
        }
      }
    }

    // ---- dphi(k)^T = Phi_q^T dW (intra) + gamma^(L-t) (R v + r_h) (inter); dk = dphi(k) phi'(k).
    // GLA: dK~ = Q~^T dW + Gamma (R v + r_h); dk = dK~ e^{-b} phi'(k) (the
    // outer-product gate: R Gamma_v V~ in place of R v), and
    // dB = dQ~ . Q~ - dK~ . K~, the gradient of the cumulative log-gate, whose
    // suffix sums give dg (below). A lane keeps the same features in every
    // chunk: 16 ft + 4 g + u2, tokens 16 jt + c.
#pragma unroll
    for (int u = 0; u < FPW; ++u) {
      const int ft = w * FPW + u;
      const int f0 = 16 * ft + 4 * g4;
      if constexpr (kKeyGate<GATE>) {
        if (ci == nch - 1) {
          // d log alpha entering from the later segments (see above)
#pragma unroll
          for (int u2 = 0; u2 < 4; ++u2) {
            const int f = f0 + u2;
            carry[u][u2] =
                later ? ((lds<float>(sm, LY::cpart_off + 4 * f) + lds<float>(sm, LY::cpart_off + 4 * (R + f))) +
                         (lds<float>(sm, LY::cpart_off + 4 * (2 * R + f)) +
                          lds<float>(sm, LY::cpart_off + 4 * (3 * R + f)))) +
                            b.z_in[(bh * b.in_head + (long long)(s + 1) * b.in_seg) / E + f] *
                                lds<float>(sm, LY::rh_off + 4 * f)
                      : 0.f;
          }
        }
      }
      // GLA walks the key tiles back to front for the suffix sums of dB
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int jt = kKeyGate<GATE> ? 3 - jj : jj;
        const int j = 16 * jt + c16;
        // a1: Q^T dW on the bf16 parts, which pass A's dQ~ . Q~ mirrors (dg);
        // a1c: the residual products (Q_lo dW + Q dW_lo) that dk adds
        f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a1c = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = jt / 2; p < 2; ++p) {
          const bf16x8 qt = tr_feat<R, true>(sm, LY::q_off, 32 * p, 16 * ft, lane);
          const bf16x8 dwb = lds<bf16x8>(sm, LY::dw_off + AT::at(j, 4 * p + g4));
          a1 = mfma16(qt, dwb, a1);
          if constexpr (LY::DK_SPLIT) {
            a1c = mfma16(tr_feat<R, true>(sm, LY::qlo_off, 32 * p, 16 * ft, lane), dwb, a1c);
            a1c = mfma16(qt, lds<bf16x8>(sm, LY::dwlo_off + AT::at(j, 4 * p + g4)), a1c);
          }
        }
#pragma unroll
        for (int ks = 0; ks < KE; ++ks)
          a2 = mfma16(lds<bf16x8>(sm, LY::rb_off + VT::at(16 * ft + c16, 4 * ks + g4)),
                      lds<bf16x8>(sm, LY::v_off + VT::at(j, 4 * ks + g4)), a2);
        float sc = 1.f;
        if constexpr (GATE == GT_DECAY) sc = exp2f(float(max(L - j, 0)) * lg2gam);
        const bf16x4 ph = lds<bf16x4>(sm, LY::k_off + FT::at(j, f0 / 8, 2 * (f0 % 8)));
        bf16x4 kd = ph;
        if constexpr (kKeyGate<GATE>) kd = lds<bf16x4>(sm, LY::kd_off + FT::at(j, f0 / 8, 2 * (f0 % 8)));
        float dk[4], bk[4];
#pragma unroll
        for (int u2 = 0; u2 < 4; ++u2) {
          if constexpr (kKeyGate<GATE>) sc = lds<float>(sm, LY::gam_off + 4 * (f0 + u2));
          const float dphi_b = a1[u2] + sc * (a2[u2] + lds<float>(sm, LY::rh_off + 4 * (f0 + u2)));
          const float dphi = dphi_b + a1c[u2];
          if constexpr (kKeyGate<GATE>) {
            dk[u2] = dphi * to_f32(kd[u2]);
            bk[u2] = dphi_b * to_f32(ph[u2]);
          } else {
            dk[u2] = dphi * phi_ew_deriv<FMAP>(to_f32(ph[u2]));
          }
        }
        if (j < L) {
          bf16* at = b.dK + (tok0 + t0 + j) * R + f0;
          store_grad4(at, dk, b.accum != 0, PF ? prevk[PF ? u : 0][jt] : load_prev4(at, b.accum != 0, true));
        }
        if constexpr (kKeyGate<GATE>) {
          // ---- dg: d log alpha_t = (d log alpha after the tile) + sum of dB over
          // the tile's tokens t' >= t (the row of 16 lanes holds tokens 16 jt + c
          // of four features); dg = d log alpha sigmoid(-g) / tau
          const f32x4 db = *reinterpret_cast<const f32x4*>(b.dB + dbq_at<R>(bh, b.n, t0 / kChunk, ft, jt, lane));
          const bf16x4 gv = lds<bf16x4>(sm, LY::gr_off + FT::at(j, f0 / 8, 2 * (f0 % 8)));
          float o[4];
#pragma unroll
          for (int u2 = 0; u2 < 4; ++u2) {
            const float x = j < L ? db[u2] - bk[u2] : 0.f;
            const float pre = row_inclusive_scan(x);
            const float tot = __shfl(pre, (lane & 48) | 15);
            o[u2] = (carry[u][u2] + ((tot - pre) + x)) * b.inv_tau * __builtin_amdgcn_rcpf(1.f + __expf(to_f32(gv[u2])));
            carry[u][u2] += tot;
          }
          if constexpr (SG) {
            // the sum over this wave's features for token j: over the lane's
            // four, its lane groups, then its feature tiles (kept in LDS by
            // the lanes of group 0, in a fixed order)
            float ts = (o[0] + o[1]) + (o[2] + o[3]);
            ts += __shfl_xor(ts, 16);
            ts += __shfl_xor(ts, 32);
            if (g4 == 0) {
              float& slot = lds<float>(sm, LY::dgs_off + 4 * (w * kChunk + j));
              slot = u == 0 ? ts : slot + ts;
            }
          } else if (j < L) {
            bf16* at = b.dg + (tok0 + t0 + j) * R + f0;
            store_grad4(at, o, b.accum != 0, PF ? prevg[PF ? u : 0][jt] : load_prev4(at, b.accum != 0, true));
          }
        }
      }
    }

    // ---- R <- gamma^L R + (gamma^t phi(q))^T [g, h]: the state entering the previous chunk
    // (GLA: R <- Gamma R + Q~^T [g, h]; outer: R <- Gamma R Gamma_v + Q~^T [G~, h])
    if constexpr (kKeyGate<GATE>) {
      state_update<R, E, GATE, NW, true, true, true>(Rs, Rz, sm, LY::q_off, LY::g_off, LY::gam_off, 1.f, lane, w,
                                                     LY::hw_off, LY::gamv_off);
    } else {
      const float gsc = GATE == GT_DECAY ? exp2f(float(L) * lg2gam) : 1.f;
      state_update<R, E, GATE, NW, true, true>(Rs, Rz, sm, GATE == GT_DECAY ? LY::qw_off : LY::q_off, LY::g_off,
                                               LY::gam_off, gsc, lane, w, LY::hw_off);
    }
    lds_barrier();
    if constexpr (SG) {
      // one gate input per token: its dg is the sum over all features (the four
      // waves' partial sums, in a fixed order; the next chunk rewrites them only
      // after its own barriers)
      if (w == 0 && lane < L) {
        const float sdg = (lds<float>(sm, LY::dgs_off + 4 * lane) + lds<float>(sm, LY::dgs_off + 4 * (kChunk + lane))) +
                          (lds<float>(sm, LY::dgs_off + 4 * (2 * kChunk + lane)) +
                           lds<float>(sm, LY::dgs_off + 4 * (3 * kChunk + lane)));
        bf16* at = b.dg + tok0 + t0 + lane;
        if constexpr (!PF) prevgs = b.accum != 0 ? *at : bf16(0.f);
        *at = (bf16)(b.accum != 0 ? sdg + to_f32(prevgs) : sdg);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// GLA: each segment's own reverse state (segments 1 .. P-1). With the
// per-feature gate the reverse state entering chunk c from its end obeys
// R_c = Gamma_c R_{c+1} + Q~_c^T [g, h] (Q~ = e^{b} phi(q), b the chunk's
// inclusive summed log-gate), so the segment's share starts from zero at its
// end and runs its chunks back to front in natural row order. The segment's
// summed log-gate goes to logG for the reverse scan. The outer-product gate
// adds its value side: R_c = (Gamma_c Gamma_v,c^T) * R_{c+1} + Q~_c^T [G~, h]
// with G~ = e^{c} g (pass A stores G~), and the segment's summed value-side
// log-gates go to logGv.
// ---------------------------------------------------------------------------
template <int R, int E, int GATE>
struct BwdRGLayout {
  static constexpr int q_off = 0;                           // Q~
  static constexpr int v_off = q_off + FeatTile<R>::BYTES;  // g (outer: G~)
  static constexpr int hw_off = v_off + FeatTile<E>::BYTES;  // [64] h
  static constexpr int gam_off = hw_off + kChunk * 4;        // [R] e^{chunk's summed log-gate}
  static constexpr int logg_off = gam_off + R * 4;           // [R] segment's summed log-gate
  static constexpr int gamv_off = logg_off + R * 4;          // outer: [E] e^{chunk's summed value-side log-gate}
  static constexpr int loggv_off = gamv_off + (GATE == GT_OUTER ? E * 4 : 0);  // outer: [E] segment's sum
  static constexpr int bytes = loggv_off + (GATE == GT_OUTER ? E * 4 : 0);
};

template <int R, int E, int GATE, int FMAP = FM_ELU1, bool SG = false>
__global__ __launch_bounds__(256) void bwd_rstate_gla(BwdArgs b) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  using LY = BwdRGLayout<R, E, GATE>;
  constexpr int NW = 4, NEB = E / 64, FR = R / NW, EV = E / NW;
  const int lane = lane_id(), w = wave_id<NW>();
  const int g4 = lane >> 4, c16 = lane & 15;
  const int s = blockIdx.x + 1;
  const long long bh = blockIdx.y;
  const int t_begin = s * b.seg_len;
  const int t_end = min(b.n, t_begin + b.seg_len);
  const long long tok0 = bh * b.n;
  const int ebase = w * (E / NW);
  CausalArgs ca{};
  ca.K = b.Q;  // the queries in the prelude's key slot, scaled by e^{+b}: Q~
  ca.V = b.G;
  ca.g = b.gl;
  ca.gv = b.gvl;
  ca.ldgv = b.ldv;
  ca.inv_tau = b.inv_tau;

  f32x4 Rs[R / 16][NEB];
#pragma unroll
  for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) Rs[rt][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 Rz[ZTiles<R, NW>::ZT];
  z_load<R, NW>(Rz, nullptr, lane, w);
  // the lane that accumulates feature w FR + lane in the prelude clears it
  if (lane < FR) lds<float>(sm, LY::logg_off + 4 * (w * FR + lane)) = 0.f;
  if constexpr (GATE == GT_OUTER) {
    if (lane < EV) lds<float>(sm, LY::loggv_off + 4 * (w * EV + lane)) = 0.f;
  }

  using Raw = RawChunk<R, E, R, FMAP, GATE, false, NW, SG>;
  const int nch = (t_end - t_begin + kChunk - 1) / kChunk;
  Raw raw;
  float hv = 0.f;
  auto load = [&](int ci) {
    const int t0 = t_begin + ci * kChunk;
    raw.load(ca, tok0, t0, t_end, lane, w);
    hv = b.h[tok0 + min(t0 + lane, t_end - 1)];
  };
  load(nch - 1);
  for (int ci = nch - 1; ci >= 0; --ci) {
    const int t0 = t_begin + ci * kChunk;
    const int L = min(kChunk, t_end - t0);
    chunk_prelude<R, E, R, FMAP, GATE, false, NW, true, kPreKPos | (GATE == GT_OUTER ? kPreVRaw : 0)>(
        raw, ca, L, 0.f, sm, 0, LY::q_off, 0, LY::v_off, LY::gam_off, LY::logg_off, lane, w, 0, 0, 0, 0,
        LY::gamv_off, LY::loggv_off);
    if (w == 0) lds<float>(sm, LY::hw_off + 4 * lane) = lane < L ? hv : 0.f;
    if (ci > 0) load(ci - 1);
    lds_barrier();
    state_update<R, E, GATE, NW, true, true, true>(Rs, Rz, sm, LY::q_off, LY::v_off, LY::gam_off, 1.f, lane, w,
                                                   LY::hw_off, LY::gamv_off);
    lds_barrier();
  }
  const long long slot = bh * b.P + s;
  float* Ro = b.R_ws + slot * R * E;
#pragma unroll
  for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i) Ro[(16 * rt + 4 * g4 + i) * E + ebase + 16 * eb + c16] = Rs[rt][eb][i];
  z_store<R, NW>(Rz, b.rh_ws + slot * R, lane, w);
  if (lane < FR) b.logG[slot * R + w * FR + lane] = lds<float>(sm, LY::logg_off + 4 * (w * FR + lane));
  if constexpr (GATE == GT_OUTER) {
    if (lane < EV) b.logGv[slot * E + w * EV + lane] = lds<float>(sm, LY::loggv_off + 4 * (w * EV + lane));
  }
}

}  // namespace la
