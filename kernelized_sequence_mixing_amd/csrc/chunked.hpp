// Chunkwise-parallel causal linear attention for gfx950.
//
// Every (batch, head) sequence is cut into 64-token chunks; each chunk is a
// dense block problem on the matrix cores:
//
//   scores   A  = (Q~ K~^T) masked to key <= query (times gamma^(i-j) for RetNet)
//   outputs  O  = A V + Q^ S_prev,   den = rowsum(A) + Q^ z_prev + eps,  o = O / den
//   state    S <- Gamma S + K^^T V,  z <- Gamma z + colsum(K^)
//
// which is the recurrence S_t = G_t S_{t-1} + phi(k_t) v_t^T of "Recurrent
// Reformulation" ("Linear Attention Mechanisms", dileepadev.github.io) with the
// gates of "Gating and Selective State Updates" on the same page, evaluated 64
// steps at a time: the intra-chunk part is the masked quadratic form of "The
// Kernel Trick for Attention" restricted to the chunk, the inter-chunk part
// reads the carried state. For the per-feature GLA gate with chunk-local
// cumulative log-gate b_t, Q~ = phi(Q) e^{b}, K~ = phi(K) e^{-b},
// K^ = phi(K) e^{b_end - b} and Gamma = e^{b_end}; for RetNet the chunk-local
// weights gamma^(i-j), gamma^(i+1) and gamma^(L-1-j) are applied directly.
//
// To fill 256 compute units with few heads, each head's sequence is split into
// P segments of whole chunks: pass 1 computes each segment's own state
// contribution, a scan chains them, and pass 3 recomputes every segment's
// outputs starting from its chained state.
//
// Workgroup = 256 threads = 4 waves. Wave w owns query rows [16w, 16w+16) of
// the chunk for the scores, and value columns [w E/4, (w+1) E/4) of the state
// and the outputs. The fp32 state lives in MFMA accumulators for the whole
// sequence; its bf16 image feeds the inter-chunk product straight from
// registers. LDS holds the chunk's operands (bf16):
//   q  [64][R+8]   Q~ (also Q^), row-major          k  [64][R+8]  K~
//   kt [R][64+8]   K^ transposed                    vt [E][64+8]  V transposed
//   a  [64][64+8]  masked scores, row-major
#pragma once

#include "common.hpp"
#include "plan.hpp"

namespace la {

enum FmapKind { FM_ELU1 = 0, FM_FAVOR = 1 };
enum GateKind { GT_NONE = 0, GT_DECAY = 1, GT_GLA = 2 };

struct CausalArgs {
  const bf16* Q;
  const bf16* K;
  const bf16* V;
  const bf16* g;
  const bf16* omega;
  const float* gamma;
  const float* S_in;       // pass 3: initial state per (head, segment); nullable
  const float* z_in;
  long long in_head;       // S_in element stride between heads
  long long in_seg;        // S_in element stride between segments
  float* S_out;            // pass 1: per-segment deltas; pass 3: final state (nullable)
  float* z_out;
  float* logG_out;         // pass 1, GLA: per-segment summed log-gates
  bf16* out;
  int H, n, P, seg_len;
  float eps, inv_tau;
};

constexpr int CP = kChunk + 8;  // row stride (elements) of the [x][t] tiles

template <int R, int E>
struct FwdLayout {
  static constexpr int RP = R + 8;
  static constexpr int q_off = 0;
  static constexpr int k_off = q_off + kChunk * RP * 2;
  static constexpr int kt_off = k_off + kChunk * RP * 2;
  static constexpr int vt_off = kt_off + R * CP * 2;
  static constexpr int a_off = vt_off + E * CP * 2;
  static constexpr int z_off = a_off + kChunk * CP * 2;
  static constexpr int gam_off = z_off + R * 4;
  static constexpr int den_off = gam_off + R * 4;
  static constexpr int bytes = den_off + kChunk * 4;
};

template <int R, int E>
struct SegLayout {
  static constexpr int kt_off = 0;
  static constexpr int vt_off = kt_off + R * CP * 2;
  static constexpr int gam_off = vt_off + E * CP * 2;
  static constexpr int logg_off = gam_off + R * 4;
  static constexpr int bytes = logg_off + R * 4;
};

// Wave barrier for LDS traffic only: every LDS access issued before it is
// complete and visible after it. Outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename T>
__device__ __forceinline__ T& lds(char* base, int byte_off) {
  return *reinterpret_cast<T*>(base + byte_off);
}

// Raw inputs of one chunk, held in registers from the global load to the LDS
// write so the next chunk's loads overlap the current chunk's math.
template <int R, int E, int DK, int FMAP, int GATE, bool WITH_Q>
struct RawChunk {
  static constexpr int FR = R / 4;       // features per wave (elu+1 lane-per-token layout)
  static constexpr int EV = E / 4;       // value columns per wave
  static constexpr int KS = DK / 32;     // projection k-steps (FAVOR)
  static constexpr bool ELU = FMAP == FM_ELU1;
  bf16x8 q[ELU && WITH_Q ? FR / 8 : 1];
  bf16x8 k[ELU ? FR / 8 : 1];
  bf16x8 g[GATE == GT_GLA ? FR / 8 : 1];
  bf16x8 xq[!ELU && WITH_Q ? 4 * KS : 1];
  bf16x8 xk[!ELU ? 4 * KS : 1];
  bf16x8 v[EV / 8];

  // Rows past the end of the sequence are read from the last valid row (always
  // in bounds) and masked by the consumer, so no instruction here touches the
  // loaded values and the loads stay in flight until the next chunk needs them.
  __device__ __forceinline__ void load(const CausalArgs& a, long long tok0, int t0, int lane, int w) {
    const int g4 = lane >> 4, c16 = lane & 15;
    {
      const long long row = tok0 + min(t0 + lane, a.n - 1);
      if constexpr (ELU) {
#pragma unroll
        for (int j = 0; j < FR / 8; ++j) {
          if constexpr (WITH_Q) q[j] = *reinterpret_cast<const bf16x8*>(a.Q + row * R + w * FR + 8 * j);
          k[j] = *reinterpret_cast<const bf16x8*>(a.K + row * R + w * FR + 8 * j);
        }
      }
      if constexpr (GATE == GT_GLA) {
#pragma unroll
        for (int j = 0; j < FR / 8; ++j) g[j] = *reinterpret_cast<const bf16x8*>(a.g + row * R + w * FR + 8 * j);
      }
#pragma unroll
      for (int j = 0; j < EV / 8; ++j) v[j] = *reinterpret_cast<const bf16x8*>(a.V + row * E + w * EV + 8 * j);
    }
    if constexpr (!ELU) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const long long row = tok0 + min(t0 + 16 * tt + c16, a.n - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if constexpr (WITH_Q) xq[tt * KS + ks] = *reinterpret_cast<const bf16x8*>(a.Q + row * DK + 32 * ks + 8 * g4);
          xk[tt * KS + ks] = *reinterpret_cast<const bf16x8*>(a.K + row * DK + 32 * ks + 8 * g4);
        }
      }
    }
  }
};

// elu+1 features, gate factors and transposes of one chunk into LDS.
//   WITH_Q: pass 3 (writes q, k, kt, vt, gam); else pass 1 (kt, vt, gam, logg).
// L = valid tokens in the chunk. Rows t >= L get phi(k) = 0 and v = 0, and a
// zero log-gate, so they add nothing to the state.
template <int R, int E, int DK, int FMAP, int GATE, bool WITH_Q>
__device__ __forceinline__ void chunk_prelude(const RawChunk<R, E, DK, FMAP, GATE, WITH_Q>& raw, const CausalArgs& a,
                                              int L, float lg2gam, char* sm, int q_off, int k_off,
                                              int kt_off, int vt_off, int gam_off, int logg_off,
                                              int lane, int w) {
  using Raw = RawChunk<R, E, DK, FMAP, GATE, WITH_Q>;
  constexpr int RP = R + 8;
  const bool valid = lane < L;
  static_assert(FMAP == FM_ELU1, "FAVOR+ chunks use the kernels of chunked_favor.hpp");
  {
    const int t = lane;
    float decay_k = 1.f;
    if constexpr (GATE == GT_DECAY) decay_k = exp2f(float(L - 1 - t) * lg2gam);
#pragma unroll
    for (int j = 0; j < Raw::FR / 8; ++j) {
      const int f0 = w * Raw::FR + 8 * j;
      float vq[8], vk[8], vkh[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        float pq = WITH_Q ? elu1(to_f32(raw.q[WITH_Q ? j : 0][u])) : 0.f;
        float pk = valid ? elu1(to_f32(raw.k[j][u])) : 0.f;
        float kh = pk;
        if constexpr (GATE == GT_DECAY) kh = pk * decay_k;
        if constexpr (GATE == GT_GLA) {
          float la = valid ? gla_log_alpha(to_f32(raw.g[j][u]), a.inv_tau) : 0.f;
          float b = wave_inclusive_scan(la);
          float bend = __shfl(b, 63);
          pq *= __expf(b);
          kh = pk * __expf(bend - b);
          pk *= __expf(-b);
          if (lane == 0) {
            lds<float>(sm, gam_off + 4 * (f0 + u)) = __expf(bend);
            if constexpr (!WITH_Q) lds<float>(sm, logg_off + 4 * (f0 + u)) += bend;
          }
        }
        vq[u] = pq;
        vk[u] = pk;
        vkh[u] = kh;
      }
      if constexpr (WITH_Q) {
        lds<bf16x8>(sm, q_off + 2 * (t * RP + f0)) =
            cat8(pack4(vq[0], vq[1], vq[2], vq[3]), pack4(vq[4], vq[5], vq[6], vq[7]));
        lds<bf16x8>(sm, k_off + 2 * (t * RP + f0)) =
            cat8(pack4(vk[0], vk[1], vk[2], vk[3]), pack4(vk[4], vk[5], vk[6], vk[7]));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) lds<bf16>(sm, kt_off + 2 * ((f0 + u) * CP + t)) = (bf16)vkh[u];
    }
  }
  // values, transposed (rows past the end are zero)
  {
    constexpr int EV = Raw::EV;
    const bf16 zero = (bf16)0.f;
#pragma unroll
    for (int j = 0; j < EV / 8; ++j)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        lds<bf16>(sm, vt_off + 2 * ((w * EV + 8 * j + u) * CP + lane)) = valid ? raw.v[j][u] : zero;
  }
}

// S (wave slab: rows all R, value columns [w E/4, (w+1) E/4)) <- Gamma S + K^^T V.
template <int R, int E, int GATE>
__device__ __forceinline__ void state_update(f32x4 (&S)[R / 16][E / 64], char* sm, int kt_off,
                                             int vt_off, int gam_off, float gscale, int lane, int w) {
  const int g4 = lane >> 4, c16 = lane & 15;
  const int ebase = w * (E / 4);
  bf16x8 vb[E / 64][2];
#pragma unroll
  for (int eb = 0; eb < E / 64; ++eb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      vb[eb][ks] = lds<bf16x8>(sm, vt_off + 2 * ((ebase + 16 * eb + c16) * CP + 32 * ks + 8 * g4));
#pragma unroll
  for (int rt = 0; rt < R / 16; ++rt) {
    bf16x8 ka[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) ka[ks] = lds<bf16x8>(sm, kt_off + 2 * ((16 * rt + c16) * CP + 32 * ks + 8 * g4));
    float gr[4] = {gscale, gscale, gscale, gscale};
    if constexpr (GATE == GT_GLA) {
#pragma unroll
      for (int i = 0; i < 4; ++i) gr[i] = lds<float>(sm, gam_off + 4 * (16 * rt + 4 * g4 + i));
    }
#pragma unroll
    for (int eb = 0; eb < E / 64; ++eb) {
      f32x4 st = S[rt][eb];
      if constexpr (GATE != GT_NONE) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st[i] *= gr[i];
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) st = mfma16(ka[ks], vb[eb][ks], st);
      S[rt][eb] = st;
    }
  }
}

// z[row] <- Gamma z[row] + sum_t K^[t][row]   (thread `row` < R owns z[row])
template <int R, int GATE>
__device__ __forceinline__ float z_update(float zr, char* sm, int kt_off, int gam_off, float gscale, int row) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < kChunk / 8; ++j) {
    bf16x8 x = lds<bf16x8>(sm, kt_off + 2 * (row * CP + 8 * j));
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += to_f32(x[u]);
  }
  float G = gscale;
  if constexpr (GATE == GT_GLA) G = lds<float>(sm, gam_off + 4 * row);
  return G * zr + acc;
}

// ---------------------------------------------------------------------------
// Pass 1: each segment's own state contribution (segments 0 .. P-2).
// ---------------------------------------------------------------------------
template <int R, int E, int DK, int FMAP, int GATE>
__global__ __launch_bounds__(256) void causal_segment_state(CausalArgs a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  using LY = SegLayout<R, E>;
  const int lane = lane_id(), w = wave_id(), tid = threadIdx.x;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int s = blockIdx.x;
  const long long bh = blockIdx.y;
  const int h = int(bh % a.H);
  const int t_begin = s * a.seg_len;
  const int t_end = min(a.n, t_begin + a.seg_len);
  const long long tok0 = bh * a.n;
  const int ebase = w * (E / 4);
  float lg2gam = 0.f;
  if constexpr (GATE == GT_DECAY) lg2gam = log2f(a.gamma[h]);

  f32x4 S[R / 16][E / 64];
#pragma unroll
  for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
    for (int eb = 0; eb < E / 64; ++eb) S[rt][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zr = 0.f;
  if (tid < R) lds<float>(sm, LY::logg_off + 4 * tid) = 0.f;
  lds_barrier();

  RawChunk<R, E, DK, FMAP, GATE, false> raw;
  raw.load(a, tok0, t_begin, lane, w);
  for (int t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int L = min(kChunk, a.n - t0);
    chunk_prelude<R, E, DK, FMAP, GATE, false>(raw, a, L, lg2gam, sm, 0, 0, LY::kt_off, LY::vt_off,
                                               LY::gam_off, LY::logg_off, lane, w);
    lds_barrier();
    if (t0 + kChunk < t_end) raw.load(a, tok0, t0 + kChunk, lane, w);
    const float gsc = GATE == GT_DECAY ? exp2f(float(L) * lg2gam) : 1.f;
    state_update<R, E, GATE>(S, sm, LY::kt_off, LY::vt_off, LY::gam_off, gsc, lane, w);
    if (tid < R) zr = z_update<R, GATE>(zr, sm, LY::kt_off, LY::gam_off, gsc, tid);
    lds_barrier();
  }
  const long long slot = bh * a.P + s;
  float* So = a.S_out + slot * R * E;
#pragma unroll
  for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
    for (int eb = 0; eb < E / 64; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i) So[(16 * rt + 4 * g4 + i) * E + ebase + 16 * eb + c16] = S[rt][eb][i];
  if (tid < R) {
    a.z_out[slot * R + tid] = zr;
    if constexpr (GATE == GT_GLA) a.logG_out[slot * R + tid] = lds<float>(sm, LY::logg_off + 4 * tid);
  }
}

// ---------------------------------------------------------------------------
// Pass 3: outputs of one segment, starting from its chained state.
// ---------------------------------------------------------------------------
template <int R, int E, int DK, int FMAP, int GATE>
__global__ __launch_bounds__(256) void causal_chunk_forward(CausalArgs a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  using LY = FwdLayout<R, E>;
  constexpr int RP = LY::RP, NEB = E / 64, KP = R / 32;
  const int lane = lane_id(), w = wave_id(), tid = threadIdx.x;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int s = blockIdx.x;
  const long long bh = blockIdx.y;
  const int h = int(bh % a.H);
  const int t_begin = s * a.seg_len;
  const int t_end = min(a.n, t_begin + a.seg_len);
  const long long tok0 = bh * a.n;
  const int ebase = w * (E / 4);
  float lg2gam = 0.f;
  if constexpr (GATE == GT_DECAY) lg2gam = log2f(a.gamma[h]);

  // ---- state carried in
  f32x4 S[R / 16][NEB];
  float zr = 0.f;
  if (a.S_in != nullptr) {
    const float* Sp = a.S_in + bh * a.in_head + s * a.in_seg;
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[rt][eb][i] = Sp[(16 * rt + 4 * g4 + i) * E + ebase + 16 * eb + c16];
    if (tid < R) zr = a.z_in[(bh * a.in_head + s * a.in_seg) / E + tid];
  } else {
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) S[rt][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (tid < R) lds<float>(sm, LY::z_off + 4 * tid) = zr;
  // bf16 image of the state as the A operand of O^T += S^T Q^^T: k-slot j of
  // lane (g, c) is feature 32p + 4g + j (j < 4) or 32p + 16 + 4g + (j - 4).
  bf16x8 Sop[KP][NEB];
  auto rebuild_sop = [&]() {
#pragma unroll
    for (int p = 0; p < KP; ++p)
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
        Sop[p][eb] = cat8(pack4(S[2 * p][eb][0], S[2 * p][eb][1], S[2 * p][eb][2], S[2 * p][eb][3]),
                          pack4(S[2 * p + 1][eb][0], S[2 * p + 1][eb][1], S[2 * p + 1][eb][2], S[2 * p + 1][eb][3]));
  };
  rebuild_sop();

  RawChunk<R, E, DK, FMAP, GATE, true> raw;
  raw.load(a, tok0, t_begin, lane, w);
  for (int t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int L = min(kChunk, a.n - t0);
    chunk_prelude<R, E, DK, FMAP, GATE, true>(raw, a, L, lg2gam, sm, LY::q_off, LY::k_off, LY::kt_off,
                                              LY::vt_off, LY::gam_off, 0, lane, w);
    lds_barrier();

    // ---- scores for query rows [16w, 16w+16): A^T tiles = K~_c Q~_w^T
    {
      bf16x8 qop[KP];
#pragma unroll
      for (int ks = 0; ks < KP; ++ks) qop[ks] = lds<bf16x8>(sm, LY::q_off + 2 * ((16 * w + c16) * RP + 32 * ks + 8 * g4));
      const int q = 16 * w + c16;
      float rs = 0.f;
      for (int c = 0; c <= w; ++c) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KP; ++ks)
          acc = mfma16(lds<bf16x8>(sm, LY::k_off + 2 * ((16 * c + c16) * RP + 32 * ks + 8 * g4)), qop[ks], acc);
        // acc[i] = A[q][key], key = 16c + 4g + i
        bf16x4 ab;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * c + 4 * g4 + i;
          float v = acc[i];
          if (key > q) v = 0.f;
          if constexpr (GATE == GT_DECAY) v *= exp2f(float(q - key) * lg2gam);
          ab[i] = (bf16)v;
          rs += to_f32(ab[i]);
        }
        lds<bf16x4>(sm, LY::a_off + 2 * (q * CP + 16 * c + 4 * g4)) = ab;
      }
      if ((w & 1) == 0) lds<bf16x4>(sm, LY::a_off + 2 * (q * CP + 16 * (w + 1) + 4 * g4)) = bf16x4{};
      float zd = 0.f;
#pragma unroll
      for (int ks = 0; ks < KP; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) zd += to_f32(qop[ks][j]) * lds<float>(sm, LY::z_off + 4 * (32 * ks + 8 * g4 + j));
      rs = sum_over_groups(rs);
      zd = sum_over_groups(zd);
      if constexpr (GATE == GT_DECAY) zd *= exp2f(float(q + 1) * lg2gam);
      if (g4 == 0) lds<float>(sm, LY::den_off + 4 * q) = rs + zd + a.eps;
    }
    lds_barrier();
    if (t0 + kChunk < t_end) raw.load(a, tok0, t0 + kChunk, lane, w);

    // ---- outputs for value columns [w E/4, (w+1) E/4): O^T = S^T Q^^T + V^T A^T
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const int q = 16 * qt + c16;
      bf16x8 qb[KP];
#pragma unroll
      for (int p = 0; p < KP; ++p)
        qb[p] = cat8(lds<bf16x4>(sm, LY::q_off + 2 * (q * RP + 32 * p + 4 * g4)),
                     lds<bf16x4>(sm, LY::q_off + 2 * (q * RP + 32 * p + 16 + 4 * g4)));
      const float den = lds<float>(sm, LY::den_off + 4 * q);
      float isc = 1.f;
      if constexpr (GATE == GT_DECAY) isc = exp2f(float(q + 1) * lg2gam);
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) {
        const int e = ebase + 16 * eb;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < KP; ++p) acc = mfma16(Sop[p][eb], qb[p], acc);
        if constexpr (GATE == GT_DECAY) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] *= isc;
        }
#pragma unroll
        for (int p2 = 0; p2 <= qt / 2; ++p2)
          acc = mfma16(lds<bf16x8>(sm, LY::vt_off + 2 * ((e + c16) * CP + 32 * p2 + 8 * g4)),
                       lds<bf16x8>(sm, LY::a_off + 2 * (q * CP + 32 * p2 + 8 * g4)), acc);
        if (q < L) {
          bf16x4 o = pack4(acc[0] / den, acc[1] / den, acc[2] / den, acc[3] / den);
          *reinterpret_cast<bf16x4*>(a.out + (tok0 + t0 + q) * E + e + 4 * g4) = o;
        }
      }
    }

    // ---- carry the state past this chunk
    const float gsc = GATE == GT_DECAY ? exp2f(float(L) * lg2gam) : 1.f;
    state_update<R, E, GATE>(S, sm, LY::kt_off, LY::vt_off, LY::gam_off, gsc, lane, w);
    rebuild_sop();
    if (tid < R) {
      zr = z_update<R, GATE>(zr, sm, LY::kt_off, LY::gam_off, gsc, tid);
      lds<float>(sm, LY::z_off + 4 * tid) = zr;
    }
    lds_barrier();
  }

  if (a.S_out != nullptr && s == a.P - 1) {
    float* So = a.S_out + bh * R * E;
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int i = 0; i < 4; ++i) So[(16 * rt + 4 * g4 + i) * E + ebase + 16 * eb + c16] = S[rt][eb][i];
    if (tid < R) a.z_out[bh * R + tid] = zr;
  }
}

// Host side: launch pass 1 / scan / pass 3 for one template instance.
template <int R, int E, int DK, int FMAP, int GATE>
la_status run_causal(const FwdPlan& p) {
  CausalArgs a{};
  a.Q = static_cast<const bf16*>(p.Q);
  a.K = static_cast<const bf16*>(p.K);
  a.V = static_cast<const bf16*>(p.V);
  a.g = static_cast<const bf16*>(p.g);
  a.omega = static_cast<const bf16*>(p.omega);
  a.gamma = p.gamma;
  a.out = static_cast<bf16*>(p.out);
  a.H = p.H;
  a.n = p.n;
  a.P = p.P;
  a.seg_len = p.seg_len;
  a.eps = p.eps;
  a.inv_tau = GATE == GT_GLA ? 1.f / p.tau : 0.f;
  const unsigned BH = unsigned(p.B) * unsigned(p.H);

  if (p.P > 1) {
    CausalArgs a1 = a;
    a1.S_out = p.ws_S;
    a1.z_out = p.ws_z;
    a1.logG_out = p.ws_logG;
    auto k1 = causal_segment_state<R, E, DK, FMAP, GATE>;
    constexpr int lds1 = SegLayout<R, E>::bytes;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(k1), hipFuncAttributeMaxDynamicSharedMemorySize, lds1) !=
        hipSuccess)
      return LA_ERR_HIP;
    hipLaunchKernelGGL(k1, dim3(p.P - 1, BH), dim3(256), lds1, p.stream, a1);
    if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
    la_status st = launch_segment_scan(p);
    if (st != LA_OK) return st;
    a.S_in = p.ws_S;
    a.z_in = p.ws_z;
    a.in_head = (long long)p.P * R * E;
    a.in_seg = (long long)R * E;
  } else {
    a.S_in = p.S0;
    a.z_in = p.z0;
    a.in_head = (long long)R * E;
    a.in_seg = 0;
  }
  a.S_out = p.S_final;
  a.z_out = p.z_final;
  auto k3 = causal_chunk_forward<R, E, DK, FMAP, GATE>;
  constexpr int lds3 = FwdLayout<R, E>::bytes;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k3), hipFuncAttributeMaxDynamicSharedMemorySize, lds3) !=
      hipSuccess)
    return LA_ERR_HIP;
  hipLaunchKernelGGL(k3, dim3(p.P, BH), dim3(256), lds3, p.stream, a);
  if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
  return LA_OK;
}

}  // namespace la
