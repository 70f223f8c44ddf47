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
// weights gamma^(i-j), gamma^(i+1) and gamma^(L-1-j) are applied directly, and
// the selective scalar gate applies e^{b_i - b_j} from its per-token b. The
// outer-product gate adds the value side: V~ = V e^{-c} per value column, the
// outputs times e^{c}, the state's columns times e^{c_end} (z keeps the key
// side only).
//
// To fill 256 compute units with few heads, each head's sequence is split into
// P segments of whole chunks: pass 1 computes each segment's own state
// contribution, a scan chains them, and pass 3 recomputes every segment's
// outputs starting from its chained state.
//
// Workgroup = NW waves: 4, or 8 for 128 x 128 states (so the per-wave share of
// the state and of the chunk's registers fits two waves per SIMD). Waves 0..3
// own query rows [16w, 16w+16) of the chunk for the scores (with 8 waves,
// waves 4..7 compute phi(q) . z for those rows), and wave w owns value columns
// [w E/NW, (w+1) E/NW) of the state and the outputs. The fp32 state lives in MFMA accumulators for the whole
// sequence; its bf16 image feeds the inter-chunk product straight from
// registers. LDS holds the chunk's operands (bf16), all [row][column]:
//   q  [64][R]     Q~ (also Q^)      k [64][R]     K~      v [64][E]   V
//   a  [64][64]    masked scores     kh [64][R]    K^ (RetNet only)
// In the output pass every tile has unpadded rows whose 16-byte chunks are
// permuted per row (FeatTile); the segment pass pads its rows instead.
// Operands that contract over tokens (the state update, V^T A^T) are read
// with the LDS transpose read (ds_read_b64_tr_b16).
// Without a gate K^ = K~; with the GLA gate K^ = Gamma K~ feature by feature,
// so the state update is S <- Gamma (S + K~^T V); RetNet weights each key row
// and keeps K^ in a tile of its own (pass 1 stores only K^, in the k tile).
#pragma once

#include <type_traits>

#include "common.hpp"
#include "plan.hpp"

namespace la {

// FM_PRE: features computed beforehand and passed in place of q and k (the
// FAVOR+ backward runs the elementwise kernels on its materialised features):
// taken as they are, like the identity, but with the normalised read-out.
enum FmapKind { FM_ELU1 = 0, FM_FAVOR = 1, FM_IDENT = 2, FM_PRE = 3 };

// Elementwise feature maps of the chunk prelude: elu+1, or the identity of the
// state-space form (whose read-out is not normalised) and of precomputed features.
template <int FMAP>
__device__ __forceinline__ float phi_ew(float x) {
  if constexpr (FMAP == FM_IDENT || FMAP == FM_PRE) return x;
  else return elu1(x);
}
// phi(x) 2^s in one exponential, and the factor e = phi'(x) 2^s: for elu+1,
// (x + 1) 2^s above zero and 2^(x log2(e) + s) below (phi' = 1 above, e^x
// below, so e is the exponential itself); for the identity, x 2^s and 2^s.
// The gated preludes need phi(q) e^{b}, phi(k) e^{-b} and e^{b} phi'(q), ...:
// one transcendental each instead of one for phi and one for the gate.
template <int FMAP>
__device__ __forceinline__ float phi_times_exp2(float x, float s, float& e) {
  if constexpr (FMAP == FM_IDENT || FMAP == FM_PRE) {
    e = __builtin_amdgcn_exp2f(s);
    return x * e;
  } else {
    // with m = min(x, 0): e = 2^(m log2(e) + s) and phi 2^s = (x - m + 1) e,
    // the two branches' values without a compare or select (x - m is the
    // positive part and keeps a NaN input a NaN)
    const float m = fminf(x, 0.f);
    e = __builtin_amdgcn_exp2f(__builtin_fmaf(m, kLog2e, s));
    return __builtin_fmaf(x - m, e, e);
  }
}
// Its derivative from the feature value: min(phi, 1) for elu+1 (1 above zero,
// exp(x) = phi below), 1 for the identity and precomputed features.
template <int FMAP>
__device__ __forceinline__ float phi_ew_deriv(float phi) {
  if constexpr (FMAP == FM_IDENT || FMAP == FM_PRE) return 1.f;
  else return fminf(phi, 1.f);
}
enum GateKind { GT_NONE = 0, GT_DECAY = 1, GT_GLA = 2, GT_SEL = 3, GT_OUTER = 4 };
// Gates with an input-dependent factor per key feature: GLA, and the
// outer-product gate, which adds a factor per value column.
template <int GATE>
constexpr bool kKeyGate = GATE == GT_GLA || GATE == GT_OUTER;
// Gates that scale every feature of a step alike (RetNet's fixed gamma, the
// selective scalar a_t): keys are weighted per token, one factor per step.
template <int GATE>
constexpr bool kScalarDecay = GATE == GT_DECAY || GATE == GT_SEL;

struct CausalArgs {
  const bf16* Q;
  const bf16* K;
  const bf16* V;
  const bf16* g;
  const bf16* gv;          // the outer-product gate's value-side input [tok][E]
  const bf16* omega;
  const float* gamma;
  const float* S_in;       // pass 3: initial state per (head, segment); nullable
  const float* z_in;
  long long in_head;       // S_in element stride between heads
  long long in_seg;        // S_in element stride between segments
  float* S_out;            // pass 1: per-segment deltas; pass 3: final state (nullable)
  float* z_out;
  float* logG_out;         // pass 1, gates with an input: per-segment summed log-gates
  float* logGv_out;        // pass 1, outer-product gate: per-segment summed value-side log-gates
  bf16* out;
  // A batch of independent sequences: with cu, blockIdx.y = b H + h and
  // sequence b is tokens cu[b] .. cu[b+1] of head h's n rows ([H][n][.]
  // layout); without it, sequence (b, h) is rows (b H + h) n .. + n. The
  // carried state of sequence b, head h is [.][H] entry slot[b] H + h (or
  // b H + h without slot); slots outside [0, nslot) mean no carried state.
  const int* cu;
  const int* slot;
  int nslot;
  int in_is_state;         // S_in is the caller's carried state (indexed like S_out), not the segment workspace
  int ldv;                 // elements between rows of V (0: d_v, dense); the backward's value-column halves
  int ldgv;                // elements between rows of gv (0: d_v, dense)
  int H, n, P, seg_len;
  int nbh;                 // sequences x heads (set by launchers whose grid is not [.][nbh])
  int r_valid;             // FAVOR+: the map's feature count when below R (features past it are zero); 0 = R
  float eps, inv_tau;
};

// Rows, length and carried-state index of the sequence of workgroup row bh.
// Offsets are clamped into [0, n] and lengths to the planned P seg_len, so a
// malformed table cannot address memory outside the inputs and outputs.
struct SeqView {
  long long tok0;  // row of the first token
  int len;         // tokens
  long long st;    // carried-state index, -1 for none
};
__device__ __forceinline__ SeqView seq_view(const CausalArgs& a, long long bh) {
  SeqView v;
  const int b = int(bh / a.H), h = int(bh % a.H);
  if (a.cu == nullptr) {
    v.tok0 = bh * a.n;
    v.len = a.n;
  } else {
    const int lo = min(max(a.cu[b], 0), a.n);
    const int hi = min(max(a.cu[b + 1], lo), a.n);
    v.tok0 = (long long)h * a.n + lo;
    v.len = min(hi - lo, a.P * a.seg_len);
  }
  v.st = bh;
  if (a.slot != nullptr) {
    const int sl = a.slot[b];
    v.st = (sl >= 0 && sl < a.nslot) ? (long long)sl * a.H + h : -1;
  }
  return v;
}

// Row padding (bf16 elements) of padded tiles: rows of 32, 64 or 128
// elements plus 8 start 4 dwords apart modulo the banks.
constexpr int kPad = 8;
constexpr int CP = kChunk + kPad;  // row stride (elements) of the score tile

// LDS tiles of 64 rows ([token][feature], [token][value column] or
// [query][key] bf16) of R columns, rows of 2R bytes without padding. The
// 16-byte chunk k of row t is stored at chunk k ^ swz(t), where swz maps the
// row bits that alias LDS banks for each row width onto chunk bits. The chunk
// kernels access these tiles as 16-byte row fragments (rows c, chunks g +
// const, c < 16, g < 4), 8-byte row fragments (16 rows, one chunk half) and
// transpose reads (rows 8 g + j and + 4, j < 4; 8-byte column groups), each
// spread over all 64 banks by this permutation, which no row padding achieves
// for all three at once (measured on gfx950: 16-byte rows are 2-way conflicted
// at a 144-byte stride, 8-byte rows at 160).
// With SWZ false the rows are instead padded by kPad elements (the segment
// pass, which reads these tiles only by transpose reads, conflict-free at that
// stride, and runs with fewer registers without the per-row permutation).
template <int R, bool SWZ = true>
struct FeatTile {
  static constexpr int ROW = 2 * R + (SWZ ? 0 : 2 * kPad);  // bytes per token row
  static constexpr int BYTES = kChunk * ROW;
  __device__ static __forceinline__ int swz(int t) {
    if constexpr (!SWZ) return 0;
    else if constexpr (R == 32) return 2 * ((t >> 2) & 1) | ((t >> 3) & 1);
    else if constexpr (R == 64) return 4 * ((t >> 1) & 1) | 2 * ((t >> 2) & 1) | ((t >> 3) & 1);
    else return 8 * ((t >> 2) & 1) | 4 * ((t >> 1) & 1) | 2 * (t & 1) | ((t >> 3) & 1);
  }
  // byte offset of byte b of 16-byte chunk k of row t
  __device__ static __forceinline__ int at(int t, int k, int b = 0) { return t * ROW + 16 * (k ^ swz(t)) + b; }
};

// Waves per workgroup of the elu+1 chunk kernels.
template <int R, int E>
struct Waves {
  static constexpr int NW = R * E >= 128 * 128 ? 8 : 4;
};

template <int R, int E, int GATE>
struct FwdLayout {
  // every [token][column] tile (q, k, kh, v, and the [query][key] scores) is
  // stored with the per-row chunk permutation of FeatTile
  static constexpr bool SWZ = true;
  static constexpr int FTB = FeatTile<R, SWZ>::BYTES;
  static constexpr int q_off = 0;
  static constexpr int k_off = q_off + FTB;
  static constexpr int v_off = k_off + FTB;
  static constexpr int kh_off = v_off + FeatTile<E, SWZ>::BYTES;
  // K^ rows of the state update: RetNet and the selective gate weight each key
  // row; the outer-product gate references its keys to the chunk end
  static constexpr int a_off = kh_off + (kScalarDecay<GATE> || GATE == GT_OUTER ? FTB : 0);
  static constexpr int z_off = a_off + FeatTile<kChunk, SWZ>::BYTES;
  static constexpr int gam_off = z_off + R * 4;
  static constexpr int rs_off = gam_off + R * 4;   // [64] score row sums
  static constexpr int zd_off = rs_off + kChunk * 4;  // [64] Q^ . z_prev
  static constexpr int bs_off = zd_off + kChunk * 4;  // selective gate: [64] cumulative log-gate
  // outer-product gate: e^{c} per token and value column (fp32, rows of E + 4:
  // 16-byte reads of 16 rows spread over the banks), e^{c_end} per column
  static constexpr int ec_off = bs_off + (GATE == GT_SEL ? kChunk * 4 : 0);
  static constexpr int gamv_off = ec_off + (GATE == GT_OUTER ? kChunk * (E + 4) * 4 : 0);
  // outer-product gate: the low bf16 half of V~ (V~ = hi + lo, hi in the v tile)
  static constexpr int vl_off = gamv_off + (GATE == GT_OUTER ? E * 4 : 0);
  static constexpr int bytes = vl_off + (GATE == GT_OUTER ? FeatTile<E, SWZ>::BYTES : 0);
};

// Pass 1: one chunk (K^ rows, V rows, gate factors) per half, then the
// segment's summed log-gates. With a per-feature gate (GLA, outer) the pass is software-pipelined
// over two halves (measured: 6% faster there; the ungated and RetNet passes,
// whose preludes are short, run 2-5% slower pipelined).
template <int R, int E, int GATE>
struct SegLayout {
  static constexpr bool PIPELINED = kKeyGate<GATE>;
  static constexpr bool SWZ = false;  // padded tiles (FeatTile)
  static constexpr int k_off = 0;     // K^ rows
  static constexpr int v_off = k_off + FeatTile<R, SWZ>::BYTES;
  static constexpr int gam_off = v_off + FeatTile<E, SWZ>::BYTES;
  static constexpr int gamv_off = gam_off + R * 4;  // outer-product gate: [E] e^{c_end}
  static constexpr int vl_off = gamv_off + (GATE == GT_OUTER ? E * 4 : 0);  // outer-product gate: lo half of V~
  static constexpr int HALF = vl_off + (GATE == GT_OUTER ? FeatTile<E, SWZ>::BYTES : 0);
  static constexpr int logg_off = (PIPELINED ? 2 : 1) * HALF;
  static constexpr int loggv_off = logg_off + R * 4;  // outer-product gate: [E] summed value-side log-gates
  static constexpr int bs_off = loggv_off + (GATE == GT_OUTER ? E * 4 : 0);  // selective gate: [64] cumulative log-gate
  static constexpr int bytes = bs_off + (GATE == GT_SEL ? kChunk * 4 : 0);
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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// MFMA operand from a [token][column] tile (FeatTile) by transpose reads
// (ds_read_b64_tr_b16): lane (g, c) receives column col0 + c (col0 a multiple of
// 16) of rows k0 + 8 g + 0..7 (k0 a multiple of 8). Within each 16-lane group
// the transpose read hands lane i element j of the 4-element piece addressed by
// lane 4 j + i / 4, so lane m = 4 j + q addresses row k0 + 8 g + j (+4 for the
// second read), columns col0 + 4 q .. + 3: half q & 1 of chunk col0 / 8 + q / 2.
template <int R, bool SWZ>
__device__ __forceinline__ bf16x8 tr_feat(char* sm, int tile_off, int k0, int col0, int lane) {
  using FT = FeatTile<R, SWZ>;
  const int g4 = lane >> 4, c16 = lane & 15, q = c16 & 3;
  const int t = k0 + 8 * g4 + (c16 >> 2), k = col0 / 8 + (q >> 1), b = 8 * (q & 1);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sm + tile_off + FT::at(t, k, b)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sm + tile_off + FT::at(t + 4, k, b)));
  return cat8(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi));
}

// Raw inputs of one chunk, held in registers from the global load to the LDS
// write so the next chunk's loads overlap the current chunk's math.
//
// Two register layouts of a chunk:
//  * row-major (elu+1 without the GLA gate): wave w holds TPW = 64 / NW tokens
//    [TPW w, TPW (w+1)), LPT = NW lanes per token; lane l holds 8-feature
//    blocks (l % LPT) + LPT j of token TPW w + l / LPT, so each load
//    instruction reads TPW rows, 16 LPT contiguous bytes of each;
//  * lane-per-token (GLA gate, whose scan runs across the 64 lanes): lane l
//    holds token l, wave w holds features [w R/NW, (w+1) R/NW); V uses this
//    layout for FAVOR+ too.
// FAVOR+ inputs X (projected inside the kernel): wave w holds tokens
// [16w, 16w+16), lane l token 16 w + l % 16, columns 32 ks + 8 (l / 16) .. + 7.
// SG (the GLA passes serving the selective gate's backward): g holds one
// input per token, used for every feature.
template <int R, int E, int DK, int FMAP, int GATE, bool WITH_Q, int NW = 4, bool SG = false>
struct RawChunk {
  static constexpr int FR = R / NW;      // features per wave (lane-per-token layout)
  static constexpr int EV = E / NW;      // value columns per wave
  static constexpr int KS = DK / 32;     // projection k-steps (FAVOR)
  static constexpr int TPW = kChunk / NW;  // tokens per wave (row-major layout)
  static constexpr int LPT = NW;           // lanes per token (row-major layout)
  static constexpr bool ELU = FMAP != FM_FAVOR;  // elementwise feature maps
  static constexpr bool ROWMAJOR = ELU && !kKeyGate<GATE>;
  // row-major: R / (8 LPT) blocks of 8 features per lane per row (= FR / 8)
  bf16x8 q[ELU && WITH_Q ? FR / 8 : 1];
  bf16x8 k[ELU ? FR / 8 : 1];
  bf16x8 g[kKeyGate<GATE> ? FR / 8 : 1];
  bf16 gs;  // SG: the token's one gate input (used for every feature)
  bf16x8 gv[GATE == GT_OUTER ? EV / 8 : 1];  // outer-product gate: value-side inputs, as v
  bf16 sg;  // selective gate: the input of token t0 + lane (every wave loads all 64)
  bf16x8 xq[!ELU && WITH_Q ? KS : 1];   // FAVOR+: token 16 w + l % 16, columns 32 ks + 8 (l / 16)
  bf16x8 xk[!ELU ? KS : 1];
  bf16x8 v[EV / 8];

  // Rows at or past row_end (the end of the segment, at most n) are read from
  // row row_end - 1 (always in bounds) and masked by the consumer, so no
  // instruction here touches the loaded values and the loads stay in flight
  // until the next chunk needs them. A load for a chunk past the segment is
  // therefore harmless, which lets the loops issue every refill
  // unconditionally.
  __device__ __forceinline__ void load(const CausalArgs& a, long long tok0, int t0, int row_end, int lane, int w) {
    const int g4 = lane >> 4, c16 = lane & 15;
    const long long ldv = a.ldv > 0 ? a.ldv : E;
    const long long ldgv = a.ldgv > 0 ? a.ldgv : E;
    if constexpr (GATE == GT_SEL) sg = a.g[tok0 + min(t0 + lane, row_end - 1)];
    if constexpr (ROWMAJOR) {
      const long long row = tok0 + min(t0 + TPW * w + lane / LPT, row_end - 1);
#pragma unroll
      for (int j = 0; j < R / (8 * LPT); ++j) {
        const int f0 = 8 * (lane % LPT + LPT * j);
        if constexpr (WITH_Q) q[j] = *reinterpret_cast<const bf16x8*>(a.Q + row * R + f0);
        k[j] = *reinterpret_cast<const bf16x8*>(a.K + row * R + f0);
      }
#pragma unroll
      for (int j = 0; j < E / (8 * LPT); ++j)
        v[j] = *reinterpret_cast<const bf16x8*>(a.V + row * ldv + 8 * (lane % LPT + LPT * j));
      return;
    }
    {
      const long long row = tok0 + min(t0 + lane, row_end - 1);
      if constexpr (ELU) {
#pragma unroll
        for (int j = 0; j < FR / 8; ++j) {
          if constexpr (WITH_Q) q[j] = *reinterpret_cast<const bf16x8*>(a.Q + row * R + w * FR + 8 * j);
          k[j] = *reinterpret_cast<const bf16x8*>(a.K + row * R + w * FR + 8 * j);
        }
      }
      if constexpr (kKeyGate<GATE> && SG) {
        gs = a.g[row];
      } else if constexpr (kKeyGate<GATE>) {
#pragma unroll
        for (int j = 0; j < FR / 8; ++j) g[j] = *reinterpret_cast<const bf16x8*>(a.g + row * R + w * FR + 8 * j);
      }
#pragma unroll
      for (int j = 0; j < EV / 8; ++j) v[j] = *reinterpret_cast<const bf16x8*>(a.V + row * ldv + w * EV + 8 * j);
      if constexpr (GATE == GT_OUTER) {
#pragma unroll
        for (int j = 0; j < EV / 8; ++j) gv[j] = *reinterpret_cast<const bf16x8*>(a.gv + row * ldgv + w * EV + 8 * j);
      }
    }
    if constexpr (!ELU) {
      const long long row = tok0 + min(t0 + 16 * w + c16, row_end - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (WITH_Q) xq[ks] = *reinterpret_cast<const bf16x8*>(a.Q + row * DK + 32 * ks + 8 * g4);
        xk[ks] = *reinterpret_cast<const bf16x8*>(a.K + row * DK + 32 * ks + 8 * g4);
      }
    }
  }
};

// elu+1 features and gate factors of one chunk into LDS ([token][column] tiles).
//   WITH_Q: pass 3 (writes q, k, v, gam; kh for RetNet); else pass 1 (k holding
//   K^, v, gam, logg).
// L = valid tokens in the chunk. Rows t >= L get phi(k) = 0 and v = 0, and a
// zero log-gate, so they add nothing to the state.
// EXTRA (GLA, backward pass), a mask of: kPreQD also writes the tile
// qd = e^{b} phi'(q), kPreKD the tile kd = e^{-b} phi'(k) (phi'(x) =
// min(phi(x), 1) for elu+1), the factors that turn gradients with respect to
// Q~ and K~ into gradients of q and k; kPreLogG adds the chunk's summed
// log-gates to logg also when WITH_Q; kPreKPos scales the key slot by e^{+b}
// (the Q~ of the reverse state, with the queries passed as keys). For the
// outer-product gate's backward: kPreVRaw stores the value slot as loaded
// (the reverse state's G~ = e^{+c} g, already scaled) while still taking the
// value-side totals; kPreNoKH skips the K^ tile and kPreVHi the lo half of V~
// (the reverse pass needs neither). kPreKLo (WITH_Q) also writes the bf16
// residual of the key slot (its fp32 value minus the stored bf16) at klo_off,
// and kPreQLo that of the query slot at qlo_off, for products that take them
// as hi + lo pairs.
constexpr int kPreQD = 1, kPreKD = 2, kPreLogG = 4, kPreKPos = 8, kPreVRaw = 16, kPreNoKH = 32, kPreVHi = 64,
              kPreKLo = 128, kPreQLo = 256;

// Eight floats as bf16 (hi) and their bf16 residuals x - hi (lo).
__device__ __forceinline__ bf16x8 bf16_residual8(const float (&x)[8], const bf16x8& hi) {
  float r[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) r[u] = x[u] - to_f32(hi[u]);
  return cat8(pack4(r[0], r[1], r[2], r[3]), pack4(r[4], r[5], r[6], r[7]));
}
template <int R, int E, int DK, int FMAP, int GATE, bool WITH_Q, int NW, bool SWZ, int EXTRA = 0, bool SG = false>
__device__ __forceinline__ void chunk_prelude(const RawChunk<R, E, DK, FMAP, GATE, WITH_Q, NW, SG>& raw,
                                              const CausalArgs& a, int L, float lg2gam, char* sm, int q_off,
                                              int k_off, int kh_off, int v_off, int gam_off, int logg_off,
                                              int lane, int w, int qd_off = 0, int kd_off = 0, int bs_off = 0,
                                              int ec_off = 0, int gamv_off = 0, int loggv_off = 0, int vl_off = 0,
                                              int klo_off = 0, int qlo_off = 0) {
  using Raw = RawChunk<R, E, DK, FMAP, GATE, WITH_Q, NW, SG>;
  constexpr int LPT = Raw::LPT;
  using FT = FeatTile<R, SWZ>;
  using VT = FeatTile<E, SWZ>;
  static_assert(FMAP != FM_FAVOR, "FAVOR+ chunks use the kernels of chunked_favor.hpp");
  if constexpr (Raw::ROWMAJOR) {
    const int t = Raw::TPW * w + lane / LPT;
    const bool valid = t < L;
    float decay_k = 1.f;
    if constexpr (GATE == GT_DECAY) decay_k = exp2f(float(max(L - 1 - t, 0)) * lg2gam);  // rows past L are dropped
    if constexpr (GATE == GT_SEL) {
      // the chunk's inclusive cumulative log-gate b, lane = token (each wave
      // scans all 64); keys are weighted e^{b_end - b_t} for the state
      const float la = keep_if(lane < L, gla_log_alpha(to_f32(raw.sg), a.inv_tau));
      const float b = wave_inclusive_scan(la);
      const float bend = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, b), 63));
      decay_k = __expf(bend - __shfl(b, t));
      if (w == 0) lds<float>(sm, bs_off + 4 * lane) = b;
      if constexpr (!WITH_Q) {
        if (64 * w + lane < R) lds<float>(sm, logg_off + 4 * (64 * w + lane)) += bend;
      }
    }
#pragma unroll
    for (int j = 0; j < R / (8 * LPT); ++j) {
      const int f0 = 8 * (lane % LPT + LPT * j);
      float vq[8], vk[8], vkh[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        vq[u] = WITH_Q ? phi_ew<FMAP>(to_f32(raw.q[WITH_Q ? j : 0][u])) : 0.f;
        vk[u] = phi_ew<FMAP>(to_f32(raw.k[j][u]));
        vkh[u] = vk[u] * decay_k;
      }
      const int fo = FT::at(t, f0 / 8);
      if constexpr (WITH_Q) {
        const bf16x8 qr = cat8(pack4(vq[0], vq[1], vq[2], vq[3]), pack4(vq[4], vq[5], vq[6], vq[7]));
        lds<bf16x8>(sm, q_off + fo) = qr;
        if constexpr ((EXTRA & kPreQLo) != 0) lds<bf16x8>(sm, qlo_off + fo) = bf16_residual8(vq, qr);
      }
      // keys past the end are zeroed after packing (four masks per eight features)
      const bf16x8 kr = keep_if(valid, cat8(pack4(vk[0], vk[1], vk[2], vk[3]), pack4(vk[4], vk[5], vk[6], vk[7])));
      const bf16x8 khr =
          keep_if(valid, cat8(pack4(vkh[0], vkh[1], vkh[2], vkh[3]), pack4(vkh[4], vkh[5], vkh[6], vkh[7])));
      if constexpr (!kScalarDecay<GATE>) {
        lds<bf16x8>(sm, k_off + fo) = kr;
      } else if constexpr (WITH_Q) {
        lds<bf16x8>(sm, k_off + fo) = kr;
        lds<bf16x8>(sm, kh_off + fo) = khr;
      } else {
        lds<bf16x8>(sm, k_off + fo) = khr;
      }
      if constexpr (WITH_Q && (EXTRA & kPreKLo) != 0) lds<bf16x8>(sm, klo_off + fo) = keep_if(valid, bf16_residual8(vk, kr));
    }
#pragma unroll
    for (int j = 0; j < E / (8 * LPT); ++j)
      lds<bf16x8>(sm, v_off + VT::at(t, lane % LPT + LPT * j)) = keep_if(valid, raw.v[j]);
    return;
  }
  const bool valid = lane < L;
  {
    const int t = lane;
    // GLA: lane f (< FR) collects the chunk's summed log-gate of this wave's
    // feature f; one store per lane after the feature loop.
    float my_bend = 0.f;
#pragma unroll
    for (int j = 0; j < Raw::FR / 8; ++j) {
      const int f0 = w * Raw::FR + 8 * j;
      float vq[8], vk[8], vkh[8], dq[8], dk[8];
      // base 2: bs[u] is the chunk's inclusive cumulative log2-gate of feature f0 + u
      float bs[8];
      if constexpr (kKeyGate<GATE>) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          float gin;
          if constexpr (SG)
            gin = to_f32(raw.gs);
          else
            gin = to_f32(raw.g[j][u]);
          bs[u] = keep_if(valid, gla_log2_alpha(gin, a.inv_tau));
        }
        wave_inclusive_scan_n(bs);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float xq = WITH_Q ? to_f32(raw.q[WITH_Q ? j : 0][u]) : 0.f;
        const float xk = to_f32(raw.k[j][u]);
        float pq, pk;
        if constexpr (kKeyGate<GATE>) {
          const float b = bs[u];
          // the chunk total is uniform across the wave: a scalar read of lane 63
          const float bend = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, b), 63));
          // Q~ = phi(q) e^{b}, K~ = phi(k) e^{-b} (K^ = e^{b_end} K~ is applied to
          // the state row after the update for GLA); eq = e^{b} phi'(q), ek = e^{-b} phi'(k)
          float eq = 0.f, ek;
          pq = WITH_Q ? phi_times_exp2<FMAP>(xq, b, eq) : 0.f;
          pk = phi_times_exp2<FMAP>(xk, (EXTRA & kPreKPos) != 0 ? b : -b, ek);
          if constexpr ((EXTRA & kPreQD) != 0) dq[u] = eq;
          if constexpr ((EXTRA & kPreKD) != 0) dk[u] = ek;
          // the outer-product gate's state update takes K^ = e^{b_end - b} phi(k) <= 1
          // (with its value side e^{-c} on top, e^{-b} would overflow first)
          if constexpr (GATE == GT_OUTER && (EXTRA & (kPreKPos | kPreNoKH)) == 0) {
            float unused;
            vkh[u] = phi_times_exp2<FMAP>(xk, bend - b, unused);
          }
          my_bend = lane == 8 * j + u ? bend : my_bend;
        } else {
          pq = WITH_Q ? phi_ew<FMAP>(xq) : 0.f;
          pk = phi_ew<FMAP>(xk);
        }
        vq[u] = pq;
        vk[u] = pk;
      }
      const int fo = FT::at(t, f0 / 8);
      if constexpr (WITH_Q) {
        const bf16x8 qr = cat8(pack4(vq[0], vq[1], vq[2], vq[3]), pack4(vq[4], vq[5], vq[6], vq[7]));
        lds<bf16x8>(sm, q_off + fo) = qr;
        if constexpr ((EXTRA & kPreQLo) != 0) lds<bf16x8>(sm, qlo_off + fo) = bf16_residual8(vq, qr);
      }
      // the outer-product gate: pass 3 writes K~ for the scores and K^ for the
      // state, pass 1 K^ only; the backward's reverse state (kPreKPos) the key
      // slot alone
      constexpr bool kh_tile = GATE == GT_OUTER && (EXTRA & (kPreKPos | kPreNoKH)) == 0;
      if constexpr (kh_tile) {
        const bf16x8 khr =
            keep_if(valid, cat8(pack4(vkh[0], vkh[1], vkh[2], vkh[3]), pack4(vkh[4], vkh[5], vkh[6], vkh[7])));
        lds<bf16x8>(sm, (WITH_Q ? kh_off : k_off) + fo) = khr;
      }
      if (!kh_tile || WITH_Q) {
        const bf16x8 kr = cat8(pack4(vk[0], vk[1], vk[2], vk[3]), pack4(vk[4], vk[5], vk[6], vk[7]));
        lds<bf16x8>(sm, k_off + fo) = keep_if(valid, kr);
        if constexpr (WITH_Q && (EXTRA & kPreKLo) != 0)
          lds<bf16x8>(sm, klo_off + fo) = keep_if(valid, bf16_residual8(vk, kr));
      }
      if constexpr (kKeyGate<GATE> && (EXTRA & kPreQD) != 0)
        lds<bf16x8>(sm, qd_off + fo) = cat8(pack4(dq[0], dq[1], dq[2], dq[3]), pack4(dq[4], dq[5], dq[6], dq[7]));
      if constexpr (kKeyGate<GATE> && (EXTRA & kPreKD) != 0)
        lds<bf16x8>(sm, kd_off + fo) = cat8(pack4(dk[0], dk[1], dk[2], dk[3]), pack4(dk[4], dk[5], dk[6], dk[7]));
    }
    if constexpr (kKeyGate<GATE>) {
      if (lane < Raw::FR) {
        lds<float>(sm, gam_off + 4 * (w * Raw::FR + lane)) = __builtin_amdgcn_exp2f(my_bend);
        if constexpr (!WITH_Q || (EXTRA & kPreLogG) != 0)
          lds<float>(sm, logg_off + 4 * (w * Raw::FR + lane)) += my_bend * kLn2;  // natural log for the scan
      }
    }
  }
  // values (rows past the end are zero). The outer-product gate's value side:
  // c, the chunk's inclusive cumulative log-gate per value column (lane =
  // token; scanned in base 2 like the key side), gives V~ = e^{-c} v as a hi + lo bf16 pair (v tile and vl tile:
  // unlike v, V~ is not exact in bf16); WITH_Q also writes e^{c} (the
  // outputs' factor), and every pass e^{c_end} per column (the state's
  // column factor; pass 1 adds c_end to the segment's summed log-gates).
  {
    constexpr int EV = Raw::EV;
    float my_cend = 0.f;
#pragma unroll
    for (int j = 0; j < EV / 8; ++j) {
      if constexpr (GATE == GT_OUTER) {
        float vs[8], ecs[8], cs[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) cs[u] = keep_if(valid, gla_log2_alpha(to_f32(raw.gv[j][u]), a.inv_tau));  // base 2
        wave_inclusive_scan_n(cs);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float c = cs[u];
          const float cend = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c), 63));
          if constexpr ((EXTRA & kPreVRaw) == 0) vs[u] = to_f32(raw.v[j][u]) * __builtin_amdgcn_exp2f(-c);
          ecs[u] = __builtin_amdgcn_exp2f(c);
          my_cend = lane == 8 * j + u ? cend : my_cend;
        }
        if constexpr ((EXTRA & kPreVRaw) != 0) {
          lds<bf16x8>(sm, v_off + VT::at(lane, w * EV / 8 + j)) = keep_if(valid, raw.v[j]);
        } else {
          const bf16x8 hi = cat8(pack4(vs[0], vs[1], vs[2], vs[3]), pack4(vs[4], vs[5], vs[6], vs[7]));
          lds<bf16x8>(sm, v_off + VT::at(lane, w * EV / 8 + j)) = keep_if(valid, hi);
          if constexpr ((EXTRA & kPreVHi) == 0) {
            float lo[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) lo[u] = vs[u] - to_f32(hi[u]);
            lds<bf16x8>(sm, vl_off + VT::at(lane, w * EV / 8 + j)) =
                keep_if(valid, cat8(pack4(lo[0], lo[1], lo[2], lo[3]), pack4(lo[4], lo[5], lo[6], lo[7])));
          }
        }
        if constexpr (WITH_Q) {
          const int eo = ec_off + 4 * (lane * (E + 4) + w * EV + 8 * j);
          lds<f32x4>(sm, eo) = f32x4{ecs[0], ecs[1], ecs[2], ecs[3]};
          lds<f32x4>(sm, eo + 16) = f32x4{ecs[4], ecs[5], ecs[6], ecs[7]};
        }
      } else {
        lds<bf16x8>(sm, v_off + VT::at(lane, w * EV / 8 + j)) = keep_if(valid, raw.v[j]);
      }
    }
    if constexpr (GATE == GT_OUTER) {
      if (lane < EV) {
        lds<float>(sm, gamv_off + 4 * (w * EV + lane)) = __builtin_amdgcn_exp2f(my_cend);
        if constexpr (!WITH_Q) lds<float>(sm, loggv_off + 4 * (w * EV + lane)) += my_cend * kLn2;
      }
    }
  }
}

// The ten lower-triangle 16x16 score tiles (query tile qi, key tile kj <= qi)
// dealt to the four waves as 3, 3, 2, 2 tiles, no wave holding two tiles of
// the same query rows, and slot 0 of wave w on query tile w (whose features
// phi(q) . z also reads):
//   wave 0: (0,0) (3,0) (2,0)   wave 1: (1,0) (3,1) (2,1)
//   wave 2: (2,2) (3,2)         wave 3: (3,3) (1,1)
__device__ __forceinline__ void score_tiles(int w, int (&qi)[3], int (&kj)[3]) {
  qi[0] = w;
  kj[0] = w < 2 ? 0 : w;
  qi[1] = w == 3 ? 1 : 3;
  kj[1] = w == 3 ? 1 : w;
  qi[2] = 2;  // waves 0 and 1 only
  kj[2] = w;
}

// z is carried on the matrix cores as the state column of a constant-1 value:
// z <- Gamma z + K^^T 1. Wave w owns the z tiles rt = w ZT .. w ZT + ZT - 1
// (16 rows each); lane (g, c) holds z[16 rt + 4 g + i] in Z[rt - w ZT][i]
// (the same in every column lane c).
template <int R, int NW = 4>
struct ZTiles {
  static constexpr int ZT = R >= 16 * NW ? R / (16 * NW) : 1;  // tiles per owning wave
  static constexpr int OWNERS = R / (16 * ZT);                 // waves that own z tiles
};

// S (wave slab: rows all R, value columns [w E/NW, (w+1) E/NW)) and this wave's
// z tiles, past one chunk:
//   no gate   S <- S + K~^T V                    z <- z + K~^T 1
//   RetNet    S <- gamma^L S + K^^T V            (kh_off holds K^ rows)
//   GLA       S <- Gamma (S + K~^T V)            Gamma = diag(e^{b_end}) from gam_off
//   outer     S <- (Gamma S + K^^T V~) Gamma_v   Gamma_v = diag(e^{c_end}) from gamv_off,
//             K^ = Gamma K~ (kh_off), V~ as hi + lo (vl_off holds lo)
// Both operands come from [token][column] tiles by transpose reads.
// S is f32x4[R / 16][E / (16 NW)], Z is f32x4[ZTiles<R, NW>::ZT].
// With ZW the z column uses per-token weights (fp32 [64] at zw_off) instead of
// the constant-1 value: z <- Gamma z + K^^T w. With PRE the GLA gate scales
// the old state only (S <- Gamma S + K~^T V), as the backward pass's reverse
// state needs; the outer-product gate with PRE likewise scales the old state
// by both sides and adds one bf16 value tile: S <- (Gamma 1^T) * S * (1 Gamma_v^T) + K~^T V.
// With KLO the key rows also have a bf16 residual tile at klo_off, added as a
// second product (the keys as a hi + lo pair).
template <int R, int E, int GATE, int NW, bool SWZ, bool ZW = false, bool PRE = false, bool KLO = false, class SArr,
          class ZArr>
__device__ __forceinline__ void state_update(SArr& S, ZArr& Z, char* sm, int kh_off, int v_off, int gam_off,
                                             float gscale, int lane, int w, int zw_off = 0, int gamv_off = 0,
                                             int vl_off = 0, int klo_off = 0) {
  constexpr int ZT = ZTiles<R, NW>::ZT, NEB = E / (16 * NW);
  const int g4 = lane >> 4;
  const int ebase = w * (E / NW);
  bf16x8 ones;
#pragma unroll
  for (int u = 0; u < 8; ++u) ones[u] = (bf16)1.f;
  bf16x8 vb[NEB][2];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) vb[eb][ks] = tr_feat<E, SWZ>(sm, v_off, 32 * ks, ebase + 16 * eb, lane);
  constexpr bool VLO = GATE == GT_OUTER && !PRE;
  bf16x8 vbl[VLO ? NEB : 1][2];  // the outer-product gate: lo half of V~
  if constexpr (VLO) {
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) vbl[eb][ks] = tr_feat<E, SWZ>(sm, vl_off, 32 * ks, ebase + 16 * eb, lane);
  }
#pragma unroll
  for (int rt = 0; rt < R / 16; ++rt) {
    bf16x8 ka[2], kal[KLO ? 2 : 1];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) ka[ks] = tr_feat<R, SWZ>(sm, kh_off, 32 * ks, 16 * rt, lane);
    if constexpr (KLO) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) kal[ks] = tr_feat<R, SWZ>(sm, klo_off, 32 * ks, 16 * rt, lane);
    }
    float gr[4] = {gscale, gscale, gscale, gscale};
    if constexpr (kKeyGate<GATE>) {
#pragma unroll
      for (int i = 0; i < 4; ++i) gr[i] = lds<float>(sm, gam_off + 4 * (16 * rt + 4 * g4 + i));
    }
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) {
      f32x4 st = S[rt][eb];
      if constexpr (GATE == GT_OUTER && PRE) {
        const float gc = lds<float>(sm, gamv_off + 4 * (ebase + 16 * eb + (lane & 15)));
#pragma unroll
        for (int i = 0; i < 4; ++i) st[i] *= gr[i] * gc;
      } else if constexpr (kScalarDecay<GATE> || (kKeyGate<GATE> && PRE) || GATE == GT_OUTER) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st[i] *= gr[i];
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) st = mfma16(ka[ks], vb[eb][ks], st);
      if constexpr (KLO) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) st = mfma16(kal[ks], vb[eb][ks], st);
      }
      if constexpr (VLO) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) st = mfma16(ka[ks], vbl[eb][ks], st);
        // the column's value-side factor
        const float gc = lds<float>(sm, gamv_off + 4 * (ebase + 16 * eb + (lane & 15)));
#pragma unroll
        for (int i = 0; i < 4; ++i) st[i] *= gc;
      } else if constexpr (kKeyGate<GATE> && !PRE) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st[i] *= gr[i];
      }
      S[rt][eb] = st;
    }
  }
  // this wave's z tiles, outside the tile loop so no branch on the wave index splits it
  if (w < ZTiles<R, NW>::OWNERS) {
#pragma unroll
    for (int j = 0; j < ZT; ++j) {
      const int rt = w * ZT + j;
      f32x4 zt = Z[j];
      float gr[4] = {gscale, gscale, gscale, gscale};
      if constexpr (kKeyGate<GATE>) {
#pragma unroll
        for (int i = 0; i < 4; ++i) gr[i] = lds<float>(sm, gam_off + 4 * (16 * rt + 4 * g4 + i));
      }
      if constexpr (kScalarDecay<GATE> || (kKeyGate<GATE> && PRE) || GATE == GT_OUTER) {
#pragma unroll
        for (int i = 0; i < 4; ++i) zt[i] *= gr[i];
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 zb = ones;
        if constexpr (ZW) {
          // k-slot jj of lane group g is token 32 ks + 8 g + jj (see tr_feat)
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) zb[jj] = (bf16)lds<float>(sm, zw_off + 4 * (32 * ks + 8 * g4 + jj));
        }
        zt = mfma16(tr_feat<R, SWZ>(sm, kh_off, 32 * ks, 16 * rt, lane), zb, zt);
        if constexpr (KLO) zt = mfma16(tr_feat<R, SWZ>(sm, klo_off, 32 * ks, 16 * rt, lane), zb, zt);
      }
      if constexpr (GATE == GT_GLA && !PRE) {  // z takes the key side only
#pragma unroll
        for (int i = 0; i < 4; ++i) zt[i] *= gr[i];
      }
      Z[j] = zt;
    }
  }
}

// z tiles of wave w to / from a flat [R] fp32 array (lanes with c == 0 write).
template <int R, int NW, class ZArr>
__device__ __forceinline__ void z_store(const ZArr& Z, float* dst, int lane, int w) {
  constexpr int ZT = ZTiles<R, NW>::ZT;
  if (w < ZTiles<R, NW>::OWNERS && (lane & 15) == 0) {
#pragma unroll
    for (int j = 0; j < ZT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[16 * (w * ZT + j) + 4 * (lane >> 4) + i] = Z[j][i];
  }
}

template <int R, int NW, class ZArr>
__device__ __forceinline__ void z_load(ZArr& Z, const float* src, int lane, int w) {
  constexpr int ZT = ZTiles<R, NW>::ZT;
#pragma unroll
  for (int j = 0; j < ZT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      Z[j][i] = (src != nullptr && w < ZTiles<R, NW>::OWNERS) ? src[16 * (w * ZT + j) + 4 * (lane >> 4) + i] : 0.f;
}

// ---------------------------------------------------------------------------
// Pass 1: each segment's own state contribution (segments 0 .. P-2).
// ---------------------------------------------------------------------------
template <int R, int E, int DK, int FMAP, int GATE>
__global__ __launch_bounds__((64 * Waves<R, E>::NW)) void causal_segment_state(CausalArgs a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  using LY = SegLayout<R, E, GATE>;
  constexpr int NW = Waves<R, E>::NW, NEB = E / (16 * NW);
  const int lane = lane_id(), w = wave_id<NW>(), tid = threadIdx.x;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int s = blockIdx.x;
  const long long bh = blockIdx.y;
  const int h = int(bh % a.H);
  const SeqView sv = seq_view(a, bh);
  const int t_begin = s * a.seg_len;
  // only segments that a later segment of the same sequence follows
  if (t_begin + a.seg_len >= sv.len) return;
  const int t_end = min(sv.len, t_begin + a.seg_len);
  const long long tok0 = sv.tok0;
  const int ebase = w * (E / NW);
  float lg2gam = 0.f;
  if constexpr (GATE == GT_DECAY) lg2gam = log2f(a.gamma[h]);

  f32x4 S[R / 16][NEB];
#pragma unroll
  for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) S[rt][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 Z[ZTiles<R, NW>::ZT];
  z_load<R, NW>(Z, nullptr, lane, w);
  if (tid < R) lds<float>(sm, LY::logg_off + 4 * tid) = 0.f;
  if constexpr (GATE == GT_OUTER) {
    if (tid < E) lds<float>(sm, LY::loggv_off + 4 * tid) = 0.f;
  }
  lds_barrier();

  // Two chunks of loads in flight: raw buffer b holds chunks of parity b;
  // after a prelude consumes one it is refilled with the chunk two ahead.
  // Refills are unconditional (past the segment they re-read its last row), so
  // every path into a prelude has the same loads outstanding and the wait
  // before it covers only that buffer.
  using Raw = RawChunk<R, E, DK, FMAP, GATE, false, NW>;
  const int nch = (t_end - t_begin + kChunk - 1) / kChunk;
  Raw raw[2];
  raw[0].load(a, tok0, t_begin, t_end, lane, w);
  __builtin_amdgcn_sched_barrier(0);  // keep the issue order: lower buffers complete first
  raw[1].load(a, tok0, t_begin + kChunk, t_end, lane, w);
  __builtin_amdgcn_sched_barrier(0);
  auto prelude = [&](Raw& rw, int ci, int half) {
    const int L = min(kChunk, sv.len - (t_begin + ci * kChunk));
    chunk_prelude<R, E, DK, FMAP, GATE, false, NW, LY::SWZ>(rw, a, L, lg2gam, sm, 0, half * LY::HALF + LY::k_off, 0,
                                                   half * LY::HALF + LY::v_off, half * LY::HALF + LY::gam_off,
                                                   LY::logg_off, lane, w, 0, 0, LY::bs_off, 0,
                                                   half * LY::HALF + LY::gamv_off, LY::loggv_off,
                                                   half * LY::HALF + LY::vl_off);
  };
  auto update = [&](int ci, int half) {
    const int L = min(kChunk, sv.len - (t_begin + ci * kChunk));
    float gsc = GATE == GT_DECAY ? exp2f(float(L) * lg2gam) : 1.f;
    if constexpr (GATE == GT_SEL) gsc = __expf(lds<float>(sm, LY::bs_off + 4 * 63));
    state_update<R, E, GATE, NW, LY::SWZ>(S, Z, sm, half * LY::HALF + LY::k_off, half * LY::HALF + LY::v_off,
                                 half * LY::HALF + LY::gam_off, gsc, lane, w, 0, half * LY::HALF + LY::gamv_off,
                                 half * LY::HALF + LY::vl_off);
  };
  if constexpr (LY::PIPELINED) {
    // while the state update of chunk ci reads half ci & 1, the prelude of
    // chunk ci + 1 writes the other half: one barrier per chunk, and the
    // prelude's VALU work can overlap the update's matrix-core work
    prelude(raw[0], 0, 0);
    raw[0].load(a, tok0, t_begin + 2 * kChunk, t_end, lane, w);
    lds_barrier();
    auto step = [&](Raw& rnext, int ci, int half) {
      if (ci + 1 < nch) prelude(rnext, ci + 1, half ^ 1);
      rnext.load(a, tok0, t_begin + (ci + 3) * kChunk, t_end, lane, w);
      update(ci, half);
      lds_barrier();
    };
    for (int ci = 0; ci < nch; ci += 2) {
      step(raw[1], ci, 0);
      if (ci + 1 < nch) step(raw[0], ci + 1, 1);
    }
  } else {
    // a step past the last chunk does nothing but its refill
    auto step = [&](Raw& rw, int ci) {
      const bool live = ci < nch;
      if (live) prelude(rw, ci, 0);
      rw.load(a, tok0, t_begin + (ci + 2) * kChunk, t_end, lane, w);
      if (live) {
        lds_barrier();
        update(ci, 0);
        lds_barrier();
      }
    };
    for (int ci = 0; ci < nch; ci += 2) {
      step(raw[0], ci);
      step(raw[1], ci + 1);
    }
  }
  const long long slot = bh * a.P + s;
  float* So = a.S_out + slot * R * E;
#pragma unroll
  for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i) So[(16 * rt + 4 * g4 + i) * E + ebase + 16 * eb + c16] = S[rt][eb][i];
  z_store<R, NW>(Z, a.z_out + slot * R, lane, w);
  if constexpr (kKeyGate<GATE> || GATE == GT_SEL) {
    if (tid < R) a.logG_out[slot * R + tid] = lds<float>(sm, LY::logg_off + 4 * tid);
  }
  if constexpr (GATE == GT_OUTER) {
    if (tid < E) a.logGv_out[slot * E + tid] = lds<float>(sm, LY::loggv_off + 4 * tid);
  }
}

// ---------------------------------------------------------------------------
// Pass 1 for the GLA gate, feature-major ("Gating and Selective State
// Updates": S_t = diag(alpha_t) S_{t-1} + phi(k_t) v_t^T). Per chunk the
// segment's state takes S <- diag(Gamma) S + K^T V with
// K^_t = e^{b_end - b_t} phi(k_t) (b the chunk's inclusive cumulative
// log-gate, Gamma = e^{b_end}; every factor <= 1), and z likewise.
//
// The feature rows of the state are independent under this gate, so each
// segment is split over R / 64 workgroups of 64 features (four waves, one
// 16-feature tile each, every value column). The chunk's k and g columns of
// the block and its v rows are staged in LDS as they load (coalesced); each
// lane then reads its feature's column for eight consecutive tokens per
// 32-token block by transpose reads, which is also the A-operand layout of
// the state update (contraction over tokens). So the cumulative log-gate is a
// running sum inside the lane plus a two-step prefix over the four lane
// groups, and K^ goes from registers to the matrix cores without an LDS round
// trip; z is the state column of a constant-1 value. LDS holds two chunks
// (one barrier per chunk).
// ---------------------------------------------------------------------------
constexpr int kGlaSegFeatures = 64;  // features per workgroup of the feature-major pass

template <int E>
struct GlaSegLayout {
  using FTR = FeatTile<kGlaSegFeatures, false>;
  using FTE = FeatTile<E, false>;
  static constexpr int k_off = 0;
  static constexpr int g_off = k_off + FTR::BYTES;
  static constexpr int v_off = g_off + FTR::BYTES;
  static constexpr int HALF = v_off + FTE::BYTES;
  static constexpr int bytes = 2 * HALF;
};

// Built for the GLA gate with 64 or 128 features.
template <int R, int GATE>
constexpr bool kGlaFeatureMajorSeg = GATE == GT_GLA && R % kGlaSegFeatures == 0;

// KLO (the backward's state recompute): K^ enters the state as a hi + lo pair.
template <int R, int E, int DK, int FMAP, bool SG = false, bool KLO = false>
__global__ __launch_bounds__(256) void gla_segment_state(CausalArgs a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  using LY = GlaSegLayout<E>;
  constexpr int FB = kGlaSegFeatures, NFB = R / FB, ET = E / 16;
  constexpr int VR = FB / 8, VE = E / 8;              // 16-byte pieces per row of the k (g) block and of v
  constexpr int PK = 64 * VR / 256, PV = 64 * VE / 256;  // pieces per thread
  using FTR = typename LY::FTR;
  using FTE = typename LY::FTE;
  const int lane = lane_id(), w = wave_id<4>(), tid = threadIdx.x;
  const int g4 = lane >> 4, c16 = lane & 15;
  // 1D grid: workgroup i runs on XCD i % 8, so the feature blocks of one
  // (head, segment), which read the same value rows, take ids 8 apart (same
  // XCD and L2, dispatched back to back)
  const int nseg = a.P - 1;
  const int grp = blockIdx.x / (8 * NFB), r8 = blockIdx.x % (8 * NFB);
  const int fb = r8 / 8;
  const long long idx = 8ll * grp + r8 % 8;
  if (idx >= (long long)nseg * a.nbh) return;
  const int s = int(idx % nseg);
  const long long bh = idx / nseg;
  const SeqView sv = seq_view(a, bh);
  const int t_begin = s * a.seg_len;
  if (t_begin + a.seg_len >= sv.len) return;  // only segments that a later one follows
  const int t_end = min(sv.len, t_begin + a.seg_len);
  const long long tok0 = sv.tok0;
  const long long ldv = a.ldv > 0 ? a.ldv : E;
  const int nch = (t_end - t_begin + kChunk - 1) / kChunk;
  const int f_lane = FB * fb + 16 * w + c16;  // this lane's feature

  f32x4 S[ET], Z = {0.f, 0.f, 0.f, 0.f};  // state rows 16 w + 4 g4 + i of the block; z of the same rows
#pragma unroll
  for (int eb = 0; eb < ET; ++eb) S[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lg = 0.f;  // summed log2-gates of feature f_lane
  bf16x8 ones;
#pragma unroll
  for (int u = 0; u < 8; ++u) ones[u] = (bf16)1.f;

  // raw rows of one chunk in registers: piece i of thread tid is piece
  // tid + 256 i of the block's tile in row-major order (rows clamped to the segment)
  bf16x8 rk[PK], rg[PK], rv[PV];
  bf16 rgs[SG ? PK : 1];  // SG: the piece's token's one gate input
  auto load = [&](int ci) {
    const int t0 = t_begin + ci * kChunk;
#pragma unroll
    for (int i = 0; i < PK; ++i) {
      const int pc = tid + 256 * i;
      const long long rowi = tok0 + min(t0 + pc / VR, t_end - 1);
      const long long at = rowi * R + FB * fb + 8 * (pc % VR);
      rk[i] = *reinterpret_cast<const bf16x8*>(a.K + at);
      if constexpr (SG)
        rgs[i] = a.g[rowi];
      else
        rg[i] = *reinterpret_cast<const bf16x8*>(a.g + at);
    }
#pragma unroll
    for (int i = 0; i < PV; ++i) {
      const int pc = tid + 256 * i;
      const long long row = tok0 + min(t0 + pc / VE, t_end - 1);
      rv[i] = *reinterpret_cast<const bf16x8*>(a.V + row * ldv + 8 * (pc % VE));
    }
  };
  auto stage = [&](int half) {
    char* base = sm + half * LY::HALF;
#pragma unroll
    for (int i = 0; i < PK; ++i) {
      const int pc = tid + 256 * i;
      lds<bf16x8>(base, LY::k_off + FTR::at(pc / VR, pc % VR)) = rk[i];
      bf16x8 gp;
      if constexpr (SG) {
#pragma unroll
        for (int u = 0; u < 8; ++u) gp[u] = rgs[i];
      } else {
        gp = rg[i];
      }
      lds<bf16x8>(base, LY::g_off + FTR::at(pc / VR, pc % VR)) = gp;
    }
#pragma unroll
    for (int i = 0; i < PV; ++i) {
      const int pc = tid + 256 * i;
      lds<bf16x8>(base, LY::v_off + FTE::at(pc / VE, pc % VE)) = rv[i];
    }
  };

  load(0);
  stage(0);
  load(1);
  lds_barrier();
  for (int ci = 0; ci < nch; ++ci) {
    const int half = ci & 1;
    if (ci + 1 < nch) stage(half ^ 1);
    load(ci + 2);  // unconditional: past the segment it re-reads its last row
    const int L = min(kChunk, sv.len - (t_begin + ci * kChunk));
    char* base = sm + half * LY::HALF;
    // MASKED: a chunk shorter than 64 tokens (the sequence's last); rows past
    // L get a zero log-gate and a zero key
    auto chunk = [&](auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
      // lane (c16, g4): feature f_lane, tokens 32 ks + 8 g4 + j
      float b[2][8];
      bf16x8 kk[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 gg = tr_feat<FB, false>(base, LY::g_off, 32 * ks, 16 * w, lane);
        kk[ks] = tr_feat<FB, false>(base, LY::k_off, 32 * ks, 16 * w, lane);
        float run = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float la = gla_log2_alpha(to_f32(gg[j]), a.inv_tau);
          run += MASKED ? keep_if(32 * ks + 8 * g4 + j < L, la) : la;
          b[ks][j] = run;
        }
      }
      // prefix of the lane totals over the four lane groups, both blocks at once
      float inc0 = b[0][7], inc1 = b[1][7];
      {
        const float u0 = __shfl_up(inc0, 16), u1 = __shfl_up(inc1, 16);
        inc0 += g4 >= 1 ? u0 : 0.f;
        inc1 += g4 >= 1 ? u1 : 0.f;
        const float v0 = __shfl_up(inc0, 32), v1 = __shfl_up(inc1, 32);
        inc0 += g4 >= 2 ? v0 : 0.f;
        inc1 += g4 >= 2 ? v1 : 0.f;
      }
      const float tot0 = __shfl(inc0, 48 + c16), tot1 = __shfl(inc1, 48 + c16);
      const float bend = tot0 + tot1;
      // exponent of K^ for token (ks, j): bend - (b[ks][j] + offset of the lane's run)
      const float r0 = bend - (inc0 - b[0][7]), r1 = bend - (tot0 + inc1 - b[1][7]);
      bf16x8 kh[2], kl[KLO ? 2 : 1];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float unused;
          e[j] = phi_times_exp2<FMAP>(to_f32(kk[ks][j]), (ks == 0 ? r0 : r1) - b[ks][j], unused);
          if constexpr (MASKED) e[j] = keep_if(32 * ks + 8 * g4 + j < L, e[j]);
        }
        kh[ks] = cat8(pack4(e[0], e[1], e[2], e[3]), pack4(e[4], e[5], e[6], e[7]));
        if constexpr (KLO) kl[ks] = bf16_residual8(e, kh[ks]);
      }
      const float gam = __builtin_amdgcn_exp2f(bend);
      lg += bend;
      float gr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) gr[i] = __shfl(gam, 4 * g4 + i);  // Gamma of state row 16 w + 4 g4 + i
#pragma unroll
      for (int eb = 0; eb < ET; ++eb) {
        f32x4 st = S[eb];
#pragma unroll
        for (int i = 0; i < 4; ++i) st[i] *= gr[i];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 vt = tr_feat<E, false>(base, LY::v_off, 32 * ks, 16 * eb, lane);
          st = mfma16(kh[ks], vt, st);
          if constexpr (KLO) st = mfma16(kl[ks], vt, st);
        }
        S[eb] = st;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Z[i] *= gr[i];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        Z = mfma16(kh[ks], ones, Z);
        if constexpr (KLO) Z = mfma16(kl[ks], ones, Z);
      }
    };
    if (L == kChunk)
      chunk(std::false_type{});
    else
      chunk(std::true_type{});
    lds_barrier();
  }
  const long long slot = bh * a.P + s;
  const int row0 = FB * fb + 16 * w + 4 * g4;
  float* So = a.S_out + slot * R * E;
#pragma unroll
  for (int eb = 0; eb < ET; ++eb)
#pragma unroll
    for (int i = 0; i < 4; ++i) So[(row0 + i) * E + 16 * eb + c16] = S[eb][i];
  if (c16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a.z_out[slot * R + row0 + i] = Z[i];
  }
  if (g4 == 0) a.logG_out[slot * R + f_lane] = lg * kLn2;  // natural log for the scan
}

// Pass 1 launch: the feature-major GLA pass where it is built, else causal_segment_state.
// SG: one gate input per token (the selective gate's backward on the GLA passes).
template <int R, int E, int DK, int FMAP, int GATE, bool SG = false, bool KLO = false>
la_status launch_segment_pass(const CausalArgs& a1, int P, unsigned BH, hipStream_t stream) {
  static_assert(!SG || kGlaFeatureMajorSeg<R, GATE>, "one gate input per token: the GLA passes only");
  if constexpr (kGlaFeatureMajorSeg<R, GATE> && FMAP != FM_FAVOR) {
    auto k1 = gla_segment_state<R, E, DK, FMAP, SG, KLO>;
    constexpr int lds1 = GlaSegLayout<E>::bytes;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(k1), hipFuncAttributeMaxDynamicSharedMemorySize, lds1) !=
        hipSuccess)
      return LA_ERR_HIP;
    CausalArgs a2 = a1;
    a2.nbh = int(BH);
    const unsigned groups = (unsigned(P - 1) * BH + 7) / 8;
    LA_LAUNCH(k1, dim3(groups * 8 * (R / kGlaSegFeatures)), dim3(256), lds1, stream, a2);
  } else {
    auto k1 = causal_segment_state<R, E, DK, FMAP, GATE>;
    constexpr int lds1 = SegLayout<R, E, GATE>::bytes;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(k1), hipFuncAttributeMaxDynamicSharedMemorySize, lds1) !=
        hipSuccess)
      return LA_ERR_HIP;
    LA_LAUNCH(k1, dim3(P - 1, BH), dim3(64 * Waves<R, E>::NW), lds1, stream, a1);
  }
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Pass 3: outputs of one segment, starting from its chained state.
// ---------------------------------------------------------------------------
template <int R, int E, int DK, int FMAP, int GATE>
__global__ __launch_bounds__((64 * Waves<R, E>::NW)) void causal_chunk_forward(CausalArgs a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  using LY = FwdLayout<R, E, GATE>;
  constexpr int NW = Waves<R, E>::NW;
  constexpr int NEB = E / (16 * NW), KP = R / 32;
  using FT = FeatTile<R, LY::SWZ>;
  using AT = FeatTile<kChunk, LY::SWZ>;
  const int lane = lane_id(), w = wave_id<NW>(), tid = threadIdx.x;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int s = blockIdx.x;
  const long long bh = blockIdx.y;
  const int h = int(bh % a.H);
  const SeqView sv = seq_view(a, bh);
  const int t_begin = s * a.seg_len;
  if (s > 0 && t_begin >= sv.len) return;  // past the end of this sequence
  const int t_end = min(sv.len, t_begin + a.seg_len);
  const long long tok0 = sv.tok0;
  const int ebase = w * (E / NW);
  float lg2gam = 0.f;
  if constexpr (GATE == GT_DECAY) lg2gam = log2f(a.gamma[h]);

  // ---- state carried in
  f32x4 S[R / 16][NEB];
  f32x4 Z[ZTiles<R, NW>::ZT];
  const long long in_idx = a.in_is_state ? sv.st : bh;
  const bool has_in = a.S_in != nullptr && in_idx >= 0;
  if (has_in) {
    const float* Sp = a.S_in + in_idx * a.in_head + s * a.in_seg;
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
  z_load<R, NW>(Z, has_in ? a.z_in + (in_idx * a.in_head + s * a.in_seg) / E : nullptr, lane, w);
  z_store<R, NW>(Z, reinterpret_cast<float*>(sm + LY::z_off), lane, w);
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

  // Loads run DEPTH chunks ahead (two buffers when the registers allow),
  // refilled unconditionally as in pass 1.
  using Raw = RawChunk<R, E, DK, FMAP, GATE, true, NW>;
  constexpr int DEPTH = 1;
  const int nch = (t_end - t_begin + kChunk - 1) / kChunk;
  Raw raw0, raw1;
  if (sv.len > 0) raw0.load(a, tok0, t_begin, t_end, lane, w);  // an empty sequence reads nothing
  __builtin_amdgcn_sched_barrier(0);  // keep the issue order: buffer 0's loads complete first
  if constexpr (DEPTH == 2) raw1.load(a, tok0, t_begin + kChunk, t_end, lane, w);
  auto step = [&](Raw& raw, int ci) {
    const int t0 = t_begin + ci * kChunk;
    const bool live = ci < nch;
    const int L = min(kChunk, sv.len - t0);
    if (live)
      chunk_prelude<R, E, DK, FMAP, GATE, true, NW, LY::SWZ>(raw, a, L, lg2gam, sm, LY::q_off, LY::k_off, LY::kh_off,
                                                    LY::v_off, LY::gam_off, 0, lane, w, 0, 0, LY::bs_off,
                                                    LY::ec_off, LY::gamv_off, 0, LY::vl_off);
    // the raw registers are free again: this refill flies during the next DEPTH chunks
    raw.load(a, tok0, t0 + DEPTH * kChunk, t_end, lane, w);
    if (!live) return;
    lds_barrier();

    // ---- scores for query rows [16 qw, 16 qw + 16): A^T tiles = K~_c Q~_qw^T
    // (waves 0..3), and Q^ . z_prev for the same rows (with 8 waves, by waves 4..7)
    {
      const int qw = w & 3;
      const bool scores = NW == 4 || w < 4, zdot = NW == 4 || w >= 4;
      bf16x8 qop[KP];
#pragma unroll
      for (int ks = 0; ks < KP; ++ks) qop[ks] = lds<bf16x8>(sm, LY::q_off + FT::at(16 * qw + c16, 4 * ks + g4));
      const int q = 16 * qw + c16;
      if (scores) {
        float rs = 0.f;
        for (int c = 0; c <= qw; ++c) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KP; ++ks)
            acc = mfma16(lds<bf16x8>(sm, LY::k_off + FT::at(16 * c + c16, 4 * ks + g4)), qop[ks], acc);
          // acc[i] = A[q][key], key = 16c + 4g + i
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = 16 * c + 4 * g4 + i;
            v[i] = acc[i];
            // RetNet: gamma^(q - key) <= 1 is formed only where key <= q, and
            // the mask is a select, so no factor above the diagonal (gamma^-15
            // there overflows for a small gamma) meets a product
            if constexpr (GATE == GT_DECAY) v[i] *= exp2f(float(max(q - key, 0)) * lg2gam);
            if (c == qw && key > q) v[i] = 0.f;  // only the diagonal tile straddles the mask
            if constexpr (GATE == GT_SEL) {
              // e^{b_q - b_key} <= 1 below the diagonal; a select (not a
              // product) above it, where the factor may overflow
              const float f = __expf(lds<float>(sm, LY::bs_off + 4 * q) - lds<float>(sm, LY::bs_off + 4 * key));
              v[i] = key <= q ? v[i] * f : 0.f;
            }
          }
          // bf16 scores, and the row sum of exactly those rounded values
          const unsigned p01 = pack2_bits(v[0], v[1]), p23 = pack2_bits(v[2], v[3]);
          rs += (lo_bf16_f32(p01) + hi_bf16_f32(p01)) + (lo_bf16_f32(p23) + hi_bf16_f32(p23));
          typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
          lds<u32x2>(sm, LY::a_off + AT::at(q, 2 * c + (g4 >> 1), 8 * (g4 & 1))) = u32x2{p01, p23};
        }
        if ((qw & 1) == 0) lds<bf16x4>(sm, LY::a_off + AT::at(q, 2 * (qw + 1) + (g4 >> 1), 8 * (g4 & 1))) = bf16x4{};
        rs = sum_over_groups(rs);
        if (g4 == 0) lds<float>(sm, LY::rs_off + 4 * q) = rs;
      }
      if (zdot) {
        float zd = 0.f;
#pragma unroll
        for (int ks = 0; ks < KP; ++ks)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            zd += to_f32(qop[ks][j]) * lds<float>(sm, LY::z_off + 4 * (32 * ks + 8 * g4 + j));
        zd = sum_over_groups(zd);
        if constexpr (GATE == GT_DECAY) zd *= exp2f(float(q + 1) * lg2gam);
        if constexpr (GATE == GT_SEL) zd *= __expf(lds<float>(sm, LY::bs_off + 4 * q));
        if (g4 == 0) lds<float>(sm, LY::zd_off + 4 * q) = zd;
      }
    }
    lds_barrier();

    // ---- outputs for value columns [w E/NW, (w+1) E/NW): O^T = S^T Q^^T + V^T A^T
    rebuild_sop();  // built here so it is not live across the prelude and the scores
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const int q = 16 * qt + c16;
      bf16x8 qb[KP];
#pragma unroll
      for (int p = 0; p < KP; ++p)
        qb[p] = cat8(lds<bf16x4>(sm, LY::q_off + FT::at(q, 4 * p + (g4 >> 1), 8 * (g4 & 1))),
                     lds<bf16x4>(sm, LY::q_off + FT::at(q, 4 * p + 2 + (g4 >> 1), 8 * (g4 & 1))));
      // one correctly rounded reciprocal per row; outputs are fl(O * fl(1 / den));
      // the state-space read-out is the numerator itself
      float inv_den = 1.f;
      if constexpr (FMAP != FM_IDENT)
        inv_den = 1.f / (lds<float>(sm, LY::rs_off + 4 * q) + lds<float>(sm, LY::zd_off + 4 * q) + a.eps);
      float isc = 1.f;
      if constexpr (GATE == GT_DECAY) isc = exp2f(float(q + 1) * lg2gam);
      if constexpr (GATE == GT_SEL) isc = __expf(lds<float>(sm, LY::bs_off + 4 * q));
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) {
        const int e = ebase + 16 * eb;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < KP; ++p) acc = mfma16(Sop[p][eb], qb[p], acc);
        if constexpr (kScalarDecay<GATE>) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] *= isc;
        }
#pragma unroll
        for (int p2 = 0; p2 <= qt / 2; ++p2) {
          const bf16x8 ab = lds<bf16x8>(sm, LY::a_off + AT::at(q, 4 * p2 + g4));
          acc = mfma16(tr_feat<E, LY::SWZ>(sm, LY::v_off, 32 * p2, e, lane), ab, acc);
          if constexpr (GATE == GT_OUTER) acc = mfma16(tr_feat<E, LY::SWZ>(sm, LY::vl_off, 32 * p2, e, lane), ab, acc);
        }
        if constexpr (GATE == GT_OUTER) {
          // both parts carry e^{-c} of the chunk start on the value side
          const f32x4 ec = lds<f32x4>(sm, LY::ec_off + 4 * (q * (E + 4) + e + 4 * g4));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] *= ec[i];
        }
        if (q < L) {
          bf16x4 o = pack4(acc[0] * inv_den, acc[1] * inv_den, acc[2] * inv_den, acc[3] * inv_den);
          *reinterpret_cast<bf16x4*>(a.out + (tok0 + t0 + q) * E + e + 4 * g4) = o;
        }
      }
    }

    // ---- carry the state past this chunk
    float gsc = GATE == GT_DECAY ? exp2f(float(L) * lg2gam) : 1.f;
    if constexpr (GATE == GT_SEL) gsc = __expf(lds<float>(sm, LY::bs_off + 4 * 63));
    state_update<R, E, GATE, NW, LY::SWZ>(S, Z, sm, kScalarDecay<GATE> || GATE == GT_OUTER ? LY::kh_off : LY::k_off,
                                 LY::v_off, LY::gam_off,
                                 gsc, lane, w, 0, LY::gamv_off, LY::vl_off);
    z_store<R, NW>(Z, reinterpret_cast<float*>(sm + LY::z_off), lane, w);  // old z no longer read this chunk
    lds_barrier();
  };
  if constexpr (DEPTH == 2) {
    for (int ci = 0; ci < nch; ci += 2) {
      step(raw0, ci);
      step(raw1, ci + 1);
    }
  } else {
    for (int ci = 0; ci < nch; ++ci) step(raw0, ci);
  }

  // the sequence's last segment stores its final state
  if (a.S_out != nullptr && sv.st >= 0 && s == (sv.len > 0 ? (sv.len - 1) / a.seg_len : 0)) {
    float* So = a.S_out + sv.st * R * E;
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int i = 0; i < 4; ++i) So[(16 * rt + 4 * g4 + i) * E + ebase + 16 * eb + c16] = S[rt][eb][i];
    z_store<R, NW>(Z, a.z_out + sv.st * R, lane, w);
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
  a.gv = static_cast<const bf16*>(p.gv);
  a.omega = static_cast<const bf16*>(p.omega);
  a.gamma = p.gamma;
  a.out = static_cast<bf16*>(p.out);
  a.cu = p.cu;
  a.slot = p.slot;
  a.nslot = p.nslot;
  a.H = p.H;
  a.n = p.n;
  a.P = p.P;
  a.seg_len = p.seg_len;
  a.eps = p.eps;
  a.inv_tau = (kKeyGate<GATE> || GATE == GT_SEL) ? 1.f / p.tau : 0.f;
  const unsigned BH = unsigned(p.nseq) * unsigned(p.H);

  if (p.P > 1) {
    CausalArgs a1 = a;
    a1.S_out = p.ws_S;
    a1.z_out = p.ws_z;
    a1.logG_out = p.ws_logG;
    a1.logGv_out = p.ws_logGv;
    la_status st = launch_segment_pass<R, E, DK, FMAP, GATE>(a1, p.P, BH, p.stream);
    if (st != LA_OK) return st;
    st = launch_segment_scan(p);
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
    a.in_is_state = 1;
  }
  a.S_out = p.S_final;
  a.z_out = p.z_final;
  auto k3 = causal_chunk_forward<R, E, DK, FMAP, GATE>;
  constexpr int lds3 = FwdLayout<R, E, GATE>::bytes;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k3), hipFuncAttributeMaxDynamicSharedMemorySize, lds3) !=
      hipSuccess)
    return LA_ERR_HIP;
  LA_LAUNCH(k3, dim3(p.P, BH), dim3(64 * Waves<R, E>::NW), lds3, p.stream, a);
  if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
  return LA_OK;
}

}  // namespace la
