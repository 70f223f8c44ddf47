// Chunkwise causal kernels for FAVOR+ features ("Choosing the Feature Map
// phi", "Linear Attention Mechanisms" (dileepadev.github.io): positive random
// features phi(x)_m = exp(w_m . x - |x|^2/2) / sqrt(r)).
//
// Same chunk algebra as the elu+1 kernels in chunked.hpp, with two changes
// forced by the features being exponentials with a wide dynamic range:
//   * every bf16 operand that carries a feature or the state is a hi + lo pair
//     (x = hi + lo, hi = bf16(x), lo = bf16(x - hi)), and products take the
//     three significant terms hi*hi + lo*hi + hi*lo, so scores, inter-chunk
//     reads and state updates keep ~16 significant bits on the matrix cores;
//   * the feature axis is processed in blocks of up to 128 features, so the
//     hi/lo tiles of one block fit in LDS; everything that contracts over the
//     features accumulates across blocks in registers.
// The projection X w^T runs on the matrix cores (exact bf16 products, fp32
// accumulation); |x|^2/2 and ln(r)/2 are subtracted before the exponential.
#pragma once

#include "chunked.hpp"

namespace la {

template <int R>
struct FavorBlock {
  static constexpr int FB = R < 128 ? R : 128;  // features per block
  static constexpr int NFB = R / FB;            // blocks
  static constexpr int RPB = FB + 8;            // row stride of [t][feature] tiles
  static constexpr int MT = FB / 64;            // 16-feature tiles per wave per block
};

template <int R, int E>
struct FavorFwdLayout {
  using F = FavorBlock<R>;
  static constexpr int qh_off = 0;
  static constexpr int ql_off = qh_off + kChunk * F::RPB * 2;
  static constexpr int kh_off = ql_off + kChunk * F::RPB * 2;
  static constexpr int kl_off = kh_off + kChunk * F::RPB * 2;
  static constexpr int kth_off = kl_off + kChunk * F::RPB * 2;
  static constexpr int ktl_off = kth_off + F::FB * CP * 2;
  static constexpr int vt_off = ktl_off + F::FB * CP * 2;
  static constexpr int a_off = vt_off + E * CP * 2;
  static constexpr int z_off = a_off + kChunk * CP * 2;
  static constexpr int den_off = z_off + R * 4;
  static constexpr int bytes = den_off + kChunk * 4;
};

template <int R, int E>
struct FavorSegLayout {
  using F = FavorBlock<R>;
  static constexpr int kth_off = 0;
  static constexpr int ktl_off = kth_off + F::FB * CP * 2;
  static constexpr int vt_off = ktl_off + F::FB * CP * 2;
  static constexpr int bytes = vt_off + E * CP * 2;
};

__device__ __forceinline__ void split2(float x, bf16& hi, bf16& lo) {
  hi = (bf16)x;
  lo = (bf16)(x - to_f32(hi));
}

__device__ __forceinline__ void split4(const float (&f)[4], bf16x4& hi, bf16x4& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16 h, l;
    split2(f[i], h, l);
    hi[i] = h;
    lo[i] = l;
  }
}

// hi/lo bf16 image of 8 state rows (two 4-row halves of adjacent 16-row tiles)
// in the k-slot order of the inter-chunk product.
__device__ __forceinline__ void split_state_op(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
  bf16x4 ha, la, hb, lb;
  float fa[4] = {a[0], a[1], a[2], a[3]}, fb[4] = {b[0], b[1], b[2], b[3]};
  split4(fa, ha, la);
  split4(fb, hb, lb);
  hi = cat8(ha, hb);
  lo = cat8(la, lb);
}

__device__ __forceinline__ f32x4 mfma3(const bf16x8& ah, const bf16x8& al, const bf16x8& bh, const bf16x8& bl,
                                       f32x4 c) {
  c = mfma16(ah, bh, c);
  c = mfma16(al, bh, c);
  c = mfma16(ah, bl, c);
  return c;
}

// FAVOR+ features of one block of one side of a chunk, as hi/lo pairs.
// Queries: row-major tiles (qh, ql). Keys: row-major tiles (kh, kl) when ROWS,
// and transposed tiles (kth, ktl) carrying the RetNet weight gamma^(L-1-t).
template <int R, int DK, int GATE, bool IS_K, bool ROWS>
__device__ __forceinline__ void favor_block_side(const bf16x8 (&x)[4 * (DK / 32)], const bf16* omega, int fb, int L,
                                                 float lg2gam, char* sm, int hi_off, int lo_off, int kth_off,
                                                 int ktl_off, int lane, int w) {
  using F = FavorBlock<R>;
  constexpr int KS = DK / 32, RPB = F::RPB;
  const int g4 = lane >> 4, c16 = lane & 15;
  // omega fragments of this wave's features in block fb (32 KB total: cache-resident)
  bf16x8 om[F::MT][KS];
#pragma unroll
  for (int mt = 0; mt < F::MT; ++mt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      om[mt][ks] = *reinterpret_cast<const bf16x8*>(
          omega + (long long)(fb * F::FB + w * (F::FB / 4) + 16 * mt + c16) * DK + 32 * ks + 8 * g4);
  const float half_log_r = 0.5f * __logf(float(R));
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float xv = to_f32(x[tt * KS + ks][u]);
        ss += xv * xv;
      }
    const float shift = 0.5f * sum_over_groups(ss) + half_log_r;
    const int t = 16 * tt + c16;
    const bool tok_ok = t < L;
    float decay_k = 1.f;
    if constexpr (GATE == GT_DECAY) decay_k = exp2f(float(L - 1 - t) * lg2gam);
#pragma unroll
    for (int mt = 0; mt < F::MT; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma16(om[mt][ks], x[tt * KS + ks], acc);
      // acc[i] = P[token t][block feature ml + i]
      const int ml = w * (F::FB / 4) + 16 * mt + 4 * g4;
      float f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[i] = __expf(acc[i] - shift);
        if (IS_K) f[i] = keep_if(tok_ok, f[i]);
      }
      if constexpr (!IS_K || ROWS) {
        bf16x4 h, l;
        split4(f, h, l);
        lds<bf16x4>(sm, hi_off + 2 * (t * RPB + ml)) = h;
        lds<bf16x4>(sm, lo_off + 2 * (t * RPB + ml)) = l;
      }
      if constexpr (IS_K) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16 h, l;
          split2(f[i] * decay_k, h, l);
          lds<bf16>(sm, kth_off + 2 * ((ml + i) * CP + t)) = h;
          lds<bf16>(sm, ktl_off + 2 * ((ml + i) * CP + t)) = l;
        }
      }
    }
  }
}

// V transposed into LDS; rows at or past L (the chunk's valid tokens) are zero.
template <int E>
__device__ __forceinline__ void write_vt(const bf16x8 (&v)[E / 32], int L, char* sm, int vt_off, int lane, int w) {
  constexpr int EV = E / 4;
  const bool valid = lane < L;
#pragma unroll
  for (int j = 0; j < EV / 8; ++j) {
    const bf16x8 vv = keep_if(valid, v[j]);
#pragma unroll
    for (int u = 0; u < 8; ++u) lds<bf16>(sm, vt_off + 2 * ((w * EV + 8 * j + u) * CP + lane)) = vv[u];
  }
}

// S rows of feature block fb (all of them, wave's value columns) <- g S + K^^T V
// with K^ as a hi/lo pair, and this wave's z tiles of the block <- g z + K^^T 1
// (z is the state column of a constant-1 value). Wave w owns block-local z
// tiles rt = w ZT .. w ZT + ZT - 1; lane (g, c) holds z[16 rt + 4 g + i].
template <int R, int E>
__device__ __forceinline__ void favor_state_block(f32x4 (&S)[R / 16][E / 64], f32x4 (&Zb)[FavorBlock<R>::FB / 64],
                                                  int fb, char* sm, int kth_off, int ktl_off, int vt_off,
                                                  float gscale, int lane, int w) {
  using F = FavorBlock<R>;
  constexpr int ZT = F::FB / 64;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int ebase = w * (E / 4);
  bf16x8 ones;
#pragma unroll
  for (int u = 0; u < 8; ++u) ones[u] = (bf16)1.f;
  bf16x8 vb[E / 64][2];
#pragma unroll
  for (int eb = 0; eb < E / 64; ++eb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      vb[eb][ks] = lds<bf16x8>(sm, vt_off + 2 * ((ebase + 16 * eb + c16) * CP + 32 * ks + 8 * g4));
#pragma unroll
  for (int rt = 0; rt < F::FB / 16; ++rt) {
    bf16x8 kh[2], kl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      kh[ks] = lds<bf16x8>(sm, kth_off + 2 * ((16 * rt + c16) * CP + 32 * ks + 8 * g4));
      kl[ks] = lds<bf16x8>(sm, ktl_off + 2 * ((16 * rt + c16) * CP + 32 * ks + 8 * g4));
    }
#pragma unroll
    for (int eb = 0; eb < E / 64; ++eb) {
      f32x4 st = S[fb * (F::FB / 16) + rt][eb];
#pragma unroll
      for (int i = 0; i < 4; ++i) st[i] *= gscale;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        st = mfma16(kh[ks], vb[eb][ks], st);
        st = mfma16(kl[ks], vb[eb][ks], st);
      }
      S[fb * (F::FB / 16) + rt][eb] = st;
    }
    if (rt / ZT == w) {
      f32x4 zt = Zb[rt % ZT];
#pragma unroll
      for (int i = 0; i < 4; ++i) zt[i] *= gscale;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        zt = mfma16(kh[ks], ones, zt);
        zt = mfma16(kl[ks], ones, zt);
      }
      Zb[rt % ZT] = zt;
    }
  }
}

// z tiles (all blocks) of wave w to / from a flat [R] fp32 array.
template <int R>
__device__ __forceinline__ void favor_z_store(const f32x4 (&Z)[FavorBlock<R>::NFB][FavorBlock<R>::FB / 64],
                                              float* dst, int lane, int w) {
  using F = FavorBlock<R>;
  constexpr int ZT = F::FB / 64;
  if ((lane & 15) == 0) {
#pragma unroll
    for (int fb = 0; fb < F::NFB; ++fb)
#pragma unroll
      for (int j = 0; j < ZT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[fb * F::FB + 16 * (w * ZT + j) + 4 * (lane >> 4) + i] = Z[fb][j][i];
  }
}

template <int R>
__device__ __forceinline__ void favor_z_load(f32x4 (&Z)[FavorBlock<R>::NFB][FavorBlock<R>::FB / 64],
                                             const float* src, int lane, int w) {
  using F = FavorBlock<R>;
  constexpr int ZT = F::FB / 64;
#pragma unroll
  for (int fb = 0; fb < F::NFB; ++fb)
#pragma unroll
    for (int j = 0; j < ZT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Z[fb][j][i] = src != nullptr ? src[fb * F::FB + 16 * (w * ZT + j) + 4 * (lane >> 4) + i] : 0.f;
}

// ---------------------------------------------------------------------------
// Pass 1 (FAVOR+): each segment's own state contribution.
// ---------------------------------------------------------------------------
template <int R, int E, int DK, int GATE>
__global__ __launch_bounds__(256) void favor_segment_state(CausalArgs a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  using LY = FavorSegLayout<R, E>;
  using F = FavorBlock<R>;
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
  f32x4 Z[F::NFB][F::FB / 64];
  favor_z_load<R>(Z, nullptr, lane, w);

  RawChunk<R, E, DK, FM_FAVOR, GT_NONE, false> raw;
  raw.load(a, tok0, t_begin, lane, w);
  for (int t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int L = min(kChunk, a.n - t0);
    const float gsc = GATE == GT_DECAY ? exp2f(float(L) * lg2gam) : 1.f;
#pragma unroll
    for (int fb = 0; fb < F::NFB; ++fb) {
      favor_block_side<R, DK, GATE, true, false>(raw.xk, a.omega, fb, L, lg2gam, sm, 0, 0, LY::kth_off, LY::ktl_off,
                                                 lane, w);
      if (fb == 0) write_vt<E>(raw.v, L, sm, LY::vt_off, lane, w);
      if (fb == F::NFB - 1 && t0 + kChunk < t_end) raw.load(a, tok0, t0 + kChunk, lane, w);
      lds_barrier();
      favor_state_block<R, E>(S, Z[fb], fb, sm, LY::kth_off, LY::ktl_off, LY::vt_off, gsc, lane, w);
      lds_barrier();
    }
  }
  const long long slot = bh * a.P + s;
  float* So = a.S_out + slot * R * E;
#pragma unroll
  for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
    for (int eb = 0; eb < E / 64; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i) So[(16 * rt + 4 * g4 + i) * E + ebase + 16 * eb + c16] = S[rt][eb][i];
  favor_z_store<R>(Z, a.z_out + slot * R, lane, w);
}

// ---------------------------------------------------------------------------
// Pass 3 (FAVOR+): outputs of one segment from its chained state.
// ---------------------------------------------------------------------------
template <int R, int E, int DK, int GATE>
__global__ __launch_bounds__(256) void favor_chunk_forward(CausalArgs a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  using LY = FavorFwdLayout<R, E>;
  using F = FavorBlock<R>;
  constexpr int RPB = F::RPB, NEB = E / 64, KPB = F::FB / 32;
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

  f32x4 S[R / 16][NEB];
  f32x4 Z[F::NFB][F::FB / 64];
  if (a.S_in != nullptr) {
    const float* Sp = a.S_in + bh * a.in_head + s * a.in_seg;
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
  favor_z_load<R>(Z, a.S_in != nullptr ? a.z_in + (bh * a.in_head + s * a.in_seg) / E : nullptr, lane, w);
  favor_z_store<R>(Z, reinterpret_cast<float*>(sm + LY::z_off), lane, w);

  RawChunk<R, E, DK, FM_FAVOR, GT_NONE, true> raw;
  raw.load(a, tok0, t_begin, lane, w);
  for (int t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int L = min(kChunk, a.n - t0);
    const int q_own = 16 * w + c16;  // this lane's query row in the score phase
    f32x4 sacc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) sacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 oacc[4][NEB];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt)
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) oacc[qt][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float zd = 0.f;

#pragma unroll
    for (int fb = 0; fb < F::NFB; ++fb) {
      const bool last = fb == F::NFB - 1;
      favor_block_side<R, DK, GATE, false, false>(raw.xq, a.omega, fb, L, lg2gam, sm, LY::qh_off, LY::ql_off, 0, 0,
                                                  lane, w);
      favor_block_side<R, DK, GATE, true, true>(raw.xk, a.omega, fb, L, lg2gam, sm, LY::kh_off, LY::kl_off,
                                                LY::kth_off, LY::ktl_off, lane, w);
      if (fb == 0) write_vt<E>(raw.v, L, sm, LY::vt_off, lane, w);
      if (last && t0 + kChunk < t_end) raw.load(a, tok0, t0 + kChunk, lane, w);
      lds_barrier();

      // ---- scores over this block's features: A^T tiles = K~_c Q~_w^T
      {
        bf16x8 qh[KPB], ql[KPB];
#pragma unroll
        for (int ks = 0; ks < KPB; ++ks) {
          qh[ks] = lds<bf16x8>(sm, LY::qh_off + 2 * (q_own * RPB + 32 * ks + 8 * g4));
          ql[ks] = lds<bf16x8>(sm, LY::ql_off + 2 * (q_own * RPB + 32 * ks + 8 * g4));
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (c <= w) {
#pragma unroll
            for (int ks = 0; ks < KPB; ++ks) {
              const int ko = 2 * ((16 * c + c16) * RPB + 32 * ks + 8 * g4);
              sacc[c] = mfma3(lds<bf16x8>(sm, LY::kh_off + ko), lds<bf16x8>(sm, LY::kl_off + ko), qh[ks], ql[ks],
                              sacc[c]);
            }
          }
        }
#pragma unroll
        for (int ks = 0; ks < KPB; ++ks)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            zd += (to_f32(qh[ks][j]) + to_f32(ql[ks][j])) *
                  lds<float>(sm, LY::z_off + 4 * (fb * F::FB + 32 * ks + 8 * g4 + j));
      }
      if (last) {
        float rs = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (c <= w) {
            bf16x4 ab;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = 16 * c + 4 * g4 + i;
              float v = sacc[c][i];
              if (c == w && key > q_own) v = 0.f;  // only the diagonal tile straddles the mask
              if constexpr (GATE == GT_DECAY) v *= exp2f(float(q_own - key) * lg2gam);
              ab[i] = (bf16)v;
              rs += to_f32(ab[i]);
            }
            lds<bf16x4>(sm, LY::a_off + 2 * (q_own * CP + 16 * c + 4 * g4)) = ab;
          }
        }
        if ((w & 1) == 0) lds<bf16x4>(sm, LY::a_off + 2 * (q_own * CP + 16 * (w + 1) + 4 * g4)) = bf16x4{};
        rs = sum_over_groups(rs);
        float zdt = sum_over_groups(zd);
        if constexpr (GATE == GT_DECAY) zdt *= exp2f(float(q_own + 1) * lg2gam);
        if (g4 == 0) lds<float>(sm, LY::den_off + 4 * q_own) = rs + zdt + a.eps;
        lds_barrier();
      }

      // ---- inter-chunk product over this block's features: O^T += S^T Q^^T
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const int q = 16 * qt + c16;
        bf16x8 qbh[KPB], qbl[KPB];
#pragma unroll
        for (int p = 0; p < KPB; ++p) {
          const int o0 = 2 * (q * RPB + 32 * p + 4 * g4), o1 = 2 * (q * RPB + 32 * p + 16 + 4 * g4);
          qbh[p] = cat8(lds<bf16x4>(sm, LY::qh_off + o0), lds<bf16x4>(sm, LY::qh_off + o1));
          qbl[p] = cat8(lds<bf16x4>(sm, LY::ql_off + o0), lds<bf16x4>(sm, LY::ql_off + o1));
        }
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
          for (int p = 0; p < KPB; ++p) {
            bf16x8 sh, sl;
            const int rt = fb * (F::FB / 16) + 2 * p;
            split_state_op(S[rt][eb], S[rt + 1][eb], sh, sl);
            oacc[qt][eb] = mfma3(sh, sl, qbh[p], qbl[p], oacc[qt][eb]);
          }
      }

      // ---- carry the state rows of this block past the chunk
      const float gsc = GATE == GT_DECAY ? exp2f(float(L) * lg2gam) : 1.f;
      // z of this block is published after the chunk's last barrier: other
      // waves may still be reading the old values in this block's score phase.
      favor_state_block<R, E>(S, Z[fb], fb, sm, LY::kth_off, LY::ktl_off, LY::vt_off, gsc, lane, w);

      if (last) {
        // ---- intra-chunk part and normalisation: O^T += V^T A^T, o = O / den
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          const int q = 16 * qt + c16;
          // one correctly rounded reciprocal per row; outputs are fl(O * fl(1 / den))
          const float inv_den = 1.f / lds<float>(sm, LY::den_off + 4 * q);
          float isc = 1.f;
          if constexpr (GATE == GT_DECAY) isc = exp2f(float(q + 1) * lg2gam);
#pragma unroll
          for (int eb = 0; eb < NEB; ++eb) {
            const int e = ebase + 16 * eb;
            f32x4 acc = oacc[qt][eb];
            if constexpr (GATE == GT_DECAY) {
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[i] *= isc;
            }
#pragma unroll
            for (int p2 = 0; p2 <= qt / 2; ++p2)
              acc = mfma16(lds<bf16x8>(sm, LY::vt_off + 2 * ((e + c16) * CP + 32 * p2 + 8 * g4)),
                           lds<bf16x8>(sm, LY::a_off + 2 * (q * CP + 32 * p2 + 8 * g4)), acc);
            if (q < L) {
              bf16x4 o = pack4(acc[0] * inv_den, acc[1] * inv_den, acc[2] * inv_den, acc[3] * inv_den);
              *reinterpret_cast<bf16x4*>(a.out + (tok0 + t0 + q) * E + e + 4 * g4) = o;
            }
          }
        }
      }
      lds_barrier();
    }
    favor_z_store<R>(Z, reinterpret_cast<float*>(sm + LY::z_off), lane, w);
  }

  if (a.S_out != nullptr && s == a.P - 1) {
    float* So = a.S_out + bh * R * E;
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int i = 0; i < 4; ++i) So[(16 * rt + 4 * g4 + i) * E + ebase + 16 * eb + c16] = S[rt][eb][i];
    favor_z_store<R>(Z, a.z_out + bh * R, lane, w);
  }
}

template <int R, int E, int DK, int GATE>
la_status run_causal_favor(const FwdPlan& p) {
  CausalArgs a{};
  a.Q = static_cast<const bf16*>(p.Q);
  a.K = static_cast<const bf16*>(p.K);
  a.V = static_cast<const bf16*>(p.V);
  a.omega = static_cast<const bf16*>(p.omega);
  a.gamma = p.gamma;
  a.out = static_cast<bf16*>(p.out);
  a.H = p.H;
  a.n = p.n;
  a.P = p.P;
  a.seg_len = p.seg_len;
  a.eps = p.eps;
  const unsigned BH = unsigned(p.B) * unsigned(p.H);
  if (p.P > 1) {
    CausalArgs a1 = a;
    a1.S_out = p.ws_S;
    a1.z_out = p.ws_z;
    auto k1 = favor_segment_state<R, E, DK, GATE>;
    constexpr int lds1 = FavorSegLayout<R, E>::bytes;
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
  auto k3 = favor_chunk_forward<R, E, DK, GATE>;
  constexpr int lds3 = FavorFwdLayout<R, E>::bytes;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k3), hipFuncAttributeMaxDynamicSharedMemorySize, lds3) !=
      hipSuccess)
    return LA_ERR_HIP;
  hipLaunchKernelGGL(k3, dim3(p.P, BH), dim3(256), lds3, p.stream, a);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // namespace la
