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
//   * the feature axis is processed in blocks of 64 features: the hi/lo tiles
//     of one block are the only per-block LDS, which keeps a workgroup near
//     54 KB so two of them share a CU. Everything that contracts over the
//     features (scores, inter-chunk product, z . phi(q)) accumulates across
//     blocks in registers.
// The projection X w^T runs on the matrix cores (exact bf16 products, fp32
// accumulation); |x|^2/2 and ln(r)/2 are subtracted before the exponential.
//
// LDS tiles are [token][column]. Operands that contract over tokens (phi(k)^T
// in the state update, V^T in the intra-chunk product) come from them by
// transpose reads. The feature tiles have unpadded 128-byte rows whose 16-byte
// chunks are permuted per row (favor_swz), so that every access pattern on
// them spreads over all LDS banks. Each wave projects its own 16 tokens (whose
// raw rows it loaded) onto all features of a block, so the raw rows never pass
// through LDS; omega comes from the cache.
#pragma once

#include "chunked.hpp"

namespace la {

template <int R>
struct FavorBlock {
  static constexpr int FB = 64;       // features per block
  static constexpr int NFB = R / FB;  // blocks
  static constexpr int FT = FB / 16;  // 16-feature tiles per block
  static constexpr int ROW = 2 * FB;  // bytes per token row of a feature tile
  static constexpr int TILE16 = 16 * ROW;  // bytes per 16 token rows
};

// Feature tiles. Block-local feature f = 16 t + 4 g + i is stored at logical
// column 32 (t >> 1) + 8 g + 4 (t & 1) + i of its token's row: the eight
// features one lane needs as an inter-chunk B operand (S tiles 2p and 2p + 1
// give the k-slots of the matrix-core product), or that it projects for two
// adjacent 16-feature tiles, form one 16-byte chunk. Logical chunk k of row r
// is stored at chunk k ^ favor_swz(r). Measured on gfx950, 16-byte row
// accesses (rows c, chunks g + const) and transpose reads of rows 4 g + j
// (j < 4) then reach all banks without conflicts, where a plain padded stride
// serves one of the two patterns at a time.
__device__ __forceinline__ int favor_swz(int r) { return 4 * ((r >> 1) & 1) | 2 * ((r >> 2) & 1); }

// Output pass. kwh/kwl (RetNet only) hold the decay-weighted key features of
// the state update; kh/kl hold the unweighted ones of the scores. zh/zl are
// the bf16 hi/lo image of z_prev (B operand of phi(q) . z on the matrix cores).
template <int R, int E, int GATE>
struct FavorFwdLayout {
  using F = FavorBlock<R>;
  static constexpr int EP = E + kPad;
  // 16 bytes between tiles: the hi and lo halves of one row are never a
  // multiple of 512 B apart, so their reads are not fused into one two-address
  // load whose halves would then have to be moved into operand order
  static constexpr int TILE = kChunk * F::ROW + 16;
  static constexpr int qh_off = 0;
  static constexpr int ql_off = qh_off + TILE;
  static constexpr int kh_off = ql_off + TILE;
  static constexpr int kl_off = kh_off + TILE;
  static constexpr int kwh_off = kl_off + TILE;
  static constexpr int kwl_off = kwh_off + (GATE == GT_DECAY ? TILE : 0);
  static constexpr int v_off = kwl_off + (GATE == GT_DECAY ? TILE : 0);
  static constexpr int zh_off = v_off + kChunk * EP * 2;
  static constexpr int zl_off = zh_off + R * 2 + 16;
  static constexpr int rsp_off = zl_off + R * 2 + 16;       // [4][64] partial score row sums
  static constexpr int zdp_off = rsp_off + 4 * kChunk * 4;  // [64] phi(q) . z
  static constexpr int a_off = zdp_off + kChunk * 4;       // [64][CP] masked scores
  static constexpr int bytes = a_off + kChunk * CP * 2;
  template <int DK>
  static constexpr int bytes_dk = bytes;
};

// Segment-state pass: kh/kl hold the (decay-weighted) key features; omega
// sits in LDS for the whole kernel when it is at most 32 KB (read per feature
// block by every wave, it cost more from the cache than the state update).
template <int R, int E>
struct FavorSegLayout {
  using F = FavorBlock<R>;
  static constexpr int EP = E + kPad;
  static constexpr int kh_off = 0;
  static constexpr int kl_off = kh_off + kChunk * F::ROW + 16;
  static constexpr int v_off = kl_off + kChunk * F::ROW + 16;
  static constexpr int om_off = v_off + kChunk * EP * 2;
  static constexpr int bytes = om_off;
  template <int DK>
  static constexpr bool om_lds = R * DK <= 16384;
  template <int DK>
  static constexpr int bytes_dk = bytes + (om_lds<DK> ? R * DK * 2 : 0);
};

// Per-lane byte offsets of every LDS access pattern, built once per feature
// block from an opaque lane index (opaque_lane): each access then adds only
// compile-time or wave-uniform constants, which fold into the instruction.
template <int EP>
struct FavorLane {
  int g4, c16;
  int row[2];  // feature tile: row c, logical chunk g + 4 h (h = 0, 1)
  int tr[2];   // feature tile transpose reads: row 4 g + (c >> 2), logical chunk 4 h + (c & 3)
  int tre;     // V tile transpose reads, rows 8 g + (c >> 2) (+4): intra-chunk product
  int tre2;    // V tile transpose reads, rows 4 g + (c >> 2) (+16): state update
  int afrag;   // row c, 8 columns at 8 g of the score tile
  int a4;      // row c, 4 columns at 4 g of the score tile
  int l4;      // 4 c (per-row floats)
  __device__ __forceinline__ FavorLane(int lane) {
    g4 = lane >> 4;
    c16 = lane & 15;
    const int rs = favor_swz(c16);
    row[0] = 128 * c16 + 16 * (g4 ^ rs);
    row[1] = 128 * c16 + 16 * ((g4 + 4) ^ rs);
    const int rt = 4 * g4 + (c16 >> 2), ts = favor_swz(rt);
    tr[0] = 128 * rt + 16 * ((c16 & 3) ^ ts);
    tr[1] = 128 * rt + 16 * ((4 + (c16 & 3)) ^ ts);
    tre = 2 * ((8 * g4 + (c16 >> 2)) * EP + 4 * (c16 & 3));
    tre2 = 2 * ((4 * g4 + (c16 >> 2)) * EP + 4 * (c16 & 3));
    afrag = 2 * (c16 * CP + 8 * g4);
    a4 = 2 * (c16 * CP + 4 * g4);
    l4 = 4 * c16;
  }
};

// MFMA operand by two transpose reads (see tr_feat), the second `gap`
// bytes after the first: k-slots 0..3 and 4..7 of the lane's group.
__device__ __forceinline__ bf16x8 tr_pair(char* sm, int addr, int gap) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sm + addr));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sm + addr + gap));
  return cat8(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi));
}

// The raw rows of this wave's tokens (16 w + c) as projection B operands,
// copied out of the prefetch registers, and each token's shift in base 2,
// (|x|^2/2 + ln(r)/2) log2(e), r = rv the map's feature count (R, or fewer
// when the kernel runs a narrower map with its extra features masked).
template <int R, int DK>
__device__ __forceinline__ float favor_take_x(const bf16x8 (&raw)[DK / 32], bf16x8 (&x)[DK / 32], int rv = R) {
  float ss = 0.f;
#pragma unroll
  for (int ks = 0; ks < DK / 32; ++ks) {
    x[ks] = raw[ks];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float xv = to_f32(raw[ks][u]);
      ss += xv * xv;
    }
  }
  return (0.5f * sum_over_groups(ss) + 0.5f * __logf(float(rv))) * 1.44269504f;
}

// hi/lo bf16 pairs of four floats (packed two per dword).
__device__ __forceinline__ void split4(const float (&f)[4], bf16x4& hi, bf16x4& lo) {
  const unsigned h01 = pack2_bits(f[0], f[1]), h23 = pack2_bits(f[2], f[3]);
  const unsigned l01 = pack2_bits(f[0] - lo_bf16_f32(h01), f[1] - hi_bf16_f32(h01));
  const unsigned l23 = pack2_bits(f[2] - lo_bf16_f32(h23), f[3] - hi_bf16_f32(h23));
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  hi = __builtin_bit_cast(bf16x4, u32x2{h01, h23});
  lo = __builtin_bit_cast(bf16x4, u32x2{l01, l23});
}

// hi/lo bf16 image of 8 state rows (two 4-row halves of adjacent 16-row tiles)
// in the k-slot order of the inter-chunk product.
__device__ __forceinline__ void split_state_op(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
  bf16x4 ha, la, hb, lb;
  const float fa[4] = {a[0], a[1], a[2], a[3]}, fb[4] = {b[0], b[1], b[2], b[3]};
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

__device__ __forceinline__ bf16x4 keep_if(bool ok, bf16x4 x) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const unsigned m = ok ? 0xffffffffu : 0u;
  return __builtin_bit_cast(bf16x4, __builtin_bit_cast(u32x2, x) & m);
}

// omega rows of feature block fb as projection A operands: om[ft][ks] holds
// row 64 fb + 16 ft + c, columns 32 ks + 8 g .. + 7 (the whole omega is 32 KB
// or less: cache-resident). Loaded one block ahead of its use.
template <int R, int DK, class LN>
__device__ __forceinline__ void favor_load_omega(bf16x8 (&om)[FavorBlock<R>::FT][DK / 32], const bf16* omega, int fb,
                                                 const LN& ln) {
  const bf16* orow = omega + (long long)(fb * FavorBlock<R>::FB + ln.c16) * DK + 8 * ln.g4;
#pragma unroll
  for (int ft = 0; ft < FavorBlock<R>::FT; ++ft)
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) om[ft][ks] = *reinterpret_cast<const bf16x8*>(orow + 16 * ft * DK + 32 * ks);
}

// omega [R][DK] in LDS: 16-byte chunk k of row r at chunk k ^ favor_om_swz(r),
// so that the projection's operand reads (rows c of a 16-row tile, chunks
// 4 ks + g, lanes in groups of rows 0..7 x g in {0, 1}) reach all banks.
template <int DK>
__device__ __forceinline__ int favor_om_swz(int r) {
  if constexpr (DK == 32) return 2 * ((r >> 2) & 1);
  else if constexpr (DK == 64) return r & 6;
  else return 2 * (r & 7);
}

template <int R, int DK>
__device__ __forceinline__ void favor_stage_omega(const bf16* omega, char* sm, int om_off, int tid) {
  constexpr int CPR = DK / 8;  // 16-byte chunks per row
#pragma unroll
  for (int c = tid; c < R * CPR; c += 256) {
    const int r = c / CPR, k = c % CPR;
    lds<bf16x8>(sm, om_off + r * DK * 2 + 16 * (k ^ favor_om_swz<DK>(r))) =
        *reinterpret_cast<const bf16x8*>(omega + (long long)r * DK + 8 * k);
  }
}

// favor_load_omega's operands, from the LDS copy.
template <int R, int DK, class LN>
__device__ __forceinline__ void favor_lds_omega(bf16x8 (&om)[FavorBlock<R>::FT][DK / 32], char* sm, int om_off,
                                                int fb, const LN& ln) {
#pragma unroll
  for (int ft = 0; ft < FavorBlock<R>::FT; ++ft)
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      const int r = fb * FavorBlock<R>::FB + 16 * ft + ln.c16;
      om[ft][ks] = lds<bf16x8>(sm, om_off + r * DK * 2 + 16 * ((4 * ks + ln.g4) ^ favor_om_swz<DK>(r)));
    }
}

// hi/lo tile chunks of eight features (two adjacent 16-feature tiles), zero
// unless ok.
__device__ __forceinline__ void favor_store_pair(char* sm, int hi_at, int lo_at, const float (&f0)[4],
                                                 const float (&f1)[4], bool ok) {
  bf16x4 h0, l0, h1, l1;
  split4(f0, h0, l0);
  split4(f1, h1, l1);
  lds<bf16x8>(sm, hi_at) = cat8(keep_if(ok, h0), keep_if(ok, h1));
  lds<bf16x8>(sm, lo_at) = cat8(keep_if(ok, l0), keep_if(ok, l1));
}

// FAVOR+ features of one side of a chunk for this wave's 16 tokens (16 w + c)
// and all 64 features of block fb, as hi/lo pairs in feature tiles: phi =
// 2^(P log2(e) - shift2) with P = x . w on the matrix cores (x: this wave's raw
// rows, omega rows from the cache). Keys past the chunk's valid rows are zero.
// With WEIGHTED, keys are also written multiplied by gamma^(L-1-t) (RetNet
// state update) into (wh_off, wl_off); with ONLY_WEIGHTED that is the only copy.
// Features at or past rv (a narrower map run on these R-wide kernels, its
// omega zero-padded to R rows) are zero.
template <int R, int DK, bool IS_K, bool WEIGHTED, bool ONLY_WEIGHTED, class LN>
__device__ __forceinline__ void favor_project(const LN& ln, const bf16x8 (&x)[DK / 32], float shift2,
                                              const bf16x8 (&om)[FavorBlock<R>::FT][DK / 32], int L, float lg2gam,
                                              char* sm, int hi_off, int lo_off, int wh_off, int wl_off, int w,
                                              int fb = 0, int rv = R) {
  using F = FavorBlock<R>;
  constexpr int KS = DK / 32;
  const int t = 16 * w + ln.c16;
  const bool ok = !IS_K || t < L;
  float wt = 1.f;
  if constexpr (WEIGHTED) wt = exp2f(float(max(L - 1 - t, 0)) * lg2gam);  // rows past L are dropped
#pragma unroll
  for (int h = 0; h < F::FT / 2; ++h) {
    float f[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma16(om[2 * h + u][ks], x[ks], acc);
      // acc[i] = P[token t][block feature 16 (2 h + u) + 4 g + i]
#pragma unroll
      for (int i = 0; i < 4; ++i) f[u][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], 1.44269504f, -shift2));
      if (R == F::FB && rv < R) {  // only the one-block kernels serve narrower maps
        const int f0 = F::FB * fb + 16 * (2 * h + u) + 4 * ln.g4;
#pragma unroll
        for (int i = 0; i < 4; ++i) f[u][i] = f0 + i < rv ? f[u][i] : 0.f;
      }
    }
    // logical chunk 4 h + g of row t
    const int at = F::TILE16 * w + ln.row[h];
    if constexpr (!ONLY_WEIGHTED) favor_store_pair(sm, hi_off + at, lo_off + at, f[0], f[1], ok);
    if constexpr (WEIGHTED) {
      float fw[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) fw[u][i] = f[u][i] * wt;
      favor_store_pair(sm, wh_off + at, wl_off + at, fw[0], fw[1], ok);
    }
    __builtin_amdgcn_sched_barrier(0);  // two feature tiles at a time: bounded live registers
  }
}

// V rows of the chunk into a row-major [token][E + kPad] tile (lane = token,
// wave w holds columns [w E/4, (w+1) E/4)). Rows past the end need no mask:
// their key features are zero and their scores are masked.
template <int E>
__device__ __forceinline__ void favor_write_v(const bf16x8 (&v)[E / 32], char* sm, int v_off, int lane, int w) {
  constexpr int EV = E / 4, EP = E + kPad;
#pragma unroll
  for (int j = 0; j < EV / 8; ++j) lds<bf16x8>(sm, v_off + 2 * (lane * EP + w * EV + 8 * j)) = v[j];
}

// S rows of feature block fb (the wave's value columns) <- g S + K^^T V with
// K^ as a hi/lo pair, and the wave's z tile of the block <- g z + K^^T 1 (z
// is the state column of a constant-1 value). Wave w owns block-local z tile
// w: lane (g, c) holds z[64 fb + 16 w + 4 g + i] in Zb. The contraction runs
// over the chunk's tokens in the order 32 ks + 16 (s >> 2) + 4 g + (s & 3) for
// k-slot s of lane group g, the same for K^ and V.
template <int R, int E, class LN>
__device__ __forceinline__ void favor_state_block(const LN& ln, f32x4 (&S)[R / 16][E / 64], f32x4& Zb, int fb,
                                                  char* sm, int kh_off, int kl_off, int v_off, float gscale, int w) {
  using F = FavorBlock<R>;
  constexpr int EP = E + kPad;
  bf16x8 ones;
#pragma unroll
  for (int u = 0; u < 8; ++u) ones[u] = (bf16)1.f;
  bf16x8 vb[E / 64][2];
  const int vbase = v_off + 2 * w * (E / 4) + ln.tre2;
#pragma unroll
  for (int eb = 0; eb < E / 64; ++eb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) vb[eb][ks] = tr_pair(sm, vbase + 2 * (32 * ks * EP + 16 * eb), 2 * 16 * EP);
#pragma unroll
  for (int rt = 0; rt < F::FT; ++rt) {
    // features 16 rt + c: logical chunk 4 (rt >> 1) + (c >> 2), half rt & 1
    bf16x8 kh[2], kl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int o = 2 * F::TILE16 * ks + ln.tr[rt >> 1] + 8 * (rt & 1);
      kh[ks] = tr_pair(sm, kh_off + o, F::TILE16);
      kl[ks] = tr_pair(sm, kl_off + o, F::TILE16);
    }
#pragma unroll
    for (int eb = 0; eb < E / 64; ++eb) {
      f32x4 st = S[fb * F::FT + rt][eb];
#pragma unroll
      for (int i = 0; i < 4; ++i) st[i] *= gscale;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        st = mfma16(kh[ks], vb[eb][ks], st);
        st = mfma16(kl[ks], vb[eb][ks], st);
      }
      S[fb * F::FT + rt][eb] = st;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // this wave's z tile (block rows 16 w .. 16 w + 15), outside the tile loop
  // so no branch on the wave index splits it
  f32x4 zt = Zb;
#pragma unroll
  for (int i = 0; i < 4; ++i) zt[i] *= gscale;
  const int zb = (w >= 2 ? ln.tr[1] : ln.tr[0]) + 8 * (w & 1);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int o = 2 * F::TILE16 * ks + zb;
    zt = mfma16(tr_pair(sm, kh_off + o, F::TILE16), ones, zt);
    zt = mfma16(tr_pair(sm, kl_off + o, F::TILE16), ones, zt);
  }
  Zb = zt;
}

// z tiles (all blocks) of wave w to / from a flat [R] fp32 array.
template <int R>
__device__ __forceinline__ void favor_z_store(const f32x4 (&Z)[FavorBlock<R>::NFB], float* dst, int lane, int w) {
  if ((lane & 15) == 0) {
#pragma unroll
    for (int fb = 0; fb < FavorBlock<R>::NFB; ++fb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[64 * fb + 16 * w + 4 * (lane >> 4) + i] = Z[fb][i];
  }
}

// bf16 hi/lo image of the wave's z tiles into LDS (zh, zl: [R] bf16 each, in
// the logical column order of the feature tiles).
template <int R>
__device__ __forceinline__ void favor_z_publish(const f32x4 (&Z)[FavorBlock<R>::NFB], char* sm, int zh_off,
                                                int zl_off, int lane, int w) {
  if ((lane & 15) == 0) {
#pragma unroll
    for (int fb = 0; fb < FavorBlock<R>::NFB; ++fb) {
      const float f[4] = {Z[fb][0], Z[fb][1], Z[fb][2], Z[fb][3]};
      bf16x4 h, l;
      split4(f, h, l);
      const int o = 2 * (64 * fb + 32 * (w >> 1) + 8 * (lane >> 4) + 4 * (w & 1));
      lds<bf16x4>(sm, zh_off + o) = h;
      lds<bf16x4>(sm, zl_off + o) = l;
    }
  }
}

template <int R>
__device__ __forceinline__ void favor_z_load(f32x4 (&Z)[FavorBlock<R>::NFB], const float* src, int lane, int w) {
#pragma unroll
  for (int fb = 0; fb < FavorBlock<R>::NFB; ++fb)
#pragma unroll
    for (int i = 0; i < 4; ++i) Z[fb][i] = src != nullptr ? src[64 * fb + 16 * w + 4 * (lane >> 4) + i] : 0.f;
}

// ---------------------------------------------------------------------------
// Pass 1 (FAVOR+): each segment's own state contribution.
// ---------------------------------------------------------------------------
template <int R, int E, int DK, int GATE>
__global__ __launch_bounds__(256) void favor_segment_state(CausalArgs a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  using LY = FavorSegLayout<R, E>;
  using F = FavorBlock<R>;
  using LN = FavorLane<E + kPad>;
  const int lane = lane_id(), w = wave_id();
  const int g4 = lane >> 4, c16 = lane & 15;
  const int s = blockIdx.x;
  const long long bh = blockIdx.y;
  const int h = int(bh % a.H);
  const SeqView sv = seq_view(a, bh);
  const int rvalid = a.r_valid > 0 ? a.r_valid : R;  // features of the map (the rest are masked)
  const int t_begin = s * a.seg_len;
  // only segments that a later segment of the same sequence follows
  if (t_begin + a.seg_len >= sv.len) return;
  const int t_end = min(sv.len, t_begin + a.seg_len);
  const long long tok0 = sv.tok0;
  const int ebase = w * (E / 4);
  float lg2gam = 0.f;
  if constexpr (GATE == GT_DECAY) lg2gam = log2f(a.gamma[h]);

  f32x4 S[R / 16][E / 64];
#pragma unroll
  for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
    for (int eb = 0; eb < E / 64; ++eb) S[rt][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 Z[F::NFB];
  favor_z_load<R>(Z, nullptr, lane, w);

  RawChunk<R, E, DK, FM_FAVOR, GT_NONE, false> raw;
  raw.load(a, tok0, t_begin, t_end, lane, w);
  constexpr bool OM_LDS = LY::template om_lds<DK>;
  bf16x8 om[F::FT][DK / 32];
  if constexpr (OM_LDS) {
    favor_stage_omega<R, DK>(a.omega, sm, LY::om_off, threadIdx.x);
    lds_barrier();
    favor_lds_omega<R, DK>(om, sm, LY::om_off, 0, LN(lane));
  } else {
    favor_load_omega<R, DK>(om, a.omega, 0, LN(lane));
  }
  for (int t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int L = min(kChunk, sv.len - t0);
    const float gsc = GATE == GT_DECAY ? exp2f(float(L) * lg2gam) : 1.f;
    bf16x8 xk[DK / 32];
    const float shk = favor_take_x<R, DK>(raw.xk, xk, rvalid);
    favor_write_v<E>(raw.v, sm, LY::v_off, lane, w);
    // the raw registers are free: the next chunk's loads fly during this one
    raw.load(a, tok0, t0 + kChunk, t_end, lane, w);
#pragma unroll
    for (int fb = 0; fb < F::NFB; ++fb) {
      const LN ln(opaque_lane(lane));
      // pass 1 keeps only the keys of the state update (decay-weighted for RetNet)
      favor_project<R, DK, true, GATE == GT_DECAY, GATE == GT_DECAY>(ln, xk, shk, om, L, lg2gam, sm, LY::kh_off,
                                                                     LY::kl_off, LY::kh_off, LY::kl_off, w, fb,
                                                                     rvalid);
      // next block (block 0 of the next chunk)
      if constexpr (OM_LDS)
        favor_lds_omega<R, DK>(om, sm, LY::om_off, fb + 1 < F::NFB ? fb + 1 : 0, ln);
      else
        favor_load_omega<R, DK>(om, a.omega, fb + 1 < F::NFB ? fb + 1 : 0, ln);
      lds_barrier();
      favor_state_block<R, E>(ln, S, Z[fb], fb, sm, LY::kh_off, LY::kl_off, LY::v_off, gsc, w);
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
__global__ __launch_bounds__(256, 2) void favor_chunk_forward(CausalArgs a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  using LY = FavorFwdLayout<R, E, GATE>;
  using F = FavorBlock<R>;
  using LN = FavorLane<E + kPad>;
  constexpr int EP = LY::EP, NEB = E / 64, KPB = F::FB / 32;
  const int lane = lane_id(), w = wave_id(), tid = threadIdx.x;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int s = blockIdx.x;
  const long long bh = blockIdx.y;
  const int h = int(bh % a.H);
  const SeqView sv = seq_view(a, bh);
  const int rvalid = a.r_valid > 0 ? a.r_valid : R;  // features of the map (the rest are masked)
  const int t_begin = s * a.seg_len;
  if (s > 0 && t_begin >= sv.len) return;  // past the end of this sequence
  const int t_end = min(sv.len, t_begin + a.seg_len);
  const long long tok0 = sv.tok0;
  const int ebase = w * (E / 4);
  float lg2gam = 0.f;
  if constexpr (GATE == GT_DECAY) lg2gam = log2f(a.gamma[h]);

  f32x4 S[R / 16][NEB];
  f32x4 Z[F::NFB];
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
  favor_z_load<R>(Z, has_in ? a.z_in + (in_idx * a.in_head + s * a.in_seg) / E : nullptr, lane, w);
  favor_z_publish<R>(Z, sm, LY::zh_off, LY::zl_off, lane, w);
  // partial row sums of query tiles this wave holds no score tile of stay zero
  lds<float>(sm, LY::rsp_off + 4 * tid) = 0.f;

  // this wave's score tiles
  const int nslot = w < 2 ? 3 : 2;
  int sqi[3], skj[3];
  score_tiles(w, sqi, skj);

  RawChunk<R, E, DK, FM_FAVOR, GT_NONE, true> raw;
  if (sv.len > 0) raw.load(a, tok0, t_begin, t_end, lane, w);  // an empty sequence reads nothing
  bf16x8 om[F::FT][DK / 32];
  favor_load_omega<R, DK>(om, a.omega, 0, LN(lane));
  for (int t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int L = min(kChunk, sv.len - t0);
    bf16x8 xq[DK / 32], xk[DK / 32];
    const float shq = favor_take_x<R, DK>(raw.xq, xq, rvalid), shk = favor_take_x<R, DK>(raw.xk, xk, rvalid);
    favor_write_v<E>(raw.v, sm, LY::v_off, lane, w);
    // the raw registers are free: the next chunk's loads fly during this one
    raw.load(a, tok0, t0 + kChunk, t_end, lane, w);
    f32x4 sacc[3];
#pragma unroll
    for (int sl = 0; sl < 3; ++sl) sacc[sl] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 oacc[4][NEB];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt)
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) oacc[qt][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 zacc = {0.f, 0.f, 0.f, 0.f};  // phi(q) . z_prev for queries 16 w + 4 g + i

#pragma unroll
    for (int fb = 0; fb < F::NFB; ++fb) {
      const LN ln(opaque_lane(lane));
      const bool last = fb == F::NFB - 1;
      favor_project<R, DK, false, false, false>(ln, xq, shq, om, L, lg2gam, sm, LY::qh_off, LY::ql_off, 0, 0, w, fb,
                                                rvalid);
      favor_project<R, DK, true, GATE == GT_DECAY, false>(ln, xk, shk, om, L, lg2gam, sm, LY::kh_off, LY::kl_off,
                                                          LY::kwh_off, LY::kwl_off, w, fb, rvalid);
      favor_load_omega<R, DK>(om, a.omega, fb + 1 < F::NFB ? fb + 1 : 0, ln);  // next block (block 0 of the next chunk)
      lds_barrier();

      // ---- scores over this block's features: A^T tiles = K~_kj Q~_qi^T, and
      // phi(q) . z_prev for query tile w (slot 0) on the matrix cores, z as a
      // hi/lo column replicated over the 16 output columns
#pragma unroll
      for (int sl = 0; sl < 3; ++sl) {
        if (sl < nslot) {
          const int ko = F::TILE16 * skj[sl], qo = F::TILE16 * sqi[sl];
#pragma unroll
          for (int ks = 0; ks < KPB; ++ks) {
            // logical columns 32 ks + 8 g .. + 7 of both sides
            const int r = ln.row[ks];
            const bf16x8 qh = lds<bf16x8>(sm, LY::qh_off + qo + r), ql = lds<bf16x8>(sm, LY::ql_off + qo + r);
            sacc[sl] = mfma3(lds<bf16x8>(sm, LY::kh_off + ko + r), lds<bf16x8>(sm, LY::kl_off + ko + r), qh, ql,
                             sacc[sl]);
            if (sl == 0) {
              const int zo = 2 * (64 * fb + 32 * ks + 8 * ln.g4);
              zacc = mfma3(qh, ql, lds<bf16x8>(sm, LY::zh_off + zo), lds<bf16x8>(sm, LY::zl_off + zo), zacc);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      __builtin_amdgcn_sched_barrier(0);  // phases stay apart: bounded register live ranges
      // ---- inter-chunk product over this block's features: O^T += S^T Q^^T
      {
        bf16x8 sh[KPB][NEB], slo[KPB][NEB];
#pragma unroll
        for (int p = 0; p < KPB; ++p)
#pragma unroll
          for (int eb = 0; eb < NEB; ++eb)
            split_state_op(S[fb * F::FT + 2 * p][eb], S[fb * F::FT + 2 * p + 1][eb], sh[p][eb], slo[p][eb]);
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
          for (int p = 0; p < KPB; ++p) {
            // features 32 p + 4 g + (0..3) and 32 p + 16 + 4 g + (0..3): logical chunk 4 p + g
            const int o = F::TILE16 * qt + ln.row[p];
            const bf16x8 qbh = lds<bf16x8>(sm, LY::qh_off + o), qbl = lds<bf16x8>(sm, LY::ql_off + o);
#pragma unroll
            for (int eb = 0; eb < NEB; ++eb) oacc[qt][eb] = mfma3(sh[p][eb], slo[p][eb], qbh, qbl, oacc[qt][eb]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- carry the state rows of this block past the chunk (z is
      // published after the chunk's last barrier: other waves still read the
      // old values in later blocks)
      __builtin_amdgcn_sched_barrier(0);
      const float gsc = GATE == GT_DECAY ? exp2f(float(L) * lg2gam) : 1.f;
      favor_state_block<R, E>(ln, S, Z[fb], fb, sm, GATE == GT_DECAY ? LY::kwh_off : LY::kh_off,
                              GATE == GT_DECAY ? LY::kwl_off : LY::kl_off, LY::v_off, gsc, w);

      __builtin_amdgcn_sched_barrier(0);
      if (last) {
        // ---- masked bf16 scores, their partial row sums, phi(q) . z
#pragma unroll
        for (int sl = 0; sl < 3; ++sl) {
          if (sl < nslot) {
            const int q = 16 * sqi[sl] + ln.c16;
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = 16 * skj[sl] + 4 * ln.g4 + i;
              v[i] = sacc[sl][i];
              // gamma^(q - key) only where key <= q; the mask selects after it
              if constexpr (GATE == GT_DECAY) v[i] *= exp2f(float(max(q - key, 0)) * lg2gam);
              if (key > q) v[i] = 0.f;  // only the diagonal tiles straddle the mask
            }
            const unsigned p01 = pack2_bits(v[0], v[1]), p23 = pack2_bits(v[2], v[3]);
            typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
            lds<u32x2>(sm, LY::a_off + 32 * sqi[sl] * CP + 32 * skj[sl] + ln.a4) = u32x2{p01, p23};
            const float rs =
                sum_over_groups((lo_bf16_f32(p01) + hi_bf16_f32(p01)) + (lo_bf16_f32(p23) + hi_bf16_f32(p23)));
            if (ln.g4 == 0) lds<float>(sm, LY::rsp_off + 256 * w + 64 * sqi[sl] + ln.l4) = rs;
          }
        }
        // upper-triangle tiles read by the intra-chunk product: (0,1) and (2,3)
        if (w >= 2) lds<bf16x4>(sm, LY::a_off + 32 * (2 * w - 4) * CP + 32 * (2 * w - 3) + ln.a4) = bf16x4{};
        {
          // zacc[i] = phi(q) . z for q = 16 w + 4 g + i (every column c alike)
          f32x4 zd = zacc;
          if constexpr (GATE == GT_DECAY) {
#pragma unroll
            for (int i = 0; i < 4; ++i) zd[i] *= exp2f(float(16 * w + 4 * ln.g4 + i + 1) * lg2gam);
          }
          if (ln.c16 == 0) lds<f32x4>(sm, LY::zdp_off + 4 * (16 * w + 4 * ln.g4)) = zd;
        }
        lds_barrier();

        // ---- intra-chunk part and normalisation: O^T += V^T A^T, o = O / den
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          const int q = 16 * qt + ln.c16;
          const int ro = LY::rsp_off + 64 * qt + ln.l4;
          const float den = (((lds<float>(sm, ro) + lds<float>(sm, ro + 256)) + lds<float>(sm, ro + 512)) +
                             lds<float>(sm, ro + 768)) +
                            lds<float>(sm, LY::zdp_off + 64 * qt + ln.l4) + a.eps;
          // one correctly rounded reciprocal per row; outputs are fl(O * fl(1 / den))
          const float inv_den = 1.f / den;
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
              acc = mfma16(tr_pair(sm, LY::v_off + 2 * (32 * p2 * EP + e) + ln.tre, 8 * EP),
                           lds<bf16x8>(sm, LY::a_off + 32 * qt * CP + 64 * p2 + ln.afrag), acc);
            if (q < L) {
              bf16x4 o = pack4(acc[0] * inv_den, acc[1] * inv_den, acc[2] * inv_den, acc[3] * inv_den);
              *reinterpret_cast<bf16x4*>(a.out + (tok0 + t0 + q) * E + e + 4 * ln.g4) = o;
            }
          }
        }
      }
      lds_barrier();
    }
    favor_z_publish<R>(Z, sm, LY::zh_off, LY::zl_off, lane, w);
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
    favor_z_store<R>(Z, a.z_out + sv.st * R, lane, w);
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
  a.r_valid = p.r_valid;
  a.out = static_cast<bf16*>(p.out);
  a.cu = p.cu;
  a.slot = p.slot;
  a.nslot = p.nslot;
  a.H = p.H;
  a.n = p.n;
  a.P = p.P;
  a.seg_len = p.seg_len;
  a.eps = p.eps;
  const unsigned BH = unsigned(p.nseq) * unsigned(p.H);
  if (p.P > 1) {
    CausalArgs a1 = a;
    a1.S_out = p.ws_S;
    a1.z_out = p.ws_z;
    auto k1 = favor_segment_state<R, E, DK, GATE>;
    constexpr int lds1 = FavorSegLayout<R, E>::template bytes_dk<DK>;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(k1), hipFuncAttributeMaxDynamicSharedMemorySize, lds1) !=
        hipSuccess)
      return LA_ERR_HIP;
    LA_LAUNCH(k1, dim3(p.P - 1, BH), dim3(256), lds1, p.stream, a1);
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
    a.in_is_state = 1;
  }
  a.S_out = p.S_final;
  a.z_out = p.z_final;
  auto k3 = favor_chunk_forward<R, E, DK, GATE>;
  constexpr int lds3 = FavorFwdLayout<R, E, GATE>::template bytes_dk<DK>;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k3), hipFuncAttributeMaxDynamicSharedMemorySize, lds3) !=
      hipSuccess)
    return LA_ERR_HIP;
  LA_LAUNCH(k3, dim3(p.P, BH), dim3(256), lds3, p.stream, a);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // namespace la
