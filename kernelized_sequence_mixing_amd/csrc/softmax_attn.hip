// Softmax attention on gfx950: the quadratic baseline that linear attention
// replaces ("Standard Self-Attention: The Quadratic Baseline", "Linear
// Attention Mechanisms", dileepadev.github.io: every query scores every key,
// a row softmax of the n x n scores weights the values; "When to Use Linear
// Attention" on the same page argues where the linear form overtakes it).
// Built to measure that crossover on this GPU at matched shapes.
//
// Flash-style: the n x n score matrix is never stored. A workgroup of four
// waves owns 128 queries (32 per wave) of one head and walks the keys in
// blocks of 64 (up to its diagonal when causal), with the running row maximum
// m and row sum l of the online softmax kept in fp32:
//   S^T = K Q^T              (bf16 MFMA, fp32; each lane holds one query's keys)
//   m' = max(m, rowmax S), p = 2^(S log2(e) scale - m'), l = 2^(m - m') l + rowsum p
//   O^T = 2^(m - m') O^T + V^T P^T   (P rounded to bf16)
// and o = O / l at the end. Computing S transposed lets each lane pass its own
// eight p values straight on as the P^T operand: the contraction over keys
// takes, in lane group g, keys 4g + 0..3 and 16 + 4g + 0..3 of each 32-key
// step, and the V^T operand is read in the same key order with the LDS
// transpose read. K and V blocks are double-buffered in LDS (one barrier per
// block); Q stays in registers.
#include "chunked.hpp"

namespace la {

struct SoftmaxArgs {
  const bf16* Q;
  const bf16* K;
  const bf16* V;
  bf16* out;
  long long heads;   // B * H
  int n;
  int nqb;           // query blocks per head
  int per_xcd;       // workgroups per XCD slot of the remapped grid
  float scale_log2;  // softmax temperature times log2(e)
  int causal;
};

constexpr int kSmQ = 128;  // queries per workgroup (32 per wave)
constexpr int kSmK = 64;   // keys per block

template <int D>
struct SmLayout {
  using FT = FeatTile<D, true>;
  static constexpr int TB = FT::BYTES;  // one [64][D] bf16 tile
  __host__ __device__ static constexpr int k_off(int buf) { return buf * 2 * TB; }
  __host__ __device__ static constexpr int v_off(int buf) { return buf * 2 * TB + TB; }
  static constexpr int bytes = 4 * TB;
};

// V^T operand of one 32-key step: lane (g, c) receives column col0 + c of
// rows r_lo + 0..3 and r_hi + 0..3 (r_lo = 32 ks + 4 g, r_hi = r_lo + 16), the
// key order of the P^T operand. Each transpose read hands the 16 lanes of a
// group column col0 + lane of a 4-row block, lane m addressing row base + m / 4
// and the 8-byte piece m % 4.
template <int D>
__device__ __forceinline__ bf16x8 tr_v_keys(const char* sm, int off, int r_lo, int r_hi, int col0, int lane) {
  using FT = FeatTile<D, true>;
  const int c16 = lane & 15, q = c16 & 3;
  const int k = col0 / 8 + (q >> 1), b = 8 * (q & 1);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sm + off + FT::at(r_lo + (c16 >> 2), k, b)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sm + off + FT::at(r_hi + (c16 >> 2), k, b)));
  return cat8(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi));
}

// Global -> registers -> LDS copy of one [64][D] key or value block (rows past
// n repeat row n - 1: their scores are masked, so they add nothing).
template <int D>
struct KvBlock {
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int PER = kSmK * CPR / 256;  // chunks per thread and tile
  bf16x8 k[PER], v[PER];
  __device__ __forceinline__ void load(const SoftmaxArgs& a, long long row0, int key0, int tid) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = tid + 256 * j, r = idx / CPR, c = idx % CPR;
      const long long row = row0 + min(key0 + r, a.n - 1);
      k[j] = *reinterpret_cast<const bf16x8*>(a.K + row * D + 8 * c);
      v[j] = *reinterpret_cast<const bf16x8*>(a.V + row * D + 8 * c);
    }
  }
  __device__ __forceinline__ void store(char* sm, int buf, int tid) const {
    using FT = FeatTile<D, true>;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = tid + 256 * j, r = idx / CPR, c = idx % CPR;
      lds<bf16x8>(sm, SmLayout<D>::k_off(buf) + FT::at(r, c)) = k[j];
      lds<bf16x8>(sm, SmLayout<D>::v_off(buf) + FT::at(r, c)) = v[j];
    }
  }
};

template <int D>
__global__ __launch_bounds__(256) void softmax_attn_forward(SoftmaxArgs a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  using FT = FeatTile<D, true>;
  using LY = SmLayout<D>;
  constexpr int KS = D / 32, DT = D / 16;
  const int lane = lane_id(), w = wave_id<4>(), tid = threadIdx.x;
  const int g4 = lane >> 4, c16 = lane & 15;

  // Grid remap: the hardware deals workgroups to the 8 XCDs round-robin by id,
  // so id -> (XCD id % 8, position id / 8) -> logical block xcd * per_xcd + pos
  // keeps consecutive logical blocks (the query blocks of one head, which read
  // the same keys and values) in one XCD's L2.
  const long long id = blockIdx.x;
  const long long logical = (id % 8) * a.per_xcd + id / 8;
  if (logical >= a.heads * a.nqb) return;
  const long long bh = logical / a.nqb;
  const int qb = a.causal ? a.nqb - 1 - int(logical % a.nqb) : int(logical % a.nqb);  // causal: longest first
  const long long row0 = bh * a.n;
  const int q0 = qb * kSmQ, qw0 = q0 + 32 * w;

  // Q^T operands: lane (g, c) holds query qw0 + 16 qt + c, columns 32 ks + 8 g .. + 7
  bf16x8 qop[2][KS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const long long row = row0 + min(qw0 + 16 * qt + c16, a.n - 1);
      qop[qt][ks] = *reinterpret_cast<const bf16x8*>(a.Q + row * D + 32 * ks + 8 * g4);
    }

  f32x4 O[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) O[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-1e30f, -1e30f}, l[2] = {0.f, 0.f};  // l: this lane's share of the row sum

  const int kend = a.causal ? min(a.n, q0 + kSmQ) : a.n;
  const int nkb = (kend + kSmK - 1) / kSmK;
  KvBlock<D> kv;
  kv.load(a, row0, 0, tid);
  kv.store(sm, 0, tid);
  lds_barrier();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    const bool more = kb + 1 < nkb;
    if (more) kv.load(a, row0, (kb + 1) * kSmK, tid);
    const int key0 = kb * kSmK;
    // a wave whose queries all precede this block has nothing to add
    if (!a.causal || key0 <= qw0 + 31) {
      // ---- S^T = K Q^T: st[kt][qt][i] = score of query 16 qt + c, key key0 + 16 kt + 4 g + i
      f32x4 st[4][2];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) st[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 kop = lds<bf16x8>(sm, LY::k_off(buf) + FT::at(16 * kt + c16, 4 * ks + g4));
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) st[kt][qt] = mfma16(kop, qop[qt][ks], st[kt][qt]);
        }
      }
      // ---- mask (causal diagonal, keys past n), online softmax in base 2
      const bool edge = (a.causal && key0 + kSmK - 1 > qw0) || key0 + kSmK > a.n;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int q = qw0 + 16 * qt + c16;
        if (edge) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = key0 + 16 * kt + 4 * g4 + i;
              if (key >= a.n || (a.causal && key > q)) st[kt][qt][i] = -INFINITY;
            }
        }
        // the row maximum of the raw scores (the temperature is positive, so it
        // commutes with the maximum and folds into the exponent's FMA below)
        float mx = -1e30f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[kt][qt][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m[qt], mx * a.scale_log2);
        const float alpha = __builtin_amdgcn_exp2f(m[qt] - mn);
        m[qt] = mn;
        float rs = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kt][qt][i], a.scale_log2, -mn));
            st[kt][qt][i] = p;
            rs += p;
          }
        l[qt] = l[qt] * alpha + rs;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[dt][qt][i] *= alpha;
      }
      // ---- O^T += V^T P^T, 32 keys per step
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        bf16x8 pb[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          pb[qt] = cat8(pack4(st[2 * ks2][qt][0], st[2 * ks2][qt][1], st[2 * ks2][qt][2], st[2 * ks2][qt][3]),
                        pack4(st[2 * ks2 + 1][qt][0], st[2 * ks2 + 1][qt][1], st[2 * ks2 + 1][qt][2],
                              st[2 * ks2 + 1][qt][3]));
        const int r_lo = 32 * ks2 + 4 * g4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8 va = tr_v_keys<D>(sm, LY::v_off(buf), r_lo, r_lo + 16, 16 * dt, lane);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) O[dt][qt] = mfma16(va, pb[qt], O[dt][qt]);
        }
      }
    }
    if (more) kv.store(sm, buf ^ 1, tid);
    lds_barrier();
  }

  // ---- o = O / l; lane (g, c) holds dims 16 dt + 4 g + i of query qw0 + 16 qt + c
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float inv = 1.f / sum_over_groups(l[qt]);
    const int q = qw0 + 16 * qt + c16;
    if (q < a.n) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<bf16x4*>(a.out + (row0 + q) * D + 16 * dt + 4 * g4) =
            pack4(O[dt][qt][0] * inv, O[dt][qt][1] * inv, O[dt][qt][2] * inv, O[dt][qt][3] * inv);
    }
  }
}

template <int D>
static la_status run_softmax(const SoftmaxPlan& p) {
  SoftmaxArgs a{};
  a.Q = static_cast<const bf16*>(p.Q);
  a.K = static_cast<const bf16*>(p.K);
  a.V = static_cast<const bf16*>(p.V);
  a.out = static_cast<bf16*>(p.out);
  a.heads = (long long)p.B * p.H;
  a.n = p.n;
  a.nqb = (p.n + kSmQ - 1) / kSmQ;
  const long long total = a.heads * a.nqb;
  a.per_xcd = int((total + 7) / 8);
  a.scale_log2 = p.scale * kLog2e;
  a.causal = p.causal;
  auto k = softmax_attn_forward<D>;
  constexpr int lds = SmLayout<D>::bytes;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, lds) !=
      hipSuccess)
    return LA_ERR_HIP;
  LA_LAUNCH(k, dim3(unsigned(8LL * a.per_xcd)), dim3(256), lds, p.stream, a);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status launch_softmax(const SoftmaxPlan& p) {
  if (p.d == 64) return run_softmax<64>(p);
  if (p.d == 128) return run_softmax<128>(p);
  return LA_ERR_UNSUPPORTED;
}

}  // namespace la
