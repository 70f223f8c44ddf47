// One recurrent step of kernelized linear attention for a batch of carried
// states, in place ("Recurrent Reformulation", "Linear Attention Mechanisms"
// (dileepadev.github.io): a rank-1 update of S, an update of z, then the
// read-out; gates per "Gating and Selective State Updates"):
//
//   S' = G S + phi(k) v^T,  z' = G z + phi(k),  o = phi(q)^T S' / (phi(q)^T z' + eps)
//
// (the outer-product gate scales entry (f, e) of S by alpha_f beta_e and z by
// alpha),
// The step streams each head's r x d_v fp32 state through once (read + write),
// so it is bound by HBM bandwidth. One workgroup per (batch, head): thread
// (row group, column quad) owns float4 column quads of R/(256/(E/4)) rows, all
// loads issued before the prologue so the whole state is in flight while the
// features are computed; the read-out reduction over rows goes through LDS.
// The states may live in a pool of slots (la_forward_batch with a few tokens per
// sequence): then the head's state is slot[b] H + h, read and/or written as
// the flags say, and a slot outside the pool means a zero state, not stored.
// With m tokens per sequence the state stays in registers across the m steps,
// taken in order (each read-out sees the state after its own token), and is
// read and written once; the next token's small inputs load during a step.
#include "vec_common.hpp"

namespace la {

struct DecodeArgs {
  float* S;
  float* z;
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* gv;  // the outer-product gate's value-side input [B][H][E]
  const void* omega;
  const float* gamma;
  void* out;
  int H, in_dt, out_dt, gate;
  float eps, inv_tau;
  const int* slot;  // nullable: state index = b H + h
  int nslot, flags;  // flags: 1 read the state, 2 write it back
  int m;             // tokens per sequence ([B][H][m][.] inputs and outputs), 1 .. kMaxStepTokens
};

template <int R, int E, int DK, int FMAP, typename InT>
__global__ __launch_bounds__(256) void decode_step_kernel(DecodeArgs a) {
  constexpr int CG = E / 4;          // float4 column quads per row
  constexpr int RPP = 256 / CG;      // rows per pass
  constexpr int PASSES = R / RPP;
  __shared__ float sxq[DK], sxk[DK];
  __shared__ float spq[R], spk[R], sal[R];
  __shared__ __attribute__((aligned(16))) float sv[E];
  __shared__ __attribute__((aligned(16))) float sbeta[E];  // value-side factors (1 without the outer-product gate)
  __shared__ __attribute__((aligned(16))) float sred[RPP * E];
  __shared__ float shalf[2], sden;
  const int tid = threadIdx.x;
  const long long bh = blockIdx.x;
  const int col4 = tid % CG, r0 = tid / CG;
  const InT* q = static_cast<const InT*>(a.q);
  const InT* k = static_cast<const InT*>(a.k);
  const InT* v = static_cast<const InT*>(a.v);

  // Small per-head inputs of the first token, then the state stream, all
  // issued back to back from one basic block (clamped indices, no branches):
  // the prologue below then waits only for the small loads while the whole
  // state slice is in flight.
  const bool gla = a.gate == LA_GATE_GLA || a.gate == LA_GATE_OUTER, sel = a.gate == LA_GATE_SEL;
  const bool outer = a.gate == LA_GATE_OUTER;
  const int iq = min(tid, DK - 1), iv = min(tid, E - 1), ir = min(tid, R - 1);
  const int m = a.m;
  // token t's small inputs: q, k, v, the gate input (GLA: one per feature;
  // selective: one per head) and the outer-product gate's value side
  InT rq, rk, rv, rg, rgv;
  auto load_token = [&](int t) {
    const long long tok = bh * m + t;
    rq = q[tok * DK + iq];
    rk = k[tok * DK + iq];
    rv = v[tok * E + iv];
    const InT* gp = gla ? static_cast<const InT*>(a.g) + tok * R + ir
                        : (sel ? static_cast<const InT*>(a.g) + tok : q + tok * DK + iq);
    rg = *gp;
    rgv = outer ? static_cast<const InT*>(a.gv)[tok * E + iv] : rv;
  };
  load_token(0);
  long long si = bh;  // this head's state
  if (a.slot != nullptr) {
    const int sl = a.slot[bh / a.H];
    si = (sl >= 0 && sl < a.nslot) ? (long long)sl * a.H + bh % a.H : -1;
  }
  const bool rd = (a.flags & 1) && si >= 0, wr = (a.flags & 2) && si >= 0;
  float4* Sh = reinterpret_cast<float4*>(a.S + (si >= 0 ? si : 0) * R * E);
  float rz = 0.f;
  float4 st[PASSES];
  if (rd) {  // uniform over the workgroup: the loads stay in one block
    rz = a.z[si * R + ir];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) st[p] = Sh[(r0 + RPP * p) * CG + col4];
  } else {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) st[p] = float4{0.f, 0.f, 0.f, 0.f};
  }

  for (int t = 0; t < m; ++t) {
    const float xq = to_f32(rq), xk = to_f32(rk), xv = to_f32(rv), xg = (gla || sel) ? to_f32(rg) : 0.f;
    const float xgv = to_f32(rgv);
    if (t + 1 < m) load_token(t + 1);  // in flight during this step

    // features and gate of this token
    // unconditional (clamped) writes keep the loads above out of branches;
    // threads past the end rewrite the last element with the same value
    sxq[iq] = xq;
    sxk[iq] = xk;
    sv[iv] = xv;
    sbeta[iv] = outer ? __expf(gla_log_alpha(xgv, a.inv_tau)) : 1.f;
    __syncthreads();
    if constexpr (FMAP == 1) {
      if (tid < 2) {
        const float* x = tid == 0 ? sxq : sxk;
        float s = 0.f;
        for (int d = 0; d < DK; ++d) s += x[d] * x[d];
        shalf[tid] = 0.5f * s;
      }
      __syncthreads();
    }
    float zdot = 0.f;
    if (tid < R) {
      float pq, pk;
      if constexpr (FMAP == 0) {
        pq = elu1(xq);
        pk = elu1(xk);
      } else if constexpr (FMAP == 2) {  // the state-space form: C = q, B = k as they are
        pq = xq;
        pk = xk;
      } else {
        float aq = 0.f, ak = 0.f;
        const InT* om = static_cast<const InT*>(a.omega) + (long long)tid * DK;
        for (int d = 0; d < DK; ++d) {
          const float w = to_f32(om[d]);
          aq += w * sxq[d];
          ak += w * sxk[d];
        }
        const float isr = rsqrtf(float(R));
        pq = __expf(aq - shalf[0]) * isr;
        pk = __expf(ak - shalf[1]) * isr;
      }
      float al = 1.f;
      if (a.gate == LA_GATE_DECAY) al = a.gamma[bh % a.H];
      if (gla || sel) al = __expf(gla_log_alpha(xg, a.inv_tau));
      spq[tid] = pq;
      spk[tid] = pk;
      sal[tid] = al;
      rz = al * rz + pk;
      zdot = pq * rz;
    }
    // denominator: block reduction of phi(q) . z'
    zdot += __shfl_xor(zdot, 1);
    zdot += __shfl_xor(zdot, 2);
    zdot += __shfl_xor(zdot, 4);
    zdot += __shfl_xor(zdot, 8);
    zdot += __shfl_xor(zdot, 16);
    zdot += __shfl_xor(zdot, 32);
    if ((tid & 63) == 0) sred[tid >> 6] = zdot;
    __syncthreads();
    if (tid == 0) {
      float d = 0.f;
      for (int w = 0; w < 4; ++w) d += sred[w];
      sden = d + a.eps;
    }
    __syncthreads();

    // rank-1 update (in registers) and partial read-out over this thread's rows
    const float4 vv = reinterpret_cast<const float4*>(sv)[col4];
    const float4 bt = reinterpret_cast<const float4*>(sbeta)[col4];
    float4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = r0 + RPP * p;
      const float al = sal[r], pk = spk[r], pq = spq[r];
      float4 s = st[p];
      s.x = al * bt.x * s.x + pk * vv.x;
      s.y = al * bt.y * s.y + pk * vv.y;
      s.z = al * bt.z * s.z + pk * vv.z;
      s.w = al * bt.w * s.w + pk * vv.w;
      st[p] = s;
      o.x += pq * s.x;
      o.y += pq * s.y;
      o.z += pq * s.z;
      o.w += pq * s.w;
    }
    reinterpret_cast<float4*>(sred)[r0 * CG + col4] = o;
    __syncthreads();
    if (tid < E) {
      float acc = 0.f;
      for (int rg = 0; rg < RPP; ++rg) acc += sred[rg * E + tid];
      // the state-space read-out y = C^T h is not normalised
      st_elem(a.out, (bh * m + t) * E + tid, a.out_dt, FMAP == 2 ? acc : acc / sden);
    }
    if (t + 1 < m) __syncthreads();  // the next step rewrites the shared vectors and sred
  }
  if (wr) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) Sh[(r0 + RPP * p) * CG + col4] = st[p];
    if (tid < R) a.z[si * R + tid] = rz;
  }
}

template <int R, int E, int DK, int FMAP>
static la_status run_decode(const DecodePlan& p) {
  const bool inp = p.gate == LA_GATE_GLA || p.gate == LA_GATE_SEL || p.gate == LA_GATE_OUTER;
  DecodeArgs a{p.S,     p.z,      p.q,        p.k,          p.v,    p.g,   p.gv,
               p.omega, p.gamma,  p.out,      p.H,          p.in_dtype,   p.out_dtype,
               p.gate,  p.eps,    inp ? 1.f / p.tau : 0.f,  p.slot, p.nslot, p.flags, p.m > 0 ? p.m : 1};
  if (p.in_dtype == LA_BF16)
    LA_LAUNCH((decode_step_kernel<R, E, DK, FMAP, bf16>), dim3(unsigned(p.B) * unsigned(p.H)), dim3(256), 0,
                       p.stream, a);
  else
    LA_LAUNCH((decode_step_kernel<R, E, DK, FMAP, float>), dim3(unsigned(p.B) * unsigned(p.H)), dim3(256),
                       0, p.stream, a);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

template <int R, int DK, int FMAP>
static la_status dec_by_dv(const DecodePlan& p) {
  switch (p.dv) {
    case 32: return run_decode<R, 32, DK, FMAP>(p);
    case 64: return run_decode<R, 64, DK, FMAP>(p);
    case 128:
      if constexpr (R * 128 <= 16384) return run_decode<R, 128, DK, FMAP>(p);
      break;
  }
  return LA_ERR_UNSUPPORTED;
}

template <int R>
static la_status dec_favor_by_dk(const DecodePlan& p) {
  switch (p.dk) {
    case 32: return dec_by_dv<R, 32, 1>(p);
    case 64: return dec_by_dv<R, 64, 1>(p);
    case 128: return dec_by_dv<R, 128, 1>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

la_status launch_decode(const DecodePlan& p) {
  if (p.fmap == LA_FMAP_ELU1) {
    switch (p.dk) {
      case 32: return dec_by_dv<32, 32, 0>(p);
      case 64: return dec_by_dv<64, 64, 0>(p);
      case 128: return dec_by_dv<128, 128, 0>(p);
    }
    return LA_ERR_UNSUPPORTED;
  }
  if (p.fmap == LA_FMAP_IDENTITY) {
    switch (p.dk) {
      case 32: return dec_by_dv<32, 32, 2>(p);
      case 64: return dec_by_dv<64, 64, 2>(p);
      case 128: return dec_by_dv<128, 128, 2>(p);
    }
    return LA_ERR_UNSUPPORTED;
  }
  switch (p.r) {
    case 32: return dec_favor_by_dk<32>(p);
    case 64: return dec_favor_by_dk<64>(p);
    case 128: return dec_favor_by_dk<128>(p);
    case 256: return dec_favor_by_dk<256>(p);
  }
  return LA_ERR_UNSUPPORTED;
}

}  // namespace la
