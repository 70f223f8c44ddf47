/*
 * linattn.h -- C ABI of the MI355X (gfx950) kernelized linear attention library.
 *
 * The library computes, for every (batch b, head h) independently,
 *
 *     o_i = phi(q_i)^T S / (phi(q_i)^T z + eps),
 *     S   = sum_j phi(k_j) v_j^T   (r x d_v),   z = sum_j phi(k_j)   (r),
 *
 * ("Linear Attention Mechanisms" (dileepadev.github.io), section "The Kernel
 * Trick for Attention"; the eps added to the denominator follows the routine in
 * "Linear Attention Mechanisms" (sadullah.online), section "The linear
 * attention trick: drop or approximate the softmax").
 *
 * Non-causal: the sums run over all j. Causal: over j <= i, optionally with a
 * per-head fixed decay (S_i = gamma_h S_{i-1} + phi(k_i) v_i^T) or a per-step
 * diagonal gate on the feature axis (S_t = diag(alpha_t) S_{t-1} + phi(k_t)
 * v_t^T), where z is decayed or gated exactly like S ("Gating and Selective
 * State Updates" on the dileepadev page; "Evolution: add decay/gating" on
 * "Attention-Free / Sub-Quadratic Architectures" (blog.vguerra.net)).
 *
 * Conventions shared by every entry point:
 *   * Tensors are dense, row-major, contiguous: Q, K [B][H][n][d_k];
 *     V [B][H][n][d_v]; out [B][H][n][d_v]; state S [B][H][r][d_v] fp32;
 *     normaliser z [B][H][r] fp32; GLA gate input g [B][H][n][r].
 *   * Every tensor pointer is a DEVICE pointer owned by the caller, 16-byte
 *     aligned. The library allocates no memory and keeps no state between
 *     calls; scratch memory is passed in as `workspace`.
 *   * Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream). Argument errors are returned synchronously before anything is
 *     launched; LA_ERR_HIP means the HIP runtime refused a launch. Faults of
 *     the device surface at the caller's next synchronisation.
 *   * NaN or Inf in the inputs propagate to the outputs; they are not checked.
 *   * Results are deterministic: no atomics, fixed reduction orders.
 *   * Functions are re-entrant; concurrent calls on different streams are
 *     safe when their output and workspace buffers do not overlap.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_ABI_VERSION 7

typedef enum la_status {
  LA_OK = 0,
  LA_ERR_INVALID_ARG = 1, /* NULL/misaligned pointer, bad size or enum, eps < 0, tau <= 0 */
  LA_ERR_UNSUPPORTED = 2, /* well-formed but outside the built set (dims, dtype mix) */
  LA_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than la_forward_workspace_size */
  LA_ERR_ALIAS = 4,       /* an output overlaps an input or another output */
  LA_ERR_HIP = 5          /* the HIP runtime reported an error for a launch */
} la_status;

typedef enum la_dtype { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

/*
 * Feature maps ("Choosing the Feature Map phi", dileepadev page):
 *   ELU1     : phi(x) = elu(x) + 1 elementwise (r == d_k).
 *   FAVOR    : phi(x)_m = exp(w_m . x - |x|^2 / 2) / sqrt(r), m = 0..r-1, the
 *              positive random features whose inner product estimates
 *              exp(q . k); omega [r][d_k] holds the rows w_m.
 *   IDENTITY : the state-space form ("State Space Models as Linear Attention",
 *              dileepadev page: h_t = A_t h_{t-1} + B_t x_t, y_t = C_t^T h_t):
 *              q = C and k = B enter unchanged and the read-out is NOT
 *              normalised, o_i = q_i^T S_i (z is still carried as the state's
 *              column of a constant-1 value and returned in z_final, but not
 *              read); causal only, r = d_k, gates as for ELU1 (the GLA gate is
 *              the selective, input-dependent diagonal A_t).
 */
typedef enum la_fmap_kind { LA_FMAP_ELU1 = 0, LA_FMAP_FAVOR = 1, LA_FMAP_IDENTITY = 2 } la_fmap_kind;

/*
 * Gates of the causal forms: the multiplier of the previous state at each step
 * ("Gating and Selective State Updates", dileepadev page; "Evolution: add
 * decay/gating", vguerra page). z is gated exactly like S unless stated.
 *   NONE  : S_t = S_{t-1} + phi(k_t) v_t^T.
 *   DECAY : S_t = gamma_h S_{t-1} + phi(k_t) v_t^T (RetNet's fixed decay).
 *   GLA   : S_t = diag(alpha_t) S_{t-1} + phi(k_t) v_t^T, a per-feature,
 *           input-dependent alpha_t = sigmoid(g_t)^(1/tau), g [B][H][n][r].
 *   SEL   : the scalar selective gate, one input-dependent
 *           a_t = sigmoid(g_t)^(1/tau) per step and head shared by all
 *           features, g [B][H][n] (decode: [B][H]): the RetNet decay made
 *           input-dependent, the selective recurrence of Mamba's kind ("State
 *           Space Models as Linear Attention", dileepadev page).
 *   OUTER : S_t = (alpha_t beta_t^T) * S_{t-1} + phi(k_t) v_t^T (elementwise):
 *           the gate matrix G_t in (0, 1)^{d x d} as the outer product of the
 *           key-side alpha_t of GLA (input g) and a value-side
 *           beta_t = sigmoid(gv_t)^(1/tau) per value column (input gv
 *           [B][H][n][d_v], decode [B][H][d_v]); z_t = alpha_t * z_{t-1} +
 *           phi(k_t) (the key side only).
 * GLA, SEL and OUTER take elementwise feature maps only.
 */
typedef enum la_gate_kind {
  LA_GATE_NONE = 0,
  LA_GATE_DECAY = 1,
  LA_GATE_GLA = 2,
  LA_GATE_SEL = 3,
  LA_GATE_OUTER = 4
} la_gate_kind;

typedef struct la_problem {
  int32_t B, H;      /* batch, heads: >= 1 */
  int32_t n;         /* sequence length: >= 1 (== 1 for la_decode_step) */
  int32_t d_k, d_v;  /* key/query and value widths */
  int32_t in_dtype;  /* la_dtype of Q, K, V, g and omega */
  int32_t out_dtype; /* la_dtype of out */
  float eps;         /* added to every denominator; finite and >= 0 */
} la_problem;

typedef struct la_feature_map {
  int32_t kind;      /* la_fmap_kind */
  int32_t r;         /* feature dimension; must equal d_k for ELU1 */
  const void* omega; /* FAVOR: device [r][d_k] in in_dtype. ELU1: must be NULL */
} la_feature_map;

typedef struct la_gate {
  int32_t kind;       /* la_gate_kind */
  float tau;          /* GLA, SEL, OUTER temperature, > 0 (ignored otherwise) */
  const float* gamma; /* DECAY: device [H] fp32, each in (0, 1] -- a documented
                         precondition, not checked (the values live on the device) */
  const void* g;      /* GLA, OUTER: device [B][H][n][r] in in_dtype (decode: [B][H][r]);
                         SEL: [B][H][n] (decode: [B][H]). Precondition of the chunked
                         causal kernels (la_forward, la_forward_batch with more than
                         16 tokens per sequence, la_backward) for GLA and OUTER, not
                         checked since g lives on the device: within every 64-token
                         chunk (tokens 64c .. 64c + 63 of each sequence) the summed
                         log alpha of each feature stays at or above -80. The
                         chunk's factors e^{+b}, e^{-b} are referenced to the chunk
                         start and stay finite in fp32 and bf16 there; below it the
                         outputs may be Inf or NaN. la_decode_step, batch steps of
                         up to 16 tokens and SEL have no such limit (SEL forms each factor
                         as e^{b_i - b_j} <= 1). */
  const void* gv;     /* OUTER: device [B][H][n][d_v] in in_dtype (decode: [B][H][d_v]),
                         with the same precondition per value column (summed
                         log beta); must be NULL
                         for every other gate (else LA_ERR_INVALID_ARG) */
} la_gate;

/* Flags of la_batch.flags. */
#define LA_SLOT_READ 1  /* each sequence starts from the state in its slot (else from zero) */
#define LA_SLOT_WRITE 2 /* each sequence's state after its last token is stored in its slot */

/*
 * A serving batch for la_forward_batch: independent causal sequences, each
 * bound to a slot of a caller-owned state pool (the recurrent state that
 * replaces a growing KV cache: "Recurrent Reformulation", dileepadev page;
 * inference throughput, "Linear Attention Mechanisms", sadullah page).
 */
typedef struct la_batch {
  const int32_t* cu_seqlens; /* NULL: p->B sequences of p->n tokens ([B][H][n][.] layout).
                                Else device [num_seqs + 1] token offsets along n, with
                                p->B == 1: sequence b is tokens cu[b] .. cu[b+1] - 1 of
                                the [1][H][n][.] tensors (packed, no padding). */
  int32_t num_seqs;          /* number of sequences; must be p->B without cu_seqlens */
  int32_t max_seqlen;        /* with cu_seqlens: an upper bound of every sequence's length,
                                1 <= max_seqlen <= p->n (used for planning); without: p->n */
  float* S;                  /* state pool: device fp32 [num_slots][H][r][d_v]; read and/or
                                written in place; may be NULL when flags == 0 */
  float* z;                  /* device fp32 [num_slots][H][r] */
  const int32_t* slot_ids;   /* device [num_seqs]: the slot of each sequence */
  int32_t num_slots;         /* >= 1 when flags != 0 */
  int32_t flags;             /* LA_SLOT_READ | LA_SLOT_WRITE, or 0 */
} la_batch;

/* ABI version of the loaded library (LA_ABI_VERSION at build time). */
int32_t la_abi_version(void);

/* Static, human-readable name of a status code. */
const char* la_status_str(int32_t status);

/*
 * Bytes of device workspace la_forward needs for this problem (0 if none).
 * Pure host computation: no HIP call is made. Same validation as la_forward
 * (pointer fields of fmap/gate are not inspected).
 */
la_status la_forward_workspace_size(const la_problem* p, const la_feature_map* fmap,
                                    int32_t causal, const la_gate* gate, size_t* bytes);

/*
 * How la_forward splits each head's sequence for the causal form: *segments
 * contiguous pieces of *segment_len tokens (the last may be shorter), each a
 * multiple of the 64-token chunk. Pure host computation; 1 for non-causal.
 */
la_status la_forward_segments(const la_problem* p, const la_feature_map* fmap,
                              int32_t causal, const la_gate* gate,
                              int32_t* segments, int32_t* segment_len);

/*
 * Full-sequence forward pass.
 *   Q, K, V       inputs (in_dtype), layouts above.
 *   fmap          feature map; gate: may be NULL (= NONE); must be NONE when causal == 0.
 *   causal        0: sums over all j ("The linear attention trick", sadullah page);
 *                 1: sums over j <= i ("Recurrent Reformulation", dileepadev page).
 *   S0, z0        optional initial state carried in (causal only; both or neither;
 *                 NULL = zero), fp32 [B][H][r][d_v] and [B][H][r].
 *   S_final, z_final  optional (both or neither): the state after the last
 *                 token (for non-causal, the full sums S and z), fp32.
 *   out           [B][H][n][d_v] in out_dtype; must not overlap any input.
 *   workspace     device scratch of at least la_forward_workspace_size bytes
 *                 (may be NULL when that size is 0), 256-byte aligned.
 * Supported (else LA_ERR_UNSUPPORTED):
 *   causal: in_dtype BF16, out_dtype BF16; d_v in {32,64,128}; ELU1 or IDENTITY with
 *           d_k in {32,64,128} and any gate; FAVOR with d_k in {32,64,128},
 *           r in {32,64,128,256}, gate NONE or DECAY; r * d_v <= 16384.
 *           d_v = 32 runs the 64-column kernels on copies whose rows are 64
 *           wide (columns 32..63 zero) of V, gate->gv, out, S0 and S_final, held
 *           in the workspace (counted by la_forward_workspace_size), and
 *           copies the 32 real columns back: results equal the d_v = 64
 *           problem with zero-padded values, column for column. FAVOR r = 32
 *           likewise runs the 64-feature kernels on omega zero-padded to 64
 *           rows, the features past 32 masked to zero and the map's 1/sqrt(r)
 *           taken at r = 32, with S0, z0, S_final, z_final padded and copied
 *           back alike: the result is the r = 32 map's.
 *   non-causal: in/out dtype F32 or BF16 (any mix); d_k in {32,64,128},
 *           d_v in {32,64,128}; FAVOR r in {32,64,128,256}; r * d_v <= 16384.
 * Numerics: bf16 MFMA products with fp32 accumulation; the state, normaliser,
 * gate factors and every denominator are fp32. The causal kernels normalise
 * each output row by one correctly rounded fp32 reciprocal of its denominator
 * and a multiply, out = fl(num * fl(1 / den)); the non-causal kernels divide,
 * out = fl(num / den) (IEEE fp32).
 */
la_status la_forward(const la_problem* p, const void* Q, const void* K, const void* V,
                     const la_feature_map* fmap, int32_t causal, const la_gate* gate,
                     const float* S0, const float* z0, float* S_final, float* z_final,
                     void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace la_forward_batch needs. Pure host computation,
 * same validation as la_forward_batch (device pointers not inspected).
 */
la_status la_forward_batch_workspace_size(const la_problem* p, const la_batch* batch,
                                          const la_feature_map* fmap, const la_gate* gate,
                                          size_t* bytes);

/*
 * The causal forward pass over a serving batch of sequences (see la_batch):
 * a ragged prefill (cu_seqlens) or a step of m tokens for each of B
 * sequences (multi-token decode; m = p->n), each sequence continuing from
 * and/or storing its state in its slot. Per sequence the result is that of
 * la_forward(causal = 1) on that sequence alone with S0 = its slot's state
 * (LA_SLOT_READ) and S_final = its slot (LA_SLOT_WRITE); the slots are updated
 * in place, after every read of them.
 *   Q, K, out, gate->g, gate->gv as la_forward on the [B][H][n][.] tensors (B = 1 with
 *   cu_seqlens); fmap, gate as la_forward; out: tokens no sequence covers are
 *   left untouched.
 * Device-side contents are not validated on the host; the kernels clamp them
 * so that no access leaves the buffers: each sequence's bounds are clamped
 * into [0, n] (an end below its start gives an empty sequence), lengths
 * above max_seqlen are cut to the planned capacity (tokens past it get no
 * output), and a slot id outside [0, num_slots) means that sequence starts
 * from zero and stores no state. Overlapping sequences give unspecified
 * outputs for the shared tokens.
 * Slot ids must be distinct within a call when LA_SLOT_WRITE is set (two
 * sequences writing one slot race).
 * A step of up to 16 tokens per sequence (no cu_seqlens, p->n <= 16) runs the
 * recurrent step of la_decode_step once per token, in order, on the slots (fp32
 * arithmetic; each state is read and written once, held in registers across
 * the tokens); longer steps and prefills run the chunked kernels.
 * A ragged batch is planned from p->n and max_seqlen (the lengths stay on the
 * device): segments sized for about one round of workgroups over all
 * sequences, as many as the longest sequence needs.
 * Supported: as la_forward with causal == 1, except d_v = 32 and FAVOR r = 32,
 * which only steps of up to 16 tokens take (LA_ERR_UNSUPPORTED otherwise).
 * Errors: LA_ERR_INVALID_ARG for a
 * malformed batch (num_seqs, max_seqlen, flags, B != 1 with cu_seqlens, NULL
 * pool pointers with flags set); LA_ERR_ALIAS when out, the pool or the
 * workspace overlap an input or each other. The library allocates nothing.
 */
la_status la_forward_batch(const la_problem* p, const la_batch* batch, const void* Q, const void* K,
                           const void* V, const la_feature_map* fmap, const la_gate* gate,
                           void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace la_backward needs for this problem. Pure host
 * computation, same validation as la_backward (pointer fields not inspected).
 */
la_status la_backward_workspace_size(const la_problem* p, const la_feature_map* fmap,
                                     int32_t causal, const la_gate* gate, size_t* bytes);

/*
 * Gradients of the forward pass, for training with the parallel form
 * ("Recurrent Reformulation", dileepadev page: trained in parallel, run as an
 * RNN). For a loss L with dL/dout = dO, writes dQ = dL/dQ, dK = dL/dK and
 * dV = dL/dV of la_forward(p, Q, K, V, fmap, 1, gate, S0, z0, ...):
 *   g_i = dO_i / den_i,  h_i = -(dO_i . o_i) / den_i,  dW_ij = g_i . v_j + h_i,
 *   dphi(q_i) = sum_{j<=i} dW_ij G_ij phi(k_j) (+ the carried state's share),
 *   dphi(k_j) = sum_{i>=j} dW_ij G_ij phi(q_i),  dv_j = sum_{i>=j} w_ij g_i,
 * with G_ij = 1 or gamma_h^(i-j) and w_ij = phi(q_i).phi(k_j) G_ij, then the
 * feature map's derivative (elu+1: 1 for x > 0, exp(x) below). With the GLA
 * gate ("Gating and Selective State Updates", dileepadev page) the weights
 * G_ij are per feature, prod_{u=j+1..i} alpha_u, and the gate's raw input g
 * also gets its gradient: with B_t = sum_{u<=t} log alpha_u,
 *   dB_t = dphi(q_t) * phi(q_t) - dphi(k_t) * phi(k_t)   (per feature),
 *   dg_u = (sum_{t>=u} dB_t) * sigmoid(-g_u) / tau.
 * The selective scalar gate is that gate with alpha_t = a_t on every feature,
 * so its dg_t is the sum over features of the per-feature dg_t (the library
 * runs the GLA passes with each token's one input used for every feature and
 * sums their dg over features in a fixed order).
 * The outer-product gate G_t = alpha_t beta_t^T adds a value-side factor
 * beta_t = sigmoid(gv_t)^(1/tau) per column (z takes the key side only):
 * with C_t = sum_{u<=t} log beta_u, the pairs carry exp(C_i - C_j) per value
 * column, dg follows the GLA rule, and
 *   dC_t = dO_t * o_t - dV_t * v_t   (per column),
 *   dgv_u = (sum_{t>=u} dC_t) * sigmoid(-gv_u) / tau.
 *   Q, K, dQ, dK [B][H][n][d_k]; V, dO, dV [B][H][n][d_v]; all BF16 (in_dtype and
 *   out_dtype must be BF16). S0, z0: the optional carried-in state of the forward
 *   (both or neither; fp32). gamma and tau are constants: no gradient is returned
 *   for them, nor for S0, z0.
 *   dg: the gradient of gate->g, BF16 in its shape ([B][H][n][r] for GLA and
 *   OUTER, [B][H][n] for SEL); required (non-NULL) with those gates and must be
 *   NULL otherwise (else LA_ERR_INVALID_ARG).
 *   dgv: the gradient of gate->gv, BF16 [B][H][n][d_v]; required with OUTER and
 *   must be NULL otherwise (else LA_ERR_INVALID_ARG).
 *   workspace: device scratch of at least la_backward_workspace_size bytes,
 *   256-byte aligned (segment states of both directions, g and h per token;
 *   GLA, SEL and OUTER: also dQ~ . Q~ per token and feature and per-segment
 *   summed log-gates; OUTER: also dO * o per token and value column (fp32)
 *   and per-segment summed value-side log-gates).
 * causal == 0 (the non-causal form, "The linear attention trick", sadullah
 * page: dphi(q_i) = S g_i + z h_i, dphi(k_j) = G v_j + hq, dv_j = G^T phi(k_j)
 * with G = sum_i phi(q_i) g_i^T, hq = sum_i phi(q_i) h_i): ELU1, no gate, no
 * S0/z0 (else LA_ERR_INVALID_ARG), in_dtype == out_dtype in {F32, BF16} with
 * the gradients in that dtype, the forward's (d_k, d_v) set; fp32 arithmetic.
 * Supported (else LA_ERR_UNSUPPORTED) for causal == 1: ELU1 or IDENTITY (the
 * state-space read-out: g_i = dO_i, h_i = 0, phi' = 1), gate NONE, DECAY, GLA,
 * SEL or OUTER, (d_k, d_v) in {(64, 64), (64, 128), (128, 64), (128, 128)}
 * (128 x 128 runs as two 64-column value halves); FAVOR ("Choosing the Feature
 * Map phi", dileepadev page) with gate NONE or DECAY, d_k in {32, 64, 128},
 * r in {64, 128}, (r, d_v) in the same set: phi(Q), phi(K) are materialised in
 * bf16 in the workspace, the passes above give dphi, and
 *   dx = sum_m dphi_m phi_m (w_m - x)
 * takes it back through the map (fp32, omega as given). Outputs must not overlap the
 * inputs, each other or the workspace (LA_ERR_ALIAS). Numerics as la_forward:
 * bf16 MFMA operands (phi, values, g, the scores and dW), fp32 accumulation,
 * states, denominators and the sums behind dg and dgv. OUTER has the forward's
 * gate-input precondition (the summed log alpha and log beta of every 64-token
 * chunk at or above -80).
 */
la_status la_backward(const la_problem* p, const void* Q, const void* K, const void* V,
                      const void* dO, const la_feature_map* fmap, int32_t causal,
                      const la_gate* gate, const float* S0, const float* z0, void* dQ,
                      void* dK, void* dV, void* dg, void* dgv, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * One recurrent step for a batch of carried states, updated IN PLACE
 * ("Recurrent Reformulation", dileepadev page: rank-1 update of S, update of
 * z, then the read-out):
 *   S' = G S + phi(k) v^T,  z' = G z + phi(k),  out = phi(q)^T S' / (phi(q)^T z' + eps)
 * with G = 1, gamma_h or diag(alpha).
 *   p->n must be 1; q, k [B][H][d_k], v [B][H][d_v], gate->g [B][H][r] (in_dtype);
 *   S [B][H][r][d_v] fp32 and z [B][H][r] fp32 are read and overwritten;
 *   out [B][H][d_v] in out_dtype.
 * Supported: in_dtype F32 or BF16, out_dtype F32 or BF16; ELU1 or IDENTITY with
 * d_k in {32,64,128}; FAVOR d_k in {32,64,128}, r in {32,64,128,256}; any gate;
 * d_v in {32,64,128}; r * d_v <= 16384. fp32 arithmetic; out = fl(num / den).
 */
la_status la_decode_step(const la_problem* p, float* S, float* z, const void* q,
                         const void* k, const void* v, const la_feature_map* fmap,
                         const la_gate* gate, void* out, void* stream);

/*
 * The feature map alone: out[i][m] = phi(X[i])_m in fp32 for `rows` rows of
 * width d_k ("Choosing the Feature Map phi", dileepadev page).
 *   X [rows][d_k] in in_dtype; out [rows][r] fp32. Same d_k / r sets as above;
 *   IDENTITY gives LA_ERR_UNSUPPORTED (nothing to apply).
 */
la_status la_feature_map_apply(const la_feature_map* fmap, int64_t rows, int32_t d_k,
                               int32_t in_dtype, const void* X, float* out, void* stream);

/*
 * Softmax attention, the quadratic baseline that linear attention replaces
 * ("Standard Self-Attention: The Quadratic Baseline", dileepadev page: every
 * query scores every key and a row softmax of the n x n scores weights the
 * values), for measuring where the linear forms overtake it ("When to Use
 * Linear Attention", same page):
 *   o_i = sum_j softmax_j(scale q_i . k_j) v_j  over j <= i (causal) or all j.
 *   Q, K, V, out [B][H][n][d] BF16 (in_dtype and out_dtype BF16, d = d_k = d_v
 *   in {64, 128}, else LA_ERR_UNSUPPORTED); scale > 0 and finite (1/sqrt(d) is
 *   the usual temperature); eps is not used.
 * The n x n scores are never stored: they are formed block by block (64 keys
 * at a time) on bf16 MFMA with fp32 accumulation, with the online softmax's
 * running maximum and row sums in fp32 and the weights rounded to bf16 for the
 * weighted sum. out must not overlap the inputs (LA_ERR_ALIAS). No workspace.
 */
la_status la_softmax_attention(const la_problem* p, const void* Q, const void* K, const void* V,
                               int32_t causal, float scale, void* out, void* stream);

/*
 * la_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid allocation). Arguments, results and errors are those of
 * la_forward; the scratch memory la_forward would take as `workspace` is a
 * fixed device array of LA_NOALLOC_SCRATCH_BYTES inside the library instead,
 * one per GPU, held until the process ends. A problem whose
 * la_forward_workspace_size exceeds that size returns LA_ERR_WORKSPACE (use
 * la_forward with a workspace). Nothing is allocated, not even on the first
 * call on a device (which only looks up the array's address). Every call on
 * one GPU uses the same array: calls that overlap in time on one GPU (other
 * streams, other host threads) race and give undefined results; calls in
 * stream order are safe (no part of the array needs to be cleared).
 */
#define LA_NOALLOC_SCRATCH_BYTES (32u << 20)
la_status la_forward_noalloc(const la_problem* p, const void* Q, const void* K, const void* V,
                             const la_feature_map* fmap, int32_t causal, const la_gate* gate,
                             const float* S0, const float* z0, float* S_final, float* z_final,
                             void* out, void* stream);

/*
 * Launch timing, for profiling (computes nothing). la_timing_begin opens a
 * bracket on the calling host thread; until la_timing_end on the same thread,
 * every kernel launch the library makes first records events[i] on its stream
 * (hipEventRecord; i counts the bracket's launches from 0). la_timing_end
 * records events[launches] on `stream` and returns the number of launches in
 * *launches (may be NULL), so hipEventElapsedTime(events[i], events[i + 1]) is
 * the time of launch i on an otherwise idle stream. The events are the
 * caller's hipEvent_t handles (created with timing enabled), at least
 * launches + 1 of them; launches past n_events - 1 are counted, not recorded.
 * Errors: LA_ERR_INVALID_ARG for a NULL event, n_events < 0, a bracket already
 * open (begin) or none open (end); LA_ERR_HIP from la_timing_end if any record
 * failed. The entry points called inside the bracket behave as always.
 */
la_status la_timing_begin(void* const* events, int32_t n_events);
la_status la_timing_end(void* stream, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
