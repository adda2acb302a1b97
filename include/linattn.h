/*
 * linattn.h -- causal linear attention with a fixed-size running state, on
 * AMD Instinct MI355X (gfx950).  Plain C ABI: device pointers, sizes and
 * status codes; no allocation, no synchronisation, no host<->device copies.
 *
 * What is computed (see the three pages this library follows):
 *   [lesson] efficient-attention lesson "Linear attention", Researcher level,
 *            "Derivation": o_i = sum_{j<=i} sim(q_i,k_j) v_j / sum_{j<=i} sim(q_i,k_j)
 *            with sim(q,k) = phi(q)^T phi(k), regrouped into the recurrence
 *            S_i = S_{i-1} + phi(k_i) v_i^T,  z_i = z_{i-1} + phi(k_i),
 *            o_i = S_i^T phi(q_i) / (z_i^T phi(q_i)).
 *   [kb]     llm-arch-kb "Linear Attention", section 2 "Derivation" (causal
 *            recurrence: the state (S, z) is an RNN hidden state of size
 *            d'(d_h + 1)) and section 3 "Reference implementation" (eps = 1e-6
 *            is added to the denominator).
 *   [card]   wikillm "Linear attention", "Implementation sketch" (optional
 *            per-token scalar decay a_t multiplies the old state and the old
 *            normaliser; decay 1 is the plain causal case, per "Decaying linear
 *            attention with a scalar state (SSD)") and "Variants / Random
 *            Fourier features (RFA)" (Gaussian random projections as the
 *            feature map; a sigmoid gate g decays the old state and scales the
 *            new term by 1 - g) and "Variants / Matrix memory with
 *            exponential gates (mLSTM)" (forget gate f, exponential input gate
 *            i, read-out divided by max(|n^T q|, 1), a stabiliser state against
 *            overflow; "Implementation sketch": the mLSTM step is this loop
 *            with the identity feature map).
 *
 * Per (batch b, head h), for t = 0 .. T-1:
 *   S <- alpha_t S + beta_t phi(k_t) v_t^T          S: d' x d_v, fp32
 *   z <- alpha_t z + beta_t phi(k_t)                z: d',       fp32
 *   o_t = (phi(q_t)^T S) / (phi(q_t)^T z + eps)     read-out after the update
 * with (alpha, beta) = (1, 1) for LA_DECAY_NONE, (a_t, 1) for LA_DECAY_SSD,
 * (g_t, 1 - g_t) for LA_GATE_RFA and (f_t, i_t) for LA_GATE_MLSTM; with
 * LA_NORM_NONE the read-out is the numerator alone, o_t = phi(q_t)^T S, and
 * with LA_NORM_MAX1 it is phi(q_t)^T S / max(|phi(q_t)^T z|, 1).
 *
 * mLSTM gates (LA_GATE_MLSTM): `decay` holds the forget-gate pre-activations
 * and `igate` the input-gate pre-activations; f_t = sigmoid(decay_t) (or
 * exp(decay_t) with fgate_exp = 1) and i_t = exp(igate_t).  The page gives
 * no formula for the stabiliser; this library keeps a per-(b, h) log-domain
 * running maximum
 *   m_t = max(log f_t + m_{t-1}, igate_t)
 * in desc->stab and stores the state scaled by e^{-m}: S and z hold
 * e^{-m_t} times the sums above (every factor applied is <= 1, so nothing
 * overflows), and the read-outs are evaluated as the same numbers, e.g.
 * phi(q)^T S / max(|phi(q)^T z|, e^{-m_t}) for LA_NORM_MAX1.  A zero state
 * (la_state_init) has m = 0.
 *
 * Feature maps:
 *   LA_PHI_ELU1: phi(x) = elu(x) + 1 (alpha = 1), element-wise, d' = d_h.
 *   LA_PHI_RFF:  phi(x) = D^{-1/2} [sin(W_h x); cos(W_h x)], W_h = rff_W[h]
 *                (D x d_h, fp32), d' = 2 D; features 0..D-1 are the sines,
 *                D..2D-1 the cosines.  No q/k scaling is applied.
 *   LA_PHI_IDENTITY: phi(x) = x, d' = d_h (the mLSTM step).
 *
 * Layouts (all row-major, contiguous, device memory, 16-byte aligned):
 *   prefill q, k [B, H, T, d_h]; v, out [B, H, T, d_v]; decay, igate [B, H, T] fp32
 *   decode  q, k [B, H, d_h];    v, out [B, H, d_v];    decay, igate [B, H]    fp32
 *   state   S [B, H, d', d_v] fp32; z [B, H, d'] fp32; stab [B, H] fp32 (mLSTM)
 * (for decode, B is the number of sequences).  q, k and v share one element
 * type (dtype); out is either dtype or fp32 (out_dtype).  Arithmetic is fp32
 * (MFMA operands bf16 for 16-bit inputs, with the intra-chunk scores split
 * into a bf16 high and low part), the state is fp32, and a 16-bit out is
 * rounded to nearest even.  Because outputs shrink like 1/sqrt(t) over long
 * sequences while early ones stay O(1), a 16-bit out carries rounding far
 * above 1e-2 of the output RMS at T ~ 1e5; fp32 out does not.
 *
 * Ownership and threading: the caller owns every buffer.  The library keeps no
 * state between calls, allocates nothing, never synchronises, and enqueues all
 * work on the caller's stream (a hipStream_t passed as void*; NULL is the null
 * stream).  Calls are thread-safe.  Buffers must not overlap, except that S
 * and z are read and written in place.
 *
 * Errors: every argument is validated on the host before anything is
 * enqueued, so a call that returns LA_EINVAL or LA_EUNSUPPORTED has had no
 * effect.  LA_EHIP means a launch failed (hipGetLastError after enqueue).
 * la_last_error() gives a human-readable reason for the calling thread's most
 * recent failure.  Non-finite values in the data are not errors: a zero
 * denominator (possible with RFF features, which can be negative) yields
 * inf/NaN outputs, as the recurrence would.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LA_OK = 0,
  LA_EINVAL = 1,        /* bad argument: NULL, size, alignment, workspace too small */
  LA_EUNSUPPORTED = 2,  /* valid but not implemented (e.g. d' or d_v too large)    */
  LA_EHIP = 3           /* a HIP launch failed                                    */
} la_status;

typedef enum { LA_F32 = 0, LA_BF16 = 1, LA_F16 = 2 } la_dtype;

typedef enum { LA_PHI_ELU1 = 0, LA_PHI_RFF = 1, LA_PHI_IDENTITY = 2 } la_phi;

typedef enum {
  LA_DECAY_NONE = 0,  /* alpha = 1,   beta = 1                          */
  LA_DECAY_SSD = 1,   /* alpha = a_t, beta = 1      (a_t >= 0 expected)  */
  LA_GATE_RFA = 2,    /* alpha = g_t, beta = 1 - g_t                     */
  LA_GATE_MLSTM = 3   /* alpha = f_t, beta = i_t = exp(igate_t), state
                         stabilised (see above)                          */
} la_decay;

typedef enum {
  LA_NORM_SUM = 0,    /* o_t = phi(q_t)^T S / (phi(q_t)^T z + eps)            */
  LA_NORM_NONE = 1,   /* o_t = phi(q_t)^T S: the normaliser is left out of the
                         read-out ([card] "Decaying linear attention with a
                         scalar state (SSD)": the normaliser-free form, which
                         relies on a normalisation layer after the read-out).
                         z is still carried and updated, so a state can move
                         between the two forms.                            */
  LA_NORM_MAX1 = 2    /* o_t = phi(q_t)^T S / max(|phi(q_t)^T z|, 1), the
                         mLSTM read-out ([card] Variants / mLSTM); eps is
                         not used                                          */
} la_norm;

typedef struct la_desc {
  int B;                 /* batch (prefill) or number of sequences (decode), >= 1 */
  int H;                 /* heads, >= 1                                           */
  int T;                 /* tokens per sequence (prefill only), >= 0              */
  int d_h;               /* query/key width, >= 1                                 */
  int d_v;               /* value width, >= 1                                     */
  la_dtype dtype;        /* element type of q, k and v                            */
  la_dtype out_dtype;    /* element type of out: dtype, or LA_F32 for any dtype   */
  la_phi phi;            /* feature map                                           */
  int rff_D;             /* RFF pairs (d' = 2 rff_D); 0 for ELU1 and IDENTITY     */
  const float* rff_W;    /* device [H, rff_D, d_h] fp32; NULL for ELU1, IDENTITY  */
  la_decay decay_kind;   /* decay / gate kind                                     */
  const float* decay;    /* device fp32 a_t, g_t or the mLSTM forget-gate
                            pre-activations; NULL iff LA_DECAY_NONE          */
  float eps;             /* added to the denominator (finite); 1e-6 on the pages  */
  int chunk;             /* prefill chunk length, 0 = default (32); 32/64/128     */
  int segments;          /* prefill segments per (b, h), 0 = automatic            */
  la_norm norm;          /* read-out form, LA_NORM_SUM (0) by default             */
  int noncausal;         /* prefill only: 0 = causal (default); 1 = non-causal,
                            every output reads the state of the whole sequence
                            (see la_prefill); needs LA_DECAY_NONE             */
  const float* igate;    /* LA_GATE_MLSTM: device fp32 input-gate
                            pre-activations, shaped like decay; else NULL   */
  int fgate_exp;         /* LA_GATE_MLSTM: forget gate f = sigmoid(decay) (0)
                            or exp(decay) (1); else 0                        */
  float* stab;           /* LA_GATE_MLSTM: device fp32 stabiliser m [B, H],
                            read and written in place like S and z; else NULL */
} la_desc;

/* Feature dimension d' of a descriptor (d_h for ELU1 and IDENTITY, 2 rff_D
 * for RFF), or -1 if the descriptor is invalid.  Host only. */
int la_feature_dim(const la_desc* desc);

/* Zero the state: S [B, H, d', d_v] and z [B, H, d'] (fp32) become 0, the
 * initial state of the recurrence ([kb] section 3: S and z start at zero);
 * with LA_GATE_MLSTM the stabiliser desc->stab [B, H] becomes 0 too.
 * Enqueued on `stream`. */
la_status la_state_init(const la_desc* desc, float* S, float* z, void* stream);

/* Bytes of device workspace la_prefill needs for `desc` (may be 0).  Host
 * only; depends on B, H, T, d', d_v, chunk and segments alone. */
la_status la_prefill_workspace_size(const la_desc* desc, size_t* bytes);

/* Execution plan la_prefill will use for `desc`: chunk length, segments per
 * (b, h), and path (1 = chunked MFMA for d' = d_v in {64, 128}: elu+1 with
 * no decay, SSD decay or the RFA gate and bf16 or fp16 inputs, or the
 * identity map with the mLSTM gates and bf16 inputs; 0 = general per-token
 * kernel).  Host only. */
la_status la_prefill_plan(const la_desc* desc, int* chunk, int* segments, int* path);

/* Causal prefill over T tokens for all (b, h):
 *   in:  q, k, v (dtype), decay/gate and rff_W through desc, the initial
 *        state (S, z, and desc->stab with mLSTM gates) -- the recurrence
 *        continues from it ([kb] section 2: the state is carried between
 *        steps);
 *   out: out [B, H, T, d_v] (out_dtype) and the final state written over
 *        (S, z) (and desc->stab).
 * The result equals T applications of the recurrence above; the chunked
 * schedule re-brackets the same sums ([lesson] Researcher level,
 * "Implementation reality": quadratic inside chunks, a scan across them).
 * `workspace` must hold la_prefill_workspace_size() bytes (NULL if 0).
 * T = 0 is a no-op.
 * With desc->noncausal = 1 the prefill is the non-causal form ([kb] section
 * 3, non-causal sketch; [lesson] Developer level, the phi(Q) (phi(K)^T V)
 * bracketing): the state first takes in all T tokens, S <- S + sum_t
 * phi(k_t) v_t^T and z <- z + sum_t phi(k_t), and then every token reads it
 * out, o_t = phi(q_t)^T S / (phi(q_t)^T z + eps) (the numerator alone with
 * LA_NORM_NONE).  The final state is the same as the causal form's.  No
 * decay or gate (LA_EINVAL otherwise). */
la_status la_prefill(const la_desc* desc, const void* q, const void* k, const void* v,
                     float* S, float* z, void* out, void* workspace,
                     size_t workspace_bytes, void* stream);

/* The three stages la_prefill enqueues, for callers that time or interleave
 * them: 1 = per-segment state contributions (reads k, v), 2 = scan of the
 * segment states (folds in the initial state), 3 = outputs and final state
 * (reads q, k, v; with mLSTM gates and several segments, stage 3 writes the
 * final stabiliser).  Running stages 1, 2, 3 in order with identical
 * arguments is exactly la_prefill; a stage with nothing to do returns LA_OK. */
la_status la_prefill_stage(const la_desc* desc, int stage, const void* q, const void* k,
                           const void* v, float* S, float* z, void* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace la_prefill_backward needs for `desc`.  Host
 * only.  The chunked path (see below): the prefill's workspace for the same
 * shapes with 32-token chunks, plus B H d' d_v + B H d' fp32 (a copy of the
 * initial state), B H nseg (d' d_v + d') fp32 (one gradient state per
 * segment) and B H T 2 fp32 (per token: the read-out's factor and the
 * divisor's gradient), each part rounded up to 256 bytes; with a decay also
 * B H nseg fp32 (each segment's log-decay), B H T 2 fp32 (per-token terms
 * of the decay gradient) and B H ceil(T / 1024) fp32 (their tile totals);
 * with the mLSTM gates also B H fp32 (a zero start stabiliser) and B H T 2
 * fp32 (log alpha'_t, beta'_t).  The per-token path: B H T (d_v + 2) fp32,
 * B H T (d_v + 4) fp32 with the mLSTM gates. */
la_status la_prefill_backward_workspace_size(const la_desc* desc, size_t* bytes);

/* Gradients of a causal prefill for training ([lesson] Developer level and
 * "Implementation reality": training runs the same function, so these are
 * the gradients of the definition).  With L = sum_t <dout_t, o_t> for the
 * prefill that `desc`, q, k, v and the initial state (S0, z0) describe:
 *   in:  q, k, v (dtype) [B, H, T, d]; dout [B, H, T, d_v] (out_dtype); the
 *        initial state S0 [B, H, d', d_v], z0 [B, H, d'] fp32, both NULL for
 *        a zero state; the decay or gate through desc;
 *   out: dq, dk [B, H, T, d_h], dv [B, H, T, d_v] fp32; ddecay [B, H, T]
 *        fp32 (dL/da_t for LA_DECAY_SSD, dL/dg_t for LA_GATE_RFA; NULL
 *        without a decay, required with one); dS0, dz0 (dL/dS0, dL/dz0;
 *        both NULL to skip).
 * mLSTM gates (LA_GATE_MLSTM, identity features; wikillm "Linear
 * attention", Variants / mLSTM): the initial state is the scaled (S0', z0')
 * with its stabiliser in desc->stab [B, H] (read only, and only with S0;
 * a zero state has stabiliser 0); ddecay holds 2 B H T floats, dL/d of the
 * forget pre-activations desc->decay then dL/d of the input pre-activations
 * desc->igate; dS0, dz0 are dL/dS0', dL/dz0' (the stabiliser's own gradient
 * is <dS0', S0'> + <dz0', z0'>).  The state is carried scaled by the
 * forward's stabiliser throughout, so no intermediate overflows where the
 * forward's does not: both paths take the recurrence with alpha'_t =
 * e^{log f_t + m_{t-1} - m_t} and beta'_t = e^{itilde_t - m_t} as decay and
 * key weight, and no gate gradient divides by a decay.
 * The decay gradient is formed through log a_t (a suffix sum of
 * <phi(q_t), dphi(q_t)> - <phi(k_t), dphi(k_t)>, divided by a_t); where a
 * decay or gate value is below 1/256 (0, a full reset, included) it is
 * taken from its definition instead, dL/da_r = <G_r, S_{r-1}> +
 * <gz_r, z_{r-1}> (the gradient of the state after r with the state before
 * it), by a walk over the tokens of r's segment, which is finite and free
 * of the division's loss of accuracy.
 * Supported: causal, elu+1 or identity features, LA_DECAY_NONE, LA_DECAY_SSD,
 * LA_GATE_RFA or LA_GATE_MLSTM, every read-out form, the widths the
 * per-token kernel takes (LA_EUNSUPPORTED otherwise: RFF, the non-causal
 * form).
 * Two paths.  Chunked (bf16 inputs, elu+1 with no decay, the SSD decay or
 * the RFA gate, or identity features with the mLSTM gates; d' = d_v in
 * {64, 128}, T > 0): the same gradients written as
 * masked-quadratic sums inside 32-token chunks and states across them, as
 * the forward ([lesson] "Implementation reality"): the prefill's segment
 * start states, a pass in token order (dq and each segment's gradient state
 * sum phi(q_t) g_t^T), a reverse scan over the segments, a pass in reverse
 * order (dk, dv) and, with a decay, a suffix sum per sequence for the decay
 * gradient; the segment plan is the prefill's for 32-token chunks
 * (desc->segments when desc->chunk is 0 or 32, 0 = default; the default
 * for any other chunk).  Otherwise one workgroup walks each (b, h) sequence token by
 * token, forward then backward.  `workspace` holds
 * la_prefill_backward_workspace_size() bytes; its contents on return are
 * scratch.  T = 0: L is an empty sum; dS0 and dz0 (if given) are written as
 * zeros and nothing else is touched (the workspace size is 0). */
la_status la_prefill_backward(const la_desc* desc, const void* q, const void* k, const void* v,
                              const float* S0, const float* z0, const void* dout, float* dq,
                              float* dk, float* dv, float* ddecay, float* dS0, float* dz0,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Size of the static device scratch behind la_prefill_noalloc: 64 MiB per
 * GPU, held from the library's first use of that GPU until the process
 * ends.  It covers the chunked prefill's workspace for every shape up to
 * B H = 256 sequences at d' = d_v = 128 with the default plan (33.8 MB for
 * B = 1, H = 8, T = 102400). */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* la_prefill for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, arguments and results as la_prefill, with the workspace
 * taken from a static per-GPU array of LA_NOALLOC_SCRATCH_BYTES instead of
 * the caller.  Calls no allocating routine.  A descriptor whose workspace
 * (la_prefill_workspace_size) exceeds that size is rejected with LA_EINVAL
 * before anything is enqueued.  The first call on a GPU looks up that GPU's
 * copy of the array (LA_EHIP if the lookup fails).  Every call on one GPU
 * shares its array, which keeps the last call's contents (nothing in it
 * needs to start at zero): calls that overlap on one GPU (several streams
 * or threads) race and must be serialised by the caller. */
la_status la_prefill_noalloc(const la_desc* desc, const void* q, const void* k, const void* v,
                             float* S, float* z, void* out, void* stream);

/* One autoregressive step for B sequences x H heads ([kb] section 2, causal
 * recurrence; [card] "When to use which": memory-bound decoding with a
 * fixed-size state): reads q, k [B, H, d_h], v [B, H, d_v] and the gate or
 * decay [B, H]; updates (S, z) (and desc->stab) in place and writes out
 * [B, H, d_v].  desc->noncausal must be 0. */
la_status la_decode_step(const la_desc* desc, const void* q, const void* k, const void* v,
                         float* S, float* z, void* out, void* stream);

/* Static name of a status code. */
const char* la_status_str(la_status status);

/* Reason for the calling thread's most recent failing call ("" if none). */
const char* la_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
