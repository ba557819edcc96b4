/*
 * liblogattn -- log-linear attention in its Mamba-2 form on AMD CDNA4 (gfx950).
 *
 * The operator, per (batch b, head h), with 0-based query t and key s:
 *
 *   o_t = sum_{s<=t} lambda[t, l(t,s)] * M^S[t,s] * (q_t . k_s) * v_s
 *
 *   M^S[t,s] = prod_{s<r<=t} a_r,  a_r = exp(log_a[r])   -- the Mamba-2 scalar
 *              gate ("Log-Linear Attention", Spanish summary, technical
 *              section 2, "Variantes", item 1; Italian summary, technical
 *              section 2, item 2: semiseparable mask of Mamba-2).
 *   l(t,s)   = 0 if s == t, else 1 + msb(t XOR s): the Fenwick-tree bucket
 *              holding key s as seen from query t; bucket l >= 1 holds
 *              2^(l-1) keys, recent keys in small buckets, old keys in large
 *              ones (Italian summary, technical section 2, item 1; Spanish
 *              summary, technical section 2, "Conceptos clave").
 *   lambda   = per-token, per-level weights: the hierarchical mask that
 *              replaces the causal mask (Italian summary, technical
 *              section 2, item 2).
 *
 * No softmax, no 1/sqrt(d) scale, no normaliser.
 *
 * Conventions for every call:
 *  - Return value: LA_OK (0) or a negative la_status.  Arguments are checked
 *    on the host before anything is enqueued; on error nothing is launched
 *    and no output is written.
 *  - Pointers are device pointers unless stated otherwise.  The caller
 *    allocates and owns every buffer; the library allocates no device memory
 *    and keeps no global mutable state, except the fixed scratch array of
 *    loglinear_fwd_noalloc (one per GPU, held until the process ends) and
 *    its per-device address.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *    stream).  Faults inside kernels surface at the caller's next
 *    synchronisation.  NaN/Inf inputs are not checked; they propagate.
 *  - Tensors are dense and contiguous in the stated layouts.
 *  - Calls that share a workspace or a state must not overlap in time.
 */
#ifndef LOGATTN_H
#define LOGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_API __attribute__((visibility("default")))

typedef enum la_status {
  LA_OK = 0,
  LA_EINVAL = -1,      /* null pointer or a non-positive count where one is required */
  LA_ESHAPE = -2,      /* unsupported head dim / chunk size, too few levels, size limit */
  LA_EDTYPE = -3,      /* dtype code not one of la_dtype */
  LA_EALIGN = -4,      /* a pointer is not aligned as documented */
  LA_EWORKSPACE = -5,  /* workspace pointer null or smaller than the queried size */
  LA_ECAPACITY = -6,   /* decode state has too few slots for the next merge */
  LA_EHIP = -7,        /* a HIP runtime call or kernel launch failed */
  LA_ESCRATCH = -8     /* the problem needs more than the fixed scratch of
                          loglinear_fwd_noalloc */
} la_status;

typedef enum la_dtype {
  LA_F32 = 0,          /* q, k, v, out in float32; float32 matrix-core products */
  LA_BF16 = 1          /* q, k, v, out in bfloat16; bf16 matrix-core products,
                          float32 accumulation */
} la_dtype;

typedef void* la_stream_t; /* hipStream_t */

/* Human-readable text for a status code (static storage; never NULL). */
LA_API const char* loglinear_strerror(int code);

/* Library version as 10000*major + 100*minor + patch. */
LA_API int loglinear_version(void);

/*
 * Workspace size for loglinear_fwd.
 *
 * Writes to *bytes (host pointer) the number of device bytes loglinear_fwd
 * needs for the given shape (0 is possible).  Supported shapes are those
 * loglinear_fwd accepts; others return the same error code it would.
 */
LA_API int loglinear_fwd_workspace(int B, int H, int64_t T, int dk, int dv, int C,
                                   int dtype, size_t* bytes);

/*
 * Chunkwise-parallel forward ("Log-Linear Attention", Italian summary,
 * technical section 2, item 3 "Training"; Spanish summary, technical
 * section 2, "Forma paralela" and "Algoritmo de entrenamiento"): the
 * sequence is cut into chunks of C tokens; pairs inside a chunk are formed
 * densely, pairs across chunks go through per-chunk states combined along the
 * Fenwick levels.  The result is the operator above, exactly up to rounding.
 *
 *   q      [B, H, T, dk]  dtype          16-byte aligned
 *   k      [B, H, T, dk]  dtype          16-byte aligned
 *   v      [B, H, T, dv]  dtype          16-byte aligned
 *   log_a  [B, H, T]      float32, <= 0 (gates a = exp(log_a) in (0, 1], as in
 *                         the model).  The kernels split each decay into
 *                         factors that are all <= 1 under this condition;
 *                         positive values may overflow them.
 *   lambda [B, H, T, L]   float32, level index innermost; L >= ceil(log2 T)+1
 *                         (levels >= ceil(log2 T)+1 are never read)
 *   out    [B, H, T, dv]  dtype, written   16-byte aligned
 *
 * Supported: dk == dv in {16, 32, 64, 128} and C in {16, 32, 64, 128}, every
 * combination except float32 with C == dk == 128, whose tiles exceed the
 * 160 KB of LDS of a workgroup (LA_ESHAPE; loglinear_fwd_workspace answers
 * the same); T >= 0 (T == 0, B == 0 or H == 0 is a no-op); T need not be a
 * multiple of C (the last chunk is partial).  T <= 2^31 - 1.
 * workspace: device memory of at least loglinear_fwd_workspace() bytes,
 * 256-byte aligned; its contents on entry do not matter.
 */
LA_API int loglinear_fwd(const void* q, const void* k, const void* v, const float* log_a,
                         const float* lambda, void* out, int B, int H, int64_t T, int dk, int dv,
                         int C, int L, int dtype, void* workspace, size_t workspace_bytes,
                         la_stream_t stream);

/*
 * loglinear_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, layouts, results and
 * errors as loglinear_fwd, except that the workspace is a fixed
 * LA_NOALLOC_SCRATCH_BYTES array in device memory that the library holds on
 * every GPU it runs on, from the first call on that GPU until the process
 * ends; nothing is allocated or freed by this call.  Shapes whose
 * loglinear_fwd_workspace() exceeds that size return LA_ESCRATCH (in bfloat16
 * at d = C = 64 it holds up to 186 (b,h) heads of 2048 tokens, 23 of 16384
 * or 2 of 131072; at d = C = 128, 73, 9 and 1).  All calls on one GPU share
 * the array: calls that overlap in time on the same GPU (two streams, or
 * several host threads) race and must be serialised by the caller.
 */
#define LA_NOALLOC_SCRATCH_BYTES (64ull << 20)
LA_API int loglinear_fwd_noalloc(const void* q, const void* k, const void* v, const float* log_a,
                                 const float* lambda, void* out, int B, int H, int64_t T, int dk,
                                 int dv, int C, int L, int dtype, la_stream_t stream);

/* Number of kernel stages loglinear_fwd enqueues for this shape (host only). */
LA_API int loglinear_fwd_num_stages(int B, int H, int64_t T, int dk, int dv, int C, int dtype,
                                    int* n_stages);

/*
 * loglinear_fwd with per-stage timing: `events` is a host array of
 * n_stages + 1 hipEvent_t handles created by the caller; events[i] is
 * recorded on `stream` before stage i and events[n_stages] after the last
 * stage.  Same arguments, results and errors as loglinear_fwd otherwise.
 */
LA_API int loglinear_fwd_staged(const void* q, const void* k, const void* v, const float* log_a,
                                const float* lambda, void* out, int B, int H, int64_t T, int dk,
                                int dv, int C, int L, int dtype, void* workspace,
                                size_t workspace_bytes, void* const* events, int n_events,
                                la_stream_t stream);

/*
 * Recurrent (decode) state: one d_k x d_v float32 matrix per Fenwick level
 * ("Log-Linear Attention", Italian summary, technical section 2, item 3
 * "Decoding": O(log T) separate recurrent states, one per level).
 *
 *   t      number of tokens already consumed (host integer)
 *   slots  [B, H, S, dk, dv] float32 device memory; slot i holds level i+1
 *   scale  [B, H, S] float32 device memory; the true bucket matrix is
 *          scale[i] * slots[i] (the gate is applied lazily to the scalar)
 * Level l >= 1 holds a bucket exactly when bit l-1 of t is set; other slots
 * are ignored.  The struct lives in host memory and is owned by the caller;
 * saving and restoring a state is copying t, slots and scale.
 */
typedef struct la_state {
  int64_t t;
  int B, H, dk, dv, S;
  float* slots;
  float* scale;
} la_state;

/* Device bytes of the slots and scale arrays for a state of this shape. */
LA_API int loglinear_state_bytes(int B, int H, int dk, int dv, int S, size_t* slot_bytes,
                                 size_t* scale_bytes);

/*
 * Initialise *st (host struct) to the empty state (t = 0) over caller-owned
 * device arrays `slots` and `scale` (16-byte aligned, sizes from
 * loglinear_state_bytes).  Enqueues a kernel that zeroes slots and sets
 * scale to 1 on `stream`.  dk == dv in {16, 32, 64, 128}; 1 <= S <= 40.
 */
LA_API int loglinear_state_init(la_state* st, int B, int H, int dk, int dv, int S, float* slots,
                                float* scale, la_stream_t stream);

/*
 * One decode step for every (b, h) at position t = st->t (Italian summary,
 * technical section 2, item 3 "Decoding"; lay part "L'essenziale": only the
 * smallest box is updated and, when needed, merged into the bigger boxes):
 *   1. every stored bucket decays by a (lazily, through scale);
 *   2. out = lambda[0] (q . k) v + sum over stored levels l of
 *      lambda[l] * scale_l * slots_l^T q;
 *   3. binary-counter carry: with k* the number of trailing one bits of t,
 *      the token and levels 1..k* merge into level k*+1 (scale 1).
 * Then st->t is incremented on the host.
 *
 *   q      [B, H, dk]   dtype      16-byte aligned
 *   k      [B, H, dk]   dtype      16-byte aligned
 *   v      [B, H, dv]   dtype      16-byte aligned
 *   a      [B, H]       float32    the gate exp(log_a) of this token, in (0, 1]
 *   lambda [B, H, S+1]  float32    weights of levels 0..S for this token
 *   out    [B, H, dv]   dtype      written, 16-byte aligned
 * LA_ECAPACITY when level k*+1 would exceed S (st->t is then unchanged).
 */
LA_API int loglinear_decode_step(la_state* st, const void* q, const void* k, const void* v,
                                 const float* a, const float* lambda, void* out, int dtype,
                                 la_stream_t stream);

/*
 * The forward that also leaves the recurrent (decode) state after the T
 * tokens in *state, so that loglinear_decode_step continues at position T:
 * a prefill hand-off (Italian summary, technical section 2, item 3: the
 * parallel form for training and the recurrent form for decoding compute
 * the same per-level states).  Slot i receives the bucket of level i+1 when
 * bit i of T is set -- the keys [((T >> i) << i) - 2^i, (T >> i) << i), each
 * weighted by its gate product up to token T-1, as a (dk, dv) matrix; the
 * slots of empty levels are left as they are (loglinear_decode_step never
 * reads them and overwrites a slot whole when its level fills).  Every scale
 * becomes 1 and state->t becomes T (on the host, once the work is enqueued).
 * With T == 0 the whole state is reset as by loglinear_state_init.  Buckets of whole chunks come from the bucket
 * nodes the forward builds, in the layer dtype (bfloat16 in LA_BF16 mode);
 * smaller ones are summed in float32 from k and v.
 *
 * state: a state of the same B, H, dk, dv (set up by loglinear_state_init
 * or by a previous call); its slots and scale are overwritten.  state->S
 * must be at least the bit length of T, else LA_ECAPACITY (nothing runs).
 * Arguments, workspace and errors otherwise as loglinear_fwd.
 */
LA_API int loglinear_fwd_state(const void* q, const void* k, const void* v, const float* log_a,
                               const float* lambda, void* out, int B, int H, int64_t T, int dk, int dv,
                               int C, int L, int dtype, void* workspace, size_t workspace_bytes,
                               la_state* state, la_stream_t stream);

/* Workspace size for loglinear_bwd (host only); errors as loglinear_bwd. */
LA_API int loglinear_bwd_workspace(int B, int H, int64_t T, int dk, int dv, int C, int dtype,
                                   size_t* bytes);

/*
 * Backward of loglinear_fwd: the gradients of a loss L with respect to q, k,
 * v, log_a and lambda, given dout = dL/dout.  Training needs them, the level
 * weights' included ("Log-Linear Attention", Spanish summary, section 5
 * "Limitaciones", first item: custom kernels for the hierarchical structure
 * and for the gradients of lambda).  With A[t,s] = lambda[t, l(t,s)] M^S[t,s]:
 *   grad_q[t]  = sum_{s<=t} A[t,s] (dout_t . v_s) k_s
 *   grad_k[s]  = sum_{t>=s} A[t,s] (dout_t . v_s) q_t
 *   grad_v[s]  = sum_{t>=s} A[t,s] (q_t . k_s) dout_t
 *   grad_lambda[t, l] = sum over the keys s of bucket l of t of
 *                       M^S[t,s] (q_t . k_s)(dout_t . v_s); 0 for empty
 *                       buckets and for levels l >= ceil(log2 T) + 1
 *   grad_log_a[r] = sum_{u>=r} (dout_u . o_u - v_u . grad_v[u])
 * (the gate of token 0 multiplies nothing, so grad_log_a[0] is 0 up to
 * rounding).  Computed chunkwise like the forward, without the forward's
 * output: dout_u . o_u = sum_l lambda[u, l] grad_lambda[u, l].
 *
 *   q, k, v, log_a, lambda  as for loglinear_fwd (inputs, not written)
 *   dout         [B, H, T, dv]  dtype     16-byte aligned
 *   grad_q       [B, H, T, dk]  dtype     written, 16-byte aligned
 *   grad_k       [B, H, T, dk]  dtype     written, 16-byte aligned
 *   grad_v       [B, H, T, dv]  dtype     written, 16-byte aligned
 *   grad_log_a   [B, H, T]      float32   written
 *   grad_lambda  [B, H, T, L]   float32   written (every entry)
 * The outputs must not overlap the inputs or each other.
 *
 * Supported: the shapes loglinear_fwd accepts with C in {16, 32, 64} (C = 128
 * returns LA_ESHAPE, and loglinear_bwd_workspace answers the same).  The chunk size only changes the
 * summation order, so a backward may use another C than its forward.
 * workspace: at least loglinear_bwd_workspace() bytes, 256-byte aligned.
 * Errors as loglinear_fwd.
 */
LA_API int loglinear_bwd(const void* q, const void* k, const void* v, const float* log_a,
                         const float* lambda, const void* dout, void* grad_q, void* grad_k,
                         void* grad_v, float* grad_log_a, float* grad_lambda, int B, int H, int64_t T,
                         int dk, int dv, int C, int L, int dtype, void* workspace,
                         size_t workspace_bytes, la_stream_t stream);

/*
 * loglinear_bwd reusing the forward pass's bucket structure (the same
 * gradients, "Log-Linear Attention", Spanish summary, section 5 on the level
 * weights' gradients).  The query side of the backward needs, for every
 * bucket, the sum of gate * k_s v_s^T over its keys: exactly the transposes
 * of the nodes the forward builds over (k, v).  So a training step that keeps
 * its forward's workspace can hand it over, and the backward skips building
 * that structure again.
 *
 *   fwd_workspace        the workspace of an earlier loglinear_fwd (or
 *                        loglinear_fwd_state) call on the same q, k, v, log_a
 *                        and lambda (same B, H, T, dk, dv, C, L and dtype),
 *                        not written since; read only.
 *                        At least loglinear_fwd_workspace() bytes, 256-byte
 *                        aligned (may be null when that size is 0).
 *   everything else      as for loglinear_bwd; workspace is this call's own
 *                        (loglinear_bwd_workspace() bytes).
 *
 * The forward's structure is used where the fused per-chunk kernel runs
 * (bfloat16, C in {32, 64}, dk <= 64, lambda rows that fit: L <= 17 at
 * C = dk = 64); elsewhere it is not read and the call is loglinear_bwd.  The
 * gradients agree with loglinear_bwd to the rounding of the two structures'
 * bfloat16 nodes (each gates its own operand).  A workspace that does not
 * hold that forward's nodes gives wrong gradients, not an error: the library
 * cannot tell.  Errors as loglinear_bwd; LA_EWORKSPACE / LA_EALIGN for
 * fwd_workspace.
 */
LA_API int loglinear_bwd_from_fwd(const void* q, const void* k, const void* v, const float* log_a,
                                  const float* lambda, const void* dout, void* grad_q, void* grad_k,
                                  void* grad_v, float* grad_log_a, float* grad_lambda, int B, int H, int64_t T,
                                  int dk, int dv, int C, int L, int dtype, const void* fwd_workspace,
                                  size_t fwd_workspace_bytes, void* workspace, size_t workspace_bytes,
                                  la_stream_t stream);

/* Workspace size for loglinear_gdn_fwd (host only); errors as loglinear_gdn_fwd. */
LA_API int loglinear_gdn_fwd_workspace(int B, int H, int64_t T, int dk, int dv, int C, int dtype,
                                       size_t* bytes);

/*
 * Log-linear Gated DeltaNet forward: the Fenwick-bucket structure laid over
 * the gated delta rule ("Log-Linear Attention", both summaries, technical
 * summary section 2, the second of the two variants).  Every bucket state
 * follows the gated delta rule's transition A_r = a_r (I - beta_r k_r k_r^T),
 * a_r = exp(log_a[r]), a key enters its bucket as beta_s k_s v_s^T, and the
 * output is the lambda-weighted sum of the buckets.  Per (b, h):
 *   out[t] = sum_{s<=t} lambda[t, l(t,s)] beta_s (q_t^T Phi(t,s) k_s) v_s,
 *   Phi(t,s) = A_t A_{t-1} ... A_{s+1}  (the identity for s = t),
 * with l(t,s) the Fenwick level of loglinear_fwd.  lambda constant reduces it
 * to the gated delta rule; with keys that never overlap it is loglinear_fwd
 * with values beta v.
 *
 *   q, k     [B, H, T, dk]  dtype     16-byte aligned; the delta rule
 *                                     expects unit-norm keys (not checked)
 *   v, out   [B, H, T, dv]  dtype     16-byte aligned; out is written
 *   log_a    [B, H, T]      float32   log of the gate (<= 0 expected)
 *   beta     [B, H, T]      float32   write strength, in [0, 1] expected
 *   lambda   [B, H, T, L]   float32   L >= ceil(log2 T) + 1
 *   C        chunk size, 16, 32 or 64; dk = dv in {16, 32, 64}
 *   workspace at least loglinear_gdn_fwd_workspace() bytes, 256-byte
 *            aligned, owned by the caller: per chunk a C x C matrix, per
 *            aligned block of 2^m full chunks a d x d state and a d x d
 *            transition, all in the layer dtype
 * Asynchronous on `stream`; every check happens on the host before any
 * launch, and on error nothing is written.  Errors: LA_EINVAL (null pointer,
 * negative count), LA_ESHAPE (dims, C, L, size limits), LA_EDTYPE,
 * LA_EALIGN, LA_EWORKSPACE, LA_EHIP (launch failure).
 */
LA_API int loglinear_gdn_fwd(const void* q, const void* k, const void* v, const float* log_a,
                             const float* beta, const float* lambda, void* out, int B, int H, int64_t T,
                             int dk, int dv, int C, int L, int dtype, void* workspace,
                             size_t workspace_bytes, la_stream_t stream);

/*
 * Log-Linear Mamba-2 layer, forward: the Mamba-2 block with its SSM replaced
 * by loglinear_fwd (Spanish summary, technical section 2, "Variantes", item
 * 1: Mamba-2's selective gate combined with the hierarchical mask; the pages
 * give no layer, so the block follows Mamba-2's published design, with one
 * more group of projected columns for the level weights).  Per sequence b and
 * token t, with d_inner = H P and head h in group g = h / (H / G):
 *   zxbcdt = u W_in^T, columns z [H P] | x [H P] | B [G N] | C [G N] | dt [H]
 *            | lam [H L]
 *   x|B|C <- silu(causal depthwise conv over time, K taps, plus bias):
 *            c[t] = conv_b + sum_{j<K} conv_w[j] xBC[t - (K-1) + j]
 *   dt_h   = softplus(dt_h + dt_bias_h);  log_a_h = -exp(A_log_h) dt_h
 *   o      = loglinear_fwd(q = C_g, k = B_g, v = dt_h x_h, log_a,
 *                          lambda = softplus(lam + lam_bias))
 *   y      = (o + D_h x_h) silu(z), divided by the root mean square over
 *            each of G equal channel groups (plus eps), times norm_w
 *   out    = y W_out^T
 * The operator runs with d_k = N, d_v = P (so N == P) and chunk size C, on
 * bfloat16 or float32 tensors as loglinear_fwd, with q and k held once per
 * group of heads (every head of group g reads C_g and B_g); projections accumulate in
 * fp32 and store the element type; the conv, gates and norm run in fp32.
 *
 *   u        [B, T, d_model]       dtype, 16-byte aligned
 *   out      [B, T, d_model]       dtype, 16-byte aligned; written
 *   weights (la_mamba2_weights, device pointers, read only):
 *     in_proj  [d_in_proj, d_model] dtype, 16-byte aligned,
 *              d_in_proj = 2 H P + 2 G N + H + H L
 *     conv_w   [H P + 2 G N, K]     dtype;  conv_b [H P + 2 G N] dtype
 *     dt_bias, A_log, D  [H] float32;  lam_bias [H, L] float32
 *     norm_w   [H P] dtype, 16-byte aligned
 *     out_proj [d_model, H P] dtype, 16-byte aligned
 *   sizes (la_mamba2_dims): d_model and H P multiples of 64 (bfloat16) or
 *     32 (float32); H P at most 2048 (bfloat16) or 1024 (float32); G
 *     divides H and H P / G is a multiple of 8; 1 <= K <= 4; P == N with
 *     (P, C, L) as loglinear_fwd accepts for T tokens; 0 <= eps <= 1
 *   workspace at least loglinear_mamba2_fwd_workspace() bytes, 256-byte
 *            aligned, owned by the caller: the projection, the operator's
 *            inputs and output, and its own workspace
 * Asynchronous on `stream`; every check happens on the host before any
 * launch, and on error nothing is written.  Errors: LA_EINVAL (null
 * pointer, non-positive size, eps out of range), LA_ESHAPE, LA_EDTYPE,
 * LA_EALIGN, LA_EWORKSPACE, LA_EHIP.  B = 0 or T = 0 writes nothing.
 */
typedef struct la_mamba2_dims {
  int B;          /* sequences */
  int64_t T;      /* tokens per sequence */
  int d_model;    /* input and output width */
  int H, P, N, G; /* heads, head dim, state size, groups of heads sharing B and C */
  int K;          /* conv taps */
  int C;          /* operator chunk size */
  int L;          /* lambda levels */
  float eps;      /* norm epsilon */
  int dtype;      /* la_dtype */
} la_mamba2_dims;

typedef struct la_mamba2_weights {
  const void* in_proj;
  const void* conv_w;
  const void* conv_b;
  const float* dt_bias;
  const float* A_log;
  const float* D;
  const float* lam_bias;
  const void* norm_w;
  const void* out_proj;
} la_mamba2_weights;

LA_API int loglinear_mamba2_fwd_workspace(const la_mamba2_dims* dims, size_t* bytes);
LA_API int loglinear_mamba2_fwd(const void* u, const la_mamba2_weights* weights, void* out,
                                const la_mamba2_dims* dims, void* workspace, size_t workspace_bytes,
                                la_stream_t stream);

/*
 * Fenwick level table for checking: out[t * T + s] = l(t, s) for s <= t and
 * -1 for s > t, as int8, computed on the device with chunks of C tokens the
 * way the forward kernels find levels.  Inside a chunk it is the level
 * function of the in-chunk masks (1 + msb of the offsets' XOR).  Across
 * chunks it is not a closed form: the table walks the bucket list of the
 * forward's output kernel (chunk buckets from the set bits of the chunk's
 * index in its group of 8, group buckets from the set bits of the group
 * index) and writes the level of the bucket that holds chunk_s, so a
 * mismatch there shows up in the table.  That enumeration equals
 * log2(C) + 1 + msb(chunk_t XOR chunk_s) for every group size, which a host
 * program checks exhaustively.
 *   out  [T, T] int8 device memory; 1 <= T <= 16384; C a power of two
 *        in [1, 2^20].
 */
LA_API int loglinear_level_table(int64_t T, int C, int8_t* out, la_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LOGATTN_H */
