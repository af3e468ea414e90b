/*
 * kda.h -- C ABI of libkda: Kimi Delta Attention (KDA) forward, decode step and
 * adjoint on AMD Instinct MI355X (gfx950), hand-written HIP kernels.
 *
 * The method (per batch b, head h; sources are the burn-kda review pages):
 *   gate     g = -exp(clamp(A_log[h], -10, 20)) * softplus(z + dt_bias[h,:])
 *            alpha = exp(g)                      ("kdafix" page, "Fix 1 -- decay form":
 *                                                 softplus first, the exp(A) multiplier outside)
 *   scale    q_hat = scale * q, default scale = K^-0.5  ("kdafix" page, "Fix 2 -- read scale")
 *   per token t (the gated delta rule):
 *            S' = diag(alpha_t) S
 *            S  = S' + beta_t k_t (v_t - S'^T k_t)^T
 *            o_t = S^T q_hat_t
 *   The chunked forward evaluates the same result in blocks of `chunk` tokens
 *   (WY form; the carry decays by exp(G_last - G), "The fused KDA adjoint" page,
 *   section 2).  Results equal the token recurrence up to floating-point rounding.
 *
 * Conventions shared by every entry point:
 *   - Layout is head-major and contiguous: q, k, z, g: (B,H,T,K); v, o: (B,H,T,V);
 *     beta: (B,H,T); state: (B,H,K,V) float32 (row = key channel, column = value
 *     channel); A_log: (H) float32; dt_bias: (H,K) float32.
 *   - `dtype` (KDA_F32 or KDA_BF16) is the element type of the activations q, k,
 *     v, z, beta and of the output o.  States, A_log, dt_bias, g, alpha and all
 *     gradients are float32 whatever `dtype` is.
 *   - Every pointer is a device pointer.  The caller allocates and owns every
 *     buffer, workspaces included; the library allocates nothing.  Between calls it
 *     keeps only process-wide counters and settings (kda_get_counters,
 *     kda_set_exchange_timeout_us) and a launch counter of the paired forward.
 *     When T = 0, pointers to buffers with a T dimension may be NULL.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously on it; a call returns once its kernels are launched.
 *   - Argument errors are reported before anything is launched, by a negative
 *     status (kda_status below).  Nothing is printed, nothing is thrown across
 *     the ABI, and there is no fallback path: an unsupported argument is an error.
 *   - Supported sizes: K, V in {8, 16, 32, 64, 128}; chunk in {16, 32, 64};
 *     B, H >= 1; T >= 0 (T = 0 writes nothing to o and copies state_in to
 *     state_out).  T need not be a multiple of chunk: the last block behaves as
 *     if padded with identity tokens (g = 0, beta = 0, q = k = v = 0), which leave
 *     the state unchanged.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = -1,       /* a required pointer is NULL */
  KDA_ERR_SHAPE = -2,      /* B, H, T, K or V out of range or unsupported */
  KDA_ERR_DTYPE = -3,      /* unknown dtype, or a dtype this entry point does not take */
  KDA_ERR_CHUNK = -4,      /* chunk not in {16, 32, 64} */
  KDA_ERR_ALIAS = -5,      /* an output buffer aliases an input it must not alias */
  KDA_ERR_HIP = -6,        /* a HIP launch or runtime call failed */
  KDA_ERR_WORKSPACE = -7,  /* workspace NULL or smaller than kda_chunk_bwd_workspace_bytes() */
  KDA_ERR_ALIGN = -8,      /* an activation pointer or a workspace is misaligned */
  KDA_ERR_EXCHANGE = -9,   /* kda_chunk_fwd_status: the two workgroups of a head failed to hand
                              blocks to each other (a bounded wait ran out, or they were not on
                              one XCD); that call's outputs are undefined */
  KDA_ERR_SCRATCH = -10    /* kda_gate_bwd_noalloc: these sizes need more than the library's
                              built-in scratch (KDA_GATE_BWD_SCRATCH_BYTES) */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* FLA's default read scale K^-0.5 as float ("kdafix" page, "Fix 2 -- read scale":
 * every path folds it into q).  Returns 0 for K <= 0.  Host-only, no GPU work. */
float kda_read_scale(int K);

/* Fused decay gate ("kdafix" page, "Fix 1 -- decay form").
 *   z        (B,H,T,K) in `dtype`
 *   A_log    (H) float32, clamped to [-10, 20] before exp
 *   dt_bias  (H,K) float32, may be NULL (= 0)
 *   g_out    (B,H,T,K) float32: g <= 0
 *   alpha_out (B,H,T,K) float32 = exp(g), may be NULL (not written)
 * K may be any value >= 1 here.  g_out/alpha_out must not alias z. */
int kda_gate(const void* z, const float* A_log, const float* dt_bias,
             float* g_out, float* alpha_out,
             int B, int H, int T, int K, int dtype, void* stream);

/* Bytes of device workspace kda_chunk_fwd / kda_chunk_fwd_scalar can use for these
 * sizes: nonzero for KDA_BF16 with V = 128 and chunk 32 or 64 (the paired path below),
 * 0 for every other call (and on bad sizes).  It grows with B*H up to 128 heads and
 * stays constant beyond (about 27.6 MB at K = 128). */
size_t kda_chunk_fwd_workspace_bytes(int B, int H, int T, int K, int V, int chunk, int dtype);

/* Chunked KDA forward: the gate, the read-scale fold, the intra-chunk WY stage
 * (decay-weighted strictly-lower beta k k^T, (I+A)^-1 by forward substitution,
 * w and u), the inter-chunk state passing and the output, fused in one kernel.
 *   q, k, z  (B,H,T,K) `dtype`;  v (B,H,T,V) `dtype`;  beta (B,H,T) `dtype`
 *   A_log (H) f32;  dt_bias (H,K) f32 or NULL (= 0)
 *   state_in  (B,H,K,V) f32, or NULL for a zero initial state
 *   scale     read scale (pass kda_read_scale(K) for the default; 0 gives o = 0)
 *   chunk     block size of the WY form, 16, 32 or 64.  The kernels block by at
 *             most 32 tokens where on-chip memory or registers require it (every
 *             KDA_BF16 call; KDA_F32 with K = 128); the result is the same function.
 *   q, k, v, z must be aligned to two elements (4 bytes for KDA_BF16, 8 for
 *   KDA_F32): the kernels load channel pairs (KDA_ERR_ALIGN otherwise).  One
 *   head's sequence must span less than 2 GiB: (T + 64) * max(K, V) * element
 *   size < 2^31, since the kernels address it with 32-bit offsets (KDA_ERR_SHAPE
 *   otherwise).
 *   o         (B,H,T,V) `dtype`; must not alias any input
 *   state_out (B,H,K,V) f32 final state, or NULL (not written); may equal state_in
 *             (each state tile is read before it is written by the same workgroup).
 *   workspace device buffer of at least kda_chunk_fwd_workspace_bytes() bytes, 256-byte
 *             aligned, or NULL.  When that size is nonzero and a workspace is given, the
 *             two value tiles of each head run as a pair of workgroups that compute the
 *             gate and WY stages of alternate blocks once and hand them to each other
 *             through the workspace (L2 of their shared XCD); with NULL, or when the size
 *             is 0, each value tile computes them itself (same results up to rounding,
 *             slower).  Contents on entry are ignored; it must not overlap any other
 *             argument (KDA_ERR_ALIAS), and two calls in flight at once must not share
 *             one (their hand-offs would mix).  A too small workspace gives
 *             KDA_ERR_WORKSPACE, a misaligned one KDA_ERR_ALIGN.  The pair's waits
 *             are bounded (kda_set_exchange_timeout_us); if one runs out the call
 *             still completes, its outputs are undefined and kda_chunk_fwd_status
 *             reports KDA_ERR_EXCHANGE.
 * Matrix products run on MFMA: bf16 operands with fp32 accumulation for
 * KDA_BF16, fp32 operands for KDA_F32.  The state is carried in fp32. */
int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* z,
                  const float* A_log, const float* dt_bias, const void* beta,
                  const float* state_in, float scale, int chunk,
                  void* o, float* state_out,
                  void* workspace, size_t workspace_bytes,
                  int B, int H, int T, int K, int V, int dtype, void* stream);

/* Bytes of device workspace kda_chunk_fwd_norm needs for these sizes: nonzero when
 * V > 64 (a head's two value tiles exchange per-token sums of squares), 0 otherwise or
 * on bad sizes or a dtype other than KDA_BF16. */
size_t kda_chunk_fwd_norm_workspace_bytes(int B, int H, int T, int K, int V, int dtype);

/* kda_chunk_fwd followed by the module's output RMSNorm, fused into the output stage
 * ("kdafix" page, "Fix 2 -- read scale": the module normalises the read right after
 * it, which absorbs a constant factor on o, such as the read scale, up to
 * O(eps / mean(o^2))).  The norm is taken over the V outputs of each token within its
 * head, with one weight row per head:
 *   o[b,h,t,:] = r[b,h,t,:] / sqrt(mean_v r[b,h,t,v]^2 + eps) * norm_weight[h,:]
 * where r = scale * (read) is the output kda_chunk_fwd would store, here kept in fp32
 * until the division; o is stored as bf16.  Same inputs, state handling, layouts and
 * checks as kda_chunk_fwd, for KDA_BF16 only (KDA_ERR_DTYPE otherwise); the blocks are
 * 32 tokens whatever `chunk` (16, 32 or 64) says.
 *   norm_weight (H,V) f32, or NULL for all ones (a model with one weight shared by all
 *               heads passes it H times); no output may overlap it.
 *   eps         >= 0 and finite (KDA_ERR_SHAPE otherwise); with eps = 0 a token whose
 *               outputs are all zero gives NaN, as the formula does.
 *   workspace   device buffer of kda_chunk_fwd_norm_workspace_bytes() bytes, 256-byte
 *               aligned, overlapping no argument; NULL when that size is 0.  It must be
 *               zero-filled before its first call (hipMemset) and serve this function
 *               only; each call leaves it ready for the next (every call advances an
 *               epoch in it, and a word counts only when it carries the current one).
 *               When V > 64
 *               the two 64-column tiles of a head run in two workgroups of one XCD,
 *               which exchange per-token sums of squares through it; two calls in flight
 *               at once must not share it.  Their waits are bounded
 *               (kda_set_exchange_timeout_us); if one runs out the call completes, its o
 *               is undefined and kda_chunk_fwd_status reports KDA_ERR_EXCHANGE.
 * o must be 8-byte aligned. */
int kda_chunk_fwd_norm(const void* q, const void* k, const void* v, const void* z,
                       const float* A_log, const float* dt_bias, const void* beta,
                       const float* state_in, float scale, int chunk,
                       const float* norm_weight, float eps,
                       void* o, float* state_out,
                       void* workspace, size_t workspace_bytes,
                       int B, int H, int T, int K, int V, int dtype, void* stream);

/* Outcome of the last call of kda_chunk_fwd / kda_chunk_fwd_scalar (paired) or
 * kda_chunk_fwd_norm (V > 64) that used this workspace: synchronizes `stream`, reads the
 * workspace's status word and clears it.
 * KDA_OK, or KDA_ERR_EXCHANGE when a wait between the workgroups of a head ran out or
 * they were not placed on one XCD (that call's outputs are undefined); KDA_ERR_HIP if
 * the synchronization or the copy fails. */
int kda_chunk_fwd_status(void* workspace, void* stream);

/* Bound of each wait of the paired forward for the other workgroup of its head, in
 * microseconds (default 1000000).  0 makes every such wait give up at once, which
 * exercises the failure path (the call then reports KDA_ERR_EXCHANGE).  Process-wide;
 * takes effect for calls made after it.  Returns KDA_OK. */
int kda_set_exchange_timeout_us(unsigned long long us);

/* One decode step of the same recurrence (the page's "decode prefill read" folds
 * the scale into q the same way).  Inputs are one token per (b,h):
 *   q, k, z (B,H,K) `dtype`;  v (B,H,V) `dtype`;  beta (B,H) `dtype`
 *   state   (B,H,K,V) f32, read and updated in place
 *   o       (B,H,V) `dtype`, must not alias an input
 * Bound by the state's HBM traffic: 2*K*V*4 bytes per head and token. */
int kda_recurrent_step(const void* q, const void* k, const void* v, const void* z,
                       const float* A_log, const float* dt_bias, const void* beta,
                       float* state, float scale, void* o,
                       int B, int H, int K, int V, int dtype, void* stream);

/* Scalar-decay special case of kda_chunk_fwd: one gate input per token and head and
 * one bias per head, so every key channel of a head decays by the same factor,
 *   g[b,h,t] = -exp(clamp(A_log[h], -10, 20)) * softplus(a[b,h,t] + dt_bias[h])
 * (the released gate of the "kdafix" page, "Fix 1 -- decay form", with an input that
 * is constant over the channels).  The result equals kda_chunk_fwd with z[b,h,t,:] =
 * a[b,h,t] and dt_bias[h,:] = dt_bias[h].
 *   a        (B,H,T) `dtype`, aligned to one element
 *   dt_bias  (H) f32 or NULL (= 0)
 * Every other argument, layout, alignment rule, error and the aliasing rules are those
 * of kda_chunk_fwd (a must not alias o or state_out). */
int kda_chunk_fwd_scalar(const void* q, const void* k, const void* v, const void* a,
                         const float* A_log, const float* dt_bias, const void* beta,
                         const float* state_in, float scale, int chunk,
                         void* o, float* state_out,
                         void* workspace, size_t workspace_bytes,
                         int B, int H, int T, int K, int V, int dtype, void* stream);

/* Decode step under the scalar decay: as kda_recurrent_step with a (B,H) `dtype` (one
 * gate input per sequence and head) and dt_bias (H) f32 or NULL. */
int kda_recurrent_step_scalar(const void* q, const void* k, const void* v, const void* a,
                              const float* A_log, const float* dt_bias, const void* beta,
                              float* state, float scale, void* o,
                              int B, int H, int K, int V, int dtype, void* stream);

/* Bytes of device workspace kda_chunk_bwd needs for these sizes (0 on bad sizes). */
size_t kda_chunk_bwd_workspace_bytes(int B, int H, int T, int K, int V, int chunk);

/* Adjoint of the forward for L = sum(o * d_o) + sum(state_out * d_state_out)
 * ("The fused KDA adjoint" page: the gradient blocks dq dk dv dg db dstate of its
 * two-chunk fixture; the intra-chunk and the reverse inter-chunk recurrence).
 * Inputs as kda_chunk_fwd, plus
 *   d_o          (B,H,T,V) in `dtype`
 *   d_state_out  (B,H,K,V) f32 or NULL (= 0)
 * Outputs, all float32, none may alias an input:
 *   dq, dk (B,H,T,K) w.r.t. the unscaled q and k;  dv (B,H,T,V);
 *   dg (B,H,T,K) w.r.t. the log-decay g;  dbeta (B,H,T);  dstate_in (B,H,K,V).
 * workspace: device buffer of at least kda_chunk_bwd_workspace_bytes(), 16-byte
 * aligned (KDA_ERR_ALIGN otherwise: the kernels read it in 16-byte vectors); its
 * contents on entry are ignored.  q, k, v and d_o must be 16-byte aligned, z 8-byte
 * (KDA_ERR_ALIGN).  B * H <= 65535.  Currently dtype must be KDA_F32.  The blocks are
 * 32 tokens whatever `chunk` (16, 32 or 64) says; a block whose decay inside it is too
 * strong for the factorised form (beyond a factor exp(60) either side of its middle)
 * is evaluated token by token, exactly. */
int kda_chunk_bwd(const void* q, const void* k, const void* v, const void* z,
                  const float* A_log, const float* dt_bias, const void* beta,
                  const float* state_in, float scale, int chunk,
                  const void* d_o, const float* d_state_out,
                  float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dstate_in,
                  void* workspace, size_t workspace_bytes,
                  int B, int H, int T, int K, int V, int dtype, void* stream);

/* Bytes of device workspace kda_gate_bwd needs for these sizes (0 when T = 0 or on
 * bad sizes). */
size_t kda_gate_bwd_workspace_bytes(int B, int H, int T, int K);

/* Adjoint of kda_gate for a cotangent dg on g ("kdafix" page, "Fix 1 -- decay form",
 * differentiated): with x = z + dt_bias and m = exp(clamp(A_log, -10, 20)),
 *   dz         (B,H,T,K) f32 = -m * sigmoid(x) * dg        (NULL: not written)
 *   dA_log     (H) f32 = sum over b, t, c of dg * g, or 0 where A_log lies outside
 *              [-10, 20] (the clamp holds the multiplier constant there)   (NULL: not written)
 *   d_dt_bias  (H,K) f32 = sum over b, t of dz  (also when dt_bias is NULL)  (NULL: not written)
 * Inputs: z (B,H,T,K) in `dtype`, A_log (H) f32, dt_bias (H,K) f32 or NULL (= 0),
 * dg (B,H,T,K) f32 (as kda_chunk_bwd returns it).  At least one output is needed.
 * workspace: device buffer of at least kda_gate_bwd_workspace_bytes() (may be NULL
 * when that is 0); contents on entry ignored.  dz may be dg itself (computed in
 * place); no other overlap between outputs, inputs and workspace is allowed.  The
 * parameter gradients are reduced in a fixed order (bitwise repeatable).  K >= 1. */
int kda_gate_bwd(const void* z, const float* A_log, const float* dt_bias, const float* dg,
                 float* dz, float* dA_log, float* d_dt_bias,
                 void* workspace, size_t workspace_bytes,
                 int B, int H, int T, int K, int dtype, void* stream);

/* Bytes of the device array kda_gate_bwd_noalloc uses in place of a workspace (per GPU). */
#define KDA_GATE_BWD_SCRATCH_BYTES ((size_t)16 << 20)

/* kda_gate_bwd without a workspace argument, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, hosts that forbid it).  The
 * per-tile partial sums go to a 16 MiB array inside the library, one per GPU, resident
 * until the process ends; this call allocates nothing.  Same arguments, outputs, checks
 * and results as kda_gate_bwd (bit-identical).  Sizes whose kda_gate_bwd_workspace_bytes()
 * exceeds KDA_GATE_BWD_SCRATCH_BYTES give KDA_ERR_SCRATCH before anything runs.  `stream`
 * must belong to the current device.  Every call on a GPU shares that GPU's array: two
 * calls that may run at the same time on one GPU (different streams, no ordering between
 * them) race and must not be made; calls in one stream are ordered and safe.  Nothing in
 * the array needs to start at zero (every partial sum is written before it is read). */
int kda_gate_bwd_noalloc(const void* z, const float* A_log, const float* dt_bias, const float* dg,
                         float* dz, float* dA_log, float* d_dt_bias,
                         int B, int H, int T, int K, int dtype, void* stream);

/* Static string for a status code ("ok", "null pointer", ...). Never NULL. */
const char* kda_status_string(int status);

/* Copies up to n counters into out and returns how many exist (KDA_NUM_COUNTERS).
 * Counters are process-wide and monotonic: calls accepted per entry point and
 * calls rejected with an error status (modelled on the page's dispatch counters,
 * "The fused KDA adjoint" page, section 6). */
#define KDA_NUM_COUNTERS 6
#define KDA_COUNTER_GATE 0
#define KDA_COUNTER_CHUNK_FWD 1
#define KDA_COUNTER_RECURRENT_STEP 2
#define KDA_COUNTER_CHUNK_BWD 3
#define KDA_COUNTER_REJECTED 4
#define KDA_COUNTER_GATE_BWD 5
int kda_get_counters(unsigned long long* out, int n);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
