/*
 * varlen_causal_attn.h -- C ABI of the MI355X (gfx950) varlen causal attention
 * forward for packed multi-user sequences.
 *
 * Operation (all entry points that compute): for every user u with rows
 * s_u = cu_seqlens[u] .. cu_seqlens[u+1]-1 and every head h,
 *     out[s_u+i, h*64 : h*64+64] = sum_{j<=i} softmax_j(scale * q_i . k_j) v_j
 * where q, k, v are head h's 64-column slices of the packed qkv rows of user u.
 * Attention is causal inside a user (diagonal included) and never crosses users.
 *   - Packed stream and offsets: cti2026 README (git.firegun.top/Days-gone/cti2026),
 *     input table (user_offsets = [0, len1, len1+len2, ..., total_tokens]).
 *   - Kernel contract (per-user segment addressing from cu_seqlens, causal
 *     pruning at the diagonal, fp32 online softmax, bf16 write-back): same README,
 *     FlashAttention_Varlen section, "operator design".
 *   - softmax(Q K^T / sqrt(d)) V: CTI-Inference-Opt inference optimisation plan
 *     (推理优化方案), section 5.2.
 *   - A max_seqlen larger than the true maximum and zero-length users leave the
 *     result unchanged: cti2026 README, CUDA Graph section ("fixed attention grid",
 *     "variable num_seqs").
 *
 * Layouts (row-major, device memory, caller-owned):
 *   qkv  bf16 [T, 3*n_heads*64]: q in columns [0, H*64), k in [H*64, 2*H*64),
 *        v in [2*H*64, 3*H*64); head h at h*64 .. h*64+63 inside each block.
 *        T = cu_seqlens[num_users].
 *   out  bf16 [T, n_heads*64]: head h at columns h*64 .. h*64+63.  Only rows
 *        that belong to a user are written; out must not overlap qkv.
 *   cu_seqlens int32 [num_users+1], cu_seqlens[0] = 0, non-decreasing; repeated
 *        values (zero-length users) are allowed.
 *
 * Execution: every compute entry point is asynchronous on `stream`.  It performs
 * no host synchronisation and reads no device data on the host.  Arguments are
 * checked on the host before any device work; the contents of cu_seqlens are a
 * precondition (a user longer than max_seqlen, or decreasing offsets, give
 * unspecified output for that user but never an access outside qkv/out rows
 * [0, cu_seqlens[num_users]) ).  The library keeps no pointer after return.
 *
 * Limits: head_dim == 64; n_heads >= 1; scale finite and > 0;
 *         0 <= max_seqlen <= VLCA_MAX_SEQLEN; T < 2^31; num_users >= 0.
 *         num_users == 0 or max_seqlen == 0 is a successful no-op.
 *
 * Return value: 0 (VLCA_OK) on success, a negative VLCA_ERR_* code otherwise;
 * varlen_causal_attn_strerror() names it.
 */
#ifndef VARLEN_CAUSAL_ATTN_H
#define VARLEN_CAUSAL_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP runtime's opaque stream handle (identical typedef to HIP's own). */
typedef struct ihipStream_t* hipStream_t;

#define VLCA_TILE_ROWS 64          /* query rows per work item, keys per K/V tile  */
#define VLCA_MAX_SEQLEN 262144     /* max_seqlen upper limit (4096 q-tiles a user) */
#define VLCA_NOALLOC_MAX_ITEMS 524288  /* worklist items of varlen_causal_attn_fwd_noalloc */

enum {
  VLCA_OK = 0,
  VLCA_ERR_NULL_POINTER = -1,    /* a required pointer is NULL (num_users > 0)       */
  VLCA_ERR_NEGATIVE_SIZE = -2,   /* num_users < 0 or max_seqlen < 0                  */
  VLCA_ERR_HEAD_DIM = -3,        /* head_dim != 64                                   */
  VLCA_ERR_N_HEADS = -4,         /* n_heads < 1 or 3*n_heads*64 columns overflow     */
  VLCA_ERR_SCALE = -5,           /* scale not finite or not > 0                      */
  VLCA_ERR_TOO_LARGE = -6,       /* max_seqlen > VLCA_MAX_SEQLEN or worklist > 2^31  */
  VLCA_ERR_CAPACITY = -7,        /* caller worklist buffer smaller than required     */
  VLCA_ERR_ALIAS = -8,           /* qkv and out are the same pointer                 */
  VLCA_ERR_WORKSPACE = -9,       /* library workspace could not be allocated        */
  VLCA_ERR_HIP = -10,            /* a HIP runtime call or kernel launch failed       */
  VLCA_ERR_SCRATCH = -11,        /* varlen_causal_attn_fwd_noalloc: the batch needs a
                                    larger worklist than VLCA_NOALLOC_MAX_ITEMS      */
  VLCA_ERR_BUCKETS = -12,        /* runner bucket sizes not positive and increasing,
                                    or more than 64 buckets                          */
  VLCA_ERR_MASK = -13,           /* mask description out of range (see vlca_mask)    */
  VLCA_ERR_SHAPE = -14,          /* neighbour kernels: d_model != 512, or an output
                                    width that is not a positive multiple of 128     */
  VLCA_ERR_ALIGN = -15           /* a pointer breaks the alignment rule below         */
};

/*
 * Alignment.  The kernels move 16-byte chunks: every bf16 tensor (qkv, out, dout,
 * dqkv, x, gamma, beta, the weights, residual, y, a graph runner's static
 * buffers) and a caller's worklist items must be 16-byte aligned; the bias
 * vectors 8-byte aligned; cu_seqlens, lse, the worklist count, num_contexts and
 * num_targets 4-byte aligned.  Else VLCA_ERR_ALIGN, before any device work.
 * (Allocations of hipMalloc and of torch satisfy all of them.)
 */

/*
 * Forward pass.  Runs the segment scheduler (a compact (user, q-tile) worklist:
 * users grouped by length class floor(log2(q-tiles)), longest class first, users
 * ascending inside a class, each user's q-tiles adjacent, last q-tile first) and
 * the attention kernel on `stream`.
 *
 * Launch plans.  Small batches (num_users <= 256 and
 * num_users*ceil(max_seqlen/64)*n_heads at most 16 items per resident
 * workgroup; varlen_causal_attn_single_kernel() tells) run as one kernel in
 * which every workgroup locates its own items.  Larger batches run the
 * scheduler kernel and the attention kernel over a worklist.
 *
 * Key-range splitting.  When the batch's users with rows, with the long items
 * split, give at most one round of resident workgroups' work units, the items
 * of more than max(ceil(t/2), 4) key tiles of a user of t q-tiles run as two
 * key-range parts on different workgroups whose softmax states are merged.  The
 * decision depends only on the lengths of the non-empty users, n_heads and the
 * device -- never on zero-length users, max_seqlen, the launch plan or graph
 * capture -- so those never change the output bits.  Split and whole items agree
 * within rounding; the worklist entry points below always run items whole.
 *
 * Library state.  Each (device, stream) has a worklist buffer with its work
 * counters and, once a call with max_seqlen > 256 has run, a split-state pool of
 * about 19 MB.  The first call on a stream that needs more allocates it
 * (hipMalloc) without synchronising; also during graph capture, when the
 * allocation is made at once (the thread's capture mode is relaxed for it) and
 * nothing is recorded into the graph.  A buffer that has to grow is replaced and
 * the old one kept until the process ends, so graphs captured earlier stay
 * valid.  Calls on one stream run in stream order and share that state; so does
 * every graph captured on that stream: replay such a graph in stream order with
 * the stream's other calls (e.g. on the same stream), never concurrently with
 * them or with another graph captured on it.  Calls on different streams use
 * different state and may overlap.
 *   qkv        device, bf16 [T, 3*n_heads*head_dim] (see Layouts)
 *   cu_seqlens device, int32 [num_users+1]
 *   num_users  number of segments U (>= 0)
 *   max_seqlen upper bound on every user's length (need not be the true maximum)
 *   n_heads    heads H (>= 1); head_dim must be 64
 *   scale      multiplier of q.k before the softmax (1/8 for head_dim 64)
 *   out        device, bf16 [T, n_heads*head_dim]
 *   stream     HIP stream (NULL = default stream)
 * Errors: the VLCA_ERR_* codes above (VLCA_ERR_WORKSPACE if an allocation
 * fails); no device work is issued when a call fails its checks.
 */
int varlen_causal_attn_fwd(const void* qkv, const int32_t* cu_seqlens, int num_users,
                           int max_seqlen, int n_heads, int head_dim, float scale,
                           void* out, hipStream_t stream);

/*
 * HSTU-style mask variants (recsys README, HSTU section: hstu_attn_varlen_func's
 * num_contexts, num_targets and window_size, and its mask list -- no mask, local
 * sliding window, causal, contextual + causal, target + causal).  A user of
 * length L with c = num_contexts[u] context tokens and g = num_targets[u]
 * candidate tokens at its end (nc = L - g; both clamped to the user) is
 * [context][history][candidates].  Query row i sees key j of its own user when
 *   window_right == 0 (causal):
 *     j < c                                        (every row sees the context),
 *     i >= c and max(c, lo(i)) <= j <= min(i, nc-1) (history, causal, windowed),
 *     i >= nc and gs(i) <= j <= i                  (its own candidate group);
 *     (so a context row sees exactly the context: bidirectional inside it)
 *   otherwise (num_contexts and num_targets NULL):
 *     lo(i) <= j <= hi(i),
 * with lo(i) = max(0, i - window_left) (window_left >= 0; -1 = no bound),
 * hi(i) = min(L-1, i + window_right) (window_right >= 0; -1 = no bound), and
 * gs(i) = nc + floor((i - nc) / target_group_size) * target_group_size.
 */
typedef struct vlca_mask {
  const int32_t* num_contexts;  /* device int32 [num_users], or NULL (no context tokens)   */
  const int32_t* num_targets;   /* device int32 [num_users], or NULL (no candidate tokens) */
  int target_group_size;        /* >= 1                                                    */
  int window_left;              /* >= -1                                                   */
  int window_right;             /* >= -1; must be 0 when num_contexts or num_targets is set */
} vlca_mask;

/*
 * Forward with a mask variant.  Arguments and layouts as for
 * varlen_causal_attn_fwd; mask (host pointer, read during the call) as above.
 * mask NULL, or the plain causal mask (no contexts, no targets, window (-1, 0)),
 * runs varlen_causal_attn_fwd itself (same bits).  Other masks run a separate
 * kernel whose result equals the definition within rounding: on the batches
 * where varlen_causal_attn_fwd runs one kernel (varlen_causal_attn_single_kernel)
 * it alone, locating its own items (no worklist, no allocation); otherwise over
 * the stream's worklist (allocated or grown on first need, never freed).  Both
 * give the same bits.  Errors as for varlen_causal_attn_fwd, plus VLCA_ERR_MASK.
 */
int varlen_causal_attn_fwd_masked(const void* qkv, const int32_t* cu_seqlens, int num_users,
                                  int max_seqlen, int n_heads, int head_dim, float scale,
                                  const vlca_mask* mask, void* out, hipStream_t stream);

/*
 * The attention's neighbours in the packed Transformer layer (cti2026 README,
 * Transformer-layer listing: residual = x; x = LayerNorm(x); qkv = Linear_qkv(x);
 * attn_out = FlashAttention_Varlen(qkv, user_offsets); x = residual +
 * Linear_out(attn_out)), with their elementwise work fused into the products.
 * All tensors bf16, row-major, device, caller-owned; T = total_tokens rows;
 * weights in nn.Linear's layout [out_features, in_features]; fp32 accumulation,
 * one rounding to bf16 of each output.  d_model must be 512.
 *
 * varlen_causal_attn_ln_qkv: qkv[T, n_out] = LayerNorm(x)[T, 512] w[n_out, 512]^T
 * + b[n_out], LayerNorm(x) = (x - mean) / sqrt(var + eps) * gamma + beta over each
 * row's 512 columns (population variance), rounded to bf16 before the product.
 * n_out = 3 * n_heads * 64 gives the forward's qkv layout; a positive multiple
 * of 128, at most 65536 (else VLCA_ERR_SHAPE).  qkv must not overlap x.
 */
int varlen_causal_attn_ln_qkv(const void* x, const void* gamma, const void* beta, float eps,
                              const void* w_qkv, const void* b_qkv, int total_tokens, int d_model,
                              int n_out, void* qkv, hipStream_t stream);

/*
 * varlen_causal_attn_out_residual: y[T, n_out] = residual[T, n_out] +
 * attn[T, 512] w[n_out, 512]^T + b[n_out] (n_out = d_model = 512 in the layer; a
 * positive multiple of 128, at most 65536).  y may be residual itself (each workgroup reads its
 * tile of residual before it writes that tile) but not attn.
 */
int varlen_causal_attn_out_residual(const void* attn, const void* w_out, const void* b_out,
                                    const void* residual, int total_tokens, int d_model, int n_out,
                                    void* y, hipStream_t stream);

/*
 * Training forward: varlen_causal_attn_fwd (same plan, split decision and output
 * bits) that also writes, for every row t of a user and head h,
 *     lse[t*n_heads + h] = ln sum_{j <= i} exp(scale * q_i . k_j)
 * (fp32 [T, n_heads], device, caller-owned; rows of no user are not written), the
 * row log-sum-exp that varlen_causal_attn_bwd uses to recompute the softmax.
 * Errors as for varlen_causal_attn_fwd; lse NULL with work to do is
 * VLCA_ERR_NULL_POINTER.
 */
int varlen_causal_attn_fwd_lse(const void* qkv, const int32_t* cu_seqlens, int num_users,
                               int max_seqlen, int n_heads, int head_dim, float scale,
                               void* out, float* lse, hipStream_t stream);

/*
 * Backward pass: with L a loss and dout = dL/dout, writes dqkv = dL/dqkv, bf16
 * [T, 3*n_heads*64] in the qkv layout (dq, dk, dv blocks; the training step of
 * the same op: the recsys README, FusedHSTULayer backward, runs the attention
 * backward between the layer's other backward kernels).  Per user and head, with
 * P the forward's causal softmax recomputed from lse:
 *     D = rowsum(dout o out),  dS = P o (dout V^T - D),
 *     dV = P^T dout,  dK = scale dS^T Q,  dQ = scale dS K.
 *   qkv, cu_seqlens, num_users, max_seqlen, n_heads, head_dim, scale: as given to
 *          varlen_causal_attn_fwd_lse;
 *   out    its bf16 output [T, n_heads*64];  lse: its fp32 [T, n_heads];
 *   dout   bf16 [T, n_heads*64];
 *   dqkv   bf16 [T, 3*n_heads*64], caller-owned, distinct from the inputs.  Every
 *          row of a user is written; rows of no user are not touched.
 * Deterministic (no atomics).  Uses the stream's worklist (as the forward's
 * scheduler plan does: allocated or grown on first need, never freed).
 * Asynchronous on `stream`; errors as for varlen_causal_attn_fwd, plus
 * VLCA_ERR_ALIAS if dqkv is one of qkv, out, dout.
 */
int varlen_causal_attn_bwd(const void* qkv, const void* out, const void* dout, const float* lse,
                           const int32_t* cu_seqlens, int num_users, int max_seqlen, int n_heads,
                           int head_dim, float scale, void* dqkv, hipStream_t stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, serving loops
 * that forbid hipMalloc): the same computation as varlen_causal_attn_fwd, with
 * the same launch plan and split decision and hence the same output bits, but
 * the worklist, work counters and split-state pool live in a fixed scratch array
 * of about 27 MB per device (loaded with the library's code object; its device
 * address is looked up once per device on the first call there).  No memory is
 * allocated and no stream is synchronised.  Every call on a device shares that
 * device's array, which keeps the last call's contents (the scheduler kernel
 * re-initialises the counters it needs; the split arrival counters are zero at
 * load and every call leaves them zero): calls that overlap on one device --
 * on different streams, or graph replays beside other calls -- race and must
 * not be made.  Limit: a batch on the scheduler plan (varlen_causal_attn_single_kernel()
 * gives 0) must need at most VLCA_NOALLOC_MAX_ITEMS worklist items
 * (num_users*ceil(max_seqlen/64)), else VLCA_ERR_SCRATCH before any device work.
 * Arguments, layouts and other errors as for varlen_causal_attn_fwd.
 */
int varlen_causal_attn_fwd_noalloc(const void* qkv, const int32_t* cu_seqlens, int num_users,
                                   int max_seqlen, int n_heads, int head_dim, float scale,
                                   void* out, hipStream_t stream);

/*
 * Worklist size (in items) needed by varlen_causal_attn_build_worklist and
 * varlen_causal_attn_fwd_worklist: num_users*ceil(max_seqlen/64).  Pure host
 * arithmetic.  Writes it to *capacity.
 */
int varlen_causal_attn_worklist_capacity(int num_users, int max_seqlen, int64_t* capacity);

/*
 * Segment scheduler alone (the same device code the forward runs).  Writes, on
 * `stream`, the compact worklist for 64-row q-tiles: items[4*i .. 4*i+3] =
 * (user, q_tile, row_start, length) for i < *count.  Order: users grouped by
 * length class floor(log2(q-tiles of the user)), highest class first; inside a
 * class, users ascending; a user's items adjacent, from its last q-tile (the
 * most key tiles) down to q-tile 0.  Users with no rows give no items; entries
 * from *count on are left untouched.  A user's tile count is clamped to
 * ceil(max_seqlen/64).
 *   items     device, int32 [capacity][4], caller-owned (may be NULL if capacity
 *             needed is 0)
 *   capacity  items available; must be >= varlen_causal_attn_worklist_capacity()
 *   count     device, int32 [1], caller-owned: number of items
 */
int varlen_causal_attn_build_worklist(const int32_t* cu_seqlens, int num_users, int max_seqlen,
                                      int32_t* items, int64_t capacity, int32_t* count,
                                      hipStream_t stream);

/*
 * Attention kernel alone, over a worklist that varlen_causal_attn_build_worklist
 * wrote (same cu_seqlens, num_users, max_seqlen) earlier in stream order; the
 * kernel reads *count on the device.  Uses no library workspace, so it may be
 * captured in a HIP graph together with the scheduler call, and one worklist can
 * serve several calls over the same batch (e.g. every layer of a model).
 * Arguments as for varlen_causal_attn_fwd, plus the caller's items/capacity/count.
 */
int varlen_causal_attn_fwd_worklist(const void* qkv, const int32_t* cu_seqlens, int num_users,
                                    int max_seqlen, int n_heads, int head_dim, float scale,
                                    const int32_t* items, int64_t capacity, const int32_t* count,
                                    void* out, hipStream_t stream);

/*
 * Which launch plan varlen_causal_attn_fwd uses on the current device for these
 * sizes: writes 1 to *single_kernel when it runs one kernel that orders its own
 * work (no worklist buffer), 0 when it runs the scheduler and the attention
 * kernel over the stream's worklist.  No device work; queries the
 * device's CU count and the kernel's occupancy once.  Errors as for the size
 * checks of varlen_causal_attn_fwd (VLCA_ERR_HIP without a device).
 */
int varlen_causal_attn_single_kernel(int num_users, int max_seqlen, int n_heads, int* single_kernel);

/*
 * Bucketed graph runner (cti2026 README, CUDA Graph section: bucketed padding,
 * fixed attention grid, no host synchronisation, variable number of users).
 * Packed batches of varying size replay one of a few captured HIP graphs:
 *   - bucket b holds up to bucket_tokens[b] tokens (strictly increasing, e.g.
 *     2560, 3072, ..., 7168); a batch of T tokens uses the smallest bucket with
 *     T <= bucket_tokens[b], whose graph runs the forward over the static buffers
 *     with the constant max_seqlen = bucket_tokens[b];
 *   - the offsets have a fixed length max_users + 1: a batch with fewer users is
 *     padded on the device with zero-length users (no host read of device data);
 *   - a batch above the top bucket, or with more than max_users users, runs the
 *     eager forward instead (with the caller's max_seqlen);
 *   - every bucket's graph is captured at creation (precapture != 0) or on its
 *     first use.
 * The output equals varlen_causal_attn_fwd's on the same batch bit for bit (the
 * forward's result does not depend on max_seqlen or zero-length users).
 *
 * qkv_static, out_static: caller-owned device buffers of at least top-bucket rows
 * of the qkv and out layouts, kept alive until the runner is destroyed; the graphs
 * read and write them.  A producer may write a batch's qkv rows straight into
 * qkv_static and read the result from out_static (run() then copies nothing);
 * other buffers are copied in and out on the stream.  The runner owns the
 * padded offsets and a stream of its own on which it captures (its graphs share
 * that stream's library state); graphs are launched on run()'s stream.  A
 * runner is used on one stream at a time; runs on it are ordered by that stream.
 * create() synchronises the device once (clearing the offsets) and allocates;
 * run() allocates only when it captures a bucket lazily.
 */
typedef struct vlca_graph_runner vlca_graph_runner;

int varlen_causal_attn_runner_create(const int32_t* bucket_tokens, int n_buckets, int max_users, int n_heads,
                                     float scale, void* qkv_static, void* out_static, int precapture,
                                     vlca_graph_runner** runner);

/*
 * Runs one batch: qkv, cu_seqlens (num_users + 1 offsets), out as for
 * varlen_causal_attn_fwd, total_tokens = cu_seqlens[num_users] (host value; it
 * picks the bucket, and offsets are clamped to it on the device), max_seqlen
 * for the eager fallback.  *bucket_used (may be NULL) receives the bucket index
 * or -1 for the eager path.  Asynchronous on `stream`.
 */
int varlen_causal_attn_runner_run(vlca_graph_runner* runner, const void* qkv, const int32_t* cu_seqlens,
                                  int num_users, int total_tokens, int max_seqlen, void* out, hipStream_t stream,
                                  int* bucket_used);

/* The bucket a batch would use (-1: the eager path).  Host arithmetic only. */
int varlen_causal_attn_runner_bucket(const vlca_graph_runner* runner, int num_users, int total_tokens, int* bucket);

/* Number of buckets whose graph has been captured. */
int varlen_causal_attn_runner_captured(const vlca_graph_runner* runner, int* n_captured);

/* Waits for the device, then frees the graphs, the offsets and the capture
 * stream (not the caller's static buffers).  NULL is a no-op. */
int varlen_causal_attn_runner_destroy(vlca_graph_runner* runner);

/* Query rows per work item (and keys per K/V tile): VLCA_TILE_ROWS. */
int varlen_causal_attn_tile_rows(void);

/* Static, NUL-terminated description of a return code. */
const char* varlen_causal_attn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* VARLEN_CAUSAL_ATTN_H */
