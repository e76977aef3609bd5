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
  VLCA_ERR_WORKSPACE = -9,       /* library workspace could not be (re)allocated,
                                    or would need to grow while the stream captures  */
  VLCA_ERR_HIP = -10             /* a HIP runtime call or kernel launch failed       */
};

/*
 * Forward pass.  Runs the segment scheduler (a compact (user, q-tile) worklist:
 * users grouped by length class floor(log2(q-tiles)), longest class first, each
 * user's q-tiles adjacent, last q-tile first) and the attention kernel on
 * `stream`.
 * Small batches (num_users <= 256 and num_users*ceil(max_seqlen/64)*n_heads at most
 * 16 items per resident workgroup; varlen_causal_attn_single_kernel() tells) run
 * as one kernel in which every workgroup locates its own items.  In a batch of
 * at most 256 users whose items, with the long ones split, fit in one round of
 * resident workgroups, the items of more than max(ceil(t/2), 4) key tiles of a
 * user of t q-tiles run as two key-range parts whose softmax states are merged
 * (on either plan, with the same decision, so max_seqlen does not change the
 * bits).  The parts meet in a fixed-size pool (about 38 MB) kept per (device,
 * stream), allocated by the first call on a stream that may split (hipMalloc;
 * while the stream is being captured and has no pool yet, the call runs its
 * items whole instead).  Split and whole items agree within rounding; the
 * worklist entry points below always run items whole.  Larger batches keep their worklist
 * in a library-owned device buffer kept per (device, stream) and grown on demand:
 * the first call on a stream with a larger num_users*ceil(max_seqlen/64) allocates
 * it (hipMalloc) after synchronising that stream, which is not allowed while the
 * stream is being captured (VLCA_ERR_WORKSPACE then -- make one eager call of the
 * same or larger size first).  Two calls that overlap on the same stream cannot
 * happen (stream order); calls on different streams use different buffers.
 *   qkv        device, bf16 [T, 3*n_heads*head_dim] (see Layouts)
 *   cu_seqlens device, int32 [num_users+1]
 *   num_users  number of segments U (>= 0)
 *   max_seqlen upper bound on every user's length (need not be the true maximum)
 *   n_heads    heads H (>= 1); head_dim must be 64
 *   scale      multiplier of q.k before the softmax (1/8 for head_dim 64)
 *   out        device, bf16 [T, n_heads*head_dim]
 *   stream     HIP stream (NULL = default stream)
 */
int varlen_causal_attn_fwd(const void* qkv, const int32_t* cu_seqlens, int num_users,
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
 * (user, q_tile, row_start, length) for i < *count, ordered by q_tile
 * descending and, within one q_tile, by user ascending; users with no rows give
 * no items; entries from *count on are left untouched.  A user's tile count is
 * clamped to ceil(max_seqlen/64).
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
 * work (no worklist buffer; at most the fixed split-state pool), 0 when it runs
 * the scheduler and the attention kernel over the library workspace.  No device work; queries the
 * device's CU count and the kernel's occupancy once.  Errors as for the size
 * checks of varlen_causal_attn_fwd (VLCA_ERR_HIP without a device).
 */
int varlen_causal_attn_single_kernel(int num_users, int max_seqlen, int n_heads, int* single_kernel);

/* Query rows per work item (and keys per K/V tile): VLCA_TILE_ROWS. */
int varlen_causal_attn_tile_rows(void);

/* Static, NUL-terminated description of a return code. */
const char* varlen_causal_attn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* VARLEN_CAUSAL_ATTN_H */
