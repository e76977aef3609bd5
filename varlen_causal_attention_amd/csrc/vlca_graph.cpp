// Bucketed graph runner for the forward pass.
//
// The cti2026 README (git.firegun.top/Days-gone/cti2026), CUDA Graph section,
// replays captured graphs instead of launching kernels one by one, and makes the
// varying packed batches fit static graphs this way: token counts are rounded up
// to buckets (2560 .. 7168 in steps of 512), each bucket has its own graph over
// fixed [S_PAD, ...] buffers captured with the constant max_seqlen = S_PAD, the
// offsets array has a fixed length with short batches padded on the device by
// zero-length users, every bucket is captured ahead of time, and batches above
// the top bucket run eagerly.  Results equal the eager path's bit for bit: here
// that holds because the forward's output does not depend on max_seqlen, on
// zero-length users or on the launch plan.
//
// Each runner captures on a stream of its own, so its graphs share that
// stream's library state (worklist, split pool) and nothing else; graphs are
// launched on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <vector>

#include "varlen_causal_attn.h"
#include "vlca_internal.h"

struct vlca_graph_runner {
  std::vector<int32_t> buckets;        // token capacity of each bucket, increasing
  std::vector<hipGraphExec_t> execs;   // per bucket; null until captured
  std::vector<hipGraph_t> graphs;
  int max_users = 0, n_heads = 0;
  float scale = 0.f;
  void* qkv = nullptr;                 // caller-owned static buffers (top bucket rows)
  void* out = nullptr;
  int32_t* cu = nullptr;               // padded offsets [max_users + 1], library-owned
  hipStream_t capture_stream = nullptr;
  int device = 0;
};

namespace {

constexpr int kMaxBuckets = 64;

size_t qkv_row_bytes(int n_heads) { return static_cast<size_t>(3) * n_heads * vlca::kHeadDim * 2; }
size_t out_row_bytes(int n_heads) { return static_cast<size_t>(n_heads) * vlca::kHeadDim * 2; }

// Captures bucket b: the forward over the static buffers with max_users users
// (padded offsets) and max_seqlen = the bucket's token count.  Nothing runs.
int capture_bucket(vlca_graph_runner* r, int b) {
  hipGraph_t g = nullptr;
  if (hipStreamBeginCapture(r->capture_stream, hipStreamCaptureModeThreadLocal) != hipSuccess) return VLCA_ERR_HIP;
  const int rc = varlen_causal_attn_fwd(r->qkv, r->cu, r->max_users, r->buckets[b], r->n_heads, vlca::kHeadDim,
                                        r->scale, r->out, r->capture_stream);
  const hipError_t e = hipStreamEndCapture(r->capture_stream, &g);
  if (rc != VLCA_OK) {
    if (g != nullptr) (void)hipGraphDestroy(g);
    return rc;
  }
  if (e != hipSuccess || g == nullptr) return VLCA_ERR_HIP;
  hipGraphExec_t x = nullptr;
  if (hipGraphInstantiate(&x, g, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(g);
    return VLCA_ERR_HIP;
  }
  r->graphs[b] = g;
  r->execs[b] = x;
  return VLCA_OK;
}

void release(vlca_graph_runner* r) {
  for (auto& x : r->execs)
    if (x != nullptr) (void)hipGraphExecDestroy(x);
  for (auto& g : r->graphs)
    if (g != nullptr) (void)hipGraphDestroy(g);
  if (r->cu != nullptr) (void)hipFree(r->cu);
  if (r->capture_stream != nullptr) (void)hipStreamDestroy(r->capture_stream);
  delete r;
}

}  // namespace

extern "C" {

int varlen_causal_attn_runner_create(const int32_t* bucket_tokens, int n_buckets, int max_users, int n_heads,
                                     float scale, void* qkv_static, void* out_static, int precapture,
                                     vlca_graph_runner** runner) {
  if (runner == nullptr || bucket_tokens == nullptr || qkv_static == nullptr || out_static == nullptr)
    return VLCA_ERR_NULL_POINTER;
  *runner = nullptr;
  if (n_buckets < 1 || n_buckets > kMaxBuckets) return VLCA_ERR_BUCKETS;
  for (int b = 0; b < n_buckets; ++b) {
    if (bucket_tokens[b] < 1 || (b > 0 && bucket_tokens[b] <= bucket_tokens[b - 1])) return VLCA_ERR_BUCKETS;
    if (bucket_tokens[b] > VLCA_MAX_SEQLEN) return VLCA_ERR_TOO_LARGE;
  }
  if (max_users < 1) return VLCA_ERR_NEGATIVE_SIZE;
  const int64_t tiles = (static_cast<int64_t>(bucket_tokens[n_buckets - 1]) + vlca::kTileRows - 1) / vlca::kTileRows;
  if (static_cast<int64_t>(max_users) * tiles > INT32_MAX) return VLCA_ERR_TOO_LARGE;
  if (n_heads < 1 || n_heads > 65536) return VLCA_ERR_N_HEADS;
  if (!std::isfinite(scale) || !(scale > 0.f)) return VLCA_ERR_SCALE;
  if (qkv_static == out_static) return VLCA_ERR_ALIAS;
  if ((reinterpret_cast<uintptr_t>(qkv_static) & 15) != 0 || (reinterpret_cast<uintptr_t>(out_static) & 15) != 0)
    return VLCA_ERR_ALIGN;

  auto* r = new vlca_graph_runner();
  r->buckets.assign(bucket_tokens, bucket_tokens + n_buckets);
  r->execs.assign(n_buckets, nullptr);
  r->graphs.assign(n_buckets, nullptr);
  r->max_users = max_users;
  r->n_heads = n_heads;
  r->scale = scale;
  r->qkv = qkv_static;
  r->out = out_static;
  if (hipGetDevice(&r->device) != hipSuccess ||
      hipStreamCreateWithFlags(&r->capture_stream, hipStreamNonBlocking) != hipSuccess) {
    r->capture_stream = nullptr;
    release(r);
    return VLCA_ERR_HIP;
  }
  void* p = nullptr;
  if (hipMalloc(&p, static_cast<size_t>(max_users + 1) * sizeof(int32_t)) != hipSuccess) {
    release(r);
    return VLCA_ERR_WORKSPACE;
  }
  r->cu = static_cast<int32_t*>(p);
  // Every user empty until the first run (a captured graph is only launched after
  // run() has written the offsets, but the buffer never holds garbage).
  if (hipMemset(r->cu, 0, static_cast<size_t>(max_users + 1) * sizeof(int32_t)) != hipSuccess) {
    release(r);
    return VLCA_ERR_HIP;
  }
  if (precapture) {
    for (int b = 0; b < n_buckets; ++b) {
      const int rc = capture_bucket(r, b);
      if (rc != VLCA_OK) {
        release(r);
        return rc;
      }
    }
  }
  *runner = r;
  return VLCA_OK;
}

int varlen_causal_attn_runner_bucket(const vlca_graph_runner* runner, int num_users, int total_tokens, int* bucket) {
  if (runner == nullptr || bucket == nullptr) return VLCA_ERR_NULL_POINTER;
  if (num_users < 0 || total_tokens < 0) return VLCA_ERR_NEGATIVE_SIZE;
  *bucket = -1;
  if (num_users > runner->max_users) return VLCA_OK;
  for (size_t b = 0; b < runner->buckets.size(); ++b) {
    if (total_tokens <= runner->buckets[b]) {
      *bucket = static_cast<int>(b);
      break;
    }
  }
  return VLCA_OK;
}

int varlen_causal_attn_runner_run(vlca_graph_runner* runner, const void* qkv, const int32_t* cu_seqlens,
                                  int num_users, int total_tokens, int max_seqlen, void* out, hipStream_t stream,
                                  int* bucket_used) {
  if (runner == nullptr) return VLCA_ERR_NULL_POINTER;
  int b = -1;
  int rc = varlen_causal_attn_runner_bucket(runner, num_users, total_tokens, &b);
  if (rc != VLCA_OK) return rc;
  if (bucket_used != nullptr) *bucket_used = b;
  if (b < 0)  // above the top bucket, or more users than the offsets hold: eager
    return varlen_causal_attn_fwd(qkv, cu_seqlens, num_users, max_seqlen, runner->n_heads, vlca::kHeadDim,
                                  runner->scale, out, stream);
  if (num_users > 0 && (qkv == nullptr || cu_seqlens == nullptr || out == nullptr)) return VLCA_ERR_NULL_POINTER;
  if (qkv != nullptr && qkv == out) return VLCA_ERR_ALIAS;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VLCA_ERR_HIP;
  if (dev != runner->device) return VLCA_ERR_HIP;
  if (runner->execs[b] == nullptr) {  // lazy capture of this bucket
    rc = capture_bucket(runner, b);
    if (rc != VLCA_OK) return rc;
  }
  const size_t T = static_cast<size_t>(total_tokens);
  if (qkv != runner->qkv && T > 0 &&
      hipMemcpyAsync(runner->qkv, qkv, T * qkv_row_bytes(runner->n_heads), hipMemcpyDeviceToDevice, stream) !=
          hipSuccess)
    return VLCA_ERR_HIP;
  if (vlca::launch_pad_offsets(cu_seqlens, num_users, total_tokens, runner->cu, runner->max_users, stream) !=
      hipSuccess)
    return VLCA_ERR_HIP;
  if (hipGraphLaunch(runner->execs[b], stream) != hipSuccess) return VLCA_ERR_HIP;
  if (out != runner->out && T > 0 &&
      hipMemcpyAsync(out, runner->out, T * out_row_bytes(runner->n_heads), hipMemcpyDeviceToDevice, stream) !=
          hipSuccess)
    return VLCA_ERR_HIP;
  return VLCA_OK;
}

int varlen_causal_attn_runner_captured(const vlca_graph_runner* runner, int* n_captured) {
  if (runner == nullptr || n_captured == nullptr) return VLCA_ERR_NULL_POINTER;
  int n = 0;
  for (auto x : runner->execs) n += x != nullptr;
  *n_captured = n;
  return VLCA_OK;
}

int varlen_causal_attn_runner_destroy(vlca_graph_runner* runner) {
  if (runner == nullptr) return VLCA_OK;
  // Graph launches may still be in flight on the caller's stream.
  const hipError_t e = hipDeviceSynchronize();
  release(runner);
  return e == hipSuccess ? VLCA_OK : VLCA_ERR_HIP;
}

}  // extern "C"
