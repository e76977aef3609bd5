// Host-only checks of the C ABI (vlca_api.cpp) against the stand-in runtime of
// hip_stub.cpp: argument errors, the launch plan, the key-range split settings
// passed to the kernels, and the per-stream worklist and split pool -- created
// without synchronising the stream, never freed while a captured graph may use
// them, and created while the stream is being captured without recording
// anything into the graph.  Built and run by tests/test_host_abi.py, with the
// address and undefined-behaviour sanitizers.  Prints "ALL OK" on success.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "hip_stub.h"
#include "varlen_causal_attn.h"

using stub::g;

static int failures = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);     \
      ++failures;                                                  \
    }                                                              \
  } while (0)

static hipStream_t stream_id(int i) { return reinterpret_cast<hipStream_t>(static_cast<intptr_t>(0x1000 + 16 * i)); }

// Dummy device pointers: the stand-in kernels never read qkv, cu_seqlens or out.
alignas(256) static char qkv_buf[64], cu_buf[64], out_buf[64];
static const void* QKV = qkv_buf;
static const int32_t* CU = reinterpret_cast<const int32_t*>(cu_buf);
static void* OUT = out_buf;

static int fwd(int users, int max_seqlen, int heads, hipStream_t s) {
  return varlen_causal_attn_fwd(QKV, CU, users, max_seqlen, heads, 64, 0.125f, OUT, s);
}

static void test_argument_errors() {
  CHECK(fwd(-1, 64, 8, nullptr) == VLCA_ERR_NEGATIVE_SIZE);
  CHECK(fwd(4, -1, 8, nullptr) == VLCA_ERR_NEGATIVE_SIZE);
  CHECK(fwd(4, VLCA_MAX_SEQLEN + 1, 8, nullptr) == VLCA_ERR_TOO_LARGE);
  CHECK(fwd(1 << 30, 262144, 8, nullptr) == VLCA_ERR_TOO_LARGE);
  CHECK(varlen_causal_attn_fwd(QKV, CU, 4, 64, 8, 32, 0.125f, OUT, nullptr) == VLCA_ERR_HEAD_DIM);
  CHECK(fwd(4, 64, 0, nullptr) == VLCA_ERR_N_HEADS);
  CHECK(fwd(4, 64, 65537, nullptr) == VLCA_ERR_N_HEADS);
  CHECK(varlen_causal_attn_fwd(QKV, CU, 4, 64, 8, 64, 0.0f, OUT, nullptr) == VLCA_ERR_SCALE);
  CHECK(varlen_causal_attn_fwd(QKV, CU, 4, 64, 8, 64, 1.0f / 0.0f, OUT, nullptr) == VLCA_ERR_SCALE);
  CHECK(varlen_causal_attn_fwd(nullptr, CU, 4, 64, 8, 64, 0.125f, OUT, nullptr) == VLCA_ERR_NULL_POINTER);
  CHECK(varlen_causal_attn_fwd(QKV, CU, 4, 64, 8, 64, 0.125f, const_cast<void*>(QKV), nullptr) == VLCA_ERR_ALIAS);
  int64_t cap = 0;
  CHECK(varlen_causal_attn_worklist_capacity(3, 129, &cap) == VLCA_OK && cap == 9);
  CHECK(varlen_causal_attn_build_worklist(CU, 3, 129, nullptr, 9, nullptr, nullptr) == VLCA_ERR_NULL_POINTER);
  alignas(16) int32_t items[4 * 8];
  int32_t count = 0;
  CHECK(varlen_causal_attn_build_worklist(CU, 3, 129, items, 8, &count, nullptr) == VLCA_ERR_CAPACITY);
  // Misaligned tensors: refused before any device work.
  CHECK(varlen_causal_attn_fwd(qkv_buf + 2, CU, 4, 64, 8, 64, 0.125f, OUT, nullptr) == VLCA_ERR_ALIGN);
  CHECK(varlen_causal_attn_fwd(QKV, CU, 4, 64, 8, 64, 0.125f, out_buf + 8, nullptr) == VLCA_ERR_ALIGN);
  CHECK(varlen_causal_attn_fwd(QKV, reinterpret_cast<const int32_t*>(cu_buf + 2), 4, 64, 8, 64, 0.125f, OUT,
                               nullptr) == VLCA_ERR_ALIGN);
  CHECK(varlen_causal_attn_build_worklist(CU, 3, 129, items + 1, 9, &count, nullptr) == VLCA_ERR_ALIGN);
  CHECK(varlen_causal_attn_fwd_worklist(QKV, CU, 3, 129, 8, 64, 0.125f, items + 2, 9, &count, OUT, nullptr) ==
        VLCA_ERR_ALIGN);
  // Nothing was launched or allocated by a refused call; no-ops launch nothing.
  CHECK(fwd(0, 64, 8, nullptr) == VLCA_OK && fwd(4, 0, 8, nullptr) == VLCA_OK);
  CHECK(g.launches.empty() && g.allocs == 0);
  // Without a device: an error, not a crash.
  g.has_device = false;
  CHECK(fwd(4, 64, 8, nullptr) == VLCA_ERR_HIP);
  g.has_device = true;
}

static void test_plans_and_split_settings() {
  stub::reset();
  // 60 users, max 452 rows: single kernel, may split (upr = 1024 / 8 = 128 units per head).
  CHECK(fwd(60, 452, 8, stream_id(1)) == VLCA_OK);
  CHECK(g.launches.size() == 1 && g.launches[0].kind == 'f');
  CHECK(g.launches[0].split.p == 2 && g.launches[0].split.upr == 128 && g.launches[0].split.min_width == 4);
  CHECK(g.launches[0].split.pool != nullptr && g.dirty_counters == 0);
  int single = -1;
  CHECK(varlen_causal_attn_single_kernel(60, 452, 8, &single) == VLCA_OK && single == 1);
  // No user can have more than 4 q-tiles: no split settings and no pool.
  stub::reset();
  CHECK(fwd(60, 256, 8, stream_id(2)) == VLCA_OK);
  CHECK(g.launches[0].kind == 'f' && g.launches[0].split.p <= 1 && g.allocs == 0);
  // The same batch with 300 zero-length users: more users than the single kernel
  // takes, so the scheduler plan -- with the same split settings (the kernels
  // decide from the users that have rows).
  stub::reset();
  CHECK(fwd(306, 1000, 8, stream_id(3)) == VLCA_OK);
  CHECK(g.launches.size() == 2 && g.launches[0].kind == 's' && g.launches[1].kind == 'a');
  CHECK(g.launches[0].split.p == 2 && g.launches[0].split.upr == 128);
  CHECK(g.launches[1].split.p == 2 && g.launches[1].split.pool == g.launches[0].split.pool);
  CHECK(varlen_causal_attn_single_kernel(306, 1000, 8, &single) == VLCA_OK && single == 0);
  // Sixteen heads: 64 units per head; 600 heads: fewer than 2 units, no splitting.
  stub::reset();
  CHECK(fwd(6, 1000, 16, stream_id(4)) == VLCA_OK && g.launches.back().split.upr == 64);
  stub::reset();
  CHECK(fwd(6, 1000, 600, stream_id(4)) == VLCA_OK && g.launches.back().split.p <= 1);
  // The caller's worklist entry point never splits and never allocates.
  stub::reset();
  std::vector<int32_t> items(4 * 64);
  int32_t count = 0;
  CHECK(varlen_causal_attn_fwd_worklist(QKV, CU, 4, 1000, 8, 64, 0.125f, items.data(), 64, &count, OUT,
                                        stream_id(5)) == VLCA_OK);
  CHECK(g.launches.size() == 1 && g.launches[0].split.p <= 1 && g.allocs == 0);
}

static void test_worklist_growth_keeps_old_buffers() {
  stub::reset();
  const hipStream_t s = stream_id(6);
  CHECK(fwd(300, 100, 8, s) == VLCA_OK);  // 600 items: first worklist (16384)
  const void* first = g.launches[0].items;
  CHECK(first != nullptr && g.allocs == 1);
  CHECK(fwd(300, 200, 8, s) == VLCA_OK);  // fits: no new allocation
  CHECK(g.allocs == 1 && g.launches.back().items == first);
  CHECK(fwd(1000, 4096, 8, s) == VLCA_OK);  // 64000 items: grows (and may split: pool too)
  const void* second = g.launches.back().items;
  CHECK(second != first);
  CHECK(g.frees == 0 && g.syncs == 0);  // no free, no synchronisation of the stream
  // A graph captured with the first worklist still finds it: write to it again.
  static_cast<char*>(const_cast<void*>(first))[0] = 2;
  // Another stream has its own worklist.
  CHECK(fwd(300, 100, 8, stream_id(7)) == VLCA_OK);
  CHECK(g.launches.back().items != first && g.launches.back().items != second);
  CHECK(g.frees == 0 && g.syncs == 0 && g.memsets <= 2 && g.dirty_counters == 0);
}

static void test_state_created_during_capture() {
  stub::reset();
  const hipStream_t s = stream_id(8);
  g.capturing = s;
  // Fresh stream, captured: the split pool and the worklist are allocated now
  // (relaxed mode), the pool's counters cleared off the captured stream.
  CHECK(fwd(306, 1000, 8, s) == VLCA_OK);
  CHECK(g.capture_violations == 0 && g.captured_memsets == 0);
  CHECK(g.allocs == 2 && g.frees == 0);
  CHECK(g.syncs == 1 && g.synced[0] != s);
  CHECK(g.launches.size() == 2 && g.launches[1].split.p == 2 && g.dirty_counters == 0);
  CHECK(g.mode == hipStreamCaptureModeGlobal);  // the thread's mode is restored
  // Growth while captured: a new worklist, nothing freed or synchronised.
  CHECK(fwd(1000, 8192, 8, s) == VLCA_OK);
  CHECK(g.capture_violations == 0 && g.frees == 0 && g.syncs == 1 && g.allocs == 3);
  g.capturing = nullptr;
  // Eager calls on that stream afterwards reuse its state.
  CHECK(fwd(306, 1000, 8, s) == VLCA_OK && g.allocs == 3 && g.dirty_counters == 0);
}

static void test_noalloc_entry_point() {
  stub::reset();
  const hipStream_t s = stream_id(9);
  char* scratch = nullptr;
  CHECK(vlca::noalloc_scratch(&scratch) == hipSuccess);
  stub::reset();
  auto na = [&](int users, int ms, int heads) {
    return varlen_causal_attn_fwd_noalloc(QKV, CU, users, ms, heads, 64, 0.125f, OUT, s);
  };
  // Single-kernel plan with split settings: the pool is the scratch array's start.
  CHECK(na(60, 452, 8) == VLCA_OK);
  CHECK(g.launches.size() == 1 && g.launches[0].kind == 'f' && g.launches[0].split.p == 2);
  CHECK(reinterpret_cast<char*>(g.launches[0].split.pool) == scratch);
  CHECK(reinterpret_cast<char*>(g.launches[0].split.ctr) == scratch + vlca::kNoAllocPoolBytes);
  // Scheduler plan: the worklist sits after the pool, its count after the items.
  CHECK(na(1000, 4096, 8) == VLCA_OK);
  CHECK(g.launches.size() == 3 && g.launches[1].kind == 's' && g.launches[2].kind == 'a');
  CHECK(reinterpret_cast<const char*>(g.launches[1].items) == scratch + vlca::kNoAllocItemsOffset);
  CHECK(g.launches[1].touched == vlca::kNoAllocItems * 16 + 4);
  CHECK(g.launches[2].split.upr == 128);
  // Too large for the scratch worklist: refused before any device work.
  const size_t before = g.launches.size();
  CHECK(na(VLCA_NOALLOC_MAX_ITEMS / 64 + 1, 4096, 8) == VLCA_ERR_SCRATCH);
  CHECK(na(VLCA_NOALLOC_MAX_ITEMS / 64, 4096, 8) == VLCA_OK);
  CHECK(g.launches.size() == before + 2);
  // Argument errors as for fwd.
  CHECK(na(4, 64, 0) == VLCA_ERR_N_HEADS && na(-1, 64, 8) == VLCA_ERR_NEGATIVE_SIZE);
  // Never allocates, frees, synchronises or sets memory -- captured or not.
  g.capturing = s;
  CHECK(na(306, 1000, 8) == VLCA_OK && na(60, 452, 8) == VLCA_OK);
  g.capturing = nullptr;
  CHECK(g.allocs == 0 && g.frees == 0 && g.syncs == 0 && g.memsets == 0 && g.capture_violations == 0);
}

static void test_graph_runner() {
  stub::reset();
  alignas(256) static char qkv_static[32], out_static[32];
  const int32_t pages[10] = {2560, 3072, 3584, 4096, 4608, 5120, 5632, 6144, 6656, 7168};
  vlca_graph_runner* r = nullptr;
  // Argument checks before any HIP call.
  const int32_t bad1[3] = {2560, 2560, 3072}, bad2[2] = {0, 64}, big[1] = {VLCA_MAX_SEQLEN + 1};
  CHECK(varlen_causal_attn_runner_create(bad1, 3, 20, 8, 0.125f, qkv_static, out_static, 1, &r) == VLCA_ERR_BUCKETS);
  CHECK(varlen_causal_attn_runner_create(bad2, 2, 20, 8, 0.125f, qkv_static, out_static, 1, &r) == VLCA_ERR_BUCKETS);
  CHECK(varlen_causal_attn_runner_create(pages, 0, 20, 8, 0.125f, qkv_static, out_static, 1, &r) == VLCA_ERR_BUCKETS);
  CHECK(varlen_causal_attn_runner_create(big, 1, 20, 8, 0.125f, qkv_static, out_static, 1, &r) == VLCA_ERR_TOO_LARGE);
  CHECK(varlen_causal_attn_runner_create(pages, 10, 0, 8, 0.125f, qkv_static, out_static, 1, &r) ==
        VLCA_ERR_NEGATIVE_SIZE);
  CHECK(varlen_causal_attn_runner_create(pages, 10, 20, 8, 0.125f, nullptr, out_static, 1, &r) ==
        VLCA_ERR_NULL_POINTER);
  CHECK(varlen_causal_attn_runner_create(pages, 10, 20, 8, 0.125f, qkv_static, qkv_static, 1, &r) == VLCA_ERR_ALIAS);
  CHECK(varlen_causal_attn_runner_create(pages, 10, 20, 8, 0.125f, qkv_static + 8, out_static, 1, &r) ==
        VLCA_ERR_ALIGN);
  CHECK(r == nullptr && g.allocs == 0 && g.launches.empty());

  // Pre-capture: one graph per bucket, each the forward with 20 users and
  // max_seqlen = the bucket, captured on the runner's own stream; nothing runs.
  CHECK(varlen_causal_attn_runner_create(pages, 10, 20, 8, 0.125f, qkv_static, out_static, 1, &r) == VLCA_OK);
  CHECK(r != nullptr && g.captures == 10 && g.graph_launches == 0 && g.capture_violations == 0);
  int n = 0;
  CHECK(varlen_causal_attn_runner_captured(r, &n) == VLCA_OK && n == 10);
  const hipStream_t cap_stream = g.launches.front().stream;
  for (const auto& l : g.launches) CHECK(l.stream == cap_stream && l.kind != 'g');
  CHECK(g.launches[0].kind == 'f' && g.launches[0].num_users == 20 && g.launches[0].max_tiles == 40);
  CHECK(g.launches.back().kind == 'a');  // 20 users x 112 tiles x 8 heads: the scheduler plan
  int b = -2;
  CHECK(varlen_causal_attn_runner_bucket(r, 20, 2560, &b) == VLCA_OK && b == 0);
  CHECK(varlen_causal_attn_runner_bucket(r, 20, 2561, &b) == VLCA_OK && b == 1);
  CHECK(varlen_causal_attn_runner_bucket(r, 3, 7168, &b) == VLCA_OK && b == 9);
  CHECK(varlen_causal_attn_runner_bucket(r, 3, 7169, &b) == VLCA_OK && b == -1);
  CHECK(varlen_causal_attn_runner_bucket(r, 21, 100, &b) == VLCA_OK && b == -1);

  // A batch of 3000 tokens and 15 users: bucket 1, offsets padded to 20 users on the
  // device, qkv copied in and out copied back (the caller's own buffers), graph replayed.
  const hipStream_t s = stream_id(10);
  g.launches.clear();
  CHECK(varlen_causal_attn_runner_run(r, QKV, CU, 15, 3000, 452, OUT, s, &b) == VLCA_OK && b == 1);
  CHECK(g.pads == 1 && g.last_pad_users == 15 && g.last_pad_total == 3000 && g.last_pad_max == 20);
  CHECK(g.copies == 2 && g.copied_bytes == int64_t(3000) * (1536 + 512) * 2);
  CHECK(g.launches.size() == 1 && g.launches[0].kind == 'g' && g.launches[0].stream == s);
  CHECK(g.launches[0].touched == 2);  // the second bucket's graph
  // The static buffers themselves: nothing copied.
  CHECK(varlen_causal_attn_runner_run(r, qkv_static, CU, 20, 2560, 452, out_static, s, &b) == VLCA_OK && b == 0);
  CHECK(g.copies == 2 && g.graph_launches == 2);
  // Above the top bucket, or too many users: the eager forward on the caller's stream.
  g.launches.clear();
  CHECK(varlen_causal_attn_runner_run(r, QKV, CU, 60, 9000, 1024, OUT, s, &b) == VLCA_OK && b == -1);
  CHECK(g.launches.size() == 1 && g.launches[0].kind == 'f' && g.launches[0].stream == s);
  CHECK(g.launches[0].max_tiles == 16 && g.graph_launches == 2);
  CHECK(varlen_causal_attn_runner_run(r, QKV, CU, 21, 100, 100, OUT, s, &b) == VLCA_OK && b == -1);
  CHECK(varlen_causal_attn_runner_destroy(r) == VLCA_OK);
  CHECK(g.execs_destroyed == 10 && g.graphs_destroyed == 10 && g.device_syncs == 1 && g.streams_destroyed == 1);

  // Lazy capture: a bucket's graph is captured on its first use only.
  stub::reset();
  CHECK(varlen_causal_attn_runner_create(pages, 10, 20, 8, 0.125f, qkv_static, out_static, 0, &r) == VLCA_OK);
  CHECK(varlen_causal_attn_runner_captured(r, &n) == VLCA_OK && n == 0 && g.captures == 0);
  CHECK(varlen_causal_attn_runner_run(r, QKV, CU, 15, 5000, 452, OUT, s, &b) == VLCA_OK && b == 5);
  CHECK(varlen_causal_attn_runner_run(r, QKV, CU, 15, 4700, 452, OUT, s, &b) == VLCA_OK && b == 5);
  CHECK(varlen_causal_attn_runner_captured(r, &n) == VLCA_OK && n == 1 && g.captures == 1 && g.graph_launches == 2);
  CHECK(g.capture_violations == 0);
  CHECK(varlen_causal_attn_runner_destroy(r) == VLCA_OK && varlen_causal_attn_runner_destroy(nullptr) == VLCA_OK);
}

static void test_training_entry_points() {
  stub::reset();
  alignas(256) static float lse_buf[16];
  alignas(256) static char dout_buf[32], dqkv_buf[32];
  const hipStream_t s = stream_id(11);
  // fwd_lse: same plan as fwd; lse required.
  CHECK(varlen_causal_attn_fwd_lse(QKV, CU, 60, 452, 8, 64, 0.125f, OUT, nullptr, s) == VLCA_ERR_NULL_POINTER);
  CHECK(varlen_causal_attn_fwd_lse(QKV, CU, 60, 452, 8, 64, 0.125f, OUT, lse_buf, s) == VLCA_OK);
  CHECK(g.launches.size() == 1 && g.launches[0].kind == 'f');
  // bwd: argument checks, then the first kernel (worklist and row pass) and the
  // gradient kernels over the stream's worklist.
  auto bwd = [&](const void* out, const void* dout, const float* lse, void* dqkv, int users, int ms) {
    return varlen_causal_attn_bwd(QKV, out, dout, lse, CU, users, ms, 8, 64, 0.125f, dqkv, s);
  };
  CHECK(bwd(OUT, nullptr, lse_buf, dqkv_buf, 60, 452) == VLCA_ERR_NULL_POINTER);
  CHECK(bwd(OUT, dout_buf, lse_buf, nullptr, 60, 452) == VLCA_ERR_NULL_POINTER);
  CHECK(bwd(OUT, dout_buf, lse_buf, dout_buf, 60, 452) == VLCA_ERR_ALIAS);
  CHECK(bwd(OUT, dout_buf, lse_buf, const_cast<void*>(QKV), 60, 452) == VLCA_ERR_ALIAS);
  const float* lse_odd = reinterpret_cast<const float*>(reinterpret_cast<const char*>(lse_buf) + 2);
  CHECK(bwd(OUT, dout_buf + 8, lse_buf, dqkv_buf, 60, 452) == VLCA_ERR_ALIGN);
  CHECK(bwd(OUT, dout_buf, lse_odd, dqkv_buf, 60, 452) == VLCA_ERR_ALIGN);
  CHECK(varlen_causal_attn_fwd_lse(QKV, CU, 60, 452, 8, 64, 0.125f, OUT, const_cast<float*>(lse_odd), s) ==
        VLCA_ERR_ALIGN);
  CHECK(bwd(OUT, dout_buf, lse_buf, dqkv_buf, 0, 452) == VLCA_OK && bwd(OUT, dout_buf, lse_buf, dqkv_buf, 60, 0) == VLCA_OK);
  g.launches.clear();
  CHECK(bwd(OUT, dout_buf, lse_buf, dqkv_buf, 60, 452) == VLCA_OK);
  CHECK(g.launches.size() == 2 && g.launches[0].kind == 'p' && g.launches[1].kind == 'b');
  CHECK(g.launches[0].max_tiles == 8 && g.launches[0].num_users == 60);  // ceil(452 / 64) q-tiles at most
  CHECK(g.launches[1].items == g.launches[0].items);
  CHECK(g.launches[1].max_tiles == 60 * 8);  // the worklist bound passed to the kernels
  CHECK(g.frees == 0 && g.syncs == 0);
}

static void test_masked_entry_point() {
  stub::reset();
  const hipStream_t s = stream_id(12);
  alignas(16) static int32_t ctx[4], tgt[4];
  auto fm = [&](const vlca_mask* m, int users, int ms) {
    return varlen_causal_attn_fwd_masked(QKV, CU, users, ms, 8, 64, 0.125f, m, OUT, s);
  };
  vlca_mask bad_group{nullptr, tgt, 0, -1, 0}, bad_left{nullptr, nullptr, 1, -2, 0},
      bad_right{ctx, nullptr, 1, -1, 3}, bad_right2{nullptr, nullptr, 1, -1, -2};
  CHECK(fm(&bad_group, 60, 452) == VLCA_ERR_MASK && fm(&bad_left, 60, 452) == VLCA_ERR_MASK);
  CHECK(fm(&bad_right, 60, 452) == VLCA_ERR_MASK && fm(&bad_right2, 60, 452) == VLCA_ERR_MASK);
  CHECK(g.launches.empty());
  // The plain causal mask (or none) is the forward itself.
  vlca_mask causal{nullptr, nullptr, 1, -1, 0};
  CHECK(fm(&causal, 60, 452) == VLCA_OK && fm(nullptr, 60, 452) == VLCA_OK);
  CHECK(g.launches.size() == 2 && g.launches[0].kind == 'f' && g.launches[1].kind == 'f');
  // A window, contexts and targets on a small batch (the causal forward's
  // single-kernel condition): the masked kernel alone, locating its own items.
  g.launches.clear();
  vlca_mask hstu{ctx, tgt, 4, 256, 0};
  CHECK(fm(&hstu, 60, 452) == VLCA_OK);
  CHECK(g.launches.size() == 1 && g.launches[0].kind == 'M');
  CHECK(g.launches[0].num_users == 60 && g.launches[0].max_tiles == 8 && g.launches[0].grid == 1024);
  CHECK(g.launches[0].layer_log2 == -1);  // 60 x 8 units per head exceed one round of 128 slots
  CHECK(fm(&hstu, 4, 1024) == VLCA_OK && g.launches.back().kind == 'M' && g.launches.back().grid == 512);
  CHECK(g.launches.back().layer_log2 == 5);  // 4 x 16 units per head fit one round: layers of 32 slots
  // Larger batches: the scheduler, then the masked kernel over its worklist.
  g.launches.clear();
  CHECK(fm(&hstu, 300, 452) == VLCA_OK);
  CHECK(g.launches.size() == 2 && g.launches[0].kind == 's' && g.launches[1].kind == 'm');
  CHECK(g.launches[1].items == g.launches[0].items && g.launches[1].num_users == 4);
  CHECK(g.launches[1].max_tiles == 256 && g.launches[1].layer_log2 == 0 && g.launches[1].grid == 1024);
  vlca_mask bidir{nullptr, nullptr, 1, -1, -1};
  CHECK(fm(&bidir, 300, 452) == VLCA_OK && g.launches.back().kind == 'm' && g.launches.back().layer_log2 == -1);
  CHECK(fm(&bidir, 60, 452) == VLCA_OK && g.launches.back().kind == 'M');
  CHECK(g.frees == 0 && g.syncs == 0);
}

// LayerNorm + qkv product and output product with residual: shape and argument
// errors launch nothing; a valid call launches one kernel with T and n_out.
static void test_neighbour_entry_points() {
  stub::reset();
  alignas(256) static char x[64], gb[64], w[64], b[64], y[64];
  CHECK(varlen_causal_attn_ln_qkv(x, gb, gb, 1e-5f, w, b, 10, 256, 1536, y, nullptr) == VLCA_ERR_SHAPE);
  CHECK(varlen_causal_attn_ln_qkv(x, gb, gb, 1e-5f, w, b, 10, 512, 1500, y, nullptr) == VLCA_ERR_SHAPE);
  CHECK(varlen_causal_attn_ln_qkv(x, gb, gb, 1e-5f, w, b, 10, 512, 0, y, nullptr) == VLCA_ERR_SHAPE);
  CHECK(varlen_causal_attn_ln_qkv(x, gb, gb, 1e-5f, w, b, 10, 512, 65536 + 128, y, nullptr) == VLCA_ERR_SHAPE);
  CHECK(varlen_causal_attn_ln_qkv(x, gb, gb, -1.f, w, b, 10, 512, 1536, y, nullptr) == VLCA_ERR_SCALE);
  CHECK(varlen_causal_attn_ln_qkv(x, gb, gb, 1e-5f, w, b, -1, 512, 1536, y, nullptr) == VLCA_ERR_NEGATIVE_SIZE);
  CHECK(varlen_causal_attn_ln_qkv(x, nullptr, gb, 1e-5f, w, b, 10, 512, 1536, y, nullptr) == VLCA_ERR_NULL_POINTER);
  CHECK(varlen_causal_attn_ln_qkv(x, gb, gb, 1e-5f, w, b, 10, 512, 1536, x, nullptr) == VLCA_ERR_ALIAS);
  CHECK(varlen_causal_attn_ln_qkv(x, gb, gb, 1e-5f, w, b, 0, 512, 1536, y, nullptr) == VLCA_OK);
  CHECK(varlen_causal_attn_out_residual(x, w, b, y, 10, 512, 640 + 64, y, nullptr) == VLCA_ERR_SHAPE);
  CHECK(varlen_causal_attn_out_residual(x, w, b, y, 10, 512, 65536 + 128, y, nullptr) == VLCA_ERR_SHAPE);
  CHECK(varlen_causal_attn_out_residual(x, w, b, y, 10, 512, 512, x, nullptr) == VLCA_ERR_ALIAS);
  CHECK(varlen_causal_attn_out_residual(x, w, nullptr, y, 10, 512, 512, y, nullptr) == VLCA_ERR_NULL_POINTER);
  CHECK(varlen_causal_attn_ln_qkv(x + 8, gb, gb, 1e-5f, w, b, 10, 512, 1536, y, nullptr) == VLCA_ERR_ALIGN);
  CHECK(varlen_causal_attn_ln_qkv(x, gb, gb, 1e-5f, w, b + 2, 10, 512, 1536, y, nullptr) == VLCA_ERR_ALIGN);
  CHECK(varlen_causal_attn_out_residual(x, w, b, y + 8, 10, 512, 512, y, nullptr) == VLCA_ERR_ALIGN);
  CHECK(g.launches.empty());
  CHECK(varlen_causal_attn_ln_qkv(x, gb, gb, 1e-5f, w, b, 10, 512, 65536, y, stream_id(9)) == VLCA_OK);
  CHECK(varlen_causal_attn_out_residual(x, w, b, y, 7, 512, 512, y, stream_id(9)) == VLCA_OK);  // y = residual
  CHECK(g.launches.size() == 2 && g.launches[0].kind == 'l' && g.launches[0].num_users == 10 &&
        g.launches[0].max_tiles == 65536 && g.launches[1].kind == 'o' && g.launches[1].num_users == 7 &&
        g.launches[1].stream == stream_id(9));
  CHECK(g.allocs == 0);
}

int main() {
  setvbuf(stdout, nullptr, _IONBF, 0);
  test_argument_errors();
  test_plans_and_split_settings();
  test_worklist_growth_keeps_old_buffers();
  test_state_created_during_capture();
  test_noalloc_entry_point();
  test_graph_runner();
  test_training_entry_points();
  test_masked_entry_point();
  test_neighbour_entry_points();
  if (failures == 0) std::printf("ALL OK\n");
  return failures == 0 ? 0 : 1;
}
