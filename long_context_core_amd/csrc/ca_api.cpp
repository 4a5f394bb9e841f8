// Host side of libca: argument validation, work-item expansion with exact
// per-item cost, longest-first ordering, workspace layout and launches.
//
// The work queue applies the pages' balancing idea at the level of compute
// units: every item's cost is its number of visible (query, key) pairs —
// attention cost is quadratic in document length, FLOPs(l) = alpha l^2 +
// beta l ("Efficient Long-context Language Model Training by Core Attention
// Disaggregation", Section 3.4) — and items are issued longest first so that
// the hardware dispatcher's greedy fill of free workgroup slots balances the
// tail (the simple greedy fill of the CMU CSD blog post on Core Attention
// Disaggregation, Figure 9 discussion).  Nothing here allocates device memory:
// the task table and the queue are uploaded into the caller's workspace.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "ca_internal.h"


namespace {

thread_local std::string g_last_error;

ca_status fail(ca_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

}  // namespace

ca_status ca::set_error(ca_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

namespace {

ca_status hip_fail(hipError_t e, const char* what) {
  return fail(CA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Sum over task rows i in [a, b] of clip(i + delta + 1, 0, kv_len): the
// number of keys each row sees (key j visible iff j <= i + delta, j < kv_len).
int64_t range_pairs(int64_t a, int64_t b, int64_t delta, int64_t kv_len) {
  if (b < a || kv_len <= 0) return 0;
  const int64_t s0 = kv_len - delta - 1;      // first row that sees all keys
  int64_t total = 0;
  const int64_t sat_lo = std::max(a, s0);
  if (b >= sat_lo) total += kv_len * (b - sat_lo + 1);
  const int64_t lo = std::max(a, -delta);     // first row that sees >= 1 key
  const int64_t hi = std::min(b, s0 - 1);
  if (hi >= lo) {
    const int64_t n = hi - lo + 1;
    const int64_t f_lo = lo + delta + 1, f_hi = hi + delta + 1;
    total += (f_lo + f_hi) * n / 2;
  }
  return total;
}

// Window and sink of task i (no mask array: causal, window 0).  The sink is
// only meaningful with a window; it is returned as a task-relative key count.
int32_t task_window(const ca_task_mask* m, int32_t i) { return m ? m[i].window : 0; }
int64_t task_sink_keys(const ca_task* t, const ca_task_mask* m, int32_t i) {
  if (!m || m[i].window <= 0) return 0;
  return std::min<int64_t>(t[i].kv_len, std::max<int64_t>(0, (int64_t)m[i].sink - t[i].kv_pos0));
}

// Keys row u = i + delta sees under the sink + sliding-window mask: the keys
// of its causal context [0, c) that are >= u - win + 1 (the window) or < sj
// (the sink).
int64_t masked_row_keys(int64_t u, int64_t kv_len, int64_t win, int64_t sj) {
  const int64_t c = std::min(kv_len, std::max<int64_t>(0, u + 1));
  const int64_t wlo = std::max<int64_t>(0, u - win + 1);
  return std::max<int64_t>(0, c - wlo) + std::max<int64_t>(0, std::min(std::min(sj, c), wlo));
}

// range_pairs under the sink + sliding-window mask, in closed form.  The
// per-row count is piecewise linear in u with integer slopes; its slope can
// change only between u = k and u = k + 1 for k in the kinks below (where
// u + 1 reaches 0 or kv_len, the window start reaches 0, the sink end or
// kv_len).  Between kinks each run of rows is an arithmetic series.
int64_t range_pairs_masked(int64_t a, int64_t b, int64_t delta, int64_t kv_len, int64_t win, int64_t sj) {
  if (win <= 0) return range_pairs(a, b, delta, kv_len);
  if (b < a || kv_len <= 0) return 0;
  const int64_t kinks[6] = {-1, kv_len - 1, win - 1, kv_len + win - 1, sj - 1, sj + win - 1};
  int64_t total = 0;
  for (int64_t r0 = a; r0 <= b;) {
    int64_t r1 = b;
    for (int64_t k : kinks)
      if (k - delta >= r0 && k - delta < r1) r1 = k - delta;
    const int64_t f0 = masked_row_keys(r0 + delta, kv_len, win, sj), f1 = masked_row_keys(r1 + delta, kv_len, win, sj);
    total += (f0 + f1) * (r1 - r0 + 1) / 2;   // even: 2 f0 n + slope n (n - 1)
    r0 = r1 + 1;
  }
  return total;
}

ca_status check_masks(const ca_task_mask* m, int32_t n) {
  if (!m) return CA_OK;
  for (int32_t i = 0; i < n; ++i)
    if (m[i].window < 0 || m[i].sink < 0) return fail(CA_ERR_INVALID, "task %d: negative window or sink", i);
  return CA_OK;
}

// Bounds that keep every size product (rows x heads x d x 4 bytes) inside
// int64: far beyond any buffer a device holds.
constexpr int64_t kMaxRows = int64_t(1) << 40;
constexpr int32_t kMaxHeads = 4096;
// Longest task (query rows and context rows): keeps the kernels' and the
// planners' int32 tile arithmetic (a length plus a tile, twice a length)
// inside int32.
constexpr int32_t kMaxTaskLen = int32_t(1) << 30;

ca_status check_shape(const ca_shape* s) {
  if (!s) return fail(CA_ERR_INVALID, "shape is NULL");
  if (s->hq < 1 || s->hkv < 1) return fail(CA_ERR_INVALID, "hq=%d hkv=%d must be >= 1", s->hq, s->hkv);
  if (s->hq % s->hkv != 0) return fail(CA_ERR_INVALID, "hkv=%d does not divide hq=%d", s->hkv, s->hq);
  if (s->d != 64 && s->d != 128) return fail(CA_ERR_UNSUPPORTED, "head dim d=%d not supported (64, 128)", s->d);
  // The kernels take row maxima of the unscaled scores: the scale must be positive.
  if (!std::isfinite(s->scale) || !(s->scale > 0.f)) return fail(CA_ERR_INVALID, "scale must be finite and > 0");
  if (s->hq > kMaxHeads) return fail(CA_ERR_INVALID, "hq=%d > %d", s->hq, kMaxHeads);
  if (s->q_rows < 0 || s->kv_rows < 0 || s->o_rows < 0)
    return fail(CA_ERR_INVALID, "negative row count");
  if (s->q_rows > kMaxRows || s->kv_rows > kMaxRows || s->o_rows > kMaxRows)
    return fail(CA_ERR_INVALID, "row count above 2^40");
  if (s->flags & ~(uint32_t)(CA_OUT_F32 | CA_LAUNCH_PERSISTENT | CA_LAUNCH_PER_ITEM))
    return fail(CA_ERR_INVALID, "unknown flags 0x%x", s->flags);
  if ((s->flags & CA_LAUNCH_PERSISTENT) && (s->flags & CA_LAUNCH_PER_ITEM))
    return fail(CA_ERR_INVALID, "CA_LAUNCH_PERSISTENT and CA_LAUNCH_PER_ITEM together");
  return CA_OK;
}

// kv_limit: rows of the space that kv_off / kv_len address (kv_rows, or the
// virtual rows of a page table).
ca_status check_tasks(const ca_shape* s, const ca_task* t, int32_t n, int64_t kv_limit) {
  if (n < 0) return fail(CA_ERR_INVALID, "n_tasks=%d < 0", n);
  if (n > 0 && !t) return fail(CA_ERR_INVALID, "tasks_host is NULL");
  for (int32_t i = 0; i < n; ++i) {
    const ca_task& k = t[i];
    if (k.q_len < 0 || k.kv_len < 0) return fail(CA_ERR_INVALID, "task %d: negative length", i);
    if (k.q_len > kMaxTaskLen || k.kv_len > kMaxTaskLen)
      return fail(CA_ERR_INVALID, "task %d: q_len=%d or kv_len=%d above 2^30", i, k.q_len, k.kv_len);
    if (k.q_off < 0 || k.kv_off < 0 || k.o_off < 0) return fail(CA_ERR_INVALID, "task %d: negative offset", i);
    // Compared as off > rows - len: the lengths are non-negative int32 and the
    // row counts non-negative, so nothing here can overflow (off + len could,
    // for offsets near INT64_MAX).
    if (k.q_off > s->q_rows - k.q_len)
      return fail(CA_ERR_INVALID, "task %d: %d query rows from row %lld past q_rows=%lld", i, k.q_len,
                  (long long)k.q_off, (long long)s->q_rows);
    if (k.kv_off > kv_limit - k.kv_len)
      return fail(CA_ERR_INVALID, "task %d: %d context rows from row %lld past %lld", i, k.kv_len,
                  (long long)k.kv_off, (long long)kv_limit);
    if (k.o_off > s->o_rows - k.q_len)
      return fail(CA_ERR_INVALID, "task %d: %d output rows from row %lld past o_rows=%lld", i, k.q_len,
                  (long long)k.o_off, (long long)s->o_rows);
    if (k.q_pos0 < -(int64_t(1) << 40) || k.q_pos0 > (int64_t(1) << 40) ||
        k.kv_pos0 < -(int64_t(1) << 40) || k.kv_pos0 > (int64_t(1) << 40))
      return fail(CA_ERR_INVALID, "task %d: positions out of range", i);
  }
  return CA_OK;
}

ca_status check_tasks(const ca_shape* s, const ca_task* t, int32_t n) { return check_tasks(s, t, n, s->kv_rows); }

constexpr int kPageAlign = 128;   // task starts and page sizes: whole 128-row tiles

// Page table checks; see ca_kv_pages.
ca_status check_page_table(const ca_shape* s, const ca_kv_pages* pg) {
  if (!pg) return fail(CA_ERR_INVALID, "pages is NULL");
  const int32_t pr = pg->page_rows;
  if (pr < kPageAlign || pr > (1 << 20) || (pr & (pr - 1)) != 0)
    return fail(CA_ERR_INVALID, "page_rows=%d must be a power of two in [128, 1 << 20]", pr);
  if (pg->n_pages < 0 || pg->n_pages > (int64_t(1) << 31) / 4)
    return fail(CA_ERR_INVALID, "n_pages=%lld out of range", (long long)pg->n_pages);
  if (pg->reserved != 0) return fail(CA_ERR_INVALID, "reserved field must be 0");
  if (pg->n_pages > 0 && !pg->table_host) return fail(CA_ERR_INVALID, "table_host is NULL");
  const int64_t phys = s->kv_rows / pr;
  for (int64_t v = 0; v < pg->n_pages; ++v)
    if (pg->table_host[v] < 0 || pg->table_host[v] >= phys)
      return fail(CA_ERR_INVALID, "page table entry %lld = %d not in [0, %lld)", (long long)v, pg->table_host[v],
                  (long long)phys);
  return CA_OK;
}

// Paged tasks start on a 128-row boundary of the virtual space.
ca_status check_paged_tasks(const ca_task* t, int32_t n) {
  for (int32_t i = 0; i < n; ++i)
    if (t[i].kv_len > 0 && t[i].kv_off % kPageAlign != 0)
      return fail(CA_ERR_INVALID, "task %d: kv_off=%lld is not a multiple of 128 (paged K/V)", i,
                  (long long)t[i].kv_off);
  return CA_OK;
}

int page_shift_of(const ca_kv_pages* pg) {
  int sh = 0;
  while ((1 << sh) < pg->page_rows) ++sh;
  return sh;
}

// Argument checks shared by the forward entry points and their workspace queries.
ca_status check_forward_args(const ca_shape* s, const ca_task* t, const ca_task_mask* m, int32_t n,
                             const ca_kv_pages* pg) {
  ca_status st = check_shape(s);
  if (st != CA_OK) return st;
  if (pg) {
    st = check_page_table(s, pg);
    if (st != CA_OK) return st;
    st = check_tasks(s, t, n, pg->n_pages * pg->page_rows);
    if (st != CA_OK) return st;
    st = check_paged_tasks(t, n);
  } else {
    st = check_tasks(s, t, n);
  }
  if (st != CA_OK) return st;
  return check_masks(m, n);
}

int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }

// Upload of a host-built work queue into the caller's workspace, through a
// ring of pinned staging buffers kept per thread and device (each grown, never
// shrunk, released when the thread ends).  An event recorded after each copy
// guards that buffer's reuse, so a call waits only when all kStagingSlots
// earlier uploads of this thread are still queued behind device work; with a
// single buffer every call waited for the previous call's copy, which put the
// host wake-up latency between consecutive small launches.
constexpr int kStagingSlots = 8;
struct Staging {
  void* buf = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};
struct StagingRing {
  Staging slot[kStagingSlots];
  int next = 0;
  StagingRing() = default;
  StagingRing(const StagingRing&) = delete;
  StagingRing& operator=(const StagingRing&) = delete;
  // At thread exit: a copy still queued reads its buffer, so wait for it
  // before the buffer goes back.  Errors cannot be reported from here.
  ~StagingRing() {
    for (Staging& st : slot) {
      if (st.pending && st.ev) (void)hipEventSynchronize(st.ev);
      if (st.buf) (void)hipHostFree(st.buf);
      if (st.ev) (void)hipEventDestroy(st.ev);
    }
  }
};
constexpr int kMaxDevices = 64;
thread_local StagingRing g_staging[kMaxDevices];

// A graph captured around the copy would keep reading a staging buffer that
// later calls overwrite, so calls that upload refuse a capturing stream (the
// prepared forward is the capturable form).  Checked before anything is
// enqueued.
ca_status check_not_capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(s, &cs);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone)
    return fail(CA_ERR_INVALID, "the stream is capturing: calls that upload a work queue are not capturable "
                                "(capture ca_forward_prepared instead)");
  return CA_OK;
}

ca_status upload(void* dst, const std::vector<char>& src, hipStream_t s) {
  ca_status cst = check_not_capturing(s);
  if (cst != CA_OK) return cst;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(CA_ERR_UNSUPPORTED, "device index %d", dev);
  StagingRing& ring = g_staging[dev];
  Staging& st = ring.slot[ring.next];
  if (st.pending) {
    // Poll briefly before blocking: with back-to-back calls of a few tens of
    // microseconds the slot frees within that time, and a blocking wait can
    // put the thread to sleep for far longer than the kernel it waits for.
    const auto t0 = std::chrono::steady_clock::now();
    while ((e = hipEventQuery(st.ev)) == hipErrorNotReady &&
           std::chrono::steady_clock::now() - t0 < std::chrono::microseconds(200)) {
    }
    if (e == hipErrorNotReady) e = hipEventSynchronize(st.ev);
    if (e != hipSuccess) return hip_fail(e, "waiting for an earlier upload");
    st.pending = false;
  }
  if (!st.ev) {
    e = hipEventCreateWithFlags(&st.ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  }
  if (st.cap < src.size()) {
    if (st.buf) (void)hipHostFree(st.buf);
    st.buf = nullptr;
    st.cap = 0;
    const size_t cap = std::max<size_t>(src.size() + src.size() / 2, 1 << 16);
    e = hipHostMalloc(&st.buf, cap, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "pinned staging allocation");
    st.cap = cap;
  }
  std::memcpy(st.buf, src.data(), src.size());
  e = hipMemcpyAsync(dst, st.buf, src.size(), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "upload of the work queue");
  e = hipEventRecord(st.ev, s);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  st.pending = true;
  ring.next = (ring.next + 1) % kStagingSlots;
  return CA_OK;
}

// ---------------------------------------------------------------------------
// Forward plan
// ---------------------------------------------------------------------------
//
// Tasks with a single query row and at most 16 query heads per KV head go to
// the split-KV decode kernel (the heads of a group share one K/V stream); all
// others go to the tiled kernel.  Decode tasks are cut into key chunks so that
// the launch has enough work items to cover the chip; chunks of one task are
// merged by log-sum-exp afterwards.

constexpr int kFwdWaves = 8;   // waves per forward workgroup (two per SIMD)
constexpr int kBwdQWaves = 8;  // waves per dQ workgroup (two per SIMD)
// Persistent forward launch: one 8-wave workgroup per compute unit of the
// MI355X (256 CUs; about 250 VGPRs per wave leave room for one such workgroup
// per CU); the workgroups claim items from the longest-first queue.  On a
// part with fewer CUs the extra workgroups wait their turn.  Chosen by
// default from 16 items per workgroup up: with the shard-major queue it
// measured +0.6 % on a 16,424-item batch and +0.7 % on a 65,728-item one
// against one workgroup per item; a few items gain nothing from claims and
// would pay the counter reset's extra launch.
constexpr size_t kPersistSlots = 256;
constexpr size_t kPersistMinItems = 16 * kPersistSlots;
// Split-KV decode: key chunks sized for about one 4-wave item per CU.  With
// the streamed (nontemporal) K/V loads, long contiguous chunks read fastest:
// on 256 single-row tasks over 16K keys each, 256 items (no chunk merge)
// 6.63 TB/s, 512 items 6.45, 1,024 items 6.15, 2,048 items 5.70.
constexpr int kDecTargetItems = 256;
constexpr int kDecMinChunk = 512;
constexpr int kDecMaxGroup = 16;

bool is_decode_task(const ca_task& k, int group, int32_t window) {
  return k.q_len == 1 && group <= kDecMaxGroup && window == 0;
}

// Query shards: maximal runs of consecutive tasks with the same q_off, o_off,
// q_len and q_pos0 (q_len > 0) are one shard, whose rows attend to the union
// of the tasks' contexts under one softmax.  Returns, per task, the number of
// tasks of the shard it starts (0 for the later tasks of a shard).
std::vector<int32_t> query_shards(const ca_task* t, int32_t n) {
  std::vector<int32_t> len((size_t)n, 1);
  for (int32_t i = 0; i < n;) {
    int32_t j = i + 1;
    if (t[i].q_len > 0)
      while (j < n && t[j].q_off == t[i].q_off && t[j].o_off == t[i].o_off && t[j].q_len == t[i].q_len &&
             t[j].q_pos0 == t[i].q_pos0)
        ++j;
    len[(size_t)i] = j - i;
    for (int32_t k = i + 1; k < j; ++k) len[(size_t)k] = 0;
    i = j;
  }
  return len;
}

// A shard of one task with a single query row goes to the split-KV decode
// kernel (when its group and mask allow); every other shard to the tiled one.
bool is_decode_shard(const ca_task* t, const ca_task_mask* m, const std::vector<int32_t>& shard, int32_t i,
                     int group) {
  return shard[(size_t)i] == 1 && is_decode_task(t[i], group, task_window(m, i));
}

// Visible pairs of query rows [r0, r1] of the shard starting at task i, per
// head (every context of the shard).
int64_t shard_range_pairs(const ca_task* t, const ca_task_mask* m, int32_t i, int32_t n_seg, int64_t r0, int64_t r1) {
  int64_t total = 0;
  for (int32_t k = i; k < i + n_seg; ++k)
    total += range_pairs_masked(r0, r1, t[k].q_pos0 - t[k].kv_pos0, t[k].kv_len, task_window(m, k),
                                task_sink_keys(t, m, k));
  return total;
}

// keys of a decode task that its single row can see: [0, vis)
int64_t decode_visible(const ca_task& k) {
  return std::min<int64_t>(k.kv_len, std::max<int64_t>(0, k.q_pos0 - k.kv_pos0 + 1));
}

// Long query shards split over key chunks (forward and dQ kernels).  An item
// whose work exceeds a quarter of one compute unit's share of the call
// (256 CUs) makes a tail no scheduling hides; its shard's visible keys are
// cut into chunks, each a run of derived tasks (sub-ranges of the shard's
// contexts, appended after the table) whose items write fp32 partials to
// staging rows; the partials are merged afterwards.  Shards with sink /
// window masks are left whole (their items are short).
constexpr int64_t kMinSplitPairs = 1 << 21;   // per item and head
constexpr int64_t kSplitShareDiv = 4 * 256;
constexpr int32_t kMaxChunks = 64;
constexpr int32_t kChunkAlign = 128;          // chunk bounds, in keys (paged tiles stay inside one page)

struct ShardSplits {
  std::vector<ca_task> tasks;              // derived tasks, indices n ..
  std::vector<ca_task_mask> masks;
  struct Split {
    int32_t task;                          // the shard's first task
    int64_t stage_row0;
    std::vector<int32_t> chunk_first, chunk_n;   // derived task runs
  };
  std::vector<Split> splits;
  std::vector<int32_t> split_of;           // per task: index into splits, or -1
  int64_t stage_rows = 0;
  int32_t max_q_len = 0;
};

// hq: query heads of the call; hpw: heads per work item.
ShardSplits plan_shard_splits(const ca_task* t, const ca_task_mask* m, int32_t n, const std::vector<int32_t>& shard,
                              int rt, int hq, int hpw, const std::vector<bool>& tiled) {
  ShardSplits S;
  S.split_of.assign((size_t)n, -1);
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i)
    if (shard[(size_t)i] > 0 && tiled[(size_t)i]) total += shard_range_pairs(t, m, i, shard[(size_t)i], 0, t[i].q_len - 1);
  // an item's work is w * hpw head-pairs, the call's total * hq
  const int64_t w_max = std::max<int64_t>(kMinSplitPairs, total / (kSplitShareDiv * hpw) * hq);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t n_seg = shard[(size_t)i];
    if (n_seg == 0 || !tiled[(size_t)i]) continue;
    bool windowed = false;
    for (int32_t k = i; k < i + n_seg; ++k) windowed |= task_window(m, k) > 0;
    if (windowed) continue;
    const ca_task& q = t[i];
    // the costliest row tile: the last, or the one before it when the last is
    // short; a tile's 32-row blocks run whole, so its rows count padded
    const int64_t last = (int64_t)(q.q_len - 1) / rt * rt;
    int64_t w = 0;
    for (int64_t r0 = last; r0 >= 0 && r0 >= last - rt; r0 -= rt) {
      const int64_t r1 = std::min<int64_t>(r0 + rt, q.q_len) - 1, rows = r1 - r0 + 1;
      w = std::max(w, shard_range_pairs(t, m, i, n_seg, r0, r1) / rows * ((rows + 31) / 32 * 32));
    }
    if (w <= w_max) continue;
    // keys the shard's last row sees, context by context
    std::vector<int64_t> nvis((size_t)n_seg);
    int64_t keys = 0;
    for (int32_t k = 0; k < n_seg; ++k) {
      const ca_task& x = t[i + k];
      nvis[(size_t)k] = std::min<int64_t>(x.kv_len, std::max<int64_t>(0, x.q_pos0 + x.q_len - x.kv_pos0));
      keys += nvis[(size_t)k];
    }
    int64_t chunks = std::min<int64_t>(kMaxChunks, (w + w_max - 1) / w_max);
    chunks = std::min<int64_t>(chunks, keys / (2 * kChunkAlign));
    if (chunks < 2) continue;
    const int64_t step = ((keys + chunks - 1) / chunks + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
    ShardSplits::Split sp;
    sp.task = i;
    // walk the contexts, cutting at multiples of `step` keys from each
    // context's start (so every cut lies on a kChunkAlign boundary)
    int64_t in_chunk = 0;
    sp.chunk_first.push_back(n + (int32_t)S.tasks.size());
    sp.chunk_n.push_back(0);
    for (int32_t k = 0; k < n_seg; ++k) {
      const ca_task& x = t[i + k];
      for (int64_t a = 0; a < nvis[(size_t)k];) {
        if (in_chunk == step) {
          sp.chunk_first.push_back(n + (int32_t)S.tasks.size());
          sp.chunk_n.push_back(0);
          in_chunk = 0;
        }
        const int64_t b = std::min<int64_t>(nvis[(size_t)k], a + (step - in_chunk));
        ca_task d = x;
        d.kv_off = x.kv_off + a;
        d.kv_len = (int32_t)(b - a);
        d.kv_pos0 = x.kv_pos0 + a;
        S.tasks.push_back(d);
        S.masks.push_back(ca_task_mask{0, 0});
        ++sp.chunk_n.back();
        in_chunk += b - a;
        a = b;
      }
    }
    if (sp.chunk_first.size() < 2) {       // nothing to split after all
      S.tasks.resize((size_t)(sp.chunk_first[0] - n));
      S.masks.resize(S.tasks.size());
      continue;
    }
    sp.stage_row0 = S.stage_rows;
    S.stage_rows += (int64_t)q.q_len * (int64_t)sp.chunk_first.size();
    S.max_q_len = std::max(S.max_q_len, q.q_len);
    S.split_of[(size_t)i] = (int32_t)S.splits.size();
    S.splits.push_back(std::move(sp));
  }
  return S;
}

struct FwdPlan {
  int hpw = 1, rt = 128, group = 1;
  std::vector<int32_t> shard;   // query_shards()
  ShardSplits splits;
  int multi = 0;               // some shard has several contexts or is split
  size_t n_items = 0;        // tiled-kernel items
  size_t n_dec_items = 0;    // decode items
  size_t n_split = 0;        // decode (task, kv head) pairs cut into > 1 chunk
  size_t n_parts = 0;        // staging slots for those chunks
  int64_t dec_chunk = 0;
  size_t n_slots = 0;        // persistent workgroups of the tiled kernel
  size_t off_tasks = 0, off_masks = 0, off_pages = 0, off_items = 0, off_dec = 0, off_split = 0, off_merge = 0,
         off_counter = 0, off_part_o = 0, off_part_l = 0, off_stage_o = 0, off_stage_l = 0, bytes = 0;
};

FwdPlan plan_forward(const ca_shape* s, const ca_task* t, const ca_task_mask* m, int32_t n,
                     const ca_kv_pages* pg = nullptr) {
  FwdPlan p;
  p.group = s->hq / s->hkv;
  p.hpw = gcd_int(p.group, kFwdWaves);
  p.rt = 32 * (kFwdWaves / p.hpw);
  p.shard = query_shards(t, n);
  int64_t dec_keys = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (t[i].q_len <= 0 || p.shard[(size_t)i] == 0) continue;
    if (p.shard[(size_t)i] > 1) p.multi = 1;
    if (is_decode_shard(t, m, p.shard, i, p.group)) {
      dec_keys += decode_visible(t[i]) * s->hkv;
      continue;
    }
  }
  std::vector<bool> tiled((size_t)n, false);
  for (int32_t i = 0; i < n; ++i)
    tiled[(size_t)i] = t[i].q_len > 0 && p.shard[(size_t)i] > 0 && !is_decode_shard(t, m, p.shard, i, p.group);
  p.splits = plan_shard_splits(t, m, n, p.shard, p.rt, s->hq, p.hpw, tiled);
  if (!p.splits.splits.empty()) p.multi = 1;
  for (int32_t i = 0; i < n; ++i) {
    if (!tiled[(size_t)i]) continue;
    const int32_t sp = p.splits.split_of[(size_t)i];
    const size_t chunks = sp >= 0 ? p.splits.splits[(size_t)sp].chunk_first.size() : 1;
    const size_t tiles = (t[i].q_len + p.rt - 1) / p.rt;
    p.n_items += tiles * (size_t)s->hkv * (size_t)(p.group / p.hpw) * chunks;
  }
  const int64_t per_item = (dec_keys + kDecTargetItems - 1) / kDecTargetItems;
  p.dec_chunk = std::max<int64_t>(kDecMinChunk, (per_item + 127) / 128 * 128);
  for (int32_t i = 0; i < n; ++i) {
    if (t[i].q_len <= 0 || !is_decode_shard(t, m, p.shard, i, p.group)) continue;
    const int64_t vis = decode_visible(t[i]);
    const int64_t chunks = std::max<int64_t>(1, (vis + p.dec_chunk - 1) / p.dec_chunk);
    p.n_dec_items += (size_t)chunks * s->hkv;
    if (chunks > 1) {
      p.n_split += s->hkv;
      p.n_parts += (size_t)chunks * s->hkv;
    }
  }
  const size_t n_all = (size_t)n + p.splits.tasks.size();   // the table and the derived tasks
  p.off_tasks = 0;
  p.off_masks = align_up(sizeof(ca_task) * n_all);
  p.off_pages = p.off_masks + (m ? align_up(sizeof(ca_task_mask) * n_all) : 0);
  p.off_items = p.off_pages + (pg ? align_up(sizeof(int32_t) * (size_t)pg->n_pages) : 0);
  p.off_dec = p.off_items + align_up(sizeof(ca::FwdItem) * p.n_items);
  p.off_split = p.off_dec + align_up(sizeof(ca::DecItem) * p.n_dec_items);
  p.off_merge = p.off_split + align_up(4 * sizeof(int32_t) * p.n_split);
  const bool persistent = (s->flags & CA_LAUNCH_PERSISTENT) ||
                          (!(s->flags & CA_LAUNCH_PER_ITEM) && p.n_items >= kPersistMinItems);
  p.n_slots = persistent ? std::min<size_t>(kPersistSlots, p.n_items) : 0;
  p.off_counter = p.off_merge + align_up(sizeof(ca::ShardMerge) * p.splits.splits.size());
  p.off_part_o = p.off_counter + align_up(8 * sizeof(uint32_t));
  p.off_part_l = p.off_part_o + align_up(sizeof(float) * p.n_parts * p.group * s->d);
  p.off_stage_o = p.off_part_l + align_up(sizeof(float) * p.n_parts * p.group);
  p.off_stage_l = p.off_stage_o + align_up(sizeof(float) * (size_t)p.splits.stage_rows * s->hq * s->d);
  p.bytes = p.off_stage_l + align_up(sizeof(float) * (size_t)p.splits.stage_rows * s->hq);
  return p;
}

// The tasks the kernels index: the table, then the derived tasks of split
// shards (masks likewise when present).
const ca_task& task_at(const ca_task* t, int32_t n, const ShardSplits& S, int32_t i) {
  return i < n ? t[i] : S.tasks[(size_t)(i - n)];
}

// Items of one shard row tile for every head group: whole, or one per key
// chunk when the shard is split.
template <class Push>
void shard_tile_items(const ca_task* t, const ca_task_mask* m, int32_t n, const ShardSplits& S, int32_t i,
                      int32_t n_seg, int32_t r0, int64_t r1, int hkv, int head_subs, int hpw, Push push) {
  const int32_t sp = S.split_of[(size_t)i];
  if (sp < 0) {
    const int64_t cost = shard_range_pairs(t, m, i, n_seg, r0, r1) * hpw + (r1 - r0 + 1) * 64;
    for (int32_t g = 0; g < hkv; ++g)
      for (int32_t hs = 0; hs < head_subs; ++hs) push(cost, ca::FwdItem{i, (int16_t)g, (int16_t)hs, r0, n_seg, -1});
    return;
  }
  const ShardSplits::Split& spl = S.splits[(size_t)sp];
  for (size_t c = 0; c < spl.chunk_first.size(); ++c) {
    int64_t pairs = 0;
    for (int32_t k = spl.chunk_first[c]; k < spl.chunk_first[c] + spl.chunk_n[c]; ++k) {
      const ca_task& x = task_at(t, n, S, k);
      pairs += range_pairs(r0, r1, x.q_pos0 - x.kv_pos0, x.kv_len);
    }
    const int64_t cost = pairs * hpw + (r1 - r0 + 1) * 64;
    const int32_t stage_row = (int32_t)(spl.stage_row0 + (int64_t)c * t[i].q_len);
    for (int32_t g = 0; g < hkv; ++g)
      for (int32_t hs = 0; hs < head_subs; ++hs)
        push(cost, ca::FwdItem{spl.chunk_first[c], (int16_t)g, (int16_t)hs, r0, spl.chunk_n[c], stage_row});
  }
}

// Merge records of the split shards (o_off: output rows; for the dQ side the
// caller passes q_off instead).
std::vector<ca::ShardMerge> shard_merges(const ca_task* t, const ShardSplits& S, bool dq) {
  std::vector<ca::ShardMerge> r;
  for (const ShardSplits::Split& sp : S.splits) {
    const ca_task& x = t[sp.task];
    r.push_back({dq ? x.q_off : x.o_off, sp.stage_row0, x.q_len, (int32_t)sp.chunk_first.size()});
  }
  return r;
}

void build_forward_items(const ca_shape* s, const ca_task* t, const ca_task_mask* m, int32_t n,
                         const FwdPlan& p, std::vector<ca::FwdItem>& items) {
  struct Keyed {
    int64_t cost;
    ca::FwdItem it;
  };
  std::vector<Keyed> tmp;
  tmp.reserve(p.n_items);
  for (int32_t i = 0; i < n; ++i) {
    const ca_task& k = t[i];
    const int32_t n_seg = p.shard[(size_t)i];
    if (k.q_len <= 0 || n_seg == 0 || is_decode_shard(t, m, p.shard, i, p.group)) continue;
    for (int32_t r0 = 0; r0 < k.q_len; r0 += p.rt) {
      const int64_t r1 = std::min<int64_t>(r0 + p.rt, k.q_len) - 1;
      // pairs of the tile (per head) plus a per-row epilogue term
      shard_tile_items(t, m, n, p.splits, i, n_seg, r0, r1, s->hkv, p.group / p.hpw, p.hpw,
                       [&](int64_t cost, const ca::FwdItem& it) { tmp.push_back({cost, it}); });
    }
  }
  // Shard-major: the costliest query shard first, its row tiles last-first
  // (the longest), then the next shard.  The KV heads of one row tile stay
  // adjacent, so they land on different XCDs (workgroups are dealt to the 8
  // XCDs in turn, and so are persistent claims), and each XCD's workgroups run
  // the row tiles of the same shard and KV head side by side: they stream the
  // same context at nearly the same pace, and its tiles are served from that
  // XCD's L2 instead of being fetched once per row tile.
  std::vector<int64_t> shard_cost((size_t)n + p.splits.tasks.size(), 0);   // by first task (derived chunks too)
  for (const Keyed& k : tmp) shard_cost[(size_t)k.it.task] += k.cost;
  std::stable_sort(tmp.begin(), tmp.end(), [&](const Keyed& a, const Keyed& b) {
    const int64_t sa = shard_cost[(size_t)a.it.task], sb = shard_cost[(size_t)b.it.task];
    if (sa != sb) return sa > sb;
    if (a.it.task != b.it.task) return a.it.task < b.it.task;
    return a.it.row0 > b.it.row0;
  });
  items.resize(tmp.size());
  for (size_t i = 0; i < tmp.size(); ++i) items[i] = tmp[i].it;
}

// Decode items (longest chunk first) and the merge records of split tasks:
// split[0..n) first staging slot, [n..2n) chunk count, [2n..3n) task,
// [3n..4n) KV head.
void build_decode_items(const ca_shape* s, const ca_task* t, const ca_task_mask* m, int32_t n,
                        const FwdPlan& p, std::vector<ca::DecItem>& items, std::vector<int32_t>& split) {
  items.clear();
  split.assign(4 * p.n_split, 0);
  size_t rec = 0;
  int32_t part = 0;
  for (int32_t i = 0; i < n; ++i) {
    const ca_task& k = t[i];
    if (k.q_len <= 0 || !is_decode_shard(t, m, p.shard, i, p.group)) continue;
    const int64_t vis = decode_visible(k);
    const int64_t chunks = std::max<int64_t>(1, (vis + p.dec_chunk - 1) / p.dec_chunk);
    for (int32_t g = 0; g < s->hkv; ++g) {
      if (chunks > 1) {
        split[rec] = part;
        split[p.n_split + rec] = (int32_t)chunks;
        split[2 * p.n_split + rec] = i;
        split[3 * p.n_split + rec] = g;
        ++rec;
      }
      for (int64_t c = 0; c < chunks; ++c) {
        ca::DecItem it{};
        it.task = i;
        it.kv_head = g;
        it.k_begin = (int32_t)(c * p.dec_chunk);
        it.k_end = (int32_t)std::min<int64_t>(vis, (c + 1) * p.dec_chunk);
        it.part = chunks > 1 ? part++ : -1;
        items.push_back(it);
      }
    }
  }
  std::stable_sort(items.begin(), items.end(), [](const ca::DecItem& a, const ca::DecItem& b) {
    return (a.k_end - a.k_begin) > (b.k_end - b.k_begin);
  });
}

constexpr uint64_t kPlanMagic = 0x43414657504c414eull;   // plan tag, checked at launch
static_assert(sizeof(ca::PreparedFwd) <= sizeof(ca_forward_plan), "ca_forward_plan too small");

}  // namespace

// Validates, plans and builds the queue on the host; see ca_internal.h.
ca_status ca::build_forward_queue(const ca_shape* s, const ca_task* t, const ca_task_mask* m, int32_t n,
                                  const ca_kv_pages* pg, const void* const* tensors, PreparedFwd& pf,
                                  std::vector<char>& host, size_t* bytes_needed) {
  *bytes_needed = 0;
  host.clear();
  ca_status st = check_forward_args(s, t, m, n, pg);
  if (st != CA_OK) return st;
  const FwdPlan p = plan_forward(s, t, m, n, pg);
  std::memset(&pf, 0, sizeof(pf));
  pf.magic = kPlanMagic;
  pf.shape = *s;
  if (p.n_items == 0 && p.n_dec_items == 0) return CA_OK;
  if (tensors)
    for (int i = 0; i < 5; ++i)
      if (!tensors[i]) return fail(CA_ERR_INVALID, "NULL tensor pointer");
  if (p.n_items > 0x7fffffffu || p.n_dec_items > 0x7fffffffu || p.n_parts > 0x7fffffffu)
    return fail(CA_ERR_UNSUPPORTED, "too many work items");
  std::vector<ca::FwdItem> items;
  build_forward_items(s, t, m, n, p, items);
  std::vector<ca::DecItem> ditems;
  std::vector<int32_t> split;
  build_decode_items(s, t, m, n, p, ditems, split);
  host.assign(p.off_part_o, 0);
  std::memcpy(host.data() + p.off_tasks, t, sizeof(ca_task) * (size_t)n);
  if (!p.splits.tasks.empty())
    std::memcpy(host.data() + p.off_tasks + sizeof(ca_task) * (size_t)n, p.splits.tasks.data(),
                sizeof(ca_task) * p.splits.tasks.size());
  if (m) {
    std::memcpy(host.data() + p.off_masks, m, sizeof(ca_task_mask) * (size_t)n);
    if (!p.splits.masks.empty())
      std::memcpy(host.data() + p.off_masks + sizeof(ca_task_mask) * (size_t)n, p.splits.masks.data(),
                  sizeof(ca_task_mask) * p.splits.masks.size());
  }
  const std::vector<ca::ShardMerge> merges = shard_merges(t, p.splits, false);
  if (!merges.empty())
    std::memcpy(host.data() + p.off_merge, merges.data(), sizeof(ca::ShardMerge) * merges.size());
  if (pg && pg->n_pages > 0)
    std::memcpy(host.data() + p.off_pages, pg->table_host, sizeof(int32_t) * (size_t)pg->n_pages);
  if (!items.empty()) std::memcpy(host.data() + p.off_items, items.data(), sizeof(ca::FwdItem) * items.size());
  if (!ditems.empty()) std::memcpy(host.data() + p.off_dec, ditems.data(), sizeof(ca::DecItem) * ditems.size());
  if (!split.empty()) std::memcpy(host.data() + p.off_split, split.data(), sizeof(int32_t) * split.size());
  pf.group = p.group;
  pf.hpw = p.hpw;
  pf.n_items = (int32_t)items.size();
  pf.n_dec_items = (int32_t)ditems.size();
  pf.n_split = (int32_t)p.n_split;
  pf.has_masks = m ? 1 : 0;
  pf.multi = p.multi;
  pf.has_pages = pg ? 1 : 0;
  pf.page_shift = pg ? page_shift_of(pg) : 0;
  pf.page_bytes = pg ? (uint32_t)(4 * pg->n_pages) : 0u;
  pf.off_tasks = p.off_tasks;
  pf.off_masks = p.off_masks;
  pf.off_pages = p.off_pages;
  pf.off_items = p.off_items;
  pf.off_dec = p.off_dec;
  pf.off_split = p.off_split;
  pf.off_part_o = p.off_part_o;
  pf.off_part_l = p.off_part_l;
  pf.off_merge = p.off_merge;
  pf.off_stage_o = p.off_stage_o;
  pf.off_stage_l = p.off_stage_l;
  pf.n_merge = (int32_t)p.splits.splits.size();
  pf.max_q_len = p.splits.max_q_len;
  pf.n_slots = (int32_t)p.n_slots;
  pf.off_counter = p.off_counter;
  *bytes_needed = p.bytes;
  return CA_OK;
}

namespace {

using ca::PreparedFwd;

// Validates, plans, builds the queue and uploads it into ws on the stream.
// With tensors given (a direct call) they are checked before the upload, so
// a rejected call changes nothing.
ca_status prepare_forward(const ca_shape* s, const ca_task* t, const ca_task_mask* m, int32_t n,
                          const ca_kv_pages* pg, void* ws, size_t ws_bytes, void* stream, PreparedFwd& pf,
                          const void* const* tensors = nullptr) {
  std::vector<char> host;
  size_t need = 0;
  ca_status st = ca::build_forward_queue(s, t, m, n, pg, tensors, pf, host, &need);
  if (st != CA_OK) return st;
  pf.ws = ws;
  if (!tensors) {
    // a plan is launched later, perhaps with another device current
    const hipError_t e = hipGetDevice(&pf.device);
    if (e != hipSuccess) {
      pf.magic = 0;
      return hip_fail(e, "hipGetDevice");
    }
  }
  if (pf.n_items == 0 && pf.n_dec_items == 0) return CA_OK;
  if (!ws || ws_bytes < need) return fail(CA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  return upload(ws, host, (hipStream_t)stream);
}

}  // namespace

// Kernel launches only: no host planning, no copies, no allocation.
ca_status ca::launch_prepared_forward(const PreparedFwd& pf, const void* Q, const void* K, const void* V, void* O,
                                      float* LSE, void* stream) {
  if (pf.n_items == 0 && pf.n_dec_items == 0) return CA_OK;
  if (!Q || !K || !V || !O || !LSE) return fail(CA_ERR_INVALID, "NULL tensor pointer");
  const ca_shape* s = &pf.shape;
  hipStream_t hs = (hipStream_t)stream;
  char* w = (char*)pf.ws;
  const float scale_log2 = s->scale * 1.4426950408889634f;
  const int out_f32 = (s->flags & CA_OUT_F32) ? 1 : 0;
  const int32_t* pages = pf.has_pages ? (const int32_t*)(w + pf.off_pages) : nullptr;
  if (pf.n_items > 0) {
    ca::FwdParams fp;
    fp.Q = (const __bf16*)Q;
    fp.K = (const __bf16*)K;
    fp.V = (const __bf16*)V;
    fp.O = O;
    fp.LSE = LSE;
    fp.tasks = (const ca_task*)(w + pf.off_tasks);
    fp.masks = pf.has_masks ? (const ca_task_mask*)(w + pf.off_masks) : nullptr;
    fp.items = (const ca::FwdItem*)(w + pf.off_items);
    fp.pages = pages;
    fp.page_bytes = pf.page_bytes;
    fp.page_shift = pf.page_shift;
    fp.n_items = pf.n_items;
    fp.hq = s->hq;
    fp.hkv = s->hkv;
    fp.group = pf.group;
    fp.hpw = pf.hpw;
    fp.scale_log2 = scale_log2;
    fp.out_f32 = out_f32;
    fp.multi = pf.multi;
    fp.stage_O = (float*)(w + pf.off_stage_o);
    fp.stage_LSE = (float*)(w + pf.off_stage_l);
    fp.counter = pf.n_slots > 0 ? (uint32_t*)(w + pf.off_counter) : nullptr;
    fp.n_slots = (int32_t)kPersistSlots;
    hipError_t e = hipSuccess;
    if (fp.counter) {
      // a kernel, not a memset: prepared launches may be captured in graphs
      e = ca::launch_zero_f32((float*)fp.counter, 8, hs);
      if (e != hipSuccess) return hip_fail(e, "claim counter reset");
    }
    e = ca::launch_forward(fp, s->d, hs);
    if (e != hipSuccess) return hip_fail(e, "forward launch");
    if (pf.n_merge > 0) {
      e = ca::launch_shard_merge((const ca::ShardMerge*)(w + pf.off_merge), pf.n_merge, pf.max_q_len, fp.stage_O,
                                 fp.stage_LSE, O, LSE, out_f32, s->hq, s->d, hs);
      if (e != hipSuccess) return hip_fail(e, "split-shard merge launch");
    }
  }
  if (pf.n_dec_items > 0) {
    ca::DecParams dp;
    dp.Q = (const __bf16*)Q;
    dp.K = (const __bf16*)K;
    dp.V = (const __bf16*)V;
    dp.O = O;
    dp.LSE = LSE;
    dp.part_O = (float*)(w + pf.off_part_o);
    dp.part_LSE = (float*)(w + pf.off_part_l);
    dp.tasks = (const ca_task*)(w + pf.off_tasks);
    dp.items = (const ca::DecItem*)(w + pf.off_dec);
    dp.pages = pages;
    dp.page_bytes = pf.page_bytes;
    dp.page_shift = pf.page_shift;
    dp.n_items = pf.n_dec_items;
    dp.hq = s->hq;
    dp.hkv = s->hkv;
    dp.group = pf.group;
    dp.scale_log2 = scale_log2;
    dp.out_f32 = out_f32;
    hipError_t e = ca::launch_decode(dp, s->d, hs);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    if (pf.n_split > 0) {
      ca::DecMergeParams mp;
      const int32_t* sp = (const int32_t*)(w + pf.off_split);
      mp.part_O = dp.part_O;
      mp.part_LSE = dp.part_LSE;
      mp.first_part = sp;
      mp.n_parts = sp + pf.n_split;
      mp.task_of = sp + 2 * pf.n_split;
      mp.head_of = sp + 3 * pf.n_split;
      mp.tasks = dp.tasks;
      mp.O = O;
      mp.LSE = LSE;
      mp.n_split = pf.n_split;
      mp.hq = s->hq;
      mp.group = pf.group;
      mp.out_f32 = out_f32;
      e = ca::launch_decode_merge(mp, s->d, hs);
      if (e != hipSuccess) return hip_fail(e, "decode merge launch");
    }
  }
  return CA_OK;
}

namespace {

ca_status forward_impl(const ca_shape* s, const ca_task* t, const ca_task_mask* m, int32_t n,
                       const ca_kv_pages* pg, const void* Q, const void* K, const void* V, void* O, float* LSE,
                       void* ws, size_t ws_bytes, void* stream) {
  PreparedFwd pf;
  const void* tensors[5] = {Q, K, V, O, LSE};
  const ca_status st = prepare_forward(s, t, m, n, pg, ws, ws_bytes, stream, pf, tensors);
  if (st != CA_OK) return st;
  return ca::launch_prepared_forward(pf, Q, K, V, O, LSE, stream);
}

// ---------------------------------------------------------------------------
// Backward plan
// ---------------------------------------------------------------------------
//
// dQ rows and dK/dV rows may be shared by several tasks (ring partials share
// query shards and KV blocks).  Tasks are split into passes whose row ranges
// are pairwise disjoint (greedy interval partitioning), so a pass can write
// without atomics; with more than one pass the gradients accumulate in fp32
// workspace buffers and are converted at the end.  With one pass the kernels
// store bf16 directly.

constexpr int kBwdKeyTile = 128;

// pass index of every task for intervals [start, start + len); len == 0 tasks
// get pass 0.  Returns the number of passes.
int partition_passes(const std::vector<std::pair<int64_t, int64_t>>& iv, std::vector<int>& pass_of) {
  const size_t n = iv.size();
  pass_of.assign(n, 0);
  std::vector<size_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) { return iv[a].first < iv[b].first; });
  std::vector<int64_t> pass_end;  // end of the last interval in each pass
  for (size_t k : order) {
    if (iv[k].second <= 0) continue;
    int chosen = -1;
    for (size_t q = 0; q < pass_end.size(); ++q)
      if (pass_end[q] <= iv[k].first) { chosen = (int)q; break; }
    if (chosen < 0) {
      chosen = (int)pass_end.size();
      pass_end.push_back(0);
    }
    pass_end[chosen] = iv[k].first + iv[k].second;
    pass_of[k] = chosen;
  }
  return std::max<int>(1, (int)pass_end.size());
}

// Physical pages read by task i of a paged table (in virtual order).
std::vector<int32_t> task_pages(const ca_task& k, const ca_kv_pages* pg) {
  std::vector<int32_t> out;
  if (k.kv_len <= 0) return out;
  const int64_t first = k.kv_off / pg->page_rows, last = (k.kv_off + k.kv_len - 1) / pg->page_rows;
  for (int64_t v = first; v <= last; ++v) out.push_back(pg->table_host[v]);
  return out;
}

// Paged K/V: dK/dV rows are physical, so tasks conflict when they share a
// physical page.  Greedy: each task (in table order) takes the first pass
// none of whose tasks uses any of its pages.  Returns the number of passes.
int partition_page_passes(const ca_task* t, int32_t n, const ca_kv_pages* pg, int64_t n_phys,
                          std::vector<int>& pass_of) {
  pass_of.assign((size_t)n, 0);
  std::vector<std::vector<uint8_t>> used;
  for (int32_t i = 0; i < n; ++i) {
    if (t[i].q_len <= 0 || t[i].kv_len <= 0) continue;
    const std::vector<int32_t> pages = task_pages(t[i], pg);
    size_t q = 0;
    for (; q < used.size(); ++q) {
      bool free = true;
      for (int32_t pp : pages)
        if (used[q][(size_t)pp]) { free = false; break; }
      if (free) break;
    }
    if (q == used.size()) used.emplace_back((size_t)n_phys, 0);
    for (int32_t pp : pages) used[q][(size_t)pp] = 1;
    pass_of[(size_t)i] = (int)q;
  }
  return std::max<int>(1, (int)used.size());
}

// Context groups of the dK/dV kernel: active tasks (q_len > 0, kv_len > 0)
// with the same context rows [kv_off, kv_off + kv_len).  A work item of a
// group sweeps the query rows of every member, so context rows that several
// tasks read (a shared sink block or question, a ring block) are written once,
// by one item.
struct KvGroups {
  std::vector<int32_t> members;        // task indices, group after group, each in table order
  std::vector<int32_t> first, count;   // per group: its members' range in `members`
  std::vector<ca_task> rep;            // per group: its first member
};

// Context groups over the candidate tasks cand (indices into t).
KvGroups kv_groups(const ca_task* t, const std::vector<int32_t>& cand) {
  KvGroups g;
  g.members = cand;
  std::stable_sort(g.members.begin(), g.members.end(), [&](int32_t a, int32_t b) {
    return t[a].kv_off != t[b].kv_off ? t[a].kv_off < t[b].kv_off : t[a].kv_len < t[b].kv_len;
  });
  for (size_t k = 0; k < g.members.size(); ++k) {
    const ca_task& x = t[g.members[k]];
    if (k == 0 || x.kv_off != g.rep.back().kv_off || x.kv_len != g.rep.back().kv_len) {
      g.first.push_back((int32_t)k);
      g.count.push_back(0);
      g.rep.push_back(x);
    }
    ++g.count.back();
  }
  return g;
}

// Context pieces for the dK/dV kernel: every context is cut at the first and
// the past-the-end rows of every other context that fall strictly inside it,
// so that contexts which overlap become runs of identical pieces (each a
// derived task: the same query rows over a sub-range of the keys, positions
// and mask kept).  Tasks whose pieces coincide form one context group, and
// groups no longer overlap, so the dK/dV items write their rows in a single
// pass: no fp32 accumulation, one launch.  (The causal-blockwise mask, whose
// windows overlap their neighbours', is the case that needs it.)  Paged calls
// keep whole contexts (their passes follow shared pages), and so does a table
// whose cuts would multiply its contexts beyond kMaxPieceFactor * n + 65,536.
constexpr int64_t kMaxPieceFactor = 4;

struct KvPieces {
  std::vector<ca_task> tasks;         // derived pieces
  std::vector<ca_task_mask> masks;    // their masks (the source task's)
  std::vector<int32_t> members;       // dK/dV candidates: table index, or first_index + k for piece k
};

KvPieces kv_pieces(const ca_task* t, const ca_task_mask* m, int32_t n, int32_t first_index, bool cut) {
  KvPieces P;
  std::vector<int64_t> pts;
  for (int32_t i = 0; i < n; ++i)
    if (t[i].q_len > 0 && t[i].kv_len > 0) {
      pts.push_back(t[i].kv_off);
      pts.push_back(t[i].kv_off + t[i].kv_len);
    }
  std::sort(pts.begin(), pts.end());
  pts.erase(std::unique(pts.begin(), pts.end()), pts.end());
  int64_t n_cuts = 0;
  for (int32_t i = 0; i < n && cut; ++i) {
    if (t[i].q_len <= 0 || t[i].kv_len <= 0) continue;
    const int64_t lo = t[i].kv_off, hi = lo + t[i].kv_len;
    n_cuts += std::lower_bound(pts.begin(), pts.end(), hi) - std::upper_bound(pts.begin(), pts.end(), lo);
  }
  if (n_cuts > kMaxPieceFactor * n + 65536 || (int64_t)first_index + n + n_cuts > INT32_MAX / 2) cut = false;
  for (int32_t i = 0; i < n; ++i) {
    const ca_task& x = t[i];
    if (x.q_len <= 0 || x.kv_len <= 0) continue;
    const int64_t lo = x.kv_off, hi = lo + x.kv_len;
    auto a = std::upper_bound(pts.begin(), pts.end(), lo);
    auto b = std::lower_bound(pts.begin(), pts.end(), hi);
    if (!cut || a == b) {
      P.members.push_back(i);
      continue;
    }
    int64_t from = lo;
    for (auto it = a;; ++it) {
      const int64_t to = it == b ? hi : *it;
      ca_task d = x;
      d.kv_off = from;
      d.kv_len = (int32_t)(to - from);
      d.kv_pos0 = x.kv_pos0 + (from - lo);
      P.members.push_back(first_index + (int32_t)P.tasks.size());
      P.tasks.push_back(d);
      P.masks.push_back(m ? m[i] : ca_task_mask{0, 0});
      if (it == b) break;
      from = to;
    }
  }
  return P;
}

// One dK/dV work unit (per KV head): 128 keys of a context group, and the
// query rows it sweeps; split units write partial slots.
struct KvUnit {
  int64_t cost;
  int32_t group, key0, member0, n_members, row_lo, row_hi;
  int32_t split;       // index of the split tile among the pass's reductions, or -1
};

struct BwdPlan {
  int group = 1, hpw = 1, rt = 128;
  int q_passes = 1, kv_passes = 1;
  std::vector<int32_t> shard;                    // query_shards()
  KvGroups groups;
  std::vector<int> q_pass_of, kv_pass_of;        // per task (shard starts) / per context group
  bool q_full = false, kv_full = false;          // every row covered by some task
  int multi = 0;                                 // a shard or a context group with several tasks, or a split
  ShardSplits splits;                            // dQ side: long shards split over key chunks
  KvPieces pieces;                               // dK/dV side: contexts cut where others start / end
  std::vector<ca_task> ext_tasks;                // table, split-shard chunks, context pieces
  std::vector<ca_task_mask> ext_masks;           // likewise (empty without masks)
  std::vector<KvUnit> units;                     // dK/dV work units (replicated per KV head)
  std::vector<std::pair<int32_t, int32_t>> split_tiles;   // (group, key0) of every split tile
  size_t n_slots = 0;                            // partial slots (per KV head included)
  size_t n_qitems = 0, n_kvitems = 0, n_reduce = 0;
  size_t off_tasks = 0, off_masks = 0, off_pages = 0, off_members = 0, off_qitems = 0, off_kvitems = 0,
         off_reduce = 0, off_qmerge = 0, off_d = 0, off_dq = 0, off_dk = 0, off_dv = 0, off_slot_k = 0,
         off_slot_v = 0, off_stage_dq = 0, bytes = 0;
};

// A tile's query rows above which its dK/dV work is split over several
// items: when the tile's work (rows x the group's heads) exceeds a quarter of
// one compute unit's share of the call (all tiles' rows x heads over 256
// CUs), so that no item alone makes a tail; at least kMinSplitRows rows per
// item.
constexpr int64_t kMinSplitRows = 8192;
constexpr int64_t kSplitShareRows = 4 * 256;

// Task-relative query rows [r_lo, r_end) of task i that see any key of the
// 128-key tile at context row k0.
std::pair<int64_t, int64_t> tile_rows(const ca_task* t, const ca_task_mask* m, int32_t i, int64_t k0) {
  const ca_task& k = t[i];
  const int64_t delta = k.q_pos0 - k.kv_pos0;
  const int32_t win = task_window(m, i);
  const int64_t sj = task_sink_keys(t, m, i);
  // rows that see the tile: i >= k0 - delta, and (window, no sink key)
  // i < last key - delta + win
  const int64_t r_lo = std::min<int64_t>(k.q_len, std::max<int64_t>(0, k0 - delta));
  int64_t r_end = k.q_len;
  if (win > 0 && k0 >= sj) {
    const int64_t last = std::min<int64_t>(k0 + kBwdKeyTile, k.kv_len) - 1;
    r_end = std::min<int64_t>(k.q_len, std::max<int64_t>(r_lo, last - delta + win));
  }
  return {r_lo, r_end};
}

// dK/dV work units of every (context group, key tile), with long tiles split
// over member ranges, or over 32-aligned row ranges of one member, into
// items of about equal rows.
void plan_kv_units(const ca_task* t, const ca_task_mask* m, int hkv, BwdPlan& p) {
  const KvGroups& G = p.groups;
  struct Tile { int32_t group, key0; int64_t rows; };
  std::vector<Tile> tiles;
  std::vector<int64_t> member_rows;   // per tile, per member (flattened)
  int64_t total = 0;
  for (size_t gi = 0; gi < G.rep.size(); ++gi)
    for (int32_t k0 = 0; k0 < G.rep[gi].kv_len; k0 += kBwdKeyTile) {
      int64_t rows = 0;
      for (int32_t q = G.first[gi]; q < G.first[gi] + G.count[gi]; ++q) {
        const auto rr = tile_rows(t, m, G.members[(size_t)q], k0);
        member_rows.push_back(rr.second - rr.first);
        rows += rr.second - rr.first;
      }
      tiles.push_back({(int32_t)gi, k0, rows});
      total += rows;
    }
  // an item's work is rows * G (one KV head), the call's total * G * hkv
  const int64_t max_rows = std::max<int64_t>(kMinSplitRows, total / kSplitShareRows * hkv);
  size_t mr = 0;
  for (const Tile& tl : tiles) {
    const int32_t first = G.first[(size_t)tl.group], count = G.count[(size_t)tl.group];
    const int64_t* rows_of = member_rows.data() + mr;
    mr += (size_t)count;
    auto unit_cost = [&](int64_t rows) { return rows * p.group * kBwdKeyTile + 64 * kBwdKeyTile; };
    if (tl.rows <= max_rows) {
      p.units.push_back({unit_cost(tl.rows), tl.group, tl.key0, first, count, 0, INT32_MAX, -1});
      continue;
    }
    const int32_t split = (int32_t)p.split_tiles.size();
    p.split_tiles.push_back({tl.group, tl.key0});
    const int64_t n_parts = (tl.rows + max_rows - 1) / max_rows;
    const int64_t chunk = (tl.rows + n_parts - 1) / n_parts;
    int32_t open0 = -1;                  // first member of the open unit
    int64_t open_rows = 0;
    auto close = [&](int32_t end) {
      if (open0 >= 0) p.units.push_back({unit_cost(open_rows), tl.group, tl.key0, first + open0, end - open0, 0,
                                         INT32_MAX, split});
      open0 = -1;
      open_rows = 0;
    };
    for (int32_t k = 0; k < count; ++k) {
      const int64_t r = rows_of[k];
      if (r > chunk) {
        close(k);
        const auto rm = tile_rows(t, m, G.members[(size_t)(first + k)], tl.key0);
        const int64_t step = (chunk + 31) / 32 * 32;
        for (int64_t a = rm.first / 32 * 32; a < rm.second; a += step)
          p.units.push_back({unit_cost(std::min(rm.second, a + step) - std::max(a, rm.first)), tl.group, tl.key0,
                             first + k, 1, (int32_t)a, (int32_t)std::min<int64_t>(rm.second, a + step), split});
        continue;
      }
      if (open0 >= 0 && open_rows + r > chunk) close(k);
      if (open0 < 0) open0 = k;
      open_rows += r;
    }
    close(count);
  }
}

BwdPlan plan_backward(const ca_shape* s, const ca_task* t, const ca_task_mask* m, int32_t n,
                      const ca_kv_pages* pg = nullptr) {
  BwdPlan p;
  p.group = s->hq / s->hkv;
  p.hpw = gcd_int(p.group, 4);
  p.rt = 32 * (kBwdQWaves / p.hpw);   // dQ work items: rows of one item
  p.shard = query_shards(t, n);
  std::vector<bool> active_q((size_t)n, false);
  for (int32_t i = 0; i < n; ++i) active_q[(size_t)i] = t[i].q_len > 0 && p.shard[(size_t)i] > 0;
  p.splits = plan_shard_splits(t, m, n, p.shard, p.rt, s->hq, p.hpw, active_q);
  if (!p.splits.splits.empty()) p.multi = 1;
  // the device's task table: the caller's, the split-shard chunks, the pieces
  p.pieces = kv_pieces(t, m, n, n + (int32_t)p.splits.tasks.size(), pg == nullptr);
  p.ext_tasks.assign(t, t + n);
  p.ext_tasks.insert(p.ext_tasks.end(), p.splits.tasks.begin(), p.splits.tasks.end());
  p.ext_tasks.insert(p.ext_tasks.end(), p.pieces.tasks.begin(), p.pieces.tasks.end());
  if (m) {
    p.ext_masks.assign(m, m + n);
    p.ext_masks.insert(p.ext_masks.end(), p.splits.masks.begin(), p.splits.masks.end());
    p.ext_masks.insert(p.ext_masks.end(), p.pieces.masks.begin(), p.pieces.masks.end());
  }
  const ca_task* et = p.ext_tasks.data();
  const ca_task_mask* em = m ? p.ext_masks.data() : nullptr;
  p.groups = kv_groups(et, p.pieces.members);
  const size_t n_groups = p.groups.rep.size();
  std::vector<std::pair<int64_t, int64_t>> qiv(n), kviv(n_groups);
  int64_t q_cover = 0, kv_cover = 0;
  for (int32_t i = 0; i < n; ++i) {
    const bool active = active_q[(size_t)i];
    qiv[i] = {t[i].q_off, active ? t[i].q_len : 0};
    if (active) {
      if (p.shard[(size_t)i] > 1) p.multi = 1;
      const int32_t sp = p.splits.split_of[(size_t)i];
      const size_t chunks = sp >= 0 ? p.splits.splits[(size_t)sp].chunk_first.size() : 1;
      p.n_qitems += (size_t)((t[i].q_len + p.rt - 1) / p.rt) * s->hkv * (p.group / p.hpw) * chunks;
      q_cover += t[i].q_len;
    }
  }
  for (size_t g = 0; g < n_groups; ++g) {
    const ca_task& x = p.groups.rep[g];
    kviv[g] = {x.kv_off, x.kv_len};
    if (p.groups.count[g] > 1) p.multi = 1;
    kv_cover += x.kv_len;
  }
  plan_kv_units(et, em, s->hkv, p);
  p.n_kvitems = p.units.size() * (size_t)s->hkv;
  p.n_reduce = p.split_tiles.size() * (size_t)s->hkv;
  for (const KvUnit& u : p.units)
    if (u.split >= 0) ++p.n_slots;
  p.n_slots *= (size_t)s->hkv;
  if (!p.split_tiles.empty()) p.multi = 1;
  p.q_passes = partition_passes(qiv, p.q_pass_of);
  p.kv_passes = pg ? partition_page_passes(p.groups.rep.data(), (int32_t)n_groups, pg, s->kv_rows / pg->page_rows,
                                           p.kv_pass_of)
                   : partition_passes(kviv, p.kv_pass_of);
  p.q_full = p.q_passes == 1 && q_cover == s->q_rows;
  p.kv_full = !pg && p.kv_passes == 1 && kv_cover == s->kv_rows;   // paged: unread page rows stay zero
  const size_t n_all = p.ext_tasks.size();   // the table and the derived tasks
  p.off_tasks = 0;
  p.off_masks = align_up(sizeof(ca_task) * n_all);
  p.off_pages = p.off_masks + (m ? align_up(sizeof(ca_task_mask) * n_all) : 0);
  p.off_members = p.off_pages + (pg ? align_up(sizeof(int32_t) * (size_t)pg->n_pages) : 0);
  p.off_qitems = p.off_members + align_up(sizeof(int32_t) * p.groups.members.size());
  p.off_kvitems = p.off_qitems + align_up(sizeof(ca::FwdItem) * p.n_qitems);
  p.off_reduce = p.off_kvitems + align_up(sizeof(ca::BwdItem) * p.n_kvitems);
  p.off_qmerge = p.off_reduce + align_up(sizeof(ca::KvReduce) * p.n_reduce);
  p.off_d = p.off_qmerge + align_up(sizeof(ca::ShardMerge) * p.splits.splits.size());
  p.off_dq = p.off_d + align_up(sizeof(float) * (size_t)s->o_rows * s->hq);
  const size_t dq_bytes = p.q_passes > 1 ? sizeof(float) * (size_t)s->q_rows * s->hq * s->d : 0;
  const size_t dkv_bytes = p.kv_passes > 1 ? sizeof(float) * (size_t)s->kv_rows * s->hkv * s->d : 0;
  const size_t slot_bytes = sizeof(float) * p.n_slots * kBwdKeyTile * s->d;
  p.off_dk = p.off_dq + align_up(dq_bytes);
  p.off_dv = p.off_dk + align_up(dkv_bytes);
  p.off_slot_k = p.off_dv + align_up(dkv_bytes);
  p.off_slot_v = p.off_slot_k + align_up(slot_bytes);
  p.off_stage_dq = p.off_slot_v + align_up(slot_bytes);
  p.bytes = p.off_stage_dq + align_up(sizeof(float) * (size_t)p.splits.stage_rows * s->hq * s->d);
  return p;
}

// Items of every pass, pass-major, each pass longest first; pass_begin has
// passes + 1 entries.
void build_backward_items(const ca_shape* s, const ca_task* t, const ca_task_mask* m, int32_t n, const BwdPlan& p,
                          const ca_kv_pages* pg, std::vector<ca::FwdItem>& qitems, std::vector<size_t>& q_begin,
                          std::vector<ca::BwdItem>& kvitems, std::vector<size_t>& kv_begin,
                          std::vector<ca::KvReduce>& reduces, std::vector<size_t>& reduce_begin,
                          std::vector<ca::ShardMerge>& qmerges, std::vector<size_t>& qmerge_begin) {
  qitems.clear();
  kvitems.clear();
  reduces.clear();
  qmerges.clear();
  q_begin.assign(1, 0);
  kv_begin.assign(1, 0);
  reduce_begin.assign(1, 0);
  qmerge_begin.assign(1, 0);
  for (int pass = 0; pass < p.q_passes; ++pass) {
    struct K { int64_t c; ca::FwdItem it; };
    std::vector<K> tmp;
    for (int32_t i = 0; i < n; ++i) {
      const ca_task& k = t[i];
      const int32_t n_seg = p.shard[(size_t)i];
      if (k.q_len <= 0 || n_seg == 0 || p.q_pass_of[i] != pass) continue;
      for (int32_t r0 = 0; r0 < k.q_len; r0 += p.rt) {
        const int64_t r1 = std::min<int64_t>(r0 + p.rt, k.q_len) - 1;
        shard_tile_items(t, m, n, p.splits, i, n_seg, r0, r1, s->hkv, p.group / p.hpw, p.hpw,
                         [&](int64_t cost, const ca::FwdItem& it) { tmp.push_back({cost, it}); });
      }
    }
    // shard-major, as the forward's queue: an XCD's workgroups stream the
    // same context for the row tiles of one shard and KV head
    std::vector<int64_t> shard_cost((size_t)n + p.splits.tasks.size(), 0);
    for (const K& k : tmp) shard_cost[(size_t)k.it.task] += k.c;
    std::stable_sort(tmp.begin(), tmp.end(), [&](const K& a, const K& b) {
      const int64_t sa = shard_cost[(size_t)a.it.task], sb = shard_cost[(size_t)b.it.task];
      if (sa != sb) return sa > sb;
      if (a.it.task != b.it.task) return a.it.task < b.it.task;
      return a.it.row0 > b.it.row0;
    });
    for (auto& k : tmp) qitems.push_back(k.it);
    q_begin.push_back(qitems.size());
    for (size_t sp = 0; sp < p.splits.splits.size(); ++sp) {
      const ShardSplits::Split& x = p.splits.splits[sp];
      if (p.q_pass_of[(size_t)x.task] != pass) continue;
      const ca_task& q = t[x.task];
      qmerges.push_back({q.q_off, x.stage_row0, q.q_len, (int32_t)x.chunk_first.size()});
    }
    qmerge_begin.push_back(qmerges.size());
  }
  // dK/dV items pass by pass, longest first; the slots of a split tile are
  // numbered consecutively (per KV head), in unit order, and its reduction
  // records follow the pass's items.
  const KvGroups& G = p.groups;
  std::vector<int32_t> slot_of_unit(p.units.size(), -1);
  std::vector<int32_t> split_slot0(p.split_tiles.size(), -1), split_n(p.split_tiles.size(), 0);
  {
    // slots grouped per (split tile, KV head): tile-major, then head, then unit
    std::vector<std::vector<size_t>> units_of(p.split_tiles.size());
    for (size_t u = 0; u < p.units.size(); ++u)
      if (p.units[u].split >= 0) units_of[(size_t)p.units[u].split].push_back(u);
    int32_t next = 0;
    for (size_t sp = 0; sp < units_of.size(); ++sp) {
      split_slot0[sp] = next;
      split_n[sp] = (int32_t)units_of[sp].size();
      for (size_t k = 0; k < units_of[sp].size(); ++k) slot_of_unit[units_of[sp][k]] = next + (int32_t)k;
      next += split_n[sp] * s->hkv;
    }
  }
  for (int pass = 0; pass < p.kv_passes; ++pass) {
    struct K { int64_t c; int32_t group; ca::BwdItem it; };
    std::vector<K> tmp;
    std::vector<int64_t> group_cost(G.rep.size(), 0);
    for (size_t u = 0; u < p.units.size(); ++u) {
      const KvUnit& un = p.units[u];
      if (p.kv_pass_of[(size_t)un.group] != pass) continue;
      group_cost[(size_t)un.group] += un.cost;
      for (int32_t g = 0; g < s->hkv; ++g) {
        const int32_t slot = un.split >= 0 ? slot_of_unit[u] + g * split_n[(size_t)un.split] : -1;
        tmp.push_back({un.cost, un.group, {un.member0, g, un.key0, un.n_members, un.row_lo, un.row_hi, slot, 0}});
      }
    }
    // group-major: the costliest context group first, its key tiles
    // costliest first; an XCD's workgroups then stream the same query rows
    // for the key tiles of one group and KV head
    std::stable_sort(tmp.begin(), tmp.end(), [&](const K& a, const K& b) {
      const int64_t ga = group_cost[(size_t)a.group], gb = group_cost[(size_t)b.group];
      if (ga != gb) return ga > gb;
      if (a.group != b.group) return a.group < b.group;
      return a.c > b.c;
    });
    for (auto& k : tmp) kvitems.push_back(k.it);
    kv_begin.push_back(kvitems.size());
    for (size_t sp = 0; sp < p.split_tiles.size(); ++sp) {
      const int32_t gi = p.split_tiles[sp].first, k0 = p.split_tiles[sp].second;
      if (p.kv_pass_of[(size_t)gi] != pass) continue;
      const ca_task& x = G.rep[(size_t)gi];
      int64_t row0 = x.kv_off + k0;
      if (pg) {
        const int64_t v = x.kv_off + k0;
        row0 = (int64_t)pg->table_host[v / pg->page_rows] * pg->page_rows + v % pg->page_rows;
      }
      for (int32_t g = 0; g < s->hkv; ++g)
        reduces.push_back({row0, split_slot0[sp] + g * split_n[sp], split_n[sp],
                           std::min<int32_t>(kBwdKeyTile, x.kv_len - k0), g});
    }
    reduce_begin.push_back(reduces.size());
  }
}

bool varlen_to_tasks(const int32_t* cu, int32_t n_docs, std::vector<ca_task>& out) {
  if (n_docs < 0 || (n_docs > 0 && !cu)) return false;
  if (n_docs > 0 && cu[0] != 0) return false;
  out.resize((size_t)n_docs);
  for (int32_t i = 0; i < n_docs; ++i) {
    if (cu[i + 1] < cu[i]) return false;
    const int32_t l = cu[i + 1] - cu[i];
    out[(size_t)i] = ca_task{cu[i], cu[i], cu[i], l, l, 0, 0};
  }
  return true;
}

// Argument checks of the backward entry points and their workspace queries:
// those of the forward, plus (paged) no task reading one physical page twice,
// since its dK/dV rows would then be written by two work items of one pass.
ca_status check_backward_args(const ca_shape* s, const ca_task* t, const ca_task_mask* m, int32_t n,
                              const ca_kv_pages* pg) {
  ca_status st = check_forward_args(s, t, m, n, pg);
  if (st != CA_OK) return st;
  if (s->flags) return fail(CA_ERR_INVALID, "flags 0x%x: CA_OUT_F32 and CA_LAUNCH_* are forward flags", s->flags);
  if (pg) {
    std::vector<uint8_t> seen((size_t)(s->kv_rows / pg->page_rows), 0);
    for (int32_t i = 0; i < n; ++i) {
      const std::vector<int32_t> pages = task_pages(t[i], pg);
      for (int32_t pp : pages) {
        if (seen[(size_t)pp]) {
          for (int32_t q : pages) seen[(size_t)q] = 0;
          return fail(CA_ERR_INVALID, "task %d reads physical page %d twice (paged backward)", i, pp);
        }
        seen[(size_t)pp] = 1;
      }
      for (int32_t pp : pages) seen[(size_t)pp] = 0;
    }
  }
  return CA_OK;
}

ca_status backward_impl(const ca_shape* s, const ca_task* t, const ca_task_mask* m, int32_t n,
                        const ca_kv_pages* pg, const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* LSE, void* dQ, void* dK, void* dV, void* ws, size_t ws_bytes,
                        void* stream) {
  ca_status st = check_backward_args(s, t, m, n, pg);
  if (st != CA_OK) return st;
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return fail(CA_ERR_INVALID, "NULL tensor pointer");
  const BwdPlan p = plan_backward(s, t, m, n, pg);
  if (!ws || ws_bytes < p.bytes)
    return fail(CA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, p.bytes);
  if (p.n_qitems > 0x7fffffffu || p.n_kvitems > 0x7fffffffu) return fail(CA_ERR_UNSUPPORTED, "too many work items");
  for (int32_t i = 0; i < n; ++i)
    if ((int64_t)t[i].kv_len * s->hkv * s->d * 2 >= (int64_t(1) << 31))
      return fail(CA_ERR_UNSUPPORTED, "task %d: context of %d rows exceeds 2 GiB per K/V", i, t[i].kv_len);
  std::vector<ca::FwdItem> qitems;
  std::vector<ca::BwdItem> kvitems;
  std::vector<size_t> q_begin, kv_begin, reduce_begin, qmerge_begin;
  std::vector<ca::KvReduce> reduces;
  std::vector<ca::ShardMerge> qmerges;
  build_backward_items(s, t, m, n, p, pg, qitems, q_begin, kvitems, kv_begin, reduces, reduce_begin, qmerges,
                       qmerge_begin);
  std::vector<char> host(p.off_d, 0);
  std::memcpy(host.data() + p.off_tasks, p.ext_tasks.data(), sizeof(ca_task) * p.ext_tasks.size());
  if (m) std::memcpy(host.data() + p.off_masks, p.ext_masks.data(), sizeof(ca_task_mask) * p.ext_masks.size());
  if (!qmerges.empty()) std::memcpy(host.data() + p.off_qmerge, qmerges.data(), sizeof(ca::ShardMerge) * qmerges.size());
  if (pg && pg->n_pages > 0)
    std::memcpy(host.data() + p.off_pages, pg->table_host, sizeof(int32_t) * (size_t)pg->n_pages);
  if (!p.groups.members.empty())
    std::memcpy(host.data() + p.off_members, p.groups.members.data(), sizeof(int32_t) * p.groups.members.size());
  if (!qitems.empty()) std::memcpy(host.data() + p.off_qitems, qitems.data(), sizeof(ca::FwdItem) * qitems.size());
  if (!kvitems.empty()) std::memcpy(host.data() + p.off_kvitems, kvitems.data(), sizeof(ca::BwdItem) * kvitems.size());
  if (!reduces.empty()) std::memcpy(host.data() + p.off_reduce, reduces.data(), sizeof(ca::KvReduce) * reduces.size());
  hipStream_t hs = (hipStream_t)stream;
  st = upload(ws, host, hs);
  if (st != CA_OK) return st;
  char* w = (char*)ws;
  float* Dv = (float*)(w + p.off_d);
  const int64_t q_elems = s->q_rows * s->hq * (int64_t)s->d;
  const int64_t kv_elems = s->kv_rows * s->hkv * (int64_t)s->d;
  hipError_t e = ca::launch_bwd_prep((const __bf16*)O, (const __bf16*)dO, Dv, s->o_rows * (int64_t)s->hq, s->d, hs);
  if (e != hipSuccess) return hip_fail(e, "backward preprocess launch");
  const bool acc_q = p.q_passes > 1, acc_kv = p.kv_passes > 1;
  // rows no kernel writes must read as zero
  if (acc_q) e = ca::launch_zero_f32((float*)(w + p.off_dq), q_elems, hs);
  else if (!p.q_full) e = ca::launch_zero_bf16((__bf16*)dQ, q_elems, hs);
  if (e != hipSuccess) return hip_fail(e, "zero fill");
  if (acc_kv) {
    e = ca::launch_zero_f32((float*)(w + p.off_dk), kv_elems, hs);
    if (e == hipSuccess) e = ca::launch_zero_f32((float*)(w + p.off_dv), kv_elems, hs);
  } else if (!p.kv_full) {
    e = ca::launch_zero_bf16((__bf16*)dK, kv_elems, hs);
    if (e == hipSuccess) e = ca::launch_zero_bf16((__bf16*)dV, kv_elems, hs);
  }
  if (e != hipSuccess) return hip_fail(e, "zero fill");

  ca::BwdParams bp;
  bp.Q = (const __bf16*)Q;
  bp.K = (const __bf16*)K;
  bp.V = (const __bf16*)V;
  bp.dO = (const __bf16*)dO;
  bp.LSE = LSE;
  bp.Dvec = Dv;
  bp.dQ = (__bf16*)dQ;
  bp.dK = (__bf16*)dK;
  bp.dV = (__bf16*)dV;
  bp.dQacc = (float*)(w + p.off_dq);
  bp.dKacc = (float*)(w + p.off_dk);
  bp.dVacc = (float*)(w + p.off_dv);
  bp.tasks = (const ca_task*)(w + p.off_tasks);
  bp.masks = m ? (const ca_task_mask*)(w + p.off_masks) : nullptr;
  bp.members = (const int32_t*)(w + p.off_members);
  bp.multi = p.multi;
  bp.slot_k = (float*)(w + p.off_slot_k);
  bp.slot_v = (float*)(w + p.off_slot_v);
  bp.stage_dQ = (float*)(w + p.off_stage_dq);
  bp.pages = pg ? (const int32_t*)(w + p.off_pages) : nullptr;
  bp.page_bytes = pg ? (uint32_t)(4 * pg->n_pages) : 0u;
  bp.page_shift = pg ? page_shift_of(pg) : 0;
  bp.hq = s->hq;
  bp.hkv = s->hkv;
  bp.group = p.group;
  bp.hpw = p.hpw;
  bp.scale = s->scale;
  bp.scale_log2 = s->scale * 1.4426950408889634f;
  const ca::FwdItem* qi = (const ca::FwdItem*)(w + p.off_qitems);
  const ca::BwdItem* ki = (const ca::BwdItem*)(w + p.off_kvitems);
  for (int pass = 0; pass < p.q_passes; ++pass) {
    ca::BwdParams pp = bp;
    pp.accumulate = acc_q ? 1 : 0;
    pp.qitems = qi + q_begin[pass];
    pp.n_qitems = (int32_t)(q_begin[pass + 1] - q_begin[pass]);
    pp.items = nullptr;
    pp.n_items = 0;
    e = ca::launch_bwd_q(pp, s->d, hs);
    if (e != hipSuccess) return hip_fail(e, "dQ launch");
    const size_t nm = qmerge_begin[pass + 1] - qmerge_begin[pass];
    if (nm > 0) {
      e = ca::launch_dq_reduce((const ca::ShardMerge*)(w + p.off_qmerge) + qmerge_begin[pass], (int32_t)nm,
                               p.splits.max_q_len, bp.stage_dQ, (__bf16*)dQ, bp.dQacc, acc_q ? 1 : 0, s->hq, s->d,
                               hs);
      if (e != hipSuccess) return hip_fail(e, "split-shard dQ reduction launch");
    }
  }
  for (int pass = 0; pass < p.kv_passes; ++pass) {
    ca::BwdParams pp = bp;
    pp.accumulate = acc_kv ? 1 : 0;
    pp.items = ki + kv_begin[pass];
    pp.n_items = (int32_t)(kv_begin[pass + 1] - kv_begin[pass]);
    pp.qitems = nullptr;
    pp.n_qitems = 0;
    e = ca::launch_bwd_kv(pp, s->d, hs);
    if (e != hipSuccess) return hip_fail(e, "dK/dV launch");
    const size_t nr = reduce_begin[pass + 1] - reduce_begin[pass];
    if (nr > 0) {
      e = ca::launch_kv_reduce((const ca::KvReduce*)(w + p.off_reduce) + reduce_begin[pass], (int32_t)nr, bp.slot_k,
                               bp.slot_v, (__bf16*)dK, (__bf16*)dV, bp.dKacc, bp.dVacc, acc_kv ? 1 : 0, s->hkv, s->d,
                               hs);
      if (e != hipSuccess) return hip_fail(e, "dK/dV reduction launch");
    }
  }
  if (acc_q) {
    e = ca::launch_f32_to_bf16(bp.dQacc, (__bf16*)dQ, q_elems, hs);
    if (e != hipSuccess) return hip_fail(e, "dQ conversion");
  }
  if (acc_kv) {
    e = ca::launch_f32_to_bf16(bp.dKacc, (__bf16*)dK, kv_elems, hs);
    if (e == hipSuccess) e = ca::launch_f32_to_bf16(bp.dVacc, (__bf16*)dV, kv_elems, hs);
    if (e != hipSuccess) return hip_fail(e, "dK/dV conversion");
  }
  return CA_OK;
}

}  // namespace

extern "C" {

size_t ca_forward_workspace(const ca_shape* shape, const ca_task* tasks_host, int32_t n_tasks) {
  return ca_forward_masked_workspace(shape, tasks_host, nullptr, n_tasks);
}

ca_status ca_forward(const ca_shape* shape, const ca_task* tasks_host, int32_t n_tasks, const void* Q,
                     const void* K, const void* V, void* O, float* LSE, void* ws, size_t ws_bytes,
                     void* stream) {
  return forward_impl(shape, tasks_host, nullptr, n_tasks, nullptr, Q, K, V, O, LSE, ws, ws_bytes, stream);
}

ca_status ca_forward_queue_info(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                                int32_t n_tasks, int64_t info[5]) {
  if (!info) return fail(CA_ERR_INVALID, "info is NULL");
  const ca_status st = check_forward_args(shape, tasks_host, masks_host, n_tasks, nullptr);
  if (st != CA_OK) return st;
  const FwdPlan p = plan_forward(shape, tasks_host, masks_host, n_tasks);
  info[0] = (int64_t)p.n_items;
  info[1] = (int64_t)p.n_dec_items;
  info[2] = (int64_t)p.n_slots;
  info[3] = p.multi;
  info[4] = (int64_t)p.splits.splits.size();
  return CA_OK;
}

size_t ca_forward_masked_workspace(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                                   int32_t n_tasks) {
  if (check_forward_args(shape, tasks_host, masks_host, n_tasks, nullptr) != CA_OK) return 0;
  return plan_forward(shape, tasks_host, masks_host, n_tasks).bytes;
}

ca_status ca_forward_masked(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                            int32_t n_tasks, const void* Q, const void* K, const void* V, void* O, float* LSE,
                            void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(shape, tasks_host, masks_host, n_tasks, nullptr, Q, K, V, O, LSE, ws, ws_bytes, stream);
}

size_t ca_forward_paged_workspace(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                                  int32_t n_tasks, const ca_kv_pages* pages) {
  if (!pages || check_forward_args(shape, tasks_host, masks_host, n_tasks, pages) != CA_OK) return 0;
  return plan_forward(shape, tasks_host, masks_host, n_tasks, pages).bytes;
}

ca_status ca_forward_paged(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                           int32_t n_tasks, const ca_kv_pages* pages, const void* Q, const void* K, const void* V,
                           void* O, float* LSE, void* ws, size_t ws_bytes, void* stream) {
  if (!pages) return fail(CA_ERR_INVALID, "pages is NULL");
  return forward_impl(shape, tasks_host, masks_host, n_tasks, pages, Q, K, V, O, LSE, ws, ws_bytes, stream);
}

ca_status ca_forward_prepare(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                             int32_t n_tasks, const ca_kv_pages* pages, void* ws, size_t ws_bytes, void* stream,
                             ca_forward_plan* plan) {
  if (!plan) return fail(CA_ERR_INVALID, "plan is NULL");
  PreparedFwd pf;
  const ca_status st = prepare_forward(shape, tasks_host, masks_host, n_tasks, pages, ws, ws_bytes, stream, pf);
  std::memset(plan, 0, sizeof(*plan));
  if (st != CA_OK) return st;
  std::memcpy(plan, &pf, sizeof(pf));
  return CA_OK;
}

ca_status ca_forward_prepared(const ca_forward_plan* plan, const void* Q, const void* K, const void* V, void* O,
                              float* LSE, void* stream) {
  if (!plan) return fail(CA_ERR_INVALID, "plan is NULL");
  PreparedFwd pf;
  std::memcpy(&pf, plan, sizeof(pf));
  if (pf.magic != kPlanMagic) return fail(CA_ERR_INVALID, "plan was not filled by ca_forward_prepare");
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != pf.device)
    return fail(CA_ERR_INVALID, "plan was prepared on device %d, device %d is current", pf.device, dev);
  return ca::launch_prepared_forward(pf, Q, K, V, O, LSE, stream);
}

size_t ca_forward_varlen_workspace(const ca_shape* shape, const int32_t* cu, int32_t n_docs) {
  std::vector<ca_task> t;
  if (!varlen_to_tasks(cu, n_docs, t)) return 0;
  return ca_forward_workspace(shape, t.data(), n_docs);
}

ca_status ca_forward_varlen(const ca_shape* shape, const int32_t* cu, int32_t n_docs, const void* Q,
                            const void* K, const void* V, void* O, float* LSE, void* ws, size_t ws_bytes,
                            void* stream) {
  std::vector<ca_task> t;
  if (!varlen_to_tasks(cu, n_docs, t))
    return fail(CA_ERR_INVALID, "cu_seqlens must start at 0 and be non-decreasing");
  return forward_impl(shape, t.data(), nullptr, n_docs, nullptr, Q, K, V, O, LSE, ws, ws_bytes, stream);
}

ca_status ca_merge(const ca_shape* shape, int32_t n_parts, int64_t n_rows, const float* O_parts,
                   const float* LSE_parts, void* O, float* LSE, void* stream) {
  if (!shape) return fail(CA_ERR_INVALID, "shape is NULL");
  if (shape->hq < 1 || shape->hq > kMaxHeads) return fail(CA_ERR_INVALID, "hq=%d not in [1, %d]", shape->hq, kMaxHeads);
  if (shape->d != 64 && shape->d != 128) return fail(CA_ERR_UNSUPPORTED, "head dim d=%d not supported", shape->d);
  if (shape->flags & ~(uint32_t)CA_OUT_F32)
    return fail(CA_ERR_INVALID, "flags 0x%x: ca_merge takes CA_OUT_F32 only", shape->flags);
  if (n_parts < 1) return fail(CA_ERR_INVALID, "n_parts=%d must be >= 1", n_parts);
  if (n_rows < 0 || n_rows > kMaxRows) return fail(CA_ERR_INVALID, "n_rows=%lld not in [0, 2^40]", (long long)n_rows);
  if (n_rows == 0) return CA_OK;
  if (!O_parts || !LSE_parts || !O || !LSE) return fail(CA_ERR_INVALID, "NULL tensor pointer");
  if (n_rows * shape->hq * (shape->d / 4) / 256 >= 0x7fffffffLL) return fail(CA_ERR_UNSUPPORTED, "too many rows");
  ca::MergeParams mp;
  mp.O_parts = O_parts;
  mp.LSE_parts = LSE_parts;
  mp.O = O;
  mp.LSE = LSE;
  mp.n_parts = n_parts;
  mp.n_rows = n_rows;
  mp.hq = shape->hq;
  mp.out_f32 = (shape->flags & CA_OUT_F32) ? 1 : 0;
  hipError_t e = ca::launch_merge(mp, shape->d, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return CA_OK;
}

size_t ca_backward_workspace(const ca_shape* shape, const ca_task* tasks_host, int32_t n_tasks) {
  return ca_backward_masked_workspace(shape, tasks_host, nullptr, n_tasks);
}

size_t ca_backward_masked_workspace(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                                    int32_t n_tasks) {
  if (check_backward_args(shape, tasks_host, masks_host, n_tasks, nullptr) != CA_OK) return 0;
  return plan_backward(shape, tasks_host, masks_host, n_tasks).bytes;
}

ca_status ca_backward(const ca_shape* s, const ca_task* t, int32_t n, const void* Q, const void* K,
                      const void* V, const void* O, const void* dO, const float* LSE, void* dQ, void* dK,
                      void* dV, void* ws, size_t ws_bytes, void* stream) {
  return backward_impl(s, t, nullptr, n, nullptr, Q, K, V, O, dO, LSE, dQ, dK, dV, ws, ws_bytes, stream);
}

ca_status ca_backward_masked(const ca_shape* s, const ca_task* t, const ca_task_mask* m, int32_t n, const void* Q,
                             const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                             void* dQ, void* dK, void* dV, void* ws, size_t ws_bytes, void* stream) {
  return backward_impl(s, t, m, n, nullptr, Q, K, V, O, dO, LSE, dQ, dK, dV, ws, ws_bytes, stream);
}

size_t ca_backward_paged_workspace(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                                   int32_t n_tasks, const ca_kv_pages* pages) {
  if (!pages || check_backward_args(shape, tasks_host, masks_host, n_tasks, pages) != CA_OK) return 0;
  return plan_backward(shape, tasks_host, masks_host, n_tasks, pages).bytes;
}

ca_status ca_backward_paged(const ca_shape* s, const ca_task* t, const ca_task_mask* m, int32_t n,
                            const ca_kv_pages* pages, const void* Q, const void* K, const void* V, const void* O,
                            const void* dO, const float* LSE, void* dQ, void* dK, void* dV, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!pages) return fail(CA_ERR_INVALID, "pages is NULL");
  return backward_impl(s, t, m, n, pages, Q, K, V, O, dO, LSE, dQ, dK, dV, ws, ws_bytes, stream);
}

int64_t ca_visible_pairs(const ca_task* tasks_host, int32_t n_tasks) {
  return ca_visible_pairs_masked(tasks_host, nullptr, n_tasks);
}

int64_t ca_visible_pairs_masked(const ca_task* tasks_host, const ca_task_mask* masks_host, int32_t n_tasks) {
  if (n_tasks < 0 || (n_tasks > 0 && !tasks_host)) return -1;
  if (masks_host)
    for (int32_t i = 0; i < n_tasks; ++i)
      if (masks_host[i].window < 0 || masks_host[i].sink < 0) return -1;
  int64_t total = 0;
  for (int32_t i = 0; i < n_tasks; ++i) {
    const ca_task& k = tasks_host[i];
    if (k.q_len < 0 || k.kv_len < 0 || k.q_len > kMaxTaskLen || k.kv_len > kMaxTaskLen) return -1;
    total += range_pairs_masked(0, (int64_t)k.q_len - 1, k.q_pos0 - k.kv_pos0, k.kv_len,
                                task_window(masks_host, i), task_sink_keys(tasks_host, masks_host, i));
  }
  return total;
}

const char* ca_status_string(ca_status s) {
  switch (s) {
    case CA_OK: return "CA_OK";
    case CA_ERR_INVALID: return "CA_ERR_INVALID";
    case CA_ERR_UNSUPPORTED: return "CA_ERR_UNSUPPORTED";
    case CA_ERR_WORKSPACE: return "CA_ERR_WORKSPACE";
    case CA_ERR_HIP: return "CA_ERR_HIP";
  }
  return "CA_UNKNOWN_STATUS";
}

const char* ca_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
