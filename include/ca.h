/*
 * ca.h — core attention on one MI355X (gfx950): the C ABI of libca.so.
 *
 * Core attention is the parameter-free softmax(Q K^T / sqrt(d)) V between the
 * QKV and output projections of a transformer layer ("Efficient Long-context
 * Language Model Training by Core Attention Disaggregation", Sections 1 and
 * 3.2).  The library computes it over a table of CA-tasks — a query shard
 * plus its key/value context, re-batched across documents into one fused
 * launch (same page, Section 3.4, "The CA-Task Abstraction" and Property 2,
 * Composability) — and returns per-row log-sum-exp so that partial results
 * merge exactly by Equation 4 ("Context Parallelism for Scalable Million-Token
 * Inference", Section 3.4 "Merge Attention", Appendix B).
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Pointers named *_host are host memory; every other pointer is device
 *    memory on the current HIP device.  The caller allocates and owns every
 *    buffer, including the workspace; the library allocates no device memory
 *    and keeps no state between calls other than a small ring of reusable
 *    pinned host staging buffers per thread and device, through which
 *    host-built work queues are copied into the workspace; a thread's ring
 *    is released when the thread ends.
 *  - Calls are asynchronous on `stream` (a hipStream_t, passed as void*; NULL
 *    is the default stream).  Buffers must stay valid until the stream work
 *    completes.  Host arrays (*_host) are only read during the call.
 *  - Arguments are validated before anything is enqueued: a call that returns
 *    an error has no side effects on device memory.  Errors are return codes;
 *    nothing is thrown across the ABI.  ca_last_error() gives a message for
 *    the last failing call on the calling thread.
 *  - bf16 means IEEE-754 binary32 truncated to its upper 16 bits (bfloat16).
 *
 * Data layout (row-major, head-interleaved, as a packed varlen batch)
 * -------------------------------------------------------------------
 *  Q  [q_rows ][hq ][d]  bf16        dQ  same layout, bf16
 *  K  [kv_rows][hkv][d]  bf16        dK  same layout, bf16
 *  V  [kv_rows][hkv][d]  bf16        dV  same layout, bf16
 *  O  [o_rows ][hq ][d]  bf16, or fp32 when flags has CA_OUT_F32
 *  LSE[o_rows ][hq]      fp32, natural log of sum_j exp(scale * q.k_j)
 *
 *  Grouped-query attention: query head h reads KV head (h * hkv) / hq, i.e.
 *  contiguous groups of hq/hkv query heads share a KV head ("Context
 *  Parallelism ...", The CP+TP Nesting Design, Figure 5).
 */
#ifndef CA_H
#define CA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CA_OK = 0,
  CA_ERR_INVALID = -1,     /* bad shape, task or pointer                     */
  CA_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. head dim)      */
  CA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required     */
  CA_ERR_HIP = -4          /* a HIP runtime call failed; see ca_last_error() */
} ca_status;

/*
 * One CA-task: a contiguous query shard q(t) and its context kv(t)
 * ("Core Attention Disaggregation", Section 3.4).  Key j of the task is
 * visible to its query i iff  kv_pos0 + j <= q_pos0 + i  (document
 * positions; the diagonal is included — a token attends to itself).
 *   - packed causal document of length l at row r:  {r, r, r, l, l, 0, 0}
 *   - shard of n queries ending at document position e (context = prefix):
 *         {q, kv, o, n, e, e - n, 0}
 *   - ring partial of query shard [a, a+n) over key block [b, b+m):
 *         {a, b, o, n, m, a, b}
 *   - decode of one token at position p over a cache block [b, b+m):
 *         {q, kv, o, 1, m, p, b}
 * A row that sees no key gets O = 0 and LSE = -inf.
 *
 * Query shards over several contexts: consecutive tasks with the same q_off,
 * o_off, q_len and q_pos0 (q_len > 0) are one query shard whose rows attend
 * to the union of the tasks' visible keys with one softmax (a key listed by
 * two of them counts twice).  The sparse masks of "DCP: Addressing Input
 * Dynamism In Long-Context Training via Dynamic Context Parallelism"
 * (Section 2.4, Figure 6c / 6d) are such unions of key ranges:
 *   - causal-blockwise, block b of a document at row r with a window
 *     starting at block w0 > 0:  {q, r, q, n, B, q - r, 0} (the sink block,
 *     all visible) followed by {q, r + w0 B, q, n, q + n - r - w0 B, q - r, w0 B}
 *     with q = r + b B;
 *   - shared question, an answer of a rows at row x after a question of qn
 *     rows at row 0:  {x, 0, x, a, qn, qn, 0} then {x, x, x, a, a, qn, qn}.
 * Apart from the tasks of one shard, output row ranges [o_off, o_off +
 * q_len) of different tasks must not overlap (documented, not checked).
 * Context ranges may overlap.
 */
typedef struct {
  int64_t q_off;   /* first row in Q (and dQ)                              */
  int64_t kv_off;  /* first row in K, V (and dK, dV)                       */
  int64_t o_off;   /* first row in O, LSE (and O, dO, LSE in backward)     */
  int32_t q_len;   /* 0 .. 2^30                                            */
  int32_t kv_len;  /* 0 .. 2^30                                            */
  int64_t q_pos0;  /* document position of query row 0                     */
  int64_t kv_pos0; /* document position of context row 0                   */
} ca_task;

/*
 * Optional per-task narrowing of the causal mask to the lambda shape of the
 * sparse masks of "Dynamic Context Parallelism" (Section 2.4, Figure 6b): an
 * attention sink plus a sliding window.  With kp = kv_pos0 + j and
 * qp = q_pos0 + i, key j is visible to query i iff
 *     kp <= qp  and  (window == 0  or  kp > qp - window  or  kp < sink):
 * the query sees its `window` latest positions (itself included) and every
 * position below `sink`.  window == 0 is the plain causal task (sink unused).
 * Causal-blockwise and shared-question masks are unions of key ranges:
 * write them as query shards over several contexts (see ca_task), one launch
 * with no partial slots and no merge.
 */
typedef struct {
  int32_t window;  /* >= 0                                                 */
  int32_t sink;    /* >= 0                                                 */
} ca_task_mask;

enum {
  CA_OUT_F32 = 1u << 0, /* forward/merge: write O as fp32 (partials for a later merge) */
  /* Forward launch of the tiled kernel (at most one of the two; results are
   * bit-identical either way).  By default the library picks: persistent
   * (one workgroup per compute unit, each claiming items from the
   * longest-first queue of its XCD and loading the next item's Q and first
   * K/V tiles under the current item's epilogue) when the call has at least
   * 4,096 work items, else one workgroup per item, dispatched by the
   * hardware. */
  CA_LAUNCH_PERSISTENT = 1u << 1,
  CA_LAUNCH_PER_ITEM = 1u << 2
};

typedef struct {
  int32_t hq;      /* query heads, >= 1                                    */
  int32_t hkv;     /* key/value heads, >= 1, divides hq                    */
  int32_t d;       /* head dimension: 64 or 128                            */
  float scale;     /* softmax scale applied to q.k, > 0 (usually 1/sqrt(d)) */
  uint32_t flags;  /* CA_OUT_F32, CA_LAUNCH_* (forward only)               */
  int64_t q_rows;  /* rows of Q (and dQ)                                   */
  int64_t kv_rows; /* rows of K, V (and dK, dV)                            */
  int64_t o_rows;  /* rows of O and LSE (and dO)                           */
} ca_shape;

/* ---------------------------------------------------------------------- */
/* Forward                                                                 */
/* ---------------------------------------------------------------------- */

/* Bytes of device workspace ca_forward needs for this task table (0 on an
 * invalid argument; check ca_forward's status for the reason). */
size_t ca_forward_workspace(const ca_shape* shape, const ca_task* tasks_host, int32_t n_tasks);

/* O and LSE for every row of every task, in one fused launch over all tasks
 * (fully masked key tiles are never visited).  A CA-task is a query shard and
 * the key/value context it attends to; any set of them, from any documents,
 * composes into one call ("Efficient Long-context Language Model Training by
 * Core Attention Disaggregation", Section 3.4, The CA-Task Abstraction and
 * Property 2, Composability); the per-row LSE is the log of the softmax
 * normaliser ("Context Parallelism for Scalable Million-Token Inference",
 * Section 3.4, Merge Attention).  Rows of O/LSE outside every task are not
 * written.  The call builds its work queue on the host and copies it into ws
 * on the stream, so it refuses a stream that is being captured into a graph
 * (CA_ERR_INVALID; ca_forward_prepare / ca_forward_prepared is the
 * capturable form).  Errors: CA_ERR_INVALID for a null pointer, hq/hkv not
 * dividing, hq above 4096, scale not finite or not positive, negative
 * lengths, row counts above 2^40 or any row range past
 * q_rows/kv_rows/o_rows; CA_ERR_UNSUPPORTED for d not in {64, 128};
 * CA_ERR_WORKSPACE when ws_bytes < ca_forward_workspace(...). */
ca_status ca_forward(const ca_shape* shape, const ca_task* tasks_host, int32_t n_tasks,
                     const void* Q, const void* K, const void* V, void* O, float* LSE,
                     void* ws, size_t ws_bytes, void* stream);

/* ca_forward with a ca_task_mask per task (masks_host may be NULL: all
 * causal).  Single-row tasks with a window run in the tiled kernel instead
 * of the split-KV decode kernel.  Errors as ca_forward, plus CA_ERR_INVALID
 * for a negative window or sink. */
size_t ca_forward_masked_workspace(const ca_shape* shape, const ca_task* tasks_host,
                                   const ca_task_mask* masks_host, int32_t n_tasks);
ca_status ca_forward_masked(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                            int32_t n_tasks, const void* Q, const void* K, const void* V, void* O,
                            float* LSE, void* ws, size_t ws_bytes, void* stream);

/* How ca_forward_masked would launch this call (host only, no device work):
 * info[0] work items of the tiled kernel, info[1] split-KV decode items,
 * info[2] persistent workgroups of the tiled kernel (0: one workgroup per
 * item), info[3] 1 when some query shard sweeps several contexts or is split
 * over key chunks, info[4] query shards split over key chunks.  The work queue
 * is the one a call would build (H1's longest-first items, "Efficient
 * Long-context Language Model Training by Core Attention Disaggregation",
 * Section 3.4).  Errors as ca_forward_masked (info untouched then). */
ca_status ca_forward_queue_info(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                                int32_t n_tasks, int64_t info[5]);

/*
 * Paged K/V: block tables as in the Blockwise Attention instruction of "DCP:
 * Addressing Input Dynamism In Long-Context Training via Dynamic Context
 * Parallelism" (Executor Design; its data blocks are per-head runs of B
 * tokens, Block Generation).  K and V are stores of physical pages of
 * page_rows rows: physical page p is rows [p * page_rows, (p + 1) * page_rows)
 * of K and of V.  Every task's kv_off and kv_len then address a virtual row
 * space of n_pages * page_rows rows, whose row v is the physical row
 *     table_host[v / page_rows] * page_rows + v % page_rows.
 * Pages may be shared by several virtual pages and tasks (a shared prefix).
 * Requirements, else CA_ERR_INVALID: page_rows a power of two in
 * [128, 1 << 20]; n_pages >= 0; every entry in [0, kv_rows / page_rows);
 * every task's [kv_off, kv_off + kv_len) inside the virtual space, with
 * kv_off a multiple of 128.  The call copies the table into the workspace;
 * the host array may be reused once the call has returned.
 */
typedef struct {
  const int32_t* table_host;  /* [n_pages] physical page of each virtual page */
  int64_t n_pages;            /* virtual pages                                 */
  int32_t page_rows;          /* rows per page                                 */
  int32_t reserved;           /* must be 0                                     */
} ca_kv_pages;

/* ca_forward_masked over paged K/V (pages must not be NULL; masks_host may
 * be).  Errors as ca_forward_masked, with the context ranges checked against
 * the virtual space instead of kv_rows, plus the page requirements above. */
size_t ca_forward_paged_workspace(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                                  int32_t n_tasks, const ca_kv_pages* pages);
ca_status ca_forward_paged(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                           int32_t n_tasks, const ca_kv_pages* pages, const void* Q, const void* K,
                           const void* V, void* O, float* LSE, void* ws, size_t ws_bytes, void* stream);

/* Packed causal documents: several documents concatenated into one chunk,
 * each token attending only to earlier tokens of its own document ("Efficient
 * Long-context Language Model Training by Core Attention Disaggregation",
 * Section 2, document packing).  Document i occupies rows [cu[i], cu[i+1])
 * of Q, K, V, O and LSE (the task {cu[i], cu[i], cu[i], l, l, 0, 0}).
 * cu_seqlens_host has n_docs + 1 non-decreasing entries starting at 0.
 * Errors and graph capture as ca_forward. */
size_t ca_forward_varlen_workspace(const ca_shape* shape, const int32_t* cu_seqlens_host,
                                   int32_t n_docs);
ca_status ca_forward_varlen(const ca_shape* shape, const int32_t* cu_seqlens_host, int32_t n_docs,
                            const void* Q, const void* K, const void* V, void* O, float* LSE,
                            void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------- */
/* Merge (Equation 4 of "Context Parallelism ...", Appendix B)             */
/* ---------------------------------------------------------------------- */

/* Combine n_parts partial results of the same n_rows query rows:
 *   O_parts  [n_parts][n_rows][hq][d] fp32   LSE_parts [n_parts][n_rows][hq] fp32
 *   O        [n_rows][hq][d] bf16 (fp32 with CA_OUT_F32)   LSE [n_rows][hq] fp32
 * With M = max_s LSE_s:  O = sum_s O_s e^(LSE_s - M) / sum_s e^(LSE_s - M),
 * LSE = M + ln sum_s e^(LSE_s - M).  A partial whose LSE is -inf weighs zero
 * and its O values are not read (so rows a forward never wrote need only
 * LSE = -inf); if all partials are empty, O = 0 and LSE = -inf.
 * Uses shape->hq, shape->d, shape->flags only.  No workspace. */
ca_status ca_merge(const ca_shape* shape, int32_t n_parts, int64_t n_rows,
                   const float* O_parts, const float* LSE_parts, void* O, float* LSE,
                   void* stream);

/* ---------------------------------------------------------------------- */
/* Backward                                                                */
/* ---------------------------------------------------------------------- */

/* Bytes of device workspace ca_backward needs (includes an fp32 dQ
 * accumulator of q_rows * hq * d floats). */
size_t ca_backward_workspace(const ca_shape* shape, const ca_task* tasks_host, int32_t n_tasks);

/* Gradients of sum(O * dO): dQ, dK, dV (bf16, accumulated in fp32).  O, dO
 * (bf16) and LSE (fp32) are the forward's outputs at rows o_off..; the
 * attention probabilities are recomputed from Q, K and the saved per-row
 * softmax statistics rather than stored ("Efficient Long-context Language
 * Model Training by Core Attention Disaggregation", Section 3.4, Property 1).
 * dK and dV sum over the query heads of each KV head's group and over every
 * task whose context covers a row.  Every row of dQ, dK and dV is written
 * (rows that no task touches get 0).  No atomics: tasks that share rows run
 * in separate passes, so results are bitwise reproducible.  Errors and graph
 * capture as for ca_forward (CA_OUT_F32 is rejected). */
ca_status ca_backward(const ca_shape* shape, const ca_task* tasks_host, int32_t n_tasks,
                      const void* Q, const void* K, const void* V, const void* O,
                      const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                      void* ws, size_t ws_bytes, void* stream);

/* ca_backward with a ca_task_mask per task (masks_host may be NULL: all
 * causal); the same mask as the forward that produced O and LSE.  Errors as
 * ca_backward, plus CA_ERR_INVALID for a negative window or sink. */
size_t ca_backward_masked_workspace(const ca_shape* shape, const ca_task* tasks_host,
                                    const ca_task_mask* masks_host, int32_t n_tasks);
ca_status ca_backward_masked(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                             int32_t n_tasks, const void* Q, const void* K, const void* V, const void* O,
                             const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                             void* ws, size_t ws_bytes, void* stream);

/* ca_backward_masked over paged K/V (see ca_kv_pages; pages must not be
 * NULL).  dK and dV are page stores laid out like K and V: the gradient of
 * virtual row v lands in its physical row.  Rows of pages no task reads are
 * zero.  Tasks may share physical pages (their contributions are summed);
 * one task must not read the same physical page twice (CA_ERR_INVALID).
 * Errors otherwise as ca_backward_masked and ca_forward_paged. */
size_t ca_backward_paged_workspace(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                                   int32_t n_tasks, const ca_kv_pages* pages);
ca_status ca_backward_paged(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                            int32_t n_tasks, const ca_kv_pages* pages, const void* Q, const void* K,
                            const void* V, const void* O, const void* dO, const float* LSE, void* dQ, void* dK,
                            void* dV, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------- */
/* Prepared forward: plan once, launch many times (HIP graph capture)      */
/* ---------------------------------------------------------------------- */
/* The decode step of "Context Parallelism for Scalable Million-Token
 * Inference" (Section 3.6) runs under captured graphs to avoid host launch
 * overhead.  ca_forward_prepare does a forward call's host work once: it
 * validates, builds the work queue and uploads it into ws (async on the
 * stream, not capturable), and fills *plan (host memory owned by the caller;
 * contents private).  ca_forward_prepared then only launches kernels (no
 * host planning, no copies, no allocation), reading the queue from the ws
 * the plan was made with, so it can be captured into a HIP graph and
 * replayed; Q, K, V, O and LSE may differ from call to call but must have the
 * shape and task table the plan was made for.  The caller keeps ws unchanged
 * while the plan is in use.  ws_bytes as for the direct call (ca_forward /
 * _masked / _paged _workspace).  The plan records the device current at
 * ca_forward_prepare (where ws lives); ca_forward_prepared must run with the
 * same device current.  Errors as for the direct call; the launch returns
 * CA_ERR_INVALID for a plan that ca_forward_prepare did not fill or that was
 * prepared on another device, and CA_ERR_HIP if the current device cannot be
 * read. */
typedef struct {
  uint64_t opaque[40];
} ca_forward_plan;

ca_status ca_forward_prepare(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                             int32_t n_tasks, const ca_kv_pages* pages, void* ws, size_t ws_bytes, void* stream,
                             ca_forward_plan* plan);
ca_status ca_forward_prepared(const ca_forward_plan* plan, const void* Q, const void* K, const void* V, void* O,
                              float* LSE, void* stream);

/* ---------------------------------------------------------------------- */
/* Forward without allocation                                               */
/* ---------------------------------------------------------------------- */
/* For callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  ca_forward_masked without
 * a workspace (masks_host may be NULL: all causal): the work queue and the
 * split-decode staging live in a fixed device array of the library, one per
 * GPU, of CA_NOALLOC_SCRATCH_BYTES, held from the library's load until the
 * process ends.  The host-built queue reaches it by value in the arguments of
 * small store kernels on `stream`, so the call makes no device or pinned
 * host allocation (the host-side planning uses ordinary heap memory), keeps
 * no host buffer alive after it returns, and may be captured into a graph
 * (replays store the same queue again, then run the same kernels).  Results
 * are bit-identical to ca_forward_masked on the same tasks.
 *   - The array is shared by every call on a GPU and keeps the last call's
 *     queue: calls that overlap on one GPU (different streams, or graphs
 *     replayed concurrently with other calls) race and give wrong results;
 *     serialise them.
 *   - The first call on each device looks the array's address up
 *     (hipGetSymbolAddress) with that device current; make that first call
 *     outside graph capture.
 * Errors as ca_forward_masked, plus CA_ERR_WORKSPACE when the call's queue
 * and staging (ca_forward_masked_workspace) exceed CA_NOALLOC_SCRATCH_BYTES,
 * CA_ERR_HIP if the array's address cannot be obtained. */
#define CA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ca_status ca_forward_noalloc(const ca_shape* shape, const ca_task* tasks_host, const ca_task_mask* masks_host,
                             int32_t n_tasks, const void* Q, const void* K, const void* V, void* O, float* LSE,
                             void* stream);

/* ---------------------------------------------------------------------- */
/* CA-task scheduling (host only; no device memory, no HIP calls)          */
/* ---------------------------------------------------------------------- */
/* The profiler cost model and the communication-aware greedy scheduler of
 * "Efficient Long-context Language Model Training by Core Attention
 * Disaggregation", Section 4.2 (The Profiler and Cost Model; The
 * Communication-Aware Greedy Scheduler, Steps 1-4) and Appendix B (Optimal
 * Shard Dimension Computation).  A batch of documents, first placed on k
 * devices in equal token blocks, is rebalanced across k attention servers by
 * migrating whole Items or Appendix-B-sized shards (or head-tail shards,
 * Section 4.1's per-document balance, when head_tail is set), the move that
 * carries the most predicted time per byte of communication first.
 *
 * Cost model: a measured grid of times (seconds) of one attention call with
 * n_q queries that are the last n_q tokens of an n_kv-token causal context,
 * at grid_q[i] x grid_kv[j] (both strictly increasing, >= 1), row-major
 * [n_gq][n_gkv].  Inside the grid: bilinear interpolation of time.  Beyond
 * it in both coordinates: FLOPs / the best measured throughput (saturated).
 * Beyond it in one coordinate: FLOPs / the throughput at the point clamped
 * into the grid.  FLOPs = flops_per_pair x visible pairs of the block, with
 * the query count capped at n_kv. */
typedef struct {
  int32_t k;               /* attention servers (>= 1)                                */
  int32_t hq, hkv, d;      /* attention shape; bytes per token sent: q hq*d*2, kv hkv*d*2 */
  double eps;              /* stop when a deficit is <= eps * target load (>= 0)      */
  double e_min;            /* migrations need E = dF / bytes > e_min                  */
  int64_t min_shard;       /* shortest query range a split may move (>= 1)           */
  int32_t max_moves;       /* cap on migrations (>= 0)                                */
  int32_t head_tail;       /* 0: a split moves the Appendix-B shard [n_kv - n_q, n_kv);
                              1: a split moves a head-tail shard, the first m and the
                              last m queries of the Item ([a, a+m) and [b-m, b)), with
                              m (a + b + 1) = alpha (b - a)(a + b + 1) / 2 pairs
                              rounded to nearest, 1 <= m <= (b - a) / 2, 2m >= min_shard */
  double flops_per_pair;   /* FLOPs the profiled call counts per visible pair (> 0)   */
} ca_sched_params;

typedef struct {
  int32_t server;          /* attention server 0..k-1                                 */
  int32_t doc;             /* document index                                          */
  int64_t q_begin, q_end;  /* query range [q_begin, q_end) of the document; its
                              context is the document prefix [0, q_end)              */
} ca_sched_item;           /* 24 bytes                                                */

/* Predicted seconds of an (n_q, n_kv) block under the cost model above; NaN
 * for an invalid grid. */
double ca_cost_time(const double* grid_q_host, int32_t n_gq, const double* grid_kv_host, int32_t n_gkv,
                    const double* grid_time_host, double flops_per_pair, int64_t n_q, int64_t n_kv);

/* Upper bound of the number of Items ca_schedule can return (-1 if invalid). */
int32_t ca_schedule_max_items(int32_t n_docs, int32_t k, int32_t max_moves);

/* Schedules the documents (lengths >= 0, in batch order) onto p->k servers.
 * Writes the Items (every document's query positions partitioned exactly
 * once), the per-server predicted loads before and after [k], the bytes moved
 * and the number of migrations.  All pointers are host memory owned by the
 * caller.  Deterministic.  Errors: CA_ERR_INVALID for bad parameters or grid;
 * CA_ERR_WORKSPACE (with *n_items set to the count needed) when the Items do
 * not fit in max_items. */
ca_status ca_schedule(const ca_sched_params* p, const int64_t* doc_lens_host, int32_t n_docs,
                      const double* grid_q_host, int32_t n_gq, const double* grid_kv_host, int32_t n_gkv,
                      const double* grid_time_host, ca_sched_item* items_host, int32_t max_items,
                      int32_t* n_items, double* load_before_host, double* load_after_host,
                      double* comm_bytes, int32_t* n_moves);

/* CA-task records of Items over the packed batch (documents back to back in
 * Q, K, V and O): q_off = o_off = start(doc) + q_begin, kv_off = start(doc),
 * q_len = q_end - q_begin, kv_len = q_end, q_pos0 = q_begin, kv_pos0 = 0.
 * Running the records of every server reproduces the causal attention of the
 * whole batch.  Errors: CA_ERR_INVALID for an Item outside its document or
 * kv_len beyond int32. */
ca_status ca_sched_tasks(const ca_sched_item* items_host, int32_t n_items, const int64_t* doc_lens_host,
                         int32_t n_docs, ca_task* tasks_host);

/* ---------------------------------------------------------------------- */
/* Context-parallel ring planning (host only; no device memory, no HIP)    */
/* ---------------------------------------------------------------------- */
/* "Context Parallelism for Scalable Million-Token Inference": the time model
 * and switching rules of ring pass-KV / pass-Q (Section 3.4, Equations 1-3,
 * Algorithm 1; Appendix C, Algorithm 5, Equation 5), load-balanced sharding
 * (Section 3.5.1), the pass-KV ring schedule (Section 3.5.2) and round-robin
 * decode sharding (Section 3.6).  Units: FLOPs = 4 T D (T + P); compute in
 * FLOP/s per rank; bandwidth in bytes/s per rank (ring SendRecv); seconds. */
typedef struct {
  int32_t n_ranks;         /* N (>= 1)                                                */
  int32_t n_heads;         /* N_H query heads (>= 1)                                  */
  int32_t n_kv_heads;      /* N_KV key/value heads (>= 1)                             */
  int32_t elem_bytes;      /* e, bytes per element of Q / K / V / O on the wire (>= 1) */
  double d_model;          /* D, model dimension (> 0)                                */
  double compute;          /* C, attention FLOP/s per rank (> 0)                      */
  double bandwidth;        /* BW, SendRecv bytes/s per rank (> 0)                     */
} ca_ring_model;

typedef struct {
  double attn_step;        /* 4 T D (T + P) / (N C): one ring step's attention        */
  double sendrecv_kv;      /* 2 (T + P) D e N_KV / (N_H BW): one pass-KV message      */
  double sendrecv_q;       /* T D e / BW: one pass-Q message                          */
  double all2all;          /* (N - 1)(D + 1) T e / BW: pass-Q's return of partials    */
  double exposed_kv;       /* (N - 1)(sendrecv_kv - attn_step), may be negative       */
  double miss_threshold;   /* Equation 1: 2 N_KV / N_H                                */
  double t_threshold;      /* Equation 2: N C N_KV e / (2 N_H BW)                      */
  double ctx_threshold;    /* Equation 3: N e C / (4 BW)                               */
  double eq5_rhs;          /* Equation 5: 2 N_KV / N_H - 4 T BW / (N C e)              */
} ca_ring_times;

enum { CA_RING_PASS_KV = 0, CA_RING_PASS_Q = 1 };

/* Every term of the model at (T new tokens, P cached tokens); T, P >= 0.
 * Errors: CA_ERR_INVALID for a bad model or NULL output. */
ca_status ca_ring_plan(const ca_ring_model* m, int64_t T, int64_t P, ca_ring_times* out);

/* pass-KV (0) or pass-Q (1) for T >= 1 new tokens over P >= 0 cached ones.
 * refined = 0: Algorithm 1 (pass-KV iff T >= t_threshold or T/(T+P) >=
 * miss_threshold).  refined = 1: Algorithm 5 (pass-KV iff T >= t_threshold,
 * else pass-Q iff exposed_kv >= all2all).  -1 on invalid arguments. */
int32_t ca_ring_select(const ca_ring_model* m, int64_t T, int64_t P, int32_t refined);

/* The same choice from measured per-step times (seconds, >= 0): each ring
 * exposes (N - 1) max(0, SendRecv - ATTN), pass-Q adds its All2All; pass-Q iff
 * strictly less exposed.  Writes both exposed times when the pointers are not
 * NULL.  -1 on invalid arguments. */
int32_t ca_ring_select_measured(int32_t n_ranks, double sendrecv_kv, double sendrecv_q, double attn,
                                double all2all, double* exposed_kv, double* exposed_q);

typedef struct {
  int32_t rank;            /* owning rank, 0..N-1                                      */
  int32_t seq;             /* sequence index                                           */
  int64_t begin, end;      /* token positions [begin, end) of the sequence, may be empty */
} ca_ring_chunk;           /* 24 bytes                                                 */

/* Load-balanced sharding of n_seqs sequences (lengths >= 0) over N ranks:
 * 2N chunks of ceil(L / 2N) positions per sequence, clipped at L; chunk k
 * belongs to rank k (k < N) or 2N - 1 - k.  Writes n_seqs * 2N chunks in
 * (sequence, k) order into caller-owned host memory. */
ca_status ca_ring_shard(int32_t n_ranks, const int64_t* lens_host, int32_t n_seqs, ca_ring_chunk* chunks_host);

/* Upper bound of the task count of one pass-KV step (-1 if invalid). */
int32_t ca_ring_kv_step_max_tasks(int32_t n_ranks, int32_t n_seqs);

/* CA-task records of pass-KV step `step` (0..N-1), slot 0 or 1, for the
 * full prefill of n_seqs packed sequences (Q, K, V, O rows back to back in
 * sequence order): every rank r's two query chunks of every sequence against
 * chunk (slot 0: src, slot 1: 2N - 1 - src) of rank src = (r - step) mod N,
 * with in-sequence positions as q_pos0 / kv_pos0.  Every non-empty query
 * chunk appears exactly once per (step, slot), so the 2N launches (fp32
 * partial outputs) merged by ca_merge give the causal attention of every
 * sequence.  Errors: CA_ERR_INVALID; CA_ERR_WORKSPACE when more than
 * max_tasks records are needed (*n_tasks then holds the bound). */
ca_status ca_ring_kv_step_tasks(int32_t n_ranks, int32_t step, int32_t slot, const int64_t* lens_host,
                                int32_t n_seqs, ca_task* tasks_host, int32_t max_tasks, int32_t* n_tasks);

/* Partial prefill ([CP] Section 3.5.1 for the new tokens, Section 3.5.2 ring):
 * sequence s brings new_lens[s] new tokens on top of cached_lens[s] cached
 * ones.  Q and O rows hold the new tokens, sequences back to back; K and V
 * rows hold each sequence's cached tokens followed by its new ones.  The new
 * tokens are sharded load-balanced; the cached tokens keep the load-balanced
 * sharding of their own earlier prefill.  Step `step`, slot 0..3: every rank
 * r's two query chunks of every sequence against, of rank (r - step) mod N,
 * its first / second cached chunk (slots 0, 1; visible to every new query) or
 * its first / second chunk of new tokens (slots 2, 3; causal).  The 4N
 * launches (fp32 partial outputs) merged by ca_merge give each new token's
 * attention over its whole sequence, the same for pass-KV and pass-Q (which
 * differ only in which rank computes a pair).  With every cached length 0
 * slots 0 and 1 hold empty contexts.  Errors as for ca_ring_kv_step_tasks. */
int32_t ca_ring_prefill_step_max_tasks(int32_t n_ranks, int32_t n_seqs);
ca_status ca_ring_prefill_step_tasks(int32_t n_ranks, int32_t step, int32_t slot, const int64_t* new_lens_host,
                                     const int64_t* cached_lens_host, int32_t n_seqs, ca_task* tasks_host,
                                     int32_t max_tasks, int32_t* n_tasks);

/* Rank that stores the decode token of batch entry seq at decode iteration
 * `iteration`: (seq + iteration) mod N.  -1 on invalid arguments. */
int32_t ca_ring_decode_rank(int32_t n_ranks, int64_t iteration, int32_t seq);

/* ---------------------------------------------------------------------- */
/* Accounting and errors                                                   */
/* ---------------------------------------------------------------------- */

/* Number of visible (query, key) pairs of a task table, per query head
 * (FLOPs = 4 d pairs hq forward, 10 d pairs hq backward).  -1 on an invalid
 * table (negative lengths or lengths above 2^30, a NULL table, a negative
 * window or sink).  Closed form: the cost does not grow with the lengths. */
int64_t ca_visible_pairs(const ca_task* tasks_host, int32_t n_tasks);
/* The same under per-task masks (masks_host may be NULL). */
int64_t ca_visible_pairs_masked(const ca_task* tasks_host, const ca_task_mask* masks_host, int32_t n_tasks);

const char* ca_status_string(ca_status status);
const char* ca_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CA_H */
