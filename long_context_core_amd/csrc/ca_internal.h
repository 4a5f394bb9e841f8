// Internal declarations shared by the host API and the HIP kernels of libca.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/ca.h"

namespace ca {

// One forward work item: a tile of query rows of one query shard (tasks
// task .. task + n_seg - 1, which share their query rows and are swept by one
// online softmax), for a subset of the query heads that share one KV head.
// The workgroup's eight waves cover hpw heads x (8 / hpw) blocks of 32 rows.
struct FwdItem {
  int32_t task;
  int16_t kv_head;
  int16_t head_sub;  // which group of hpw heads inside the KV head's group
  int32_t row0;      // first task-relative query row
  int32_t n_seg;     // contexts of the shard (consecutive tasks)
  int32_t stage_row; // -1; or a key chunk of a split shard: its fp32 partial
                     // output goes to staging row stage_row + query row
};

// A query shard split over key chunks: chunk c's partial outputs are staging
// rows stage_row0 + c * q_len + (0 .. q_len - 1); the forward merges them by
// Equation 4 into O / LSE rows o_off.., the dQ kernel's are summed into dQ
// rows q_off...
struct ShardMerge {
  int64_t o_off;     // output rows (forward) / dQ rows (backward)
  int64_t stage_row0;
  int32_t q_len, n_chunks;
};

// Split-KV decode work item: one task (a single query row), one KV head, all
// query heads of its group, keys [k_begin, k_end) of the task's context.
// Writes a partial (O, LSE) to slot `part` of the decode staging area, or
// straight to the output when the task is not split.
struct DecItem {
  int32_t task;
  int32_t kv_head;
  int32_t k_begin;
  int32_t k_end;
  int32_t part;    // staging slot, or -1: write the final O/LSE of the task
  int32_t pad[3];
};

// Backward work item (dK/dV kernel): 128 context rows of a context group
// (tasks with the same context rows, listed at members[member0 ..
// member0 + n_members)), one KV head; it sweeps the query rows of every
// member.  A tile whose query rows are too many for one item is split into
// several items over member ranges (or, for one member, row ranges [row_lo,
// row_hi)) that write fp32 partial dK / dV to a slot; a reduction sums the
// slots in order.
struct BwdItem {
  int32_t member0;
  int32_t kv_head;
  int32_t key0;      // first context-relative row of the tile
  int32_t n_members;
  int32_t row_lo, row_hi;  // task-relative query rows swept (all: 0, INT32_MAX)
  int32_t slot;            // -1: write dK / dV; else the partial slot
  int32_t pad;
};

// Reduction of the partial slots of one split (tile, KV head): dK / dV of
// rows row0 .. row0 + n_keys - 1 = sum of slots slot0 .. slot0 + n_slots - 1.
struct KvReduce {
  int64_t row0;      // physical K/V row of the tile's first key
  int32_t slot0, n_slots, n_keys, kv_head;
};

struct FwdParams {
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  void* O;
  float* LSE;
  const ca_task* tasks;
  const ca_task_mask* masks;   // per task, or nullptr: causal only
  const FwdItem* items;
  const int32_t* pages;   // K/V block table (virtual page -> physical page), or nullptr: rows are physical
  uint32_t page_bytes;    // bytes of the table
  int32_t page_shift;     // log2 of the rows per page
  int32_t n_items;
  int32_t hq, hkv, group, hpw;
  float scale_log2;   // softmax scale * log2(e)
  int32_t out_f32;
  int32_t multi;      // some item has n_seg > 1 or a staging row
  float* stage_O;     // [stage rows][hq][d] fp32 partials of split shards
  float* stage_LSE;   // [stage rows][hq]
  uint32_t* counter;  // persistent launch: 8 claim counters, one per XCD (zero at launch); nullptr: one
                      // workgroup per item
  int32_t n_slots;    // persistent workgroups (a multiple of 8; the grid is min(n_slots, n_items))
};

struct DecParams {
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  void* O;
  float* LSE;
  float* part_O;      // [n_parts][group][d] fp32 staging for split tasks
  float* part_LSE;    // [n_parts][group]
  const ca_task* tasks;
  const DecItem* items;
  const int32_t* pages;   // as in FwdParams
  uint32_t page_bytes;
  int32_t page_shift;
  int32_t n_items;
  int32_t hq, hkv, group;
  float scale_log2;
  int32_t out_f32;
};

struct DecMergeParams {
  const float* part_O;
  const float* part_LSE;
  const int32_t* first_part;   // per split task: first staging slot
  const int32_t* n_parts;      // per split task: number of slots
  const int32_t* task_of;      // per split task: task index
  const int32_t* head_of;      // per split task: KV head
  const ca_task* tasks;
  void* O;
  float* LSE;
  int32_t n_split;
  int32_t hq, group;
  int32_t out_f32;
};

struct MergeParams {
  const float* O_parts;
  const float* LSE_parts;
  void* O;
  float* LSE;
  int32_t n_parts;
  int64_t n_rows;
  int32_t hq;
  int32_t out_f32;
};

struct BwdParams {
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  const __bf16* dO;
  const float* LSE;
  const float* Dvec;  // [o_rows][hq] rowsum(dO * O)
  __bf16* dQ;
  __bf16* dK;
  __bf16* dV;
  float* dQacc;       // [q_rows][hq][d] fp32, used when accumulate != 0 (dQ kernel)
  float* dKacc;       // [kv_rows][hkv][d] fp32, used when accumulate != 0 (dK/dV kernel)
  float* dVacc;
  const ca_task* tasks;
  const ca_task_mask* masks;   // per task, or nullptr: causal only
  const int32_t* members;      // task indices of the context groups (dK/dV items)
  const int32_t* pages;   // as in FwdParams
  uint32_t page_bytes;
  int32_t page_shift;
  const BwdItem* items;   // dK/dV kernel
  int32_t n_items;
  float* slot_k;          // [slots][128][d] fp32 partial dK of split items (scaled), and dV
  float* slot_v;
  float* stage_dQ;        // [stage rows][hq][d] fp32 partial dQ of split shards (scaled)
  const FwdItem* qitems;  // dQ kernel
  int32_t n_qitems;
  int32_t hq, hkv, group, hpw;
  float scale;
  float scale_log2;
  int32_t accumulate;
  int32_t multi;          // a shard (dQ items) or a context group (dK/dV items) of several tasks
};

// A forward call whose work queue is built: what its launch needs once the
// queue is in a device buffer (ws): the shape, the queue layout and counts.
// Plain data, so it can live in the caller's ca_forward_plan.
struct PreparedFwd {
  uint64_t magic;
  void* ws;                 // device buffer holding the queue (and decode staging)
  int32_t device;           // current device at preparation: ws lives there
  ca_shape shape;
  int32_t group, hpw;
  int32_t n_items, n_dec_items, n_split;
  int32_t has_masks, has_pages, page_shift;
  uint32_t page_bytes;
  int32_t multi;            // some query shard has several contexts or is split
  int32_t n_merge;          // split shards
  int32_t max_q_len;        // longest split shard
  int32_t n_slots;          // persistent workgroups (0: one workgroup per item)
  uint64_t off_tasks, off_masks, off_pages, off_items, off_dec, off_split, off_merge, off_part_o, off_part_l,
      off_stage_o, off_stage_l, off_counter;
};

// Validates a forward call (tensors: Q, K, V, O, LSE, or nullptr to skip the
// pointer checks) and builds its work queue on the host: `host` receives the
// bytes that must be at the start of the device buffer before the launch
// (task table, masks, page table, work items, decode merge records), and
// *bytes_needed the whole buffer size (the rest is staging the kernels write
// before reading).  Fills pf except pf.ws and pf.device.  No HIP calls.
ca_status build_forward_queue(const ca_shape* s, const ca_task* t, const ca_task_mask* m, int32_t n,
                              const ca_kv_pages* pg, const void* const* tensors, PreparedFwd& pf,
                              std::vector<char>& host, size_t* bytes_needed);

// The kernel launches of a built queue whose bytes are in pf.ws: no host
// planning, no copies, no allocation.
ca_status launch_prepared_forward(const PreparedFwd& pf, const void* Q, const void* K, const void* V, void* O,
                                  float* LSE, void* stream);

// Kernel launchers (defined in the .hip files).
hipError_t launch_forward(const FwdParams& p, int d, hipStream_t s);
hipError_t launch_decode(const DecParams& p, int d, hipStream_t s);
hipError_t launch_decode_merge(const DecMergeParams& p, int d, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, int d, hipStream_t s);
hipError_t launch_bwd_prep(const __bf16* O, const __bf16* dO, float* Dv, int64_t n_pairs, int d, hipStream_t s);
hipError_t launch_bwd_kv(const BwdParams& p, int d, hipStream_t s);
hipError_t launch_bwd_q(const BwdParams& p, int d, hipStream_t s);
hipError_t launch_shard_merge(const ShardMerge* recs, int32_t n_recs, int32_t max_q_len, const float* stage_O,
                              const float* stage_LSE, void* O, float* LSE, int out_f32, int hq, int d, hipStream_t s);
hipError_t launch_dq_reduce(const ShardMerge* recs, int32_t n_recs, int32_t max_q_len, const float* stage_dQ,
                            __bf16* dQ, float* dQacc, int accumulate, int hq, int d, hipStream_t s);
hipError_t launch_kv_reduce(const KvReduce* recs, int32_t n_recs, const float* slot_k, const float* slot_v,
                            __bf16* dK, __bf16* dV, float* dKacc, float* dVacc, int accumulate, int hkv, int d,
                            hipStream_t s);
hipError_t launch_f32_to_bf16(const float* src, __bf16* dst, int64_t n, hipStream_t s);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);
hipError_t launch_zero_bf16(__bf16* p, int64_t n, hipStream_t s);

// Records the thread's last-error text (ca_last_error) and returns st.
ca_status set_error(ca_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace ca
