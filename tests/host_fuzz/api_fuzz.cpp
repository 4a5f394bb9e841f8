// Host-only fuzz of argument validation and work planning (workspace queries,
// visible-pair counts) under ASan/UBSan; kernel launchers are stubs.
#include <cstdint>
#include <cstdio>
#include <random>
#include <algorithm>
#include <vector>
#include "ca_internal.h"
namespace ca {
hipError_t launch_forward(const FwdParams&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_decode(const DecParams&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_decode_merge(const DecMergeParams&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_merge(const MergeParams&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_prep(const __bf16*, const __bf16*, float*, int64_t, int, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_kv(const BwdParams&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_q(const BwdParams&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_f32_to_bf16(const float*, __bf16*, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_zero_f32(float*, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_zero_bf16(__bf16*, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_shard_merge(const ShardMerge*, int32_t, int32_t, const float*, const float*, void*, float*, int, int,
                              int, hipStream_t) { return hipSuccess; }
hipError_t launch_dq_reduce(const ShardMerge*, int32_t, int32_t, const float*, __bf16*, float*, int, int, int,
                            hipStream_t) { return hipSuccess; }
hipError_t launch_kv_reduce(const KvReduce*, int32_t, const float*, const float*, __bf16*, __bf16*, float*, float*, int,
                            int, int, hipStream_t) { return hipSuccess; }
}
int main() {
  std::mt19937_64 rng(11);
  auto U = [&](int64_t a, int64_t b) { return std::uniform_int_distribution<int64_t>(a, b)(rng); };
  size_t sink = 0;
  for (int it = 0; it < 4000; ++it) {
    ca_shape s{};
    s.hkv = (int)U(1, 8); s.hq = s.hkv * (int)U(1, 16); s.d = U(0, 5) ? 128 : 64; s.scale = U(0, 20) ? 0.088f : -1.f;
    s.flags = U(0, 7); s.q_rows = U(0, 100000); s.kv_rows = U(0, 100000); s.o_rows = s.q_rows * U(1, 3);
    if (!U(0, 30)) s.q_rows = INT64_MAX - U(0, 10);    // huge row counts are rejected, not multiplied
    if (!U(0, 30)) s.hq = s.hkv * (int)U(1 << 12, 1 << 20);
    int n = (int)U(0, 30);
    std::vector<ca_task> t(n + 1);
    std::vector<ca_task_mask> m(n + 1);
    for (int i = 0; i < n; ++i) {
      ca_task& x = t[i];
      x.q_len = (int)U(U(0, 50) ? 0 : -3, 3000); x.kv_len = (int)U(U(0, 50) ? 0 : -3, 9000);
      x.q_off = U(0, 1) ? U(0, 100000) : U(-5, 5); x.kv_off = U(0, 100000); x.o_off = U(0, 100000);
      if (!U(0, 8)) {   // offsets at and near INT64_MAX: range checks must not overflow
        int64_t* off[3] = {&x.q_off, &x.kv_off, &x.o_off};
        *off[U(0, 2)] = INT64_MAX - U(0, 4000);
      }
      if (!U(0, 40)) {  // lengths near INT32_MAX: rejected before any tile arithmetic
        int32_t* len[2] = {&x.q_len, &x.kv_len};
        *len[U(0, 1)] = INT32_MAX - (int32_t)U(0, 200);
      }
      x.q_pos0 = U(0, 20000); x.kv_pos0 = U(0, 20000);
      m[i].window = (int)U(0, 3) ? 0 : (int)U(-1, 5000); m[i].sink = (int)U(-1, 100);
    }
    sink += ca_forward_workspace(&s, t.data(), n);
    sink += ca_forward_masked_workspace(&s, t.data(), m.data(), n);
    sink += ca_backward_workspace(&s, t.data(), n);
    sink += ca_backward_masked_workspace(&s, t.data(), m.data(), n);
    sink += (size_t)ca_visible_pairs(t.data(), n);
    sink += (size_t)ca_visible_pairs_masked(t.data(), m.data(), n);
    std::vector<int32_t> cu(n + 2);
    cu[0] = 0;
    for (int i = 1; i <= n; ++i) cu[i] = cu[i - 1] + (int32_t)U(U(0, 40) ? 0 : -2, 500);
    sink += ca_forward_varlen_workspace(&s, cu.data(), n);
    std::vector<int32_t> table(64);
    for (auto& x : table) x = (int32_t)U(-1, 70);
    ca_kv_pages pg{table.data(), (int64_t)U(0, 64), (int32_t)(U(0, 3) ? 128 << U(0, 3) : U(1, 300)), 0};
    sink += ca_forward_paged_workspace(&s, t.data(), m.data(), n, &pg);
    sink += ca_backward_paged_workspace(&s, t.data(), m.data(), n, &pg);
  }
  // valid by construction: every task inside its buffers
  int valid_nonzero = 0;
  for (int it = 0; it < 4000; ++it) {
    ca_shape s{};
    s.hkv = (int)U(1, 8); s.hq = s.hkv * (int)U(1, 16); s.d = U(0, 1) ? 128 : 64; s.scale = 0.088f;
    s.flags = U(0, 7); s.q_rows = U(1, 20000); s.kv_rows = U(1, 20000); s.o_rows = s.q_rows;
    int n = (int)U(1, 20);
    std::vector<ca_task> t(n);
    std::vector<ca_task_mask> m(n);
    for (int i = 0; i < n; ++i) {
      ca_task& x = t[i];
      x.q_len = (int)U(0, s.q_rows); x.q_off = U(0, s.q_rows - x.q_len); x.o_off = x.q_off;
      x.kv_len = (int)U(0, s.kv_rows); x.kv_off = U(0, s.kv_rows - x.kv_len);
      x.q_pos0 = U(0, 30000); x.kv_pos0 = U(0, 30000);
      if (U(0, 1)) x.q_len = std::min<int32_t>(x.q_len, 1);
      m[i].window = (int)U(0, 2) ? 0 : (int)U(1, 5000); m[i].sink = (int)U(0, 100);
    }
    size_t a = ca_forward_workspace(&s, t.data(), n), b = ca_forward_masked_workspace(&s, t.data(), m.data(), n);
    sink += a + b + ca_backward_workspace(&s, t.data(), n) + ca_backward_masked_workspace(&s, t.data(), m.data(), n);
    sink += (size_t)ca_visible_pairs(t.data(), n) + (size_t)ca_visible_pairs_masked(t.data(), m.data(), n);
    valid_nonzero += a > 0;
  }
  // query shards over several contexts (runs of tasks sharing their query
  // rows) and context groups (tasks sharing their context rows)
  for (int it = 0; it < 3000; ++it) {
    ca_shape s{};
    s.hkv = (int)U(1, 4); s.hq = s.hkv * (int)U(1, 8); s.d = U(0, 1) ? 128 : 64; s.scale = 0.088f;
    s.q_rows = U(1, 5000); s.kv_rows = U(1, 5000); s.o_rows = s.q_rows;
    std::vector<ca_task> t;
    std::vector<ca_task_mask> m;
    const int n_shards = (int)U(1, 12);
    for (int k = 0; k < n_shards; ++k) {
      ca_task base{};
      base.q_len = (int)U(0, std::min<int64_t>(s.q_rows, 700));
      base.q_off = U(0, s.q_rows - base.q_len); base.o_off = base.q_off;
      base.q_pos0 = U(0, 9000);
      const int n_seg = (int)U(1, 4);
      for (int j = 0; j < n_seg; ++j) {
        ca_task x = base;
        if (!t.empty() && !U(0, 3)) { x.kv_off = t.back().kv_off; x.kv_len = t.back().kv_len; }
        else { x.kv_len = (int)U(0, s.kv_rows); x.kv_off = U(0, s.kv_rows - x.kv_len); }
        x.kv_pos0 = U(0, 9000);
        t.push_back(x);
        m.push_back({(int)U(0, 2) ? 0 : (int)U(1, 3000), (int)U(0, 50)});
      }
    }
    const int n = (int)t.size();
    sink += ca_forward_workspace(&s, t.data(), n) + ca_forward_masked_workspace(&s, t.data(), m.data(), n);
    sink += ca_backward_workspace(&s, t.data(), n) + ca_backward_masked_workspace(&s, t.data(), m.data(), n);
    sink += (size_t)ca_visible_pairs_masked(t.data(), m.data(), n);
  }
  std::printf("api host fuzz done %zu (valid cases with a workspace: %d)\n", sink % 7, valid_nonzero);
  return 0;
}
