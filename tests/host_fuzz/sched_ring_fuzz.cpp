// Host-only fuzz of the scheduler and ring planning under ASan/UBSan.
#include <cstdarg>
#include <cstdio>
#include <random>
#include <vector>
#include "ca.h"
namespace ca { ca_status set_error(ca_status st, const char*, ...) { return st; } }
int main() {
  std::mt19937_64 rng(7);
  auto U = [&](int64_t a, int64_t b) { return std::uniform_int_distribution<int64_t>(a, b)(rng); };
  for (int it = 0; it < 3000; ++it) {
    int n = (int)U(0, 40);
    std::vector<int64_t> docs(n);
    for (auto& d : docs) d = U(0, 1) ? U(0, 300) : U(0, 200000);
    int k = (int)U(1, 16);
    double gq[3] = {64, 1024, 16384}, gkv[3] = {64, 8192, 262144}, gt[9];
    for (int i = 0; i < 9; ++i) gt[i] = 1e-5 * (i + 1);
    ca_sched_params p{};
    p.k = k; p.hq = 32; p.hkv = 8; p.d = 128; p.eps = U(0, 3) * 0.02; p.e_min = 0; p.min_shard = U(1, 256);
    p.max_moves = (int)U(0, 50); p.head_tail = (int)U(0, 1); p.flops_per_pair = 4 * 128 * 32;
    int cap = ca_schedule_max_items(n, k, p.max_moves);
    std::vector<ca_sched_item> items(cap > 0 ? cap : 1);
    std::vector<double> lb(k), la(k);
    int32_t ni = 0, mv = 0; double comm = 0;
    if (ca_schedule(&p, docs.data(), n, gq, 3, gkv, 3, gt, items.data(), cap, &ni, lb.data(), la.data(), &comm, &mv) == CA_OK) {
      std::vector<ca_task> tasks(ni > 0 ? ni : 1);
      ca_sched_tasks(items.data(), ni, docs.data(), n, tasks.data());
    }
    int N = (int)U(1, 9);
    std::vector<ca_ring_chunk> ch(2 * N * (size_t)n + 1);
    std::vector<int64_t> lens(n);
    for (auto& l : lens) l = U(0, 5000);
    ca_ring_shard(N, lens.data(), n, ch.data());
    int mt = ca_ring_kv_step_max_tasks(N, n);
    std::vector<ca_task> rt(mt > 0 ? mt : 1);
    int32_t nt = 0;
    for (int s = 0; s < N; ++s) for (int sl = 0; sl < 2; ++sl) ca_ring_kv_step_tasks(N, s, sl, lens.data(), n, rt.data(), mt, &nt);
    ca_ring_model m{N, 128, 8, 2, 16384.0, 1e15, 1e11};
    ca_ring_times t;
    ca_ring_plan(&m, U(0, 100000), U(0, 1000000), &t);
    ca_ring_select(&m, U(1, 100000), U(0, 1000000), (int)U(0, 1));
  }
  std::printf("host fuzz done\n");
  return 0;
}
