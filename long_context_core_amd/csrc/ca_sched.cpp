// Host-side CA-task scheduler: the profiler's cost model, the optimal shard
// size of a partial migration and the communication-aware greedy placement of
// CA-tasks on attention servers ("Efficient Long-context Language Model
// Training by Core Attention Disaggregation", Section 4.2: The Profiler and
// Cost Model; The Communication-Aware Greedy Scheduler, Steps 1-4; Appendix B,
// Optimal Shard Dimension Computation).
//
// Readings where the pages leave a step open:
//  * Items.  Documents are packed in batch order and device j owns the j-th
//    block of ceil(T / k) tokens; each maximal piece of a document on a device
//    is an Item: query range [a, b) of its document, context [0, b).
//  * Load.  An Item's load is the cost model's predicted time for
//    (n_q, n_kv) = (b - a, b).
//  * Communication.  n_q s_q + n_kv s_kv bytes, s_q = hq d 2, s_kv = hkv d 2,
//    so beta = hkv / hq as the pages state.
//  * Split.  alpha = dF / F(t) is used as the FLOPs fraction of Appendix B;
//    the real optimum (or the cheaper feasible boundary) is rounded to whole
//    tokens, the sub-Item is queries [n_kv - n_q, n_kv), the rest stays on the
//    source as up to two Items; splits shorter than min_shard are not
//    candidates.
//  * Head-tail split (head_tail set).  The shard is the first m and the last
//    m queries of the Item [a, b), [a, a + m) and [b - m, b) (Section 4.1's
//    head-tail balance of a document, applied to an Item), which hold
//    m (a + b + 1) of its (b - a)(a + b + 1) / 2 visible pairs; m is
//    alpha (b - a) / 2 rounded to nearest, clamped to [1, (b - a) / 2].  The
//    middle [a + m, b - m) stays on the source; the communication is 2 m
//    queries and the context [0, b).
//  * Order and ties.  Deficit servers once each, largest deficit first; for
//    each, the best candidate (highest E) over all Items on servers above the
//    target is migrated until the deficit is within eps * target, no
//    candidate beats e_min, or max_moves is reached.  Ties: lower source
//    server, then older Item.
// All arithmetic is plain double, evaluated in a fixed order, so the choices
// are reproducible one for one by any implementation of the same steps.

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <vector>

#include "ca_internal.h"

namespace {

struct CostModel {
  const double* q;
  const double* kv;
  const double* t;   // [nq][nkv]
  int nq, nkv;
  double fpp;
  double peak = 0.0;

  double at(int i, int j) const { return t[(size_t)i * nkv + j]; }
  // FLOPs of the block; more queries than context counts as n_kv queries
  double flops(double x, double y) const {
    const double m = std::min(x, y);
    return fpp * (m * y - m * (m - 1.0) / 2.0);
  }

  void init() {
    double best = 0.0;
    for (int i = 0; i < nq; ++i)
      for (int j = 0; j < nkv; ++j) {
        const double tp = flops(q[i], kv[j]) / at(i, j);
        if (tp > best) best = tp;
      }
    peak = best;
  }

  static int bracket(const double* axis, int n, double x) {
    int i = 0;
    while (i + 2 < n && axis[i + 1] < x) ++i;
    return i;
  }

  double interp(double x, double y) const {
    if (nq == 1 && nkv == 1) return at(0, 0);
    if (nq == 1) {
      const int j = bracket(kv, nkv, y);
      const double v = (y - kv[j]) / (kv[j + 1] - kv[j]);
      return at(0, j) * (1.0 - v) + at(0, j + 1) * v;
    }
    if (nkv == 1) {
      const int i = bracket(q, nq, x);
      const double u = (x - q[i]) / (q[i + 1] - q[i]);
      return at(i, 0) * (1.0 - u) + at(i + 1, 0) * u;
    }
    const int i = bracket(q, nq, x);
    const int j = bracket(kv, nkv, y);
    const double u = (x - q[i]) / (q[i + 1] - q[i]);
    const double v = (y - kv[j]) / (kv[j + 1] - kv[j]);
    return at(i, j) * (1.0 - u) * (1.0 - v) + at(i + 1, j) * u * (1.0 - v) + at(i, j + 1) * (1.0 - u) * v +
           at(i + 1, j + 1) * u * v;
  }

  // Predicted time: bilinear inside the grid; FLOPs / peak beyond it in both
  // coordinates (saturated); FLOPs / the throughput at the clamped point when
  // beyond it in one coordinate.
  double time(int64_t n_q, int64_t n_kv) const {
    if (n_q <= 0) return 0.0;
    const double x = (double)n_q, y = (double)n_kv;
    const bool in_q = q[0] <= x && x <= q[nq - 1];
    const bool in_kv = kv[0] <= y && y <= kv[nkv - 1];
    if (in_q && in_kv) return interp(x, y);
    if (x > q[nq - 1] && y > kv[nkv - 1]) return flops(x, y) / peak;
    const double cx = std::min(std::max(x, q[0]), q[nq - 1]);
    double cy = std::min(std::max(y, kv[0]), kv[nkv - 1]);
    if (cy < cx) cy = cx;   // keep the clamped block causal-feasible
    const double tp = flops(cx, cy) / interp(cx, cy);
    return flops(x, y) / tp;
  }
};

// Appendix B: (n_q, n_kv) with n_q (2 n_kv - n_q) = alpha L_q (2 L_kv - L_q)
// that minimises n_q + beta n_kv under 0 < n_q <= L_q,
// n_q + L_kv - L_q <= n_kv <= L_kv.
void optimal_shard(double alpha, int64_t L_q, int64_t L_kv, double beta, double* out_nq, double* out_nkv) {
  const double Lq = (double)L_q, Lkv = (double)L_kv;
  const double C = alpha * Lq * (2.0 * Lkv - Lq);
  const double lo_off = (double)(L_kv - L_q);
  const double tol = 1e-9 * std::max(1.0, Lkv);
  auto kv_of = [&](double nq) { return (C / nq + nq) / 2.0; };
  auto feasible = [&](double nq, double nkv) {
    return 0.0 < nq && nq <= Lq + tol && nq + lo_off - tol <= nkv && nkv <= Lkv + tol;
  };
  const double nq_int = std::sqrt(alpha * beta * Lq * (2.0 * Lkv - Lq) / (beta + 2.0));
  if (nq_int > 0.0 && feasible(nq_int, kv_of(nq_int))) {
    *out_nq = nq_int;
    *out_nkv = kv_of(nq_int);
    return;
  }
  bool have = false;
  double bc = 0.0, bq = 0.0, bkv = 0.0;
  auto consider = [&](double c, double nq, double nkv) {
    if (!have || c < bc || (c == bc && (nq < bq || (nq == bq && nkv < bkv)))) {
      have = true;
      bc = c;
      bq = nq;
      bkv = nkv;
    }
  };
  const double sq_end = (double)(L_kv * L_kv) - C;
  const double nq_end = Lkv - std::sqrt(std::max(sq_end, 0.0));
  if (feasible(nq_end, Lkv)) consider(nq_end + beta * Lkv, nq_end, Lkv);
  const double nq_start = -lo_off + std::sqrt(lo_off * lo_off + C);
  if (feasible(nq_start, nq_start + lo_off)) consider(nq_start + beta * (nq_start + lo_off), nq_start, nq_start + lo_off);
  if (!have) {
    *out_nq = Lq;
    *out_nkv = Lkv;
    return;
  }
  *out_nq = bq;
  *out_nkv = bkv;
}

// Half-width m of the head-tail shard of Item [a, b) holding a fraction alpha
// of its pairs: alpha (b - a) / 2 to nearest, clamped to [1, (b - a) / 2].
int64_t head_tail_shard(double alpha, int64_t a, int64_t b) {
  const int64_t half = (b - a) / 2;
  const int64_t m = (int64_t)std::floor(alpha * (double)(b - a) / 2.0 + 0.5);
  return std::min(std::max(m, (int64_t)1), half);
}

void round_shard(double nq, double nkv, int64_t L_q, int64_t L_kv, int64_t* n_q, int64_t* n_kv) {
  int64_t a = (int64_t)std::floor(nq + 0.5);
  a = std::min(std::max(a, (int64_t)1), L_q);
  int64_t b = (int64_t)std::floor(nkv + 0.5);
  b = std::min(std::max(b, a + L_kv - L_q), L_kv);
  *n_q = a;
  *n_kv = b;
}

ca_status check_grid(const double* gq, int32_t n_gq, const double* gkv, int32_t n_gkv, const double* gt,
                     double fpp) {
  if (!gq || !gkv || !gt) return ca::set_error(CA_ERR_INVALID, "NULL cost-model grid");
  if (n_gq < 1 || n_gkv < 1) return ca::set_error(CA_ERR_INVALID, "empty cost-model grid");
  for (int i = 0; i < n_gq; ++i)
    if (!(gq[i] >= 1.0) || (i > 0 && !(gq[i] > gq[i - 1])))
      return ca::set_error(CA_ERR_INVALID, "grid_q must be >= 1 and strictly increasing");
  for (int j = 0; j < n_gkv; ++j)
    if (!(gkv[j] >= 1.0) || (j > 0 && !(gkv[j] > gkv[j - 1])))
      return ca::set_error(CA_ERR_INVALID, "grid_kv must be >= 1 and strictly increasing");
  for (int64_t i = 0; i < (int64_t)n_gq * n_gkv; ++i)
    if (!(gt[i] > 0.0) || !std::isfinite(gt[i])) return ca::set_error(CA_ERR_INVALID, "grid times must be finite and > 0");
  if (!(fpp > 0.0) || !std::isfinite(fpp)) return ca::set_error(CA_ERR_INVALID, "flops_per_pair must be > 0");
  return CA_OK;
}

}  // namespace

extern "C" {

double ca_cost_time(const double* grid_q_host, int32_t n_gq, const double* grid_kv_host, int32_t n_gkv,
                    const double* grid_time_host, double flops_per_pair, int64_t n_q, int64_t n_kv) {
  if (check_grid(grid_q_host, n_gq, grid_kv_host, n_gkv, grid_time_host, flops_per_pair) != CA_OK) return NAN;
  CostModel m{grid_q_host, grid_kv_host, grid_time_host, n_gq, n_gkv, flops_per_pair};
  m.init();
  return m.time(n_q, n_kv);
}

int32_t ca_schedule_max_items(int32_t n_docs, int32_t k, int32_t max_moves) {
  if (n_docs < 0 || k < 1 || max_moves < 0) return -1;
  const int64_t n = (int64_t)n_docs + k + 2 * (int64_t)max_moves;
  return n > 0x7fffffff ? -1 : (int32_t)n;
}

ca_status ca_schedule(const ca_sched_params* p, const int64_t* doc_lens_host, int32_t n_docs,
                      const double* grid_q_host, int32_t n_gq, const double* grid_kv_host, int32_t n_gkv,
                      const double* grid_time_host, ca_sched_item* items_host, int32_t max_items,
                      int32_t* n_items, double* load_before_host, double* load_after_host, double* comm_bytes,
                      int32_t* n_moves) {
  if (!p) return ca::set_error(CA_ERR_INVALID, "params is NULL");
  if (p->k < 1) return ca::set_error(CA_ERR_INVALID, "k=%d must be >= 1", p->k);
  if (p->hq < 1 || p->hkv < 1 || p->d < 1) return ca::set_error(CA_ERR_INVALID, "hq, hkv, d must be >= 1");
  if (!(p->eps >= 0.0) || !std::isfinite(p->e_min) || p->min_shard < 1 || p->max_moves < 0)
    return ca::set_error(CA_ERR_INVALID, "eps >= 0, finite e_min, min_shard >= 1, max_moves >= 0 required");
  if (p->head_tail != 0 && p->head_tail != 1) return ca::set_error(CA_ERR_INVALID, "head_tail must be 0 or 1");
  const bool head_tail = p->head_tail == 1;
  if (n_docs < 0 || (n_docs > 0 && !doc_lens_host)) return ca::set_error(CA_ERR_INVALID, "bad document list");
  if (!items_host || !n_items || !load_before_host || !load_after_host || !comm_bytes || !n_moves)
    return ca::set_error(CA_ERR_INVALID, "NULL output pointer");
  for (int32_t i = 0; i < n_docs; ++i)
    if (doc_lens_host[i] < 0 || doc_lens_host[i] > (int64_t)1 << 40)
      return ca::set_error(CA_ERR_INVALID, "document %d length %lld out of range", i, (long long)doc_lens_host[i]);
  {
    const ca_status st = check_grid(grid_q_host, n_gq, grid_kv_host, n_gkv, grid_time_host, p->flops_per_pair);
    if (st != CA_OK) return st;
  }
  CostModel m{grid_q_host, grid_kv_host, grid_time_host, n_gq, n_gkv, p->flops_per_pair};
  m.init();
  const int k = p->k;
  const double s_q = (double)((int64_t)p->hq * p->d * 2);
  const double s_kv = (double)((int64_t)p->hkv * p->d * 2);
  const double beta = s_kv / s_q;

  // Initial items: equal token blocks of the packed batch.
  std::vector<ca_sched_item> items;
  int64_t T = 0;
  for (int32_t i = 0; i < n_docs; ++i) T += doc_lens_host[i];
  const int64_t per = T > 0 ? (T + k - 1) / k : 0;
  int64_t start = 0;
  for (int32_t doc = 0; doc < n_docs; ++doc) {
    const int64_t L = doc_lens_host[doc];
    int64_t a = 0;
    while (a < L) {
      const int64_t dev = per > 0 ? std::min((start + a) / per, (int64_t)k - 1) : 0;
      const int64_t dev_end = dev < k - 1 ? (dev + 1) * per : T;
      const int64_t b = std::min(L, dev_end - start);
      items.push_back(ca_sched_item{(int32_t)dev, doc, a, b});
      a = b;
    }
    start += L;
  }
  auto F = [&](const ca_sched_item& it) { return m.time(it.q_end - it.q_begin, it.q_end); };

  std::vector<double> load(k, 0.0);
  for (const auto& it : items) load[it.server] += F(it);
  for (int s = 0; s < k; ++s) load_before_host[s] = load[s];
  double total = 0.0;
  for (int s = 0; s < k; ++s) total += load[s];
  const double target = total / k;
  std::vector<int> order(k);
  for (int s = 0; s < k; ++s) order[s] = s;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
    const double kx = -(target - load[x]), ky = -(target - load[y]);
    return kx < ky || (kx == ky && x < y);
  });
  double comm = 0.0;
  int32_t moves = 0;
  std::vector<int> deficits;
  for (int s : order)
    if (load[s] < target) deficits.push_back(s);
  for (int dst : deficits) {
    while (moves < p->max_moves) {
      const double D = target - load[dst];
      if (D <= p->eps * target) break;
      bool have = false;
      double bE = 0.0, bV = 0.0;
      int bsrc = 0;
      size_t bidx = 0;
      bool bwhole = false;
      int64_t bnq = 0, bnkv = 0;
      for (size_t idx = 0; idx < items.size(); ++idx) {
        const ca_sched_item& it = items[idx];
        const int src = it.server;
        const double S = load[src] - target;
        if (src == dst || S <= 0.0) continue;
        const double Ft = F(it);
        if (Ft <= 0.0) continue;
        const double dF = std::min(std::min(Ft, S), D);
        const int64_t L_q = it.q_end - it.q_begin, L_kv = it.q_end;
        int64_t n_q, n_kv;
        bool whole;
        if (dF == Ft) {
          n_q = L_q;
          n_kv = L_kv;
          whole = true;
        } else if (head_tail) {
          if (L_q < 2) continue;
          const int64_t m = head_tail_shard(dF / Ft, it.q_begin, it.q_end);
          n_q = 2 * m;
          n_kv = L_kv;
          whole = (n_q == L_q);
          if (!whole && n_q < p->min_shard) continue;
        } else {
          double nq, nkv;
          optimal_shard(dF / Ft, L_q, L_kv, beta, &nq, &nkv);
          round_shard(nq, nkv, L_q, L_kv, &n_q, &n_kv);
          whole = (n_q == L_q);
          if (!whole && n_q < p->min_shard) continue;
        }
        const double V = (double)n_q * s_q + (double)n_kv * s_kv;
        const double E = dF / V;
        if (E <= p->e_min) continue;
        if (!have || E > bE || (E == bE && (src < bsrc || (src == bsrc && idx < bidx)))) {
          have = true;
          bE = E;
          bV = V;
          bsrc = src;
          bidx = idx;
          bwhole = whole;
          bnq = n_q;
          bnkv = n_kv;
        }
      }
      if (!have) break;
      ca_sched_item it = items[bidx];
      load[bsrc] -= F(it);
      if (bwhole) {
        items[bidx].server = dst;
        load[dst] += F(items[bidx]);
      } else if (head_tail) {
        const int64_t m = bnq / 2;
        items.erase(items.begin() + (ptrdiff_t)bidx);
        if (it.q_end - m > it.q_begin + m) {
          const ca_sched_item mid{bsrc, it.doc, it.q_begin + m, it.q_end - m};
          load[bsrc] += F(mid);
          items.insert(items.begin() + (ptrdiff_t)bidx, mid);
        }
        const ca_sched_item head{dst, it.doc, it.q_begin, it.q_begin + m};
        const ca_sched_item tail{dst, it.doc, it.q_end - m, it.q_end};
        items.push_back(head);
        load[dst] += F(head);
        items.push_back(tail);
        load[dst] += F(tail);
      } else {
        const int64_t sa = bnkv - bnq, sb = bnkv;
        items.erase(items.begin() + (ptrdiff_t)bidx);
        std::vector<ca_sched_item> pieces;
        if (sa > it.q_begin) pieces.push_back(ca_sched_item{bsrc, it.doc, it.q_begin, sa});
        if (it.q_end > sb) pieces.push_back(ca_sched_item{bsrc, it.doc, sb, it.q_end});
        for (const auto& pc : pieces) load[bsrc] += F(pc);
        items.insert(items.begin() + (ptrdiff_t)bidx, pieces.begin(), pieces.end());
        const ca_sched_item nw{dst, it.doc, sa, sb};
        items.push_back(nw);
        load[dst] += F(nw);
      }
      comm += bV;
      ++moves;
    }
  }
  *n_items = (int32_t)items.size();
  if ((int64_t)items.size() > (int64_t)max_items)
    return ca::set_error(CA_ERR_WORKSPACE, "%zu items do not fit in max_items=%d", items.size(), max_items);
  std::copy(items.begin(), items.end(), items_host);
  for (int s = 0; s < k; ++s) load_after_host[s] = load[s];
  *comm_bytes = comm;
  *n_moves = moves;
  return CA_OK;
}

ca_status ca_sched_tasks(const ca_sched_item* items_host, int32_t n_items, const int64_t* doc_lens_host,
                         int32_t n_docs, ca_task* tasks_host) {
  if (n_items < 0 || n_docs < 0) return ca::set_error(CA_ERR_INVALID, "negative count");
  if (n_items > 0 && (!items_host || !tasks_host || !doc_lens_host))
    return ca::set_error(CA_ERR_INVALID, "NULL pointer");
  std::vector<int64_t> starts((size_t)n_docs + 1, 0);
  for (int32_t i = 0; i < n_docs; ++i) starts[i + 1] = starts[i] + doc_lens_host[i];
  for (int32_t i = 0; i < n_items; ++i) {
    const ca_sched_item& it = items_host[i];
    if (it.doc < 0 || it.doc >= n_docs || it.q_begin < 0 || it.q_begin >= it.q_end ||
        it.q_end > doc_lens_host[it.doc] || it.q_end > 0x7fffffff)
      return ca::set_error(CA_ERR_INVALID, "item %d out of range", i);
    const int64_t base = starts[it.doc];
    ca_task t;
    t.q_off = base + it.q_begin;
    t.kv_off = base;
    t.o_off = base + it.q_begin;
    t.q_len = (int32_t)(it.q_end - it.q_begin);
    t.kv_len = (int32_t)it.q_end;
    t.q_pos0 = it.q_begin;
    t.kv_pos0 = 0;
    tasks_host[i] = t;
  }
  return CA_OK;
}

}  // extern "C"
