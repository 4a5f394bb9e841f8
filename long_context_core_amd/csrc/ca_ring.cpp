// Host-side context-parallel ring planning: what one GPU's share of a ring
// needs from the host ("Context Parallelism for Scalable Million-Token
// Inference"):
//  * Section 3.4: the per-step time model of ring pass-KV and pass-Q, the
//    thresholds of Equations 1-3 and the switching heuristic (Algorithm 1);
//  * Appendix C: the exposed pass-KV time against the All2All that pass-Q's
//    merge needs (Algorithm 5, Equation 5);
//  * Section 3.5.1: load-balanced sharding, 2N chunks per sequence, rank i
//    holding chunks i and 2N - 1 - i;
//  * Section 3.5.2: the pass-KV ring, rank i holding the KV of rank
//    (i - s) mod N at step s, written as CA-task tables over the packed
//    sequences so one GPU can run every rank's share of a step in one launch;
//  * Section 3.6: round-robin sharding of batched decode tokens.
//
// Readings where the pages leave a step open:
//  * FLOPs = 4 T D (T + P), C in FLOP/s per rank, BW in bytes/s per rank.
//  * A ring step hides its SendRecv when its attention takes at least as
//    long; otherwise each of the N - 1 steps exposes the difference.  The
//    refined choice takes pass-Q iff the exposed pass-KV time is at least the
//    All2All time (Equation 5 is this comparison with (D + 1) / D taken as 1).
//  * A sequence of L tokens is cut into 2N chunks of ceil(L / 2N) positions;
//    chunks are clipped at L, so padded positions hold no token.
//  * At decode iteration t the token of batch entry b goes to rank
//    (b + t) mod N.
// All arithmetic is plain double in a fixed order.

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "ca_internal.h"

namespace {

ca_status check_model(const ca_ring_model* m) {
  if (!m) return ca::set_error(CA_ERR_INVALID, "ring model is NULL");
  if (m->n_ranks < 1 || m->n_heads < 1 || m->n_kv_heads < 1 || m->elem_bytes < 1)
    return ca::set_error(CA_ERR_INVALID, "n_ranks, n_heads, n_kv_heads, elem_bytes must be >= 1");
  if (!(m->d_model > 0.0) || !(m->compute > 0.0) || !(m->bandwidth > 0.0) || !std::isfinite(m->d_model) ||
      !std::isfinite(m->compute) || !std::isfinite(m->bandwidth))
    return ca::set_error(CA_ERR_INVALID, "d_model, compute and bandwidth must be finite and > 0");
  return CA_OK;
}

struct Model {
  double N, NH, NKV, e, D, C, BW;
  explicit Model(const ca_ring_model& m)
      : N(m.n_ranks), NH(m.n_heads), NKV(m.n_kv_heads), e(m.elem_bytes), D(m.d_model), C(m.compute),
        BW(m.bandwidth) {}
  double attn_step(double T, double P) const { return 4.0 * T * D * (T + P) / (N * C); }
  double sendrecv_kv(double T, double P) const { return 2.0 * (T + P) * D * e * NKV / (NH * BW); }
  double sendrecv_q(double T) const { return T * D * e / BW; }
  double all2all(double T) const { return (N - 1.0) * (D + 1.0) * T * e / BW; }
  double exposed_kv(double T, double P) const { return (N - 1.0) * (sendrecv_kv(T, P) - attn_step(T, P)); }
  double miss_threshold() const { return 2.0 * NKV / NH; }
  double t_threshold() const { return N * C * NKV * e / (2.0 * NH * BW); }
  double ctx_threshold() const { return N * e * C / (4.0 * BW); }
  double eq5_rhs(double T) const { return 2.0 * NKV / NH - 4.0 * T * BW / (N * C * e); }
};

int64_t chunk_len(int64_t L, int32_t N) { return L > 0 ? (L + 2 * (int64_t)N - 1) / (2 * (int64_t)N) : 0; }

}  // namespace

extern "C" {

ca_status ca_ring_plan(const ca_ring_model* m, int64_t T, int64_t P, ca_ring_times* out) {
  const ca_status st = check_model(m);
  if (st != CA_OK) return st;
  if (!out) return ca::set_error(CA_ERR_INVALID, "output is NULL");
  if (T < 0 || P < 0) return ca::set_error(CA_ERR_INVALID, "T=%lld and P=%lld must be >= 0", (long long)T,
                                           (long long)P);
  const Model md(*m);
  const double t = (double)T, p = (double)P;
  out->attn_step = md.attn_step(t, p);
  out->sendrecv_kv = md.sendrecv_kv(t, p);
  out->sendrecv_q = md.sendrecv_q(t);
  out->all2all = md.all2all(t);
  out->exposed_kv = md.exposed_kv(t, p);
  out->miss_threshold = md.miss_threshold();
  out->t_threshold = md.t_threshold();
  out->ctx_threshold = md.ctx_threshold();
  out->eq5_rhs = md.eq5_rhs(t);
  return CA_OK;
}

int32_t ca_ring_select(const ca_ring_model* m, int64_t T, int64_t P, int32_t refined) {
  if (check_model(m) != CA_OK) return -1;
  if (T < 1 || P < 0 || (refined != 0 && refined != 1)) {
    ca::set_error(CA_ERR_INVALID, "T >= 1, P >= 0 and refined in {0, 1} required");
    return -1;
  }
  const Model md(*m);
  const double t = (double)T, p = (double)P;
  if (t >= md.t_threshold()) return CA_RING_PASS_KV;
  if (!refined) return t / (t + p) >= md.miss_threshold() ? CA_RING_PASS_KV : CA_RING_PASS_Q;
  return md.exposed_kv(t, p) >= md.all2all(t) ? CA_RING_PASS_Q : CA_RING_PASS_KV;
}

int32_t ca_ring_select_measured(int32_t n_ranks, double sendrecv_kv, double sendrecv_q, double attn, double all2all,
                                double* exposed_kv, double* exposed_q) {
  if (n_ranks < 1 || !(sendrecv_kv >= 0.0) || !(sendrecv_q >= 0.0) || !(attn >= 0.0) || !(all2all >= 0.0)) {
    ca::set_error(CA_ERR_INVALID, "n_ranks >= 1 and non-negative times required");
    return -1;
  }
  const double steps = (double)(n_ranks - 1);
  const double k = steps * std::fmax(0.0, sendrecv_kv - attn);
  const double q = steps * std::fmax(0.0, sendrecv_q - attn) + all2all;
  if (exposed_kv) *exposed_kv = k;
  if (exposed_q) *exposed_q = q;
  return q < k ? CA_RING_PASS_Q : CA_RING_PASS_KV;
}

ca_status ca_ring_shard(int32_t n_ranks, const int64_t* lens_host, int32_t n_seqs, ca_ring_chunk* chunks_host) {
  if (n_ranks < 1 || n_seqs < 0) return ca::set_error(CA_ERR_INVALID, "n_ranks >= 1 and n_seqs >= 0 required");
  if (n_seqs > 0 && (!lens_host || !chunks_host)) return ca::set_error(CA_ERR_INVALID, "NULL pointer");
  for (int32_t s = 0; s < n_seqs; ++s)
    if (lens_host[s] < 0 || lens_host[s] > ((int64_t)1 << 40))
      return ca::set_error(CA_ERR_INVALID, "sequence %d length %lld out of range", s, (long long)lens_host[s]);
  const int32_t K = 2 * n_ranks;
  for (int32_t s = 0; s < n_seqs; ++s) {
    const int64_t L = lens_host[s], c = chunk_len(L, n_ranks);
    for (int32_t k = 0; k < K; ++k) {
      ca_ring_chunk& ch = chunks_host[(int64_t)s * K + k];
      ch.rank = k < n_ranks ? k : K - 1 - k;
      ch.seq = s;
      ch.begin = std::min((int64_t)k * c, L);
      ch.end = std::min((int64_t)(k + 1) * c, L);
    }
  }
  return CA_OK;
}

int32_t ca_ring_kv_step_max_tasks(int32_t n_ranks, int32_t n_seqs) {
  if (n_ranks < 1 || n_seqs < 0) return -1;
  const int64_t n = 2 * (int64_t)n_ranks * n_seqs;
  return n > 0x7fffffff ? -1 : (int32_t)n;
}

ca_status ca_ring_kv_step_tasks(int32_t n_ranks, int32_t step, int32_t slot, const int64_t* lens_host,
                                int32_t n_seqs, ca_task* tasks_host, int32_t max_tasks, int32_t* n_tasks) {
  if (n_ranks < 1 || n_seqs < 0 || step < 0 || step >= n_ranks || (slot != 0 && slot != 1))
    return ca::set_error(CA_ERR_INVALID, "n_ranks >= 1, n_seqs >= 0, 0 <= step < n_ranks, slot in {0, 1}");
  if (!n_tasks || (n_seqs > 0 && (!lens_host || !tasks_host))) return ca::set_error(CA_ERR_INVALID, "NULL pointer");
  for (int32_t s = 0; s < n_seqs; ++s)
    if (lens_host[s] < 0 || lens_host[s] > 0x7fffffff)
      return ca::set_error(CA_ERR_INVALID, "sequence %d length %lld out of range", s, (long long)lens_host[s]);
  const int32_t K = 2 * n_ranks;
  int32_t n = 0;
  for (int32_t r = 0; r < n_ranks; ++r) {
    const int32_t src = ((r - step) % n_ranks + n_ranks) % n_ranks;   // KV of rank (r - step) mod N
    const int32_t kv_chunk = slot == 0 ? src : K - 1 - src;
    int64_t base = 0;
    for (int32_t s = 0; s < n_seqs; ++s) {
      const int64_t L = lens_host[s], c = chunk_len(L, n_ranks);
      const int64_t kb = std::min((int64_t)kv_chunk * c, L), ke = std::min((int64_t)(kv_chunk + 1) * c, L);
      for (int32_t h = 0; h < 2; ++h) {
        const int32_t q_chunk = h == 0 ? r : K - 1 - r;
        const int64_t qb = std::min((int64_t)q_chunk * c, L), qe = std::min((int64_t)(q_chunk + 1) * c, L);
        if (qe <= qb) continue;
        if (n >= max_tasks) {
          *n_tasks = ca_ring_kv_step_max_tasks(n_ranks, n_seqs);
          return ca::set_error(CA_ERR_WORKSPACE, "more than max_tasks=%d tasks", max_tasks);
        }
        ca_task& t = tasks_host[n++];
        t.q_off = base + qb;
        t.kv_off = base + kb;
        t.o_off = base + qb;
        t.q_len = (int32_t)(qe - qb);
        t.kv_len = (int32_t)(ke - kb);
        t.q_pos0 = qb;
        t.kv_pos0 = kb;
      }
      base += L;
    }
  }
  *n_tasks = n;
  return CA_OK;
}

int32_t ca_ring_prefill_step_max_tasks(int32_t n_ranks, int32_t n_seqs) {
  return ca_ring_kv_step_max_tasks(n_ranks, n_seqs);
}

ca_status ca_ring_prefill_step_tasks(int32_t n_ranks, int32_t step, int32_t slot, const int64_t* new_lens_host,
                                     const int64_t* cached_lens_host, int32_t n_seqs, ca_task* tasks_host,
                                     int32_t max_tasks, int32_t* n_tasks) {
  if (n_ranks < 1 || n_seqs < 0 || step < 0 || step >= n_ranks || slot < 0 || slot > 3)
    return ca::set_error(CA_ERR_INVALID, "n_ranks >= 1, n_seqs >= 0, 0 <= step < n_ranks, 0 <= slot < 4");
  if (!n_tasks || (n_seqs > 0 && (!new_lens_host || !cached_lens_host || !tasks_host)))
    return ca::set_error(CA_ERR_INVALID, "NULL pointer");
  for (int32_t s = 0; s < n_seqs; ++s)
    if (new_lens_host[s] < 0 || cached_lens_host[s] < 0 || new_lens_host[s] + cached_lens_host[s] > 0x7fffffff)
      return ca::set_error(CA_ERR_INVALID, "sequence %d lengths out of range", s);
  const int32_t K = 2 * n_ranks;
  int32_t n = 0;
  for (int32_t r = 0; r < n_ranks; ++r) {
    const int32_t src = ((r - step) % n_ranks + n_ranks) % n_ranks;   // KV of rank (r - step) mod N
    const int32_t kv_chunk = (slot & 1) == 0 ? src : K - 1 - src;
    int64_t q_base = 0, kv_base = 0;
    for (int32_t s = 0; s < n_seqs; ++s) {
      const int64_t T = new_lens_host[s], P = cached_lens_host[s];
      const int64_t ct = chunk_len(T, n_ranks), cp = chunk_len(P, n_ranks);
      // slots 0, 1: the source rank's cached chunks (positions < P, visible to
      // every new query); slots 2, 3: its chunks of the new tokens (causal)
      int64_t kb, ke;
      if (slot < 2) {
        kb = std::min((int64_t)kv_chunk * cp, P);
        ke = std::min((int64_t)(kv_chunk + 1) * cp, P);
      } else {
        kb = P + std::min((int64_t)kv_chunk * ct, T);
        ke = P + std::min((int64_t)(kv_chunk + 1) * ct, T);
      }
      for (int32_t h = 0; h < 2; ++h) {
        const int32_t q_chunk = h == 0 ? r : K - 1 - r;
        const int64_t qb = std::min((int64_t)q_chunk * ct, T), qe = std::min((int64_t)(q_chunk + 1) * ct, T);
        if (qe <= qb) continue;
        if (n >= max_tasks) {
          *n_tasks = ca_ring_prefill_step_max_tasks(n_ranks, n_seqs);
          return ca::set_error(CA_ERR_WORKSPACE, "more than max_tasks=%d tasks", max_tasks);
        }
        ca_task& t = tasks_host[n++];
        t.q_off = q_base + qb;
        t.kv_off = kv_base + kb;
        t.o_off = q_base + qb;
        t.q_len = (int32_t)(qe - qb);
        t.kv_len = (int32_t)(ke - kb);
        t.q_pos0 = P + qb;
        t.kv_pos0 = kb;
      }
      q_base += T;
      kv_base += P + T;
    }
  }
  *n_tasks = n;
  return CA_OK;
}

int32_t ca_ring_decode_rank(int32_t n_ranks, int64_t iteration, int32_t seq) {
  if (n_ranks < 1 || iteration < 0 || seq < 0) {
    ca::set_error(CA_ERR_INVALID, "n_ranks >= 1, iteration >= 0 and seq >= 0 required");
    return -1;
  }
  return (int32_t)(((int64_t)seq + iteration) % n_ranks);
}

}  // extern "C"
