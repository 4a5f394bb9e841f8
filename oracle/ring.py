"""Context-parallel ring planning as the oracle states it — TEST INFRASTRUCTURE
ONLY.

"Context Parallelism for Scalable Million-Token Inference":

* Section 3.4 (analytical model): per-step attention and SendRecv times of
  ring pass-KV and pass-Q, Equation 1 (the miss-rate threshold 2 N_KV / N_H),
  Equation 2 (the new-token threshold that hides pass-KV), Equation 3 (the
  context threshold that hides pass-Q) and the switching heuristic
  (Algorithm 1);
* Appendix C: the exposed pass-KV time against the All2All of pass-Q's merge
  (Algorithm 5, Equation 5);
* Section 3.5.1: load-balanced sharding (2N chunks, rank i holds chunks i and
  2N - 1 - i, each sequence padded to a multiple of 2N);
* Section 3.5.2: the pass-KV ring (rank i meets the KV of rank (i - s) mod N
  at step s);
* Section 3.6: round-robin sharding of batched decode tokens (the offset
  moves by one each decode iteration).

Readings where the pages leave a step open:
* Units.  FLOPs = 4 T D (T + P) with D the model dimension, C in FLOP/s per
  rank, BW in bytes/s per rank, e bytes per element; times in seconds.
* Exposed time.  A ring step hides its SendRecv when the step's attention
  takes at least as long; otherwise (N - 1) steps each expose the difference.
  The refined choice takes pass-Q iff the exposed pass-KV time is at least
  the All2All time; Equation 5 is the same comparison with (D + 1) / D taken
  as 1, and the oracle keeps both.
* Padding.  A sequence of L tokens is cut into 2N chunks of c = ceil(L / 2N)
  positions; chunk k covers [min(k c, L), min((k + 1) c, L)), so padded
  positions hold no token.
* Round robin.  At decode iteration t the token of batch entry b goes to rank
  (b + t) mod N.
* The empirical classifier of Appendix D is not restated: with the printed
  coefficients it does not separate the printed Table 4 points under a
  natural, base-2 or base-10 logarithm.
"""

import math

PASS_KV = 0
PASS_Q = 1


class RingModel:
    """N ranks, N_H query heads, N_KV key/value heads, e bytes per element,
    D model dimension, C attention FLOP/s per rank, BW SendRecv bytes/s per
    rank."""

    def __init__(self, n_ranks, n_heads, n_kv_heads, elem_bytes, d_model, compute, bandwidth):
        self.N = int(n_ranks)
        self.NH = int(n_heads)
        self.NKV = int(n_kv_heads)
        self.e = float(elem_bytes)
        self.D = float(d_model)
        self.C = float(compute)
        self.BW = float(bandwidth)

    # Section 3.4: one ring step on one rank.
    def attn_step(self, T, P):
        """T / N queries against (T + P) / N keys: 4 T D (T + P) / (N C)."""
        return 4.0 * T * self.D * (T + P) / (self.N * self.C)

    def sendrecv_kv(self, T, P):
        """K and V of (T + P) tokens at N_KV / N_H of the query width."""
        return 2.0 * (T + P) * self.D * self.e * self.NKV / (self.NH * self.BW)

    def sendrecv_q(self, T, P):
        return T * self.D * self.e / self.BW

    def all2all(self, T):
        """Appendix C: partial outputs and their LSE, (D + 1) values per token."""
        return (self.N - 1) * (self.D + 1.0) * T * self.e / self.BW

    def exposed_kv(self, T, P):
        """Appendix C, as printed: (N - 1) (SendRecv_KV - ATTN), possibly negative."""
        return (self.N - 1) * (self.sendrecv_kv(T, P) - self.attn_step(T, P))

    # Thresholds.
    def miss_threshold(self):
        """Equation 1: pass-KV sends fewer bytes iff T / (T + P) >= 2 N_KV / N_H."""
        return 2.0 * self.NKV / self.NH

    def t_threshold(self):
        """Equation 2: pass-KV is hidden iff T >= N C N_KV e / (2 N_H BW)."""
        return self.N * self.C * self.NKV * self.e / (2.0 * self.NH * self.BW)

    def ctx_threshold(self):
        """Equation 3: pass-Q is hidden iff T + P >= N e C / (4 BW)."""
        return self.N * self.e * self.C / (4.0 * self.BW)

    def eq5_rhs(self, T):
        """Equation 5: pass-Q iff T / (T + P) <= 2 N_KV / N_H - 4 T BW / (N C e)."""
        return 2.0 * self.NKV / self.NH - 4.0 * T * self.BW / (self.N * self.C * self.e)


def select_simple(m, T, P):
    """Algorithm 1: pass-KV if T reaches the Equation 2 threshold or the miss
    rate reaches the Equation 1 threshold, else pass-Q."""
    if T >= m.t_threshold() or T / float(T + P) >= m.miss_threshold():
        return PASS_KV
    return PASS_Q


def select_refined(m, T, P):
    """Algorithm 5: pass-KV when its communication is hidden; otherwise pass-Q
    iff the exposed pass-KV time is at least the All2All time."""
    if T >= m.t_threshold():
        return PASS_KV
    return PASS_Q if m.exposed_kv(T, P) >= m.all2all(T) else PASS_KV


def select_eq5(m, T, P):
    """Algorithm 5 with the closed form of Equation 5."""
    if T >= m.t_threshold():
        return PASS_KV
    return PASS_Q if T / float(T + P) <= m.eq5_rhs(T) else PASS_KV


def select_measured(n_ranks, sendrecv_kv, sendrecv_q, attn, all2all):
    """The comparison of Table 5 on measured per-step times: each ring exposes
    (N - 1) max(0, SendRecv - ATTN); pass-Q adds its All2All.  Returns
    (choice, exposed pass-KV, exposed pass-Q); ties go to pass-KV."""
    k = (n_ranks - 1) * max(0.0, sendrecv_kv - attn)
    q = (n_ranks - 1) * max(0.0, sendrecv_q - attn) + all2all
    return (PASS_Q if q < k else PASS_KV), k, q


# Section 3.5.1: load-balanced sharding.
def chunk_len(L, N):
    return -(-int(L) // (2 * int(N))) if L > 0 else 0


def shard(lens, N):
    """[(rank, seq, begin, end)] for every sequence and chunk k = 0 .. 2N-1,
    in (seq, k) order; rank i holds chunks i and 2N - 1 - i."""
    out = []
    for s, L in enumerate(lens):
        c = chunk_len(L, N)
        for k in range(2 * N):
            rank = k if k < N else 2 * N - 1 - k
            out.append((rank, s, min(k * c, L), min((k + 1) * c, L)))
    return out


def kv_step_source(rank, step, N):
    """Section 3.5.2: at step s rank i holds the KV of rank (i - s) mod N."""
    return (rank - step) % N


def decode_rank(seq, iteration, N):
    """Section 3.6: round-robin owner of a batch entry's decode token."""
    return (seq + iteration) % N


def causal_pairs(begin, end):
    """Visible (query, key) pairs of queries [begin, end) of one causal
    sequence, keys from position 0: sum over p of (p + 1)."""
    return (end - begin) * (begin + end + 1) // 2 if end > begin else 0


def rank_pairs(lens, N):
    """Causal pairs each rank's query chunks hold, summed over sequences."""
    load = [0] * N
    for rank, s, b, e in shard(lens, N):
        load[rank] += causal_pairs(b, e)
    return load
