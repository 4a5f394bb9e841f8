"""50-digit brute-force attention with mpmath, for inputs of a few tokens.

Independent of the oracle: it walks every (output row, head, key) triple of
the whole K buffer, decides visibility from document positions it derives
itself, and forms the softmax with arbitrary-precision exp/log.  Used only to
pin the oracle (tests)."""

import mpmath as mp

mp.mp.dps = 50


def _val(x):
    if isinstance(x, mp.mpf):
        return x
    return mp.mpf(float(x))


def _groups(tasks):
    """Consecutive tasks naming the same query rows (q_off, o_off, q_len,
    q_pos0, q_len > 0) form one query that attends to all their contexts."""
    rows = [tuple(int(x) for x in t[:7]) for t in tasks]
    out = []
    for t in rows:
        if out and t[3] > 0 and all(out[-1][-1][c] == t[c] for c in (0, 2, 3, 5)):
            out[-1].append(t)
        else:
            out.append([t])
    return out


def attention(tasks, Q, K, V, scale):
    """Returns dict {(o_row, h): (O list of mpf, LSE mpf)}."""
    out = {}
    hq, d = Q.shape[1], Q.shape[2]
    hkv = K.shape[1]
    group = hq // hkv
    sc = mp.mpf(scale) if not isinstance(scale, mp.mpf) else scale
    for grp in _groups(tasks):
        q_off, _, o_off, q_len, _, q_pos0, _ = grp[0]
        for i in range(q_len):
            my_pos = q_pos0 + i
            for h in range(hq):
                g = h // group
                keys = []          # (K/V row, score) over every context of the query
                for (_, kv_off, _, _, kv_len, _, kv_pos0) in grp:
                    for j in range(kv_len):
                        if kv_pos0 + j > my_pos:
                            continue
                        s = mp.mpf(0)
                        for c in range(d):
                            s += _val(Q[q_off + i, h, c]) * _val(K[kv_off + j, g, c])
                        keys.append((kv_off + j, s * sc))
                if not keys:
                    out[(o_off + i, h)] = ([mp.mpf(0)] * d, -mp.inf)
                    continue
                z = mp.fsum(mp.exp(s) for _, s in keys)
                o = [mp.fsum(mp.exp(s) * _val(V[row, g, c]) for row, s in keys) / z
                     for c in range(d)]
                out[(o_off + i, h)] = (o, mp.log(z))
    return out


def loss(tasks, Q, K, V, dO, scale):
    """L = sum over covered rows of <O, dO>, in 50 digits."""
    res = attention(tasks, Q, K, V, scale)
    total = mp.mpf(0)
    for (row, h), (o, _) in res.items():
        for c, oc in enumerate(o):
            total += oc * _val(dO[row, h, c])
    return total


def loss_listed(rows_keys, Q, K, V, dO, scale):
    """L = sum_r <O_r, dO_r> in 50 digits, where O_r is the softmax attention
    of query row r over exactly the key rows listed in rows_keys[r]
    (GQA: query head h reads KV head h // (hq // hkv))."""
    hq, d = Q.shape[1], Q.shape[2]
    group = hq // K.shape[1]
    sc = mp.mpf(scale) if not isinstance(scale, mp.mpf) else scale
    total = mp.mpf(0)
    for r, keys in enumerate(rows_keys):
        if not keys:
            continue
        for h in range(hq):
            g = h // group
            s = [sc * mp.fsum(_val(Q[r, h, c]) * _val(K[k, g, c]) for c in range(d)) for k in keys]
            z = mp.fsum(mp.exp(x) for x in s)
            for c in range(d):
                oc = mp.fsum(mp.exp(x) * _val(V[k, g, c]) for x, k in zip(s, keys)) / z
                total += oc * _val(dO[r, h, c])
    return total
