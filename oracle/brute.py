"""Pure-Python brute force for tiny grouped-query attention cases.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Uses nothing but the
``math`` module and nested lists, so that it shares no code path with the C
oracle or with numpy/torch.  It follows the same definition, written out
independently:

* group size G = h_q / h_kv, query head h uses key/value head h // G
  ("Modern LLM architecture (1): GQA and RMSNorm", §2.3;
  "Attention in Qwen, DeepSeek and LLaMA3", §2.2);
* weights w_j = exp(s_j) / sum_t exp(s_t) with s_j = scale * <q, k_j> over the
  visible keys ("Modern LLM architecture (1)", §2.1);
* output = sum_j w_j v_j.

Inputs are nested lists (or anything indexable the same way); outputs are
nested lists of floats.
"""
import math


def _softmax_average(q, keys, values, scale):
    """sum_j softmax_j(scale * <q, k_j>) * v_j over the given keys; [] keys -> zeros."""
    d_v = len(values[0]) if values else len(q)
    if not keys:
        return [0.0] * d_v, []
    scores = [scale * math.fsum(qc * kc for qc, kc in zip(q, key)) for key in keys]
    top = max(scores)
    expd = [math.exp(s - top) for s in scores]
    total = math.fsum(expd)
    weights = [e / total for e in expd]
    out = [math.fsum(w * val[c] for w, val in zip(weights, values)) for c in range(d_v)]
    return out, weights


def prefill(q, k, v, causal, scale):
    """q [B][L][h_q][d], k/v [B][L][h_kv][d] -> (o [B][L][h_q][d], probs [B][h_q][L][L])."""
    B, L, h_q = len(q), len(q[0]), len(q[0][0])
    h_kv = len(k[0][0])
    if h_q % h_kv:
        raise ValueError("h_q must be a multiple of h_kv")
    G = h_q // h_kv
    o = [[[None] * h_q for _ in range(L)] for _ in range(B)]
    probs = [[[[0.0] * L for _ in range(L)] for _ in range(h_q)] for _ in range(B)]
    for b in range(B):
        for h in range(h_q):
            g = h // G
            for i in range(L):
                last = i + 1 if causal else L
                keys = [k[b][j][g] for j in range(last)]
                vals = [v[b][j][g] for j in range(last)]
                out, w = _softmax_average(q[b][i][h], keys, vals, scale)
                o[b][i][h] = out
                for j, wj in enumerate(w):
                    probs[b][h][i][j] = wj
    return o, probs


def prefill_cached(q, k, v, causal, scale):
    """q [B][Lq][h_q][d], k/v [B][Lk][h_kv][d] -> o [B][Lq][h_q][d]; query row i is
    position Lk - Lq + i (the Lq newest of Lk positions)."""
    B, Lq, h_q = len(q), len(q[0]), len(q[0][0])
    Lk, h_kv = len(k[0]), len(k[0][0])
    if h_q % h_kv or Lq > Lk:
        raise ValueError("need h_q a multiple of h_kv and Lq <= Lk")
    G = h_q // h_kv
    o = [[[None] * h_q for _ in range(Lq)] for _ in range(B)]
    for b in range(B):
        for h in range(h_q):
            g = h // G
            for i in range(Lq):
                pos = Lk - Lq + i
                last = pos + 1 if causal else Lk
                out, _ = _softmax_average(q[b][i][h], [k[b][j][g] for j in range(last)],
                                          [v[b][j][g] for j in range(last)], scale)
                o[b][i][h] = out
    return o


def decode(q, k_cache, v_cache, seqlens):
    """q [B][h_q][d], caches [B][h_kv][S][d], seqlens [B] -> o [B][h_q][d]."""
    B, h_q, d = len(q), len(q[0]), len(q[0][0])
    h_kv = len(k_cache[0])
    G = h_q // h_kv
    scale = 1.0 / math.sqrt(d)
    o = []
    for b in range(B):
        n = int(seqlens[b])
        row = []
        for h in range(h_q):
            g = h // G
            out, _ = _softmax_average(q[b][h], [k_cache[b][g][j] for j in range(n)],
                                      [v_cache[b][g][j] for j in range(n)], scale)
            row.append(out)
        o.append(row)
    return o


def rope(x, cos, sin):
    """x [B][L][H][d], cos/sin [L][d/2] -> rotated copy: for pair i at position p,
    out[i] = x[2i] cos - x[2i+1] sin and out[d/2 + i] = x[2i] sin + x[2i+1] cos
    ("Attention in Qwen, DeepSeek and LLaMA3", §1)."""
    out = []
    for xb in x:
        ob = []
        for p, xp in enumerate(xb):
            op = []
            for vec in xp:
                half = len(vec) // 2
                first = [vec[2 * i] * cos[p][i] - vec[2 * i + 1] * sin[p][i] for i in range(half)]
                second = [vec[2 * i] * sin[p][i] + vec[2 * i + 1] * cos[p][i] for i in range(half)]
                op.append(first + second)
            ob.append(op)
        out.append(ob)
    return out


def prefill_mask(q, k, v, mask, causal, scale):
    """q [B][Lq][h_q][d], k/v [B][Lk][h_kv][d], mask [B][Lq][Lk] -> o [B][Lq][h_q][d].

    Key j is visible to query row i of sequence b iff mask[b][i][j] is nonzero
    and, when causal, j <= Lk - Lq + i (the pages' masked_fill(mask == 0,
    -inf) convention, "Implementing GQA from scratch in PyTorch", §3.3); a row
    with no visible key is zeros."""
    B, Lq, h_q = len(q), len(q[0]), len(q[0][0])
    Lk, h_kv = len(k[0]), len(k[0][0])
    if h_q % h_kv or Lq > Lk:
        raise ValueError("need h_q a multiple of h_kv and Lq <= Lk")
    G = h_q // h_kv
    o = [[[None] * h_q for _ in range(Lq)] for _ in range(B)]
    for b in range(B):
        for i in range(Lq):
            seen = [j for j in range(Lk)
                    if mask[b][i][j] and (not causal or j <= Lk - Lq + i)]
            for h in range(h_q):
                g = h // G
                out, _ = _softmax_average(q[b][i][h], [k[b][j][g] for j in seen],
                                          [v[b][j][g] for j in seen], scale)
                o[b][i][h] = out
    return o
