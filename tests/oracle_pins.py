"""Pins that tie the fp64 oracle to what the pages and the mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
something other than itself: a hand-derived closed form stored under
``tests/golden/`` (with its citation), a library routine that the method
reduces to in a special case (torch's fp64 scaled_dot_product_attention for
MHA, MQA and its enable_gqa form), an invariant of softmax attention, or the
independent pure-Python brute force.

``test_oracle_pins.py`` runs every pin under pytest.  ``test_oracle_mutants.py``
runs this file as a script against deliberately broken copies of the C oracle
(``python tests/oracle_pins.py <path/to/lib.so>``) and expects a failure for
each, which shows the pins catch plausible mistakes.
"""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np
import torch
import torch.nn.functional as F

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from oracle import brute  # noqa: E402

GOLDEN = os.path.join(HERE, "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed, std=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * std


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol:.1e}"


def _sdpa(q, k, v, causal, scale, enable_gqa=False):
    """torch fp64 SDPA on [B, L, H, d] tensors (test-only library routine)."""
    tq = torch.from_numpy(np.ascontiguousarray(q)).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.ascontiguousarray(k)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(np.ascontiguousarray(v)).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale,
                                       enable_gqa=enable_gqa)
    return o.permute(0, 2, 1, 3).contiguous().numpy()


# ---------------------------------------------------------------- golden pins

def pin_hand_2x2():
    g = _golden("hand_2x2.json")
    q, k, v = (np.array(g[n]) for n in ("q", "k", "v"))
    tol = g["tolerance"]
    o, p = oracle.prefill(q, k, v, causal=False, scale=g["scale"], return_probs=True)
    _close(o, g["expected_noncausal"], tol, "hand 2x2 non-causal")
    _close(p, g["expected_probs_noncausal"], tol, "hand 2x2 probabilities")
    o = oracle.prefill(q, k, v, causal=True, scale=g["scale"])
    _close(o, g["expected_causal"], tol, "hand 2x2 causal")
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0]), "causal row 0 must equal V[0] exactly"
    for causal, key in ((False, "expected_noncausal"), (True, "expected_causal")):
        ob, _ = brute.prefill(g["q"], g["k"], g["v"], causal, g["scale"])
        _close(ob, g[key], tol, f"brute force hand 2x2 causal={causal}")


def _head_map_tensors(g):
    L = len(g["k_per_kv_head"][0])
    h_q = len(g["q_per_head"])
    q = np.array([[g["q_per_head"] for _ in range(L)]])  # [1, L, h_q, d]
    k = np.array([np.array(g["k_per_kv_head"]).transpose(1, 0, 2)])  # [1, L, h_kv, d]
    v = np.array([np.array(g["v_per_kv_head"]).transpose(1, 0, 2)])
    return q, k, v, L, h_q


def pin_head_map():
    g = _golden("head_map_4q2kv.json")
    q, k, v, L, h_q = _head_map_tensors(g)
    tol = g["tolerance"]
    o = oracle.prefill(q, k, v, causal=False, scale=g["scale"])
    for i in range(L):
        _close(o[0, i], g["expected_noncausal_per_head"], tol, f"head map non-causal row {i}")
    o = oracle.prefill(q, k, v, causal=True, scale=g["scale"])
    exp = np.array(g["expected_causal_per_head_per_row"]).transpose(1, 0, 2)  # [L, h_q, d]
    _close(o[0], exp, tol, "head map causal")
    ob, _ = brute.prefill(q.tolist(), k.tolist(), v.tolist(), True, g["scale"])
    _close(np.array(ob)[0], exp, tol, "brute force head map causal")


def pin_decode_golden():
    g = _golden("decode_cache_3seq.json")
    B = len(g["seqlens"])
    kc = np.array([[g["k_rows"]] for _ in range(B)])  # [B, 1, S, d]
    vc = np.array([[g["v_rows"]] for _ in range(B)])
    q = np.array(g["q"])
    o = oracle.decode(q, kc, vc, g["seqlens"])
    _close(o, g["expected"], g["tolerance"], "decode golden")
    ob = brute.decode(g["q"], kc.tolist(), vc.tolist(), g["seqlens"])
    _close(ob, g["expected"], g["tolerance"], "brute force decode golden")


# ------------------------------------------------------- library reductions

def pin_mha_reduction():
    """h_kv == h_q: per-head softmax attention == torch fp64 SDPA."""
    B, L, H, d = 2, 9, 3, 8
    q, k, v = _rand((B, L, H, d), 1), _rand((B, L, H, d), 2), _rand((B, L, H, d), 3)
    for causal in (False, True):
        o = oracle.prefill(q, k, v, causal=causal, scale=0.3)
        _close(o, _sdpa(q, k, v, causal, 0.3), 1e-12, f"MHA vs SDPA causal={causal}")


def pin_mqa_reduction():
    """h_kv == 1: equals attention against one key/value head broadcast with expand."""
    B, L, H, d = 2, 7, 4, 6
    q, k, v = _rand((B, L, H, d), 4), _rand((B, L, 1, d), 5), _rand((B, L, 1, d), 6)
    kx, vx = np.broadcast_to(k, (B, L, H, d)), np.broadcast_to(v, (B, L, H, d))
    for causal in (False, True):
        o = oracle.prefill(q, k, v, causal=causal, scale=1 / math.sqrt(d))
        _close(o, _sdpa(q, kx, vx, causal, 1 / math.sqrt(d)), 1e-12,
               f"MQA vs expanded SDPA causal={causal}")


def pin_gqa_library():
    """General group sizes against torch's own grouped form (enable_gqa) and the brute force."""
    for (B, L, h_q, h_kv, d, seed) in ((2, 11, 6, 2, 5, 7), (1, 13, 8, 4, 4, 8),
                                       (2, 5, 6, 3, 3, 9)):
        q = _rand((B, L, h_q, d), seed)
        k = _rand((B, L, h_kv, d), seed + 1)
        v = _rand((B, L, h_kv, d), seed + 2)
        for causal in (False, True):
            o = oracle.prefill(q, k, v, causal=causal, scale=0.4)
            ref = _sdpa(q, k, v, causal, 0.4, enable_gqa=True)
            _close(o, ref, 1e-12, f"GQA {h_q}/{h_kv} vs SDPA enable_gqa causal={causal}")
    q, k, v = _rand((1, 4, 4, 3), 20), _rand((1, 4, 2, 3), 21), _rand((1, 4, 2, 3), 22)
    ob, _ = brute.prefill(q.tolist(), k.tolist(), v.tolist(), True, 0.7)
    _close(oracle.prefill(q, k, v, causal=True, scale=0.7), ob, 1e-12, "C oracle vs brute force")


# ------------------------------------------------------------------ properties

def pin_rows_sum_to_one():
    q, k, v = _rand((2, 10, 4, 6), 30), _rand((2, 10, 2, 6), 31), _rand((2, 10, 2, 6), 32)
    for causal in (False, True):
        _, p = oracle.prefill(q, k, v, causal=causal, scale=0.5, return_probs=True)
        _close(p.sum(-1), np.ones(p.shape[:-1]), 1e-14, f"softmax rows sum to 1 causal={causal}")
        assert (p >= 0).all()
        if causal:
            L = p.shape[-1]
            assert np.all(p[..., np.triu_indices(L, 1)[0], np.triu_indices(L, 1)[1]] == 0.0), \
                "masked probabilities must be exactly zero"


def pin_k_zero_mean():
    """K == 0: every visible key has weight 1/n, output = mean of the visible V rows."""
    B, L, h_q, h_kv, d = 2, 8, 4, 2, 5
    q, v = _rand((B, L, h_q, d), 40), _rand((B, L, h_kv, d), 41)
    k = np.zeros((B, L, h_kv, d))
    G = h_q // h_kv
    o = oracle.prefill(q, k, v, causal=False, scale=0.9)
    for h in range(h_q):
        _close(o[:, :, h], np.broadcast_to(v[:, :, h // G].mean(1, keepdims=True), (B, L, d)),
               1e-12, "K=0 non-causal mean")
    o = oracle.prefill(q, k, v, causal=True, scale=0.9)
    for h in range(h_q):
        cum = np.cumsum(v[:, :, h // G], axis=1) / np.arange(1, L + 1)[None, :, None]
        _close(o[:, :, h], cum, 1e-12, "K=0 causal running mean")
    S = 12
    kc, vc = np.zeros((B, h_kv, S, d)), _rand((B, h_kv, S, d), 42)
    lens = [5, 12]
    od = oracle.decode(q[:, 0], kc, vc, lens)
    for b in range(B):
        for h in range(h_q):
            _close(od[b, h], vc[b, h // G, :lens[b]].mean(0), 1e-12, "K=0 decode mean")


def pin_causal_row0():
    B, L, h_q, h_kv, d = 3, 6, 8, 2, 7
    q, k, v = _rand((B, L, h_q, d), 50), _rand((B, L, h_kv, d), 51), _rand((B, L, h_kv, d), 52)
    o = oracle.prefill(q, k, v, causal=True, scale=0.125)
    for h in range(h_q):
        assert np.array_equal(o[:, 0, h], v[:, 0, h // (h_q // h_kv)]), "causal row 0 != V[0]"


def pin_identical_heads():
    B, L, h_q, h_kv, d = 2, 9, 8, 2, 4
    G = h_q // h_kv
    qg = _rand((B, L, h_kv, 1, d), 60)
    q = np.repeat(qg, G, axis=3).reshape(B, L, h_q, d)
    k, v = _rand((B, L, h_kv, d), 61), _rand((B, L, h_kv, d), 62)
    for causal in (False, True):
        o = oracle.prefill(q, k, v, causal=causal, scale=0.3)
        for h in range(h_q):
            assert np.array_equal(o[:, :, h], o[:, :, (h // G) * G]), "heads of a group differ"
        # heads of different groups differ (the key/value heads differ)
        assert not np.allclose(o[:, :, 0], o[:, :, G])


def pin_invariances():
    B, L, h_q, h_kv, d = 2, 10, 6, 3, 5
    q, k, v = _rand((B, L, h_q, d), 70), _rand((B, L, h_kv, d), 71), _rand((B, L, h_kv, d), 72)
    for causal in (False, True):
        base = oracle.prefill(q, k, v, causal=causal, scale=0.4)
        u = _rand((d,), 73)
        _close(oracle.prefill(q, k + u, v, causal=causal, scale=0.4), base, 1e-11,
               f"key shift invariance causal={causal}")
        _close(oracle.prefill(3.0 * q, k, v, causal=causal, scale=0.4 / 3.0), base, 1e-11,
               f"q scaling invariance causal={causal}")
        c = np.full_like(v, 2.5)
        _close(oracle.prefill(q, k, c, causal=causal, scale=0.4), np.full_like(q, 2.5), 1e-12,
               "constant V rows")
    perm = np.random.default_rng(74).permutation(L)
    base = oracle.prefill(q, k, v, causal=False, scale=0.4)
    _close(oracle.prefill(q, k[:, perm], v[:, perm], causal=False, scale=0.4), base, 1e-12,
           "key/value permutation invariance")
    S = 9
    kc, vc = _rand((B, h_kv, S, d), 75), _rand((B, h_kv, S, d), 76)
    lens = [9, 6]
    od = oracle.decode(q[:, 0], kc, vc, lens)
    kp, vp = kc.copy(), vc.copy()
    for b in range(B):
        p = np.random.default_rng(77 + b).permutation(lens[b])
        kp[b, :, :lens[b]] = kc[b][:, p]
        vp[b, :, :lens[b]] = vc[b][:, p]
    _close(oracle.decode(q[:, 0], kp, vp, lens), od, 1e-12, "decode permutation invariance")


def pin_cross_path():
    """decode of the last position == row L-1 of causal prefill over the same keys."""
    B, L, h_q, h_kv, d = 2, 12, 8, 2, 6
    q, k, v = _rand((B, L, h_q, d), 80), _rand((B, L, h_kv, d), 81), _rand((B, L, h_kv, d), 82)
    o = oracle.prefill(q, k, v, causal=True, scale=1 / math.sqrt(d))
    kc = np.ascontiguousarray(k.transpose(0, 2, 1, 3))
    vc = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    od = oracle.decode(q[:, L - 1], kc, vc, [L] * B)
    _close(od, o[:, L - 1], 1e-12, "decode vs last causal prefill row")
    od = oracle.decode(q[:, 4], kc, vc, [5] * B)
    _close(od, o[:, 4], 1e-12, "decode with seqlen 5 vs causal prefill row 4")


def pin_rows_match_full():
    B, L, h_q, h_kv, d = 2, 7, 4, 2, 3
    q, k, v = _rand((B, L, h_q, d), 90), _rand((B, L, h_kv, d), 91), _rand((B, L, h_kv, d), 92)
    full = oracle.prefill(q, k, v, causal=True, scale=0.6)
    rows = [(1, 6, 3), (1, 0, 3), (0, 2, 1), (0, 5, 1), (1, 3, 0)]
    qr = np.array([q[b, i, h] for b, i, h in rows])
    out = oracle.prefill_rows(qr, rows, k, v, h_q, causal=True, scale=0.6)
    _close(out, np.array([full[b, i, h] for b, i, h in rows]), 0.0, "rows entry vs full entry")


def pin_decode_tail_ignored():
    B, h_q, h_kv, S, d = 3, 4, 2, 8, 4
    q = _rand((B, h_q, d), 100)
    kc, vc = _rand((B, h_kv, S, d), 101), _rand((B, h_kv, S, d), 102)
    lens = [3, 8, 0]
    base = oracle.decode(q, kc, vc, lens)
    kp, vp = kc.copy(), vc.copy()
    for b in range(B):
        kp[b, :, lens[b]:] = np.nan
        vp[b, :, lens[b]:] = np.nan
    o = oracle.decode(q, kp, vp, lens)
    assert np.array_equal(o, base), "rows beyond seqlens leaked into the output"
    assert np.array_equal(o[2], np.zeros((h_q, d))), "seqlen 0 must give zeros"


def pin_argument_errors():
    q, k = np.zeros((1, 2, 3, 4)), np.zeros((1, 2, 2, 4))
    try:
        oracle.prefill(q, k, k, causal=False, scale=1.0)
    except ValueError:
        pass
    else:
        raise AssertionError("h_q % h_kv != 0 must be rejected")


# ------------------------------------------------- prefill against cached keys

def pin_chunk_golden():
    """Hand-derived 2-of-3 case: bottom-right causal alignment, closed forms."""
    g = _golden("chunk_2_of_3.json")
    q, k, v = np.array(g["q"]), np.array(g["k"]), np.array(g["v"])
    for causal, key in ((True, "expected_causal"), (False, "expected_noncausal")):
        _close(oracle.prefill_cached(q, k, v, causal, g["scale"]), g[key], g["tolerance"],
               f"chunk golden causal={causal}")
        _close(brute.prefill_cached(q.tolist(), k.tolist(), v.tolist(), causal, g["scale"]),
               g[key], g["tolerance"], f"brute chunk golden causal={causal}")


def pin_chunked_equals_full():
    """Chunk by chunk against the growing key set == one full prefill, row for row."""
    B, L, h_q, h_kv, d = 2, 37, 4, 2, 8
    q, k, v = _rand((B, L, h_q, d), 110), _rand((B, L, h_kv, d), 111), _rand((B, L, h_kv, d), 112)
    scale = 1 / math.sqrt(d)
    full = oracle.prefill(q, k, v, causal=True, scale=scale)
    for c0, c1 in ((0, 10), (10, 11), (11, 30), (30, 37)):
        part = oracle.prefill_cached(q[:, c0:c1], k[:, :c1], v[:, :c1], True, scale)
        _close(part, full[:, c0:c1], 1e-13, f"causal chunk [{c0},{c1}) vs full prefill")
    full_nc = oracle.prefill(q, k, v, causal=False, scale=scale)
    part = oracle.prefill_cached(q[:, 5:9], k, v, False, scale)
    _close(part, full_nc[:, 5:9], 1e-13, "non-causal rows against all keys vs full prefill")


def pin_chunk_single_query_is_decode():
    """One new query against n keys == decode over a cache of n rows."""
    B, n, h_q, h_kv, d = 3, 9, 8, 2, 16
    q, k, v = _rand((B, 1, h_q, d), 120), _rand((B, n, h_kv, d), 121), _rand((B, n, h_kv, d), 122)
    o = oracle.prefill_cached(q, k, v, True, 1 / math.sqrt(d))
    kc = np.ascontiguousarray(k.transpose(0, 2, 1, 3))
    vc = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    _close(o[:, 0], oracle.decode(q[:, 0], kc, vc, [n] * B), 1e-13, "L_q = 1 vs decode")


def pin_chunk_brute_and_library():
    """Random tiny shapes: the brute force, and fp64 SDPA with a bottom-right mask."""
    B, Lq, Lk, h_q, h_kv, d = 2, 3, 7, 4, 2, 5
    q, k, v = _rand((B, Lq, h_q, d), 130), _rand((B, Lk, h_kv, d), 131), _rand((B, Lk, h_kv, d), 132)
    for causal in (True, False):
        o = oracle.prefill_cached(q, k, v, causal, 0.4)
        _close(o, brute.prefill_cached(q.tolist(), k.tolist(), v.tolist(), causal, 0.4), 1e-12,
               f"chunk vs brute causal={causal}")
        mask = None
        if causal:  # key j visible to row i iff j <= Lk - Lq + i
            mask = torch.tensor([[j <= Lk - Lq + i for j in range(Lk)] for i in range(Lq)])
        tq = torch.from_numpy(q).permute(0, 2, 1, 3)
        tk = torch.from_numpy(k).permute(0, 2, 1, 3)
        tv = torch.from_numpy(v).permute(0, 2, 1, 3)
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.4,
                                             enable_gqa=True).permute(0, 2, 1, 3).numpy()
        _close(o, ref, 1e-12, f"chunk vs SDPA causal={causal}")


def pin_chunk_rows_match_full():
    B, Lq, Lk, h_q, h_kv, d = 2, 5, 11, 4, 1, 3
    q, k, v = _rand((B, Lq, h_q, d), 140), _rand((B, Lk, h_kv, d), 141), _rand((B, Lk, h_kv, d), 142)
    full = oracle.prefill_cached(q, k, v, True, 0.7)
    rows = [(1, 4, 3), (0, 0, 0), (1, 2, 1)]
    qr = np.array([q[b, i, h] for b, i, h in rows])
    out = oracle.prefill_cached_rows(qr, rows, k, v, h_q, Lq, True, 0.7)
    _close(out, np.array([full[b, i, h] for b, i, h in rows]), 0.0, "chunk rows vs full")


# ----------------------------------------------------------- decode with append

def pin_append_cross_path():
    """Appending token n to a cache of n rows and decoding == causal prefill row n,
    and the grown cache holds rows 0..n exactly."""
    B, n, h_q, h_kv, d, S = 2, 11, 8, 2, 16, 20
    q, k, v = (_rand((B, n + 1, h_q, d), 150), _rand((B, n + 1, h_kv, d), 151),
               _rand((B, n + 1, h_kv, d), 152))
    full = oracle.prefill(q, k, v, causal=True, scale=1 / math.sqrt(d))
    kc = np.zeros((B, h_kv, S, d))
    vc = np.zeros((B, h_kv, S, d))
    kc[:, :, :n] = k[:, :n].transpose(0, 2, 1, 3)
    vc[:, :, :n] = v[:, :n].transpose(0, 2, 1, 3)
    o, kc2, vc2 = oracle.decode_append(q[:, n], k[:, n], v[:, n], kc, vc, [n] * B)
    _close(o, full[:, n], 1e-12, "append + decode vs causal prefill row n")
    assert np.array_equal(kc2[:, :, :n + 1], k[:, :n + 1].transpose(0, 2, 1, 3))
    assert np.array_equal(vc2[:, :, :n + 1], v[:, :n + 1].transpose(0, 2, 1, 3))
    assert np.array_equal(kc2[:, :, n + 1:], kc[:, :, n + 1:]), "rows past the append changed"


def pin_append_to_empty_cache():
    """With nothing cached the token attends only to itself: o = v_new of its group, exactly."""
    B, h_q, h_kv, d, S = 3, 6, 2, 8, 5
    q, kn, vn = _rand((B, h_q, d), 160), _rand((B, h_kv, d), 161), _rand((B, h_kv, d), 162)
    kc = np.full((B, h_kv, S, d), np.nan)
    vc = np.full((B, h_kv, S, d), np.nan)
    o, _, _ = oracle.decode_append(q, kn, vn, kc, vc, [0] * B)
    G = h_q // h_kv
    for h in range(h_q):
        assert np.array_equal(o[:, h], vn[:, h // G]), "empty cache: output must be v_new"


def pin_append_brute_and_tail():
    """Against the brute force over a grown cache built by hand; NaN rows past
    the appended one never leak in; a length of S is rejected."""
    B, h_q, h_kv, d, S = 3, 4, 2, 5, 9
    q, kn, vn = _rand((B, h_q, d), 170), _rand((B, h_kv, d), 171), _rand((B, h_kv, d), 172)
    kc, vc = _rand((B, h_kv, S, d), 173), _rand((B, h_kv, S, d), 174)
    lens = [0, 4, 8]
    kp, vp = kc.copy(), vc.copy()
    for b, n in enumerate(lens):
        kp[b, :, n + 1:] = np.nan
        vp[b, :, n + 1:] = np.nan
    o, _, _ = oracle.decode_append(q, kn, vn, kp, vp, lens)
    kg, vg = kc.tolist(), vc.tolist()
    for b, n in enumerate(lens):
        for g in range(h_kv):
            kg[b][g][n] = kn[b, g].tolist()
            vg[b][g][n] = vn[b, g].tolist()
    _close(o, brute.decode(q.tolist(), kg, vg, [n + 1 for n in lens]), 1e-12,
           "append vs brute force over a hand-grown cache")
    try:
        oracle.decode_append(q, kn, vn, kc, vc, [S, 0, 0])
    except ValueError:
        pass
    else:
        raise AssertionError("seqlens[b] == S leaves no row to append into: must be rejected")


def pin_token_major_brute():
    """Token-major cache [B, S, h_kv, d] against the brute force over the same
    rows read out by index, and against the head-major entry on the transposed
    copy; NaN rows past a length never leak in."""
    B, h_q, h_kv, d, S = 3, 6, 2, 5, 7
    q = _rand((B, h_q, d), 180)
    kt, vt = _rand((B, S, h_kv, d), 181), _rand((B, S, h_kv, d), 182)
    lens = [0, 3, 7]
    for b, n in enumerate(lens):
        kt[b, n:] = np.nan
        vt[b, n:] = np.nan
    o = oracle.decode_token_major(q, kt, vt, lens)
    kg = [[[kt[b, j, g].tolist() for j in range(S)] for g in range(h_kv)] for b in range(B)]
    vg = [[[vt[b, j, g].tolist() for j in range(S)] for g in range(h_kv)] for b in range(B)]
    _close(o, brute.decode(q.tolist(), kg, vg, lens), 1e-12, "token-major vs brute force")
    o2 = oracle.decode(q, np.ascontiguousarray(kt.transpose(0, 2, 1, 3)),
                       np.ascontiguousarray(vt.transpose(0, 2, 1, 3)), lens)
    _close(o, o2, 0.0, "token-major vs head-major on the transposed cache")


def _scatter_to_pages(kc, vc, lens, page_size, seed, spare=3):
    """Scatter head-major caches [B, h_kv, S, d] into a shuffled page pool
    [num_pages, h_kv, page_size, d]; unused pages and rows past a length are NaN."""
    B, h_kv, S, d = kc.shape
    max_blocks = -(-S // page_size)
    need = [-(-n // page_size) for n in lens]
    num_pages = sum(need) + spare
    perm = np.random.default_rng(seed).permutation(num_pages)
    kp = np.full((num_pages, h_kv, page_size, d), np.nan)
    vp = np.full_like(kp, np.nan)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    nxt = 0
    for b, n in enumerate(lens):
        for i in range(need[b]):
            page = int(perm[nxt])
            nxt += 1
            table[b, i] = page
            rows = min(page_size, n - i * page_size)
            kp[page, :, :rows] = kc[b, :, i * page_size:i * page_size + rows]
            vp[page, :, :rows] = vc[b, :, i * page_size:i * page_size + rows]
    return kp, vp, table


def pin_paged_brute():
    """Paged cache with group-aligned pages ("Attention in Qwen, DeepSeek and
    LLaMA3", §4.3) on a shuffled pool: equal to the brute force and to the
    head-major entry over the logical cache; unused pages and rows past a
    length (NaN) never leak in; a page index outside the pool is rejected."""
    B, h_q, h_kv, d, S, P = 4, 8, 2, 6, 20, 4
    q = _rand((B, h_q, d), 190)
    kc, vc = _rand((B, h_kv, S, d), 191), _rand((B, h_kv, S, d), 192)
    lens = [0, 5, 8, 19]
    kp, vp, table = _scatter_to_pages(kc, vc, lens, P, 193)
    o = oracle.decode_paged(q, kp, vp, table, lens)
    _close(o, brute.decode(q.tolist(), kc.tolist(), vc.tolist(), lens), 1e-12,
           "paged vs brute force over the logical cache")
    _close(o, oracle.decode(q, kc, vc, lens), 0.0, "paged vs head-major over the logical cache")
    bad = table.copy()
    bad[3, 0] = kp.shape[0]
    try:
        oracle.decode_paged(q, kp, vp, bad, lens)
    except ValueError:
        pass
    else:
        raise AssertionError("a page index outside the pool must be rejected")


def pin_paged_shared_prefix():
    """Two sequences whose tables share their first pages (a shared prefix)
    give the outputs of two separate caches holding the same rows."""
    h_q, h_kv, d, P = 4, 1, 3, 2
    q = _rand((2, h_q, d), 195)
    pool_k, pool_v = _rand((5, h_kv, P, d), 196), _rand((5, h_kv, P, d), 197)
    table = np.array([[3, 0, 4], [3, 0, 1]], dtype=np.int32)
    lens = [5, 6]
    o = oracle.decode_paged(q, pool_k, pool_v, table, lens)
    kc = np.stack([np.concatenate([pool_k[p] for p in table[b]], axis=1) for b in range(2)])
    vc = np.stack([np.concatenate([pool_v[p] for p in table[b]], axis=1) for b in range(2)])
    _close(o, brute.decode(q.tolist(), kc.tolist(), vc.tolist(), lens), 1e-12,
           "shared-prefix pages vs brute force")


def _rope_tables(L, d, offset=0, base=10000.0):
    """cos, sin [L, d/2] for angles (p + offset) * base^(-2i/d) (test-side inputs)."""
    pos = np.arange(L, dtype=np.float64)[:, None] + offset
    freq = base ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)
    ang = pos * freq[None, :]
    return np.cos(ang), np.sin(ang)


def pin_rope_golden():
    """Hand-derived rotations and a 2-position prefill (tests/golden/rope_by_hand.json)."""
    g = _golden("rope_by_hand.json")
    x = np.array(g["x"])
    cv, sv = np.array(g["cos_vec"]), np.array(g["sin_vec"])
    both = np.concatenate([x, x], axis=1)  # the vector at positions 0 and 1
    r = oracle.rope(both, cv, sv)
    _close(r[0, 1, 0], g["expected_vector_p1"], 1e-15, "rope of the vector at position 1")
    _close(r[0, 0, 0], g["expected_vector_p0"], 0.0, "rope with cos 1, sin 0")
    o, k_rot = oracle.prefill_rope(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]),
                                   np.array(g["cos_attn"]), np.array(g["sin_attn"]), True, 1.0)
    _close(o, g["expected_o"], 1e-15, "rope prefill output")
    _close(k_rot, g["expected_k_rot"], 1e-15, "rotated keys")


def pin_rope_identity_tables():
    """cos = 1, sin = 0 turns the rotation into the fixed permutation evens-then-odds:
    the rotated keys are that permutation of k exactly, and the attention equals
    the plain prefill (a common permutation of q and k leaves every dot product)."""
    B, L, h_q, h_kv, d = 2, 9, 6, 3, 8
    q, k, v = _rand((B, L, h_q, d), 200), _rand((B, L, h_kv, d), 201), _rand((B, L, h_kv, d), 202)
    ones, zeros = np.ones((L, d // 2)), np.zeros((L, d // 2))
    perm = list(range(0, d, 2)) + list(range(1, d, 2))
    for causal in (False, True):
        o, k_rot = oracle.prefill_rope(q, k, v, ones, zeros, causal, 0.4)
        _close(k_rot, k[..., perm], 0.0, "identity tables: rotated keys = permuted keys")
        _close(o, oracle.prefill(q, k, v, causal=causal, scale=0.4), 1e-13,
               "identity tables: attention unchanged")


def pin_rope_relative_position():
    """With tables from angles theta_i * p, shifting every position by the same
    offset leaves the attention output unchanged (scores depend on m - n only),
    while the rotated keys do change; each pair keeps its norm."""
    B, L, h_q, h_kv, d = 1, 12, 4, 2, 16
    q, k, v = _rand((B, L, h_q, d), 210), _rand((B, L, h_kv, d), 211), _rand((B, L, h_kv, d), 212)
    c0, s0 = _rope_tables(L, d)
    c1, s1 = _rope_tables(L, d, offset=37)
    for causal in (False, True):
        o0, kr0 = oracle.prefill_rope(q, k, v, c0, s0, causal, 0.25)
        o1, kr1 = oracle.prefill_rope(q, k, v, c1, s1, causal, 0.25)
        _close(o0, o1, 1e-12, "rope: a common position shift leaves the attention")
        assert float(np.max(np.abs(kr0 - kr1))) > 1e-3, "the shift must move the rotated keys"
    half = d // 2
    n_in = k[..., 0::2] ** 2 + k[..., 1::2] ** 2
    n_out = kr0[..., :half] ** 2 + kr0[..., half:] ** 2
    _close(n_in, n_out, 1e-12, "rope keeps the norm of every pair")


def pin_rope_brute():
    """Against the pure-Python rotation followed by the brute-force prefill."""
    B, L, h_q, h_kv, d = 2, 5, 4, 2, 6
    q, k, v = _rand((B, L, h_q, d), 220), _rand((B, L, h_kv, d), 221), _rand((B, L, h_kv, d), 222)
    c, sn = _rope_tables(L, d, offset=3, base=100.0)
    for causal in (False, True):
        o, k_rot = oracle.prefill_rope(q, k, v, c, sn, causal, 0.5)
        qb = brute.rope(q.tolist(), c.tolist(), sn.tolist())
        kb = brute.rope(k.tolist(), c.tolist(), sn.tolist())
        ob, _ = brute.prefill(qb, kb, v.tolist(), causal, 0.5)
        _close(k_rot, kb, 1e-15, "rotated keys vs brute force")
        _close(o, ob, 1e-12, "rope prefill vs brute force")


def pin_varlen_equals_truncated():
    """A padded batch with lengths: each valid row equals the prefill of its
    sequence cut to its length; padding (NaN) never leaks in; a padded row
    sees every valid key (causal: as the last valid row's key set); a length
    of 0 gives zero rows."""
    B, L, h_q, h_kv, d = 4, 9, 6, 2, 5
    q, k, v = _rand((B, L, h_q, d), 230), _rand((B, L, h_kv, d), 231), _rand((B, L, h_kv, d), 232)
    lens = [9, 4, 1, 0]
    kp, vp = k.copy(), v.copy()
    for b, n in enumerate(lens):
        kp[b, n:] = np.nan
        vp[b, n:] = np.nan
    for causal in (False, True):
        o = oracle.prefill_varlen(q, kp, vp, lens, causal, 0.6)
        assert np.isfinite(o).all(), "padding leaked into the output"
        for b, n in enumerate(lens):
            if n == 0:
                _close(o[b], np.zeros_like(o[b]), 0.0, "length 0 gives zero rows")
                continue
            alone = oracle.prefill(q[b:b + 1, :n], k[b:b + 1, :n], v[b:b + 1, :n], causal=causal,
                                   scale=0.6)
            _close(o[b:b + 1, :n], alone, 1e-13, f"seq {b}: valid rows vs the cut sequence")
            # a padded row attends to all n valid keys (brute force, by hand)
            for i in range(n, L):
                for h in range(h_q):
                    g = h // (h_q // h_kv)
                    want, _ = brute._softmax_average(q[b, i, h].tolist(),
                                                     [k[b, j, g].tolist() for j in range(n)],
                                                     [v[b, j, g].tolist() for j in range(n)], 0.6)
                    _close(o[b, i, h], want, 1e-12, f"seq {b} padded row {i} head {h}")


def pin_varlen_library():
    """Against torch's fp64 SDPA with an explicit boolean mask (key padding, and
    causal), on sequences of nonzero length."""
    B, L, h_q, h_kv, d = 3, 11, 4, 4, 7
    q, k, v = _rand((B, L, h_q, d), 240), _rand((B, L, h_kv, d), 241), _rand((B, L, h_kv, d), 242)
    lens = [11, 6, 1]
    for causal in (False, True):
        o = oracle.prefill_varlen(q, k, v, lens, causal, 0.3)
        keep = torch.zeros(B, 1, L, L, dtype=torch.bool)
        for b, n in enumerate(lens):
            keep[b, :, :, :n] = True
        if causal:
            keep &= torch.ones(L, L, dtype=torch.bool).tril()
        tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=keep, scale=0.3)
        _close(o, ref.permute(0, 2, 1, 3).numpy(), 1e-12, f"varlen vs masked SDPA causal={causal}")
        rows = [(1, 0, 0), (1, 5, 3), (1, 10, 2), (2, 7, 1), (0, 10, 3)]
        qr = np.array([q[b, i, h] for (b, i, h) in rows])
        _close(oracle.prefill_varlen_rows(qr, rows, k, v, lens, h_q, causal, 0.3),
               np.array([o[b, i, h] for (b, i, h) in rows]), 0.0, "varlen rows vs full")


def pin_rope_decode_step():
    """A decode step with rotary embedding continues a rotary prefill: with the
    cache holding the prefill's rotated keys of positions 0..n-1, appending
    token n (rotated at position n) and attending gives the prefill's row n,
    and the appended cache row is the prefill's rotated key n.  With identity
    tables it is the plain decode with append of permuted q and k."""
    B, n, h_q, h_kv, d, S = 2, 9, 6, 2, 8, 12
    q, k, v = (_rand((B, n + 1, h_q, d), 250), _rand((B, n + 1, h_kv, d), 251),
               _rand((B, n + 1, h_kv, d), 252))
    c, sn = _rope_tables(S, d)
    full, k_rot = oracle.prefill_rope(q, k, v, c[:n + 1], sn[:n + 1], True, 1 / math.sqrt(d))
    kc = np.full((B, h_kv, S, d), np.nan)
    vc = np.full((B, h_kv, S, d), np.nan)
    kc[:, :, :n] = k_rot[:, :n].transpose(0, 2, 1, 3)
    vc[:, :, :n] = v[:, :n].transpose(0, 2, 1, 3)
    o, kc2, vc2 = oracle.decode_append_rope(q[:, n], k[:, n], v[:, n], kc, vc, [n] * B, c, sn)
    _close(o, full[:, n], 1e-12, "rotary decode step vs rotary prefill row n")
    _close(kc2[:, :, n], k_rot[:, n], 0.0, "appended row = the prefill's rotated key n")
    _close(vc2[:, :, n], v[:, n], 0.0, "appended value row")
    ones, zeros = np.ones((S, d // 2)), np.zeros((S, d // 2))
    perm = list(range(0, d, 2)) + list(range(1, d, 2))
    o1, k1, _ = oracle.decode_append_rope(q[:, n], k[:, n], v[:, n], kc, vc, [n] * B, ones, zeros)
    o2, k2, _ = oracle.decode_append(q[:, n][..., perm], k[:, n][..., perm], v[:, n], kc, vc,
                                     [n] * B)
    _close(o1, o2, 0.0, "identity tables: plain decode of permuted q, k")
    _close(k1[:, :, :n + 1], k2[:, :, :n + 1], 0.0, "identity tables: appended permuted key")


def pin_mask_golden():
    """The hand-worked keep-mask case: closed-form weights, a fully hidden row
    that is zero, and the causal mask applied on top of the keep-mask."""
    g = _golden("mask_by_hand.json")
    q, k, v, m = (np.array(g[n]) for n in ("q", "k", "v", "mask"))
    tol = g["tolerance"]
    for causal, key in ((False, "expected_noncausal"), (True, "expected_causal")):
        o = oracle.prefill_mask(q, k, v, m, causal, g["scale"])
        _close(o, g[key], tol, f"mask by hand causal={causal}")
        ob = brute.prefill_mask(g["q"], g["k"], g["v"], g["mask"], causal, g["scale"])
        _close(ob, g[key], tol, f"brute force mask by hand causal={causal}")
    assert np.array_equal(oracle.prefill_mask(q, k, v, m, False, 1.0)[0, 1],
                          np.zeros((2, 2))), "a row with no visible key is exactly zero"


def _random_mask(shape, seed, density=0.5):
    g = np.random.default_rng(seed)
    return (g.random(shape) < density).astype(np.uint8)


def pin_mask_library():
    """Against torch's fp64 SDPA with a boolean attn_mask (the keep-mask, and
    bottom-right causal folded in) and enable_gqa for the head map, on an
    asymmetric random mask with L_q < L_k; rows with no visible key are zero."""
    B, Lq, Lk, h_q, h_kv, d = 2, 9, 13, 6, 2, 5
    q, k, v = (_rand((B, Lq, h_q, d), 260), _rand((B, Lk, h_kv, d), 261),
               _rand((B, Lk, h_kv, d), 262))
    m = _random_mask((B, Lq, Lk), 263, 0.45)
    m[1, 4] = 0  # one row with no visible key
    for causal in (False, True):
        keep = torch.from_numpy(m != 0)
        if causal:
            i = torch.arange(Lq)[:, None]
            j = torch.arange(Lk)[None, :]
            keep = keep & (j <= Lk - Lq + i)[None]
        o = oracle.prefill_mask(q, k, v, m, causal, 0.4)
        tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=keep[:, None], scale=0.4,
                                             enable_gqa=True).permute(0, 2, 1, 3).numpy()
        empty = ~keep.any(dim=-1).numpy()  # [B, Lq]
        assert empty[1, 4], "the emptied row must have no visible key"
        _close(o[~empty], ref[~empty], 1e-12, f"mask vs masked SDPA causal={causal}")
        _close(o[empty], np.zeros_like(o[empty]), 0.0, "rows with no visible key are zero")


def pin_mask_reductions():
    """Masks that other entry points express: all ones is the prefill against
    L_k keys, lengths are the padded variable-length prefill, and the lower
    triangle without the causal flag is the causal prefill (bit for bit: the
    same keys in the same order)."""
    B, L, h_q, h_kv, d = 3, 10, 4, 2, 6
    q, k, v = _rand((B, L, h_q, d), 270), _rand((B, L, h_kv, d), 271), _rand((B, L, h_kv, d), 272)
    for causal in (False, True):
        ones = np.ones((B, L, L), np.uint8)
        _close(oracle.prefill_mask(q, k, v, ones, causal, 0.5),
               oracle.prefill(q, k, v, causal=causal, scale=0.5), 0.0, "all-ones mask")
        lens = [10, 3, 0]
        bylen = np.zeros((B, L, L), np.uint8)
        for b, n in enumerate(lens):
            bylen[b, :, :n] = 1
        _close(oracle.prefill_mask(q, k, v, bylen, causal, 0.5),
               oracle.prefill_varlen(q, k, v, lens, causal, 0.5), 0.0, "length mask")
    tril = np.broadcast_to(np.tril(np.ones((L, L), np.uint8)), (B, L, L))
    _close(oracle.prefill_mask(q, k, v, tril, False, 0.5),
           oracle.prefill(q, k, v, causal=True, scale=0.5), 0.0, "lower-triangle mask")
    qc, kc, vc = q[:, 6:], k, v
    onesc = np.ones((B, 4, L), np.uint8)
    _close(oracle.prefill_mask(qc, kc, vc, onesc, True, 0.5),
           oracle.prefill_cached(qc, kc, vc, True, 0.5), 0.0, "all-ones mask, L_q < L_k")


def pin_mask_brute():
    """Against the pure-Python brute force on random masks (causal and not,
    L_q < L_k), and the rows entry against the full entry."""
    B, Lq, Lk, h_q, h_kv, d = 2, 5, 8, 6, 3, 4
    q, k, v = (_rand((B, Lq, h_q, d), 280), _rand((B, Lk, h_kv, d), 281),
               _rand((B, Lk, h_kv, d), 282))
    m = _random_mask((B, Lq, Lk), 283, 0.4)
    for causal in (False, True):
        o = oracle.prefill_mask(q, k, v, m, causal, 0.7)
        ob = brute.prefill_mask(q.tolist(), k.tolist(), v.tolist(), m.tolist(), causal, 0.7)
        _close(o, ob, 1e-12, f"mask vs brute force causal={causal}")
        rows = [(0, 0, 0), (1, 4, 5), (0, 2, 3), (1, 1, 2)]
        qr = np.array([q[b, i, h] for (b, i, h) in rows])
        _close(oracle.prefill_mask_rows(qr, rows, k, v, m, h_q, causal, 0.7),
               np.array([o[b, i, h] for (b, i, h) in rows]), 0.0, "mask rows vs full")
    _, p = oracle.prefill_mask(q, k, v, m, True, 0.7, return_probs=True)
    sums = p.sum(axis=-1)
    vis = np.array([[(m[b, i] * (np.arange(Lk) <= Lk - Lq + i)).any() for i in range(Lq)]
                    for b in range(B)])
    ok = sums[np.broadcast_to(vis[:, None], sums.shape)]
    _close(ok, np.ones_like(ok), 1e-15, "mask rows sum to 1")
    hidden = (m[:, None] == 0) | (np.arange(Lk)[None, None, None] >
                                  (Lk - Lq + np.arange(Lq))[None, None, :, None])
    assert np.all(p[np.broadcast_to(hidden, p.shape)] == 0.0), "hidden keys get weight 0"


ALL_PINS = [pin_hand_2x2, pin_head_map, pin_decode_golden, pin_mha_reduction,
            pin_mqa_reduction, pin_gqa_library, pin_rows_sum_to_one, pin_k_zero_mean,
            pin_causal_row0, pin_identical_heads, pin_invariances, pin_cross_path,
            pin_rows_match_full, pin_decode_tail_ignored, pin_argument_errors,
            pin_chunk_golden, pin_chunked_equals_full, pin_chunk_single_query_is_decode,
            pin_chunk_brute_and_library, pin_chunk_rows_match_full, pin_append_cross_path,
            pin_append_to_empty_cache, pin_append_brute_and_tail, pin_token_major_brute,
            pin_paged_brute, pin_paged_shared_prefix, pin_rope_golden,
            pin_rope_identity_tables, pin_rope_relative_position, pin_rope_brute,
            pin_varlen_equals_truncated, pin_varlen_library, pin_rope_decode_step,
            pin_mask_golden, pin_mask_library, pin_mask_reductions, pin_mask_brute]


def main(argv):
    """Run every pin against the oracle library at argv[1]; exit 1 if any fails."""
    if len(argv) > 1:
        oracle._LIB_PATH = argv[1]
    failed = []
    for pin in ALL_PINS:
        try:
            pin()
        except AssertionError as e:
            failed.append(f"{pin.__name__}: {e}")
    for f in failed:
        print("FAIL", f)
    print("pins failed: %d of %d" % (len(failed), len(ALL_PINS)))
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
