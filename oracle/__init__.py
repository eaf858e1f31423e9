"""Plain fp64 CPU oracle for the grouped-query attention core.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
(the HIP library and its Python binding) never imports it, and this package
imports nothing from the product: the two share no code.

Two independent implementations live here:

* ``gqa_oracle.c`` -- the fp64 C oracle (OpenMP over independent rows), loaded
  with ctypes.  It explicitly repeats every key/value head once per query head
  of its group, then evaluates softmax(q k^T * scale) v row by row
  ("Modern LLM architecture (1): GQA and RMSNorm", §2.1 formula and §2.3
  repeat_interleave module).
* ``brute.py`` -- a pure-Python (``math`` only) brute force for tiny inputs.

All functions take and return float64 numpy arrays in the layouts of the
library's entry points: prefill q, o [B, L, h_q, d] and k, v [B, L, h_kv, d];
decode q, o [B, h_q, d] (the one new position per sequence), caches
[B, h_kv, S, d] (token-major form [B, S, h_kv, d]; paged form
[num_pages, h_kv, page_size, d] with a block table [B, max_blocks]) and
seqlens [B].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgqa_oracle.so")
_DEFAULT_LIB = _LIB_PATH

# No -ffast-math and no FP contraction: the C code's operation order is the
# order that is evaluated.
_CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with the host gcc into ``oracle/libgqa_oracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # the in-tree library is rebuilt when missing or older than its source (a
    # library named explicitly, such as a test's mutant, is loaded as it is)
    if _LIB_PATH == _DEFAULT_LIB and (not os.path.exists(_LIB_PATH) or
                                      os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.gqa_oracle_prefill.argtypes = [P, P, P, P, I, I, I, I, I, I, ctypes.c_double, P]
    lib.gqa_oracle_prefill.restype = I
    lib.gqa_oracle_prefill_rows.argtypes = [P, P, ctypes.c_int64, P, P, I, I, I, I, I, I,
                                           ctypes.c_double, P, P]
    lib.gqa_oracle_prefill_rows.restype = I
    lib.gqa_oracle_prefill_cached.argtypes = [P, P, P, P, I, I, I, I, I, I, I,
                                              ctypes.c_double, P]
    lib.gqa_oracle_prefill_cached.restype = I
    lib.gqa_oracle_prefill_cached_rows.argtypes = [P, P, ctypes.c_int64, P, P, I, I, I, I, I,
                                                   I, I, ctypes.c_double, P]
    lib.gqa_oracle_prefill_cached_rows.restype = I
    lib.gqa_oracle_decode.argtypes = [P, P, P, P, P, I, I, I, I, I]
    lib.gqa_oracle_decode_append.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I]
    lib.gqa_oracle_decode_append.restype = I
    lib.gqa_oracle_decode.restype = I
    lib.gqa_oracle_decode_token_major.argtypes = [P, P, P, P, P, I, I, I, I, I]
    lib.gqa_oracle_decode_token_major.restype = I
    lib.gqa_oracle_decode_paged.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I]
    lib.gqa_oracle_decode_paged.restype = I
    lib.gqa_oracle_prefill_varlen.argtypes = [P, P, P, P, P, I, I, I, I, I, I, ctypes.c_double]
    lib.gqa_oracle_prefill_varlen.restype = I
    lib.gqa_oracle_prefill_varlen_rows.argtypes = [P, P, ctypes.c_int64, P, P, P, I, I, I, I, I,
                                                   I, ctypes.c_double, P]
    lib.gqa_oracle_prefill_varlen_rows.restype = I
    lib.gqa_oracle_decode_append_rope.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I]
    lib.gqa_oracle_decode_append_rope.restype = I
    lib.gqa_oracle_rope.argtypes = [P, P, P, P, I, I, I, I]
    lib.gqa_oracle_rope.restype = I
    lib.gqa_oracle_prefill_rope.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I,
                                            ctypes.c_double]
    lib.gqa_oracle_prefill_rope.restype = I
    lib.gqa_oracle_prefill_mask.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, ctypes.c_double,
                                            P]
    lib.gqa_oracle_prefill_mask.restype = I
    lib.gqa_oracle_prefill_mask_rows.argtypes = [P, P, ctypes.c_int64, P, P, P, I, I, I, I, I, I,
                                                 I, ctypes.c_double, P, P]
    lib.gqa_oracle_prefill_mask_rows.restype = I
    lib.gqa_oracle_num_threads.argtypes = []
    lib.gqa_oracle_num_threads.restype = I
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """Threads the oracle's parallel loops use (OpenMP's maximum)."""
    return int(_load().gqa_oracle_num_threads())


def prefill(q, k, v, causal: bool, scale: float, return_probs: bool = False):
    """Full prefill.  q [B,L,h_q,d], k/v [B,L,h_kv,d] -> o [B,L,h_q,d] (float64).

    With ``return_probs`` also returns the softmax matrices [B, h_q, L, L]
    (zero where a key is masked).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, L, h_q, d = q.shape
    h_kv = k.shape[2]
    if k.shape != (B, L, h_kv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, L, h_kv, d] matching q")
    o = np.empty_like(q)
    probs = np.empty((B, h_q, L, L)) if return_probs else None
    rc = _load().gqa_oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, L, h_q, h_kv, d,
                                    int(bool(causal)), float(scale),
                                    _ptr(probs) if probs is not None else None)
    if rc != 0:
        raise ValueError("oracle prefill rejected its arguments (rc=%d)" % rc)
    return (o, probs) if return_probs else o


def prefill_rows(q_rows, rows_bih, k, v, h_q: int, causal: bool, scale: float):
    """Prefill output of selected rows only.

    q_rows [n, d] holds the query vectors of the rows (b, i, h) listed in
    rows_bih [n, 3]; k/v are the full [B, L, h_kv, d] tensors.  Returns [n, d].
    """
    q_rows = _f64(q_rows)
    rows = np.ascontiguousarray(np.asarray(rows_bih, dtype=np.int64).reshape(-1, 3))
    k, v = _f64(k), _f64(v)
    B, L, h_kv, d = k.shape
    n = rows.shape[0]
    if q_rows.shape != (n, d):
        raise ValueError("q_rows must be [n, d]")
    out = np.empty((n, d))
    rc = _load().gqa_oracle_prefill_rows(_ptr(q_rows), _ptr(rows), n, _ptr(k), _ptr(v), B, L,
                                         h_q, h_kv, d, int(bool(causal)), float(scale),
                                         _ptr(out), None)
    if rc != 0:
        raise ValueError("oracle prefill_rows rejected its arguments (rc=%d)" % rc)
    return out


def prefill_cached(q, k, v, causal: bool, scale: float, return_probs: bool = False):
    """Prefill of L_q new positions against L_k keys (1 <= L_q <= L_k).

    q [B,L_q,h_q,d], k/v [B,L_k,h_kv,d] -> o [B,L_q,h_q,d] (float64).  Query
    row i sits at position L_k - L_q + i, so causally it sees keys
    0 .. L_k - L_q + i.  With ``return_probs`` also returns [B, h_q, L_q, L_k].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Lq, h_q, d = q.shape
    Lk, h_kv = k.shape[1], k.shape[2]
    if k.shape != (B, Lk, h_kv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, L_k, h_kv, d] matching q")
    o = np.empty_like(q)
    probs = np.empty((B, h_q, Lq, Lk)) if return_probs else None
    rc = _load().gqa_oracle_prefill_cached(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, Lq, Lk, h_q,
                                           h_kv, d, int(bool(causal)), float(scale),
                                           _ptr(probs) if probs is not None else None)
    if rc != 0:
        raise ValueError("oracle prefill_cached rejected its arguments (rc=%d)" % rc)
    return (o, probs) if return_probs else o


def prefill_cached_rows(q_rows, rows_bih, k, v, h_q: int, Lq: int, causal: bool, scale: float):
    """prefill_cached output of selected rows (b, i, h), 0 <= i < Lq; returns [n, d]."""
    q_rows = _f64(q_rows)
    rows = np.ascontiguousarray(np.asarray(rows_bih, dtype=np.int64).reshape(-1, 3))
    k, v = _f64(k), _f64(v)
    B, Lk, h_kv, d = k.shape
    n = rows.shape[0]
    if q_rows.shape != (n, d):
        raise ValueError("q_rows must be [n, d]")
    out = np.empty((n, d))
    rc = _load().gqa_oracle_prefill_cached_rows(_ptr(q_rows), _ptr(rows), n, _ptr(k), _ptr(v),
                                                B, Lq, Lk, h_q, h_kv, d, int(bool(causal)),
                                                float(scale), _ptr(out))
    if rc != 0:
        raise ValueError("oracle prefill_cached_rows rejected its arguments (rc=%d)" % rc)
    return out


def decode(q, k_cache, v_cache, seqlens):
    """Decode.  q [B,h_q,d], caches [B,h_kv,S,d], seqlens [B] -> o [B,h_q,d]."""
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    B, h_q, d = q.shape
    _, h_kv, S, _ = kc.shape
    if kc.shape != (B, h_kv, S, d) or vc.shape != kc.shape or sl.shape != (B,):
        raise ValueError("decode shapes do not match")
    o = np.empty_like(q)
    rc = _load().gqa_oracle_decode(_ptr(q), _ptr(kc), _ptr(vc), _ptr(sl), _ptr(o), B, h_q,
                                   h_kv, S, d)
    if rc != 0:
        raise ValueError("oracle decode rejected its arguments (rc=%d)" % rc)
    return o


def prefill_varlen(q, k, v, kv_lens, causal: bool, scale: float):
    """Padded variable-length prefill: q [B,L,h_q,d], k/v [B,L,h_kv,d], kv_lens [B];
    key j of sequence b is visible iff j < kv_lens[b] (and j <= i when causal)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    kl = np.ascontiguousarray(np.asarray(kv_lens, dtype=np.int32))
    B, L, h_q, d = q.shape
    h_kv = k.shape[2]
    if k.shape != (B, L, h_kv, d) or v.shape != k.shape or kl.shape != (B,):
        raise ValueError("prefill_varlen shapes do not match")
    o = np.empty_like(q)
    rc = _load().gqa_oracle_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(kl), _ptr(o), B, L,
                                           h_q, h_kv, d, int(bool(causal)), float(scale))
    if rc != 0:
        raise ValueError("oracle prefill_varlen rejected its arguments (rc=%d)" % rc)
    return o


def prefill_varlen_rows(q_rows, rows_bih, k, v, kv_lens, h_q: int, causal: bool, scale: float):
    """Selected rows (b, i, h) of the padded variable-length prefill.  Returns [n, d]."""
    q_rows = _f64(q_rows)
    rows = np.ascontiguousarray(np.asarray(rows_bih, dtype=np.int64).reshape(-1, 3))
    k, v = _f64(k), _f64(v)
    kl = np.ascontiguousarray(np.asarray(kv_lens, dtype=np.int32))
    B, L, h_kv, d = k.shape
    n = rows.shape[0]
    if q_rows.shape != (n, d) or kl.shape != (B,):
        raise ValueError("prefill_varlen_rows shapes do not match")
    out = np.empty((n, d))
    rc = _load().gqa_oracle_prefill_varlen_rows(_ptr(q_rows), _ptr(rows), n, _ptr(k), _ptr(v),
                                                _ptr(kl), B, L, h_q, h_kv, d, int(bool(causal)),
                                                float(scale), _ptr(out))
    if rc != 0:
        raise ValueError("oracle prefill_varlen_rows rejected its arguments (rc=%d)" % rc)
    return out


def _mask_u8(mask, B, Lq, Lk):
    m = np.asarray(mask)
    if m.shape != (B, Lq, Lk):
        raise ValueError("mask must be [B, L_q, L_k]")
    return np.ascontiguousarray(m != 0, dtype=np.uint8)


def prefill_mask(q, k, v, mask, causal: bool, scale: float, return_probs: bool = False):
    """Prefill with a keep-mask: q [B,L_q,h_q,d], k/v [B,L_k,h_kv,d], mask
    [B,L_q,L_k] (key j visible to row i iff mask[b,i,j] != 0, and j <= L_k -
    L_q + i when causal) -> o [B,L_q,h_q,d]; a row with no visible key is zero.
    With ``return_probs`` also returns [B, h_q, L_q, L_k]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Lq, h_q, d = q.shape
    Lk, h_kv = k.shape[1], k.shape[2]
    if k.shape != (B, Lk, h_kv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, L_k, h_kv, d] matching q")
    m = _mask_u8(mask, B, Lq, Lk)
    o = np.empty_like(q)
    probs = np.empty((B, h_q, Lq, Lk)) if return_probs else None
    rc = _load().gqa_oracle_prefill_mask(_ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(o), B, Lq, Lk,
                                         h_q, h_kv, d, int(bool(causal)), float(scale),
                                         _ptr(probs) if probs is not None else None)
    if rc != 0:
        raise ValueError("oracle prefill_mask rejected its arguments (rc=%d)" % rc)
    return (o, probs) if return_probs else o


def prefill_mask_rows(q_rows, rows_bih, k, v, mask, h_q: int, causal: bool, scale: float):
    """Selected rows (b, i, h) of the keep-mask prefill; mask [B, L_q, L_k].
    Returns [n, d]."""
    q_rows = _f64(q_rows)
    rows = np.ascontiguousarray(np.asarray(rows_bih, dtype=np.int64).reshape(-1, 3))
    k, v = _f64(k), _f64(v)
    B, Lk, h_kv, d = k.shape
    Lq = np.asarray(mask).shape[1]
    m = _mask_u8(mask, B, Lq, Lk)
    n = rows.shape[0]
    if q_rows.shape != (n, d):
        raise ValueError("q_rows must be [n, d]")
    out = np.empty((n, d))
    rc = _load().gqa_oracle_prefill_mask_rows(_ptr(q_rows), _ptr(rows), n, _ptr(k), _ptr(v),
                                              _ptr(m), B, Lq, Lk, h_q, h_kv, d,
                                              int(bool(causal)), float(scale), _ptr(out), None)
    if rc != 0:
        raise ValueError("oracle prefill_mask_rows rejected its arguments (rc=%d)" % rc)
    return out


def rope(x, cos, sin):
    """Rotary embedding of x [B, L, H, d] with tables cos, sin [L, d/2] (see the C source)."""
    x, ct, st = _f64(x), _f64(cos), _f64(sin)
    B, L, H, d = x.shape
    if d % 2 or ct.shape != (L, d // 2) or st.shape != ct.shape:
        raise ValueError("rope shapes do not match")
    out = np.empty_like(x)
    rc = _load().gqa_oracle_rope(_ptr(x), _ptr(ct), _ptr(st), _ptr(out), B, L, H, d)
    if rc != 0:
        raise ValueError("oracle rope rejected its arguments (rc=%d)" % rc)
    return out


def prefill_rope(q, k, v, cos, sin, causal, scale):
    """Prefill with q and k rotated first.  Returns (o [B,L,h_q,d], k_rot [B,L,h_kv,d])."""
    q, k, v, ct, st = _f64(q), _f64(k), _f64(v), _f64(cos), _f64(sin)
    B, L, h_q, d = q.shape
    h_kv = k.shape[2]
    if (k.shape != (B, L, h_kv, d) or v.shape != k.shape or ct.shape != (L, d // 2)
            or st.shape != ct.shape):
        raise ValueError("prefill_rope shapes do not match")
    o = np.empty_like(q)
    k_rot = np.empty_like(k)
    rc = _load().gqa_oracle_prefill_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(ct), _ptr(st), _ptr(o),
                                         _ptr(k_rot), B, L, h_q, h_kv, d, int(bool(causal)),
                                         float(scale))
    if rc != 0:
        raise ValueError("oracle prefill_rope rejected its arguments (rc=%d)" % rc)
    return o, k_rot


def decode_append_rope(q, k_new, v_new, k_cache, v_cache, seqlens, cos, sin):
    """Decode step with rotary embedding: q [B,h_q,d] and k_new [B,h_kv,d]
    rotated with row seqlens[b] of cos, sin [S, d/2], the rotated key appended
    at row seqlens[b], then attend.  Returns (o, k_cache', v_cache') (copies)."""
    q, kn, vn = _f64(q), _f64(k_new), _f64(v_new)
    kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
    ct, st = _f64(cos), _f64(sin)
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    B, h_q, d = q.shape
    _, h_kv, S, _ = kc.shape
    if (kc.shape != (B, h_kv, S, d) or vc.shape != kc.shape or kn.shape != (B, h_kv, d)
            or vn.shape != kn.shape or sl.shape != (B,) or ct.shape != (S, d // 2)
            or st.shape != ct.shape):
        raise ValueError("decode_append_rope shapes do not match")
    o = np.empty_like(q)
    rc = _load().gqa_oracle_decode_append_rope(_ptr(q), _ptr(kn), _ptr(vn), _ptr(kc), _ptr(vc),
                                               _ptr(sl), _ptr(ct), _ptr(st), _ptr(o), B, h_q,
                                               h_kv, S, d)
    if rc != 0:
        raise ValueError("oracle decode_append_rope rejected its arguments (rc=%d)" % rc)
    return o, kc, vc


def decode_token_major(q, k_cache, v_cache, seqlens):
    """Decode over a token-major cache.  q [B,h_q,d], caches [B,S,h_kv,d], seqlens [B]."""
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    B, h_q, d = q.shape
    _, S, h_kv, _ = kc.shape
    if kc.shape != (B, S, h_kv, d) or vc.shape != kc.shape or sl.shape != (B,):
        raise ValueError("decode_token_major shapes do not match")
    o = np.empty_like(q)
    rc = _load().gqa_oracle_decode_token_major(_ptr(q), _ptr(kc), _ptr(vc), _ptr(sl), _ptr(o),
                                               B, h_q, h_kv, S, d)
    if rc != 0:
        raise ValueError("oracle decode_token_major rejected its arguments (rc=%d)" % rc)
    return o


def decode_paged(q, k_pages, v_pages, block_table, seqlens):
    """Decode over a paged cache with group-aligned pages.

    q [B,h_q,d]; k_pages, v_pages [num_pages, h_kv, page_size, d]; block_table
    [B, max_blocks] (block i of sequence b holds its positions
    [i*page_size, (i+1)*page_size)); seqlens [B].
    """
    q, kp, vp = _f64(q), _f64(k_pages), _f64(v_pages)
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    B, h_q, d = q.shape
    num_pages, h_kv, page_size, _ = kp.shape
    if (kp.shape != (num_pages, h_kv, page_size, d) or vp.shape != kp.shape or bt.ndim != 2
            or bt.shape[0] != B or sl.shape != (B,)):
        raise ValueError("decode_paged shapes do not match")
    o = np.empty_like(q)
    rc = _load().gqa_oracle_decode_paged(_ptr(q), _ptr(kp), _ptr(vp), _ptr(bt), _ptr(sl),
                                         _ptr(o), B, h_q, h_kv, page_size, bt.shape[1],
                                         num_pages, d)
    if rc != 0:
        raise ValueError("oracle decode_paged rejected its arguments (rc=%d)" % rc)
    return o


def decode_append(q, k_new, v_new, k_cache, v_cache, seqlens):
    """Decode with append.  q [B,h_q,d], k_new/v_new [B,h_kv,d], caches [B,h_kv,S,d],
    seqlens [B] (before the append, each < S).

    Returns (o [B,h_q,d], k_cache', v_cache'): the caches with the new rows
    written at row seqlens[b] (copies; the inputs are not modified), and the
    output of attending over rows [0, seqlens[b] + 1).
    """
    q, kn, vn = _f64(q), _f64(k_new), _f64(v_new)
    kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    B, h_q, d = q.shape
    _, h_kv, S, _ = kc.shape
    if (kc.shape != (B, h_kv, S, d) or vc.shape != kc.shape or kn.shape != (B, h_kv, d)
            or vn.shape != kn.shape or sl.shape != (B,)):
        raise ValueError("decode_append shapes do not match")
    o = np.empty_like(q)
    rc = _load().gqa_oracle_decode_append(_ptr(q), _ptr(kn), _ptr(vn), _ptr(kc), _ptr(vc),
                                          _ptr(sl), _ptr(o), B, h_q, h_kv, S, d)
    if rc != 0:
        raise ValueError("oracle decode_append rejected its arguments (rc=%d)" % rc)
    return o, kc, vc
