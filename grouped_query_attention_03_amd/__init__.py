"""MI355X (gfx950) grouped-query attention core: Python binding of ``libgqa_hip.so``.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/gqa.h``.  PyTorch supplies device memory
and the current stream.  There is no fallback: if the library is missing or
the device is not a gfx950 GPU, the calls raise.

    prefill(q, k, v, causal=..., scale=None, out=None)
        q [B, L, h_q, d], k/v [B, L, h_kv, d] (bf16 or fp32, contiguous, on the
        GPU) -> o [B, L, h_q, d].  Query head h reads key/value head
        h // (h_q // h_kv).
    prefill_chunk(q, k, v, causal=..., scale=None, out=None)
        q [B, L_q, h_q, d] against k/v [B, L_k, h_kv, d] (L_q <= L_k): the L_q
        newest positions attend to all L_k keys (causally, row i sees keys
        0 .. L_k - L_q + i).
    decode(q, k_cache, v_cache, seqlens, out=None, workspace=None, num_splits=0)
        q [B, 1, h_q, d] bf16, caches [B, h_kv, S, d] bf16, seqlens [B] int32
        -> o [B, 1, h_q, d].
    prefill_varlen(q, k, v, kv_lens, causal=..., scale=None, out=None)
        padded batch; key j of sequence b visible iff j < kv_lens[b].
    prefill_mask(q, k, v, mask, causal=..., scale=None, out=None)
        q [B, L_q, h_q, d] against k/v [B, L_k, h_kv, d]; key j visible to query
        row i of sequence b only where mask[b, i, j] != 0 (mask [B, L_q, L_k]
        or [L_q, L_k], bool or uint8, on the GPU), and causally as in
        prefill_chunk; a row with no visible key is zero.
    prefill_rope(q, k, v, cos, sin, causal=..., scale=None, out=None, k_rot=None)
        q and k rotated (tables cos, sin [L, d/2]), then prefill; returns
        (o, k_rot).
    decode_append_rope(q, k_new, v_new, k_cache, v_cache, seqlens, cos, sin, ...)
        decode with append, q and k_new rotated at position seqlens[b] first.
    decode_noalloc(q, k_cache, v_cache, seqlens, out=..., num_splits=0)
        as decode, with the library's fixed scratch as workspace: allocates nothing.
    decode_token_major(q, k_cache, v_cache, seqlens, ...)
        as decode, with caches [B, S, h_kv, d].
    decode_paged(q, k_pages, v_pages, block_table, seqlens, ...)
        as decode, over pools [num_pages, h_kv, page_size, d] and a block
        table [B, max_blocks].
    decode_append(q, k_new, v_new, k_cache, v_cache, seqlens, ...)
        writes k_new/v_new [B, 1, h_kv, d] at cache row seqlens[b], then attends
        over rows [0, seqlens[b] + 1).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libgqa_hip.so")

GQA_F32 = 0
GQA_BF16 = 1

_lib = None


class GQAError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {status_string(status)}")


def lib() -> ctypes.CDLL:
    """Load ``libgqa_hip.so`` (building it first only if it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    L = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.gqa_prefill.argtypes = [P, P, P, P, I, I, I, I, I, I, I, F, P]
    L.gqa_prefill.restype = I
    L.gqa_prefill_chunk.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, F, P]
    L.gqa_prefill_chunk.restype = I
    L.gqa_decode.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, P, ctypes.c_size_t, P]
    L.gqa_decode.restype = I
    L.gqa_decode_append.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, P,
                                    ctypes.c_size_t, P]
    L.gqa_decode_append.restype = I
    L.gqa_decode_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, P]
    L.gqa_decode_noalloc.restype = I
    L.gqa_decode_noalloc_max_bytes.argtypes = []
    L.gqa_decode_noalloc_max_bytes.restype = ctypes.c_size_t
    L.gqa_decode_token_major.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, P, ctypes.c_size_t, P]
    L.gqa_decode_token_major.restype = I
    L.gqa_decode_paged.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, P, ctypes.c_size_t, P]
    L.gqa_decode_paged.restype = I
    L.gqa_prefill_varlen.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, P]
    L.gqa_prefill_varlen.restype = I
    LL = ctypes.c_longlong
    SZ = ctypes.c_size_t
    L.gqa_prefill_mask.argtypes = [P, P, P, P, LL, LL, P, I, I, I, I, I, I, I, I, F, P, SZ, P]
    L.gqa_prefill_mask.restype = I
    L.gqa_prefill_mask_workspace_bytes.argtypes = [I, I, I]
    L.gqa_prefill_mask_workspace_bytes.restype = ctypes.c_size_t
    L.gqa_prefill_rope.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P]
    L.gqa_prefill_rope.restype = I
    L.gqa_decode_append_rope.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P,
                                         ctypes.c_size_t, P]
    L.gqa_decode_append_rope.restype = I
    L.gqa_decode_rope_workspace_bytes.argtypes = [I, I, I, I, I]
    L.gqa_decode_rope_workspace_bytes.restype = ctypes.c_size_t
    L.gqa_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    L.gqa_decode_workspace_bytes.restype = ctypes.c_size_t
    L.gqa_decode_default_splits.argtypes = []
    L.gqa_decode_default_splits.restype = I
    L.gqa_status_string.argtypes = [I]
    L.gqa_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().gqa_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GQA_BF16
    if t.dtype == torch.float32:
        return GQA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(t: torch.Tensor, name: str, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same(ref: torch.Tensor, *named):
    """Every (tensor, name) pair shares ref's dtype and device."""
    for t, name in named:
        if t.dtype != ref.dtype:
            raise TypeError(f"{name} must have dtype {ref.dtype}, got {t.dtype}")
        if t.device != ref.device:
            raise ValueError(f"{name} must be on {ref.device}, got {t.device}")


def _on_device(ref: torch.Tensor, *named):
    """Every (tensor, name) pair sits on ref's device."""
    for t, name in named:
        if t.device != ref.device:
            raise ValueError(f"{name} must be on {ref.device}, got {t.device}")


def _check_out(out, like: torch.Tensor, name: str = "out"):
    """A caller-supplied output must be a contiguous GPU tensor of like's shape and dtype."""
    _check(out, name, like.dim())
    if out.shape != like.shape or out.dtype != like.dtype:
        raise ValueError(f"{name} must match {tuple(like.shape)} {like.dtype}, got "
                         f"{tuple(out.shape)} {out.dtype}")
    if out.device != like.device:
        raise ValueError(f"{name} must be on {like.device}")


def _workspace(workspace, need: int, like: torch.Tensor):
    """The caller's workspace (a GPU tensor of at least need bytes), or a new one."""
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=like.device)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise ValueError("workspace must be a GPU tensor")
    if workspace.device != like.device:
        raise ValueError(f"workspace must be on {like.device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} "
                         f"bytes, {need} needed")
    return workspace


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def prefill(q, k, v, *, causal: bool, scale: float | None = None, out=None):
    _check(q, "q", 4)
    _check(k, "k", 4)
    _check(v, "v", 4)
    B, L, h_q, d = q.shape
    h_kv = k.shape[2]
    if tuple(k.shape) != (B, L, h_kv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, L, h_kv, d] with q's B, L and d")
    _same(q, (k, "k"), (v, "v"))
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(q.device):  # the library launches on the current device
        st = lib().gqa_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, L, h_q,
                               h_kv, d, _dtype_code(q), int(bool(causal)), float(scale), _stream(q))
    if st != 0:
        raise GQAError(st, "gqa_prefill")
    return out


def prefill_chunk(q, k, v, *, causal: bool, scale: float | None = None, out=None):
    """The L_q newest positions against all L_k keys: q [B,L_q,h_q,d], k/v
    [B,L_k,h_kv,d] -> o [B,L_q,h_q,d]; causally, query row i sees keys
    0 .. L_k - L_q + i."""
    _check(q, "q", 4)
    _check(k, "k", 4)
    _check(v, "v", 4)
    B, Lq, h_q, d = q.shape
    Lk, h_kv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Lk, h_kv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, L_k, h_kv, d] with q's B and d")
    _same(q, (k, "k"), (v, "v"))
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(q.device):  # the library launches on the current device
        st = lib().gqa_prefill_chunk(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Lq,
                                     Lk, h_q, h_kv, d, _dtype_code(q), int(bool(causal)),
                                     float(scale), _stream(q))
    if st != 0:
        raise GQAError(st, "gqa_prefill_chunk")
    return out


def decode_workspace_bytes(B: int, h_q: int, h_kv: int, d: int, num_splits: int = 0) -> int:
    return int(lib().gqa_decode_workspace_bytes(B, h_q, h_kv, d, num_splits))


def decode_default_splits() -> int:
    return int(lib().gqa_decode_default_splits())


def decode(q, k_cache, v_cache, seqlens, *, out=None, workspace=None, num_splits: int = 0):
    _check(q, "q", 4)
    _check(k_cache, "k_cache", 4)
    _check(v_cache, "v_cache", 4)
    _check(seqlens, "seqlens", 1)
    B, one, h_q, d = q.shape
    if one != 1:
        raise ValueError("q must be [B, 1, h_q, d]")
    _, h_kv, S, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, h_kv, S, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, h_kv, S, d] with q's B and d")
    if seqlens.dtype != torch.int32 or seqlens.shape[0] != B:
        raise ValueError("seqlens must be int32 [B]")
    _same(q, (k_cache, "k_cache"), (v_cache, "v_cache"))
    _on_device(q, (seqlens, "seqlens"))
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q)
    need = decode_workspace_bytes(B, h_q, h_kv, d, num_splits)
    workspace = _workspace(workspace, need, q)
    with torch.cuda.device(q.device):  # the library launches on the current device
        st = lib().gqa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                              seqlens.data_ptr(), out.data_ptr(), B, h_q, h_kv, S, d, _dtype_code(q),
                              int(num_splits), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                              _stream(q))
    if st != 0:
        raise GQAError(st, "gqa_decode")
    return out


def decode_noalloc_max_bytes() -> int:
    return int(lib().gqa_decode_noalloc_max_bytes())


def decode_noalloc(q, k_cache, v_cache, seqlens, *, out, num_splits: int = 0):
    """decode() with the library's fixed scratch as its workspace: the call
    allocates nothing (out must be given).  Calls that overlap on one GPU race;
    a call needing more than decode_noalloc_max_bytes() of workspace raises."""
    _check(q, "q", 4)
    _check(k_cache, "k_cache", 4)
    _check(v_cache, "v_cache", 4)
    _check(seqlens, "seqlens", 1)
    B, one, h_q, d = q.shape
    if one != 1:
        raise ValueError("q must be [B, 1, h_q, d]")
    _, h_kv, S, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, h_kv, S, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, h_kv, S, d] with q's B and d")
    if seqlens.dtype != torch.int32 or seqlens.shape[0] != B:
        raise ValueError("seqlens must be int32 [B]")
    _same(q, (k_cache, "k_cache"), (v_cache, "v_cache"))
    _on_device(q, (seqlens, "seqlens"))
    _check_out(out, q)
    with torch.cuda.device(q.device):  # the library launches on the current device
        st = lib().gqa_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                      seqlens.data_ptr(), out.data_ptr(), B, h_q, h_kv, S, d,
                                      _dtype_code(q), int(num_splits), _stream(q))
    if st != 0:
        raise GQAError(st, "gqa_decode_noalloc")
    return out


def decode_append(q, k_new, v_new, k_cache, v_cache, seqlens, *, out=None, workspace=None,
                  num_splits: int = 0):
    """Append the new token's rows at seqlens[b] of the caches (in place), then
    attend over rows [0, seqlens[b] + 1).  q [B,1,h_q,d], k_new/v_new
    [B,1,h_kv,d], caches [B,h_kv,S,d] bf16, seqlens [B] int32 (before the
    append, each < S; not modified) -> o [B,1,h_q,d]."""
    _check(q, "q", 4)
    _check(k_new, "k_new", 4)
    _check(v_new, "v_new", 4)
    _check(k_cache, "k_cache", 4)
    _check(v_cache, "v_cache", 4)
    _check(seqlens, "seqlens", 1)
    B, one, h_q, d = q.shape
    if one != 1:
        raise ValueError("q must be [B, 1, h_q, d]")
    _, h_kv, S, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, h_kv, S, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, h_kv, S, d] with q's B and d")
    if tuple(k_new.shape) != (B, 1, h_kv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [B, 1, h_kv, d]")
    if seqlens.dtype != torch.int32 or seqlens.shape[0] != B:
        raise ValueError("seqlens must be int32 [B]")
    _same(q, (k_cache, "k_cache"), (v_cache, "v_cache"), (k_new, "k_new"), (v_new, "v_new"))
    _on_device(q, (seqlens, "seqlens"))
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q)
    need = decode_workspace_bytes(B, h_q, h_kv, d, num_splits)
    workspace = _workspace(workspace, need, q)
    with torch.cuda.device(q.device):  # the library launches on the current device
        st = lib().gqa_decode_append(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                     k_cache.data_ptr(), v_cache.data_ptr(), seqlens.data_ptr(),
                                     out.data_ptr(), B, h_q, h_kv, S, d, _dtype_code(q),
                                     int(num_splits), workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(), _stream(q))
    if st != 0:
        raise GQAError(st, "gqa_decode_append")
    return out


def _decode_out_ws(q, out, workspace, B, h_q, h_kv, d, num_splits):
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q)
    need = decode_workspace_bytes(B, h_q, h_kv, d, num_splits)
    workspace = _workspace(workspace, need, q)
    return out, workspace


def decode_token_major(q, k_cache, v_cache, seqlens, *, out=None, workspace=None,
                       num_splits: int = 0):
    """Decode over a token-major cache: q [B,1,h_q,d], caches [B,S,h_kv,d] bf16,
    seqlens [B] int32 -> o [B,1,h_q,d]."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _check(t, n, 4)
    _check(seqlens, "seqlens", 1)
    B, one, h_q, d = q.shape
    _, S, h_kv, _ = k_cache.shape
    if one != 1 or tuple(k_cache.shape) != (B, S, h_kv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("need q [B, 1, h_q, d] and caches [B, S, h_kv, d]")
    if seqlens.dtype != torch.int32 or seqlens.shape[0] != B:
        raise ValueError("seqlens must be int32 [B]")
    _same(q, (k_cache, "k_cache"), (v_cache, "v_cache"))
    _on_device(q, (seqlens, "seqlens"))
    out, workspace = _decode_out_ws(q, out, workspace, B, h_q, h_kv, d, num_splits)
    with torch.cuda.device(q.device):  # the library launches on the current device
        st = lib().gqa_decode_token_major(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                          seqlens.data_ptr(), out.data_ptr(), B, h_q, h_kv, S, d,
                                          _dtype_code(q), int(num_splits), workspace.data_ptr(),
                                          workspace.numel() * workspace.element_size(), _stream(q))
    if st != 0:
        raise GQAError(st, "gqa_decode_token_major")
    return out


def decode_paged(q, k_pages, v_pages, block_table, seqlens, *, out=None, workspace=None,
                 num_splits: int = 0):
    """Decode over a paged cache with group-aligned pages: q [B,1,h_q,d], pools
    [num_pages, h_kv, page_size, d] bf16, block_table [B, max_blocks] int32,
    seqlens [B] int32 -> o [B,1,h_q,d]."""
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _check(t, n, 4)
    _check(block_table, "block_table", 2)
    _check(seqlens, "seqlens", 1)
    B, one, h_q, d = q.shape
    _, h_kv, page_size, _ = k_pages.shape
    if one != 1 or k_pages.shape[3] != d or v_pages.shape != k_pages.shape:
        raise ValueError("need q [B, 1, h_q, d] and pools [num_pages, h_kv, page_size, d]")
    if block_table.dtype != torch.int32 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_blocks]")
    if seqlens.dtype != torch.int32 or seqlens.shape[0] != B:
        raise ValueError("seqlens must be int32 [B]")
    _same(q, (k_pages, "k_pages"), (v_pages, "v_pages"))
    _on_device(q, (seqlens, "seqlens"), (block_table, "block_table"))
    out, workspace = _decode_out_ws(q, out, workspace, B, h_q, h_kv, d, num_splits)
    with torch.cuda.device(q.device):  # the library launches on the current device
        st = lib().gqa_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                                    block_table.data_ptr(), seqlens.data_ptr(), out.data_ptr(), B,
                                    h_q, h_kv, page_size, block_table.shape[1], d, _dtype_code(q),
                                    int(num_splits), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream(q))
    if st != 0:
        raise GQAError(st, "gqa_decode_paged")
    return out


def prefill_rope(q, k, v, cos, sin, *, causal: bool, scale=None, out=None, k_rot=None):
    """Prefill with q and k rotated first (bf16).  q [B,L,h_q,d], k/v
    [B,L,h_kv,d], cos/sin [L, d/2] fp32.  Returns (o [B,L,h_q,d], k_rot
    [B,L,h_kv,d]: the rotated keys)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, 4)
    _check(cos, "cos", 2)
    _check(sin, "sin", 2)
    B, L, h_q, d = q.shape
    h_kv = k.shape[2]
    if tuple(k.shape) != (B, L, h_kv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, L, h_kv, d] with q's B, L and d")
    if (cos.dtype != torch.float32 or sin.dtype != torch.float32
            or tuple(cos.shape) != (L, d // 2) or sin.shape != cos.shape):
        raise ValueError("cos and sin must be float32 [L, d/2]")
    _same(q, (k, "k"), (v, "v"))
    _on_device(q, (cos, "cos"), (sin, "sin"))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if k_rot is None:
        k_rot = torch.empty_like(k)
    _check_out(out, q)
    _check_out(k_rot, k, "k_rot")
    with torch.cuda.device(q.device):  # the library launches on the current device
        st = lib().gqa_prefill_rope(q.data_ptr(), k.data_ptr(), v.data_ptr(), cos.data_ptr(),
                                    sin.data_ptr(), out.data_ptr(), k_rot.data_ptr(), B, L, h_q, h_kv,
                                    d, _dtype_code(q), int(bool(causal)), float(scale), _stream(q))
    if st != 0:
        raise GQAError(st, "gqa_prefill_rope")
    return out, k_rot


def prefill_varlen(q, k, v, kv_lens, *, causal: bool, scale=None, out=None):
    """Padded variable-length prefill: q [B,L,h_q,d], k/v [B,L,h_kv,d], kv_lens
    [B] int32 (key j of sequence b visible iff j < kv_lens[b]) -> o."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, 4)
    _check(kv_lens, "kv_lens", 1)
    B, L, h_q, d = q.shape
    h_kv = k.shape[2]
    if tuple(k.shape) != (B, L, h_kv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, L, h_kv, d] with q's B, L and d")
    if kv_lens.dtype != torch.int32 or kv_lens.shape[0] != B:
        raise ValueError("kv_lens must be int32 [B]")
    _same(q, (k, "k"), (v, "v"))
    _on_device(q, (kv_lens, "kv_lens"))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q)
    with torch.cuda.device(q.device):  # the library launches on the current device
        st = lib().gqa_prefill_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      kv_lens.data_ptr(), B, L, h_q, h_kv, d, _dtype_code(q),
                                      int(bool(causal)), float(scale), _stream(q))
    if st != 0:
        raise GQAError(st, "gqa_prefill_varlen")
    return out


def mask_layout(mask: torch.Tensor, B: int, Lq: int, Lk: int):
    """(uint8 tensor, row stride, batch stride) of a keep-mask [B, L_q, L_k] as
    the kernels read it.

    The kernels read each mask row as 16-byte pieces: the row stride (bytes)
    must be a multiple of 16 and at least L_k, the batch stride a multiple of
    16 (0 shares one mask across the batch), and the storage must hold
    (B - 1) * batch stride + L_q * row stride bytes.  A mask laid out that way
    is used in place (a bool mask as its uint8 view); any other is copied into
    rows padded to a multiple of 16 bytes."""
    if mask.dtype not in (torch.bool, torch.uint8):
        raise TypeError("mask must be bool or uint8")
    m = mask.view(torch.uint8) if mask.dtype == torch.bool else mask
    pad = -(-Lk // 16) * 16
    sr = m.stride(1) if Lq > 1 else pad
    sb = m.stride(0) if B > 1 else 0
    ok = (m.stride(2) == 1 or Lk == 1) and sr % 16 == 0 and sr >= Lk and sb % 16 == 0 \
        and sb >= 0 and m.data_ptr() % 16 == 0
    if ok:
        avail = m.untyped_storage().nbytes() - m.storage_offset()
        ok = avail >= (B - 1) * sb + Lq * sr
    if not ok:
        buf = torch.zeros(B, Lq, pad, dtype=torch.uint8, device=m.device)
        buf[..., :Lk] = m
        m, sr, sb = buf, pad, Lq * pad
    return m, sr, sb


def prefill_mask_workspace_bytes(B: int, L_q: int, L_k: int) -> int:
    return int(lib().gqa_prefill_mask_workspace_bytes(B, L_q, L_k))


def prefill_mask(q, k, v, mask, *, causal: bool, scale=None, out=None, workspace=None):
    """Prefill with a keep-mask.  q [B,L_q,h_q,d], k/v [B,L_k,h_kv,d] (L_q <=
    L_k, causal rows bottom-right aligned as in prefill_chunk), mask
    [B,L_q,L_k] or [L_q,L_k] (shared by the batch), bool or uint8 on the GPU:
    key j is visible to query row i of sequence b only where the mask is
    nonzero.  A row with no visible key is zero.  k and v must be finite
    everywhere (a hidden key has weight exactly 0, and 0 * NaN is NaN).
    workspace: a GPU tensor of at least prefill_mask_workspace_bytes(B, L_q,
    L_k) bytes for the mask's summary, or None for a new one.
    -> o [B,L_q,h_q,d]."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, 4)
    B, Lq, h_q, d = q.shape
    Lk, h_kv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Lk, h_kv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, L_k, h_kv, d] with q's B and d")
    _same(q, (k, "k"), (v, "v"))
    if not isinstance(mask, torch.Tensor):
        raise TypeError("mask must be a torch.Tensor")
    if mask.dim() == 2:
        mask = mask.unsqueeze(0).expand(B, Lq, Lk)
    if tuple(mask.shape) != (B, Lq, Lk):
        raise ValueError(f"mask must be [B, L_q, L_k] = {(B, Lq, Lk)} or [L_q, L_k], got "
                         f"{tuple(mask.shape)}")
    if not mask.is_cuda:
        raise ValueError("mask must be on the GPU")
    _on_device(q, (mask, "mask"))
    m, row_stride, batch_stride = mask_layout(mask, B, Lq, Lk)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q)
    need = prefill_mask_workspace_bytes(B, Lq, Lk)
    workspace = _workspace(workspace, need, q)
    with torch.cuda.device(q.device):  # the library launches on the current device
        st = lib().gqa_prefill_mask(q.data_ptr(), k.data_ptr(), v.data_ptr(), m.data_ptr(),
                                    int(row_stride), int(batch_stride), out.data_ptr(), B, Lq, Lk,
                                    h_q, h_kv, d, _dtype_code(q), int(bool(causal)), float(scale),
                                    workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                    _stream(q))
    if st != 0:
        raise GQAError(st, "gqa_prefill_mask")
    return out


def decode_rope_workspace_bytes(B, h_q, h_kv, d, num_splits=0) -> int:
    return int(lib().gqa_decode_rope_workspace_bytes(B, h_q, h_kv, d, num_splits))


def decode_append_rope(q, k_new, v_new, k_cache, v_cache, seqlens, cos, sin, *, out=None,
                       workspace=None, num_splits: int = 0):
    """Decode step with rotary embedding: q [B,1,h_q,d] and k_new [B,1,h_kv,d]
    rotated at position seqlens[b] (tables cos, sin [S, d/2] fp32), the rotated
    key and v_new appended at cache row seqlens[b] (in place), then attend over
    rows [0, seqlens[b] + 1) -> o [B,1,h_q,d]."""
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _check(t, n, 4)
    _check(seqlens, "seqlens", 1)
    _check(cos, "cos", 2)
    _check(sin, "sin", 2)
    B, one, h_q, d = q.shape
    _, h_kv, S, _ = k_cache.shape
    if one != 1 or tuple(k_cache.shape) != (B, h_kv, S, d) or v_cache.shape != k_cache.shape:
        raise ValueError("need q [B, 1, h_q, d] and caches [B, h_kv, S, d]")
    if tuple(k_new.shape) != (B, 1, h_kv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [B, 1, h_kv, d]")
    if (cos.dtype != torch.float32 or sin.dtype != torch.float32
            or tuple(cos.shape) != (S, d // 2) or sin.shape != cos.shape):
        raise ValueError("cos and sin must be float32 [S, d/2]")
    if seqlens.dtype != torch.int32 or seqlens.shape[0] != B:
        raise ValueError("seqlens must be int32 [B]")
    _same(q, (k_cache, "k_cache"), (v_cache, "v_cache"), (k_new, "k_new"), (v_new, "v_new"))
    _on_device(q, (seqlens, "seqlens"), (cos, "cos"), (sin, "sin"))
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q)
    need = decode_rope_workspace_bytes(B, h_q, h_kv, d, num_splits)
    workspace = _workspace(workspace, need, q)
    with torch.cuda.device(q.device):  # the library launches on the current device
        st = lib().gqa_decode_append_rope(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                          k_cache.data_ptr(), v_cache.data_ptr(), seqlens.data_ptr(),
                                          cos.data_ptr(), sin.data_ptr(), out.data_ptr(), B, h_q, h_kv,
                                          S, d, _dtype_code(q), int(num_splits), workspace.data_ptr(),
                                          workspace.numel() * workspace.element_size(), _stream(q))
    if st != 0:
        raise GQAError(st, "gqa_decode_append_rope")
    return out
