"""Seeded synthetic inputs and the workload table for the GQA core.

This module only draws random numbers and casts them; it holds none of the
attention arithmetic.  Both the oracle-side tests and the GPU-side tests and
benchmark take their inputs from here, so the two sides see identical bytes.

Recipe (one fixed rule for every workload):

* a CPU ``torch.Generator`` seeded with the workload's seed;
* draws in float32 with ``torch.randn`` in the order q, k, v (decode: the
  per-sequence lengths first, with ``torch.randint`` over [lo, hi] inclusive,
  then q, k_cache, v_cache; decode with append: then also k_new, v_new);
* a standard deviation other than 1 is applied in float32 before the cast;
* the cast to bfloat16 is torch's round-to-nearest-even.

The chunked prefill runs the last 2048 of 32768 positions of the 64/8-head
shape against all 32768 keys, the exact form of processing a long sequence
chunk by chunk ("Implementing GQA from scratch", §4.3; "What is Grouped-Query
Attention", §3.2).

Shapes follow the pages' workloads: the worked example of "Implementing GQA
from scratch" (§5: B=32, L=1024, 8 heads, d_model=512, 4 key/value heads), the
Llama-2-7B style 32/8 head split with d=128 ("What is Grouped-Query
Attention", §2.3 and §3.4), the A100 prefill length 4096 and the Qwen2-72B
64/8 head split ("Attention in Qwen, DeepSeek and LLaMA3", §2.2 and §2.3), at
32K context.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    # "prefill", "prefill_chunk", "prefill_rope", "prefill_varlen", "prefill_mask",
    # "decode", "decode_append" or "decode_paged"
    path: str
    dtype: str  # "f32" or "bf16"
    B: int
    h_q: int
    h_kv: int
    d: int
    L: int = 1  # prefill sequence length (prefill_chunk: the new positions L_q)
    Lk: int = 0  # prefill_chunk: keys per sequence L_k (the new positions are the last L_q)
    S: int = 0  # decode cache capacity
    causal: bool = False
    std: float = 1.0
    # decode: inclusive [lo, hi] of the lengths (decode_append: before the append);
    # prefill_varlen: of the valid lengths in the padded batch; prefill_mask: of
    # the packed documents' lengths
    seqlen_range: tuple = (0, 0)
    seed: int = 0
    page_size: int = 0  # decode_paged: rows per page
    description: str = field(default="", compare=False)

    @property
    def G(self) -> int:
        return self.h_q // self.h_kv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    "tiny_prefill_f32": Workload(
        "tiny_prefill_f32", "prefill", "f32", B=1, L=128, h_q=8, h_kv=2, d=64, causal=True,
        std=1.0, seed=1,
        description="tiny fp32 causal prefill, B=1 L=128 h_q=8 h_kv=2 d=64"),
    "worked_example_prefill_bf16": Workload(
        "worked_example_prefill_bf16", "prefill", "bf16", B=32, L=1024, h_q=8, h_kv=4, d=64,
        causal=False, std=1.0, seed=2,
        description="bf16 non-causal prefill, B=32 L=1024 h_q=8 h_kv=4 d=64"),
    "llama2_7b_prefill_bf16": Workload(
        "llama2_7b_prefill_bf16", "prefill", "bf16", B=1, L=4096, h_q=32, h_kv=8, d=128,
        causal=True, std=1.0 / math.sqrt(2.0), seed=3,
        description="bf16 causal prefill, B=1 L=4096 h_q=32 h_kv=8 d=128"),
    "batched_decode_bf16": Workload(
        "batched_decode_bf16", "decode", "bf16", B=64, h_q=32, h_kv=8, d=128, S=8192,
        std=1.0, seqlen_range=(1024, 8192), seed=4,
        description="bf16 decode, B=64 h_q=32 h_kv=8 d=128 S=8192 lengths U{1024..8192}"),
    "long_context_prefill_bf16": Workload(
        "long_context_prefill_bf16", "prefill", "bf16", B=1, L=32768, h_q=64, h_kv=8, d=128,
        causal=True, std=1.0 / math.sqrt(2.0), seed=5,
        description="bf16 causal prefill, B=1 L=32768 h_q=64 h_kv=8 d=128"),
    "chunked_prefill_bf16": Workload(
        "chunked_prefill_bf16", "prefill_chunk", "bf16", B=1, L=2048, Lk=32768, h_q=64, h_kv=8,
        d=128, causal=True, std=1.0 / math.sqrt(2.0), seed=6,
        description="bf16 causal chunked prefill: the last 2048 of 32768 positions, "
                    "B=1 h_q=64 h_kv=8 d=128"),
    "batched_decode_append_bf16": Workload(
        "batched_decode_append_bf16", "decode_append", "bf16", B=64, h_q=32, h_kv=8, d=128,
        S=8192, std=1.0, seqlen_range=(1023, 8191), seed=7,
        description="bf16 decode with the new token's key/value appended, B=64 h_q=32 h_kv=8 "
                    "d=128 S=8192 lengths U{1023..8191} before the append"),
    "llama2_7b_prefill_rope_bf16": Workload(
        "llama2_7b_prefill_rope_bf16", "prefill_rope", "bf16", B=1, L=4096, h_q=32, h_kv=8,
        d=128, causal=True, std=1.0 / math.sqrt(2.0), seed=3,
        description="bf16 causal prefill with rotary embedding (tables for base 10000), "
                    "B=1 L=4096 h_q=32 h_kv=8 d=128"),
    "varlen_prefill_bf16": Workload(
        "varlen_prefill_bf16", "prefill_varlen", "bf16", B=16, L=2048, h_q=32, h_kv=8, d=128,
        causal=True, std=1.0 / math.sqrt(2.0), seqlen_range=(128, 2048), seed=8,
        description="bf16 causal prefill of a padded batch, B=16 L=2048 lengths U{128..2048} "
                    "h_q=32 h_kv=8 d=128"),
    "long_context_group_prefill_bf16": Workload(
        "long_context_group_prefill_bf16", "prefill", "bf16", B=1, L=32768, h_q=8, h_kv=1, d=128,
        causal=True, std=1.0 / math.sqrt(2.0), seed=9,
        description="bf16 causal prefill of one key/value group of the long-context shape "
                    "(an eighth of its heads), B=1 L=32768 h_q=8 h_kv=1 d=128"),
    "batched_decode_paged_bf16": Workload(
        "batched_decode_paged_bf16", "decode_paged", "bf16", B=64, h_q=32, h_kv=8, d=128,
        S=8192, std=1.0, seqlen_range=(1024, 8192), seed=4, page_size=64,
        description="bf16 decode over a paged cache: the batched-decode inputs in a shuffled "
                    "pool of 64-row group-aligned pages"),
    "document_masked_prefill_bf16": Workload(
        "document_masked_prefill_bf16", "prefill_mask", "bf16", B=1, L=4096, h_q=32, h_kv=8,
        d=128, causal=True, std=1.0 / math.sqrt(2.0), seqlen_range=(128, 1024), seed=10,
        description="bf16 causal prefill with a keep-mask: documents of lengths U{128..1024} "
                    "packed into one sequence, each position seeing only its own document, "
                    "B=1 L=4096 h_q=32 h_kv=8 d=128"),
}

# Order in which the workloads are listed everywhere: the five of the core
# path, then the chunked prefill against existing keys, the decode that
# appends the new token's key/value rows itself and the decode over pages.
WORKLOAD_ORDER = ["tiny_prefill_f32", "worked_example_prefill_bf16", "llama2_7b_prefill_bf16",
                  "batched_decode_bf16", "long_context_prefill_bf16", "chunked_prefill_bf16",
                  "batched_decode_append_bf16", "batched_decode_paged_bf16",
                  "llama2_7b_prefill_rope_bf16", "varlen_prefill_bf16",
                  "long_context_group_prefill_bf16", "document_masked_prefill_bf16"]


def _draw(gen, shape, std, dtype):
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(torch.tensor(std, dtype=torch.float32))
    return x.to(dtype)


def prefill_inputs(B, L, h_q, h_kv, d, seed, std=1.0, dtype=torch.bfloat16):
    """Seeded CPU tensors q [B,L,h_q,d], k, v [B,L,h_kv,d] of the given dtype."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    q = _draw(gen, (B, L, h_q, d), std, dtype)
    k = _draw(gen, (B, L, h_kv, d), std, dtype)
    v = _draw(gen, (B, L, h_kv, d), std, dtype)
    return q, k, v


def prefill_chunk_inputs(B, Lq, Lk, h_q, h_kv, d, seed, std=1.0, dtype=torch.bfloat16):
    """Seeded CPU tensors q [B,Lq,h_q,d] (the last Lq positions), k, v [B,Lk,h_kv,d]."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    q = _draw(gen, (B, Lq, h_q, d), std, dtype)
    k = _draw(gen, (B, Lk, h_kv, d), std, dtype)
    v = _draw(gen, (B, Lk, h_kv, d), std, dtype)
    return q, k, v


def decode_inputs(B, h_q, h_kv, S, d, seed, seqlen_range, std=1.0, dtype=torch.bfloat16):
    """Seeded CPU tensors: seqlens [B] int32, q [B,1,h_q,d], k_cache, v_cache [B,h_kv,S,d]."""
    lo, hi = seqlen_range
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    seqlens = torch.randint(lo, hi + 1, (B,), generator=gen, dtype=torch.int64).to(torch.int32)
    q = _draw(gen, (B, 1, h_q, d), std, dtype)
    k_cache = _draw(gen, (B, h_kv, S, d), std, dtype)
    v_cache = _draw(gen, (B, h_kv, S, d), std, dtype)
    return seqlens, q, k_cache, v_cache


def decode_append_inputs(B, h_q, h_kv, S, d, seed, seqlen_range, std=1.0,
                         dtype=torch.bfloat16):
    """decode_inputs' tensors (lengths before the append), then the new token's
    k_new, v_new [B,1,h_kv,d] drawn from the same generator after them."""
    lo, hi = seqlen_range
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    seqlens = torch.randint(lo, hi + 1, (B,), generator=gen, dtype=torch.int64).to(torch.int32)
    q = _draw(gen, (B, 1, h_q, d), std, dtype)
    k_cache = _draw(gen, (B, h_kv, S, d), std, dtype)
    v_cache = _draw(gen, (B, h_kv, S, d), std, dtype)
    k_new = _draw(gen, (B, 1, h_kv, d), std, dtype)
    v_new = _draw(gen, (B, 1, h_kv, d), std, dtype)
    return seqlens, q, k_new, v_new, k_cache, v_cache


def rope_tables(L, d, base=10000.0):
    """cos, sin [L, d/2] float32 for the angles p * base^(-2i/d) (position p,
    pair i), evaluated in float64 and rounded to float32: the input tables of a
    rotary embedding, as a model would pass them."""
    pos = torch.arange(L, dtype=torch.float64)[:, None]
    freq = base ** (-2.0 * torch.arange(d // 2, dtype=torch.float64) / d)
    ang = pos * freq[None, :]
    return torch.cos(ang).to(torch.float32), torch.sin(ang).to(torch.float32)


def to_pages(k_cache, v_cache, seqlens, page_size, seed, spare=0):
    """Move head-major caches [B, h_kv, S, d] into a pool of group-aligned pages.

    Returns (k_pages, v_pages [num_pages, h_kv, page_size, d], block_table
    [B, max_blocks] int32).  The pages a sequence needs (ceil(len / page_size))
    take physical slots in a seeded random order; ``spare`` extra pages are
    left over.  Rows of a page past the sequence end, spare pages and table
    entries past a sequence's last block hold zeros (table: -1).  Pure data
    movement: no arithmetic of the method.
    """
    B, h_kv, S, d = k_cache.shape
    max_blocks = -(-S // page_size)
    need = [-(-int(n) // page_size) for n in seqlens.tolist()]
    num_pages = sum(need) + spare
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    perm = torch.randperm(num_pages, generator=gen)
    k_pages = torch.zeros(num_pages, h_kv, page_size, d, dtype=k_cache.dtype)
    v_pages = torch.zeros_like(k_pages)
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    nxt = 0
    for b, n in enumerate(seqlens.tolist()):
        for i in range(need[b]):
            page = int(perm[nxt])
            nxt += 1
            table[b, i] = page
            rows = min(page_size, n - i * page_size)
            k_pages[page, :, :rows] = k_cache[b, :, i * page_size:i * page_size + rows]
            v_pages[page, :, :rows] = v_cache[b, :, i * page_size:i * page_size + rows]
    return k_pages, v_pages, table


def document_lengths(L, lo, hi, seed):
    """Lengths of documents packed into L positions: draws U{lo..hi} from a
    generator seeded ``seed`` until they cover L, the last one cut to fit."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    lens, total = [], 0
    while total < L:
        n = int(torch.randint(lo, hi + 1, (1,), generator=gen))
        n = min(n, L - total)
        lens.append(n)
        total += n
    return lens


def document_mask(lens):
    """uint8 [L, L] keep-mask of packed documents: 1 where row and column lie
    in the same document (a block-diagonal pattern; pure data layout)."""
    L = sum(lens)
    doc = torch.repeat_interleave(torch.arange(len(lens)), torch.tensor(lens))
    return (doc[:, None] == doc[None, :]).to(torch.uint8).reshape(L, L)


def random_mask(shape, density, seed):
    """uint8 keep-mask of the given shape, each byte 1 with probability density."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    return (torch.rand(*shape, generator=gen) < density).to(torch.uint8)


def workload_inputs(w: Workload):
    """Inputs of a named workload, as CPU tensors (see prefill_inputs/decode_inputs)."""
    if w.path == "prefill":
        return prefill_inputs(w.B, w.L, w.h_q, w.h_kv, w.d, w.seed, w.std, w.torch_dtype())
    if w.path == "prefill_chunk":
        return prefill_chunk_inputs(w.B, w.L, w.Lk, w.h_q, w.h_kv, w.d, w.seed, w.std,
                                    w.torch_dtype())
    if w.path == "prefill_varlen":
        q, k, v = prefill_inputs(w.B, w.L, w.h_q, w.h_kv, w.d, w.seed, w.std, w.torch_dtype())
        lo, hi = w.seqlen_range
        gen = torch.Generator(device="cpu").manual_seed(int(w.seed) + 1000)
        lens = torch.randint(lo, hi + 1, (w.B,), generator=gen, dtype=torch.int64)
        return q, k, v, lens.to(torch.int32)
    if w.path == "prefill_mask":
        q, k, v = prefill_inputs(w.B, w.L, w.h_q, w.h_kv, w.d, w.seed, w.std, w.torch_dtype())
        lo, hi = w.seqlen_range
        masks = [document_mask(document_lengths(w.L, lo, hi, w.seed + 1000 + b))
                 for b in range(w.B)]
        return q, k, v, torch.stack(masks)
    if w.path == "prefill_rope":
        q, k, v = prefill_inputs(w.B, w.L, w.h_q, w.h_kv, w.d, w.seed, w.std, w.torch_dtype())
        cos, sin = rope_tables(w.L, w.d)
        return q, k, v, cos, sin
    if w.path == "decode_paged":
        seqlens, q, kc, vc = decode_inputs(w.B, w.h_q, w.h_kv, w.S, w.d, w.seed, w.seqlen_range,
                                           w.std, w.torch_dtype())
        kp, vp, table = to_pages(kc, vc, seqlens, w.page_size, w.seed + 1000)
        return seqlens, q, kp, vp, table
    if w.path == "decode_append":
        return decode_append_inputs(w.B, w.h_q, w.h_kv, w.S, w.d, w.seed, w.seqlen_range, w.std,
                                    w.torch_dtype())
    return decode_inputs(w.B, w.h_q, w.h_kv, w.S, w.d, w.seed, w.seqlen_range, w.std,
                         w.torch_dtype())


def sample_rows(n, B, L, h_q, seed, include=()):
    """Seeded (b, i, h) triples for sampled checks, sorted by (b, h, i).

    ``include`` adds fixed triples (for example the first and last position).
    """
    gen = torch.Generator(device="cpu").manual_seed(int(seed) + 1000003)
    b = torch.randint(0, B, (n,), generator=gen)
    i = torch.randint(0, L, (n,), generator=gen)
    h = torch.randint(0, h_q, (n,), generator=gen)
    rows = {(int(x), int(y), int(z)) for x, y, z in zip(b, i, h)}
    rows.update(tuple(int(t) for t in r) for r in include)
    return sorted(rows, key=lambda r: (r[0], r[2], r[1]))
