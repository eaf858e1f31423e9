"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Both sides see the same seeded inputs from ``gqa_workloads``; the oracle gets
the exact values the GPU received (bf16 upcast exactly to float64).

Tolerances (whole compared tensor): fp32 max-abs <= 1e-4; bf16 max-abs <= 2e-2
and relative L2 <= 1e-2.  Small shapes are compared in full (several tiles,
ragged tails, every group size class).  The named workloads run at their full
sizes in the launch configuration the benchmark times: the worked example, the
Llama-2-shaped layer (plain and rotary), the packed-documents keep-mask prefill
and every decode workload are compared in full (decode: every sequence, 8 at a
time); the 32K-position workloads, the chunked and the padded variable-length
prefill are compared on one seeded row of every work-group plus seeded samples,
and are checked for every output written.
"""
import math

import numpy as np
import pytest
import torch

import gqa_workloads as wl
import grouped_query_attention_03_amd as gqa
import oracle

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_MAXABS = 2e-2
BF16_RELL2 = 1e-2


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def check(out, ref, dtype, what):
    o = np.asarray(out, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert o.shape == r.shape, f"{what}: shape {o.shape} vs {r.shape}"
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - r)
    maxabs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(o - r) / max(np.linalg.norm(r), 1e-300))
    say(f"  {what}: max-abs {maxabs:.3e} rel-L2 {rel:.3e}")
    if dtype == "f32":
        assert maxabs <= F32_TOL, f"{what}: max-abs {maxabs:.3e} > {F32_TOL}"
    else:
        assert maxabs <= BF16_MAXABS, f"{what}: max-abs {maxabs:.3e} > {BF16_MAXABS}"
        assert rel <= BF16_RELL2, f"{what}: rel-L2 {rel:.3e} > {BF16_RELL2}"


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def run_prefill(q, k, v, causal, scale, dev):
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.full_like(qd, float("nan"))  # every element must be overwritten
    gqa.prefill(qd, kd, vd, causal=causal, scale=scale, out=out)
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------------ prefill, full

PREFILL_SMALL = [
    # B, L, h_q, h_kv, d, dtype, causal
    (1, 128, 8, 2, 64, "f32", True),       # the tiny fp32 workload's shape
    (2, 77, 4, 4, 128, "f32", True),
    (1, 300, 6, 2, 64, "f32", False),
    (1, 1, 8, 1, 128, "f32", True),
    (2, 300, 8, 2, 128, "bf16", True),     # G = 4, ragged tail
    (1, 257, 8, 4, 64, "bf16", False),     # G = 2
    (1, 1000, 16, 2, 128, "bf16", True),   # G = 8
    (1, 129, 16, 1, 64, "bf16", True),     # G = 16 (MQA), two work-groups per group
    (2, 17, 4, 4, 128, "bf16", False),     # MHA
    (1, 1, 8, 2, 128, "bf16", True),       # L = 1
    (1, 200, 6, 2, 128, "bf16", True),     # G = 3
    (1, 150, 12, 2, 64, "bf16", False),    # G = 6
    (3, 64, 8, 8, 64, "bf16", True),       # exactly one tile
    (1, 513, 32, 8, 128, "bf16", True),
    (2, 99, 3, 1, 64, "bf16", True),       # G = 3 (odd: one head per work-group), d = 64
    (1, 161, 10, 2, 128, "bf16", False),   # G = 5, ragged tail, non-causal
    (3, 65, 8, 2, 64, "bf16", True),       # one full tile plus one key, three sequences
    (1, 2, 64, 8, 128, "bf16", True),      # L = 2 with G = 8: every wave but one past the end
]


@pytest.mark.parametrize("case", PREFILL_SMALL, ids=lambda c: "B{}_L{}_hq{}_hkv{}_d{}_{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_prefill_matches_oracle(case, dev):
    B, L, h_q, h_kv, d, dtype, causal = case
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    std = 1.0 if dtype == "f32" else 1 / math.sqrt(2)
    seed = 1000 + 7 * L + h_q
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, seed, std, tdt)
    scale = 1 / math.sqrt(d)
    say(f"prefill {case} seed {seed}")
    out = run_prefill(q, k, v, causal, scale, dev)
    ref = oracle.prefill(f64(q), f64(k), f64(v), causal=causal, scale=scale)
    check(f64(out), ref, dtype, f"prefill {case}")


def test_prefill_non_default_scale(dev):
    q, k, v = wl.prefill_inputs(1, 190, 8, 2, 128, 77, 1.0, torch.bfloat16)
    say("prefill scale 0.05 B1 L190 8/2 d128")
    out = run_prefill(q, k, v, True, 0.05, dev)
    check(f64(out), oracle.prefill(f64(q), f64(k), f64(v), causal=True, scale=0.05), "bf16",
          "prefill scale 0.05")


def test_prefill_causal_row0_is_v0_exactly(dev):
    B, L, h_q, h_kv, d = 2, 100, 8, 2, 128
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, 31, 1.0, torch.bfloat16)
    say("prefill causal row 0")
    out = run_prefill(q, k, v, True, 1 / math.sqrt(d), dev).cpu()
    for h in range(h_q):
        assert torch.equal(out[:, 0, h], v[:, 0, h // (h_q // h_kv)])


def test_prefill_is_deterministic(dev):
    q, k, v = wl.prefill_inputs(1, 700, 16, 4, 128, 32, 1.0, torch.bfloat16)
    say("prefill determinism")
    o1 = run_prefill(q, k, v, True, 0.088, dev)
    o2 = run_prefill(q, k, v, True, 0.088, dev)
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("scale_kind", ["default", "power_of_two"])
def test_prefill_running_max_jumps(d, causal, scale_kind, dev):
    """Keys that grow along the sequence, plus one spike key, so a row's max
    rises by more than the lazy-rescale threshold in later tiles, and for most
    rows once by far more than the fp32 exponent range (2^128): the rescale
    and the recomputed-tile paths of the online softmax must agree with the
    plain row softmax, for scores of hundreds of log2 units.

    At the default scale 1/sqrt(d) the kernel multiplies the fp32 scores by
    scale*log2(e); at scale = ln(2)/8 that factor is 1/8, a power of two, and
    the kernel folds it into q instead (exact in bf16): both must match."""
    B, L, h_q, h_kv = 1, 700, 8, 2
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, 35 + d, 1 / math.sqrt(2), torch.bfloat16)
    grow = 1.0 + torch.arange(L, dtype=torch.float32) / 40.0
    grow[517] *= 60.0
    k = (k.float() * grow[None, :, None, None]).to(torch.bfloat16)
    scale = 1 / math.sqrt(d) if scale_kind == "default" else math.log(2) / 8
    say(f"prefill rising keys d{d} causal={causal} scale={scale}")
    out = run_prefill(q, k, v, causal, scale, dev)
    ref = oracle.prefill(f64(q), f64(k), f64(v), causal=causal, scale=scale)
    check(f64(out), ref, "bf16", f"prefill rising keys d{d} scale {scale_kind}")


def test_prefill_head_map_discriminates(dev):
    """Key/value head 0 has all-zero keys, so heads 0..G-1 must return running means of V0."""
    B, L, h_q, h_kv, d = 1, 96, 8, 2, 64
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, 33, 1.0, torch.bfloat16)
    k[:, :, 0] = 0
    say("prefill head-map discriminator")
    out = f64(run_prefill(q, k, v, True, 0.125, dev))
    v0 = f64(v)[:, :, 0]
    running_mean = np.cumsum(v0, axis=1) / np.arange(1, L + 1)[None, :, None]
    for h in range(h_q // h_kv):
        check(out[:, :, h], running_mean, "bf16", f"head {h} reads kv head 0")
    check(out, oracle.prefill(f64(q), f64(k), f64(v), causal=True, scale=0.125), "bf16",
          "head-map case vs oracle")


# ---------------------------------------------------------- named workloads, full size

def workgroup_rows(B, L, h_q, h_kv, seed):
    """One seeded (b, i, h) row from every prefill work-group: a work-group
    holds GW query heads of one group (GW the largest power of two dividing
    G, at most 8) times 256 / GW consecutive positions."""
    G = h_q // h_kv
    gw = 1
    while gw < 8 and G % (2 * gw) == 0:
        gw *= 2
    bm = 256 // gw
    gen = torch.Generator().manual_seed(int(seed) + 77)
    rows = []
    for b in range(B):
        for kvh in range(h_kv):
            for sub in range(G // gw):
                for p0 in range(0, L, bm):
                    n = min(bm, L - p0)
                    i = p0 + int(torch.randint(0, n, (1,), generator=gen))
                    h = kvh * G + sub * gw + int(torch.randint(0, gw, (1,), generator=gen))
                    rows.append((b, i, h))
    return rows


def _full_prefill(name, dev):
    """A named workload compared in full: every output row against the oracle."""
    w = wl.WORKLOADS[name]
    q, k, v = wl.workload_inputs(w)
    say(f"prefill workload {name} ({w.description}) seed {w.seed}: every row")
    out = run_prefill(q, k, v, w.causal, w.scale, dev)
    ref = oracle.prefill(f64(q), f64(k), f64(v), causal=w.causal, scale=w.scale)
    check(f64(out), ref, w.dtype, f"{name}: all {out.numel() // w.d} rows")


def _sampled_prefill(name, n_rows, dev):
    w = wl.WORKLOADS[name]
    q, k, v = wl.workload_inputs(w)
    say(f"prefill workload {name} ({w.description}) seed {w.seed}")
    out = run_prefill(q, k, v, w.causal, w.scale, dev)
    # seeded rows, the corners, and one row of every work-group
    rows = wl.sample_rows(n_rows, w.B, w.L, w.h_q, w.seed,
                          include=[(0, 0, 0), (w.B - 1, w.L - 1, w.h_q - 1), (0, w.L - 1, 0),
                                   *workgroup_rows(w.B, w.L, w.h_q, w.h_kv, w.seed)])
    idx = torch.tensor(rows)
    q_rows = q[idx[:, 0], idx[:, 1], idx[:, 2]]
    o_rows = out.cpu()[idx[:, 0], idx[:, 1], idx[:, 2]]
    ref = oracle.prefill_rows(f64(q_rows), rows, f64(k), f64(v), w.h_q, causal=w.causal,
                              scale=w.scale)
    check(f64(o_rows), ref, w.dtype, f"{name}: {len(rows)} sampled rows")
    assert not torch.isnan(out).any(), f"{name}: output not fully written"


def test_workload_tiny_prefill_f32_full(dev):
    w = wl.WORKLOADS["tiny_prefill_f32"]
    q, k, v = wl.workload_inputs(w)
    say(f"prefill workload {w.name}")
    out = run_prefill(q, k, v, w.causal, w.scale, dev)
    check(f64(out), oracle.prefill(f64(q), f64(k), f64(v), causal=w.causal, scale=w.scale),
          "f32", w.name)


def test_workload_worked_example_prefill(dev):
    _full_prefill("worked_example_prefill_bf16", dev)


def test_workload_llama2_prefill(dev):
    _full_prefill("llama2_7b_prefill_bf16", dev)


def test_workload_long_context_prefill(dev):
    _sampled_prefill("long_context_prefill_bf16", 96, dev)


def test_workload_long_context_group_prefill(dev):
    """One key/value group of the long-context shape: the share of one device
    when the heads are split by group (G = 8, a single key/value head)."""
    _sampled_prefill("long_context_group_prefill_bf16", 128, dev)


# ------------------------------------------------ prefill against existing keys

def run_prefill_chunk(q, k, v, causal, scale, dev):
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.full_like(qd, float("nan"))
    gqa.prefill_chunk(qd, kd, vd, causal=causal, scale=scale, out=out)
    torch.cuda.synchronize()
    return out


CHUNK_SMALL = [
    # B, L_q, L_k, h_q, h_kv, d, dtype, causal
    (1, 1, 200, 8, 2, 128, "bf16", True),      # one new token
    (2, 70, 300, 8, 4, 64, "bf16", True),      # ragged chunk and keys
    (1, 64, 128, 8, 1, 64, "bf16", True),      # tile-aligned, MQA
    (1, 33, 1000, 32, 8, 128, "bf16", False),
    (1, 129, 129, 16, 2, 128, "bf16", True),   # L_q == L_k
    (1, 250, 251, 6, 2, 128, "bf16", True),    # G = 3
    (2, 17, 80, 4, 4, 64, "f32", True),
    (1, 50, 77, 8, 2, 128, "f32", False),
]


@pytest.mark.parametrize("case", CHUNK_SMALL, ids=lambda c: "B{}_Lq{}_Lk{}_hq{}_hkv{}_d{}_{}_c{}".format(*c))
def test_prefill_chunk_matches_oracle(case, dev):
    B, Lq, Lk, h_q, h_kv, d, dt, causal = case
    seed = 3000 + Lq + Lk + h_q
    dtype = torch.float32 if dt == "f32" else torch.bfloat16
    q, k, v = wl.prefill_chunk_inputs(B, Lq, Lk, h_q, h_kv, d, seed, dtype=dtype)
    say(f"prefill_chunk {case} seed {seed}")
    out = run_prefill_chunk(q, k, v, causal, 1 / math.sqrt(d), dev)
    ref = oracle.prefill_cached(f64(q), f64(k), f64(v), causal, 1 / math.sqrt(d))
    check(f64(out), ref, dt, f"prefill_chunk {case}")


def test_prefill_chunk_square_is_prefill(dev):
    # the same kernel and work map: bit-identical results
    q, k, v = wl.prefill_inputs(1, 300, 8, 2, 128, 3100)
    say("prefill_chunk square vs prefill")
    a = run_prefill(q, k, v, True, 0.09, dev)
    b = run_prefill_chunk(q, k, v, True, 0.09, dev)
    assert torch.equal(a, b)


def test_chunked_prefill_reproduces_full_prefill(dev):
    # run one sequence chunk by chunk against the keys so far: every chunk's
    # rows must match the full causal prefill's rows (oracle) to tolerance
    B, L, h_q, h_kv, d = 1, 700, 16, 4, 128
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, 3200)
    say("chunked prefill vs full causal prefill")
    ref = oracle.prefill(f64(q), f64(k), f64(v), causal=True, scale=1 / math.sqrt(d))
    parts = []
    for c0, c1 in ((0, 100), (100, 101), (101, 356), (356, 700)):
        parts.append(run_prefill_chunk(q[:, c0:c1].contiguous(), k[:, :c1].contiguous(),
                                       v[:, :c1].contiguous(), True, 1 / math.sqrt(d), dev).cpu())
    check(f64(torch.cat(parts, dim=1)), ref, "bf16", "chunked vs full causal prefill")


def test_workload_chunked_prefill(dev):
    w = wl.WORKLOADS["chunked_prefill_bf16"]
    q, k, v = wl.workload_inputs(w)
    say(f"prefill_chunk workload {w.name} ({w.description}) seed {w.seed}")
    out = run_prefill_chunk(q, k, v, w.causal, w.scale, dev)
    rows = wl.sample_rows(96, w.B, w.L, w.h_q, w.seed,
                          include=[(0, 0, 0), (0, w.L - 1, w.h_q - 1),
                                   *workgroup_rows(w.B, w.L, w.h_q, w.h_kv, w.seed)])
    idx = torch.tensor(rows)
    q_rows = q[idx[:, 0], idx[:, 1], idx[:, 2]]
    o_rows = out.cpu()[idx[:, 0], idx[:, 1], idx[:, 2]]
    ref = oracle.prefill_cached_rows(f64(q_rows), rows, f64(k), f64(v), w.h_q, w.L, w.causal,
                                     w.scale)
    check(f64(o_rows), ref, w.dtype, f"{w.name}: {len(rows)} sampled rows")
    assert not torch.isnan(out).any(), f"{w.name}: output not fully written"


# ------------------------------------------------------------------------- decode

def run_decode(seqlens, q, kc, vc, dev, splits=0, out_fill=float("nan")):
    qd, kd, vd, sd = q.to(dev), kc.to(dev), vc.to(dev), seqlens.to(dev)
    out = torch.full_like(qd, out_fill)
    gqa.decode(qd, kd, vd, sd, out=out, num_splits=splits)
    torch.cuda.synchronize()
    return out


def decode_ref(seqlens, q, kc, vc, bsel=None):
    if bsel is None:
        bsel = list(range(q.shape[0]))
    bi = torch.tensor(bsel)
    return oracle.decode(f64(q[bi, 0]), f64(kc[bi]), f64(vc[bi]), seqlens[bi].numpy())


def test_workload_batched_decode(dev):
    w = wl.WORKLOADS["batched_decode_bf16"]
    seqlens, q, kc, vc = wl.workload_inputs(w)
    say(f"decode workload {w.name} ({w.description}) total keys {int(seqlens.sum())}")
    out = run_decode(seqlens, q, kc, vc, dev).cpu()
    assert not torch.isnan(out).any()
    # every sequence, 8 at a time (bounds the fp64 copies of the caches)
    refs = [decode_ref(seqlens, q, kc, vc, list(range(b0, min(b0 + 8, w.B))))
            for b0 in range(0, w.B, 8)]
    check(f64(out[:, 0]), np.concatenate(refs), "bf16", f"{w.name}: all {w.B} sequences")


def test_decode_reuses_one_workspace(dev):
    """One workspace serves many calls: its contents on entry are ignored, so a
    second, smaller call (other lengths, fewer sequences, a zero length) and a
    repeat of the first give the results of fresh workspaces, bit for bit,
    also when the workspace starts out full of NaN bytes."""
    B, h_q, h_kv, S, d = 6, 32, 8, 1100, 128
    need = gqa.decode_workspace_bytes(B, h_q, h_kv, d)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)
    s1, q1, k1, v1 = wl.decode_inputs(B, h_q, h_kv, S, d, 4100, (1, S))
    s2, q2, k2, v2 = wl.decode_inputs(3, h_q, h_kv, S, d, 4101, (1, S))
    s2[0] = 0
    q1d, k1d, v1d, s1d = q1.to(dev), k1.to(dev), v1.to(dev), s1.to(dev)
    q2d, k2d, v2d, s2d = q2.to(dev), k2.to(dev), v2.to(dev), s2.to(dev)
    say("decode: repeated calls on one workspace")
    fresh1 = gqa.decode(q1d, k1d, v1d, s1d)
    fresh2 = gqa.decode(q2d, k2d, v2d, s2d)
    for rep in range(3):
        a = gqa.decode(q1d, k1d, v1d, s1d, workspace=ws)
        b = gqa.decode(q2d, k2d, v2d, s2d, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(a, fresh1), f"call {2 * rep} differs from a fresh workspace"
        assert torch.equal(b, fresh2), f"call {2 * rep + 1} differs from a fresh workspace"
    assert torch.equal(fresh2[0].cpu(), torch.zeros_like(fresh2[0].cpu()))
    check(f64(fresh1.cpu()[:, 0]), decode_ref(s1, q1, k1, v1), "bf16", "decode reusing a workspace")


DECODE_SMALL = [
    # B, h_q, h_kv, S, d, seqlens
    (6, 32, 8, 1100, 128, [0, 1, 511, 512, 513, 1100]),
    (3, 8, 8, 700, 64, [700, 64, 65]),        # G = 1
    (2, 32, 1, 300, 128, [300, 17]),          # G = 32: two query-head subgroups
    (2, 16, 2, 1000, 64, [999, 1000]),        # G = 8
    (4, 12, 4, 96, 128, [96, 95, 33, 32]),    # G = 3
]


@pytest.mark.parametrize("case", DECODE_SMALL, ids=lambda c: "B{}_hq{}_hkv{}_S{}_d{}".format(*c[:5]))
def test_decode_matches_oracle(case, dev):
    B, h_q, h_kv, S, d, lens = case
    seed = 2000 + S + h_q
    _, q, kc, vc = wl.decode_inputs(B, h_q, h_kv, S, d, seed, (1, S))
    seqlens = torch.tensor(lens, dtype=torch.int32)
    # poison every cache row beyond its sequence length: it must never be read
    for b, n in enumerate(lens):
        kc[b, :, n:] = float("nan")
        vc[b, :, n:] = float("nan")
    say(f"decode {case} seed {seed}")
    out = run_decode(seqlens, q, kc, vc, dev).cpu()
    check(f64(out[:, 0]), decode_ref(seqlens, q, kc, vc), "bf16", f"decode {case}")
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.equal(out[b], torch.zeros_like(out[b]))


def test_decode_many_sequences(dev):
    # more sequences than one wave has lanes: the block-list totals and the
    # per-wave start search run over several 64-sequence chunks
    B, h_q, h_kv, S, d = 150, 8, 2, 160, 64
    g = torch.Generator().manual_seed(77)
    lens = torch.randint(0, S + 1, (B,), generator=g).to(torch.int32)
    lens[[0, 63, 64, 65, 127, 128, 149]] = torch.tensor([0, S, 0, 1, 33, 0, S], dtype=torch.int32)
    _, q, kc, vc = wl.decode_inputs(B, h_q, h_kv, S, d, 78, (1, S))
    say(f"decode many sequences B={B}")
    for splits in (0, 7, 300):
        out = run_decode(lens, q, kc, vc, dev, splits=splits).cpu()
        check(f64(out[:, 0]), decode_ref(lens, q, kc, vc), "bf16", f"decode B={B} splits={splits}")
        for b in range(B):
            if int(lens[b]) == 0:
                assert torch.equal(out[b], torch.zeros_like(out[b]))


def test_decode_split_count_does_not_change_the_result(dev):
    B, h_q, h_kv, S, d = 4, 32, 8, 3000, 128
    seqlens, q, kc, vc = wl.decode_inputs(B, h_q, h_kv, S, d, 41, (1, S))
    ref = decode_ref(seqlens, q, kc, vc)
    outs = {}
    for ns in (1, 3, 64, 1000, 5000, 0):
        say(f"decode split identity num_splits {ns}")
        outs[ns] = run_decode(seqlens, q, kc, vc, dev, splits=ns).cpu()
        check(f64(outs[ns][:, 0]), ref, "bf16", f"num_splits {ns} vs oracle")
    for ns in outs:
        check(f64(outs[ns]), f64(outs[1]), "bf16", f"num_splits {ns} vs num_splits 1")


def test_decode_is_deterministic(dev):
    seqlens, q, kc, vc = wl.decode_inputs(8, 32, 8, 2048, 128, 42, (1, 2048))
    say("decode determinism")
    assert torch.equal(run_decode(seqlens, q, kc, vc, dev), run_decode(seqlens, q, kc, vc, dev))


def test_decode_lengths_outside_their_range_are_clamped(dev):
    """A length outside [0, S] is clamped into it on the device: the result is
    that of the clamped length, bit for bit, in the head-major, paged and
    append forms, and the append writes nothing for such a sequence."""
    B, h_q, h_kv, S, d, P = 6, 32, 8, 320, 128, 64
    big = 2 ** 31 - 1
    seqlens, q, kc, vc = wl.decode_inputs(B, h_q, h_kv, S, d, 4200, (1, S))
    lens = torch.tensor([S + 5, -7, S, big, 0, 150], dtype=torch.int32)
    clamped = lens.clamp(0, S)
    say(f"decode lengths {lens.tolist()} against {clamped.tolist()}")
    out = run_decode(lens, q, kc, vc, dev)
    assert torch.equal(out, run_decode(clamped, q, kc, vc, dev))
    # paged: every table entry names a page, so the clamped length may use them all
    kp, vp, table = wl.to_pages(kc, vc, torch.full((B,), S, dtype=torch.int32), P, 4201)
    kp, vp, table = kp.to(dev), vp.to(dev), table.to(dev)
    qd = q.to(dev)
    o1 = gqa.decode_paged(qd, kp, vp, table, lens.to(dev))
    o2 = gqa.decode_paged(qd, kp, vp, table, clamped.to(dev))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(o1, out)
    # append: lengths before the append belong in [0, S - 1]
    _, q, kn, vn, kc, vc = wl.decode_append_inputs(B, h_q, h_kv, S, d, 4202, (0, S - 1))
    lens = torch.tensor([S, -3, S - 1, big, 0, 150], dtype=torch.int32)
    clamped = lens.clamp(0, S - 1)
    outside = (lens < 0) | (lens > S - 1)
    say(f"decode_append lengths {lens.tolist()} against {clamped.tolist()}")
    o1, kc1, vc1 = run_decode_append(lens, q, kn, vn, kc, vc, dev)
    o2, kc2, vc2 = run_decode_append(clamped, q, kn, vn, kc, vc, dev)
    assert torch.equal(o1, o2)
    for b in range(B):
        if outside[b]:  # nothing written
            assert torch.equal(kc1[b], kc[b]) and torch.equal(vc1[b], vc[b]), f"sequence {b}"
        else:
            assert torch.equal(kc1[b], kc2[b]) and torch.equal(vc1[b], vc2[b]), f"sequence {b}"


def test_decode_equals_last_row_of_causal_prefill(dev):
    B, L, h_q, h_kv, d = 2, 777, 32, 8, 128
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, 43, 1.0, torch.bfloat16)
    say("decode vs causal prefill last row")
    po = run_prefill(q, k, v, True, 1 / math.sqrt(d), dev).cpu()
    kc = k.transpose(1, 2).contiguous()
    vc = v.transpose(1, 2).contiguous()
    seqlens = torch.full((B,), L, dtype=torch.int32)
    do = run_decode(seqlens, q[:, L - 1:L].contiguous(), kc, vc, dev).cpu()
    check(f64(do), f64(po[:, L - 1:L]), "bf16", "decode vs prefill row L-1")


# -------------------------------------------------------------- decode with append

def run_decode_append(seqlens, q, kn, vn, kc, vc, dev, splits=0):
    """Returns (o, k_cache after, v_cache after) on the CPU; the inputs are not modified."""
    qd, knd, vnd, sd = q.to(dev), kn.to(dev), vn.to(dev), seqlens.to(dev)
    kcd, vcd = kc.to(dev).clone(), vc.to(dev).clone()
    out = torch.full_like(qd, float("nan"))
    gqa.decode_append(qd, knd, vnd, kcd, vcd, sd, out=out, num_splits=splits)
    torch.cuda.synchronize()
    return out.cpu(), kcd.cpu(), vcd.cpu()


def append_ref(seqlens, q, kn, vn, kc, vc):
    return oracle.decode_append(f64(q[:, 0]), f64(kn[:, 0]), f64(vn[:, 0]), f64(kc), f64(vc),
                                seqlens.numpy())


def check_cache_exact(got, ref, what):
    g = f64(got)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} vs {ref.shape}"
    assert np.array_equal(g, ref, equal_nan=True), (
        f"{what}: {int((~((g == ref) | (np.isnan(g) & np.isnan(ref)))).sum())} elements differ")


APPEND_SMALL = [
    # B, h_q, h_kv, S, d, lengths before the append
    (6, 32, 8, 1100, 128, [0, 1, 511, 512, 31, 1099]),  # empty cache, block edges, last free row
    (3, 8, 8, 700, 64, [699, 63, 64]),                  # G = 1
    (2, 32, 1, 300, 128, [299, 16]),                    # G = 32: two query-head subgroups
    (2, 16, 2, 1000, 64, [998, 0]),                     # G = 8
    (4, 12, 4, 96, 128, [95, 94, 32, 31]),              # G = 3
]


@pytest.mark.parametrize("case", APPEND_SMALL, ids=lambda c: "B{}_hq{}_hkv{}_S{}_d{}".format(*c[:5]))
def test_decode_append_matches_oracle(case, dev):
    B, h_q, h_kv, S, d, lens = case
    seed = 3000 + S + h_q
    _, q, kn, vn, kc, vc = wl.decode_append_inputs(B, h_q, h_kv, S, d, seed, (0, S - 1))
    seqlens = torch.tensor(lens, dtype=torch.int32)
    # poison the row the append overwrites and every row after it: the cache
    # copy of the new row must not be read, nor any row beyond it
    for b, n in enumerate(lens):
        kc[b, :, n:] = float("nan")
        vc[b, :, n:] = float("nan")
    say(f"decode_append {case} seed {seed}")
    o_ref, kc_ref, vc_ref = append_ref(seqlens, q, kn, vn, kc, vc)
    for splits in (0, 1, 7, 1000):
        out, kc_out, vc_out = run_decode_append(seqlens, q, kn, vn, kc, vc, dev, splits)
        check(f64(out[:, 0]), o_ref, "bf16", f"decode_append {case} splits {splits}")
        check_cache_exact(kc_out, kc_ref, f"k_cache after append, splits {splits}")
        check_cache_exact(vc_out, vc_ref, f"v_cache after append, splits {splits}")


def test_decode_append_equals_decode_of_the_grown_cache(dev):
    # the fused form reads the new rows from k_new/v_new and the plain decode
    # from the cache; the values, blocks and slices are the same, so the
    # results are bit-identical
    B, h_q, h_kv, S, d = 5, 32, 8, 2000, 128
    seqlens, q, kn, vn, kc, vc = wl.decode_append_inputs(B, h_q, h_kv, S, d, 51, (0, S - 1))
    seqlens[0] = 0
    seqlens[1] = S - 1
    say("decode_append vs decode of the grown cache")
    out, kc_out, vc_out = run_decode_append(seqlens, q, kn, vn, kc, vc, dev)
    grown = run_decode(seqlens + 1, q, kc_out, vc_out, dev).cpu()
    assert torch.equal(out, grown)


def test_decode_append_is_deterministic_and_idempotent(dev):
    seqlens, q, kn, vn, kc, vc = wl.decode_append_inputs(4, 16, 4, 900, 64, 52, (0, 899))
    say("decode_append determinism")
    dq, dkn, dvn, ds = q.to(dev), kn.to(dev), vn.to(dev), seqlens.to(dev)
    kcd, vcd = kc.to(dev), vc.to(dev)
    o1 = gqa.decode_append(dq, dkn, dvn, kcd, vcd, ds)
    k1, v1 = kcd.clone(), vcd.clone()
    o2 = gqa.decode_append(dq, dkn, dvn, kcd, vcd, ds)  # the same rows written again
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(k1, kcd) and torch.equal(v1, vcd)


def test_workload_batched_decode_append(dev):
    w = wl.WORKLOADS["batched_decode_append_bf16"]
    seqlens, q, kn, vn, kc, vc = wl.workload_inputs(w)
    say(f"decode_append workload {w.name} ({w.description})")
    sd = seqlens.to(dev)
    kcd, vcd = kc.to(dev), vc.to(dev)
    out = torch.empty_like(q, device=dev)
    gqa.decode_append(q.to(dev), kn.to(dev), vn.to(dev), kcd, vcd, sd, out=out)
    torch.cuda.synchronize()
    out = out.cpu()
    # the caches at full size: row seqlens[b] of every head now holds the new
    # row and no other element changed (a property that holds at any size)
    b_idx = torch.arange(w.B, device=dev)
    for name, got, before, new in (("k", kcd, kc, kn), ("v", vcd, vc, vn)):
        exp = before.to(dev)
        exp[b_idx, :, sd.long()] = new.to(dev)[:, 0]
        assert torch.equal(got.view(torch.int16), exp.view(torch.int16)), f"{name}_cache"
        del exp
    # every sequence's output, and the whole cache slabs of 8 sampled
    # sequences, against the oracle (8 sequences at a time)
    o_refs = []
    for b0 in range(0, w.B, 8):
        bi = torch.arange(b0, min(b0 + 8, w.B))
        o_ref, _, _ = append_ref(seqlens[bi], q[bi], kn[bi], vn[bi], kc[bi], vc[bi])
        o_refs.append(o_ref)
    check(f64(out[:, 0]), np.concatenate(o_refs), "bf16", f"{w.name}: all {w.B} sequences")
    order = torch.argsort(seqlens).tolist()
    picks = torch.randperm(w.B, generator=torch.Generator().manual_seed(w.seed))[:6].tolist()
    bsel = sorted({order[0], order[-1], *picks})
    bi = torch.tensor(bsel)
    _, kc_ref, vc_ref = append_ref(seqlens[bi], q[bi], kn[bi], vn[bi], kc[bi], vc[bi])
    check_cache_exact(kcd[bi.to(dev)].cpu(), kc_ref, "k_cache slabs of the sampled sequences")
    check_cache_exact(vcd[bi.to(dev)].cpu(), vc_ref, "v_cache slabs of the sampled sequences")


def _at_address_with_bit31_set(t, dev):
    """A device copy of t placed where bit 31 of the address's low word is set
    (a 2 GiB + size buffer always holds such a 256-byte-aligned place)."""
    n = t.numel() * t.element_size()
    buf = torch.empty((1 << 31) + n + 256, dtype=torch.uint8, device=dev)
    base = buf.data_ptr()
    x = base if base & (1 << 31) else (base & ~0xFFFFFFFF) | (1 << 31)
    x = (x + 255) // 256 * 256
    assert x & (1 << 31) and x + n <= base + buf.numel()
    view = buf[x - base:x - base + n].view(t.dtype).view(t.shape)
    view.copy_(t)
    return buf, view


def test_decode_append_cache_addresses_with_bit31_set(dev):
    # regression: the new rows' store address was once built from a signed
    # 32-bit low word, which corrupted caches placed at such addresses
    B, h_q, h_kv, S, d = 3, 8, 8, 700, 64
    seqlens, q, kn, vn, kc, vc = wl.decode_append_inputs(B, h_q, h_kv, S, d, 53, (0, S - 1))
    seqlens[0] = S - 1
    say("decode_append with caches at addresses whose bit 31 is set")
    o_ref, kc_ref, vc_ref = append_ref(seqlens, q, kn, vn, kc, vc)
    kbuf, kcd = _at_address_with_bit31_set(kc, dev)
    vbuf, vcd = _at_address_with_bit31_set(vc, dev)
    out = gqa.decode_append(q.to(dev), kn.to(dev), vn.to(dev), kcd, vcd, seqlens.to(dev))
    torch.cuda.synchronize()
    check(f64(out[:, 0]), o_ref, "bf16", "decode_append output")
    check_cache_exact(kcd.cpu(), kc_ref, "k_cache after append")
    check_cache_exact(vcd.cpu(), vc_ref, "v_cache after append")
    del kbuf, vbuf


# ----------------------------------------------------- decode over other layouts

TOKEN_MAJOR = [
    # B, h_q, h_kv, S, d, lengths
    (4, 32, 8, 700, 128, [0, 1, 333, 700]),
    (3, 8, 8, 300, 64, [300, 64, 65]),     # G = 1
    (2, 32, 1, 200, 128, [200, 17]),       # G = 32
    (3, 12, 4, 96, 64, [96, 95, 31]),      # G = 3
]


@pytest.mark.parametrize("case", TOKEN_MAJOR, ids=lambda c: "B{}_hq{}_hkv{}_S{}_d{}".format(*c[:5]))
def test_decode_token_major_matches_oracle(case, dev):
    B, h_q, h_kv, S, d, lens = case
    seed = 4000 + S + h_q
    _, q, kc, vc = wl.decode_inputs(B, h_q, h_kv, S, d, seed, (1, S))
    seqlens = torch.tensor(lens, dtype=torch.int32)
    kt = kc.transpose(1, 2).contiguous()  # [B, S, h_kv, d]
    vt = vc.transpose(1, 2).contiguous()
    for b, n in enumerate(lens):
        kt[b, n:] = float("nan")
        vt[b, n:] = float("nan")
    say(f"decode token-major {case} seed {seed}")
    ref = oracle.decode_token_major(f64(q[:, 0]), f64(kt), f64(vt), seqlens.numpy())
    qd, ktd, vtd, sd = q.to(dev), kt.to(dev), vt.to(dev), seqlens.to(dev)
    for splits in (0, 5, 999):
        out = gqa.decode_token_major(qd, ktd, vtd, sd, num_splits=splits)
        torch.cuda.synchronize()
        check(f64(out.cpu()[:, 0]), ref, "bf16", f"token-major {case} splits {splits}")
    # the same blocks and arithmetic as the head-major entry on the transposed cache
    hm = run_decode(seqlens, q, kt.transpose(1, 2).contiguous(), vt.transpose(1, 2).contiguous(),
                    dev).cpu()
    assert torch.equal(gqa.decode_token_major(qd, ktd, vtd, sd).cpu(), hm)


def test_decode_token_major_over_prefill_keys(dev):
    # prefill's k/v [B, L, h_kv, d] are a token-major cache as they stand: the
    # last position's decode equals the causal prefill's last row
    B, L, h_q, h_kv, d = 2, 777, 32, 8, 128
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, 43, 1.0, torch.bfloat16)
    say("token-major decode over prefill keys vs causal prefill last row")
    po = run_prefill(q, k, v, True, 1 / math.sqrt(d), dev).cpu()
    seqlens = torch.full((B,), L, dtype=torch.int32, device=dev)
    do = gqa.decode_token_major(q[:, L - 1:L].contiguous().to(dev), k.to(dev), v.to(dev), seqlens)
    torch.cuda.synchronize()
    check(f64(do.cpu()), f64(po[:, L - 1:L]), "bf16", "token-major decode vs prefill row L-1")


PAGED = [
    # B, h_q, h_kv, S, d, page_size, lengths
    (5, 32, 8, 600, 128, 64, [0, 1, 64, 65, 600]),
    (3, 8, 8, 300, 64, 32, [300, 31, 33]),        # G = 1, smallest pages
    (2, 32, 1, 512, 128, 256, [512, 257]),        # G = 32, large pages
    (4, 12, 4, 200, 64, 96, [200, 96, 95, 1]),    # G = 3, pages of 3 blocks
]


@pytest.mark.parametrize("case", PAGED, ids=lambda c: "B{}_hq{}_hkv{}_S{}_d{}_P{}".format(*c[:6]))
def test_decode_paged_matches_oracle(case, dev):
    B, h_q, h_kv, S, d, P, lens = case
    seed = 5000 + S + h_q + P
    _, q, kc, vc = wl.decode_inputs(B, h_q, h_kv, S, d, seed, (1, S))
    seqlens = torch.tensor(lens, dtype=torch.int32)
    kp, vp, table = wl.to_pages(kc, vc, seqlens, P, seed, spare=3)
    # rows past each length, spare pages: poisoned, never read
    used = set(int(x) for x in table.flatten().tolist() if x >= 0)
    for page in range(kp.shape[0]):
        if page not in used:
            kp[page] = float("nan")
            vp[page] = float("nan")
    for b, n in enumerate(lens):
        if n % P:
            last = int(table[b, (n - 1) // P])
            kp[last, :, n % P:] = float("nan")
            vp[last, :, n % P:] = float("nan")
    say(f"decode paged {case} seed {seed} pages {kp.shape[0]}")
    ref = oracle.decode_paged(f64(q[:, 0]), f64(kp), f64(vp), table.numpy(), seqlens.numpy())
    qd, kpd, vpd, td, sd = q.to(dev), kp.to(dev), vp.to(dev), table.to(dev), seqlens.to(dev)
    for splits in (0, 3, 1000):
        out = gqa.decode_paged(qd, kpd, vpd, td, sd, num_splits=splits)
        torch.cuda.synchronize()
        check(f64(out.cpu()[:, 0]), ref, "bf16", f"paged {case} splits {splits}")
    # bit-identical to the head-major entry over the logical cache
    hm = run_decode(seqlens, q, kc, vc, dev).cpu()
    assert torch.equal(gqa.decode_paged(qd, kpd, vpd, td, sd).cpu(), hm)


def test_decode_paged_shared_prefix(dev):
    # two sequences whose tables start with the same pages
    h_q, h_kv, d, P = 16, 2, 128, 32
    g = torch.Generator().manual_seed(61)
    pool_k = torch.randn(6, h_kv, P, d, generator=g).to(torch.bfloat16)
    pool_v = torch.randn(6, h_kv, P, d, generator=g).to(torch.bfloat16)
    q = torch.randn(2, 1, h_q, d, generator=g).to(torch.bfloat16)
    table = torch.tensor([[4, 0, 5, -1], [4, 0, 2, 3]], dtype=torch.int32)
    lens = torch.tensor([80, 127], dtype=torch.int32)
    say("decode paged shared prefix")
    ref = oracle.decode_paged(f64(q[:, 0]), f64(pool_k), f64(pool_v), table.numpy(), lens.numpy())
    out = gqa.decode_paged(q.to(dev), pool_k.to(dev), pool_v.to(dev), table.to(dev), lens.to(dev))
    torch.cuda.synchronize()
    check(f64(out.cpu()[:, 0]), ref, "bf16", "paged shared prefix")


def test_workload_batched_decode_paged(dev):
    w = wl.WORKLOADS["batched_decode_paged_bf16"]
    seqlens, q, kp, vp, table = wl.workload_inputs(w)
    say(f"decode workload {w.name} ({w.description}) pages {kp.shape[0]}")
    out = gqa.decode_paged(q.to(dev), kp.to(dev), vp.to(dev), table.to(dev), seqlens.to(dev))
    torch.cuda.synchronize()
    out = out.cpu()
    # the same inputs as batched_decode_bf16, so the contiguous decode gives the same bits
    dw = wl.WORKLOADS["batched_decode_bf16"]
    s2, q2, kc, vc = wl.workload_inputs(dw)
    assert torch.equal(s2, seqlens) and torch.equal(q2, q)
    assert torch.equal(out, run_decode(s2, q2, kc, vc, dev).cpu())
    # every sequence against the oracle, 8 at a time; the oracle gets only the
    # pages those sequences use, renumbered
    refs = []
    for b0 in range(0, w.B, 8):
        bi = torch.arange(b0, min(b0 + 8, w.B))
        sub = table[bi]
        used = sorted(set(int(x) for x in sub.flatten().tolist() if x >= 0))
        remap = {p: i for i, p in enumerate(used)}
        sub = torch.tensor([[remap.get(int(x), -1) for x in row] for row in sub.tolist()],
                           dtype=torch.int32)
        idx = torch.tensor(used)
        refs.append(oracle.decode_paged(f64(q[bi, 0]), f64(kp[idx]), f64(vp[idx]), sub.numpy(),
                                        seqlens[bi].numpy()))
    check(f64(out[:, 0]), np.concatenate(refs), "bf16", f"{w.name}: all {w.B} sequences")


# ------------------------------------------------------ prefill with rotary embedding

def check_rotated_keys(got, ref, what):
    """bf16 keys rotated in fp32 and rounded once: within one bf16 rounding of
    the fp64 rotation (half an ulp of the result, plus the fp32 arithmetic)."""
    g, r = f64(got), np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape and np.isfinite(g).all(), what
    bound = np.abs(r) * 2.0 ** -8 + 1e-6
    bad = int((np.abs(g - r) > bound).sum())
    say(f"  {what}: max-abs {float(np.abs(g - r).max()):.3e}, {bad} beyond one bf16 rounding")
    assert bad == 0, f"{what}: {bad} elements beyond one bf16 rounding of the oracle"


ROPE_SMALL = [
    # B, L, h_q, h_kv, d, causal
    (2, 200, 8, 2, 128, True),
    (1, 333, 8, 8, 64, False),   # G = 1, ragged tail
    (2, 130, 32, 4, 128, False),
    (1, 77, 6, 3, 64, True),     # G = 2, one partial tile
]


@pytest.mark.parametrize("case", ROPE_SMALL, ids=lambda c: "B{}_L{}_hq{}_hkv{}_d{}_c{}".format(*c))
def test_prefill_rope_matches_oracle(case, dev):
    B, L, h_q, h_kv, d, causal = case
    seed = 6000 + L + h_q
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, seed, 1.0 / math.sqrt(2.0), torch.bfloat16)
    cos, sin = wl.rope_tables(L, d)
    scale = 1 / math.sqrt(d)
    say(f"prefill rope {case} seed {seed}")
    out, k_rot = gqa.prefill_rope(q.to(dev), k.to(dev), v.to(dev), cos.to(dev), sin.to(dev),
                                  causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, kr_ref = oracle.prefill_rope(f64(q), f64(k), f64(v), f64(cos), f64(sin), causal,
                                        scale)
    check(f64(out.cpu()), o_ref, "bf16", f"rope prefill {case}")
    check_rotated_keys(k_rot.cpu(), kr_ref, f"rotated keys {case}")


def test_prefill_rope_identity_tables_is_permuted_prefill(dev):
    # cos = 1, sin = 0: the rotation is the evens-then-odds permutation, exact in
    # fp32, so the rotary call gives the plain prefill of permuted q and k bit for bit
    B, L, h_q, h_kv, d = 2, 300, 16, 4, 128
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, 71, 1.0, torch.bfloat16)
    ones = torch.ones(L, d // 2, dtype=torch.float32)
    zeros = torch.zeros(L, d // 2, dtype=torch.float32)
    perm = list(range(0, d, 2)) + list(range(1, d, 2))
    say("rope identity tables vs permuted plain prefill")
    for causal in (True, False):
        out, k_rot = gqa.prefill_rope(q.to(dev), k.to(dev), v.to(dev), ones.to(dev), zeros.to(dev),
                                      causal=causal, scale=0.1)
        plain = run_prefill(q[..., perm].contiguous(), k[..., perm].contiguous(), v, causal, 0.1,
                            dev)
        assert torch.equal(k_rot.cpu(), k[..., perm])
        assert torch.equal(out.cpu(), plain.cpu())


def test_workload_llama2_prefill_rope(dev):
    w = wl.WORKLOADS["llama2_7b_prefill_rope_bf16"]
    q, k, v, cos, sin = wl.workload_inputs(w)
    say(f"prefill workload {w.name} ({w.description}) seed {w.seed}")
    out, k_rot = gqa.prefill_rope(q.to(dev), k.to(dev), v.to(dev), cos.to(dev), sin.to(dev),
                                  causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    out, k_rot = out.cpu(), k_rot.cpu()
    kr_ref = oracle.rope(f64(k), f64(cos), f64(sin))
    check_rotated_keys(k_rot, kr_ref, f"{w.name}: all rotated keys")
    q_rot = oracle.rope(f64(q), f64(cos), f64(sin))
    ref = oracle.prefill(q_rot, kr_ref, f64(v), causal=w.causal, scale=w.scale)
    check(f64(out), ref, "bf16", f"{w.name}: all {out.numel() // w.d} rows")


# ------------------------------------------------ prefill of variable-length sequences

VARLEN_SMALL = [
    # B, L, h_q, h_kv, d, dtype, causal, lengths
    (7, 200, 32, 8, 128, "bf16", True, [200, 0, 1, 63, 64, 65, 137]),
    (4, 333, 8, 8, 64, "bf16", False, [333, 1, 256, 100]),    # G = 1
    (3, 130, 16, 2, 128, "bf16", False, [0, 130, 64]),         # G = 8
    (3, 96, 8, 2, 64, "f32", True, [96, 33, 0]),
]


@pytest.mark.parametrize("case", VARLEN_SMALL,
                         ids=lambda c: "B{}_L{}_hq{}_hkv{}_d{}_{}_c{}".format(*c[:7]))
def test_prefill_varlen_matches_oracle(case, dev):
    B, L, h_q, h_kv, d, dtype, causal, lens = case
    seed = 7000 + L + h_q
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, seed, 1.0, tdt)
    kv_lens = torch.tensor(lens, dtype=torch.int32)
    for b, n in enumerate(lens):  # padding keys and values: never read into a result
        k[b, n:] = float("nan")
        v[b, n:] = float("nan")
    scale = 1 / math.sqrt(d)
    say(f"prefill varlen {case} seed {seed}")
    out = gqa.prefill_varlen(q.to(dev), k.to(dev), v.to(dev), kv_lens.to(dev), causal=causal,
                             scale=scale)
    torch.cuda.synchronize()
    ref = oracle.prefill_varlen(f64(q), f64(k), f64(v), lens, causal, scale)
    check(f64(out.cpu()), ref, dtype, f"varlen {case}")
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.equal(out[b].cpu(), torch.zeros_like(out[b].cpu()))


def test_prefill_varlen_full_lengths_is_prefill(dev):
    B, L, h_q, h_kv, d = 2, 300, 32, 8, 128
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, 72, 1.0, torch.bfloat16)
    kv_lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    say("varlen with every length L vs plain prefill")
    for causal in (True, False):
        a = gqa.prefill_varlen(q.to(dev), k.to(dev), v.to(dev), kv_lens, causal=causal, scale=0.09)
        b = run_prefill(q, k, v, causal, 0.09, dev)
        assert torch.equal(a.cpu(), b.cpu())


def test_workload_varlen_prefill(dev):
    w = wl.WORKLOADS["varlen_prefill_bf16"]
    q, k, v, kv_lens = wl.workload_inputs(w)
    say(f"prefill workload {w.name} ({w.description}) lengths {kv_lens.tolist()}")
    out = gqa.prefill_varlen(q.to(dev), k.to(dev), v.to(dev), kv_lens.to(dev), causal=w.causal,
                             scale=w.scale)
    torch.cuda.synchronize()
    out = out.cpu()
    assert not torch.isnan(out).any()
    # sampled rows, plus the last valid and first padded row of the shortest sequence
    b0 = int(torch.argmin(kv_lens))
    n0 = int(kv_lens[b0])
    rows = wl.sample_rows(192, w.B, w.L, w.h_q, w.seed,
                          include=[(b0, n0 - 1, 0), (b0, min(n0, w.L - 1), w.h_q - 1),
                                   (w.B - 1, w.L - 1, 3),
                                   *workgroup_rows(w.B, w.L, w.h_q, w.h_kv, w.seed)])
    idx = torch.tensor(rows)
    ref = oracle.prefill_varlen_rows(f64(q[idx[:, 0], idx[:, 1], idx[:, 2]]), rows, f64(k), f64(v),
                                     kv_lens.numpy(), w.h_q, w.causal, w.scale)
    check(f64(out[idx[:, 0], idx[:, 1], idx[:, 2]]), ref, "bf16", f"{w.name}: {len(rows)} rows")


# ------------------------------------------------------------------ maximum sizes

def test_decode_largest_split_count(dev):
    # num_splits at its limit (2^20 slices: most waves get an empty slice and
    # exit; the workspace is about 4 GiB)
    B, h_q, h_kv, S, d = 2, 8, 2, 700, 64
    seqlens, q, kc, vc = wl.decode_inputs(B, h_q, h_kv, S, d, 81, (1, S))
    say(f"decode num_splits 2^20, workspace {gqa.decode_workspace_bytes(B, h_q, h_kv, d, 1 << 20)}")
    out = run_decode(seqlens, q, kc, vc, dev, splits=1 << 20).cpu()
    check(f64(out[:, 0]), decode_ref(seqlens, q, kc, vc), "bf16", "decode num_splits 2^20")


@pytest.mark.parametrize("h_q,h_kv", [(64, 1), (128, 2)])
def test_prefill_wide_group(h_q, h_kv, dev):
    # G = 64: eight work-groups of 8 heads share each key/value head
    B, L, d = 1, 300, 128
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, 82 + h_q, 1.0, torch.bfloat16)
    say(f"prefill wide group h_q {h_q} h_kv {h_kv}")
    for causal in (True, False):
        out = run_prefill(q, k, v, causal, 1 / math.sqrt(d), dev).cpu()
        check(f64(out), oracle.prefill(f64(q), f64(k), f64(v), causal=causal, scale=1 / math.sqrt(d)),
              "bf16", f"prefill G=64 h_q={h_q} causal={causal}")


@pytest.mark.parametrize("h_q,h_kv,d", [(64, 1, 128), (128, 2, 64)])
def test_decode_wide_group(h_q, h_kv, d, dev):
    # G = 64: four subgroups of 16 query heads per key/value head
    B, S = 3, 500
    seqlens, q, kc, vc = wl.decode_inputs(B, h_q, h_kv, S, d, 84 + h_q, (1, S))
    seqlens[0] = 1
    seqlens[2] = S
    say(f"decode wide group h_q {h_q} h_kv {h_kv} d {d}")
    for splits in (0, 17):
        out = run_decode(seqlens, q, kc, vc, dev, splits=splits).cpu()
        check(f64(out[:, 0]), decode_ref(seqlens, q, kc, vc), "bf16",
              f"decode G=64 h_q={h_q} splits={splits}")


# ------------------------------------------------ decode step with rotary embedding

APPEND_ROPE = [
    # B, h_q, h_kv, S, d, lengths before the append
    (5, 32, 8, 700, 128, [0, 1, 63, 64, 699]),
    (3, 8, 8, 300, 64, [299, 31, 100]),       # G = 1
    (2, 32, 1, 200, 128, [150, 7]),           # G = 32
]


@pytest.mark.parametrize("case", APPEND_ROPE, ids=lambda c: "B{}_hq{}_hkv{}_S{}_d{}".format(*c[:5]))
def test_decode_append_rope_matches_oracle(case, dev):
    B, h_q, h_kv, S, d, lens = case
    seed = 8000 + S + h_q
    _, q, kn, vn, kc, vc = wl.decode_append_inputs(B, h_q, h_kv, S, d, seed, (0, S - 1))
    seqlens = torch.tensor(lens, dtype=torch.int32)
    for b, n in enumerate(lens):
        kc[b, :, n:] = float("nan")
        vc[b, :, n:] = float("nan")
    cos, sin = wl.rope_tables(S, d)
    say(f"decode_append_rope {case} seed {seed}")
    o_ref, kc_ref, vc_ref = oracle.decode_append_rope(f64(q[:, 0]), f64(kn[:, 0]), f64(vn[:, 0]),
                                                      f64(kc), f64(vc), seqlens.numpy(), f64(cos),
                                                      f64(sin))
    for splits in (0, 9):
        kcd, vcd = kc.to(dev), vc.to(dev)
        out = gqa.decode_append_rope(q.to(dev), kn.to(dev), vn.to(dev), kcd, vcd, seqlens.to(dev),
                                     cos.to(dev), sin.to(dev), num_splits=splits)
        torch.cuda.synchronize()
        check(f64(out.cpu()[:, 0]), o_ref, "bf16", f"decode_append_rope {case} splits {splits}")
        # the appended keys are within one bf16 rounding of the fp64 rotation;
        # every other element of the caches is exactly the oracle's
        kg, vg = kcd.cpu(), vcd.cpu()
        k_expect = kc_ref.copy()
        for b, n in enumerate(lens):
            check_rotated_keys(kg[b, :, n], kc_ref[b, :, n], f"appended key of seq {b}")
            k_expect[b, :, n] = f64(kg[b, :, n])
        check_cache_exact(kg, k_expect, "k_cache after the rotary append")
        check_cache_exact(vg, vc_ref, "v_cache after the rotary append")


def test_decode_append_rope_continues_rotary_prefill(dev):
    # the rotary prefill of n positions leaves its rotated keys in the cache;
    # the decode step of token n then matches the rotary prefill of n + 1
    # positions at row n, and appends exactly that prefill's rotated key n
    B, n, h_q, h_kv, d, S = 2, 300, 32, 8, 128, 512
    q, k, v = wl.prefill_inputs(B, n + 1, h_q, h_kv, d, 91, 1.0 / math.sqrt(2.0), torch.bfloat16)
    cos, sin = wl.rope_tables(S, d)
    say("rotary decode step vs rotary prefill")
    full, k_rot = gqa.prefill_rope(q.to(dev), k.to(dev), v.to(dev), cos[:n + 1].contiguous().to(dev),
                                   sin[:n + 1].contiguous().to(dev), causal=True)
    kc = torch.zeros(B, h_kv, S, d, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    kc[:, :, :n] = k_rot[:, :n].transpose(1, 2)
    vc[:, :, :n] = v[:, :n].to(dev).transpose(1, 2)
    seqlens = torch.full((B,), n, dtype=torch.int32, device=dev)
    out = gqa.decode_append_rope(q[:, n:n + 1].contiguous().to(dev), k[:, n:n + 1].contiguous().to(dev),
                                 v[:, n:n + 1].contiguous().to(dev), kc, vc, seqlens, cos.to(dev),
                                 sin.to(dev))
    torch.cuda.synchronize()
    check(f64(out.cpu()), f64(full[:, n:n + 1].cpu()), "bf16", "decode step vs prefill row n")
    assert torch.equal(kc[:, :, n].cpu(), k_rot[:, n].cpu())


# --------------------------------------------------------------- graph capture

def test_graph_capture_replays_match_eager(dev):
    # the entry points allocate nothing and never synchronise, so a prefill and
    # a paged decode captured in one HIP graph replay with the eager results,
    # replay after replay, with eager work on the outputs in between
    B, L, h_q, h_kv, d = 2, 256, 16, 4, 128
    q, k, v = (t.to(dev) for t in wl.prefill_inputs(B, L, h_q, h_kv, d, 95, 1.0, torch.bfloat16))
    seqlens, dq, kc, vc = wl.decode_inputs(4, 32, 8, 1024, 128, 96, (1, 1024))
    kp, vp, table = wl.to_pages(kc, vc, seqlens, 64, 97)
    seqlens, dq, kp, vp, table = (t.to(dev) for t in (seqlens, dq, kp, vp, table))
    po, do = torch.empty_like(q), torch.empty_like(dq)
    ws = torch.empty(gqa.decode_workspace_bytes(4, 32, 8, 128), dtype=torch.uint8, device=dev)

    def step():
        gqa.prefill(q, k, v, causal=True, out=po)
        gqa.decode_paged(dq, kp, vp, table, seqlens, out=do, workspace=ws)

    say("graph capture of prefill + paged decode")
    step()
    torch.cuda.synchronize()
    ref_p, ref_d = po.clone(), do.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(4):
        po.zero_()
        do.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(po, ref_p) and torch.equal(do, ref_d)


# ------------------------------------------------------------ prefill with a keep-mask

def run_prefill_mask(q, k, v, mask, causal, scale, dev):
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.full_like(qd, float("nan"))
    gqa.prefill_mask(qd, kd, vd, mask.to(dev), causal=causal, scale=scale, out=out)
    torch.cuda.synchronize()
    return out


def _case_mask(B, Lq, Lk, density, kind, seed):
    """A keep-mask [B, Lq, Lk] (uint8, CPU): random bytes of the given density,
    or packed documents ("blocks"); row 3 of sequence 0 hides every key."""
    if kind == "blocks":
        rows = []
        for b in range(B):
            lens = wl.document_lengths(Lk, 16, 96, seed + b)
            rows.append(wl.document_mask(lens)[Lk - Lq:])
        m = torch.stack(rows)
    else:
        m = wl.random_mask((B, Lq, Lk), density, seed)
        # nonzero keep values other than 1 mean keep too
        m = m * torch.randint(1, 256, m.shape, generator=torch.Generator().manual_seed(seed),
                              dtype=torch.int64).to(torch.uint8).clamp(min=1)
    if Lq > 3:
        m[0, 3] = 0
    return m


MASK_SMALL = [
    # B, L_q, L_k, h_q, h_kv, d, dtype, causal, density, kind
    (2, 300, 300, 8, 2, 128, "bf16", True, 0.5, "random"),     # G = 4
    (1, 257, 257, 8, 4, 64, "bf16", False, 0.3, "random"),     # G = 2, ragged tail
    (2, 100, 333, 16, 2, 128, "bf16", True, 0.6, "random"),    # L_q < L_k, rows padded to 336
    (1, 200, 200, 6, 2, 128, "bf16", False, 0.5, "blocks"),    # G = 3: 256 rows a work-group
    (3, 65, 65, 8, 8, 64, "bf16", True, 0.5, "random"),        # MHA
    (1, 129, 129, 16, 1, 64, "bf16", False, 0.05, "random"),   # G = 16, sparse
    (1, 700, 700, 16, 2, 128, "bf16", True, 1.0, "blocks"),    # G = 8, block-diagonal documents
    (2, 77, 90, 4, 2, 64, "f32", True, 0.5, "random"),
    (1, 50, 50, 8, 2, 128, "f32", False, 0.5, "blocks"),
]


@pytest.mark.parametrize("case", MASK_SMALL, ids=lambda c: "B{}_Lq{}_Lk{}_hq{}_hkv{}_d{}_{}_c{}_{}".format(
    *c[:8], c[9]))
def test_prefill_mask_matches_oracle(case, dev):
    B, Lq, Lk, h_q, h_kv, d, dt, causal, density, kind = case
    seed = 5000 + Lq + Lk + h_q
    dtype = torch.float32 if dt == "f32" else torch.bfloat16
    q, k, v = wl.prefill_chunk_inputs(B, Lq, Lk, h_q, h_kv, d, seed, dtype=dtype)
    m = _case_mask(B, Lq, Lk, density, kind, seed)
    say(f"prefill_mask {case} seed {seed}")
    out = run_prefill_mask(q, k, v, m, causal, 1 / math.sqrt(d), dev)
    ref = oracle.prefill_mask(f64(q), f64(k), f64(v), m.numpy(), causal, 1 / math.sqrt(d))
    check(f64(out), ref, dt, f"prefill_mask {case}")
    if Lq > 3:
        assert torch.equal(out[0, 3].cpu(), torch.zeros_like(out[0, 3].cpu())), \
            "a row with no visible key must be zero"


def test_prefill_mask_shared_2d_mask(dev):
    """One [L_q, L_k] mask for the whole batch (batch stride 0)."""
    B, L, h_q, h_kv, d = 3, 190, 8, 2, 128
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, 5101)
    m2 = wl.random_mask((L, L), 0.4, 5102)
    say("prefill_mask with one mask for the batch")
    out = run_prefill_mask(q, k, v, m2, True, 0.09, dev)
    ref = oracle.prefill_mask(f64(q), f64(k), f64(v), m2.expand(B, L, L).numpy(), True, 0.09)
    check(f64(out), ref, "bf16", "shared 2-D mask")


def test_prefill_mask_all_ones_is_chunk(dev):
    """Every byte nonzero: the chunked prefill's result, bit for bit."""
    for (B, Lq, Lk, h_q, h_kv, d, dtype) in ((2, 150, 300, 8, 2, 128, torch.bfloat16),
                                            (1, 257, 257, 8, 4, 64, torch.bfloat16),
                                            (1, 70, 99, 4, 1, 64, torch.float32)):
        q, k, v = wl.prefill_chunk_inputs(B, Lq, Lk, h_q, h_kv, d, 5200 + Lq, dtype=dtype)
        ones = torch.full((B, Lq, Lk), 7, dtype=torch.uint8)
        for causal in (True, False):
            say(f"prefill_mask all ones {B, Lq, Lk, h_q, h_kv, d, dtype} causal={causal}")
            a = run_prefill_mask(q, k, v, ones, causal, 0.1, dev)
            b = run_prefill_chunk(q, k, v, causal, 0.1, dev)
            assert torch.equal(a, b)


def test_prefill_mask_lengths_is_varlen(dev):
    """A key-padding mask given as bytes: the variable-length prefill, bit for bit."""
    B, L, h_q, h_kv, d = 4, 300, 8, 2, 128
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, 5300)
    lens = torch.tensor([300, 1, 64, 129], dtype=torch.int32)
    m = torch.zeros(B, L, L, dtype=torch.uint8)
    for b, n in enumerate(lens.tolist()):
        m[b, :, :n] = 1
    for causal in (True, False):
        say(f"prefill_mask lengths vs varlen causal={causal}")
        a = run_prefill_mask(q, k, v, m, causal, 0.1, dev)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        b = gqa.prefill_varlen(qd, kd, vd, lens.to(dev), causal=causal, scale=0.1)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


@pytest.mark.parametrize("d", [128, 64])
def test_prefill_mask_lower_triangle_with_padding_bytes(d, dev):
    """A mask that is exactly the causal pattern, in rows padded with random
    bytes past L_k: with the causal flag every listed tile has all its keys
    visible (no mask bytes loaded); without it the diagonal tiles are partly
    visible.  Both equal the causal chunked prefill bit for bit, and the
    padding bytes play no part."""
    B, L, h_q, h_kv = 2, 300, 8, 2
    q, k, v = wl.prefill_inputs(B, L, h_q, h_kv, d, 5600 + d)
    g = torch.Generator().manual_seed(5601)
    big = torch.randint(0, 2, (B, L, L + 52), generator=g, dtype=torch.int64).to(torch.uint8)
    big[..., :L] = torch.tril(torch.ones(L, L, dtype=torch.uint8))
    big = big.to(dev)
    m = big[..., :L]  # row stride 352 bytes, used in place
    assert gqa.mask_layout(m, B, L, L)[0].data_ptr() == big.data_ptr()
    want = run_prefill_chunk(q, k, v, True, 0.1, dev)
    for causal in (True, False):
        say(f"prefill_mask lower triangle d={d} causal={causal}")
        assert torch.equal(run_prefill_mask(q, k, v, m, causal, 0.1, dev), want)


def test_prefill_mask_more_query_tiles_than_the_ordering_ranks(dev):
    """4100 (sequence, query tile) items, more than the ranking pass orders
    (4096): the work-groups take them in the static order instead.  All-ones
    masks give the chunked prefill bit for bit; a random mask matches the
    oracle on a sample of sequences (each sequence is independent)."""
    B, Lq, Lk, h_q, h_kv, d = 4100, 32, 64, 8, 1, 64  # G = 8: 32-row query tiles
    q, k, v = wl.prefill_chunk_inputs(B, Lq, Lk, h_q, h_kv, d, 5700)
    say("prefill_mask with 4100 query tiles")
    ones = torch.ones(B, Lq, Lk, dtype=torch.uint8)
    assert torch.equal(run_prefill_mask(q, k, v, ones, True, 0.125, dev),
                       run_prefill_chunk(q, k, v, True, 0.125, dev))
    m = wl.random_mask((B, Lq, Lk), 0.3, 5701)
    out = run_prefill_mask(q, k, v, m, True, 0.125, dev).cpu()
    sel = torch.tensor([0, 1, 2047, 4095, 4096, 4099] + list(range(100, 4100, 137)))
    ref = oracle.prefill_mask(f64(q[sel]), f64(k[sel]), f64(v[sel]), m[sel].numpy(), True, 0.125)
    check(f64(out[sel]), ref, "bf16", "4100 query tiles, sampled sequences")


@pytest.mark.parametrize("B", [1, 5, 7])
def test_prefill_mask_fewer_items_than_xcds(B, dev):
    """Fewer (query tile, head) work items than XCDs (one query tile of one
    key/value head per sequence): the persistent prefill runs B work-groups,
    each taking the items of its own XCD's counter, and every item is done."""
    Lq, Lk, h_q, h_kv, d = 30, 100, 4, 1, 128  # G = 4: one 64-row query tile
    q, k, v = wl.prefill_chunk_inputs(B, Lq, Lk, h_q, h_kv, d, 5800 + B)
    m = wl.random_mask((B, Lq, Lk), 0.5, 5801 + B)
    say(f"prefill_mask with {B} work items")
    for causal in (True, False):
        out = run_prefill_mask(q, k, v, m, causal, 0.1, dev)
        ref = oracle.prefill_mask(f64(q), f64(k), f64(v), m.numpy(), causal, 0.1)
        check(f64(out), ref, "bf16", f"{B} work items, causal={causal}")


def _scattered_mask(B, Lq, Lk, period, density, hidden_rows, seed):
    """Keys visible only in key tiles t with t % period == 2 (with the given
    density inside them), and rows [0, hidden_rows) of every sequence see no
    key: a work-group's list of visible tiles has gaps, and the work-groups
    of the hidden rows list none."""
    m = wl.random_mask((B, Lq, Lk), density, seed)
    tile = torch.arange(Lk) // 64
    m = m * (tile % period == 2).to(torch.uint8)[None, None, :]
    m[:, :hidden_rows] = 0
    return m


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [128, 64])
def test_prefill_mask_scattered_tiles(causal, d, dev):
    """Only every fifth key tile holds visible keys: the list of tiles a
    work-group walks skips the others, so ring slots follow list positions,
    not tile indices; rows 0..95 see nothing (whole work-groups with an
    empty list)."""
    B, Lq, Lk, h_q, h_kv = 2, 700, 1500, 8, 2
    q, k, v = wl.prefill_chunk_inputs(B, Lq, Lk, h_q, h_kv, d, 5400 + d)
    m = _scattered_mask(B, Lq, Lk, 5, 0.5, 96, 5401)
    say(f"prefill_mask scattered tiles d={d} causal={causal}")
    out = run_prefill_mask(q, k, v, m, causal, 0.1, dev)
    ref = oracle.prefill_mask(f64(q), f64(k), f64(v), m.numpy(), causal, 0.1)
    check(f64(out), ref, "bf16", f"scattered tiles d={d} causal={causal}")
    assert torch.all(out[:, :96].cpu() == 0), "rows that see no key must be zero"


def test_prefill_mask_long_rows_list_every_tile(dev):
    """Rows of more than 4096 key tiles (262,244 keys): the work-group lists
    every tile instead of scanning, and the result still matches."""
    B, Lq, Lk, h_q, h_kv, d = 1, 40, 4096 * 64 + 100, 4, 1, 64
    q, k, v = wl.prefill_chunk_inputs(B, Lq, Lk, h_q, h_kv, d, 5500)
    m = wl.random_mask((B, Lq, Lk), 0.002, 5501)
    m[:, 5] = 0
    say("prefill_mask with 4098 key tiles per row")
    out = run_prefill_mask(q, k, v, m, False, 0.125, dev)
    ref = oracle.prefill_mask(f64(q), f64(k), f64(v), m.numpy(), False, 0.125)
    check(f64(out), ref, "bf16", "4098 key tiles per row")
    assert torch.all(out[:, 5].cpu() == 0)


def test_workload_document_masked_prefill(dev):
    """The packed-documents workload at full size, every output against the oracle."""
    w = wl.WORKLOADS["document_masked_prefill_bf16"]
    q, k, v, m = wl.workload_inputs(w)
    say(f"prefill_mask workload {w.name} ({w.description}) seed {w.seed}")
    out = run_prefill_mask(q, k, v, m, w.causal, w.scale, dev)
    ref = oracle.prefill_mask(f64(q), f64(k), f64(v), m.numpy(), w.causal, w.scale)
    check(f64(out), ref, w.dtype, f"{w.name}: all {out.numel() // w.d} rows")


# ------------------------------------------------------------ binding argument checks

def test_binding_rejects_mismatched_buffers(dev):
    """Caller-supplied outputs, rotated-key buffers and workspaces of the wrong
    shape, dtype or device are refused before anything is launched."""
    B, L, h_q, h_kv, d = 2, 64, 8, 2, 64
    q, k, v = (t.to(dev) for t in wl.prefill_inputs(B, L, h_q, h_kv, d, 9100))
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    short = torch.empty(B, L - 1, h_q, d, dtype=q.dtype, device=dev)
    f32 = torch.empty(B, L, h_q, d, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        gqa.prefill_varlen(q, k, v, lens, causal=True, out=short)
    with pytest.raises(ValueError):
        gqa.prefill_varlen(q, k, v, lens, causal=True, out=f32)
    cos, sin = (t.to(dev) for t in wl.rope_tables(L, d))
    with pytest.raises(ValueError):
        gqa.prefill_rope(q, k, v, cos, sin, causal=True, out=f32)
    with pytest.raises(ValueError):
        gqa.prefill_rope(q, k, v, cos, sin, causal=True,
                         k_rot=torch.empty(B, L, h_kv, d - 8, dtype=q.dtype, device=dev))
    with pytest.raises(ValueError):
        gqa.prefill_mask(q, k, v, torch.ones(B, L, L, dtype=torch.bool, device=dev),
                         causal=True, out=short)
    seqlens, qd, kc, vc = (t.to(dev) for t in wl.decode_inputs(B, h_q, h_kv, 128, d, 9101,
                                                               (1, 128)))
    need = gqa.decode_workspace_bytes(B, h_q, h_kv, d)
    with pytest.raises(ValueError):
        gqa.decode(qd, kc, vc, seqlens, workspace=torch.empty(need, dtype=torch.uint8))
    with pytest.raises(ValueError):
        gqa.decode(qd, kc, vc, seqlens, workspace=torch.empty(need - 1, dtype=torch.uint8,
                                                              device=dev))
    with pytest.raises(TypeError):
        gqa.decode(qd, kc.float(), vc, seqlens)
    kn = torch.zeros(B, 1, h_kv, d, dtype=qd.dtype, device=dev)
    with pytest.raises(ValueError):
        gqa.decode_append_rope(qd, kn, kn, kc, vc, seqlens, *(t.to(dev) for t in
                                                              wl.rope_tables(128, d)),
                               out=torch.empty(B, 1, h_q, d, dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
