"""gqa_decode_noalloc (the decode whose workspace is the library's fixed
scratch) against gqa_decode with a workspace of its own, through the C ABI.

Two calls in a row, the second with a smaller input (fewer sequences, a zero
length, another head dimension and group size): each must give gqa_decode's
result bit for bit (the same kernels on the same arguments), and match the
fp64 oracle within the bf16 tolerance.  A call needing more workspace than the
scratch holds is refused before anything is launched.
"""
import ctypes

import numpy as np
import pytest
import torch

import gqa_workloads as wl
import grouped_query_attention_03_amd as gqa
import oracle

pytestmark = pytest.mark.gpu

GQA_ERR_SCRATCH = 10


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _noalloc(q, kc, vc, seqlens, out, splits=0):
    B, _, h_q, d = q.shape
    _, h_kv, S, _ = kc.shape
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    return gqa.lib().gqa_decode_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                                        seqlens.data_ptr(), out.data_ptr(), B, h_q, h_kv, S, d,
                                        gqa.GQA_BF16, splits, stream)


def test_noalloc_decode_matches_decode_on_two_calls(dev):
    cases = [
        # B, h_q, h_kv, S, d, seed, lengths (None: drawn)
        (16, 32, 8, 2048, 128, 9500, None),
        (3, 12, 4, 300, 64, 9501, [0, 300, 33]),   # smaller: G = 3, d = 64, a zero length
    ]
    for (B, h_q, h_kv, S, d, seed, lens) in cases:
        seqlens, q, kc, vc = wl.decode_inputs(B, h_q, h_kv, S, d, seed, (1, S))
        if lens is not None:
            seqlens = torch.tensor(lens, dtype=torch.int32)
        print(f"noalloc decode B={B} h_q={h_q} h_kv={h_kv} S={S} d={d} seed={seed}", flush=True)
        qd, kd, vd, sd = q.to(dev), kc.to(dev), vc.to(dev), seqlens.to(dev)
        out = torch.full_like(qd, float("nan"))
        assert _noalloc(qd, kd, vd, sd, out) == 0
        ref = gqa.decode(qd, kd, vd, sd)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "gqa_decode_noalloc differs from gqa_decode"
        want = oracle.decode(q[:, 0].double().numpy(), kc.double().numpy(), vc.double().numpy(),
                             seqlens.numpy())
        got = out[:, 0].cpu().double().numpy()
        err = float(np.abs(got - want).max())
        rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
        print(f"  max-abs {err:.3e} rel-L2 {rel:.3e}", flush=True)
        assert err <= 2e-2 and rel <= 1e-2


def test_noalloc_decode_refuses_more_than_its_scratch(dev):
    B, h_q, h_kv, S, d = 2, 8, 2, 64, 64
    seqlens, q, kc, vc = (t.to(dev) for t in wl.decode_inputs(B, h_q, h_kv, S, d, 9502, (1, S)))
    out = torch.full_like(q, float("nan"))
    # 2^20 splits need about 4 GiB of workspace: refused, nothing launched
    assert _noalloc(q, kc, vc, seqlens, out, splits=1 << 20) == GQA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    with pytest.raises(gqa.GQAError):
        gqa.decode_noalloc(q, kc, vc, seqlens, out=out, num_splits=1 << 20)
