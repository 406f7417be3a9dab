"""GPU parity of the float32 backward (fa_bwd and fa_bwd_blocksparse with
float32 tensors) against the fp64 oracle's gradients, at the fp32 bar
(max-abs 1e-5 on dQ, dK, dV): O and LSE come from the fp32 forward of the
same inputs, the oracle recomputes everything in fp64.  Cases span ragged
N, one key, causal and not, both head sizes, block masks with empty block
rows and columns, the fp32 workload's shape, and the separately callable
passes against the fused call."""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_amd import fa, workloads
from tests.test_gpu_parity import compare, dev, f64, gen  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    sys.stdout.flush()
    yield


def _f32_bwd_case(dev, B, H, N, d, seed, causal, mask=None, bm=128, bn=128,
                  sigma=1.0):
    x = gen(B, H, N, d, seed, dtype="f32", sigma=sigma, with_do=True, dev=dev)
    scale = 1 / math.sqrt(d)
    if mask is None:
        o, lse = fa.fa_fwd(x["q"], x["k"], x["v"], scale=scale, causal=causal)
        dq, dk, dv = fa.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse,
                               scale=scale, causal=causal)
    else:
        m_t = torch.from_numpy(mask).to(dev)
        o, lse = fa.fa_fwd_blocksparse(x["q"], x["k"], x["v"], m_t, bm, bn,
                                       scale=scale, causal=causal)
        dq, dk, dv = fa.fa_bwd_blocksparse(x["q"], x["k"], x["v"], o, x["do"],
                                           lse, m_t, bm, bn, scale=scale,
                                           causal=causal)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            ref = oracle.attention_bwd_head(
                *(f64(x[n][b, h]) for n in ("q", "k", "v", "do")), scale,
                causal, mask, bm, bn)
            for name, got, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
                compare(f"{name}[{b},{h}]", f64(got[b, h]), r, fp32=True)
    return x, (o, lse), (dq, dk, dv)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 77, 128, 200, 385])
def test_f32_bwd_shapes(dev, N, d, causal):
    _f32_bwd_case(dev, 1, 2, N, d, seed=500 + N + d, causal=causal)


def test_f32_bwd_workload_shape_1x1x256x64(dev):
    # The fp32 workload's shape and inputs, differentiated in both masks.
    w = workloads.workload("fp32_1x1x256x64")
    for causal in (False, True):
        _f32_bwd_case(dev, w["B"], w["H"], w["N"], w["d"], w["seed"], causal)


def test_f32_bwd_single_key_closed_form(dev):
    # N = 1: P = 1, so dQ = dK = 0 exactly in exact arithmetic and dV = dO.
    x, _, (dq, dk, dv) = _f32_bwd_case(dev, 2, 1, 1, 64, seed=11, causal=True)
    assert float(dq.abs().max()) <= 1e-6 and float(dk.abs().max()) <= 1e-6
    compare("dV vs dO", f64(dv), f64(x["do"]), fp32=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_bwd_block_masks(dev, d, causal):
    # 3 x 3 blocks of 128 (N = 300, ragged last block): block row 1 sees
    # nothing, block column 2 is seen by nobody.
    mask = np.array([[1, 1, 0], [0, 0, 0], [1, 1, 0]], dtype=np.uint8)
    _, _, (dq, dk, dv) = _f32_bwd_case(dev, 1, 2, 300, d, seed=90 + d,
                                       causal=causal, mask=mask)
    assert torch.count_nonzero(dq[:, :, 128:256]) == 0
    assert torch.count_nonzero(dk[:, :, 256:]) == 0
    assert torch.count_nonzero(dv[:, :, 256:]) == 0


def test_f32_bwd_256_blocks(dev):
    mask = np.array([[1, 0], [1, 1]], dtype=np.uint8)
    _f32_bwd_case(dev, 1, 1, 400, 64, seed=95, causal=False, mask=mask,
                  bm=256, bn=256)


def test_f32_bwd_passes_equal_fused_call(dev):
    B, H, N, d = 1, 2, 200, 128
    x = gen(B, H, N, d, seed=96, dtype="f32", with_do=True, dev=dev)
    o, lse = fa.fa_fwd(x["q"], x["k"], x["v"], causal=True)
    dq, dk, dv = fa.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse,
                           causal=True)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8,
                     device=dev)
    dq2, dk2, dv2 = (torch.empty_like(t) for t in (dq, dk, dv))
    fa.fa_bwd_preprocess(o, x["do"], lse, ws)
    fa.fa_bwd_dkdv(x["q"], x["k"], x["v"], x["do"], ws, dk2, dv2, causal=True)
    fa.fa_bwd_dq(x["q"], x["k"], x["v"], x["do"], ws, dq2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    # the combined preprocess + dQ call, then the dK/dV pass
    ws.fill_(0x55)
    dq3, dk3, dv3 = (torch.empty_like(t) for t in (dq, dk, dv))
    fa.fa_bwd_dq_stats(x["q"], x["k"], x["v"], o, x["do"], lse, ws, dq3,
                       causal=True)
    fa.fa_bwd_dkdv(x["q"], x["k"], x["v"], x["do"], ws, dk3, dv3, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq3) and torch.equal(dk, dk3) and torch.equal(dv, dv3)


def test_f32_bwd_repeatable(dev):
    # No atomics: repeated calls are bitwise identical.
    x = gen(1, 2, 333, 64, seed=97, dtype="f32", with_do=True, dev=dev)
    o, lse = fa.fa_fwd(x["q"], x["k"], x["v"], causal=True)
    a = fa.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, causal=True)
    b = fa.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, causal=True)
    torch.cuda.synchronize()
    for u, w in zip(a, b):
        assert torch.equal(u, w)
