"""GPU parity of the block-sparse backward (fa_bwd_blocksparse) against the
fp64 oracle's masked gradients, plus the identities the mask fixes: an
all-ones mask is the dense backward (bitwise at d = 64: same tiles, same
order; at d = 128 the dense dQ pass sums the keys of half its causal query
tiles from the diagonal down, float32 rounding apart, and the dense dK/dV
pass is the 256-key kernel, whose statistics enter the products, so P and
dS round to bf16 differently in a few elements), a diagonal mask is the dense backward of each diagonal chunk, and queries
(keys) that see nothing get zero dQ (dK, dV)."""

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


def _sparse_case(dev, B, H, N, d, seed, causal, mask, bm, bn, heads=None):
    x = gen(B, H, N, d, seed, with_do=True, dev=dev)
    scale = 1 / math.sqrt(d)
    m_t = torch.from_numpy(mask).to(dev)
    o, lse = fa.fa_fwd_blocksparse(x["q"], x["k"], x["v"], m_t, bm, bn,
                                   scale=scale, causal=causal)
    dq, dk, dv = fa.fa_bwd_blocksparse(x["q"], x["k"], x["v"], o, x["do"],
                                       lse, m_t, bm, bn, scale=scale,
                                       causal=causal)
    torch.cuda.synchronize()
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        ref = oracle.attention_bwd_head(
            *(f64(x[n][b, h]) for n in ("q", "k", "v", "do")), scale, causal,
            mask, bm, bn)
        for name, got, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            compare(f"{name}[{b},{h}]", f64(got[b, h]), r)
    return x, (o, lse), (dq, dk, dv)


def _mask(t_m, t_n, seed, empty_row=None, empty_col=None):
    r = np.random.default_rng(seed)
    m = (r.random((t_m, t_n)) < 0.5).astype(np.uint8)
    for i in range(min(t_m, t_n)):
        m[i, i] = 1
    if empty_row is not None:
        m[empty_row, :] = 0
    if empty_col is not None:
        m[:, empty_col] = 0
    return m


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,bm,bn", [(512, 128, 128), (500, 128, 128),
                                     (640, 256, 128), (640, 128, 256)])
def test_sparse_bwd_random_masks(dev, N, bm, bn, d, causal):
    t_m, t_n = -(-N // bm), -(-N // bn)
    mask = _mask(t_m, t_n, seed=N + bm + 3 * bn + d, empty_row=t_m - 1,
                 empty_col=0 if not causal else None)
    _sparse_case(dev, 1, 2, N, d, seed=700 + N + d, causal=causal,
                 mask=mask, bm=bm, bn=bn)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_sparse_bwd_all_ones_is_dense(dev, d, causal):
    B, H, N = 1, 3, 700
    x = gen(B, H, N, d, seed=71, with_do=True, dev=dev)
    scale = 1 / math.sqrt(d)
    T = -(-N // 128)
    ones = torch.ones(T, T, dtype=torch.uint8, device=dev)
    o, lse = fa.fa_fwd(x["q"], x["k"], x["v"], scale=scale, causal=causal)
    dense = fa.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, scale=scale,
                      causal=causal)
    sp = fa.fa_bwd_blocksparse(x["q"], x["k"], x["v"], o, x["do"], lse, ones,
                               scale=scale, causal=causal)
    none = fa.fa_bwd_blocksparse(x["q"], x["k"], x["v"], o, x["do"], lse,
                                 None, scale=scale, causal=causal)
    for a, b, c, name in zip(dense, sp, none, ("dQ", "dK", "dV")):
        err = float((a - b).abs().max())
        if name == "dQ" and causal and d == 128:
            # Same terms, another summation order: float32 rounding only.
            assert err <= 1e-5 * float(a.abs().max()), (name, err)
        elif name != "dQ" and d == 128:
            # Another kernel: bf16 rounding of P and dS in a few elements.
            assert err <= 1e-2 * float(a.abs().max()), (name, err)
        else:
            assert torch.equal(a, b), f"all-ones mask {name} differs from dense"
        assert torch.equal(a, c), f"mask=None {name} differs from dense"


@pytest.mark.parametrize("d", [64, 128])
def test_sparse_bwd_diagonal_is_chunked_dense(dev, d):
    T, H, N = 4, 2, 512
    x = gen(1, H, N, d, seed=72, with_do=True, dev=dev)
    scale = 1 / math.sqrt(d)
    diag = torch.eye(T, dtype=torch.uint8, device=dev)
    o, lse = fa.fa_fwd_blocksparse(x["q"], x["k"], x["v"], diag, scale=scale)
    sp = fa.fa_bwd_blocksparse(x["q"], x["k"], x["v"], o, x["do"], lse, diag,
                               scale=scale)
    chunk = lambda t: t.reshape(H * T, 1, 128, d).contiguous()  # noqa: E731
    oc, lc = fa.fa_fwd(chunk(x["q"]), chunk(x["k"]), chunk(x["v"]),
                       scale=scale)
    dc = fa.fa_bwd(chunk(x["q"]), chunk(x["k"]), chunk(x["v"]), oc,
                   chunk(x["do"]), lc, scale=scale)
    torch.cuda.synchronize()
    for a, b, name in zip(sp, dc, ("dQ", "dK", "dV")):
        compare(f"diagonal {name}", f64(a.reshape(b.shape)), f64(b))


def test_sparse_bwd_nothing_visible_gives_zero(dev):
    # Block row 1 sees nothing (dQ rows 128..255 are exactly 0); block
    # column 2 is seen by nobody (dK, dV rows 256..383 are exactly 0).
    N, d = 384, 64
    mask = np.array([[1, 1, 0], [0, 0, 0], [1, 1, 0]], dtype=np.uint8)
    _, _, (dq, dk, dv) = _sparse_case(dev, 1, 2, N, d, seed=73, causal=False,
                                      mask=mask, bm=128, bn=128)
    assert torch.count_nonzero(dq[:, :, 128:256]) == 0
    assert torch.count_nonzero(dk[:, :, 256:]) == 0
    assert torch.count_nonzero(dv[:, :, 256:]) == 0
