"""The tiles the bf16 kernels visit, counted by the kernels themselves.

Under the causal rule a block of queries needs only the key blocks at or
before its last query ([REAPER] "3 · FlashAttention", causal-mask question:
T(T+1)/2 of T^2 square blocks), and the block-sparse forms only the blocks
whose mask entry is nonzero ([XYZ], block-sparse section).  The counting
instances (fa_fwd_tile_visits, fa_bwd_tile_visits) run the same kernels and
report, per work tile, how many tiles of the other operand they visited.
Checked against the oracle's block rule (oracle.causal_tiles_visited, whose
square case is pinned to T(T+1)/2) and against counts made here from the
mask; their outputs must equal the plain calls bitwise.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_amd import fa
from tests.test_gpu_parity import dev, gen  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    sys.stdout.flush()
    yield


def _needed(i, rows, j, cols, n, causal, mask, bm, bn):
    """Whether work tile i (rows per tile) needs tile j (cols per tile):
    under the causal rule the tile's first key is at or before the block's
    last query; with a mask the covering mask entry is nonzero."""
    if causal and j * cols > min((i + 1) * rows, n) - 1:
        return False
    if mask is not None and not mask[(i * rows) // bm, (j * cols) // bn]:
        return False
    return True


def _expected(n, rows, cols, causal, mask=None, bm=128, bn=128):
    ti, tj = -(-n // rows), -(-n // cols)
    return np.array([[_needed(i, rows, j, cols, n, causal, mask, bm, bn)
                      for j in range(tj)] for i in range(ti)])


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_causal_visits_half_the_tiles(dev, d):
    N = 2048
    x = gen(1, 2, N, d, seed=601 + d, dev=dev)
    rows, cols = fa.fa_tile_grid(0, d)
    for causal in (True, False):
        o, lse, visits = fa.fa_fwd_tile_visits(x["q"], x["k"], x["v"],
                                               causal=causal)
        o_ref, l_ref = fa.fa_fwd(x["q"], x["k"], x["v"], causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        got = visits.cpu().numpy()
        exp = _expected(N, rows, cols, causal).sum(axis=1)
        assert np.array_equal(got[0, 0], exp) and np.array_equal(got[0, 1], exp)
        total = int(got[0, 0].sum())
        if causal:
            assert total == oracle.causal_tiles_visited(N, rows, cols)
            if rows == cols:
                T = N // rows
                assert total == T * (T + 1) // 2
        else:
            assert total == (N // rows) * (N // cols)
        print(f"  d={d} causal={causal} {rows}x{cols} tiles: {total} visited",
              flush=True)


def test_metric_shape_visits(dev):
    # B=2 H=32 N=8192 d=128 causal: every head's count against the block
    # rule, forward and both gradient passes; in units of square blocks of
    # its key-tile width c the dK/dV pass covers exactly T(T+1)/2 of them
    # per head (T = N / c; its query stages divide c).
    B, H, N, d = 2, 32, 8192, 128
    x = gen(B, H, N, d, seed=3, sigma=0.5, with_do=True, dev=dev)
    o, lse, vf = fa.fa_fwd_tile_visits(x["q"], x["k"], x["v"], causal=True)
    dq, dk, dv, vkv, vq = fa.fa_bwd_tile_visits(x["q"], x["k"], x["v"], o,
                                                x["do"], lse, causal=True)
    torch.cuda.synchronize()
    r0, c0 = fa.fa_tile_grid(0, d)
    r1, c1 = fa.fa_tile_grid(1, d)
    r2, c2 = fa.fa_tile_grid(2, d)
    want_f = oracle.causal_tiles_visited(N, r0, c0)
    want_kv = oracle.causal_tiles_visited(N, r1, c1)
    want_q = oracle.causal_tiles_visited(N, r2, c2)
    assert (vf.sum(dim=2) == want_f).all(), "forward"
    assert (vkv.sum(dim=2) == want_kv).all(), "dK/dV pass"
    assert (vq.sum(dim=2) == want_q).all(), "dQ pass"
    T = N // c1
    assert c1 % r1 == 0
    assert want_kv * r1 * c1 == T * (T + 1) // 2 * c1 * c1
    per_kt = _expected(N, r1, c1, True).sum(axis=0)
    assert np.array_equal(vkv[1, 31].cpu().numpy(), per_kt)
    print(f"  forward {want_f} tiles of {r0}x{c0}, dK/dV {want_kv} of "
          f"{r1}x{c1}, dQ {want_q} of {r2}x{c2} per head", flush=True)


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_visits_and_results(dev, d):
    N = 1000  # ragged: the last tiles are partial
    x = gen(1, 3, N, d, seed=611 + d, with_do=True, dev=dev)
    _, c1 = fa.fa_tile_grid(1, d)
    r1, _ = fa.fa_tile_grid(1, d)
    r2, c2 = fa.fa_tile_grid(2, d)
    for causal in (True, False):
        o, lse = fa.fa_fwd(x["q"], x["k"], x["v"], causal=causal)
        dq, dk, dv, vkv, vq = fa.fa_bwd_tile_visits(
            x["q"], x["k"], x["v"], o, x["do"], lse, causal=causal)
        ref = fa.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse,
                        causal=causal)
        torch.cuda.synchronize()
        for a, b in zip((dq, dk, dv), ref):
            assert torch.equal(a, b)
        exp_kv = _expected(N, r1, c1, causal).sum(axis=0)
        exp_q = _expected(N, r2, c2, causal).sum(axis=1)
        for h in range(3):
            assert np.array_equal(vkv[0, h].cpu().numpy(), exp_kv)
            assert np.array_equal(vq[0, h].cpu().numpy(), exp_q)


@pytest.mark.parametrize("d", [64, 128])
def test_blocksparse_visits(dev, d):
    N, bm, bn = 1024, 256, 128
    x = gen(1, 2, N, d, seed=621 + d, with_do=True, dev=dev)
    rng = np.random.default_rng(7)
    mask = (rng.random((N // bm, N // bn)) < 0.4).astype(np.uint8)
    mask[1] = 0                      # a block row with nothing visible
    mask[:, 3] = 0                   # a block column nobody sees
    mask[0, 0] = mask[2, 5] = 1
    m_t = torch.from_numpy(mask).to(dev)
    for causal in (False, True):
        o, lse, vf = fa.fa_fwd_tile_visits(x["q"], x["k"], x["v"], m_t, bm,
                                           bn, causal=causal)
        o_ref, l_ref = fa.fa_fwd_blocksparse(x["q"], x["k"], x["v"], m_t, bm,
                                             bn, causal=causal)
        dq, dk, dv, vkv, vq = fa.fa_bwd_tile_visits(
            x["q"], x["k"], x["v"], o, x["do"], lse, m_t, bm, bn,
            causal=causal)
        g_ref = fa.fa_bwd_blocksparse(x["q"], x["k"], x["v"], o, x["do"], lse,
                                      m_t, bm, bn, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        for a, b in zip((dq, dk, dv), g_ref):
            assert torch.equal(a, b)
        r0, c0 = fa.fa_tile_grid(0, d, sparse=True)
        r1, c1 = fa.fa_tile_grid(1, d, sparse=True)
        r2, c2 = fa.fa_tile_grid(2, d, sparse=True)
        ef = _expected(N, r0, c0, causal, mask, bm, bn).sum(axis=1)
        ekv = _expected(N, r1, c1, causal, mask, bm, bn).sum(axis=0)
        eq = _expected(N, r2, c2, causal, mask, bm, bn).sum(axis=1)
        for h in range(2):
            assert np.array_equal(vf[0, h].cpu().numpy(), ef), "forward"
            assert np.array_equal(vkv[0, h].cpu().numpy(), ekv), "dK/dV"
            assert np.array_equal(vq[0, h].cpu().numpy(), eq), "dQ"
        assert int(vf[0, 0, (bm // r0):(2 * bm // r0)].sum()) == 0
