"""GPU parity of attention with dropout on P (fa_fwd_dropout, fa_bwd_dropout)
against the fp64 dropout oracle, at the bf16 bar (rel-RMS 5e-3; max-abs
2e-2 times 1/(1-p): the kept probabilities are scaled by 1/(1-p) before
their bf16 products, and so are the outputs and their rounding errors),
plus exact checks of the keep mask itself: with Q = 0 every visible
probability is 1/n and one-hot V (or dO) turns outputs into counts of kept
elements, which must equal the oracle's counts exactly, so a single wrong
mask element anywhere in the forward, the dK/dV pass or the dQ pass fails.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from tests.test_gpu_parity import (BF16_MAX_ABS, BF16_REL_RMS, compare,  # noqa: F401
                                   dev, f64, gen)
from exact_io_aware_amd import fa

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    sys.stdout.flush()
    yield


def _compare_drop(name, got, ref, t):
    """compare() with the max-abs bar scaled by 1/(1-p) = 256/(256-t)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{name}: -inf"
    ok = ~np.isneginf(ref)
    g, r = got[ok], ref[ok]
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    if g.size == 0:
        return
    err = float(np.max(np.abs(g - r)))
    norm = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(g - r) / norm) if norm > 0 else 0.0
    bar = BF16_MAX_ABS * 256.0 / (256 - t)
    print(f"  {name}: max-abs {err:.3e} (bar {bar:.2e}) rel-rms {rel:.3e}",
          flush=True)
    assert err <= bar, f"{name}: max-abs {err:.3e} > {bar:.2e}"
    assert rel <= BF16_REL_RMS, f"{name}: rel-rms {rel:.3e}"


def _case(dev, B, H, N, d, causal, p, drop_seed, in_seed, check_bwd=True):
    x = gen(B, H, N, d, in_seed, with_do=True, dev=dev)
    scale = 1 / math.sqrt(d)
    t = oracle.dropout_threshold(p)
    o, lse = fa.fa_fwd_dropout(x["q"], x["k"], x["v"], p, drop_seed,
                               scale=scale, causal=causal)
    grads = None
    if check_bwd:
        grads = fa.fa_bwd_dropout(x["q"], x["k"], x["v"], o, x["do"], lse, p,
                                  drop_seed, scale=scale, causal=causal)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            args = [f64(x[n][b, h]) for n in ("q", "k", "v")]
            O, L = oracle.attention_fwd_dropout_head(*args, scale, causal, t,
                                                     drop_seed, b * H + h)
            _compare_drop(f"O[{b},{h}]", f64(o[b, h]), O, t)
            compare(f"LSE[{b},{h}]", f64(lse[b, h]), L)
            if check_bwd:
                ref = oracle.attention_bwd_dropout_head(
                    *args, f64(x["do"][b, h]), scale, causal, t, drop_seed,
                    b * H + h)
                for name, g, r in zip(("dQ", "dK", "dV"), grads, ref):
                    _compare_drop(f"{name}[{b},{h}]", f64(g[b, h]), r, t)
    return x, (o, lse), grads


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,p", [(1, 0.5), (77, 0.1), (200, 0.25),
                                 (385, 0.9), (600, 0.1)])
def test_dropout_shapes(dev, N, p, d, causal):
    _case(dev, 2, 2, N, d, causal, p, drop_seed=0x5EED0000 + N,
          in_seed=700 + N + d)


def test_dropout_seed_high_word(dev):
    # Seeds above 2^32 (the key's second word) and the largest t.
    _case(dev, 1, 3, 256, 128, True, 255 / 256, drop_seed=(7 << 40) | 12345,
          in_seed=11)


def test_dropout_p0_equals_plain(dev):
    x = gen(2, 2, 300, 128, 12, with_do=True, dev=dev)
    o0, l0 = fa.fa_fwd(x["q"], x["k"], x["v"], causal=True)
    o1, l1 = fa.fa_fwd_dropout(x["q"], x["k"], x["v"], 0.0, 99, causal=True)
    g0 = fa.fa_bwd(x["q"], x["k"], x["v"], o0, x["do"], l0, causal=True)
    g1 = fa.fa_bwd_dropout(x["q"], x["k"], x["v"], o1, x["do"], l1, 0.0, 99,
                           causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)


def test_dropout_deterministic_and_seeded(dev):
    x = gen(1, 2, 512, 64, 13, with_do=True, dev=dev)
    run = [fa.fa_fwd_dropout(x["q"], x["k"], x["v"], 0.3, s, causal=False)
           for s in (5, 5, 5 + (1 << 32))]
    torch.cuda.synchronize()
    assert torch.equal(run[0][0], run[1][0])
    assert not torch.equal(run[0][0], run[2][0]), "seed high word ignored"
    assert torch.equal(run[0][1], run[2][1]), "LSE must not depend on dropout"


def _counts_ref(bh, N, d, seed, t, causal, by_col):
    """Kept elements per (row, column class): for row i and c < d, the number
    of kept j = c (mod d) (by_col=False), or for key j the number of kept
    i = c (mod d) (by_col=True); only visible elements count."""
    keep = oracle.dropout_keep(bh, N, N, seed, t)
    if causal:
        keep &= np.tril(np.ones((N, N), dtype=bool))
    if by_col:
        keep = keep.T
    return keep.reshape(N, N // d, d).sum(axis=1)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_mask_exact_forward(dev, d, causal):
    # Q = 0: P_ij = 1/(visible keys of row i); V_j = e_(j mod d), so
    # O_ic * n_i * (256 - t) / 256 counts the kept keys j = c (mod d).
    B, H, N, p, seed = 2, 3, 1024, 0.2, 0xABCDEF0123
    t = oracle.dropout_threshold(p)
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device=dev)
    k = torch.randn(B, H, N, d, device=dev).bfloat16()
    v = torch.zeros(N, d, device=dev)
    v[torch.arange(N), torch.arange(N) % d] = 1.0
    v = v.bfloat16().expand(B, H, N, d).contiguous()
    o, _ = fa.fa_fwd_dropout(q, k, v, p, seed, causal=causal)
    torch.cuda.synchronize()
    n_vis = (np.arange(N) + 1.0) if causal else np.full(N, float(N))
    for b in range(B):
        for h in range(H):
            got = np.rint(f64(o[b, h]) * n_vis[:, None] * (256 - t) / 256)
            ref = _counts_ref(b * H + h, N, d, seed, t, causal, False)
            bad = np.argwhere(got != ref)
            assert bad.size == 0, f"head {b},{h}: mask differs at {bad[:5]}"


@pytest.mark.parametrize("d", [64, 128])
def test_dropout_mask_exact_dkdv(dev, d):
    # Q = 0, non-causal, N = 1024: P = 2^-10 exactly; dO_i = e_(i mod d), so
    # dV_jc * N * (256 - t) / 256 counts the kept queries i = c (mod d) of
    # key j.
    B, H, N, p, seed = 1, 3, 1024, 0.3, 77
    t = oracle.dropout_threshold(p)
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device=dev)
    k = torch.randn(B, H, N, d, device=dev).bfloat16()
    v = torch.randn(B, H, N, d, device=dev).bfloat16()
    do = torch.zeros(N, d, device=dev)
    do[torch.arange(N), torch.arange(N) % d] = 1.0
    do = do.bfloat16().expand(B, H, N, d).contiguous()
    o, lse = fa.fa_fwd_dropout(q, k, v, p, seed)
    _, _, dv = fa.fa_bwd_dropout(q, k, v, o, do, lse, p, seed)
    torch.cuda.synchronize()
    for h in range(H):
        got = np.rint(f64(dv[0, h]) * N * (256 - t) / 256)
        ref = _counts_ref(h, N, d, seed, t, False, True)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"head {h}: mask differs at {bad[:5]}"


@pytest.mark.parametrize("d", [64, 128])
def test_dropout_mask_dq(dev, d):
    # Q = 0, K and V one-hot (K_j = V_j = e_(j mod d)), dO = 1: dP_ij =
    # Z_ij/(1-p), dS_ij = (Z_ij/(1-p) - D_i)/N and dQ_ic = scale * sum over
    # j = c (mod d) of dS_ij.  One wrong mask element moves dQ_ic by
    # scale/(N(1-p)); the bound below is 0.4 of that.
    B, H, N, p, seed = 1, 2, 1024, 0.1, 4242
    t = oracle.dropout_threshold(p)
    scale = 1 / math.sqrt(d)
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device=dev)
    e = torch.zeros(N, d, device=dev)
    e[torch.arange(N), torch.arange(N) % d] = 1.0
    k = e.bfloat16().expand(B, H, N, d).contiguous()
    v = k.clone()
    do = torch.ones(B, H, N, d, dtype=torch.bfloat16, device=dev)
    o, lse = fa.fa_fwd_dropout(q, k, v, p, seed)
    dq, _, _ = fa.fa_bwd_dropout(q, k, v, o, do, lse, p, seed)
    torch.cuda.synchronize()
    step = scale / (N * (256 - t) / 256)
    for h in range(H):
        ref = oracle.attention_bwd_dropout_head(
            f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), f64(do[0, h]), scale,
            False, t, seed, h)[0]
        err = float(np.max(np.abs(f64(dq[0, h]) - ref)))
        print(f"  dQ[{h}] max-abs {err:.3e} (one mask element: {step:.3e})")
        assert err <= 0.4 * step, f"head {h}: dQ off by {err:.3e}"


def test_dropout_metric_shape_sampled_rows(dev):
    # B=2 H=32 N=8192 d=128 causal, p = 0.1: sampled rows of O, LSE and dQ
    # of two heads against the oracle's row-restricted forward and dQ.
    B, H, N, d, p, seed = 2, 32, 8192, 128, 0.1, 2024
    t = oracle.dropout_threshold(p)
    scale = 1 / math.sqrt(d)
    x = gen(B, H, N, d, 3, sigma=0.5, with_do=True, dev=dev)
    o, lse = fa.fa_fwd_dropout(x["q"], x["k"], x["v"], p, seed, causal=True)
    dq, _, _ = fa.fa_bwd_dropout(x["q"], x["k"], x["v"], o, x["do"], lse, p,
                                 seed, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.sort(np.concatenate([[0, 1, 255, 256, N - 1],
                                   rng.choice(N, 27, replace=False)]))
    for b, h in ((0, 0), (1, 31)):
        args = [f64(x[n][b, h]) for n in ("q", "k", "v")]
        O, L = oracle.attention_fwd_dropout_head(*args, scale, True, t, seed,
                                                 b * H + h, rows=rows)
        _compare_drop(f"O rows [{b},{h}]", f64(o[b, h])[rows], O, t)
        compare(f"LSE rows [{b},{h}]", f64(lse[b, h])[rows], L)
        dQ = oracle.attention_dq_dropout_rows(*args, f64(x["do"][b, h]), scale,
                                              True, t, seed, b * H + h, rows)
        # The edge rows see one or two keys, where dQ is (near) zero and the
        # rounding of D (formed from the stored bf16 O) dominates: the
        # relative bar applies to the uniformly drawn rows, max-abs to all.
        edge = np.isin(rows, [0, 1, 255, 256, N - 1])
        _compare_drop(f"dQ rows [{b},{h}]", f64(dq[b, h])[rows][~edge],
                      dQ[~edge], t)
        err = float(np.max(np.abs(f64(dq[b, h])[rows][edge] - dQ[edge])))
        assert err <= BF16_MAX_ABS, f"dQ edge rows [{b},{h}]: {err:.3e}"
