"""GPU parity of fa_fwd_general / fa_bwd_general against the fp64 oracle.

The general calls take Nq queries against Nk keys (under the causal rule the
queries are the last Nq of the Nk tokens, [REAPER] 3.6: a prompt fed in
chunks, or decoding), an optional block mask and optional dropout, together.
Bars as everywhere: fp32 max-abs 1e-5; bf16 max-abs 2e-2 (x 256/(256-t)
with dropout) and rel-RMS 5e-3.  Reference values: the oracle's
``attention_decode_head`` rows for the offset forward (as the split-KV
tests), ``attention_fwd_head`` / ``attention_bwd_head`` with ``q_pos0`` for
everything else, and the dropout oracle with the same mask, offset and seed.
Exact checks: with Q = 0 and one-hot V the dropout forward counts kept
elements, which must equal the oracle's counts at the same offset; with
Nq = Nk, no mask and no dropout the general calls equal fa_fwd / fa_bwd
bitwise.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_amd import fa
from tests.test_gpu_dropout import _compare_drop
from tests.test_gpu_parity import compare, dev, f64, gen  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    sys.stdout.flush()
    yield


def _inputs(B, H, Nq, Nk, d, seed, dtype="bf16", dev=None):
    x = gen(B, H, max(Nq, Nk), d, seed, dtype, with_do=True, dev=dev)
    return {"q": x["q"][:, :, :Nq].contiguous(),
            "k": x["k"][:, :, :Nk].contiguous(),
            "v": x["v"][:, :, :Nk].contiguous(),
            "do": x["do"][:, :, :Nq].contiguous()}


def _mask(Nq, Nk, bm, bn, seed, empty_row=None):
    rng = np.random.default_rng(seed)
    m = (rng.random((-(-Nq // bm), -(-Nk // bn))) < 0.5).astype(np.uint8)
    m[0, 0] = 1
    m[-1, -1] = 1
    if empty_row is not None:
        m[empty_row] = 0
    return m


def _check(dev, B, H, Nq, Nk, d, causal, mask=None, bm=128, bn=128, p=0.0,
           seed=0, dtype="bf16", in_seed=1, heads=None, bwd=True):
    x = _inputs(B, H, Nq, Nk, d, in_seed, dtype, dev)
    scale = 1 / math.sqrt(d)
    fp32 = dtype == "f32"
    m_t = torch.from_numpy(mask).to(dev) if mask is not None else None
    kw = dict(scale=scale, causal=causal, block_mask=m_t, block_m=bm,
              block_n=bn, p_drop=p, seed=seed)
    o, lse = fa.fa_fwd_general(x["q"], x["k"], x["v"], **kw)
    grads = (fa.fa_bwd_general(x["q"], x["k"], x["v"], o, x["do"], lse, **kw)
             if bwd else None)
    torch.cuda.synchronize()
    off = Nk - Nq
    t = oracle.dropout_threshold(p)
    for b, h in heads or [(b, h) for b in range(B) for h in range(H)]:
        q, k, v, do = (f64(x[n][b, h]) for n in ("q", "k", "v", "do"))
        tag = f"({b},{h}) {Nq}x{Nk} d={d} causal={causal}"
        if t > 0:
            O, L = oracle.attention_fwd_dropout_head(
                q, k, v, scale, causal, t, seed, b * H + h, None, mask, bm,
                bn, off)
            _compare_drop("O " + tag, f64(o[b, h]), O, t)
        else:
            O, L = oracle.attention_fwd_head(q, k, v, scale, causal, mask, bm,
                                             bn, q_pos0=off)
            compare("O " + tag, f64(o[b, h]), O, fp32)
        compare("LSE " + tag, f64(lse[b, h]), L, fp32)
        if not bwd:
            continue
        if t > 0:
            ref = oracle.attention_bwd_dropout_head(
                q, k, v, do, scale, causal, t, seed, b * H + h, mask, bm, bn,
                off)
            for name, g, r in zip(("dQ", "dK", "dV"), grads, ref):
                _compare_drop(f"{name} {tag}", f64(g[b, h]), r, t)
        else:
            ref = oracle.attention_bwd_head(q, k, v, do, scale, causal, mask,
                                            bm, bn, q_pos0=off)
            for name, g, r in zip(("dQ", "dK", "dV"), grads, ref):
                compare(f"{name} {tag}", f64(g[b, h]), r, fp32)
    return x, (o, lse), grads


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nq,Nk", [(300, 1000), (1, 777), (64, 2048),
                                   (511, 513), (1000, 1000), (257, 4096)])
def test_offset_causal_against_decode_rows(dev, d, Nq, Nk):
    # The forward rows equal the oracle's decoding definition (queries =
    # the last Nq tokens); the backward against the offset oracle.
    x, (o, lse), _ = _check(dev, 1, 2, Nq, Nk, d, True, in_seed=Nq + Nk + d)
    for h in range(2):
        O, L = oracle.attention_decode_head(f64(x["q"][0, h]),
                                            f64(x["k"][0, h]),
                                            f64(x["v"][0, h]), 1 / math.sqrt(d),
                                            True)
        compare(f"O vs decode rows h={h}", f64(o[0, h]), O)
        compare(f"LSE vs decode rows h={h}", f64(lse[0, h]), L)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nq,Nk", [(500, 200), (200, 700), (129, 1)])
def test_cross_lengths_noncausal(dev, d, Nq, Nk):
    _check(dev, 2, 2, Nq, Nk, d, False, in_seed=3 * Nq + Nk)


@pytest.mark.parametrize("d", [64, 128])
def test_chunked_prompt_equals_whole(dev, d):
    # A causal prompt of 1000 tokens fed in chunks of 300, 300, 400, each
    # against the keys of the chunks so far, gives the whole prompt's rows.
    B, H, N = 1, 3, 1000
    x = gen(B, H, N, d, seed=41 + d, dev=dev)
    o_all, l_all = fa.fa_fwd(x["q"], x["k"], x["v"], causal=True)
    rows = []
    for a, e in ((0, 300), (300, 600), (600, 1000)):
        o, lse = fa.fa_fwd_general(x["q"][:, :, a:e].contiguous(),
                                   x["k"][:, :, :e].contiguous(),
                                   x["v"][:, :, :e].contiguous(), causal=True)
        rows.append((a, e, o, lse))
    torch.cuda.synchronize()
    for h in range(H):
        O, L = oracle.attention_fwd_head(f64(x["q"][0, h]), f64(x["k"][0, h]),
                                         f64(x["v"][0, h]), 1 / math.sqrt(d),
                                         True)
        for a, e, o, lse in rows:
            compare(f"chunk [{a},{e}) h={h} O", f64(o[0, h]), O[a:e])
            compare(f"chunk [{a},{e}) h={h} LSE", f64(lse[0, h]), L[a:e])
            diff = float((o[0, h].float() - o_all[0, h, a:e].float()).abs().max())
            assert diff <= 2e-2, f"chunk [{a},{e}) vs whole: {diff:.3e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_offset_block_mask(dev, d, causal):
    Nq, Nk, bm, bn = 384, 1000, 128, 256
    mask = _mask(Nq, Nk, bm, bn, seed=d + causal, empty_row=1)
    _check(dev, 1, 2, Nq, Nk, d, causal, mask, bm, bn, in_seed=77 + d)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(512, 512), (300, 1000)])
def test_dropout_with_block_mask(dev, d, causal, Nq, Nk):
    mask = _mask(Nq, Nk, 128, 128, seed=Nq + d, empty_row=1)
    _check(dev, 1, 2, Nq, Nk, d, causal, mask, p=0.15, seed=0xC0FFEE + d,
           in_seed=91 + d)


@pytest.mark.parametrize("d", [64, 128])
def test_dropout_offset_no_mask(dev, d):
    _check(dev, 2, 2, 200, 650, d, True, p=0.25, seed=(3 << 33) + d,
           in_seed=13 + d)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("off", [0, 5, 131])
def test_dropout_offset_mask_exact(dev, d, off):
    # Q = 0 with a block mask and the causal rule at offset `off`: every
    # visible probability of row i is 1/n_i, and V_j = e_(j mod d) turns
    # O_ic * n_i * (256 - t) / 256 into the count of kept visible keys
    # j = c (mod d), which must equal the oracle's count exactly (the keep
    # bits come from the counter with word 3 = off).
    B, H, Nq, bm, bn, p, seed = 1, 2, 512, 128, 128, 0.2, 0xFEED
    Nk = Nq + off
    t = oracle.dropout_threshold(p)
    mask = _mask(Nq, Nk, bm, bn, seed=off)
    q = torch.zeros(B, H, Nq, d, dtype=torch.bfloat16, device=dev)
    k = torch.randn(B, H, Nk, d, device=dev).bfloat16()
    v = torch.zeros(Nk, d, device=dev)
    v[torch.arange(Nk), torch.arange(Nk) % d] = 1.0
    v = v.bfloat16().expand(B, H, Nk, d).contiguous()
    o, _ = fa.fa_fwd_general(q, k, v, causal=True,
                             block_mask=torch.from_numpy(mask).to(dev),
                             p_drop=p, seed=seed)
    torch.cuda.synchronize()
    vis = oracle.visible(np.arange(Nq), Nk, True, mask, bm, bn, q_pos0=off)
    n_vis = vis.sum(axis=1).astype(np.float64)
    live = n_vis > 0
    for h in range(H):
        keep = oracle.dropout_keep(h, Nq, Nk, seed, t, off) & vis
        pad = (-Nk) % d
        ref = np.pad(keep, ((0, 0), (0, pad))).reshape(Nq, -1, d).sum(axis=1)
        got = np.rint(f64(o[0, h]) * n_vis[:, None] * (256 - t) / 256)
        bad = np.argwhere(got[live] != ref[live])
        assert bad.size == 0, f"head {h} off {off}: mask differs at {bad[:5]}"
        assert np.all(f64(o[0, h])[~live] == 0.0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_offset_and_mask(dev, d, causal):
    Nq, Nk = 200, 600
    _check(dev, 1, 2, Nq, Nk, d, causal, dtype="f32", in_seed=5 + d)
    mask = _mask(Nq, Nk, 128, 128, seed=9 + d, empty_row=0)
    _check(dev, 1, 2, Nq, Nk, d, causal, mask, dtype="f32", in_seed=6 + d)


@pytest.mark.parametrize("d", [64, 128])
def test_square_plain_call_is_bitwise_fa_fwd_bwd(dev, d):
    B, H, N = 2, 2, 700
    x = gen(B, H, N, d, seed=17 + d, with_do=True, dev=dev)
    for causal in (False, True):
        o0, l0 = fa.fa_fwd(x["q"], x["k"], x["v"], causal=causal)
        o1, l1 = fa.fa_fwd_general(x["q"], x["k"], x["v"], causal=causal)
        g0 = fa.fa_bwd(x["q"], x["k"], x["v"], o0, x["do"], l0, causal=causal)
        g1 = fa.fa_bwd_general(x["q"], x["k"], x["v"], o1, x["do"], l1,
                               causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
        for a, b in zip(g0, g1):
            assert torch.equal(a, b)


def test_offset_metric_head_shape(dev):
    # A 1024-token chunk at the end of an 8192-token context, B=1 H=8
    # d=128 causal: whole heads, forward and backward.
    _check(dev, 1, 8, 1024, 8192, 128, True, in_seed=123,
           heads=[(0, 0), (0, 7)])
