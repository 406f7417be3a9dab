"""GPU parity of the split-KV forward (fa_fwd_splitkv) against the fp64
oracle's decoding attention: a short block of Nq queries, the last Nq
positions of the sequence, against Nk keys cut into chunks whose results
are merged by the two-part softmax rule.  Cases span one and several query
tiles, one key tile per chunk up to hundreds, ragged key tails, causal rows
that a whole chunk hides, and the full decoding workload (sampled heads)."""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_amd import fa, workloads
from tests.test_gpu_parity import compare, dev, f64  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    sys.stdout.flush()
    yield


def _decode_case(dev, B, H, Nq, Nk, d, causal, splits, seed, heads=None):
    x = workloads.make_decode_inputs(B, H, Nq, Nk, d, seed, device=dev)
    scale = 1 / math.sqrt(d)
    o, lse = fa.fa_fwd_splitkv(x["q"], x["k"], x["v"], scale=scale,
                               causal=causal, n_splits=splits)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (B, H, Nq, d) and tuple(lse.shape) == (B, H, Nq)
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        O, L = oracle.attention_decode_head(
            f64(x["q"][b, h]), f64(x["k"][b, h]), f64(x["v"][b, h]), scale,
            causal)
        compare(f"O[{b},{h}]", f64(o[b, h]), O)
        compare(f"LSE[{b},{h}]", f64(lse[b, h]), L)
    return x, o, lse


@pytest.mark.parametrize("Nq,Nk,d,causal,splits", [
    (1, 1000, 128, False, 0),      # one query, ragged key tail, auto chunks
    (1, 4096, 64, True, 0),
    (1, 1, 64, False, 0),          # a single key
    (4, 777, 128, True, 3),        # a few queries, capped chunk count
    (5, 33, 128, False, 1000),     # one tile per chunk, 1-key last tile
    (37, 300, 64, True, 0),        # two query tiles, causal offset 263
    (64, 128, 128, True, 4),       # chunks hidden from the first rows
    (64, 64, 128, True, 0),        # Nq = Nk: the square causal rule
    (100, 5000, 128, True, 7),
    (32, 2048, 64, False, 64),
    # one query (the vector chunk pass): capped chunk counts, one tile per
    # chunk with a 1-key last tile, and the automatic plan at a small B*H
    (1, 777, 128, True, 5),
    (1, 33, 64, False, 1000),
    (1, 5000, 64, False, 0),
    (1, 16384, 128, True, 0),
    (1, 16, 128, True, 0),         # one key group exactly
    (1, 5, 128, False, 3),         # fewer keys than one group's slots
    (1, 96, 64, False, 3),         # one group per chunk at d = 64
])
def test_splitkv_shapes(dev, Nq, Nk, d, causal, splits):
    _decode_case(dev, 2, 3, Nq, Nk, d, causal, splits, seed=900 + Nq + Nk)


@pytest.mark.parametrize("d", [64, 128])
def test_splitkv_square_matches_fwd(dev, d):
    # With Nq = Nk both paths compute the same rows; each agrees with the
    # oracle, and they agree with each other to the bf16 bar.
    B, H, N = 1, 2, 300
    x = workloads.make_decode_inputs(B, H, N, N, d, seed=31, device=dev)
    scale = 1 / math.sqrt(d)
    for causal in (False, True):
        o1, l1 = fa.fa_fwd(x["q"], x["k"], x["v"], scale=scale, causal=causal)
        o2, l2 = fa.fa_fwd_splitkv(x["q"], x["k"], x["v"], scale=scale,
                                   causal=causal, n_splits=3)
        torch.cuda.synchronize()
        compare("O split vs fwd", f64(o2), f64(o1))
        compare("LSE split vs fwd", f64(l2), f64(l1))


def test_splitkv_chunk_count_invariance(dev):
    # Every chunk count gives the oracle's result (the merge is exact up to
    # rounding), from one chunk to one 32-key tile per chunk.
    B, H, Nq, Nk, d = 1, 2, 3, 640, 128
    x = workloads.make_decode_inputs(B, H, Nq, Nk, d, seed=32, device=dev)
    scale = 1 / math.sqrt(d)
    ref = [oracle.attention_decode_head(f64(x["q"][0, h]), f64(x["k"][0, h]),
                                        f64(x["v"][0, h]), scale, True)
           for h in range(H)]
    for splits in (1, 2, 5, 20):
        assert fa.fa_fwd_splitkv_chunks(B, H, Nq, Nk, d, splits) == splits
        o, lse = fa.fa_fwd_splitkv(x["q"], x["k"], x["v"], scale=scale,
                                   causal=True, n_splits=splits)
        torch.cuda.synchronize()
        for h in range(H):
            compare(f"O splits={splits} h={h}", f64(o[0, h]), ref[h][0])
            compare(f"LSE splits={splits} h={h}", f64(lse[0, h]), ref[h][1])


def test_splitkv_reused_workspace(dev):
    # One workspace serves two calls of different shapes back to back.
    d = 64
    need = max(fa.fa_fwd_splitkv_workspace_bytes(2, 2, 1, 3000, d, 0),
               fa.fa_fwd_splitkv_workspace_bytes(1, 3, 7, 500, d, 0))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    for (B, H, Nq, Nk), seed in (((2, 2, 1, 3000), 33), ((1, 3, 7, 500), 34)):
        x = workloads.make_decode_inputs(B, H, Nq, Nk, d, seed, device=dev)
        o, lse = fa.fa_fwd_splitkv(x["q"], x["k"], x["v"], causal=True,
                                   workspace=ws)
        torch.cuda.synchronize()
        for b in range(B):
            for h in range(H):
                O, L = oracle.attention_decode_head(
                    f64(x["q"][b, h]), f64(x["k"][b, h]), f64(x["v"][b, h]),
                    1 / math.sqrt(d), True)
                compare(f"O[{b},{h}]", f64(o[b, h]), O)
                compare(f"LSE[{b},{h}]", f64(lse[b, h]), L)


def test_splitkv_decode_workload(dev):
    # The decoding workload at full size in the launch configuration the
    # benchmark times (automatic chunks); four heads against the oracle,
    # every row finite.
    w = workloads.workload("decode_16x32x1x16384x128")
    x = workloads.make_decode_inputs(w["B"], w["H"], w["Nq"], w["Nk"], w["d"],
                                     w["seed"], w["sigma"], device=dev)
    o, lse = fa.fa_fwd_splitkv(x["q"], x["k"], x["v"], scale=w["scale"],
                               causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(6)
    for _ in range(4):
        b, h = int(rng.integers(w["B"])), int(rng.integers(w["H"]))
        O, L = oracle.attention_decode_head(
            f64(x["q"][b, h]), f64(x["k"][b, h]), f64(x["v"][b, h]),
            w["scale"], True)
        compare(f"O[{b},{h}]", f64(o[b, h]), O)
        compare(f"LSE[{b},{h}]", f64(lse[b, h]), L)


@pytest.mark.parametrize("d", [64, 128])
def test_splitkv_one_query_large_scores(dev, d):
    # Scores spread over a wide range (Q and K scaled by 3: S has a standard
    # deviation of about 9 at scale 1/sqrt(d)), so the running max moves
    # many times inside each chunk.
    B, H, Nk = 2, 2, 3000
    x = workloads.make_decode_inputs(B, H, 1, Nk, d, seed=35, device=dev)
    q = (x["q"].float() * 3).to(torch.bfloat16)
    k = (x["k"].float() * 3).to(torch.bfloat16)
    scale = 1 / math.sqrt(d)
    o, lse = fa.fa_fwd_splitkv(q, k, x["v"], scale=scale, causal=True)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            O, L = oracle.attention_decode_head(f64(q[b, h]), f64(k[b, h]),
                                                f64(x["v"][b, h]), scale, True)
            compare(f"O[{b},{h}]", f64(o[b, h]), O)
            compare(f"LSE[{b},{h}]", f64(lse[b, h]), L)


@pytest.mark.parametrize("d", [64, 128])
def test_splitkv_one_query_matches_general(dev, d):
    # The vector chunk pass (one query) and the matrix-core forward with the
    # query at the end of the sequence compute the same row; each agrees with
    # the oracle, and they agree with each other to the bf16 bar.
    B, H, Nk = 2, 3, 2500
    x = workloads.make_decode_inputs(B, H, 1, Nk, d, seed=36, device=dev)
    scale = 1 / math.sqrt(d)
    o1, l1 = fa.fa_fwd_general(x["q"], x["k"], x["v"], scale=scale,
                               causal=True)
    for splits in (0, 1, 7):
        o2, l2 = fa.fa_fwd_splitkv(x["q"], x["k"], x["v"], scale=scale,
                                   causal=True, n_splits=splits)
        torch.cuda.synchronize()
        compare(f"O vector vs general, splits={splits}", f64(o2), f64(o1))
        compare(f"LSE vector vs general, splits={splits}", f64(l2), f64(l1))
