"""The longest and largest problems: more than 2^31 elements per tensor at
N = 65536, so that every element offset past 2^31 is exercised (heads 256
and beyond start past it).  Checked against the fp64 oracle where it can be
evaluated one row at a time:
  * O, LSE and dQ at a uniform sample of query rows (full bar: the sample
    estimates the whole-tensor rel-RMS) and at edge rows (max-abs bar);
    each row is O(N d) for the oracle;
  * under the causal rule dK, dV of the last 64
    keys, which only the last 64 queries see, so their whole gradient comes
    from those rows;
and for every key through identities of the exact gradient that hold at
any size: sum_j dK_j = 0 (each row of dS sums to 0) and
sum_j dV_j = sum_i dO_i (each row of P sums to 1)."""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_amd import fa, workloads
from tests.test_gpu_parity import BF16_MAX_ABS, compare, dev, f64  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    sys.stdout.flush()
    yield


N = 65536
# Edge rows (first keys, tile boundaries, the end) and a uniform sample.  The
# bf16 bar's rel-RMS is defined over the whole tensor; the uniform sample
# estimates it, while the hand-picked rows are a biased sample (short rows
# have the largest dQ and the largest share of the D = dO . O rounding,
# D being formed from the stored bf16 O), so they get the max-abs bar only.
EDGE = [0, 1, 127, 128, 4097, 32768, 65471, 65535]


def _uniform(seed, count=48):
    return sorted(set(np.random.default_rng(seed).integers(0, N, count)
                      .tolist()) - set(EDGE))


def _max_abs(name, got, ref):
    err = float(np.max(np.abs(np.asarray(got) - np.asarray(ref))))
    print(f"  {name}: max-abs {err:.3e}", flush=True)
    assert err <= BF16_MAX_ABS, f"{name}: max-abs {err:.3e}"


def test_max_size_fwd_bwd_causal_d128(dev):
    B, H, d = 1, 272, 128
    scale = 1 / math.sqrt(d)
    x = workloads.make_inputs_device(B, H, N, d, seed=8, with_do=True,
                                     device=dev)
    assert x["q"].numel() > 2 ** 31
    o, lse = fa.fa_fwd(x["q"], x["k"], x["v"], scale=scale, causal=True)
    dq, dk, dv = fa.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse,
                           scale=scale, causal=True)
    torch.cuda.synchronize()
    uni = _uniform(8)
    tail = list(range(N - 64, N))
    for h in (0, 135, 255, 256, 271):
        qh, kh, vh, doh = (f64(x[n][0, h]) for n in ("q", "k", "v", "do"))
        O, L = oracle.attention_fwd_head(qh, kh, vh, scale, True, rows=uni)
        compare(f"O uniform rows h={h}", f64(o[0, h, uni]), O)
        compare(f"LSE uniform rows h={h}", f64(lse[0, h, uni]), L)
        O, L = oracle.attention_fwd_head(qh, kh, vh, scale, True, rows=EDGE)
        _max_abs(f"O edge rows h={h}", f64(o[0, h, EDGE]), O)
        _max_abs(f"LSE edge rows h={h}", f64(lse[0, h, EDGE]), L)
        sel = sorted(set(uni + EDGE + tail))
        dq_r, dk_t, dv_t = oracle.attention_bwd_rows(qh, kh, vh, doh, scale,
                                                     sel, True)
        pos = {r: t for t, r in enumerate(sel)}
        iu = [pos[r] for r in uni]
        ie = [pos[r] for r in EDGE]
        compare(f"dQ uniform rows h={h}", f64(dq[0, h, uni]), dq_r[iu])
        _max_abs(f"dQ edge rows h={h}", f64(dq[0, h, EDGE]), dq_r[ie])
        compare(f"dK last 64 keys h={h}", f64(dk[0, h, N - 64:]), dk_t[N - 64:])
        compare(f"dV last 64 keys h={h}", f64(dv[0, h, N - 64:]), dv_t[N - 64:])
        # Identities over all keys (loose: they catch wrong or missing tiles,
        # whose error is of the order of the norm itself).
        dkh, dvh = dk[0, h].double(), dv[0, h].double()
        r_k = float(dkh.sum(0).norm() / dkh.norm())
        r_v = float((dvh.sum(0) - x["do"][0, h].double().sum(0)).norm()
                    / dvh.norm())
        print(f"  identities h={h}: |sum dK|/|dK| {r_k:.2e}, "
              f"|sum dV - sum dO|/|dV| {r_v:.2e}", flush=True)
        assert r_k < 0.1 and r_v < 0.1


def test_max_size_fwd_noncausal_d64(dev):
    B, H, d = 2, 272, 64
    scale = 1 / math.sqrt(d)
    x = workloads.make_inputs_device(B, H, N, d, seed=9, device=dev)
    assert x["q"].numel() > 2 ** 31
    o, lse = fa.fa_fwd(x["q"], x["k"], x["v"], scale=scale)
    torch.cuda.synchronize()
    uni = _uniform(9)
    for b, h in ((0, 0), (0, 271), (1, 0), (1, 271)):
        qh, kh, vh = (f64(x[n][b, h]) for n in ("q", "k", "v"))
        O, L = oracle.attention_fwd_head(qh, kh, vh, scale, False, rows=uni)
        compare(f"O uniform rows ({b},{h})", f64(o[b, h, uni]), O)
        compare(f"LSE uniform rows ({b},{h})", f64(lse[b, h, uni]), L)
        O, L = oracle.attention_fwd_head(qh, kh, vh, scale, False, rows=EDGE)
        _max_abs(f"O edge rows ({b},{h})", f64(o[b, h, EDGE]), O)
        _max_abs(f"LSE edge rows ({b},{h})", f64(lse[b, h, EDGE]), L)


@pytest.mark.parametrize("d", [64, 128])
def test_many_tiny_heads(dev, d):
    # 65536 heads of 16 rows: the largest grids (one workgroup per head in
    # every pass) and per-head offsets up to 2^20 heads * 16 rows * d.
    B, H, n = 256, 256, 16
    scale = 1 / math.sqrt(d)
    x = workloads.make_inputs_device(B, H, n, d, seed=10 + d, with_do=True,
                                     device=dev)
    for causal in (False, True):
        o, lse = fa.fa_fwd(x["q"], x["k"], x["v"], scale=scale, causal=causal)
        dq, dk, dv = fa.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse,
                               scale=scale, causal=causal)
        torch.cuda.synchronize()
        for b, h in ((0, 0), (0, 255), (131, 77), (255, 255)):
            args = [f64(x[k][b, h]) for k in ("q", "k", "v", "do")]
            O, L = oracle.attention_fwd_head(*args[:3], scale, causal)
            compare(f"O ({b},{h})", f64(o[b, h]), O)
            compare(f"LSE ({b},{h})", f64(lse[b, h]), L)
            for name, got, r in zip(("dQ", "dK", "dV"), (dq, dk, dv),
                                    oracle.attention_bwd_head(*args, scale,
                                                              causal)):
                compare(f"{name} ({b},{h})", f64(got[b, h]), r)
