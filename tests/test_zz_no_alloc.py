"""fa_bwd_noalloc (the backward that allocates nothing) against fa_bwd.

Both run the same kernels; fa_bwd_noalloc takes its per-row workspace from
the library's own device scratch instead of the caller.  Two calls in a row
(the second smaller, so the scratch holds the first call's rows) must each
equal fa_bwd bitwise, and so must a call at the scratch's row limit.  The
last case also checks the result against the fp64 oracle at the bf16 bar.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_amd import fa, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.library()
    return torch.device("cuda:0")


def _case(dev, B, H, N, d, seed, causal, dtype="bf16"):
    print(f"\n[gpu case] fa_bwd_noalloc B={B} H={H} N={N} d={d} "
          f"causal={causal} {dtype}", flush=True)
    sys.stdout.flush()
    x = workloads.make_inputs(B, H, N, d, seed, dtype=dtype, with_do=True,
                              device=dev)
    scale = 1 / math.sqrt(d)
    o, lse = fa.fa_fwd(x["q"], x["k"], x["v"], scale=scale, causal=causal)
    ref = fa.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, scale=scale,
                    causal=causal)
    got = [torch.full_like(t, float("nan")) for t in ref]
    fa.fa_bwd_noalloc(x["q"], x["k"], x["v"], o, x["do"], lse, *got,
                      scale=scale, causal=causal)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), f"{name}: fa_bwd_noalloc != fa_bwd"
    return x, got, scale


def test_two_calls_second_smaller(dev):
    _case(dev, 2, 4, 1000, 128, seed=501, causal=True)
    _case(dev, 1, 2, 300, 64, seed=502, causal=False)
    _case(dev, 1, 1, 77, 64, seed=503, causal=True, dtype="f32")


def test_at_the_row_limit(dev):
    # B*H*N = 2^20 rows: the whole scratch.
    B, H, N, d = 1, 128, 8192, 64
    x, got, scale = _case(dev, B, H, N, d, seed=504, causal=True)
    for h in (0, 127):
        q, k, v, do = (x[n][0, h].double().cpu().numpy()
                       for n in ("q", "k", "v", "do"))
        ref = oracle.attention_bwd_head(q, k, v, do, scale, True)
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            gg = g[0, h].double().cpu().numpy()
            err = float(np.max(np.abs(gg - r)))
            rel = float(np.linalg.norm(gg - r) / np.linalg.norm(r))
            print(f"  head {h} {name}: max-abs {err:.3e} rel-rms {rel:.3e}",
                  flush=True)
            assert err <= 2e-2 and rel <= 5e-3, name


def test_too_large_is_rejected(dev):
    B, H, N, d = 1, 1, (1 << 20) + 128, 64
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(B, H, N, dtype=torch.float32, device=dev)
    g = torch.zeros(B, H, N, d, dtype=torch.float32, device=dev)
    with pytest.raises(fa.FAError) as e:
        fa.fa_bwd_noalloc(q, q, q, q, q, lse, g, g, g)
    assert e.value.status == 9
