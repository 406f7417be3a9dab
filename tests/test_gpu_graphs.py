"""The hot path under HIP-graph capture: the library enqueues only kernel
launches (no memsets, no allocations of its own), so a forward + backward
step (with or without dropout), and the split-KV decode, can be captured once
and replayed.  Every
replay is compared bitwise with the eager result, with the program's own
eager work and synchronisations between replays."""

import sys

import pytest
import torch

from exact_io_aware_amd import fa, workloads
from tests.test_gpu_parity import dev, gen  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    sys.stdout.flush()
    yield


def _replay_and_check(graph, outs, refs, noise):
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))        # eager work between replays
        noise.mul_(1.0001)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, refs)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs"


@pytest.mark.parametrize("causal", [False, True])
def test_graph_fwd_bwd_step(dev, causal):
    B, H, N, d = 2, 3, 384, 128
    x = gen(B, H, N, d, seed=81, with_do=True, dev=dev)
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    ref = [o.clone(), lse.clone(),
           *fa.fa_bwd(q, k, v, o, do, lse, causal=causal)]
    torch.cuda.synchronize()
    o_g, lse_g = torch.empty_like(o), torch.empty_like(lse)
    grads = [torch.empty(q.shape, dtype=torch.float32, device=dev)
             for _ in range(3)]
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8,
                     device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):         # warm-up on the capture stream
        fa.fa_fwd(q, k, v, causal=causal, out=o_g, lse=lse_g)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_fwd(q, k, v, causal=causal, out=o_g, lse=lse_g)
        fa.fa_bwd(q, k, v, o_g, do, lse_g, causal=causal, workspace=ws,
                  dq=grads[0], dk=grads[1], dv=grads[2])
    noise = torch.ones(1024, device=dev)
    _replay_and_check(g, [o_g, lse_g, *grads], ref, noise)


def test_graph_splitkv_decode(dev):
    B, H, Nq, Nk, d = 2, 4, 1, 3000, 128
    x = workloads.make_decode_inputs(B, H, Nq, Nk, d, seed=82, device=dev)
    o, lse = fa.fa_fwd_splitkv(x["q"], x["k"], x["v"], causal=True)
    ref = [o.clone(), lse.clone()]
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, 0),
                     dtype=torch.uint8, device=dev)
    o_g, lse_g = torch.empty_like(o), torch.empty_like(lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_fwd_splitkv(x["q"], x["k"], x["v"], causal=True, workspace=ws,
                          out=o_g, lse=lse_g)
    noise = torch.ones(1024, device=dev)
    _replay_and_check(g, [o_g, lse_g], ref, noise)


def test_graph_dropout_step(dev):
    # The dropout mask is a function of (seed, head, row, key) alone, so
    # replays reproduce the eager step bit for bit.
    B, H, N, d, p, seed = 1, 4, 320, 128, 0.2, 123456789
    x = gen(B, H, N, d, seed=83, with_do=True, dev=dev)
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    o, lse = fa.fa_fwd_dropout(q, k, v, p, seed, causal=True)
    ref = [o.clone(), lse.clone(),
           *fa.fa_bwd_dropout(q, k, v, o, do, lse, p, seed, causal=True)]
    torch.cuda.synchronize()
    o_g, lse_g = torch.empty_like(o), torch.empty_like(lse)
    grads = [torch.empty(q.shape, dtype=torch.float32, device=dev)
             for _ in range(3)]
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8,
                     device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):         # warm-up on the capture stream
        fa.fa_fwd_dropout(q, k, v, p, seed, causal=True, out=o_g, lse=lse_g)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_fwd_dropout(q, k, v, p, seed, causal=True, out=o_g, lse=lse_g)
        fa.fa_bwd_dropout(q, k, v, o_g, do, lse_g, p, seed, causal=True,
                          workspace=ws, dq=grads[0], dk=grads[1], dv=grads[2])
    noise = torch.ones(1024, device=dev)
    _replay_and_check(g, [o_g, lse_g, *grads], ref, noise)
