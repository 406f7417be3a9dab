"""Seeded synthetic inputs shaped like the pages' attention workloads.

This module holds input generation only: shapes, seeds, distributions and
block masks.  It contains none of the attention arithmetic, so the HIP path,
the CPU oracle, the tests and the benchmark can all draw their inputs from it
without sharing any part of the method.

Recipe (the same for every workload):
  * a CPU ``torch.Generator`` seeded with the workload's seed draws Q, K, V
    (then dO for backward workloads) in that order with ``torch.randn`` in
    float32, shape (B, H, N, d);
  * each tensor is multiplied by ``sigma`` and then rounded to the workload
    dtype (round-to-nearest-even for bfloat16);
  * block masks are uint8 with the diagonal always on and a fixed count of
    off-diagonal blocks, round(frac * (T*T - T)), drawn without replacement by
    ``numpy.random.default_rng(seed)``.

Decoding workloads (one or a few new query tokens against a long context)
draw Q of shape (B, H, Nq, d) first, then K and V of shape (B, H, Nk, d),
from the same kind of generator.

Shapes follow the pages' workloads: a small fp32 single head (the simplified
one-row-per-block kernel of the page "FlashAttention：在线 softmax 与
IO-aware 注意力" runs fp32 at d = 64), the GPT-2 head shape at sequence 1K
(d = 64), long-sequence d = 128 heads at 8K and 4K, and a 16K block-sparse
setting like the long-range experiments of the page "FlashAttention:
IOを意識した高速かつメモリ効率の高い厳密なアテンション".  Synthetic
Gaussian tensors stand in for any dataset; none is used.
"""

import math

import numpy as np
import torch

__all__ = ["WORKLOADS", "DECODE_WORKLOADS", "CONTEXT_WORKLOADS", "workload",
           "make_inputs",
           "make_inputs_device", "make_decode_inputs", "block_mask",
           "workload_mask"]


def _w(name, B, H, N, d, dtype, causal, passes, seed, sigma=1.0,
       sparse=None):
    return dict(name=name, B=B, H=H, N=N, d=d, dtype=dtype, causal=causal,
                passes=passes, seed=seed, sigma=sigma,
                scale=1.0 / math.sqrt(d), sparse=sparse)


# The five workloads, keyed by a stable name.
WORKLOADS = {
    "fp32_1x1x256x64": _w("fp32_1x1x256x64", 1, 1, 256, 64, "f32",
                          (False,), ("fwd",), seed=1),
    "gpt2_8x16x1024x64": _w("gpt2_8x16x1024x64", 8, 16, 1024, 64, "bf16",
                            (False, True), ("fwd",), seed=2),
    "causal_2x32x8192x128": _w("causal_2x32x8192x128", 2, 32, 8192, 128,
                               "bf16", (True,), ("fwd", "bwd"), seed=3,
                               sigma=0.5),
    "bwd_4x16x4096x128": _w("bwd_4x16x4096x128", 4, 16, 4096, 128, "bf16",
                            (True,), ("fwd", "bwd"), seed=4),
    "sparse_1x16x16384x64": _w("sparse_1x16x16384x64", 1, 16, 16384, 64,
                               "bf16", (False,), ("fwd", "bwd"), seed=5,
                               sparse=dict(block=128, frac=0.25, seed=5)),
}


# Decoding: one new token per sequence against a 16K-token context, 16
# sequences of 32 heads of d = 128 (the long-context d = 128 head shape of
# the workloads above; [REAPER] section 3.6 describes the decoding shape, a
# single query row against the full K and V, without sizes).
DECODE_WORKLOADS = {
    "decode_16x32x1x16384x128": dict(
        name="decode_16x32x1x16384x128", B=16, H=32, Nq=1, Nk=16384, d=128,
        dtype="bf16", causal=(True,), passes=("decode",), seed=6, sigma=1.0,
        scale=1.0 / math.sqrt(128)),
}


# Context: the single fp32 head (N = 2048, d = 64) on which the simplified
# one-row-per-block kernel of the page "FlashAttention：在线 softmax 与
# IO-aware 注意力" reports its time and its max-abs error against standard
# attention (section 3).
CONTEXT_WORKLOADS = {
    "fp32_1x1x2048x64": _w("fp32_1x1x2048x64", 1, 1, 2048, 64, "f32",
                           (False,), ("fwd",), seed=7),
    # The metric shape with dropout on P (drop probability 0.1, a typical
    # training value; the pages give none), to price the fused dropout.
    "dropout_2x32x8192x128": dict(
        _w("dropout_2x32x8192x128", 2, 32, 8192, 128, "bf16", (True,),
           ("fwd", "bwd"), seed=3, sigma=0.5), p_drop=0.1, drop_seed=2024),
}


def workload(name):
    for table in (DECODE_WORKLOADS, CONTEXT_WORKLOADS):
        if name in table:
            return dict(table[name])
    return dict(WORKLOADS[name])


_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def make_inputs(B, H, N, d, seed, sigma=1.0, dtype="bf16", with_do=False,
                device="cpu"):
    """Q, K, V (and dO) drawn as described in the module docstring.

    Returns a dict of tensors on ``device`` in the requested dtype.
    """
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    names = ("q", "k", "v", "do") if with_do else ("q", "k", "v")
    out = {}
    for n in names:
        x = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x = x * sigma
        out[n] = x.to(_DTYPES[dtype]).to(device)
    return out


def make_inputs_device(B, H, N, d, seed, sigma=1.0, dtype="bf16",
                       with_do=False, device="cuda:0"):
    """Q, K, V (and dO) drawn on the device itself, for shapes too large to
    draw on the host in reasonable time: a ``torch.Generator`` of that
    device seeded with `seed` draws them in the order Q, K, V, dO with
    ``torch.randn`` (float32), each multiplied by sigma and rounded to the
    dtype.  (Not the same numbers as ``make_inputs`` for the same seed.)"""
    g = torch.Generator(device=device).manual_seed(int(seed))
    names = ("q", "k", "v", "do") if with_do else ("q", "k", "v")
    out = {}
    for n in names:
        x = torch.randn((B, H, N, d), generator=g, dtype=torch.float32,
                        device=device)
        if sigma != 1.0:
            x.mul_(sigma)
        out[n] = x.to(_DTYPES[dtype])
        del x
    return out


def make_decode_inputs(B, H, Nq, Nk, d, seed, sigma=1.0, dtype="bf16",
                       device="cpu"):
    """Q (B, H, Nq, d), then K and V (B, H, Nk, d), drawn as described in the
    module docstring."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    out = {}
    for n, rows in (("q", Nq), ("k", Nk), ("v", Nk)):
        x = torch.randn((B, H, rows, d), generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x = x * sigma
        out[n] = x.to(_DTYPES[dtype]).to(device)
    return out


def block_mask(t_m, t_n, seed, frac, diagonal=True):
    """uint8 block mask of shape (t_m, t_n).

    With ``diagonal`` the blocks (i, i) are always on; then
    round(frac * number of other blocks) of the other blocks are switched on,
    chosen uniformly without replacement.
    """
    m = np.zeros((t_m, t_n), dtype=np.uint8)
    idx = np.arange(t_m * t_n)
    if diagonal:
        diag = [i * t_n + i for i in range(min(t_m, t_n))]
        m.flat[diag] = 1
        idx = np.setdiff1d(idx, diag)
    count = int(round(frac * idx.size))
    rng = np.random.default_rng(seed)
    m.flat[rng.choice(idx, count, replace=False)] = 1
    return m


def workload_mask(w):
    """The block mask of a block-sparse workload (None for dense ones)."""
    sp = w.get("sparse")
    if not sp:
        return None
    t = -(-w["N"] // sp["block"])
    return block_mask(t, t, sp["seed"], sp["frac"])


def workload_inputs(name, with_do=None, device="cpu"):
    """Inputs of a named workload (dO included for backward workloads)."""
    w = workload(name)
    if with_do is None:
        with_do = "bwd" in w["passes"]
    return make_inputs(w["B"], w["H"], w["N"], w["d"], w["seed"], w["sigma"],
                       w["dtype"], with_do, device)
