"""Pins for the dropout oracle (``oracle/dropout.py``).

Every check takes the dropout oracle module as its argument, so the same
checks run against the real oracle (``test_oracle.py``) and against broken
copies of it (``test_oracle_mutations.py``).

Sources of truth, none of which is the dropout oracle itself:
  * the published known-answer values of Philox4x32-10
    (``tests/golden/philox4x32_10_kat.json``, with their citation);
  * the element-to-counter mapping evaluated with plain Python integers
    element by element;
  * the dropout-free oracle (``oracle/attention.py``, pinned on its own) for
    t = 0 and for the softmax statistics, which dropout leaves unchanged;
  * probability: the kept fraction is binomial with p = 1 - t/256, and the
    dropped-and-rescaled output is unbiased over seeds;
  * central finite differences of the dropout forward for its backward;
  * brute force with plain Python loops on a tiny case.
"""

import itertools
import json
import math
import os

import numpy as np

from oracle import attention as plain

KAT = os.path.join(os.path.dirname(__file__), "golden",
                   "philox4x32_10_kat.json")


def _close(x, y, tol, what):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, f"{what}: shape {x.shape} vs {y.shape}"
    err = np.max(np.abs(x - y)) if x.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def check_philox_kat(drp):
    """The generator reproduces the published known-answer vectors."""
    with open(KAT) as f:
        vectors = json.load(f)["vectors"]
    for vec in vectors:
        ctr = np.array([int(w, 16) for w in vec["counter"]], dtype=np.uint64)
        key = tuple(int(w, 16) for w in vec["key"])
        got = drp.philox4x32_10(ctr, key)
        want = [int(w, 16) for w in vec["out"]]
        assert [int(w) for w in got] == want, (
            f"Philox4x32-10 {vec['counter']} {vec['key']}: "
            f"{[hex(int(w)) for w in got]} != {vec['out']}")


def _philox_py(ctr, key):
    """Philox4x32-10 on Python integers, one call (for the mapping check;
    the known-answer check pins the vectorised generator itself)."""
    x0, x1, x2, x3 = ctr
    k0, k1 = key
    for _ in range(10):
        p0, p1 = 0xD2511F53 * x0, 0xCD9E8D57 * x2
        x0, x1, x2, x3 = ((p1 >> 32) ^ x1 ^ k0, p1 & 0xFFFFFFFF,
                          (p0 >> 32) ^ x3 ^ k1, p0 & 0xFFFFFFFF)
        k0, k1 = (k0 + 0x9E3779B9) & 0xFFFFFFFF, (k1 + 0xBB67AE85) & 0xFFFFFFFF
    return x0, x1, x2, x3


def check_mask_layout(drp):
    """Element (bh, i, j) takes byte (j & 3) of word (i & 3) of the call with
    counter (i >> 2, j >> 2, bh, q_pos0) and key (seed low, seed high)."""
    seed = 0x0123456789ABCDEF
    rows = [0, 1, 2, 3, 5, 6, 17, 130, 1023, 4097]
    cols = [0, 1, 2, 3, 4, 7, 9, 255, 1000, 8191]
    for bh, off in ((0, 0), (3, 0), (63, 0), (3, 5), (1, 4096)):
        got = (drp.dropout_bytes(bh, rows, cols, seed) if off == 0 else
               drp.dropout_bytes(bh, rows, cols, seed, off))
        for a, i in enumerate(rows):
            for b, j in enumerate(cols):
                w = _philox_py((i >> 2, j >> 2, bh, off),
                               (seed & 0xFFFFFFFF, seed >> 32))[i & 3]
                want = (w >> (8 * (j & 3))) & 0xFF
                assert int(got[a, b]) == want, (
                    f"byte of (bh={bh}, i={i}, j={j}, q_pos0={off}): "
                    f"{int(got[a, b])} != {want}")


def check_keep_fraction(drp):
    """t = 0 keeps every element; otherwise the kept fraction is binomial
    with p = 1 - t/256 (within 5 standard deviations on 2^20 elements), and
    the bytes are uniform over 0..255 (chi-square with 255 degrees of
    freedom below its 0.9999 quantile, ~360)."""
    n = 1024
    for t in (0, 1, 26, 128, 255):
        z = drp.dropout_keep(7, n, n, 12345 + t, t)
        frac = z.mean()
        if t == 0:
            assert z.all(), "t = 0 must keep every element"
            continue
        p = 1.0 - t / 256.0
        sd = math.sqrt(p * (1 - p) / z.size)
        assert abs(frac - p) <= 5 * sd, f"t={t}: kept {frac:.5f}, want {p:.5f}"
    u = drp.dropout_bytes(2, np.arange(n), np.arange(n), 99).ravel()
    counts = np.bincount(u, minlength=256)
    e = u.size / 256.0
    chi2 = float(((counts - e) ** 2 / e).sum())
    assert chi2 < 360.0, f"byte histogram chi-square {chi2:.1f}"


def check_threshold(drp):
    """t = round(256 p), in [0, 255]."""
    assert drp.dropout_threshold(0.0) == 0
    assert drp.dropout_threshold(0.1) == 26
    assert drp.dropout_threshold(0.5) == 128
    assert drp.dropout_threshold(255 / 256) == 255
    for bad in (-0.1, 0.999, 1.0):
        try:
            drp.dropout_threshold(bad)
        except ValueError:
            continue
        raise AssertionError(f"p = {bad} accepted")


def check_no_dropout_is_plain(drp):
    """t = 0 gives the dropout-free oracle's O, LSE and gradients; for any t
    the LSE is that of the undropped softmax."""
    r = np.random.default_rng(31)
    for n, d, causal in ((1, 4, False), (9, 8, True), (37, 16, False)):
        q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
        O0, L0 = plain.attention_fwd_head(q, k, v, 0.5, causal)
        O, L = drp.attention_fwd_dropout_head(q, k, v, 0.5, causal, 0, 5, 1)
        _close(O, O0, 1e-13, "t=0 O")
        _close(L, L0, 1e-13, "t=0 LSE")
        g0 = plain.attention_bwd_head(q, k, v, do, 0.5, causal)
        g = drp.attention_bwd_dropout_head(q, k, v, do, 0.5, causal, 0, 5, 1)
        for name, a, b in zip(("dQ", "dK", "dV"), g, g0):
            _close(a, b, 1e-12, f"t=0 {name}")
        _, Lt = drp.attention_fwd_dropout_head(q, k, v, 0.5, causal, 77, 5, 1)
        _close(Lt, L0, 1e-13, "LSE with dropout")


def check_unbiased(drp):
    """E[P~] = P: the mean over 600 seeds of the dropped output is the
    undropped output (within 5 standard errors per element)."""
    r = np.random.default_rng(32)
    n, d, t = 12, 4, 64
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    O0, _ = plain.attention_fwd_head(q, k, v, 0.8, True)
    outs = np.stack([drp.attention_fwd_dropout_head(q, k, v, 0.8, True, t,
                                                    1000 + s, 2)[0]
                     for s in range(600)])
    se = outs.std(axis=0) / math.sqrt(outs.shape[0]) + 1e-12
    z = np.abs(outs.mean(axis=0) - O0) / se
    assert z.max() <= 5.0, f"dropout mean off by {z.max():.1f} standard errors"


def check_finite_differences(drp):
    """With the mask fixed by the seed, central differences of
    L = sum(O * dO) match the dropout backward (relative 1e-6)."""
    r = np.random.default_rng(33)
    h = 1e-6
    for n, d, causal, t in ((2, 3, True, 128), (5, 2, False, 90),
                            (8, 4, True, 200)):
        q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
        grads = dict(zip("qkv", drp.attention_bwd_dropout_head(
            q, k, v, do, 0.7, causal, t, 4242, 5)))
        base = {"q": q, "k": k, "v": v}
        for name in "qkv":
            fd = np.zeros((n, d))
            for idx in itertools.product(range(n), range(d)):
                xp = {a: b.copy() for a, b in base.items()}
                xm = {a: b.copy() for a, b in base.items()}
                xp[name][idx] += h
                xm[name][idx] -= h
                Lp = np.sum(drp.attention_fwd_dropout_head(
                    xp["q"], xp["k"], xp["v"], 0.7, causal, t, 4242, 5)[0] * do)
                Lm = np.sum(drp.attention_fwd_dropout_head(
                    xm["q"], xm["k"], xm["v"], 0.7, causal, t, 4242, 5)[0] * do)
                fd[idx] = (Lp - Lm) / (2 * h)
            err = np.max(np.abs(fd - grads[name]))
            ref = max(1.0, np.max(np.abs(fd)))
            assert err / ref <= 1e-6, f"FD d{name} n={n} t={t}: {err:.2e}"


def check_brute_force_python(drp):
    """Plain Python loops for a tiny causal case: softmax of the visible
    scores, elements dropped by the mask, survivors scaled by 256/(256-t)."""
    r = np.random.default_rng(34)
    n, d, t, seed, bh = 6, 3, 100, 77, 4
    q, k, v = (r.standard_normal((n, d)).tolist() for _ in range(3))
    keep = drp.dropout_keep(bh, n, n, seed, t)
    O, _ = drp.attention_fwd_dropout_head(np.array(q), np.array(k),
                                          np.array(v), 0.9, True, t, seed, bh)
    for i in range(n):
        s = [0.9 * sum(q[i][c] * k[j][c] for c in range(d))
             for j in range(i + 1)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        tot = sum(e)
        for c in range(d):
            want = sum((e[j] / tot) * (256.0 / (256 - t)) * v[j][c]
                       for j in range(i + 1) if keep[i, j])
            assert abs(O[i, c] - want) <= 1e-12, f"O[{i},{c}]"


def check_row_subsets(drp):
    """The row-restricted forward and dQ equal the full-head results on those
    rows (the full-head functions are pinned above)."""
    r = np.random.default_rng(35)
    for n, d, causal, t in ((40, 8, True, 51), (33, 4, False, 200)):
        q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
        rows = np.array([0, 3, 4, 17, n - 1])
        O, L = drp.attention_fwd_dropout_head(q, k, v, 0.6, causal, t, 9, 3)
        Or, Lr = drp.attention_fwd_dropout_head(q, k, v, 0.6, causal, t, 9, 3,
                                                rows=rows)
        _close(Or, O[rows], 1e-13, "forward rows")
        _close(Lr, L[rows], 1e-13, "LSE rows")
        dq = drp.attention_bwd_dropout_head(q, k, v, do, 0.6, causal, t, 9,
                                            3)[0]
        dqr = drp.attention_dq_dropout_rows(q, k, v, do, 0.6, causal, t, 9, 3,
                                            rows)
        _close(dqr, dq[rows], 1e-12, "dQ rows")


def check_d_identity(drp):
    """sum_j P_ij dP_ij = sum_c dO_ic O_ic: the row statistic the backward
    needs can be formed from the dropout forward's output (P from the
    dropout-free oracle, Z from the mask function, dP from its definition)."""
    r = np.random.default_rng(36)
    n, d, t, seed, bh = 23, 6, 77, 31337, 2
    for causal in (False, True):
        q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
        S = 0.5 * (q @ k.T)
        S = np.where(plain.visible(np.arange(n), n, causal), S, -np.inf)
        S = S - S.max(axis=1, keepdims=True)
        P = np.exp(S) / np.exp(S).sum(axis=1, keepdims=True)
        Z = drp.dropout_keep(bh, n, n, seed, t)
        dP = np.where(Z, do @ v.T, 0.0) * 256.0 / (256.0 - t)
        O, _ = drp.attention_fwd_dropout_head(q, k, v, 0.5, causal, t, seed, bh)
        _close((P * dP).sum(axis=1), (do * O).sum(axis=1), 1e-12, "D identity")


def _torch_dropout(q, k, v, do, scale, vis, keep, t):
    """PyTorch float64 autograd of O = (Z * softmax(S) * 256/(256-t)) V with
    S = scale Q K^T masked by the element mask ``vis`` (every row has a
    visible key)."""
    import torch
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True)
                  for x in (q, k, v))
    S = (scale * tq @ tk.T).masked_fill(~torch.tensor(vis), float("-inf"))
    P = torch.softmax(S, dim=1)
    Pd = P * torch.tensor(keep, dtype=torch.float64) * (256.0 / (256.0 - t))
    o = Pd @ tv
    o.backward(torch.tensor(do, dtype=torch.float64))
    lse = torch.logsumexp(S, dim=1)
    return (o.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(),
            tk.grad.numpy(), tv.grad.numpy())


def check_block_mask_and_offset(drp):
    """Dropout with a block mask and with fewer queries than keys (the causal
    rule at position q_pos0 + r): forward, LSE and gradients against
    PyTorch's float64 autograd of the definition, with the element mask built
    here with Python loops and Z taken from the keep function at the same
    offset (its layout pinned above element by element).  Rows with no
    visible key get O = 0, LSE = -inf and dQ = 0; the row-restricted dQ
    takes the same mask and offset."""
    r = np.random.default_rng(37)
    d, bm_, bn_, t, seed, bh = 4, 2, 3, 90, 2024, 3
    for n_q, n_k in ((5, 9), (7, 7), (2, 6)):
        off = n_k - n_q
        q, do = r.standard_normal((n_q, d)), r.standard_normal((n_q, d))
        k, v = r.standard_normal((n_k, d)), r.standard_normal((n_k, d))
        mask = (r.random((-(-n_q // bm_), -(-n_k // bn_))) < 0.6).astype(
            np.uint8)
        mask[0, 0] = 1
        mask[-1, :] = 0                       # the last rows see nothing
        keep = drp.dropout_keep(bh, n_q, n_k, seed, t, off)
        for causal in (False, True):
            vis = np.array([[(not causal or j <= off + i) and
                             mask[i // bm_][j // bn_] != 0
                             for j in range(n_k)] for i in range(n_q)])
            live = vis.any(axis=1)
            assert not live.all()
            e2 = vis.copy()
            e2[~live] = True
            To, Tl, Tdq, Tdk, Tdv = _torch_dropout(
                q, k, v, np.where(live[:, None], do, 0.0), 0.7, e2, keep, t)
            kw = dict(block_mask=mask, block_m=bm_, block_n=bn_, q_pos0=off)
            O, L = drp.attention_fwd_dropout_head(q, k, v, 0.7, causal, t,
                                                  seed, bh, **kw)
            dq, dk, dv = drp.attention_bwd_dropout_head(q, k, v, do, 0.7,
                                                        causal, t, seed, bh,
                                                        **kw)
            tag = f"masked dropout {n_q}x{n_k} causal={causal}"
            _close(O[live], To[live], 1e-12, tag + " O")
            _close(L[live], Tl[live], 1e-12, tag + " LSE")
            assert np.all(O[~live] == 0.0) and np.all(np.isneginf(L[~live]))
            _close(dq[live], Tdq[live], 1e-12, tag + " dQ")
            assert np.all(dq[~live] == 0.0), tag + " empty dQ"
            _close(dk, Tdk, 1e-12, tag + " dK")
            _close(dv, Tdv, 1e-12, tag + " dV")
            rows = np.array([0, n_q - 1])
            dqr = drp.attention_dq_dropout_rows(q, k, v, do, 0.7, causal, t,
                                                seed, bh, rows, **kw)
            _close(dqr, dq[rows], 1e-12, tag + " dQ rows")
            Or, Lr = drp.attention_fwd_dropout_head(q, k, v, 0.7, causal, t,
                                                    seed, bh, rows=rows, **kw)
            _close(Or, O[rows], 1e-13, tag + " forward rows")


ALL_CHECKS = [
    check_philox_kat,
    check_mask_layout,
    check_keep_fraction,
    check_threshold,
    check_no_dropout_is_plain,
    check_unbiased,
    check_finite_differences,
    check_brute_force_python,
    check_row_subsets,
    check_d_identity,
    check_block_mask_and_offset,
]
