"""Pins for the fp64 oracle: checks against what the pages and mathematics fix.

Every check takes the oracle module as its argument, so the same checks run
against the real oracle (``test_oracle.py``) and against deliberately broken
copies of it (``test_oracle_mutations.py``, which requires each planted
mistake to fail at least one check).

Sources of truth used here, none of which is the oracle itself:
  * the numbers printed in the worked examples of the page
    "출력을 누적해 메모리 이동을 줄이는 FlashAttention" (Fig. 1, 2, 3),
    stored with their citations in ``tests/golden/worked_examples.json``;
  * closed forms (equal scores give the mean of V, a single key gives V,
    adding a constant to a score row leaves O unchanged and raises LSE by it;
    the page "3 · FlashAttention", section 3.3, shows the rescale identity);
  * central finite differences of the forward for the backward;
  * PyTorch's own CPU float64 attention and autograd (a library routine);
  * brute force with plain Python loops on tiny inputs.
"""

import itertools
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "worked_examples.json")
PRINTED_TOL = 5e-4 + 1e-9          # 3 printed decimals
EXACT_TOL = 1e-12


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _close(x, y, tol, what):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, f"{what}: shape {x.shape} vs {y.shape}"
    err = np.max(np.abs(x - y)) if x.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# Worked examples (printed values)
# ---------------------------------------------------------------------------

def check_fig1_divide_last(orc):
    g = _golden()["fig1_divide_last"]
    q = np.array([[1.0]])
    k = np.array(g["scores"], dtype=float)[:, None]      # q.k_j = score j
    v = np.array(g["values"], dtype=float)
    trace = []
    O, lse, _ = orc.tiled_fwd_head(q, k, v, 1.0, 1, 2, trace=trace)
    _close(O[0], g["output"], PRINTED_TOL, "fig1 tiled O")
    _close(trace[-1]["l"][0], g["exp_sum"], PRINTED_TOL, "fig1 exp sum")
    _close(trace[-1]["a"][0], g["unnormalised_a"], PRINTED_TOL, "fig1 a")
    O2, _ = orc.attention_fwd_head(q, k, v, 1.0)
    _close(O2[0], g["output"], PRINTED_TOL, "fig1 materialised O")
    # With V = identity the output row is the probability row itself.
    P, _ = orc.attention_fwd_head(q, k, np.eye(2), 1.0)
    _close(P[0], g["probabilities"], PRINTED_TOL, "fig1 probabilities")
    # exp values after subtracting the max: exp(s - m) = P * l
    _close(P[0] * trace[-1]["l"][0], g["exp_after_max_shift"], PRINTED_TOL,
           "fig1 exp(s - m)")


def check_fig2_streamed_pairs(orc):
    g = _golden()["fig2_streamed_pairs"]
    q = np.array([[1.0]])
    k = np.array(g["scores"], dtype=float)[:, None]
    v = np.array(g["values"], dtype=float)
    trace = []
    O, lse, visited = orc.tiled_fwd_head(q, k, v, 1.0, 1, g["chunk"],
                                         trace=trace)
    assert visited == 3 and len(trace) == 3
    for t, exp in zip(trace, g["after_pair"]):
        _close(t["m"][0], exp["m"], 0.0, "fig2 m")
        _close(t["l"][0], exp["l"], PRINTED_TOL, "fig2 l")
        _close(t["a"][0], exp["a"], PRINTED_TOL, "fig2 a")
        if "rescale" in exp:
            _close(t["alpha"][0], exp["rescale"], PRINTED_TOL, "fig2 alpha")
            _close(t["l_rescaled"][0], exp["l_rescaled"], PRINTED_TOL,
                   "fig2 rescaled l")
            _close(t["a_rescaled"][0], exp["a_rescaled"], PRINTED_TOL,
                   "fig2 rescaled a")
        if "new_exp_sum" in exp:
            _close(t["l"][0] - t["l_rescaled"][0], exp["new_exp_sum"],
                   PRINTED_TOL, "fig2 new exp sum")
            _close(t["a"][0] - t["a_rescaled"][0], exp["new_a_term"],
                   PRINTED_TOL, "fig2 new a term")
    _close(O[0], g["output"], PRINTED_TOL, "fig2 tiled O")
    O2, lse2 = orc.attention_fwd_head(q, k, v, 1.0)
    _close(O2[0], g["output"], PRINTED_TOL, "fig2 materialised O")
    # LSE of the scores equals m + ln(l) of the final printed state.
    last = g["after_pair"][-1]
    _close(lse2[0], last["m"] + math.log(last["l"]), 1e-3, "fig2 LSE")


def check_fig3_two_query_tile(orc):
    g = _golden()["fig3_two_query_tile"]
    Q, K, V = (np.array(g[x], dtype=float) for x in ("Q", "K", "V"))
    for key, val in g["printed_inputs"].items():
        src = {"Q": Q, "K": K, "V": V}[key[0]]
        _close(src[int(key[1])], val, 0.0, f"fig3 printed {key}")
    S = Q @ K.T
    _close(S[:, :2], g["scores_tile1"], 0.0, "fig3 scores tile 1")
    _close(S[:, 2:], g["scores_tile2"], 0.0, "fig3 scores tile 2")
    trace = []
    O, _, visited = orc.tiled_fwd_head(Q, K, V, 1.0, g["Br"], g["Bc"],
                                       trace=trace)
    assert visited == 2
    t1, t2 = trace
    _close(t1["m"], g["tile1"]["m"], 0.0, "fig3 tile1 m")
    _close(t1["l"], g["tile1"]["l"], PRINTED_TOL, "fig3 tile1 l")
    _close(t1["a"], g["tile1"]["a"], PRINTED_TOL, "fig3 tile1 a")
    _close(t2["alpha"], g["tile2"]["rescale"], PRINTED_TOL, "fig3 alpha")
    _close(t2["m"], g["tile2"]["m"], 0.0, "fig3 tile2 m")
    _close(t2["l"], g["tile2"]["l"], PRINTED_TOL, "fig3 tile2 l")
    _close(t2["a"], g["tile2"]["a"], PRINTED_TOL, "fig3 tile2 a")
    _close(O, g["output"], PRINTED_TOL, "fig3 tiled O")
    O2, _ = orc.attention_fwd_head(Q, K, V, 1.0)
    _close(O2, g["output"], PRINTED_TOL, "fig3 materialised O")
    # exp values of the first tile: exp(S - m) per row
    P1, _ = orc.attention_fwd_head(Q, K[:2], np.eye(2), 1.0)
    _close(P1 * np.array(g["tile1"]["l"])[:, None], g["tile1"]["exps"],
           PRINTED_TOL, "fig3 tile1 exps")


# ---------------------------------------------------------------------------
# Closed forms and invariants
# ---------------------------------------------------------------------------

def check_single_key(orc):
    """N = 1: O = V and LSE = scale * q.k; dQ = dK = 0 and dV = dO."""
    r = _rng(11)
    for d in (1, 3, 8):
        q, k, v, do = (r.standard_normal((1, d)) for _ in range(4))
        scale = 0.37
        for causal in (False, True):
            O, lse = orc.attention_fwd_head(q, k, v, scale, causal)
            _close(O, v, EXACT_TOL, "N=1 O")
            _close(lse, [scale * float(q[0] @ k[0])], EXACT_TOL, "N=1 LSE")
            dq, dk, dv = orc.attention_bwd_head(q, k, v, do, scale, causal)
            _close(dq, np.zeros_like(q), EXACT_TOL, "N=1 dQ")
            _close(dk, np.zeros_like(k), EXACT_TOL, "N=1 dK")
            _close(dv, do, EXACT_TOL, "N=1 dV")


def check_causal_first_row(orc):
    """Causal row 0 sees only key 0: O_0 = V_0, LSE_0 = scale q_0.k_0."""
    r = _rng(12)
    q, k, v = (r.standard_normal((7, 5)) for _ in range(3))
    O, lse = orc.attention_fwd_head(q, k, v, 0.5, causal=True)
    _close(O[0], v[0], EXACT_TOL, "causal row 0 O")
    _close(lse[0], 0.5 * float(q[0] @ k[0]), EXACT_TOL, "causal row 0 LSE")


def check_equal_scores(orc):
    """Q = 0 makes every score 0: O_i is the mean of the visible V rows and
    LSE_i = ln(number of visible keys)."""
    r = _rng(13)
    n, d = 9, 4
    k, v = r.standard_normal((n, d)), r.standard_normal((n, 3))
    q = np.zeros((n, d))
    O, lse = orc.attention_fwd_head(q, k, v, 0.8)
    _close(O, np.tile(v.mean(axis=0), (n, 1)), EXACT_TOL, "equal scores O")
    _close(lse, np.full(n, math.log(n)), EXACT_TOL, "equal scores LSE")
    O, lse = orc.attention_fwd_head(q, k, v, 0.8, causal=True)
    prefix = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    _close(O, prefix, EXACT_TOL, "equal scores causal O")
    _close(lse, np.log(np.arange(1, n + 1)), EXACT_TOL,
           "equal scores causal LSE")


def check_normalisation(orc):
    """Rows of P sum to 1 (V = identity exposes P); V = 1 gives O = 1."""
    r = _rng(14)
    n, d = 11, 6
    q, k = r.standard_normal((n, d)), r.standard_normal((n, d))
    for causal in (False, True):
        P, _ = orc.attention_fwd_head(q, k, np.eye(n), 1.3, causal)
        _close(P.sum(axis=1), np.ones(n), 1e-14, "rows of P sum to 1")
        assert np.all(P >= 0)
        if causal:
            assert np.all(np.triu(P, 1) == 0.0), "causal P above diagonal"
        O, _ = orc.attention_fwd_head(q, k, np.ones((n, 2)), 1.3, causal)
        _close(O, np.ones((n, 2)), 1e-14, "V = 1 gives O = 1")


def check_shift_invariance(orc):
    """Adding c to every score of row i leaves O_i unchanged and adds c to
    LSE_i.  The shift is injected through an extra coordinate: keys get a
    last coordinate of 1 and query i a last coordinate of c / scale."""
    r = _rng(15)
    n, d, scale = 8, 5, 0.25
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    q[:, -1] = 0.0
    k[:, -1] = 1.0
    O0, l0 = orc.attention_fwd_head(q, k, v, scale)
    for c in (-50.0, 7.0, 1e3):
        for i in (0, 3, n - 1):
            qs = q.copy()
            qs[i, -1] = c / scale
            O1, l1 = orc.attention_fwd_head(qs, k, v, scale)
            _close(O1, O0, 1e-12, f"shift {c} O")
            expect = l0.copy()
            expect[i] += c
            _close(l1, expect, 1e-12 * max(1.0, abs(c)), f"shift {c} LSE")


def _torch_reference(q, k, v, do, scale, causal, elem_mask=None):
    import torch
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True)
                  for x in (q, k, v))
    mask = None
    n_q, n_k = q.shape[0], k.shape[0]
    allowed = torch.ones(n_q, n_k, dtype=torch.bool)
    if causal:
        allowed &= torch.ones(n_q, n_k, dtype=torch.bool).tril()
    if elem_mask is not None:
        allowed &= torch.tensor(elem_mask)
    mask = allowed
    o = torch.nn.functional.scaled_dot_product_attention(
        tq[None], tk[None], tv[None], attn_mask=mask[None], scale=scale)[0]
    o.backward(torch.tensor(do, dtype=torch.float64))
    lse = torch.logsumexp(
        (scale * tq @ tk.T).masked_fill(~mask, float("-inf")), dim=1)
    return (o.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(),
            tk.grad.numpy(), tv.grad.numpy())


def check_vs_torch_library(orc):
    """PyTorch's float64 CPU attention and autograd agree with the oracle
    (forward, LSE and all three gradients), causal and not, N != d."""
    r = _rng(16)
    for (n, d, dv) in ((13, 4, 3), (6, 9, 9), (32, 16, 16)):
        q, k = r.standard_normal((n, d)), r.standard_normal((n, d))
        v, do = r.standard_normal((n, dv)), r.standard_normal((n, dv))
        for causal in (False, True):
            scale = 1.0 / math.sqrt(d)
            To, Tl, Tdq, Tdk, Tdv = _torch_reference(q, k, v, do, scale,
                                                     causal)
            O, lse = orc.attention_fwd_head(q, k, v, scale, causal)
            dq, dk, dv_ = orc.attention_bwd_head(q, k, v, do, scale, causal)
            _close(O, To, 1e-12, "torch O")
            _close(lse, Tl, 1e-12, "torch LSE")
            _close(dq, Tdq, 1e-12, "torch dQ")
            _close(dk, Tdk, 1e-12, "torch dK")
            _close(dv_, Tdv, 1e-12, "torch dV")


def check_brute_force_python(orc):
    """Plain Python loops (no NumPy) on a tiny causal and non-causal case."""
    r = _rng(17)
    n, d = 4, 3
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    scale = 0.9
    for causal in (False, True):
        O, lse = orc.attention_fwd_head(q, k, v, scale, causal)
        for i in range(n):
            keys = [j for j in range(n) if (j <= i or not causal)]
            s = [scale * sum(q[i][t] * k[j][t] for t in range(d))
                 for j in keys]
            w = [math.exp(x) for x in s]
            tot = sum(w)
            for c in range(d):
                ref = sum(w[a] * v[j][c] for a, j in enumerate(keys)) / tot
                assert abs(O[i][c] - ref) < 1e-12, "brute force O"
            assert abs(lse[i] - math.log(tot)) < 1e-12, "brute force LSE"


# ---------------------------------------------------------------------------
# Backward: finite differences and identities
# ---------------------------------------------------------------------------

def check_finite_differences(orc):
    """Central differences of L = sum(O * dO) (h = 1e-6) match the oracle's
    gradients to a relative error of 1e-6 on tiny shapes."""
    r = _rng(18)
    h = 1e-6
    for n, d, causal in ((1, 2, False), (2, 3, True), (3, 4, False),
                         (5, 2, True), (8, 3, False), (8, 4, True)):
        scale = 0.7
        q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
        dq, dk, dv = orc.attention_bwd_head(q, k, v, do, scale, causal)
        grads = {"q": dq, "k": dk, "v": dv}
        base = {"q": q, "k": k, "v": v}
        for name in ("q", "k", "v"):
            fd = np.zeros((n, d))
            for idx in itertools.product(range(n), range(d)):
                xp = {kk: vv.copy() for kk, vv in base.items()}
                xm = {kk: vv.copy() for kk, vv in base.items()}
                xp[name][idx] += h
                xm[name][idx] -= h
                Lp = np.sum(orc.attention_fwd_head(
                    xp["q"], xp["k"], xp["v"], scale, causal)[0] * do)
                Lm = np.sum(orc.attention_fwd_head(
                    xm["q"], xm["k"], xm["v"], scale, causal)[0] * do)
                fd[idx] = (Lp - Lm) / (2 * h)
            err = np.max(np.abs(fd - grads[name]))
            ref = max(1.0, np.max(np.abs(fd)))
            assert err / ref <= 1e-6, (
                f"FD d{name} n={n} d={d} causal={causal}: {err:.2e}")


def check_bwd_identities(orc):
    """Each row of dS sums to zero, so the dK rows sum to zero per head; with
    Q = 0 every score is 0, so dK = 0 and (non-causal) every dV row is the
    mean of the dO rows."""
    r = _rng(19)
    n, d = 10, 6
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    for causal in (False, True):
        _, dk, _ = orc.attention_bwd_head(q, k, v, do, 0.6, causal)
        _close(dk.sum(axis=0), np.zeros(d), 1e-12, "sum of dK rows")
    _, dk, dv = orc.attention_bwd_head(np.zeros((n, d)), k, v, do, 0.6)
    _close(dk, np.zeros((n, d)), 1e-13, "Q = 0 gives dK = 0")
    _close(dv, np.tile(do.mean(axis=0), (n, 1)), 1e-13,
           "Q = 0 gives dV = mean dO")


# ---------------------------------------------------------------------------
# Tiling: exactness across tile shapes, FA1 = FA2 = definition
# ---------------------------------------------------------------------------

def check_tile_invariance(orc):
    """Blockwise results equal the materialising definition for any tile
    shape, ragged tails included ([TLDR] online-softmax section: the tiled
    result equals the all-columns softmax)."""
    r = _rng(20)
    n, d = 23, 5
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    bm = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    for causal in (False, True):
        for mask in (None, bm):
            kw = dict(block_mask=mask, block_m=8, block_n=8)
            O_ref, l_ref = orc.attention_fwd_head(q, k, v, 0.4, causal, **kw)
            for Br, Bc in ((1, 1), (2, 2), (3, 5), (16, 4), (4, 16),
                           (n, n), (64, 64)):
                O, l, _ = orc.tiled_fwd_head(q, k, v, 0.4, Br, Bc, causal,
                                             **kw)
                _close(O, O_ref, EXACT_TOL, f"FA2 tiles {Br}x{Bc}")
                _close(np.nan_to_num(l, neginf=-1e300),
                       np.nan_to_num(l_ref, neginf=-1e300), EXACT_TOL,
                       f"FA2 LSE {Br}x{Bc}")
                O1, l1 = orc.tiled_fwd_fa1_head(q, k, v, 0.4, Br, Bc, causal,
                                                **kw)
                _close(O1, O_ref, EXACT_TOL, f"FA1 tiles {Br}x{Bc}")
                _close(np.nan_to_num(l1, neginf=-1e300),
                       np.nan_to_num(l_ref, neginf=-1e300), EXACT_TOL,
                       f"FA1 LSE {Br}x{Bc}")


def check_causal_tile_count(orc):
    """Causal block skipping keeps exactly T(T+1)/2 of T*T square tiles (the
    page "3 · FlashAttention", causal question: about half of the blocks)."""
    for T in (1, 2, 5, 8):
        B = 4
        assert orc.causal_tiles_visited(T * B, B, B) == T * (T + 1) // 2
        r = _rng(21 + T)
        q, k, v = (r.standard_normal((T * B, 3)) for _ in range(3))
        _, _, visited = orc.tiled_fwd_head(q, k, v, 1.0, B, B, causal=True)
        assert visited == T * (T + 1) // 2
        _, _, visited = orc.tiled_fwd_head(q, k, v, 1.0, B, B, causal=False)
        assert visited == T * T


# ---------------------------------------------------------------------------
# Block-sparse masks
# ---------------------------------------------------------------------------

def check_block_sparse(orc):
    """All-ones mask equals dense; diagonal-only mask equals dense attention
    on each diagonal chunk; every 2 x 2 block mask at N = 8 with 4 x 4 blocks
    (and a ragged N = 7) agrees with PyTorch's attention under the expanded
    element mask; a row with no visible key gives O = 0, LSE = -inf."""
    r = _rng(30)
    n, d, blk = 12, 3, 4
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    T = n // blk
    ones = np.ones((T, T), dtype=np.uint8)
    for causal in (False, True):
        O_a, l_a = orc.attention_fwd_head(q, k, v, 0.5, causal, ones, blk, blk)
        O_d, l_d = orc.attention_fwd_head(q, k, v, 0.5, causal)
        _close(O_a, O_d, 0.0, "all-ones mask O")
        _close(l_a, l_d, 0.0, "all-ones mask LSE")
    diag = np.eye(T, dtype=np.uint8)
    O_g, l_g = orc.attention_fwd_head(q, k, v, 0.5, False, diag, blk, blk)
    for t in range(T):
        s = slice(t * blk, (t + 1) * blk)
        O_c, l_c = orc.attention_fwd_head(q[s], k[s], v[s], 0.5)
        _close(O_g[s], O_c, EXACT_TOL, "diagonal mask O")
        _close(l_g[s], l_c, EXACT_TOL, "diagonal mask LSE")
    for n_case in (8, 7):
        qq, kk, vv, dd = (x[:n_case] for x in (q, k, v, do))
        for bits in range(16):
            m = np.array([(bits >> b) & 1 for b in range(4)],
                         dtype=np.uint8).reshape(2, 2)
            elem = np.zeros((n_case, n_case), dtype=bool)
            for i in range(n_case):
                for j in range(n_case):
                    elem[i, j] = m[i // 4, j // 4] == 1
            for causal in (False, True):
                vis = elem & (np.tri(n_case, dtype=bool) if causal else True)
                O, lse = orc.attention_fwd_head(qq, kk, vv, 0.5, causal, m,
                                                4, 4)
                dq, dk, dv = orc.attention_bwd_head(qq, kk, vv, dd, 0.5,
                                                    causal, m, 4, 4)
                live = vis.any(axis=1)
                assert np.all(O[~live] == 0.0), "empty row O != 0"
                assert np.all(np.isneginf(lse[~live])), "empty row LSE"
                assert np.all(dq[~live] == 0.0), "empty row dQ"
                if live.any():
                    # PyTorch gives NaN on rows with nothing visible; compare
                    # the live rows, give empty rows a harmless mask and a
                    # zero upstream gradient so they add nothing to dK, dV.
                    e2 = vis.copy()
                    e2[~live] = True
                    To, Tl, Tdq, Tdk, Tdv = _torch_reference(
                        qq, kk, vv, np.where(live[:, None], dd, 0.0), 0.5,
                        False, e2)
                    _close(O[live], To[live], 1e-12, f"mask {bits} O")
                    _close(lse[live], Tl[live], 1e-12, f"mask {bits} LSE")
                    _close(dq[live], Tdq[live], 1e-12, f"mask {bits} dQ")
                    _close(dk, Tdk, 1e-12, f"mask {bits} dK")
                    _close(dv, Tdv, 1e-12, f"mask {bits} dV")


def check_decode(orc):
    """Decoding (Nq queries = the last Nq of Nk tokens, [REAPER] 3.6):
    with Nq = Nk it is the square problem; its rows equal the last Nq rows of
    the square causal problem over the same tokens; a single causal query
    sees every key; and it agrees with PyTorch's float64 attention under the
    explicit bottom-right mask (key j visible to row r iff j <= Nk - Nq + r,
    built here with Python loops)."""
    r = _rng(40)
    d = 5
    for n_k in (1, 6, 13):
        k, v = r.standard_normal((n_k, d)), r.standard_normal((n_k, 3))
        q_all = r.standard_normal((n_k, d))
        for causal in (False, True):
            O_sq, l_sq = orc.attention_fwd_head(q_all, k, v, 0.6, causal)
            O_d, l_d = orc.attention_decode_head(q_all, k, v, 0.6, causal)
            _close(O_d, O_sq, 0.0, "decode Nq = Nk O")
            _close(l_d, l_sq, 0.0, "decode Nq = Nk LSE")
            for n_q in range(1, n_k + 1):
                q = q_all[n_k - n_q:]
                O, l = orc.attention_decode_head(q, k, v, 0.6, causal)
                _close(O, O_sq[n_k - n_q:], EXACT_TOL, "decode = last rows O")
                _close(l, l_sq[n_k - n_q:], EXACT_TOL, "decode = last rows LSE")
        O1, l1 = orc.attention_decode_head(q_all[-1:], k, v, 0.6, True)
        O0, l0 = orc.attention_decode_head(q_all[-1:], k, v, 0.6, False)
        _close(O1, O0, 0.0, "one causal query sees every key")
        _close(l1, l0, 0.0, "one causal query LSE")
    n_q, n_k = 3, 8
    q, k = r.standard_normal((n_q, d)), r.standard_normal((n_k, d))
    v, do = r.standard_normal((n_k, 4)), r.standard_normal((n_q, 4))
    elem = np.array([[j <= n_k - n_q + i for j in range(n_k)]
                     for i in range(n_q)])
    To, Tl, _, _, _ = _torch_reference(q, k, v, do, 0.45, False, elem)
    O, lse = orc.attention_decode_head(q, k, v, 0.45, True)
    _close(O, To, 1e-12, "decode vs torch O")
    _close(lse, Tl, 1e-12, "decode vs torch LSE")


def check_bwd_rows(orc):
    """The row-restricted backward against PyTorch's float64 autograd (mask
    expanded here with Python loops): dQ of chosen rows equals the full dQ
    at those rows; the rows' contributions to dK and dV, summed over a
    partition of all rows, equal the full dK and dV; under the causal rule
    the last T rows alone give the whole dK, dV of the last T keys.  Causal
    and not, with and without a block mask."""
    r = _rng(41)
    n, d, dv, blk = 11, 5, 3, 4
    q, k = r.standard_normal((n, d)), r.standard_normal((n, d))
    v, do = r.standard_normal((n, dv)), r.standard_normal((n, dv))
    bm = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    for causal in (False, True):
        for mask in (None, bm):
            elem = None
            if mask is not None:
                elem = np.array([[mask[i // blk][j // blk] != 0
                                  for j in range(n)] for i in range(n)])
            _, _, Tdq, Tdk, Tdv = _torch_reference(q, k, v, do, 0.7, causal,
                                                   elem)
            sel = [0, 3, 7, 10]
            dq_rows, _, _ = orc.attention_bwd_rows(q, k, v, do, 0.7, sel,
                                                   causal, mask, blk, blk)
            _close(dq_rows, Tdq[sel], 1e-12, "bwd rows dQ")
            dk_sum, dv_sum = np.zeros_like(k), np.zeros_like(v)
            for part in ([0, 1, 2, 3, 4], [5, 6], [7, 8, 9, 10]):
                _, dk_p, dv_p = orc.attention_bwd_rows(q, k, v, do, 0.7, part,
                                                       causal, mask, blk, blk)
                dk_sum += dk_p
                dv_sum += dv_p
            _close(dk_sum, Tdk, 1e-12, "bwd rows: dK contributions sum")
            _close(dv_sum, Tdv, 1e-12, "bwd rows: dV contributions sum")
            if causal:
                _, dk_t, dv_t = orc.attention_bwd_rows(
                    q, k, v, do, 0.7, [8, 9, 10], causal, mask, blk, blk)
                _close(dk_t[8:], Tdk[8:], 1e-12, "causal tail keys dK")
                _close(dv_t[8:], Tdv[8:], 1e-12, "causal tail keys dV")


def check_batched_wrappers(orc):
    """The batched forms ``attention_fwd`` and ``attention_bwd`` (every
    workload parity test and the smoke test go through them) against
    PyTorch's float64 attention and autograd, head by head: distinct data in
    every (b, h), non-square blocks (block_m = 4, block_n = 2, so a swap of
    the two changes the visible set), a block row with no visible key, causal
    and not, a ragged N; the element mask is expanded here with Python
    loops.  Also: ``heads`` restricts the work and leaves the other heads
    NaN, and ``workers`` > 1 gives the same values."""
    r = _rng(42)
    B, H, n, d, dv = 2, 3, 11, 4, 3
    bm_, bn_ = 4, 2
    Q, K = r.standard_normal((B, H, n, d)), r.standard_normal((B, H, n, d))
    V, dO = r.standard_normal((B, H, n, dv)), r.standard_normal((B, H, n, dv))
    mask = (r.random((3, 6)) < 0.6).astype(np.uint8)
    mask[1] = 0                                  # rows 4..7 see no key
    mask[0, 0] = mask[2, 5] = 1
    assert not np.array_equal(mask, mask.T[:3, :3])
    scale = 0.55
    for causal in (False, True):
        for m in (None, mask):
            O, lse = orc.attention_fwd(Q, K, V, scale, causal, m, bm_, bn_)
            dq, dk, dv_ = orc.attention_bwd(Q, K, V, dO, scale, causal, m,
                                            bm_, bn_)
            for b in range(B):
                for h in range(H):
                    vis = np.array([[(j <= i or not causal) and
                                     (m is None or m[i // bm_][j // bn_] != 0)
                                     for j in range(n)] for i in range(n)])
                    live = vis.any(axis=1)
                    e2 = vis.copy()
                    e2[~live] = True
                    To, Tl, Tdq, Tdk, Tdv = _torch_reference(
                        Q[b, h], K[b, h], V[b, h],
                        np.where(live[:, None], dO[b, h], 0.0), scale, False,
                        e2)
                    tag = f"batched ({b},{h}) causal={causal} mask={m is not None}"
                    _close(O[b, h][live], To[live], 1e-12, tag + " O")
                    _close(lse[b, h][live], Tl[live], 1e-12, tag + " LSE")
                    assert np.all(O[b, h][~live] == 0.0), tag + " empty O"
                    assert np.all(np.isneginf(lse[b, h][~live])), tag
                    _close(dq[b, h][live], Tdq[live], 1e-12, tag + " dQ")
                    assert np.all(dq[b, h][~live] == 0.0), tag + " empty dQ"
                    _close(dk[b, h], Tdk, 1e-12, tag + " dK")
                    _close(dv_[b, h], Tdv, 1e-12, tag + " dV")
    O_all, l_all = orc.attention_fwd(Q, K, V, scale, True, mask, bm_, bn_)
    O_one, l_one = orc.attention_fwd(Q, K, V, scale, True, mask, bm_, bn_,
                                     heads=[(1, 2)])
    assert np.array_equal(O_one[1, 2], O_all[1, 2])
    assert np.isnan(O_one[0]).all() and np.isnan(l_one[1, :2]).all()
    O_t, l_t = orc.attention_fwd(Q, K, V, scale, True, mask, bm_, bn_,
                                 workers=4)
    _close(O_t, O_all, 1e-13, "threaded O")
    _close(np.nan_to_num(l_t, neginf=-1e300),
           np.nan_to_num(l_all, neginf=-1e300), 1e-13, "threaded LSE")
    g_all = orc.attention_bwd(Q, K, V, dO, scale, True, mask, bm_, bn_)
    g_t = orc.attention_bwd(Q, K, V, dO, scale, True, mask, bm_, bn_,
                            workers=4)
    for a, t in zip(g_all, g_t):
        _close(t, a, 1e-13, "threaded gradients")


def check_offset_queries(orc):
    """Fewer queries than keys, the queries being the last Nq tokens
    (q_pos0 = Nk - Nq; decoding and prompts fed in chunks, [REAPER] 3.6):
    forward and backward against PyTorch's float64 attention and autograd
    under the explicit element mask (the causal rule at position q_pos0 + r
    AND a block mask of ceil(Nq/bm) x ceil(Nk/bn) entries, built here with
    Python loops), including rows that see no key; the causal forward equals
    ``attention_decode_head``; the causal backward equals that of the square
    problem over all Nk tokens whose first Nk - Nq query rows carry dO = 0
    (such rows contribute nothing to dK and dV); the row-restricted backward
    and the batched wrappers take the same offset."""
    r = _rng(43)
    d, dv, bm_, bn_, scale = 4, 3, 2, 3, 0.6
    for n_q, n_k in ((3, 8), (5, 5), (1, 7), (6, 13)):
        off = n_k - n_q
        q, k = r.standard_normal((n_q, d)), r.standard_normal((n_k, d))
        v, do = r.standard_normal((n_k, dv)), r.standard_normal((n_q, dv))
        mask = (r.random((-(-n_q // bm_), -(-n_k // bn_))) < 0.6).astype(
            np.uint8)
        mask[0, 0] = 1
        for causal in (False, True):
            for m in (None, mask):
                vis = np.array([[(not causal or j <= off + i) and
                                 (m is None or m[i // bm_][j // bn_] != 0)
                                 for j in range(n_k)] for i in range(n_q)])
                live = vis.any(axis=1)
                e2 = vis.copy()
                e2[~live] = True
                To, Tl, Tdq, Tdk, Tdv = _torch_reference(
                    q, k, v, np.where(live[:, None], do, 0.0), scale, False,
                    e2)
                tag = f"offset {n_q}x{n_k} causal={causal} mask={m is not None}"
                O, lse = orc.attention_fwd_head(q, k, v, scale, causal, m, bm_,
                                                bn_, q_pos0=off)
                dq, dk, dv_ = orc.attention_bwd_head(q, k, v, do, scale,
                                                     causal, m, bm_, bn_,
                                                     q_pos0=off)
                _close(O[live], To[live], 1e-12, tag + " O")
                _close(lse[live], Tl[live], 1e-12, tag + " LSE")
                assert np.all(O[~live] == 0.0), tag + " empty O"
                assert np.all(np.isneginf(lse[~live])), tag + " empty LSE"
                _close(dq[live], Tdq[live], 1e-12, tag + " dQ")
                assert np.all(dq[~live] == 0.0), tag + " empty dQ"
                _close(dk, Tdk, 1e-12, tag + " dK")
                _close(dv_, Tdv, 1e-12, tag + " dV")
                dq_r, dk_r, dv_r = orc.attention_bwd_rows(
                    q, k, v, do, scale, np.arange(n_q), causal, m, bm_, bn_,
                    q_pos0=off)
                _close(dq_r, dq, 1e-12, tag + " rows dQ")
                _close(dk_r, dk, 1e-12, tag + " rows dK")
                _close(dv_r, dv_, 1e-12, tag + " rows dV")
        O_d, l_d = orc.attention_decode_head(q, k, v, scale, True)
        O, lse = orc.attention_fwd_head(q, k, v, scale, True, q_pos0=off)
        _close(O, O_d, EXACT_TOL, "offset forward = decode O")
        _close(lse, l_d, EXACT_TOL, "offset forward = decode LSE")
        q_full = np.concatenate([r.standard_normal((off, d)), q])
        do_full = np.concatenate([np.zeros((off, dv)), do])
        gq, gk, gv = orc.attention_bwd_head(q_full, k, v, do_full, scale, True)
        dq, dk, dv_ = orc.attention_bwd_head(q, k, v, do, scale, True,
                                             q_pos0=off)
        _close(dq, gq[off:], EXACT_TOL, "offset = padded square dQ")
        _close(dk, gk, EXACT_TOL, "offset = padded square dK")
        _close(dv_, gv, EXACT_TOL, "offset = padded square dV")
    B, H, n_q, n_k = 2, 2, 3, 7
    Q, dO = r.standard_normal((B, H, n_q, d)), r.standard_normal((B, H, n_q, dv))
    K, V = r.standard_normal((B, H, n_k, d)), r.standard_normal((B, H, n_k, dv))
    O, lse = orc.attention_fwd(Q, K, V, scale, True, q_pos0=n_k - n_q)
    g = orc.attention_bwd(Q, K, V, dO, scale, True, q_pos0=n_k - n_q)
    for b in range(B):
        for h in range(H):
            vis = np.array([[j <= n_k - n_q + i for j in range(n_k)]
                            for i in range(n_q)])
            To, Tl, Tdq, Tdk, Tdv = _torch_reference(
                Q[b, h], K[b, h], V[b, h], dO[b, h], scale, False, vis)
            tag = f"batched offset ({b},{h})"
            _close(O[b, h], To, 1e-12, tag + " O")
            _close(lse[b, h], Tl, 1e-12, tag + " LSE")
            for a, t, nm in zip(g, (Tdq, Tdk, Tdv), ("dQ", "dK", "dV")):
                _close(a[b, h], t, 1e-12, f"{tag} {nm}")


ALL_CHECKS = [
    check_fig1_divide_last,
    check_fig2_streamed_pairs,
    check_fig3_two_query_tile,
    check_single_key,
    check_causal_first_row,
    check_equal_scores,
    check_normalisation,
    check_shift_invariance,
    check_vs_torch_library,
    check_brute_force_python,
    check_finite_differences,
    check_bwd_identities,
    check_tile_invariance,
    check_causal_tile_count,
    check_block_sparse,
    check_decode,
    check_bwd_rows,
    check_batched_wrappers,
    check_offset_queries,
]
