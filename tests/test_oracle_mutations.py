"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is the oracle's source with one plausible slip (a dropped term, a
wrong sign or index, a transposed operand).  The mutated source is executed
as a throw-away module on the CPU and run through the pin checks of
``oracle_pins``; the test passes when some check rejects it.  This shows that
the pins constrain every part of the oracle, not only that the oracle passes
them.
"""

import os
import types

import pytest

from tests import oracle_pins, oracle_pins_dropout

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle",
                        "attention.py")

# (description, original text, replacement, which occurrence)
MUTATIONS = [
    ("fwd: scale dropped", "S = scale * (q[r] @ k.T)", "S = (q[r] @ k.T)", 0),
    ("bwd: scale dropped in recomputed S", "S = scale * (q[r] @ k.T)",
     "S = (q[r] @ k.T)", 1),
    ("fwd: P transposed in O = P V", "O[c0:c0 + r.size] = P @ v",
     "O[c0:c0 + r.size] = P.T @ v", 0),
    ("causal: strict inequality", "cols[None, :] <= q_pos0 + rows[:, None]",
     "cols[None, :] < q_pos0 + rows[:, None]", 0),
    ("causal: reversed", "cols[None, :] <= q_pos0 + rows[:, None]",
     "cols[None, :] >= q_pos0 + rows[:, None]", 0),
    ("causal: query offset subtracted",
     "cols[None, :] <= q_pos0 + rows[:, None]",
     "cols[None, :] <= rows[:, None] - q_pos0", 0),
    ("decode: offset from the wrong end", "q_pos0=n_k - n_q", "q_pos0=0", 0),
    ("block mask: indices swapped",
     "bm[rows[:, None] // block_m, cols[None, :] // block_n]",
     "bm[cols[None, :] // block_n, rows[:, None] // block_m]", 0),
    ("LSE: max term dropped", "m + np.log(l))", "np.log(l))", 0),
    ("softmax: not normalised", "P = E / np.where(empty, 1.0, l)[:, None]",
     "P = E", 0),
    ("softmax: max added instead of subtracted",
     "E = np.exp(S - m_shift[:, None])", "E = np.exp(S + m_shift[:, None])",
     0),
    ("bwd: dV = P dO", "dv += P.T @ do[r]", "dv += P @ do[r]", 0),
    ("bwd: dP sign", "dP = do[r] @ v.T", "dP = -do[r] @ v.T", 0),
    ("bwd: D term dropped", "dS = P * (dP - D[:, None])", "dS = P * dP", 0),
    ("bwd: D over the wrong axis", "D = (P * dP).sum(axis=1)",
     "D = (P * dP).sum(axis=0)", 0),
    ("bwd: dQ with dS transposed", "dq[r] = scale * (dS @ k)",
     "dq[r] = scale * (dS.T @ k)", 0),
    ("bwd: dK without transpose", "dk += scale * (dS.T @ q[r])",
     "dk += scale * (dS @ q[r])", 0),
    ("bwd: dK scale dropped", "dk += scale * (dS.T @ q[r])",
     "dk += (dS.T @ q[r])", 0),
    ("tiled: alpha inverted", "alpha = np.exp(m - shift)",
     "alpha = np.exp(shift - m)", 0),
    ("tiled: accumulator not rescaled", "a = a_scaled + Pt @ v[j0:j1]",
     "a = a + Pt @ v[j0:j1]", 0),
    ("tiled: exp-sum not rescaled", "l = l_scaled + Pt.sum(axis=1)",
     "l = l + Pt.sum(axis=1)", 0),
    ("tiled: causal block skip too eager",
     "return (not causal) or j0 <= i1 - 1", "return (not causal) or j0 <= i0",
     0),
    ("bwd rows: scale dropped in S", "S = scale * (q[r] @ k.T)",
     "S = (q[r] @ k.T)", 2),
    ("bwd rows: D term dropped", "dS = P * (dP - D[:, None])", "dS = P * dP",
     1),
    ("bwd rows: dQ scale dropped", "dq_rows = scale * (dS @ k)",
     "dq_rows = (dS @ k)", 0),
    ("bwd rows: dK part without transpose", "dk_part = scale * (dS.T @ q[r])",
     "dk_part = scale * (dS.T @ q)", 0),
    ("bwd rows: dV part from P not transposed", "dv_part = P.T @ do[r]",
     "dv_part = P.T @ do[r][::-1]", 0),
    ("FA1: old sum not rescaled", "l_new = c_old * l + c_blk * l_blk",
     "l_new = l + c_blk * l_blk", 0),
    ("FA1: output not un-normalised",
     "num = (l * c_old)[:, None] * o", "num = c_old[:, None] * o", 0),
    ("batched fwd: block sizes swapped",
     "block_mask, block_m, block_n,\n                                  row_chunk",
     "block_mask, block_n, block_m,\n                                  row_chunk", 0),
    ("batched fwd: causal rule dropped",
     "scale, causal,\n                                  block_mask",
     "scale, False,\n                                  block_mask", 0),
    ("batched fwd: keys of the neighbouring head",
     "attention_fwd_head(Q[idx], K[idx], V[idx]",
     "attention_fwd_head(Q[idx], K[idx[:-1] + ((idx[-1] + 1) % K.shape[-3],)], V[idx]", 0),
    ("batched fwd: LSE of another head",
     "O[idx], LSE[idx] = o, lse", "O[idx], LSE[idx[::-1]] = o, lse", 0),
    ("batched bwd: block sizes swapped",
     "causal, block_mask, block_m, block_n,\n                                  row_chunk",
     "causal, block_mask, block_n, block_m,\n                                  row_chunk", 0),
    ("batched bwd: dO of the neighbouring head",
     "V[idx], dO[idx], scale", "V[idx], dO[idx[:-1] + ((idx[-1] + 1) % dO.shape[-3],)], scale", 0),
    ("batched bwd: dK and dV slots swapped",
     "dQ[idx], dK[idx], dV[idx] = dq, dk, dv",
     "dQ[idx], dK[idx], dV[idx] = dq, dv, dk", 0),
    ("batched bwd: causal rule dropped",
     "dO[idx], scale,\n                                  causal,",
     "dO[idx], scale,\n                                  False,", 0),
    ("offset fwd: query offset ignored", "q_pos0), S, NEG_INF)",
     "0), S, NEG_INF)", 0),
    ("offset bwd: query offset ignored", "q_pos0), S, NEG_INF)",
     "0), S, NEG_INF)", 1),
    ("offset bwd rows: query offset ignored", "q_pos0), S, NEG_INF)",
     "0), S, NEG_INF)", 2),
    ("offset bwd: offset counted from the wrong end", "q_pos0), S, NEG_INF)",
     "-q_pos0), S, NEG_INF)", 1),
    ("batched fwd: offset not passed", "row_chunk=row_chunk, q_pos0=q_pos0)",
     "row_chunk=row_chunk)", 0),
    ("batched bwd: offset not passed", "row_chunk=row_chunk, q_pos0=q_pos0)",
     "row_chunk=row_chunk)", 1),
]


def _mutant(old, new, occurrence):
    with open(SRC_PATH) as f:
        src = f.read()
    parts = src.split(old)
    assert len(parts) - 1 > occurrence, f"pattern not in oracle: {old!r}"
    mutated = old.join(parts[:occurrence + 1]) + new + old.join(
        parts[occurrence + 1:])
    assert mutated != src
    mod = types.ModuleType("oracle_mutant")
    exec(compile(mutated, "<oracle mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("desc,old,new,occ", MUTATIONS,
                         ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(desc, old, new, occ):
    mod = _mutant(old, new, occ)
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception:       # AssertionError, or a crash on bad shapes
            return
    pytest.fail(f"no pin catches the planted mistake: {desc}")


DROPOUT_SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(__file__)),
                                "oracle", "dropout.py")

# Planted mistakes in the dropout oracle (same scheme).
DROPOUT_MUTATIONS = [
    ("philox: multipliers swapped", "p0 = x0 * np.uint64(_M0)",
     "p0 = x0 * np.uint64(_M1)", 0),
    ("philox: key not advanced", "k0 = (k0 + _W0) & _MASK32", "k0 = k0", 0),
    ("philox: permutation slip", "x1 = lo1", "x1 = lo0", 0),
    ("philox: nine rounds", "for _ in range(10):", "for _ in range(9):", 0),
    ("philox: key words swapped", "x0 = hi1 ^ x1 ^ np.uint64(k0)",
     "x0 = hi1 ^ x1 ^ np.uint64(k1)", 0),
    ("mapping: row and column blocks swapped",
     "ctr = np.stack([R, C, np.full_like(R, bh)",
     "ctr = np.stack([C, R, np.full_like(R, bh)", 0),
    ("mapping: word from the column", "(rows & 3)[:, None]]",
     "(cols & 3)[None, :]]", 0),
    ("mapping: byte from the row", "shift = (8 * (cols & 3))",
     "shift = (8 * (rows[:1] & 3))", 0),
    ("mapping: seed halves swapped",
     "(seed & _MASK32, (seed >> 32) & _MASK32)",
     "((seed >> 32) & _MASK32, seed & _MASK32)", 0),
    ("keep: strict comparison", "q_pos0) >= t\n\n\ndef attention_fwd", "q_pos0) > t\n\n\ndef attention_fwd", 0),
    ("threshold: truncated", "t = int(np.rint(256.0 * float(p)))",
     "t = int(256.0 * float(p))", 0),
    ("fwd: survivors not rescaled", "Pd = np.where(Z, P, 0.0) * (256.0 / (256.0 - t))",
     "Pd = np.where(Z, P, 0.0)", 0),
    ("fwd: LSE of the dropped row", "m + np.log(l))",
     "m + np.log((Pd * l[:, None]).sum(axis=1)))", 0),
    ("bwd: dP not masked", "dP = np.where(Z, dPd, 0.0) * c", "dP = dPd", 0),
    ("bwd: dP not rescaled", "dP = np.where(Z, dPd, 0.0) * c",
     "dP = np.where(Z, dPd, 0.0)", 0),
    ("bwd: dV from the undropped P", "dv = Pd.T @ do", "dv = P.T @ do", 0),
    ("bwd: D from the dropped P", "D = (P * dP).sum(axis=1)",
     "D = (Pd * dP).sum(axis=1)", 0),
    ("dq rows: dP not rescaled", "dP = np.where(Z, do[r] @ v.T, 0.0) * c",
     "dP = np.where(Z, do[r] @ v.T, 0.0)", 0),
    ("dq rows: D term dropped", "dS = P * (dP - D[:, None])\n    return",
     "dS = P * dP\n    return", 0),
    ("fwd rows: mask of the first rows", "Z = dropout_bytes(bh, r, np.arange(n_k), seed, q_pos0) >= t",
     "Z = dropout_bytes(bh, np.arange(len(r)), np.arange(n_k), seed, q_pos0) >= t", 0),
    ("fwd: key blocks collapsed", "block_n,\n                         q_pos0), S, NEG_INF)",
     "block_n * 0 + 10**6,\n                         q_pos0), S, NEG_INF)", 0),
    ("bwd: block sizes swapped",
     "causal, block_mask, block_m, block_n,\n                         q_pos0), S, NEG_INF)",
     "causal, block_mask, block_n, block_m,\n                         q_pos0), S, NEG_INF)", 1),
    ("bwd: query offset ignored", "q_pos0), S, NEG_INF)", "0), S, NEG_INF)", 1),
    ("dq rows: query offset ignored", "q_pos0), S, NEG_INF)", "0), S, NEG_INF)", 2),
    ("fwd: Z indexed by position", "Z = dropout_bytes(bh, r, np.arange(n_k), seed, q_pos0) >= t\n    Pd",
     "Z = dropout_bytes(bh, r + q_pos0, np.arange(n_k), seed, q_pos0) >= t\n    Pd", 0),
    ("fwd: Z without the offset", "Z = dropout_bytes(bh, r, np.arange(n_k), seed, q_pos0) >= t\n    Pd",
     "Z = dropout_bytes(bh, r, np.arange(n_k), seed) >= t\n    Pd", 0),
    ("bwd: Z without the offset", "Z = dropout_keep(bh, n_q, n_k, seed, t, q_pos0)",
     "Z = dropout_keep(bh, n_q, n_k, seed, t)", 0),
    ("mapping: offset not in the counter", "np.full_like(R, q_pos0)],", "np.zeros_like(R)],", 0),
]


def _dropout_mutant(old, new, occurrence):
    with open(DROPOUT_SRC_PATH) as f:
        src = f.read()
    parts = src.split(old)
    assert len(parts) - 1 > occurrence, f"pattern not in oracle: {old!r}"
    mutated = old.join(parts[:occurrence + 1]) + new + old.join(
        parts[occurrence + 1:])
    assert mutated != src
    # run outside the package: the relative import names the real module
    mutated = mutated.replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("oracle_dropout_mutant")
    exec(compile(mutated, "<dropout oracle mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("desc,old,new,occ", DROPOUT_MUTATIONS,
                         ids=[m[0] for m in DROPOUT_MUTATIONS])
def test_dropout_mutant_is_caught(desc, old, new, occ):
    mod = _dropout_mutant(old, new, occ)
    for check in oracle_pins_dropout.ALL_CHECKS:
        try:
            check(mod)
        except Exception:
            return
    pytest.fail(f"no pin catches the planted mistake: {desc}")
