"""Plain fp64 CPU oracle for attention with dropout on the probabilities.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library and imports nothing from it.

[XYZ] (key ideas, kernel fusion) lists dropout among the steps fused into the
one attention kernel, next to the matrix products, the mask and the softmax.
The pages define neither the dropout nor its random numbers.  Readings taken
here:

  * Dropout acts on the probability matrix: P~ = Z * P / (1 - p) with
    Z_ij in {0, 1} drawn independently, P(Z_ij = 0) = p, and O = P~ V.  The
    softmax statistics (m, l, LSE) are those of P itself, before dropout.
    This is the usual definition of dropout (units zeroed with probability
    p, survivors scaled by 1/(1-p) so that E[P~] = P) applied to P.
  * The random numbers come from the counter-based generator Philox4x32-10
    (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1,
    2, 3", SC 2011): one call maps a 128-bit counter and a 64-bit key to
    four 32-bit words.  Element (bh, i, j) of head bh (batch-major flattened
    index b*H + h), query row i (the row of Q) and key column j uses the call
    with counter (i >> 2, j >> 2, bh, q_pos0) and key (seed mod 2^32,
    seed >> 32); word (i & 3) of its output, byte (j & 3) of that word (bits
    8(j&3) .. 8(j&3)+7) is the element's random byte u.  So one call covers a
    4 x 4 block of the score matrix, and the mask does not depend on any
    tiling.  q_pos0 is the position of query row 0 in the key sequence (0
    when queries and keys are the same tokens): queries fed in chunks at
    different offsets draw from disjoint counters.
  * The drop probability is quantised to t / 256 with t = round(256 p), an
    integer in [0, 255]: the element is kept iff u >= t, and survivors are
    scaled by 256 / (256 - t).

Gradients: with the mask Z fixed, L = sum(O * dO) gives
  dV = P~^T dO,   dP~ = dO V^T,   dP = Z * dP~ / (1 - p),
  D_i = sum_j P_ij dP_ij,   dS = P * (dP - D),
  dQ = scale * dS K,   dK = scale * dS^T Q.
D also equals sum_k dO_ik O_ik (the pins check this identity).
"""

import numpy as np

from .attention import visible, _softmax_rows, _f64, NEG_INF

__all__ = [
    "philox4x32_10",
    "dropout_threshold",
    "dropout_bytes",
    "dropout_keep",
    "attention_fwd_dropout_head",
    "attention_bwd_dropout_head",
    "attention_dq_dropout_rows",
]

# Philox4x32 constants (Salmon et al. 2011, section 5: the two multipliers
# of the round function and the two Weyl increments of the key schedule).
_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds.  ctr: integer array (..., 4) of 32-bit
    counter words; key: (k0, k1).  Returns a uint32 array (..., 4).

    One round multiplies counter words 0 and 2 by the two multipliers (full
    64-bit products split into high and low halves) and permutes:
      (x0, x1, x2, x3) -> (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2),
                           hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)),
    after which the key advances by the Weyl increments (k0 += W0,
    k1 += W1, mod 2^32).  Ten rounds, the first with the key as given.
    """
    x = np.asarray(ctr, dtype=np.uint64) & _MASK32
    x0, x1, x2, x3 = (x[..., c].copy() for c in range(4))
    k0, k1 = int(key[0]) & _MASK32, int(key[1]) & _MASK32
    for _ in range(10):
        p0 = x0 * np.uint64(_M0)               # < 2^64: exact in uint64
        p1 = x2 * np.uint64(_M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(_MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(_MASK32)
        x0 = hi1 ^ x1 ^ np.uint64(k0)
        x1 = lo1
        x2 = hi0 ^ x3 ^ np.uint64(k1)
        x3 = lo0
        k0 = (k0 + _W0) & _MASK32
        k1 = (k1 + _W1) & _MASK32
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def dropout_threshold(p):
    """The integer threshold t = round(256 p) of a drop probability p; the
    quantised probability is t / 256.  Valid for 0 <= p and t <= 255."""
    t = int(np.rint(256.0 * float(p)))
    if not (0.0 <= float(p) and t <= 255):
        raise ValueError("drop probability must round to t in [0, 255]")
    return t


def dropout_bytes(bh, rows, cols, seed, q_pos0=0):
    """The random byte u of every element (bh, i, j), i in rows, j in cols
    (uint8 array of shape (len(rows), len(cols))), following the element to
    counter mapping stated in the module docstring."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    rb = np.unique(rows >> 2)
    cb = np.unique(cols >> 2)
    R, C = np.meshgrid(rb, cb, indexing="ij")
    ctr = np.stack([R, C, np.full_like(R, bh), np.full_like(R, q_pos0)],
                   axis=-1)
    words = philox4x32_10(ctr, (seed & _MASK32, (seed >> 32) & _MASK32))
    ri = np.searchsorted(rb, rows >> 2)
    ci = np.searchsorted(cb, cols >> 2)
    w = words[ri[:, None], ci[None, :], (rows & 3)[:, None]]
    shift = (8 * (cols & 3)).astype(np.uint32)[None, :]
    return ((w >> shift) & 0xFF).astype(np.uint8)


def dropout_keep(bh, n_q, n_k, seed, t, q_pos0=0):
    """Boolean keep mask Z (n_q, n_k) of head bh: u >= t."""
    return dropout_bytes(bh, np.arange(n_q), np.arange(n_k), seed,
                         q_pos0) >= t


def attention_fwd_dropout_head(q, k, v, scale, causal, t, seed, bh, rows=None,
                               block_mask=None, block_m=128, block_n=128,
                               q_pos0=0):
    """O and LSE of one head with dropout on P (module docstring):
      S = scale Q K^T (masked entries -inf),  P = softmax(S),
      O = (Z * P * 256 / (256 - t)) V,  LSE_i = ln(sum_j exp(S_ij)).
    Returns O (n_q, dv) and LSE (n_q,), float64; with ``rows`` only those
    query rows (each row of O depends on its own row of S alone).  The
    visible set is that of ``attention.visible`` (causal rule at position
    q_pos0 + row, block mask); Z is that of ``dropout_bytes`` with the same
    q_pos0."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n_q, n_k = q.shape[0], k.shape[0]
    r = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    S = scale * (q[r] @ k.T)
    S = np.where(visible(r, n_k, causal, block_mask, block_m, block_n,
                         q_pos0), S, NEG_INF)
    P, m, l = _softmax_rows(S)
    Z = dropout_bytes(bh, r, np.arange(n_k), seed, q_pos0) >= t
    Pd = np.where(Z, P, 0.0) * (256.0 / (256.0 - t))
    O = Pd @ v
    with np.errstate(divide="ignore"):
        LSE = np.where(np.isneginf(m), NEG_INF, m + np.log(l))
    return O, LSE


def attention_bwd_dropout_head(q, k, v, do, scale, causal, t, seed, bh,
                               block_mask=None, block_m=128, block_n=128,
                               q_pos0=0):
    """dQ, dK, dV of one head with dropout on P, for L = sum(O * dO) with the
    mask Z fixed (chain rule in the module docstring); visible set and Z as
    in ``attention_fwd_dropout_head``."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n_q, n_k = q.shape[0], k.shape[0]
    r = np.arange(n_q)
    S = scale * (q @ k.T)
    S = np.where(visible(r, n_k, causal, block_mask, block_m, block_n,
                         q_pos0), S, NEG_INF)
    P, _, _ = _softmax_rows(S)
    Z = dropout_keep(bh, n_q, n_k, seed, t, q_pos0)
    c = 256.0 / (256.0 - t)
    Pd = np.where(Z, P, 0.0) * c
    dv = Pd.T @ do
    dPd = do @ v.T
    dP = np.where(Z, dPd, 0.0) * c
    D = (P * dP).sum(axis=1)
    dS = P * (dP - D[:, None])
    dq = scale * (dS @ k)
    dk = scale * (dS.T @ q)
    return dq, dk, dv


def attention_dq_dropout_rows(q, k, v, do, scale, causal, t, seed, bh, rows,
                              block_mask=None, block_m=128, block_n=128,
                              q_pos0=0):
    """dQ of the given query rows of one head with dropout on P: row i of dQ
    needs only row i of P, dP and D (same chain rule as
    ``attention_bwd_dropout_head``), so heads too long to materialise can be
    checked row by row."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n_k = k.shape[0]
    r = np.asarray(rows, dtype=np.int64)
    S = scale * (q[r] @ k.T)
    S = np.where(visible(r, n_k, causal, block_mask, block_m, block_n,
                         q_pos0), S, NEG_INF)
    P, _, _ = _softmax_rows(S)
    Z = dropout_bytes(bh, r, np.arange(n_k), seed, q_pos0) >= t
    c = 256.0 / (256.0 - t)
    dP = np.where(Z, do[r] @ v.T, 0.0) * c
    D = (P * dP).sum(axis=1)
    dS = P * (dP - D[:, None])
    return scale * (dS @ k)
