"""Plain, slow fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library and imports nothing from it.

Every function here is the plain definition written out in NumPy float64,
materialising the score matrix S and the probability matrix P (in row chunks
where N is large, which bounds memory without changing the definition).

Pages cited (titles as published):
  [TLDR]   "FlashAttention：メモリ効率的なアテンション計算" (tech-tldr.com)
  [XYZ]    "FlashAttention: IOを意識した高速かつメモリ効率の高い厳密なアテンション"
           (xyznot.com, summary of arXiv 2205.14135)
  [REAPER] "3 · FlashAttention" (mkdocs.reaper.mx, GPU course, chapter 3)
  [LLMSYS] "출력을 누적해 메모리 이동을 줄이는 FlashAttention"
           (llm-systems-engineering.pages.dev)
  [Q67]    "FlashAttention：在线 softmax 与 IO-aware 注意力" (quant67.com)

Readings of points the pages leave open:
  * The saved per-row statistic is one natural-log logsumexp of the *scaled*
    scores, LSE_i = m_i + ln(l_i); the pages save the pair (m, l)
    ([TLDR] backward section, [XYZ] key ideas, [Q67] section 5).
  * Causal means key j is visible to query i iff j <= i (equal lengths,
    top-left aligned); [REAPER] only states the block rule j <= i.  When
    there are fewer queries than keys (decoding, [REAPER] 3.6, and likewise
    a prompt fed in chunks), the Nq queries are the last Nq of the Nk
    tokens: query row r sits at position q_pos0 + r with q_pos0 = Nk - Nq
    and sees key j iff j <= q_pos0 + r (the square rule at that position).
  * A block mask M has shape ceil(N/block_m) x ceil(N/block_n); key j is
    visible to query i iff M[i // block_m, j // block_n] != 0, and it combines
    with the causal rule by AND ([XYZ] block-sparse extension).
  * A row that sees no key at all has O_i = 0 and LSE_i = -inf (the pages are
    silent; this is the value of the empty sum convention).
  * The backward is the exact gradient of L = sum(O * dO) with respect to
    Q, K, V (the pages give no formulas, only that S and P are recomputed;
    [TLDR] backward section, [REAPER] section 3.4, [Q67] section 5).  No
    gradient flows into LSE.

Parity pins for every function live in ``tests/oracle_pins.py``.
"""

import numpy as np

__all__ = [
    "visible",
    "attention_fwd_head",
    "attention_fwd",
    "attention_bwd_head",
    "attention_bwd",
    "attention_bwd_rows",
    "tiled_fwd_head",
    "tiled_fwd_fa1_head",
    "causal_tiles_visited",
    "attention_decode_head",
]

NEG_INF = -np.inf


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Visibility (masking)
# ---------------------------------------------------------------------------

def visible(rows, n_keys, causal=False, block_mask=None, block_m=128,
            block_n=128, q_pos0=0):
    """Boolean matrix vis[r, j]: key j is visible to query rows[r].

    Causal rule: j <= i ([REAPER], causal-mask question of the chapter
    summary: query block i needs only key blocks j <= i; read element-wise),
    where i = q_pos0 + row is the query's position in the key sequence
    (q_pos0 = 0 when queries and keys are the same tokens; a decoding step's
    Nq new queries are the last Nq positions, q_pos0 = Nk - Nq).
    Block-sparse rule: the entry of the block mask covering (i, j) is nonzero
    ([XYZ], section "Block-Sparse FlashAttention").  Both apply by AND.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.arange(n_keys, dtype=np.int64)
    vis = np.ones((rows.size, n_keys), dtype=bool)
    if causal:
        vis &= cols[None, :] <= q_pos0 + rows[:, None]
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        vis &= bm[rows[:, None] // block_m, cols[None, :] // block_n]
    return vis


# ---------------------------------------------------------------------------
# Materialising forward: the definition
# ---------------------------------------------------------------------------

def _softmax_rows(S):
    """Safe softmax of each row of S (entries may be -inf).

    Subtracts the row maximum before exponentiating ([TLDR] online-softmax
    section; [LLMSYS] Fig. 1).  Returns (P, m, l) with P = exp(S - m) / l,
    m the row maximum and l the sum of exp(S - m).  A row whose entries are
    all -inf gives P = 0, m = -inf, l = 0.
    """
    m = S.max(axis=1)
    empty = np.isneginf(m)
    m_shift = np.where(empty, 0.0, m)
    E = np.exp(S - m_shift[:, None])          # exp(-inf) = 0 for masked keys
    l = E.sum(axis=1)
    P = E / np.where(empty, 1.0, l)[:, None]
    return P, m, l


def attention_fwd_head(q, k, v, scale, causal=False, block_mask=None,
                       block_m=128, block_n=128, rows=None, row_chunk=1024,
                       q_pos0=0):
    """O and LSE of one head, optionally for a subset of query rows.

    The three steps of standard attention ([Q67] section 1; [REAPER] 3.1):
      S = scale * Q K^T,   P = softmax(S) row-wise,   O = P V,
    with masked scores set to -inf before the softmax, and
      LSE_i = m_i + ln(sum_j exp(S_ij - m_i)) = ln(sum_j exp(S_ij)).
    q: (Nq, d), k: (Nk, d), v: (Nk, dv).  Returns O (len(rows), dv) and
    LSE (len(rows),), both float64.  Under the causal rule query row r sits
    at position q_pos0 + r of the key sequence (``visible``).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n_q, n_k = q.shape[0], k.shape[0]
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((rows.size, v.shape[1]))
    LSE = np.full(rows.size, NEG_INF)
    for c0 in range(0, rows.size, row_chunk):
        r = rows[c0:c0 + row_chunk]
        S = scale * (q[r] @ k.T)
        S = np.where(visible(r, n_k, causal, block_mask, block_m, block_n,
                             q_pos0), S, NEG_INF)
        P, m, l = _softmax_rows(S)
        O[c0:c0 + r.size] = P @ v
        with np.errstate(divide="ignore"):
            LSE[c0:c0 + r.size] = np.where(np.isneginf(m), NEG_INF,
                                           m + np.log(l))
    return O, LSE


def attention_decode_head(q, k, v, scale, causal=False):
    """O and LSE of one head for Nq queries against Nk >= Nq keys, the
    queries being the last Nq tokens of the sequence ([REAPER] 3.6: in
    decoding Q is one token, or a few, while K and V span the whole context).
    The definition is that of ``attention_fwd_head``; under the causal rule
    query row r sits at position Nk - Nq + r."""
    q, k = _f64(q), _f64(k)
    n_q, n_k = q.shape[0], k.shape[0]
    assert n_k >= n_q, "decoding queries are the last Nq of the Nk tokens"
    v = _f64(v)
    O = np.zeros((n_q, v.shape[1]))
    LSE = np.full(n_q, NEG_INF)
    r = np.arange(n_q)
    S = scale * (q @ k.T)
    S = np.where(visible(r, n_k, causal, q_pos0=n_k - n_q), S, NEG_INF)
    P, m, l = _softmax_rows(S)
    O[:] = P @ v
    with np.errstate(divide="ignore"):
        LSE[:] = np.where(np.isneginf(m), NEG_INF, m + np.log(l))
    return O, LSE


def _each_head(fn, heads, workers):
    """fn(idx) for every head index, in order.  Heads are independent, so
    with workers > 1 they run on a thread pool (NumPy's matrix products and
    ufuncs release the interpreter lock), each with a single BLAS thread."""
    heads = list(heads)
    if workers <= 1 or len(heads) <= 1:
        return [fn(idx) for idx in heads]
    import concurrent.futures
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1, user_api="blas")
    except ImportError:  # pragma: no cover - threadpoolctl is optional
        limit = contextlib.nullcontext()
    with limit, concurrent.futures.ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, heads))


def attention_fwd(Q, K, V, scale, causal=False, block_mask=None, block_m=128,
                  block_n=128, heads=None, row_chunk=1024, workers=1,
                  q_pos0=0):
    """Batched forward over leading dims: Q (..., Nq, d), K and V
    (..., Nk, d); each head is ``attention_fwd_head`` of that head's slices
    (``q_pos0`` as there).

    ``heads`` optionally restricts the work to a list of leading-index tuples
    (the other heads of the returned arrays stay NaN); ``workers`` > 1 runs
    the heads on that many threads.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    lead = Q.shape[:-2]
    O = np.full(lead + (Q.shape[-2], V.shape[-1]), np.nan)
    LSE = np.full(lead + (Q.shape[-2],), np.nan)
    idxs = list(np.ndindex(*lead) if heads is None else heads)

    def one(idx):
        return attention_fwd_head(Q[idx], K[idx], V[idx], scale, causal,
                                  block_mask, block_m, block_n,
                                  row_chunk=row_chunk, q_pos0=q_pos0)
    for idx, (o, lse) in zip(idxs, _each_head(one, idxs, workers)):
        O[idx], LSE[idx] = o, lse
    return O, LSE


# ---------------------------------------------------------------------------
# Materialising backward: the exact gradient of the definition
# ---------------------------------------------------------------------------

def attention_bwd_head(q, k, v, do, scale, causal=False, block_mask=None,
                       block_m=128, block_n=128, row_chunk=1024, q_pos0=0):
    """dQ, dK, dV of one head for the loss L = sum(O * dO).

    The pages only say that S and P are rebuilt from saved row statistics
    rather than stored ([TLDR] backward section; [REAPER] 3.4; [Q67]
    section 5).  The gradient itself follows from O = P V, P = softmax(S),
    S = scale * Q K^T by the chain rule:
      dV = P^T dO,   dP = dO V^T,   D_i = sum_j P_ij dP_ij,
      dS = P * (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
    Masked entries have P = 0 and contribute nothing.  P is recomputed here
    from its definition, row chunk by row chunk.  q, do: (Nq, .); k, v:
    (Nk, .); ``q_pos0`` as in ``attention_fwd_head``.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n_q, n_k = q.shape[0], k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, n_q, row_chunk):
        r = np.arange(r0, min(n_q, r0 + row_chunk))
        S = scale * (q[r] @ k.T)
        S = np.where(visible(r, n_k, causal, block_mask, block_m, block_n,
                             q_pos0), S, NEG_INF)
        P, _, _ = _softmax_rows(S)
        dv += P.T @ do[r]
        dP = do[r] @ v.T
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        dq[r] = scale * (dS @ k)
        dk += scale * (dS.T @ q[r])
    return dq, dk, dv


def attention_bwd_rows(q, k, v, do, scale, rows, causal=False,
                       block_mask=None, block_m=128, block_n=128, q_pos0=0):
    """The backward restricted to a set of query rows, for heads too long to
    materialise: dQ of those rows, and their contributions to dK and dV.

    Same chain rule as ``attention_bwd_head``, applied to the rows given:
    dQ_i depends only on row i of P and dP, so dQ[rows] is exact; dK and dV
    are sums over query rows, so the returned dk_part = scale * dS[rows]^T
    q[rows] and dv_part = P[rows]^T dO[rows] are the contributions of those
    rows only (under the causal rule, the contributions of rows [N-T, N)
    are the whole dK, dV of keys [N-T, N), which no earlier row sees).
    Work and memory are O(len(rows) * N * d).  ``q_pos0`` as in
    ``attention_fwd_head``.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    r = np.asarray(rows, dtype=np.int64)
    n_k = k.shape[0]
    S = scale * (q[r] @ k.T)
    S = np.where(visible(r, n_k, causal, block_mask, block_m, block_n,
                         q_pos0), S, NEG_INF)
    P, _, _ = _softmax_rows(S)
    dP = do[r] @ v.T
    D = (P * dP).sum(axis=1)
    dS = P * (dP - D[:, None])
    dq_rows = scale * (dS @ k)
    dk_part = scale * (dS.T @ q[r])
    dv_part = P.T @ do[r]
    return dq_rows, dk_part, dv_part


def attention_bwd(Q, K, V, dO, scale, causal=False, block_mask=None,
                  block_m=128, block_n=128, heads=None, row_chunk=1024,
                  workers=1, q_pos0=0):
    """Batched backward over leading dims: each head is
    ``attention_bwd_head`` of that head's slices (``heads``, ``workers`` and
    ``q_pos0`` as in ``attention_fwd``)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    lead = Q.shape[:-2]
    dQ = np.full(Q.shape, np.nan)
    dK = np.full(K.shape, np.nan)
    dV = np.full(V.shape, np.nan)
    idxs = list(np.ndindex(*lead) if heads is None else heads)

    def one(idx):
        return attention_bwd_head(Q[idx], K[idx], V[idx], dO[idx], scale,
                                  causal, block_mask, block_m, block_n,
                                  row_chunk=row_chunk, q_pos0=q_pos0)
    for idx, (dq, dk, dv) in zip(idxs, _each_head(one, idxs, workers)):
        dQ[idx], dK[idx], dV[idx] = dq, dk, dv
    return dQ, dK, dV


# ---------------------------------------------------------------------------
# Tiled forward, online softmax: test scaffolding for the exactness claim
# ---------------------------------------------------------------------------

def _key_block_needed(i0, i1, j0, causal):
    """Causal block skip: a key block is needed iff its first key j0 is
    visible to the last query i1 - 1 of the row block ([REAPER], causal
    question: inner loop j from 0 to i)."""
    return (not causal) or j0 <= i1 - 1


def tiled_fwd_head(q, k, v, scale, Br, Bc, causal=False, block_mask=None,
                   block_m=128, block_n=128, trace=None):
    """FA2-form tiled forward with an unnormalised accumulator.

    Outer loop over query blocks of Br rows, inner loop over key/value blocks
    of Bc rows ([TLDR] tiling section; [REAPER] 3.2).  Per row, with m the
    running max, l the running exp-sum and a the running unnormalised
    weighted sum of V ([LLMSYS] Fig. 2 and Fig. 3; [TLDR] online-softmax
    section; [REAPER] 3.3; [Q67] section 2):
        m_new = max(m, rowmax(S_j))
        alpha = exp(m - m_new)
        l     = alpha * l + rowsum(exp(S_j - m_new))
        a     = alpha * a + exp(S_j - m_new) V_j
        m     = m_new
    and once at the end O = a / l.  Tiles need not divide N (the last one is
    ragged).  If ``trace`` is a list, one dict per visited tile is appended
    with the state after rescaling by alpha and after adding the tile.
    Returns (O, LSE, number of visited tiles).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n_q, n_k, dv = q.shape[0], k.shape[0], v.shape[1]
    O = np.zeros((n_q, dv))
    LSE = np.full(n_q, NEG_INF)
    visited = 0
    for i0 in range(0, n_q, Br):
        i1 = min(n_q, i0 + Br)
        rows = np.arange(i0, i1)
        m = np.full(i1 - i0, NEG_INF)
        l = np.zeros(i1 - i0)
        a = np.zeros((i1 - i0, dv))
        for j0 in range(0, n_k, Bc):
            j1 = min(n_k, j0 + Bc)
            if not _key_block_needed(i0, i1, j0, causal):
                continue
            visited += 1
            S = scale * (q[i0:i1] @ k[j0:j1].T)
            vis = visible(rows, n_k, causal, block_mask, block_m,
                          block_n)[:, j0:j1]
            S = np.where(vis, S, NEG_INF)
            m_new = np.maximum(m, S.max(axis=1))
            # Rows that have seen no visible key yet keep m = -inf; shift
            # them by 0 so that exp(-inf - 0) = 0 rather than NaN.
            shift = np.where(np.isneginf(m_new), 0.0, m_new)
            alpha = np.exp(m - shift)
            Pt = np.exp(S - shift[:, None])
            l_scaled, a_scaled = alpha * l, alpha[:, None] * a
            l = l_scaled + Pt.sum(axis=1)
            a = a_scaled + Pt @ v[j0:j1]
            m = m_new
            if trace is not None:
                trace.append(dict(i0=i0, j0=j0, m=m.copy(), alpha=alpha,
                                  l_rescaled=l_scaled, a_rescaled=a_scaled,
                                  l=l.copy(), a=a.copy()))
        empty = l == 0.0
        O[i0:i1] = a / np.where(empty, 1.0, l)[:, None]
        with np.errstate(divide="ignore"):
            LSE[i0:i1] = np.where(empty, NEG_INF, m + np.log(l))
    return O, LSE, visited


def tiled_fwd_fa1_head(q, k, v, scale, Br, Bc, causal=False, block_mask=None,
                       block_m=128, block_n=128):
    """FA1-form tiled forward: a normalised running output.

    Per key block, block-local statistics m~ = rowmax(S), P~ = exp(S - m~),
    l~ = rowsum(P~); then the running statistics merge by the two-part rule
        m_new = max(m, m~),  l_new = exp(m - m_new) l + exp(m~ - m_new) l~
    and the output is kept normalised,
        O <- diag(l_new)^-1 (diag(l) exp(m - m_new) O + exp(m~ - m_new) P~ V)
    ([XYZ], section "incremental softmax tracking", steps 1-4).  Must agree
    with ``tiled_fwd_head`` and with the materialising definition.
    Returns (O, LSE).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n_q, n_k, dv = q.shape[0], k.shape[0], v.shape[1]
    O = np.zeros((n_q, dv))
    LSE = np.full(n_q, NEG_INF)
    for i0 in range(0, n_q, Br):
        i1 = min(n_q, i0 + Br)
        rows = np.arange(i0, i1)
        m = np.full(i1 - i0, NEG_INF)
        l = np.zeros(i1 - i0)
        o = np.zeros((i1 - i0, dv))
        for j0 in range(0, n_k, Bc):
            j1 = min(n_k, j0 + Bc)
            if not _key_block_needed(i0, i1, j0, causal):
                continue
            S = scale * (q[i0:i1] @ k[j0:j1].T)
            vis = visible(rows, n_k, causal, block_mask, block_m,
                          block_n)[:, j0:j1]
            S = np.where(vis, S, NEG_INF)
            m_blk = S.max(axis=1)
            blk_empty = np.isneginf(m_blk)
            P_blk = np.exp(S - np.where(blk_empty, 0.0, m_blk)[:, None])
            l_blk = P_blk.sum(axis=1)
            m_new = np.maximum(m, m_blk)
            shift = np.where(np.isneginf(m_new), 0.0, m_new)
            c_old = np.exp(m - shift)
            c_blk = np.where(blk_empty, 0.0,
                             np.exp(np.where(blk_empty, 0.0, m_blk) - shift))
            l_new = c_old * l + c_blk * l_blk
            num = (l * c_old)[:, None] * o + c_blk[:, None] * (P_blk @ v[j0:j1])
            o = num / np.where(l_new == 0.0, 1.0, l_new)[:, None]
            m, l = m_new, l_new
        O[i0:i1] = o
        with np.errstate(divide="ignore"):
            LSE[i0:i1] = np.where(l == 0.0, NEG_INF, m + np.log(l))
    return O, LSE


def causal_tiles_visited(n, Br, Bc):
    """Number of (query block, key block) pairs the causal block skip keeps."""
    count = 0
    for i0 in range(0, n, Br):
        i1 = min(n, i0 + Br)
        for j0 in range(0, n, Bc):
            if _key_block_needed(i0, i1, j0, True):
                count += 1
    return count
