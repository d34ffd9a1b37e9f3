"""Plain float64 softmax attention: the definition written out, S and P materialised.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy only; no blocking,
fusion or reordering beyond what each docstring states.

Notation (all pages): Q [B, Hq, N, d], K and V [B, Hkv, N, d], scale a positive
number, S = scale * Q K^T, P = softmax(S) over keys, O = P V.  With grouped
heads, query head h reads key/value head h // (Hq // Hkv) ([FA-LLM], entry
"Grouped-Query Attention": query heads are divided into groups that share one
key/value head; groups are contiguous runs of query heads).  Causal: key j is
visible to query i iff j <= i ([Digest], "Limits", which lists causal masks;
queries and keys have the same length, so there is no alignment choice).

The log-sum-exp statistic is LSE_i = m_i + ln(l_i) in natural-log units of
the scaled scores ([FA-legal], paragraph on the backward pass: only the
softmax normalisation statistics (m, l) are kept; [FA-LLM], third paragraph:
the log-sum-exp trick).
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 256   # rows materialised at once; each block still holds full rows of S and P


def _log(x):
    """Natural log with log(0) = -inf and no warning (a row that sees no key has LSE = -inf)."""
    with np.errstate(divide="ignore"):
        return np.log(x)


class BlockMask:
    """A block-sparse pattern: key j is visible to query i iff mask[i // bs, j // bs].

    [FA-legal], entry "Block-sparse": a sparsity mask over the blocks of the
    attention matrix says which blocks are computed.  Used as the ``window``
    argument; with the causal mask both conditions apply.
    """

    def __init__(self, mask, bs):
        self.mask = np.asarray(mask, dtype=bool)
        self.bs = int(bs)


def _band(window):
    """(W, S) of a ``window`` argument: an int W, or a pair (W, S)."""
    if isinstance(window, (tuple, list)):
        return int(window[0]), int(window[1])
    return int(window), 0


def _band_visible(keys, rows, window):
    """Sliding window with global tokens: j > i - W, or j < S; or a block mask (causal part applied by the caller)."""
    if isinstance(window, BlockMask):
        return window.mask[rows // window.bs, keys // window.bs]
    W, S = _band(window)
    return (keys > rows - W) | (keys < S)


def _visible(rows: np.ndarray, n_keys: int, causal: bool, window=None) -> np.ndarray | None:
    """Boolean mask [len(rows), n_keys] of visible keys, or None when all are.

    ``window`` (with the causal mask only) is the sliding window of local
    attention, optionally with global tokens ([FA-legal], entry
    "Block-sparse": sliding-window (local) attention and global tokens are
    named sparsity patterns): an int W, or a pair (W, S).  Key j is visible to
    query i iff j <= i and (i - W < j or j < S): the S leading tokens are
    seen by every later query.
    """
    if window is not None and not causal and not isinstance(window, BlockMask):
        raise ValueError("the sliding window is defined with the causal mask")
    keys = np.arange(n_keys)[None, :]
    if not causal:
        return None if window is None else _band_visible(keys, rows[:, None], window)
    vis = keys <= rows[:, None]
    if window is not None:
        vis &= _band_visible(keys, rows[:, None], window)
    return vis


@np.errstate(divide="ignore")
def probabilities(qh, kg, scale, causal, rows=None, window=None):
    """Rows of S and P = softmax(S), plus the row max m and row sum l.

    [IO-aware], "The Memory Bandwidth Bottleneck", steps 1-2: S = Q K^T, then
    P = softmax(S).  The softmax is the two-pass form that [FA-legal] (online
    softmax paragraph) contrasts with the online one: first the row maximum,
    then exponentials of S - m and their sum.  Masked scores are -inf and
    contribute exp(-inf) = 0.
    """
    qh = np.asarray(qh, dtype=np.float64)
    kg = np.asarray(kg, dtype=np.float64)
    n = kg.shape[0]
    rows = np.arange(qh.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    S = scale * (qh[rows] @ kg.T)
    vis = _visible(rows, n, causal, window)
    if vis is not None:
        S = np.where(vis, S, -np.inf)
    m = S.max(axis=1)
    seen = np.isfinite(m)                               # rows that see at least one key
    E = np.exp(S - np.where(seen, m, 0.0)[:, None])
    l = E.sum(axis=1)
    P = E / np.where(seen, l, 1.0)[:, None]
    return S, P, m, l


def head_rows_forward(qh, kg, vg, rows, causal, scale, window=None):
    """O and LSE for the given query rows of one head, in row blocks.

    [IO-aware], "The Memory Bandwidth Bottleneck", step 3: O = P V.
    LSE_i = m_i + ln l_i.
    """
    rows = np.asarray(rows, dtype=np.int64)
    vg = np.asarray(vg, dtype=np.float64)
    O = np.empty((rows.size, vg.shape[1]))
    L = np.empty(rows.size)
    for s in range(0, rows.size, ROW_BLOCK):
        r = rows[s:s + ROW_BLOCK]
        _, P, m, l = probabilities(qh, kg, scale, causal, r, window)
        O[s:s + r.size] = P @ vg
        L[s:s + r.size] = m + _log(l)
    return O, L


def forward(q, k, v, causal, scale, window=None):
    """Full forward over [B, Hq, N, d]: returns O [B, Hq, N, d] and LSE [B, Hq, N]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    O = np.empty((B, Hq, N, v.shape[3]))
    L = np.empty((B, Hq, N))
    rows = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            O[b, h], L[b, h] = head_rows_forward(q[b, h], k[b, g], v[b, g], rows, causal, scale, window)
    return O, L


def decode_forward(q, k, v, causal, scale):
    """New query rows against a key/value cache: O [B, Hq, Nq, d] and LSE [B, Hq, Nq].

    q is [B, Hq, Nq, d]; k and v are the cache, [B, Hkv, Nk, d].  [FA-LLM],
    entry "KV Cache": the keys and values of all earlier tokens are kept and
    each new token attends to them; [Digest], "Limits": decode-time attention
    over that cache.  The new rows are the last Nq positions of the sequence,
    so with the causal mask row i sees cache keys j <= Nk - Nq + i; without
    it every row sees all Nk keys.  Plain definition per (batch, head): S =
    scale * q k^T over the visible keys, two-pass softmax, O = P v,
    LSE = m + ln l.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, _ = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    O = np.empty((B, Hq, Nq, v.shape[3]))
    L = np.empty((B, Hq, Nq))
    pos = np.arange(Nk - Nq, Nk)                      # positions of the new rows
    for b in range(B):
        for h in range(Hq):
            g = h // G
            S = scale * (q[b, h] @ k[b, g].T)
            if causal:
                S = np.where(np.arange(Nk)[None, :] <= pos[:, None], S, -np.inf)
            m = S.max(axis=1)
            E = np.exp(S - m[:, None])
            l = E.sum(axis=1)
            O[b, h] = (E / l[:, None]) @ v[b, g]
            L[b, h] = m + np.log(l)
    return O, L


def decode_paged_forward(q, k_cache, v_cache, block_table, seq_lens, causal, scale):
    """Decode against a paged cache: O [B, Hq, Nq, d] and LSE [B, Hq, Nq].

    [FA-LLM], entry "PagedAttention": the KV cache is kept in fixed-size,
    non-contiguous blocks; sequence b's key j is row j % bs of block
    block_table[b][j // bs] of the pool k_cache / v_cache [nblk, Hkv, bs, d],
    and it has seq_lens[b] keys ([Digest], "Limits": batch-varying lengths).
    Per sequence the keys are gathered in order, then the plain definition as
    in ``decode_forward``: causal row i sees keys j <= n - Nq + i.  A row that
    sees no key gets O = 0 and LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, Nq, _ = q.shape
    Hkv, bs = k_cache.shape[1], k_cache.shape[2]
    G = Hq // Hkv
    O = np.zeros((B, Hq, Nq, v_cache.shape[3]))
    L = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        blocks = [int(x) for x in block_table[b][:(n + bs - 1) // bs]]
        kb = np.concatenate([np.asarray(k_cache[x], dtype=np.float64) for x in blocks], axis=1)[:, :n]
        vb = np.concatenate([np.asarray(v_cache[x], dtype=np.float64) for x in blocks], axis=1)[:, :n]
        vis = np.ones((Nq, n), dtype=bool)
        if causal:
            vis = np.arange(n)[None, :] <= (n - Nq + np.arange(Nq))[:, None]
        rows = vis.any(axis=1)
        for h in range(Hq):
            S = np.where(vis, scale * (q[b, h] @ kb[h // G].T), -np.inf)[rows]
            m = S.max(axis=1)
            E = np.exp(S - m[:, None])
            l = E.sum(axis=1)
            O[b, h, rows] = (E / l[:, None]) @ vb[h // G]
            L[b, h, rows] = m + np.log(l)
    return O, L


def forward_online(q, k, v, causal, scale, block_sizes):
    """Forward by the tiled online softmax, key blocks taken in order.

    [IO-aware], "Flash Attention Algorithm" and "Online Softmax"; [FA-legal],
    online softmax paragraph and glossary entry "Online softmax": keep a
    running maximum m and running sum l per query row; for each key block,
    take the new maximum m' = max(m, rowmax(S_blk)), rescale what was
    accumulated so far by exp(m - m'), add the block's exp(S_blk - m') to the
    sum and exp(S_blk - m') V_blk to the output accumulator; at the end divide
    the accumulator by l.  Rows with no visible key yet have m = -inf and no
    accumulated mass (their rescale factor is taken as 0 and their exponent
    base as 0 so that -inf - -inf never occurs).

    ``block_sizes`` lists the key-block lengths; they must sum to N.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, N, d = q.shape
    assert sum(block_sizes) == N
    G = Hq // k.shape[1]
    O = np.empty((B, Hq, N, v.shape[3]))
    L = np.empty((B, Hq, N))
    rows = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, v.shape[3]))
            j0 = 0
            for bs in block_sizes:
                cols = np.arange(j0, j0 + bs)
                S = scale * (q[b, h] @ k[b, g, j0:j0 + bs].T)
                if causal:
                    S = np.where(cols[None, :] <= rows[:, None], S, -np.inf)
                m_new = np.maximum(m, S.max(axis=1))
                base = np.where(np.isneginf(m_new), 0.0, m_new)
                alpha = np.where(np.isneginf(m), 0.0, np.exp(m - base))
                Pt = np.exp(S - base[:, None])
                l = alpha * l + Pt.sum(axis=1)
                acc = alpha[:, None] * acc + Pt @ v[b, g, j0:j0 + bs]
                m = m_new
                j0 += bs
            O[b, h] = acc / l[:, None]
            L[b, h] = m + np.log(l)
    return O, L


def backward(q, k, v, do, causal, scale, window=None):
    """Gradients of O = softmax(scale Q K^T [+mask]) V for a loss with dL/dO = dO.

    The pages do not print the backward; [FA-legal] (backward paragraph and
    entry "Recomputation") and [Digest] ("Method", item 4) say only that P is
    recomputed from Q, K and the stored statistics.  This is the chain rule of
    the forward definition, P materialised:
      dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic (= sum_j P_ij dP_ij),
      dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,
    and, with grouped heads, dK and dV of a key/value head are the sums over
    the query heads of its group.  Returns dq, dk, dv and D [B, Hq, N].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    Dall = np.empty((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            _, P, _, _ = probabilities(q[b, h], k[b, g], scale, causal, window=window)
            O = P @ v[b, g]
            dv[b, g] += P.T @ do[b, h]
            dP = do[b, h] @ v[b, g].T
            D = (do[b, h] * O).sum(axis=1)
            dS = P * (dP - D[:, None])
            dq[b, h] = scale * (dS @ k[b, g])
            dk[b, g] += scale * (dS.T @ q[b, h])
            Dall[b, h] = D
    return dq, dk, dv, Dall


def head_rows_backward_dq(qh, kg, vg, doh, rows, causal, scale, window=None):
    """dQ rows of one head (and their O, LSE, D), from full rows of P.

    Same chain rule as ``backward`` restricted to the given query rows: D of
    those rows uses this oracle's own O of those rows.
    """
    rows = np.asarray(rows, dtype=np.int64)
    kg = np.asarray(kg, dtype=np.float64)
    vg = np.asarray(vg, dtype=np.float64)
    doh = np.asarray(doh, dtype=np.float64)
    dQ = np.empty((rows.size, kg.shape[1]))
    O = np.empty((rows.size, vg.shape[1]))
    L = np.empty(rows.size)
    Dr = np.empty(rows.size)
    for s in range(0, rows.size, ROW_BLOCK):
        r = rows[s:s + ROW_BLOCK]
        _, P, m, l = probabilities(qh, kg, scale, causal, r, window)
        Or = P @ vg
        dP = doh[r] @ vg.T
        D = (doh[r] * Or).sum(axis=1)
        dS = P * (dP - D[:, None])
        dQ[s:s + r.size] = scale * (dS @ kg)
        O[s:s + r.size] = Or
        L[s:s + r.size] = m + _log(l)
        Dr[s:s + r.size] = D
    return dQ, O, L, Dr


def head_full_stats(qh, kg, vg, doh, causal, scale, window=None):
    """LSE and D = rowsum(dO * O) for every row of one head (row blocks, full rows of P)."""
    n = np.asarray(qh).shape[0]
    O, L = head_rows_forward(qh, kg, vg, np.arange(n), causal, scale, window)
    D = (np.asarray(doh, dtype=np.float64) * O).sum(axis=1)
    return L, D


def head_cols_backward_dkdv(q_heads, kg, vg, do_heads, stats, cols, causal, scale, window=None):
    """dK and dV rows (key positions ``cols``) of one key/value head.

    For each query head h of the group, with its full-row LSE and D
    (``stats[h] = (LSE, D)``): P[:, j] = exp(S[:, j] - LSE), dP[:, j] =
    dO v_j, dS[:, j] = P[:, j] (dP[:, j] - D); dV_j = sum_i P_ij dO_i and
    dK_j = scale sum_i dS_ij Q_i, summed over the group's query heads.
    P from LSE is the recomputation of [FA-legal] entry "Recomputation".
    """
    cols = np.asarray(cols, dtype=np.int64)
    kg = np.asarray(kg, dtype=np.float64)
    vg = np.asarray(vg, dtype=np.float64)
    n = kg.shape[0]
    rows = np.arange(n)
    dK = np.zeros((cols.size, kg.shape[1]))
    dV = np.zeros((cols.size, vg.shape[1]))
    for qh, doh, (L, D) in zip(q_heads, do_heads, stats):
        qh = np.asarray(qh, dtype=np.float64)
        doh = np.asarray(doh, dtype=np.float64)
        S = scale * (qh @ kg[cols].T)                      # [n, |cols|]
        vis = None
        if causal:
            vis = cols[None, :] <= rows[:, None]
            if window is not None:
                vis &= _band_visible(cols[None, :], rows[:, None], window)
        elif window is not None:
            vis = _band_visible(cols[None, :], rows[:, None], window)
        if vis is not None:
            S = np.where(vis, S, -np.inf)
        L_ = np.asarray(L)
        seen = np.isfinite(L_)                          # rows that see no key at all have P = 0
        P = np.where(seen[:, None], np.exp(S - np.where(seen, L_, 0.0)[:, None]), 0.0)
        dP = doh @ vg[cols].T
        dS = P * (dP - np.asarray(D)[:, None])
        dV += P.T @ doh
        dK += scale * (dS.T @ qh)
    return dK, dV


def attention_matrix_bytes(n: int, bytes_per_element: int) -> int:
    """Bytes of one head's N x N score matrix that standard attention writes.

    [IO-aware], "The Memory Bandwidth Bottleneck": standard attention writes
    S and P (N x N) to HBM; this is the size of one such matrix.
    """
    return int(n) * int(n) * int(bytes_per_element)
