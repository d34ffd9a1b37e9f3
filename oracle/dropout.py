"""Attention dropout for the float64 oracle: a counter-based mask and the forward and backward through it.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[FA-LLM], opening paragraphs: the fused kernel does the matrix products,
masking, softmax and dropout in one program; [Digest], "Limits": dropout is
one of the features a kernel must handle.  Neither page specifies the random
numbers, the drop rule or where the rescale goes.  Readings taken here:

- Random numbers: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
  random numbers: as easy as 1, 2, 3", SC 2011): a 4 x 32-bit counter, a
  2 x 32-bit key, ten rounds.  Each round multiplies counter words 0 and 2 by
  0xD2511F53 and 0xCD9E8D57 into 64-bit products and forms the new counter
  from their high and low halves, the other two words and the key; the key
  is bumped by the Weyl constants 0x9E3779B9 and 0xBB67AE85 between rounds.
- One call serves a 4 x 4 block of the score matrix, one byte per element:
  the element (query i, key j) of batch entry b and query head h takes byte
  4 (i mod 4) + (j mod 4) of Philox(counter = (j div 4, i div 4, b * Hq + h, 0),
  key = (seed mod 2^32, seed div 2^32)), byte 4 w + e being bits 8 e .. 8 e + 7
  of output word w.
- The element is kept iff that byte is >= t = floor(256 p), so it is dropped
  with probability p' = t / 256: p rounded down to a multiple of 1/256 (p
  itself for p on that grid; no dropout for p < 1/256).
- Dropout acts on the normalised probabilities: O = ((Z o P) / (1 - p')) V,
  Z the keep mask; the rescale uses p', so E[Z / (1 - p')] = 1 exactly.  The
  row statistic LSE is that of the undropped softmax, so the backward
  recomputes P from it as without dropout.
"""
from __future__ import annotations

import numpy as np

from .attention import probabilities

_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Philox4x32-10 on arrays: ``ctr`` is four uint32 arrays (broadcastable), ``key`` two; returns four uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) for x in ctr]
    k0, k1 = (np.asarray(x, dtype=np.uint64) for x in key)
    c0, c1, c2, c3 = np.broadcast_arrays(*c)
    for _ in range(10):
        p0 = np.uint64(_M0) * c0                        # < 2^64: exact in uint64
        p1 = np.uint64(_M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0) & _MASK, lo1, (hi0 ^ c3 ^ k1) & _MASK, lo0
        k0 = (k0 + np.uint64(_W0)) & _MASK
        k1 = (k1 + np.uint64(_W1)) & _MASK
    return [x.astype(np.uint32) for x in (c0, c1, c2, c3)]


def drop_threshold(p: float) -> int:
    """The keep threshold t = floor(256 p) for a drop probability 0 <= p < 1 (a byte is kept iff >= t)."""
    if not 0.0 <= p < 1.0:
        raise ValueError("the drop probability must be in [0, 1)")
    return int(np.floor(p * 256.0))


def drop_probability(p: float) -> float:
    """p' = floor(256 p) / 256, the probability with which an element is dropped (and the rescale's p)."""
    return drop_threshold(p) / 256.0


def keep_mask(b: int, h: int, Hq: int, rows, n_keys: int, p: float, seed: int) -> np.ndarray:
    """Boolean keep mask Z [len(rows), n_keys] of batch entry b, query head h."""
    rows = np.asarray(rows, dtype=np.uint64)[:, None]
    keys = np.arange(n_keys, dtype=np.uint64)[None, :]
    words = philox4x32_10((keys >> np.uint64(2), rows >> np.uint64(2), np.uint64(b * Hq + h), np.uint64(0)),
                          (np.uint64(seed & 0xFFFFFFFF), np.uint64(seed >> 32)))
    sel = (rows & np.uint64(3)).astype(np.int64)                    # word i mod 4 ...
    w = np.choose(np.broadcast_to(sel, words[0].shape), words).astype(np.uint64)
    byte = (w >> (np.uint64(8) * (keys & np.uint64(3)))) & np.uint64(0xFF)   # ... byte j mod 4 of it
    return byte >= np.uint64(drop_threshold(p))


def forward_dropout(q, k, v, causal, scale, p, seed):
    """O [B, Hq, N, d] and the (undropped) LSE [B, Hq, N] of attention with dropout on P."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, N, _ = q.shape
    G = Hq // k.shape[1]
    O = np.empty((B, Hq, N, v.shape[3]))
    L = np.empty((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            _, P, m, l = probabilities(q[b, h], k[b, h // G], scale, causal)
            Z = keep_mask(b, h, Hq, np.arange(N), k.shape[2], p, seed)
            Pd = np.where(Z, P, 0.0) / (1.0 - drop_probability(p))
            O[b, h] = Pd @ np.asarray(v[b, h // G], dtype=np.float64)
            L[b, h] = m + np.log(l)
    return O, L


def head_backward_dropout(qh, kg, vg, doh, b, h, Hq, causal, scale, p, seed):
    """One query head's share of the backward through dropout: (dq_h, dk_h, dv_h, O_h).

    qh, doh [N, d] of (batch b, query head h); kg, vg [N, d] of its K/V head.
    The chain rule of O = ((Z o P) / (1 - p')) V, Z fixed by the seed: with
    Pd = Z o P / (1 - p'), dV = Pd^T dO, dPd = dO V^T, dP = Z o dPd / (1 - p'), and
    through the softmax dS = P o (dP - D) with D_i = sum_j P_ij dP_ij = dO_i . O_i;
    then dQ = scale dS K and dK = scale dS^T Q.  dk_h, dv_h are this head's terms
    of its K/V head's gradients (a group sums them over its query heads)."""
    qh, kg, vg, doh = (np.asarray(x, dtype=np.float64) for x in (qh, kg, vg, doh))
    N = qh.shape[0]
    _, P, _, _ = probabilities(qh, kg, scale, causal)
    Z = keep_mask(b, h, Hq, np.arange(N), kg.shape[0], p, seed)
    pp = drop_probability(p)
    Pd = np.where(Z, P, 0.0) / (1.0 - pp)
    O = Pd @ vg
    dv = Pd.T @ doh
    dP = np.where(Z, doh @ vg.T, 0.0) / (1.0 - pp)
    D = np.sum(doh * O, axis=1)
    dS = P * (dP - D[:, None])
    return scale * (dS @ kg), scale * (dS.T @ qh), dv, O


def backward_dropout(q, k, v, do, causal, scale, p, seed):
    """dQ, dK, dV of O = ((Z o P) / (1 - p')) V for a loss with dL/dO = dO; returns (dq, dk, dv, O).

    Every (batch, query head) through head_backward_dropout; the K/V gradients
    of a group sum over its query heads."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, N, _ = q.shape
    G = Hq // k.shape[1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    O = np.empty((B, Hq, N, v.shape[3]))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            dq[b, h], dkh, dvh, O[b, h] = head_backward_dropout(q[b, h], k[b, g], v[b, g], do[b, h], b, h, Hq,
                                                                causal, scale, p, seed)
            dk[b, g] += dkh
            dv[b, g] += dvh
    return dq, dk, dv, O
