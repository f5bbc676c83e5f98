"""Textbook decode attention in float64 (oracle; test infrastructure only).

Definition followed (the pages print no formula; this is the plain reading of
attention that "reads the logical sequence as if it were contiguous" —
"Paged Attention: Virtual Memory for the KV Cache", §The fix borrowed from
operating systems; glossary "What is Paged Attention?"):

    for query head r of a sequence with context length n, kv head h = r // g
    (g = query heads per kv head, grouped-query attention as named in
    §What it does not fix):
        s_t = scale * sum_d q[r, d] * K[t, h, d]          t < n
        p_t = exp(s_t - max_t s_t)
        out[r, :] = sum_t p_t * V[t, h, :] / sum_t p_t

n = 0 gives a zero row (a reading: the pages never attend over nothing).

The split form computes, for consecutive partitions of ``part`` tokens,
m_p = max s, l_p = sum exp(s - m_p), acc_p = sum exp(s - m_p) V, and merges
them with M = max_p m_p: out = sum_p acc_p e^{m_p - M} / sum_p l_p e^{m_p - M}.
"""
from __future__ import annotations

import numpy as np

__all__ = ["decode_attention", "split_k", "lse_merge", "decode_attention_split"]


def _scores(q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """q [Hq, D], K [n, Hkv, D] -> s [Hq, n] (float64)."""
    Hq = q.shape[0]
    n, Hkv, _ = K.shape
    g = Hq // Hkv
    s = np.empty((Hq, n), dtype=np.float64)
    for r in range(Hq):
        h = r // g
        s[r] = (K[:, h, :] @ q[r]) * scale
    return s


def decode_attention(q, K, V, scale: float) -> np.ndarray:
    """One sequence: q [Hq, D], K/V [n, Hkv, D] (any float dtype) -> [Hq, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, D = q.shape
    n, Hkv, _ = K.shape
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    out = np.zeros((Hq, D), dtype=np.float64)
    if n == 0:
        return out
    g = Hq // Hkv
    s = _scores(q, K, scale)
    for r in range(Hq):
        p = np.exp(s[r] - s[r].max())
        out[r] = (p @ V[:, r // g, :]) / p.sum()
    return out


def prefill_attention(Q, K, V, scale: float) -> np.ndarray:
    """A chunk of new tokens at the end of an n-token context: Q [L, Hq, D],
    K/V [n, Hkv, D] (the chunk's own keys and values last) -> [L, Hq, D]
    float64.  Row t sits at position n - L + t and sees positions 0 .. itself:
    the causal attention of a decoder, which the pages do not spell out (the
    step before decode, "Paged Attention as a Memory Manager", §How the Kernel
    Executes Paged Attention), so each row is exactly the decode result over
    the context up to and including its own position."""
    Q = np.asarray(Q, dtype=np.float64)
    L, n = Q.shape[0], K.shape[0]
    if L > n:
        raise ValueError("the chunk is longer than its context")
    out = np.zeros(Q.shape, dtype=np.float64)
    for t in range(L):
        out[t] = decode_attention(Q[t], K[: n - L + t + 1], V[: n - L + t + 1], scale)
    return out


def split_k(q, K, V, scale: float, part: int):
    """Partials of one sequence over partitions of ``part`` tokens.

    Returns (m [P, Hq], l [P, Hq], acc [P, Hq, D]) in float64, P = ceil(n/part)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, D = q.shape
    n, Hkv, _ = K.shape
    g = Hq // Hkv
    P = -(-n // part)
    m = np.empty((P, Hq))
    l = np.empty((P, Hq))
    acc = np.empty((P, Hq, D))
    s = _scores(q, K, scale)
    for p in range(P):
        lo, hi = p * part, min(n, (p + 1) * part)
        for r in range(Hq):
            sp = s[r, lo:hi]
            m[p, r] = sp.max()
            e = np.exp(sp - m[p, r])
            l[p, r] = e.sum()
            acc[p, r] = e @ V[lo:hi, r // g, :]
    return m, l, acc


def lse_merge(m, l, acc) -> np.ndarray:
    """Merge partials (m [P, Hq], l [P, Hq], acc [P, Hq, D]) -> out [Hq, D]."""
    m = np.asarray(m, dtype=np.float64)
    if m.shape[0] == 0:
        return np.zeros(acc.shape[1:], dtype=np.float64)
    M = m.max(axis=0)                          # [Hq]
    w = np.exp(m - M[None, :])                 # [P, Hq]
    L = (np.asarray(l) * w).sum(axis=0)        # [Hq]
    num = (np.asarray(acc) * w[:, :, None]).sum(axis=0)
    return num / L[:, None]


def decode_attention_split(q, K, V, scale: float, part: int) -> np.ndarray:
    n = np.asarray(K).shape[0]
    if n == 0:
        return np.zeros(np.asarray(q).shape, dtype=np.float64)
    return lse_merge(*split_k(q, K, V, scale, part))
