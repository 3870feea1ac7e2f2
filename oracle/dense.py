"""Dense-mask brute force -- TEST INFRASTRUCTURE, tiny inputs only.

This is the construction the Kev article (icman.com.cn) prints in sections
2.3 and 5.3: a T x T block-diagonal matrix that is 1 inside each question's
interval and 0 across intervals, multiplied element-wise by the lower
triangle of ones (causal AND isolation).  The 0/1 mask is turned into the
additive form of the primer's section 2.1 formula (0 where allowed, -inf
where blocked), and softmax(Q K^T / sqrt(d_h) + M) V is evaluated per head
with whole matrices in float64.  Grouped KV heads are repeated to the query
head count (the isolation article's section 7.1 copy-versus-view note),
with query head h reading KV head h // (heads // kv_heads).

It returns the probability matrix as well, so tests can check that every
blocked entry is exactly 0.0 (primer section 2.1 prints that check for the
causal case).
"""
from __future__ import annotations

import numpy as np


def block_diag_mask(intervals, total_len: int) -> np.ndarray:
    """1 inside each [start, end) question block, 0 elsewhere."""
    m = np.zeros((total_len, total_len), dtype=np.float64)
    for start, end in intervals:
        m[start:end, start:end] = 1.0
    return m


def isolation_mask(intervals, total_len: int) -> np.ndarray:
    """Block-diagonal mask times the causal lower triangle (a logical AND)."""
    causal = np.tril(np.ones((total_len, total_len), dtype=np.float64))
    return block_diag_mask(intervals, total_len) * causal


def intervals_from_cu(cu) -> list[tuple[int, int]]:
    cu = [int(x) for x in cu]
    return [(cu[s], cu[s + 1]) for s in range(len(cu) - 1)]


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu, heads: int, kv_heads: int):
    """q[T, heads, d], k/v[T, kv_heads, d] as float64.  Returns (out[T, heads, d], P[heads, T, T])."""
    T, _, d = q.shape
    allowed = isolation_mask(intervals_from_cu(cu), T)
    M = np.where(allowed > 0, 0.0, -np.inf)
    G = heads // kv_heads
    k_rep = np.repeat(k, G, axis=1)          # [T, heads, d], head h <- kv head h // G
    v_rep = np.repeat(v, G, axis=1)
    out = np.zeros((T, heads, d), dtype=np.float64)
    P = np.zeros((heads, T, T), dtype=np.float64)
    for h in range(heads):
        scores = q[:, h, :] @ k_rep[:, h, :].T / np.sqrt(d) + M
        if T == 0:
            continue
        row_max = scores.max(axis=1, keepdims=True)
        row_max = np.where(np.isfinite(row_max), row_max, 0.0)
        e = np.exp(scores - row_max)
        p = e / e.sum(axis=1, keepdims=True)
        P[h] = p
        out[:, h, :] = p @ v_rep[:, h, :]
    return out, P
