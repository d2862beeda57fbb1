"""Plain CPU float64 oracle for block-causal ReLU linear attention.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this module; only
the tests and the benchmark's CPU-baseline leg do. It shares no code with
the HIP path and uses nothing but NumPy (and the forward oracle's decoding).

Source: the Linear-DiT 4K blog, section "技术演进", says SANA-Video extends
Sana's linear attention to Block Causal Linear Attention (with a causal
Mix-FFN) for video generation; no page gives its formula. Reading taken
where the page is silent: the n tokens of a batch item form consecutive
blocks of L tokens (a video frame is such a block; the last block may be
shorter); a query in block c attends to every key in blocks 0..c, in its own
block as much as in the earlier ones. Per (b, h), with the forward's
phi = ReLU and eps:

  S_c   = sum_{n in blocks <= c} phi(k_n)^T [v_n | 1]      (an inclusive prefix
                                                          sum of block states)
  out_i = phi(q_i) S_c(i)[:, :d] / (phi(q_i) . S_c(i)[:, d] + eps)

L = n gives the forward pass of oracle/linattn.py; L = 1 gives token-causal
attention (query i sees keys 0..i). token_causal_rows computes single rows of
that token-causal attention straight from the definition, for sequences whose
per-token prefix states would not fit in memory.

Pins (tests/test_oracle_block_causal.py): the explicit masked n x n form
(mask[i][n] = block(n) <= block(i)) on small inputs; L = n against the
non-causal oracle; L = 1 against a lower-triangular mask; the first block
against the non-causal attention of that block alone; no output depends on
later blocks (changing them leaves earlier outputs bitwise unchanged);
invariance to the choice of L within one block-aligned split; the rows of
token_causal_rows against the lower-triangular masked form. A test plants
mistakes in this module and checks that the pins catch each one.
"""
from __future__ import annotations

import numpy as np

from .linattn import phi, to_f64


def block_states(k: np.ndarray, v: np.ndarray, L: int) -> np.ndarray:
    """Per-block augmented states phi(K_c)^T [V_c | 1] of one head:
    [blocks, d, d+1]."""
    n, d = k.shape
    nb = (n + L - 1) // L
    pk = phi(k)
    va = np.concatenate([v, np.ones((n, 1))], axis=1)
    st = np.empty((nb, d, d + 1))
    for c in range(nb):
        st[c] = pk[c * L:(c + 1) * L].T @ va[c * L:(c + 1) * L]
    return st


def prefix_states(states: np.ndarray) -> np.ndarray:
    """Inclusive prefix sum over blocks: blocks 0..c for entry c."""
    return np.cumsum(states, axis=0)


def apply_prefix(q: np.ndarray, prefix: np.ndarray, L: int, eps: float) -> np.ndarray:
    """Each query row against the prefix state of its own block."""
    n, d = q.shape
    pq = phi(q)
    out = np.empty((n, d))
    for c in range(prefix.shape[0]):
        rows = slice(c * L, (c + 1) * L)
        num = pq[rows] @ prefix[c][:, :d]
        den = pq[rows] @ prefix[c][:, d]
        out[rows] = num / (den + eps)[:, None]
    return out


def block_causal_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, L: int,
                      eps: float) -> np.ndarray:
    return apply_prefix(q, prefix_states(block_states(k, v, L)), L, eps)


def block_causal_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, L: int,
                      eps: float) -> np.ndarray:
    """Block-causal attention on float64 tensors laid out [B, N, H, d]."""
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have the same [B, N, H, d] shape")
    B, N, H, d = q.shape
    out = np.empty((B, N, H, d))
    for b in range(B):
        for h in range(H):
            out[b, :, h] = block_causal_head(q[b, :, h], k[b, :, h], v[b, :, h], L, eps)
    return out


def block_causal_from_inputs(q: np.ndarray, k: np.ndarray, v: np.ndarray, L: int,
                             eps: float, dtype: str) -> np.ndarray:
    """From raw inputs (bf16 bits or float32), one head at a time."""
    B, N, H, d = q.shape
    out = np.empty((B, N, H, d))
    for b in range(B):
        for h in range(H):
            out[b, :, h] = block_causal_head(to_f64(q[b, :, h], dtype), to_f64(k[b, :, h], dtype),
                                             to_f64(v[b, :, h], dtype), L, eps)
    return out


def token_causal_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows, eps: float) -> np.ndarray:
    """Token-causal attention (blocks of one token) of one head, [n, d]
    float64, at the listed query rows only, each from its own definition:
    S_i = phi(K[0..i])^T [V[0..i] | 1], out_i = phi(q_i) S_i[:, :d] /
    (phi(q_i) . S_i[:, d] + eps). Cost O(i d^2) per row, memory O(i d): the
    way to check single outputs of sequences too long for the prefix states
    of every token. Returns [len(rows), d]."""
    n, d = q.shape
    out = np.empty((len(rows), d))
    for r, i in enumerate(rows):
        if not 0 <= i < n:
            raise IndexError(f"row {i} outside 0..{n - 1}")
        pk = phi(k[:i + 1])
        s = pk.T @ np.concatenate([v[:i + 1], np.ones((i + 1, 1))], axis=1)
        pq = phi(q[i])
        out[r] = (pq @ s[:, :d]) / (pq @ s[:, d] + eps)
    return out


def masked_quadratic_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                          eps: float) -> np.ndarray:
    """The explicit n x n form with a 0/1 mask (mask[i][n] = 1 where query i
    sees key n): out = ((W * mask) V) / ((W * mask) 1 + eps), W = phi(Q) phi(K)^T.
    [B, N, H, d] float64."""
    B, N, H, d = q.shape
    out = np.empty((B, N, H, d))
    for b in range(B):
        for h in range(H):
            w = (phi(q[b, :, h]) @ phi(k[b, :, h]).T) * mask
            out[b, :, h] = (w @ v[b, :, h]) / (w.sum(axis=1) + eps)[:, None]
    return out
