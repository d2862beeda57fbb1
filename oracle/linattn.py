"""Plain CPU float64 oracle for Sana's ReLU linear self-attention (forward).

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this module; only
the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP path: it decodes bfloat16 itself and uses
nothing but NumPy.

What is computed, per batch item b and head h, with x_n = x[b, n, h, :]:

  phi(x)  = max(x, 0)                       feature map
  KV      = sum_n phi(k_n) (outer) v_n      d x d state       (a)
  ksum    = sum_n phi(k_n)                  length-d state    (b)
  out_i   = phi(q_i) KV / (phi(q_i) . ksum + eps)

Sources (the web pages on Sana):
  * Sana course notes (papers-3lj.pages.dev, "08 Sana 高效高分辨率生成"),
    section "Linear Attention 的原理": phi = ReLU, KV = phi(K)^T V is a d x d
    matrix independent of n, and A = phi(Q) KV.
  * Linear-DiT 4K blog (blog.hotdry.top, "linear diffusion transformer 4k
    efficient generation"), section "核心架构：Linear Attention 与 DC-AE 的协同
    设计": the normalised form phi(Q)(phi(K)^T V) / (phi(Q) phi(K)^T 1), whose
    denominator is phi(q_i) . ksum since phi(K)^T 1 = ksum.
  * Sana paper review (phd-frog.tistory.com/40), section 2.2 "Efficient
    Linear DiT Design", "선형 어텐션 블럭": ReLU linear attention, the shared
    terms (a) and (b) computed once and reused by every query, O(N).

Readings where the pages are silent:
  * eps is on no page. It is added to the denominator, outside the dot
    product: den + eps (not max(den, eps)).
  * d is the per-head width; heads never interact. Batches never interact.
  * No positional term is applied to q or k (NoPE: Sana review, section 2.2
    "Positional Encoding을 없앤 DiT").
  * Attention is non-causal: every query sees all n tokens.
  * A query row with phi(q_i) = 0 gives num = 0 and den + eps = eps, so the
    output row is exactly 0 for eps > 0 (0/0 = NaN for eps = 0).

Pins: every function here is checked by the CPU tests against something
other than itself - the explicit n x n quadratic form, exact rational brute
force on tiny inputs, closed forms (N = 1, constant inputs, one-hot queries)
and invariants (convex-combination bound, positive scaling of K or Q, dead
query rows, dead key tokens, permutation, linearity in V). A test also plants
mistakes in this module and checks that the pins catch each one.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------- decoding


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float64, exactly.

    A bfloat16 value is the upper 16 bits of an IEEE binary32 value, so
    shifting the bits up by 16 gives the binary32 value exactly, and binary32
    widens to binary64 exactly."""
    b = np.asarray(bits).astype(np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Input tensor (bf16 bits as uint16, or float32 values) -> float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ------------------------------------------------------------ the method


def phi(x: np.ndarray) -> np.ndarray:
    """Feature map phi = ReLU (course notes, "Linear Attention 的原理")."""
    return np.maximum(x, 0.0)


def kv_state(k: np.ndarray, v: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Shared terms of one head: KV = phi(K)^T V (d x d) and ksum = phi(K)^T 1.

    k, v: [n, d] float64. The state's size does not depend on n (course
    notes, "Linear Attention 的原理"; blog, normalised formula)."""
    pk = phi(k)
    kv = pk.T @ v
    ksum = pk.sum(axis=0)
    return kv, ksum


def apply_state(q: np.ndarray, kv: np.ndarray, ksum: np.ndarray, eps: float) -> np.ndarray:
    """out_i = phi(q_i) KV / (phi(q_i) . ksum + eps) for q: [m, d] float64."""
    pq = phi(q)
    num = pq @ kv
    den = pq @ ksum
    return num / (den + eps)[:, None]


def linattn_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, eps: float) -> np.ndarray:
    """The forward pass on float64 tensors laid out [B, N, H, d]."""
    B, N, H, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same [B, N, H, d] shape")
    out = np.empty((B, N, H, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kv, ksum = kv_state(k[b, :, h, :], v[b, :, h, :])
            out[b, :, h, :] = apply_state(q[b, :, h, :], kv, ksum, eps)
    return out


def state_fp64(k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Augmented state per (b, h): [B, H, d, d+1], column d holding ksum.

    This is phi(K)^T [V | 1]: the ones column appended to V turns the
    normaliser into one more column of the same contraction."""
    B, N, H, d = k.shape
    st = np.empty((B, H, d, d + 1), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kv, ksum = kv_state(k[b, :, h, :], v[b, :, h, :])
            st[b, h, :, :d] = kv
            st[b, h, :, d] = ksum
    return st


def apply_rows(q_rows: np.ndarray, state: np.ndarray, eps: float) -> np.ndarray:
    """Output rows for selected queries.

    q_rows: [m, H, d] float64 token rows of one batch item; state: [H, d, d+1].
    Returns [m, H, d]."""
    m, H, d = q_rows.shape
    out = np.empty((m, H, d), dtype=np.float64)
    for h in range(H):
        out[:, h, :] = apply_state(q_rows[:, h, :], state[h, :, :d], state[h, :, d], eps)
    return out


# ----------------------------------------------------- bits-level drivers


def linattn_from_inputs(q: np.ndarray, k: np.ndarray, v: np.ndarray, eps: float,
                        dtype: str) -> np.ndarray:
    """Forward pass on raw inputs (bf16 bits or float32), decoded one head at
    a time to bound memory. Returns float64 [B, N, H, d]."""
    B, N, H, d = q.shape
    out = np.empty((B, N, H, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kv, ksum = kv_state(to_f64(k[b, :, h, :], dtype), to_f64(v[b, :, h, :], dtype))
            out[b, :, h, :] = apply_state(to_f64(q[b, :, h, :], dtype), kv, ksum, eps)
    return out


def state_from_inputs(k: np.ndarray, v: np.ndarray, dtype: str,
                      heads: Optional[Sequence[Tuple[int, int]]] = None,
                      token_block: int = 1 << 18) -> np.ndarray:
    """Augmented state [B, H, d, d+1] from raw inputs, one head at a time.

    Long sequences are summed in token blocks (the state is additive over
    tokens, which is what makes it independent of n). ``heads`` restricts the
    work to the listed (b, h) pairs; other entries are left NaN."""
    B, N, H, d = k.shape
    st = np.full((B, H, d, d + 1), np.nan, dtype=np.float64)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        acc_kv = np.zeros((d, d))
        acc_ks = np.zeros(d)
        for n0 in range(0, N, token_block):
            n1 = min(N, n0 + token_block)
            kv, ksum = kv_state(to_f64(k[b, n0:n1, h, :], dtype), to_f64(v[b, n0:n1, h, :], dtype))
            acc_kv += kv
            acc_ks += ksum
        st[b, h, :, :d] = acc_kv
        st[b, h, :, d] = acc_ks
    return st


# ------------------------------------------------- the unreordered form


def quadratic_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, eps: float) -> np.ndarray:
    """The same attention without the associativity reorder.

    Forms the n x n weight matrix W = phi(Q) phi(K)^T per (b, h), its row
    sums r = W 1, and out = (W V) / (r + eps). Quadratic in n: tiny inputs
    only. This is the form linear attention avoids (course notes, "Linear
    Attention 的原理": the n x n intermediate replaced by a d x d one)."""
    B, N, H, d = q.shape
    out = np.empty((B, N, H, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            w = phi(q[b, :, h, :]) @ phi(k[b, :, h, :]).T
            r = w.sum(axis=1)
            out[b, :, h, :] = (w @ v[b, :, h, :]) / (r + eps)[:, None]
    return out
