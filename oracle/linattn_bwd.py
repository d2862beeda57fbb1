"""Plain CPU float64 oracle for the backward pass of Sana's ReLU linear
self-attention: the gradients of the forward definition.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this module; only
the tests and the benchmark's CPU-baseline leg do. It shares no code with
the HIP path and uses nothing but NumPy (and the forward oracle's decoding).

The forward, per batch item b and head h (see oracle/linattn.py):

  phi(x) = max(x, 0),  S = phi(K)^T V  (d x d),  z = phi(K)^T 1  (d)
  num_i = phi(q_i) S,  den_i = phi(q_i) . z + eps,  out_i = num_i / den_i

Given the gradient g_i = dL/dout_i of a scalar loss L, the chain rule gives,
term by term:

  dnum_i  = g_i / den_i                                  (d)
  dden_i  = -(g_i . num_i) / den_i^2 = -(g_i . out_i) / den_i
  dphi(q_i) = S dnum_i + z dden_i        i.e. [S | z] [dnum_i | dden_i]^T
  dS      = sum_i phi(q_i)^T dnum_i      (d x d)
  dz      = sum_i phi(q_i) dden_i        (d)
  dphi(k_n) = dS v_n + dz                i.e. [dS | dz] [v_n | 1]^T
  dv_n    = phi(k_n) dS
  dq_i = dphi(q_i) * [q_i > 0],   dk_n = dphi(k_n) * [k_n > 0]

Sources: the forward is the one on the pages (course notes, "Linear
Attention 的原理"; Linear-DiT 4K blog, "核心架构"; Sana paper review, section
2.2 "선형 어텐션 블럭"). The review's section 2.2 "Triton을 통한 학습/추론
가속화" fuses this attention's kernels for training as well as inference,
which needs these gradients; no page writes them out, so they are derived
here from the forward definition.

Readings where the pages are silent:
  * The derivative of ReLU at exactly 0 is taken as 0 (the gradient passes
    only where x > 0), the usual subgradient choice.
  * eps is a constant (no gradient).
  * g has the shape and dtype of out; the loss is otherwise arbitrary.

Pins (tests/test_oracle_bwd.py), none of which restates these formulas:
central finite differences of the forward oracle's loss sum(g * out), per
element and along random directions; torch float64 autograd through the
explicit n x n quadratic form; and three exact identities that follow from
homogeneity: sum_c q_ic dq_ic = (g_i . out_i) eps / den_i (scaling phi(q_i)),
sum_n phi(k_n) . dphi(k_n) = sum_i (g_i . out_i) eps / den_i (scaling all of
phi(K)), and sum_n v_n . dv_n = sum_i g_i . out_i (out is linear in V). A
test plants mistakes in this module and checks that the pins catch each one.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .linattn import phi, to_f64


# ------------------------------------------------- the steps, one head


def relu_mask(x: np.ndarray) -> np.ndarray:
    """d phi / dx: 1 where x > 0, else 0 (0 at x == 0, a reading)."""
    return (x > 0).astype(np.float64)


def output_grads(g: np.ndarray, num: np.ndarray, den: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """dL/dnum_i = g_i / den_i and dL/dden_i = -(g_i . num_i) / den_i^2."""
    dnum = g / den[:, None]
    dden = -(g * num).sum(axis=1) / (den * den)
    return dnum, dden


def phi_q_grad(dnum: np.ndarray, dden: np.ndarray, kv: np.ndarray,
               ksum: np.ndarray) -> np.ndarray:
    """dL/dphi(q_i): num_i = phi(q_i) S and den_i = phi(q_i) . z + eps give
    S dnum_i + z dden_i."""
    return dnum @ kv.T + dden[:, None] * ksum[None, :]


def state_grads(pq: np.ndarray, dnum: np.ndarray, dden: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """dL/dS = sum_i phi(q_i)^T dnum_i and dL/dz = sum_i phi(q_i) dden_i."""
    return pq.T @ dnum, pq.T @ dden


def phi_k_grad(v: np.ndarray, dkv: np.ndarray, dksum: np.ndarray) -> np.ndarray:
    """dL/dphi(k_n): S = sum_n phi(k_n)^T v_n and z = sum_n phi(k_n) give
    dS v_n + dz."""
    return v @ dkv.T + dksum[None, :]


def v_grad(pk: np.ndarray, dkv: np.ndarray) -> np.ndarray:
    """dL/dv_n = phi(k_n) dS."""
    return pk @ dkv


def backward_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray,
                  eps: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(dq, dk, dv) of one head; every argument [n, d] float64."""
    pq, pk = phi(q), phi(k)
    kv = pk.T @ v
    ksum = pk.sum(axis=0)
    num = pq @ kv
    den = pq @ ksum + eps
    dnum, dden = output_grads(g, num, den)
    dq = phi_q_grad(dnum, dden, kv, ksum) * relu_mask(q)
    dkv, dksum = state_grads(pq, dnum, dden)
    dk = phi_k_grad(v, dkv, dksum) * relu_mask(k)
    dv = v_grad(pk, dkv)
    return dq, dk, dv


def state_grad_head(q: np.ndarray, g: np.ndarray, kv: np.ndarray, ksum: np.ndarray,
                    eps: float) -> np.ndarray:
    """[dS | dz] of one head as a d x (d+1) matrix, from q, g and the
    forward state (the quantity the backward's token reduction computes)."""
    pq = phi(q)
    num = pq @ kv
    den = pq @ ksum + eps
    dnum, dden = output_grads(g, num, den)
    dkv, dksum = state_grads(pq, dnum, dden)
    return np.concatenate([dkv, dksum[:, None]], axis=1)


# -------------------------------------------------------------- drivers


def linattn_bwd_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray,
                     eps: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients on float64 tensors laid out [B, N, H, d]."""
    if not (q.shape == k.shape == v.shape == g.shape):
        raise ValueError("q, k, v and g must have the same [B, N, H, d] shape")
    B, N, H, d = q.shape
    dq, dk, dv = (np.empty((B, N, H, d), dtype=np.float64) for _ in range(3))
    for b in range(B):
        for h in range(H):
            dq[b, :, h], dk[b, :, h], dv[b, :, h] = backward_head(
                q[b, :, h], k[b, :, h], v[b, :, h], g[b, :, h], eps)
    return dq, dk, dv


def linattn_bwd_from_inputs(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray,
                            eps: float, dtype: str):
    """Gradients from raw inputs (bf16 bits or float32), decoded one head at
    a time to bound memory. Returns three float64 [B, N, H, d] arrays."""
    B, N, H, d = q.shape
    dq, dk, dv = (np.empty((B, N, H, d), dtype=np.float64) for _ in range(3))
    for b in range(B):
        for h in range(H):
            dq[b, :, h], dk[b, :, h], dv[b, :, h] = backward_head(
                to_f64(q[b, :, h], dtype), to_f64(k[b, :, h], dtype),
                to_f64(v[b, :, h], dtype), to_f64(g[b, :, h], dtype), eps)
    return dq, dk, dv
