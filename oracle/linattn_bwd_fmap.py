"""Plain CPU float64 oracle for the backward pass with other feature maps.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this module; only
the tests and the benchmark's CPU-baseline leg do. It shares no code with
the HIP path and uses nothing but NumPy (and the other oracles' decoding,
feature maps and chain-rule steps).

The forward is the feature-map forward of oracle/linattn_feature_maps.py
(course notes, "Linear Attention 的原理": ELU + 1 and cos named as
alternatives to ReLU; blog, "核心架构": the normalised form). Its gradients
follow from the chain rule exactly as for ReLU (oracle/linattn_bwd.py), with
the map's derivative in place of ReLU's mask:

  dnum_i, dden_i, dS, dz       as for ReLU, from phi(q), phi(k) of this map
  dq_i = (S dnum_i + z dden_i) * phi'(q_i)
  dk_n = (dS v_n + dz) * phi'(k_n)
  dv_n = phi(k_n) dS

with phi'(x), element by element:
  "relu"  1 where x > 0, else 0 (0 at x == 0, the ReLU oracle's reading)
  "elu1"  1 where x > 0, exp(x) at or below 0 (continuous at 0, value 1)
  "cos"   -sin(x)

No page writes these gradients: the review's section 2.2 (Triton section)
fuses this attention for training, and the notes ask for the kernel function
as a parameter, so the backward is derived here for each map.

Pins (tests/test_oracle_bwd_fmap.py), none of which restates these formulas:
central finite differences of the feature-map forward oracle's loss
sum(g * out), along random directions and per element on tiny inputs; torch
float64 autograd through a torch form of the forward definition; "relu"
equal to the ReLU backward oracle. A test plants mistakes in this module and
checks that the pins catch each one.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .linattn import to_f64
from .linattn_bwd import output_grads, phi_k_grad, phi_q_grad, state_grads, v_grad
from .linattn_feature_maps import feature_map


def dphi_relu(x: np.ndarray) -> np.ndarray:
    return (x > 0).astype(np.float64)


def dphi_elu1(x: np.ndarray) -> np.ndarray:
    """d(ELU(x) + 1)/dx with alpha = 1: 1 above 0, exp(x) at or below 0."""
    return np.where(x > 0.0, 1.0, np.exp(np.minimum(x, 0.0)))


def dphi_cos(x: np.ndarray) -> np.ndarray:
    return -np.sin(x)


DERIVATIVES = {"relu": dphi_relu, "elu1": dphi_elu1, "cos": dphi_cos}


def derivative(name: str):
    try:
        return DERIVATIVES[name]
    except KeyError:
        raise ValueError(f"unknown feature map {name!r}") from None


def backward_head_fmap(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, eps: float,
                       fmap: str) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(dq, dk, dv) of one head with feature map `fmap`; every argument
    [n, d] float64."""
    phi, dphi = feature_map(fmap), derivative(fmap)
    pq, pk = phi(q), phi(k)
    kv = pk.T @ v
    ksum = pk.sum(axis=0)
    num = pq @ kv
    den = pq @ ksum + eps
    dnum, dden = output_grads(g, num, den)
    dq = phi_q_grad(dnum, dden, kv, ksum) * dphi(q)
    dkv, dksum = state_grads(pq, dnum, dden)
    dk = phi_k_grad(v, dkv, dksum) * dphi(k)
    dv = v_grad(pk, dkv)
    return dq, dk, dv


def linattn_bwd_fmap_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray,
                          eps: float, fmap: str) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients on float64 tensors laid out [B, N, H, d]."""
    if not (q.shape == k.shape == v.shape == g.shape):
        raise ValueError("q, k, v and g must have the same [B, N, H, d] shape")
    B, N, H, d = q.shape
    dq, dk, dv = (np.empty((B, N, H, d), dtype=np.float64) for _ in range(3))
    for b in range(B):
        for h in range(H):
            dq[b, :, h], dk[b, :, h], dv[b, :, h] = backward_head_fmap(
                q[b, :, h], k[b, :, h], v[b, :, h], g[b, :, h], eps, fmap)
    return dq, dk, dv


def linattn_bwd_fmap_from_inputs(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray,
                                 eps: float, dtype: str, fmap: str):
    """Gradients from raw inputs (bf16 bits or float32), decoded one head at
    a time. Returns three float64 [B, N, H, d] arrays."""
    B, N, H, d = q.shape
    dq, dk, dv = (np.empty((B, N, H, d), dtype=np.float64) for _ in range(3))
    for b in range(B):
        for h in range(H):
            dq[b, :, h], dk[b, :, h], dv[b, :, h] = backward_head_fmap(
                to_f64(q[b, :, h], dtype), to_f64(k[b, :, h], dtype),
                to_f64(v[b, :, h], dtype), to_f64(g[b, :, h], dtype), eps, fmap)
    return dq, dk, dv
