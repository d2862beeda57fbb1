"""Plain CPU float64 oracle for linear attention with other feature maps.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this module; only
the tests and the benchmark's CPU-baseline leg do. It shares no code with
the HIP path and uses nothing but NumPy (and the forward oracle's decoding).

Source: the Sana course notes (papers-3lj.pages.dev, "08 Sana 高效高分辨率生成"),
section "Linear Attention 的原理", take phi = ReLU and note that other
non-linear kernels such as ELU + 1 and cos can stand in for it; the same
notes' design note asks for a linear attention that takes the kernel
function as a parameter. The attention itself is the forward's (blog,
"核心架构"): per batch item b and head h,

  KV    = sum_n phi(k_n) (outer) v_n,   ksum = sum_n phi(k_n)
  out_i = phi(q_i) KV / (phi(q_i) . ksum + eps)

with one of these feature maps, applied element by element:

  "relu"  phi(x) = max(x, 0)
  "elu1"  phi(x) = ELU(x) + 1 = x + 1 for x > 0, exp(x) for x <= 0 (ELU with
          alpha = 1, its usual form; the notes name the function only)
  "cos"   phi(x) = cos(x)

Readings where the notes are silent: ELU's alpha is 1; cos is applied to
each channel as it stands (no reweighting, no scaling); eps is added as in
the forward. With cos, phi can be negative, so den can be 0 or negative:
the formula is evaluated as it stands (no clamp), and a row whose den + eps
is 0 gives inf or NaN.

Pins (tests/test_oracle_feature_maps.py): "relu" equals the forward oracle
bit for bit; every map against the explicit n x n form built with the map
(tiny inputs); the maps' values at points where they are known exactly;
Q = K = 0, where every map gives phi = 1 and out is the mean of V scaled by
N d / (N d + eps); cos's period (K + 2 pi changes nothing); linearity in V
and invariance under a permutation of the (K, V) rows. A test plants
mistakes in this module and checks that the pins catch each one.
"""
from __future__ import annotations

import numpy as np

from .linattn import to_f64


def phi_relu(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0)


def phi_elu1(x: np.ndarray) -> np.ndarray:
    """ELU(x) + 1 with alpha = 1: x + 1 above 0, exp(x) at or below 0 (the
    two branches meet at x = 0 with value 1)."""
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def phi_cos(x: np.ndarray) -> np.ndarray:
    return np.cos(x)


FEATURE_MAPS = {"relu": phi_relu, "elu1": phi_elu1, "cos": phi_cos}


def feature_map(name: str):
    try:
        return FEATURE_MAPS[name]
    except KeyError:
        raise ValueError(f"unknown feature map {name!r}") from None


def state_head(k: np.ndarray, v: np.ndarray, fmap: str):
    """KV = phi(K)^T V and ksum = phi(K)^T 1 of one head ([n, d] inputs)."""
    pk = feature_map(fmap)(k)
    return pk.T @ v, pk.sum(axis=0)


def apply_head(q: np.ndarray, kv: np.ndarray, ksum: np.ndarray, eps: float,
               fmap: str) -> np.ndarray:
    pq = feature_map(fmap)(q)
    return (pq @ kv) / (pq @ ksum + eps)[:, None]


def linattn_fmap_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, eps: float,
                      fmap: str) -> np.ndarray:
    """The forward pass with feature map `fmap` on float64 [B, N, H, d]."""
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have the same [B, N, H, d] shape")
    B, N, H, d = q.shape
    out = np.empty((B, N, H, d))
    for b in range(B):
        for h in range(H):
            kv, ksum = state_head(k[b, :, h], v[b, :, h], fmap)
            out[b, :, h] = apply_head(q[b, :, h], kv, ksum, eps, fmap)
    return out


def linattn_fmap_from_inputs(q: np.ndarray, k: np.ndarray, v: np.ndarray, eps: float,
                             dtype: str, fmap: str) -> np.ndarray:
    """From raw inputs (bf16 bits or float32), decoded one head at a time."""
    B, N, H, d = q.shape
    out = np.empty((B, N, H, d))
    for b in range(B):
        for h in range(H):
            kv, ksum = state_head(to_f64(k[b, :, h], dtype), to_f64(v[b, :, h], dtype), fmap)
            out[b, :, h] = apply_head(to_f64(q[b, :, h], dtype), kv, ksum, eps, fmap)
    return out
