"""Plain CPU float64 oracle for the QKV projection followed by the attention
(the projection whose epilogue produces the ReLU(K)^T V state).

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this module; only
the tests and the benchmark's CPU-baseline leg do. It shares no code with
the HIP path and uses nothing but NumPy and the forward oracle.

Source: the Sana paper review (phd-frog.tistory.com/40), section 4: the
deployment kernels fold linear attention's ReLU(K)^T V product into the QKV
projection layer (with linear attention and the key-value projection kept
at full precision). The projection is the linear map of a Linear DiT
block's token features x (width C) to q, k and v (width D = H d each); the
attention is the forward of oracle/linattn.py.

  [q | k | v] = x W^T            W: [3 D][C], rows 0..D-1 give q, D..2D-1 k,
                                 2D..3D-1 v; within each, head h holds rows
                                 h d .. h d + d - 1
  q, k, v rounded to bf16        (the projection's output type)
  out = forward(q, k, v, eps)

Readings where the review is silent: the weight has the [out][in] layout
of a linear layer with no bias (the pages name none); q, k and v are rounded
to bfloat16, round-to-nearest-even, as a bf16 projection would store them,
so the fused kernel computes what the unfused bf16 pipeline computes.

Pins (tests/test_oracle_qkv.py): the projection against a triple loop on
tiny inputs; the bf16 rounding against torch's conversion on
float32-representable values and against exact ties; a selection W (rows of
the identity) that makes q, k, v slices of x, where the whole path equals
the forward oracle on those slices; the state of the projected k, v against
the forward oracle's. A test plants mistakes in this module and checks that
the pins catch each one.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from . import linattn as L


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (ties to even), as float64. bf16
    keeps 8 significant bits: with a = m 2^e, m in [0.5, 1), m is rounded to
    a multiple of 2^-8 (numpy rounds half to even). Zero stays zero; the
    inputs here never leave bf16's exponent range."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def project(x: np.ndarray, w: np.ndarray, H: int, d: int = 32) -> Tuple[np.ndarray, ...]:
    """x: [B, N, C], w: [3 H d, C] float64 -> unrounded q, k, v [B, N, H, d]."""
    B, N, C = x.shape
    D = H * d
    if w.shape != (3 * D, C):
        raise ValueError(f"w must be [3 H d, C] = [{3 * D}, {C}]")
    y = x.reshape(B * N, C) @ w.T                       # [B N, 3 D]
    return tuple(y[:, i * D:(i + 1) * D].reshape(B, N, H, d) for i in range(3))


def qkv_attention_fp64(x: np.ndarray, w: np.ndarray, H: int, eps: float,
                       d: int = 32) -> Tuple[np.ndarray, np.ndarray]:
    """(q rounded to bf16, out) for float64 x [B, N, C] and w [3 H d, C]."""
    q, k, v = (round_bf16(t) for t in project(x, w, H, d))
    return q, L.linattn_fp64(q, k, v, eps)


def qkv_attention_from_inputs(x: np.ndarray, w: np.ndarray, H: int, eps: float,
                              d: int = 32) -> Tuple[np.ndarray, np.ndarray]:
    """From bf16 bits (uint16) of x and w."""
    return qkv_attention_fp64(L.bf16_bits_to_f64(x), L.bf16_bits_to_f64(w), H, eps, d)
