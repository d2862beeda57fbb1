"""Seeded synthetic workloads for ReLU linear self-attention.

This module only draws input tensors. It holds none of the attention
arithmetic, so both the HIP path and the CPU oracle can take its output
without sharing any of the method's code.

Shapes follow the pages on Sana:
  * tokens per image come from the 32x-compression autoencoder with patch 1
    (Sana review, section 2.1.2 "AutoEncoder Design Philosophy": 1024px ->
    32x32 tokens; Linear-DiT 4K blog, section on DC-AE: 4K -> 16k tokens);
  * the 1.6B model is 2240 channels wide (Sana review, section 5 "Model
    details"), split here into 70 heads of 32 channels;
  * the long case is the video token count of the Sana course notes' memory
    table (16 frames x 65,536 tokens = 1,048,576).

Layout of every tensor: ``[B][N][H][d]`` row-major, i.e. a token row of
``D = H*d`` channels per (b, n).

Recipe (all draws in float64, then rounded to float32, then - for bf16
workloads - rounded to bfloat16 with round-to-nearest-even):
  * token rows ``r = b*N + n`` are cut into chunks of ``CHUNK_ROWS`` rows;
    chunk ``c`` of tensor ``t`` (q=0, k=1, v=2; g=4, the upstream gradient
    dL/dout that the backward pass takes, N(0, 1) unless stated) draws from
    ``PCG64(SeedSequence([seed, t, c]))``, so generation is chunk-parallel and
    the result does not depend on the number of worker threads;
  * ``normal(mu, sigma)``: ``mu + sigma * standard_normal``;
  * ``student_t(nu)``: ``z / sqrt(g / (nu/2))`` with ``z`` standard normal and
    ``g ~ Gamma(nu/2, 1)``, the textbook construction (chi-square over its
    degrees of freedom is ``2g/nu``);
  * "rows made all-negative": exactly ``round(frac * B * N)`` token rows,
    chosen without replacement by ``PCG64(SeedSequence([seed, 3, 0]))``,
    get every channel replaced by ``-|x|`` (the sign bit set);
  * the QKV projection's inputs (``projection_inputs``): token features x
    ``[B][N][C]`` ~ N(0, 1) (tensor 5) and the weight ``[3 D][C]`` ~
    N(0, 1/C) (tensor 6, so each projected channel has unit variance), drawn
    in chunks of ``CHUNK_ROWS`` rows the same way, always bfloat16.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import numpy as np

CHUNK_ROWS = 8192
TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "g": 4, "x": 5, "w": 6}
MASK_STREAM = 3


@dataclass(frozen=True)
class Dist:
    kind: str  # "normal" | "student_t"
    a: float = 0.0  # normal: mean;  student_t: degrees of freedom
    b: float = 1.0  # normal: standard deviation

    def describe(self) -> str:
        if self.kind == "normal":
            return f"N({self.a:g}, {self.b:g}^2)"
        return f"t(nu={self.a:g})"


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    N: int
    H: int
    d: int
    dtype: str  # "f32" | "bf16"
    eps: float
    q: Dist
    k: Dist
    v: Dist
    mask_tensor: Optional[str] = None  # which tensor gets all-negative rows
    mask_frac: float = 0.0
    g: Dist = Dist("normal", 0.0, 1.0)  # upstream gradient (backward pass only)

    @property
    def D(self) -> int:
        return self.H * self.d

    @property
    def shape(self) -> Tuple[int, int, int, int]:
        return (self.B, self.N, self.H, self.d)

    @property
    def itemsize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def n_masked(self) -> int:
        return int(round(self.mask_frac * self.B * self.N))

    def algorithmic_bytes(self) -> int:
        """Read q, k, v once and write out once."""
        return 4 * self.B * self.N * self.H * self.d * self.itemsize

    def replace(self, **kw) -> "Workload":
        fields = dict(self.__dict__)
        fields.update(kw)
        return Workload(**fields)


EPS = 1e-6
STD = Dist("normal", 0.0, 1.0)

WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        # 16x16 latent, two heads, fp32; small enough for the explicit n x n form.
        Workload("tiny_f32", 1, 1, 256, 2, 32, "f32", EPS, STD, STD, STD),
        # Sana-0.6B-shaped 1024px block, CFG pair; 5% of K rows all-negative.
        Workload("sana06_1024px", 2, 2, 1024, 36, 32, "bf16", EPS, STD, STD, STD,
                 mask_tensor="k", mask_frac=0.05),
        # Sana-1.6B-shaped 1024px batch of 16; 2% of Q rows all-negative.
        Workload("sana16_1024px_b16", 3, 16, 1024, 70, 32, "bf16", EPS, STD, STD,
                 Dist("normal", 0.0, 0.5), mask_tensor="q", mask_frac=0.02),
        # 4096px latent (128x128 tokens), width 2240: the headline shape.
        Workload("latent_4096px", 4, 2, 16384, 70, 32, "bf16", EPS,
                 Dist("normal", 0.1, 1.0), Dist("normal", 0.1, 1.0), STD),
        # 16 frames of 256x256 tokens, flattened, non-causal; heavy-tailed Q, K.
        Workload("video_1m_tokens", 5, 1, 1 << 20, 36, 32, "bf16", EPS,
                 Dist("student_t", 4.0), Dist("student_t", 4.0), STD),
    ]
}
ORDER = ["tiny_f32", "sana06_1024px", "sana16_1024px_b16", "latent_4096px",
         "video_1m_tokens"]
HEADLINE = "latent_4096px"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.

    Finite inputs only (the workloads never produce NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _draw(dist: Dist, rng: np.random.Generator, n: int) -> np.ndarray:
    if dist.kind == "normal":
        z = rng.standard_normal(n)
        if dist.b != 1.0:
            z *= dist.b
        if dist.a != 0.0:
            z += dist.a
        return z
    if dist.kind == "student_t":
        half = dist.a / 2.0
        z = rng.standard_normal(n)
        g = rng.standard_gamma(half, n)
        g /= half
        np.sqrt(g, out=g)
        z /= g
        return z
    raise ValueError(f"unknown distribution {dist.kind!r}")


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate_tensor(w: Workload, which: str, rows: Optional[Tuple[int, int]] = None,
                    workers: Optional[int] = None) -> np.ndarray:
    """Draw tensor ``which`` ('q', 'k', 'v', or 'g' for the backward's
    upstream gradient) of workload ``w``.

    Returns uint16 bf16 bits or float32 values, shaped ``[rows, H, d]`` over
    the flattened token rows ``r = b*N + n`` in ``rows = (r0, r1)`` (default:
    all rows, reshaped to ``[B, N, H, d]``). ``r0`` must be a multiple of
    ``CHUNK_ROWS``. The all-negative row mask is applied when ``which`` is the
    workload's masked tensor.
    """
    tid = TENSOR_IDS[which]
    dist = getattr(w, which)
    total = w.B * w.N
    r0, r1 = (0, total) if rows is None else rows
    if r0 % CHUNK_ROWS or not (0 <= r0 <= r1 <= total):
        raise ValueError("row range must start on a chunk boundary and lie inside the tensor")
    D = w.D
    out_dtype = np.float32 if w.dtype == "f32" else np.uint16
    out = np.empty((r1 - r0, D), dtype=out_dtype)

    def one(c: int) -> None:
        a = c * CHUNK_ROWS
        b = min(a + CHUNK_ROWS, r1)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, tid, c])))
        vals = _draw(dist, rng, (b - a) * D).astype(np.float32).reshape(b - a, D)
        if w.dtype == "f32":
            out[a - r0:b - r0] = vals
        else:
            out[a - r0:b - r0] = f32_to_bf16_bits(vals)

    chunks = range(r0 // CHUNK_ROWS, (r1 + CHUNK_ROWS - 1) // CHUNK_ROWS)
    nw = workers or _workers()
    if nw == 1 or len(chunks) == 1:
        for c in chunks:
            one(c)
    else:
        with ThreadPoolExecutor(nw) as ex:
            list(ex.map(one, chunks))

    if w.mask_tensor == which and w.n_masked:
        sel = masked_rows(w)
        sel = sel[(sel >= r0) & (sel < r1)] - r0
        if w.dtype == "f32":
            out[sel] = -np.abs(out[sel])
        else:
            out[sel] |= np.uint16(0x8000)
    if rows is None:
        return out.reshape(w.B, w.N, w.H, w.d)
    return out.reshape(r1 - r0, w.H, w.d)


def masked_rows(w: Workload) -> np.ndarray:
    """Sorted flattened token rows (b*N + n) that are made all-negative."""
    if not w.mask_tensor or not w.n_masked:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, MASK_STREAM, 0])))
    return np.sort(rng.choice(w.B * w.N, size=w.n_masked, replace=False)).astype(np.int64)


def generate(w: Workload, workers: Optional[int] = None, grad: bool = False) -> Dict[str, np.ndarray]:
    """The input tensors of ``w`` as ``{'q','k','v'}`` (plus ``'g'`` with
    ``grad``) -> [B, N, H, d]."""
    names = ("q", "k", "v", "g") if grad else ("q", "k", "v")
    return {t: generate_tensor(w, t, workers=workers) for t in names}


def custom(name: str, B: int, N: int, H: int, dtype: str = "bf16", seed: int = 11,
           eps: float = EPS, q: Dist = STD, k: Dist = STD, v: Dist = STD, d: int = 32,
           mask_tensor: Optional[str] = None, mask_frac: float = 0.0) -> Workload:
    """A workload of arbitrary shape with the same recipe (for ragged cases)."""
    return Workload(name, seed, B, N, H, d, dtype, eps, q, k, v, mask_tensor, mask_frac)


def generate_matrix(seed: int, tid: int, rows: int, width: int, dist: Dist,
                    workers: Optional[int] = None) -> np.ndarray:
    """A [rows, width] bf16 matrix (uint16 bits) drawn chunk by chunk of
    CHUNK_ROWS rows from PCG64(SeedSequence([seed, tid, chunk]))."""
    out = np.empty((rows, width), dtype=np.uint16)

    def one(c: int) -> None:
        a = c * CHUNK_ROWS
        b = min(a + CHUNK_ROWS, rows)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, c])))
        out[a:b] = f32_to_bf16_bits(_draw(dist, rng, (b - a) * width).astype(np.float32)
                                    .reshape(b - a, width))

    chunks = range((rows + CHUNK_ROWS - 1) // CHUNK_ROWS)
    nw = workers or _workers()
    if nw == 1 or len(chunks) <= 1:
        for c in chunks:
            one(c)
    else:
        with ThreadPoolExecutor(nw) as ex:
            list(ex.map(one, chunks))
    return out


def projection_inputs(w: Workload, C: int, workers: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of the QKV projection for workload w's attention shape:
    {'x': [B, N, C], 'w': [3 D, C]}, bf16 bits."""
    x = generate_matrix(w.seed, TENSOR_IDS["x"], w.B * w.N, C, STD, workers)
    wt = generate_matrix(w.seed, TENSOR_IDS["w"], 3 * w.D, C, Dist("normal", 0.0, C ** -0.5),
                         workers)
    return {"x": x.reshape(w.B, w.N, C), "w": wt}
