"""The seeded input generator: reproducible, chunk-independent, exact masks."""
import numpy as np
import pytest

from relu_linear_attention_attn_amd import workloads as W


def test_five_workloads_have_the_stated_shapes():
    got = {n: (w.B, w.N, w.H, w.d, w.dtype) for n, w in W.WORKLOADS.items()}
    assert got == {
        "tiny_f32": (1, 256, 2, 32, "f32"),
        "sana06_1024px": (2, 1024, 36, 32, "bf16"),
        "sana16_1024px_b16": (16, 1024, 70, 32, "bf16"),
        "latent_4096px": (2, 16384, 70, 32, "bf16"),
        "video_1m_tokens": (1, 1048576, 36, 32, "bf16"),
    }
    assert W.WORKLOADS[W.HEADLINE].D == 2240
    assert W.WORKLOADS[W.HEADLINE].algorithmic_bytes() == 4 * 2 * 16384 * 2240 * 2


def test_seed_reproduces():
    w = W.custom("r", 2, 100, 3, seed=9)
    a, b = W.generate(w), W.generate(w)
    for t in "qkv":
        assert np.array_equal(a[t], b[t])
    assert not np.array_equal(a["q"], a["k"])


def test_thread_count_does_not_matter():
    w = W.custom("r", 1, 3 * W.CHUNK_ROWS + 5, 1, seed=2)
    a = W.generate_tensor(w, "v", workers=1)
    b = W.generate_tensor(w, "v", workers=4)
    assert np.array_equal(a, b)


def test_row_ranges_equal_slices_of_the_whole():
    w = W.custom("r", 2, W.CHUNK_ROWS + 100, 2, seed=3, mask_tensor="k", mask_frac=0.1)
    full = W.generate_tensor(w, "k").reshape(-1, 2, 32)
    total = w.B * w.N
    part = W.generate_tensor(w, "k", rows=(W.CHUNK_ROWS, total))
    assert np.array_equal(part, full[W.CHUNK_ROWS:])
    with pytest.raises(ValueError):
        W.generate_tensor(w, "k", rows=(5, 10))


@pytest.mark.parametrize("name,which,count", [("sana06_1024px", "k", 102),
                                               ("sana16_1024px_b16", "q", 328)])
def test_mask_counts_are_exact(name, which, count):
    w = W.WORKLOADS[name]
    assert w.n_masked == count
    rows = W.masked_rows(w)
    assert len(rows) == count and len(np.unique(rows)) == count
    if w.B * w.N <= 4096:  # the small one: check every element of the tensor
        x = W.generate_tensor(w, which).reshape(w.B * w.N, -1)
        neg = np.all((x & 0x8000) != 0, axis=1)
        assert set(np.nonzero(neg)[0]) >= set(rows)
        # rows outside the mask are not all-negative (1152 fair coin flips)
        assert neg.sum() == count


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e30).astype(np.float32),
                        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                                  1.0 - 2 ** -9], dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_bf16_bits(x), want)


def test_distributions_have_the_stated_moments():
    w = W.custom("m", 1, W.CHUNK_ROWS, 8, dtype="f32", seed=5,
                 q=W.Dist("normal", 0.1, 1.0), v=W.Dist("normal", 0.0, 0.5),
                 k=W.Dist("student_t", 4.0))
    q = W.generate_tensor(w, "q").ravel().astype(np.float64)
    v = W.generate_tensor(w, "v").ravel().astype(np.float64)
    k = W.generate_tensor(w, "k").ravel().astype(np.float64)
    n = q.size
    assert abs(q.mean() - 0.1) < 5 / np.sqrt(n) and abs(q.std() - 1.0) < 0.01
    assert abs(v.mean()) < 5 * 0.5 / np.sqrt(n) and abs(v.std() - 0.5) < 0.005
    # t(4): variance nu/(nu-2) = 2; P(|t| > 2.776) = 0.05 (two-sided 95% point)
    assert abs(np.mean(np.abs(k) > 2.776445) - 0.05) < 0.002
    assert abs(np.median(k)) < 0.01


def test_upstream_gradient_stream():
    """g (the backward's dL/dout) has its own seeded stream: chunk-parallel
    generation matches serial, it differs from q, k and v, and it is
    N(0, 1)."""
    w = W.custom("gstream", 2, 9000, 3, dtype="f32", seed=21)
    a = W.generate_tensor(w, "g", workers=1)
    b = W.generate_tensor(w, "g", workers=4)
    assert np.array_equal(a, b)
    for t in ("q", "k", "v"):
        assert not np.array_equal(a, W.generate_tensor(w, t, workers=1))
    assert abs(float(a.mean())) < 0.01 and abs(float(a.std()) - 1.0) < 0.01
    x = W.generate(w, grad=True)
    assert set(x) == {"q", "k", "v", "g"} and np.array_equal(x["g"], a)
