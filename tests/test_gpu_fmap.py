"""GPU parity of the forward pass with other feature maps (ReLU, ELU + 1,
cos; sana_linattn_fwd_fmap) against the CPU float64 feature-map oracle,
element by element, on the same seeded bits.

Tolerances: fp32 as for the forward (rel-L2 <= 1e-5, max-abs <= 1e-5 *
max|ref|). bf16 ReLU and ELU + 1: the forward's (rel-L2 <= 5e-3 and
max-abs <= 1e-2); that max-abs rests on |out| < 4 (the bf16 half-ulp there
is 2^-9 |out| < 0.0078), which holds because these maps' weights are
positive and out is a convex combination of V. bf16 cos: rel-L2 <= 5e-3 and
max-abs <= max(1e-2, 2^-8 max|ref|): cos weights can be negative, so outputs
can leave that range, and the bound follows the largest output's half-ulp
with a factor 2 for the fp32 arithmetic before the rounding. The inputs keep
cos's denominator well away from 0 (den is at least a third of the sum of
its terms' magnitudes on every row here, checked in the test)."""
import numpy as np
import pytest

import oracle.linattn_feature_maps as FM
import relu_linear_attention_attn_amd as R
from relu_linear_attention_attn_amd import workloads as W

from gpu_util import decode, metrics, to_device, to_host, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a ROCm GPU"
    R.lib()
    yield


def _check(got, ref, dtype, what, fmap):
    maxabs, rel, refmax = metrics(got, ref)
    msg = f"{what}: max-abs {maxabs:.3e}, rel-L2 {rel:.3e}, max|ref| {refmax:.3e}"
    print(msg, flush=True)
    assert np.all(np.isfinite(got)), msg + " (non-finite output)"
    if dtype == "bf16":
        bound = max(1e-2, 2.0 ** -8 * refmax) if fmap == "cos" else 1e-2
        assert rel <= 5e-3 and maxabs <= bound, msg
    else:
        assert rel <= 1e-5 and maxabs <= 1e-5 * max(refmax, 1e-30), msg


def _cos_conditioning(x, dtype):
    q, k = decode(x["q"], dtype), decode(x["k"], dtype)
    cq, ks = np.cos(q), np.cos(k).sum(axis=1, keepdims=True)
    den = (cq * ks).sum(-1)
    return float((den / (np.abs(cq) * np.abs(ks)).sum(-1)).min())


SHAPES = [(1, 1, 1), (1, 2, 2), (2, 15, 3), (1, 17, 1), (3, 100, 5), (2, 1000, 7), (2, 4099, 4),
          (1, 33000, 3), (2, 1024, 36)]


@pytest.mark.parametrize("fmap", ["relu", "elu1", "cos"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,N,H", SHAPES)
def test_fmap_matches_oracle(B, N, H, dtype, fmap):
    if dtype == "f32" and N * H * B > 200000:
        pytest.skip("fp32 covered by the smaller shapes")
    w = W.custom(f"fm_{B}_{N}_{H}", B, N, H, dtype=dtype, seed=700 + N + H,
                 q=W.Dist("normal", 0.1, 1.0), k=W.Dist("normal", 0.1, 1.0))
    print(f"\n[case] fmap {fmap} {dtype} B={B} N={N} H={H}", flush=True)
    x = W.generate(w)
    if fmap == "cos":
        assert _cos_conditioning(x, dtype) > 0.3
    dev = {t: to_device(x[t], dtype) for t in "qkv"}
    out = R.forward_fmap(dev["q"], dev["k"], dev["v"], fmap, eps=w.eps)
    torch().cuda.synchronize()
    ref = FM.linattn_fmap_from_inputs(x["q"], x["k"], x["v"], w.eps, dtype, fmap)
    _check(decode(to_host(out, dtype), dtype), ref, dtype, f"{fmap} {dtype} B={B} N={N} H={H}",
           fmap)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_relu_map_is_the_split_forward_bitwise(dtype):
    w = W.custom("fm_relu_eq", 2, 5000, 7, dtype=dtype, seed=71)
    x = W.generate(w)
    dev = {t: to_device(x[t], dtype) for t in "qkv"}
    a = R.forward_fmap(dev["q"], dev["k"], dev["v"], "relu", eps=w.eps)
    b = R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps, variant=R.VARIANT_SPLIT)
    torch().cuda.synchronize()
    assert np.array_equal(to_host(a, dtype), to_host(b, dtype))


def test_fmap_repeat_bitwise_and_events():
    w = W.custom("fm_rep", 2, 8192, 6, seed=72)
    x = W.generate(w)
    dev = {t: to_device(x[t], "bf16") for t in "qkv"}
    for fmap in ("elu1", "cos"):
        runs = []
        for _ in range(3):
            runs.append(to_host(R.forward_fmap(dev["q"], dev["k"], dev["v"], fmap, eps=w.eps),
                                "bf16"))
        assert all(np.array_equal(runs[0], r) for r in runs[1:])
        ev = [torch().cuda.Event(enable_timing=True) for _ in range(3)]
        out = R.forward_fmap(dev["q"], dev["k"], dev["v"], fmap, eps=w.eps, events=ev)
        torch().cuda.synchronize()
        assert np.array_equal(to_host(out, "bf16"), runs[0])
        assert all(ev[i].elapsed_time(ev[i + 1]) > 0 for i in range(2))


def test_elu1_headline_shape_sampled_heads():
    """The 4096px latent shape (2 x 16384 tokens, 70 heads) with ELU + 1: two
    heads of each batch item compared in full."""
    w = W.WORKLOADS["latent_4096px"]
    x = W.generate(w)
    dev = {t: to_device(x[t], "bf16") for t in "qkv"}
    got = decode(to_host(R.forward_fmap(dev["q"], dev["k"], dev["v"], "elu1", eps=w.eps), "bf16"),
                 "bf16")
    for h in (0, w.H - 1):
        sl = (slice(None), slice(None), slice(h, h + 1))
        ref = FM.linattn_fmap_from_inputs(x["q"][sl], x["k"][sl], x["v"][sl], w.eps, "bf16",
                                          "elu1")
        _check(got[sl], ref, "bf16", f"latent_4096px elu1 head {h}", "elu1")
