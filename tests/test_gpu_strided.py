"""GPU parity of the strided forward (sana_linattn_fwd_strided): q, k, v read
in place from one packed [B][N][3][H][d] tensor (the output layout of a fused
QKV linear layer) or with a padded token stride, against the CPU float64
oracle element by element on the same seeded bits, and bitwise against the
contiguous split forward on copies of the same tensors (same plan, same
kernels, only the addressing differs).

Tolerances as for the forward: bf16 max-abs <= 1e-2 and rel-L2 <= 5e-3;
fp32 rel-L2 <= 1e-5 and max-abs <= 1e-5 * max|ref|."""
import numpy as np
import pytest

import oracle.linattn as L
import oracle.linattn_feature_maps as FM
import relu_linear_attention_attn_amd as R
from relu_linear_attention_attn_amd import workloads as W

from gpu_util import assert_close, decode, to_device, to_host, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a ROCm GPU"
    R.lib()
    yield


def _packed(x, dtype, pad=0):
    """q, k, v of x laid side by side per token, [B][N][3 H d + pad], with
    the padding filled with a large finite value that must never be read;
    returns the buffer and the three (B, N, H, d) views."""
    t = torch()
    B, N, H, d = x["q"].shape
    D = H * d
    parts = [to_device(x[n], dtype).reshape(B, N, D) for n in "qkv"]
    buf = t.full((B, N, 3 * D + pad), 1e4, dtype=parts[0].dtype, device="cuda")
    for i, p in enumerate(parts):
        buf[:, :, i * D:(i + 1) * D] = p
    views = [buf[:, :, i * D:(i + 1) * D].view(B, N, H, d) for i in range(3)]
    return buf, views


CASES = [  # (B, N, H, dtype, pad)
    (2, 4096, 6, "bf16", 0), (2, 4096, 6, "f32", 0), (3, 5000, 7, "bf16", 0),
    (3, 5000, 7, "f32", 0), (1, 64, 2, "bf16", 0), (1, 1, 1, "bf16", 0), (2, 17, 1, "f32", 0),
    (2, 1000, 5, "bf16", 8), (2, 1000, 5, "f32", 4), (1, 4099, 36, "bf16", 24),
]


@pytest.mark.parametrize("B,N,H,dtype,pad", CASES)
def test_strided_matches_oracle_and_contiguous(B, N, H, dtype, pad):
    w = W.custom(f"st_{B}_{N}_{H}", B, N, H, dtype=dtype, seed=900 + N + H + pad,
                 q=W.Dist("normal", 0.1, 1.0), k=W.Dist("normal", 0.1, 1.0))
    print(f"\n[case] strided {dtype} B={B} N={N} H={H} pad={pad}", flush=True)
    x = W.generate(w)
    buf, (q, k, v) = _packed(x, dtype, pad)
    assert N == 1 or q.stride(1) == 3 * H * 32 + pad
    out = R.forward_strided(q, k, v, eps=w.eps)
    torch().cuda.synchronize()
    got = to_host(out, dtype)
    ref = L.linattn_from_inputs(x["q"], x["k"], x["v"], w.eps, dtype)
    assert_close(decode(got, dtype), ref, dtype, f"strided B={B} N={N} H={H} pad={pad}")
    c = R.forward(q.contiguous(), k.contiguous(), v.contiguous(), eps=w.eps,
                  variant=R.VARIANT_SPLIT)
    torch().cuda.synchronize()
    assert np.array_equal(got, to_host(c, dtype)), "strided and contiguous differ"


@pytest.mark.parametrize("fmap", ["elu1", "cos"])
def test_strided_other_feature_maps(fmap):
    w = W.custom("st_fm", 2, 3000, 5, seed=951, q=W.Dist("normal", 0.1, 1.0),
                 k=W.Dist("normal", 0.1, 1.0))
    print(f"\n[case] strided fmap {fmap}", flush=True)
    x = W.generate(w)
    buf, (q, k, v) = _packed(x, "bf16")
    out = R.forward_strided(q, k, v, fmap=fmap, eps=w.eps)
    torch().cuda.synchronize()
    got = to_host(out, "bf16")
    ref = FM.linattn_fmap_from_inputs(x["q"], x["k"], x["v"], w.eps, "bf16", fmap)
    g = decode(got, "bf16")
    assert np.max(np.abs(g - ref)) <= max(1e-2, 2.0 ** -8 * np.max(np.abs(ref)))
    c = R.forward_fmap(q.contiguous(), k.contiguous(), v.contiguous(), fmap, eps=w.eps)
    torch().cuda.synchronize()
    assert np.array_equal(got, to_host(c, "bf16"))


def test_strided_contiguous_layout_is_the_forward():
    """ld = H d (plain contiguous tensors) through the strided entry point."""
    w = W.custom("st_ld_hd", 2, 5000, 7, seed=952)
    x = W.generate(w)
    dev = {t: to_device(x[t], "bf16") for t in "qkv"}
    a = R.forward_strided(dev["q"], dev["k"], dev["v"], eps=w.eps)
    b = R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps, variant=R.VARIANT_SPLIT)
    torch().cuda.synchronize()
    assert np.array_equal(to_host(a, "bf16"), to_host(b, "bf16"))


def test_strided_latent_4096px_sampled_heads():
    """The 1.6B model's 4096px latent (B=2, N=16384, H=70) from one packed
    [B][N][3 x 2240] projection output: bitwise equal to the contiguous split
    forward, and two heads compared in full against the oracle."""
    w = W.WORKLOADS["latent_4096px"]
    print(f"\n[case] strided latent {w.shape}", flush=True)
    x = W.generate(w)
    buf, (q, k, v) = _packed(x, "bf16")
    out = R.forward_strided(q, k, v, eps=w.eps)
    c = R.forward(q.contiguous(), k.contiguous(), v.contiguous(), eps=w.eps,
                  variant=R.VARIANT_SPLIT)
    torch().cuda.synchronize()
    got = to_host(out, "bf16")
    assert np.array_equal(got, to_host(c, "bf16"))
    for h in (0, w.H - 1):
        sl = (slice(None), slice(None), slice(h, h + 1))
        ref = L.linattn_from_inputs(x["q"][sl], x["k"][sl], x["v"][sl], w.eps, "bf16")
        assert_close(decode(got[sl], "bf16"), ref, "bf16", f"latent head {h}")


def test_strided_binding_rejects_mixed_strides():
    w = W.custom("st_mix", 1, 64, 2, seed=953)
    x = W.generate(w)
    buf, (q, k, v) = _packed(x, "bf16")
    with pytest.raises(ValueError):
        R.forward_strided(q, k.contiguous(), v, eps=w.eps)
    with pytest.raises(ValueError):
        R.forward_strided(q.transpose(2, 3), k, v, eps=w.eps)
