"""Seeded random shapes through every entry point, against the CPU float64
oracles: the forward (each variant and dtype), the strided forward on a
packed projection output with a random row padding, the other feature maps,
block-causal attention with a random block length, token-causal attention,
the backward (ReLU, ELU + 1, cos; from a saved state bitwise as recomputing), and the QKV projection path. The shapes are drawn from a fixed seed, with token
counts near the kernels' boundaries (multiples of the 16-token tile, the
256-token projection tile, the fused variant's 1024-token limit) more often
than elsewhere, and small enough for the oracle to finish in seconds.

Tolerances are the ones each entry point's own parity file states: bf16
max-abs <= 1e-2 and rel-L2 <= 5e-3, fp32 rel-L2 <= 1e-5 (gpu_util); other
maps max-abs <= max(1e-2, 2^-8 max|ref|); token-causal per element
2^-8 |ref| + 2e-3; the backward's and the QKV q's term-scaled bounds
(imported from those files)."""
import numpy as np
import pytest

import oracle.linattn as L
import oracle.linattn_block_causal as BC
import oracle.linattn_bwd as LB
import oracle.linattn_feature_maps as FM
import oracle.linattn_qkv as QK
import relu_linear_attention_attn_amd as R
from relu_linear_attention_attn_amd import workloads as W

from gpu_util import assert_close, decode, to_device, to_host, torch

pytestmark = pytest.mark.gpu

COUNT = 12  # shapes per entry point


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a ROCm GPU"
    R.lib()
    yield


def _draw(seed: int):
    """(B, N, H) triples: N near 16 k, 256 k or 1024 half the time."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(COUNT):
        B = int(rng.integers(1, 4))
        H = int(rng.integers(1, 10))
        if rng.random() < 0.5:
            base = int(rng.choice([16, 256, 1024])) * int(rng.integers(1, 3))
            N = max(1, base + int(rng.integers(-2, 3)))
        else:
            N = int(rng.integers(1, 2500))
        out.append((B, N, H))
    return out


def _workload(tag, B, N, H, dtype, seed):
    return W.custom(f"rand_{tag}_{B}_{N}_{H}", B, N, H, dtype=dtype, seed=seed,
                    q=W.Dist("normal", 0.1, 1.0), k=W.Dist("normal", 0.1, 1.0))


@pytest.mark.parametrize("i", range(COUNT))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_random(i, dtype):
    B, N, H = _draw(1001)[i]
    w = _workload("fwd", B, N, H, dtype, 2000 + i)
    print(f"\n[case] random forward {dtype} B={B} N={N} H={H}", flush=True)
    x = W.generate(w)
    dev = {t: to_device(x[t], dtype) for t in "qkv"}
    ref = L.linattn_from_inputs(x["q"], x["k"], x["v"], w.eps, dtype)
    for name, var in (("auto", R.VARIANT_AUTO), ("split", R.VARIANT_SPLIT),
                      ("fused", R.VARIANT_FUSED)):
        out = R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps, variant=var)
        torch().cuda.synchronize()
        assert_close(decode(to_host(out, dtype), dtype), ref, dtype,
                     f"B={B} N={N} H={H} {dtype} {name}")


@pytest.mark.parametrize("i", range(COUNT))
def test_strided_random(i):
    B, N, H = _draw(1002)[i]
    rng = np.random.default_rng(3000 + i)
    dtype = "bf16" if i % 2 == 0 else "f32"
    pad = int(rng.integers(0, 5)) * (8 if dtype == "bf16" else 4)
    w = _workload("strided", B, N, H, dtype, 3000 + i)
    print(f"\n[case] random strided {dtype} B={B} N={N} H={H} pad={pad}", flush=True)
    x = W.generate(w)
    t = torch()
    D = H * 32
    parts = [to_device(x[n], dtype).reshape(B, N, D) for n in "qkv"]
    buf = t.full((B, N, 3 * D + pad), 3e4, dtype=parts[0].dtype, device="cuda")
    for j, p in enumerate(parts):
        buf[:, :, j * D:(j + 1) * D] = p
    q, k, v = (buf[:, :, j * D:(j + 1) * D].view(B, N, H, 32) for j in range(3))
    out = R.forward_strided(q, k, v, eps=w.eps)
    t.cuda.synchronize()
    ref = L.linattn_from_inputs(x["q"], x["k"], x["v"], w.eps, dtype)
    assert_close(decode(to_host(out, dtype), dtype), ref, dtype,
                 f"strided B={B} N={N} H={H} pad={pad} {dtype}")


@pytest.mark.parametrize("i", range(COUNT))
def test_feature_maps_random(i):
    B, N, H = _draw(1003)[i]
    fmap = ("elu1", "cos")[i % 2]
    w = _workload("fmap", B, N, H, "bf16", 4000 + i)
    print(f"\n[case] random fmap {fmap} B={B} N={N} H={H}", flush=True)
    x = W.generate(w)
    dev = {t: to_device(x[t], "bf16") for t in "qkv"}
    out = R.forward_fmap(dev["q"], dev["k"], dev["v"], fmap, eps=w.eps)
    torch().cuda.synchronize()
    ref = FM.linattn_fmap_from_inputs(x["q"], x["k"], x["v"], w.eps, "bf16", fmap)
    got = decode(to_host(out, "bf16"), "bf16")
    diff = got - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30))
    maxabs = float(np.max(np.abs(diff)))
    msg = f"{fmap} B={B} N={N} H={H}: max-abs {maxabs:.3e}, rel-L2 {rel:.3e}"
    print(msg, flush=True)
    assert rel <= 5e-3 and maxabs <= max(1e-2, 2.0 ** -8 * float(np.max(np.abs(ref)))), msg


@pytest.mark.parametrize("i", range(COUNT))
def test_block_causal_random(i):
    B, N, H = _draw(1004)[i]
    rng = np.random.default_rng(5000 + i)
    divisors = [L_ for L_ in range(1, N + 1) if N % L_ == 0]
    block = int(divisors[int(rng.integers(0, len(divisors)))])
    if N // block > 512:  # keep the oracle's per-block loop short
        block = N
    w = _workload("bc", B, N, H, "bf16", 5000 + i)
    print(f"\n[case] random block-causal B={B} N={N} H={H} block={block}", flush=True)
    x = W.generate(w)
    dev = {t: to_device(x[t], "bf16") for t in "qkv"}
    out = R.forward_block_causal(dev["q"], dev["k"], dev["v"], block, eps=w.eps)
    torch().cuda.synchronize()
    ref = BC.block_causal_from_inputs(x["q"], x["k"], x["v"], block, w.eps, "bf16")
    assert_close(decode(to_host(out, "bf16"), "bf16"), ref, "bf16",
                 f"block-causal B={B} N={N} H={H} block={block}")


@pytest.mark.parametrize("i", range(COUNT))
def test_causal_random(i):
    from test_gpu_causal import assert_causal_close

    B, N, H = _draw(1007)[i]
    w = _workload("causal", B, N, H, "bf16", 7000 + i)
    print(f"\n[case] random token-causal B={B} N={N} H={H}", flush=True)
    x = W.generate(w)
    dev = {t: to_device(x[t], "bf16") for t in "qkv"}
    out = R.forward_causal(dev["q"], dev["k"], dev["v"], eps=w.eps)
    torch().cuda.synchronize()
    ref = BC.block_causal_from_inputs(x["q"], x["k"], x["v"], 1, w.eps, "bf16")
    assert_causal_close(decode(to_host(out, "bf16"), "bf16"), ref,
                        f"token-causal B={B} N={N} H={H}")


@pytest.mark.parametrize("i", range(COUNT))
def test_backward_random(i):
    from test_gpu_bwd import _check

    B, N, H = _draw(1005)[i]
    w = _workload("bwd", B, N, H, "bf16", 6000 + i)
    print(f"\n[case] random backward B={B} N={N} H={H}", flush=True)
    x = W.generate(w, grad=True)
    dev = {t: to_device(x[t], "bf16") for t in "qkvg"}
    dq, dk, dv = R.backward(dev["q"], dev["k"], dev["v"], dev["g"], eps=w.eps)
    torch().cuda.synchronize()
    got = [to_host(t, "bf16") for t in (dq, dk, dv)]
    ref = LB.linattn_bwd_from_inputs(x["q"], x["k"], x["v"], x["g"], w.eps, "bf16")
    _check(got, ref, x, w.eps, f"B={B} N={N} H={H}")


@pytest.mark.parametrize("i", range(COUNT))
def test_backward_fmap_random(i):
    import oracle.linattn_bwd_fmap as LBF
    from test_gpu_bwd_fmap import _check as _check_fmap, _cos_conditioning

    B, N, H = _draw(1007)[i]
    fmap = ("elu1", "cos")[i % 2]
    w = _workload("bwdfm", B, N, H, "bf16", 6500 + i)
    print(f"\n[case] random backward {fmap} B={B} N={N} H={H}", flush=True)
    x = W.generate(w, grad=True)
    if fmap == "cos":
        assert _cos_conditioning(x) > 0.3
    dev = {t: to_device(x[t], "bf16") for t in "qkvg"}
    dq, dk, dv = R.backward(dev["q"], dev["k"], dev["v"], dev["g"], eps=w.eps, fmap=fmap)
    torch().cuda.synchronize()
    got = [to_host(t, "bf16") for t in (dq, dk, dv)]
    ref = LBF.linattn_bwd_fmap_from_inputs(x["q"], x["k"], x["v"], x["g"], w.eps, "bf16", fmap)
    _check_fmap(got, ref, x, w.eps, fmap, f"{fmap} B={B} N={N} H={H}")


@pytest.mark.parametrize("i", range(COUNT))
def test_backward_saved_state_random(i):
    """The backward from kv_state's saved state gives the recomputing
    backward's bits."""
    B, N, H = _draw(1009)[i]
    w = _workload("bwdst", B, N, H, "bf16", 7000 + i)
    print(f"\n[case] random backward from a saved state B={B} N={N} H={H}", flush=True)
    x = W.generate(w, grad=True)
    dev = {t: to_device(x[t], "bf16") for t in "qkvg"}
    a = R.backward(dev["q"], dev["k"], dev["v"], dev["g"], eps=w.eps)
    b = R.backward(dev["q"], dev["k"], dev["v"], dev["g"], eps=w.eps,
                   state=R.kv_state(dev["k"], dev["v"]))
    torch().cuda.synchronize()
    for name, s, t in zip(("dq", "dk", "dv"), a, b):
        assert np.array_equal(to_host(s, "bf16"), to_host(t, "bf16")), name


@pytest.mark.parametrize("i", range(COUNT))
def test_qkv_random(i):
    from test_gpu_qkv import _check_q, _dev, _terms

    B, N, H = _draw(1006)[i]
    rng = np.random.default_rng(7000 + i)
    C = 8 * int(rng.integers(1, 97))  # 8 .. 768 channels, multiples of 8
    w = W.custom(f"rand_qkv_{B}_{N}_{C}_{H}", B, N, H, seed=7000 + i)
    print(f"\n[case] random qkv B={B} N={N} C={C} H={H}", flush=True)
    x = W.projection_inputs(w, C)
    q, out = R.forward_qkv(_dev(x["x"]), _dev(x["w"]), H, eps=w.eps)
    torch().cuda.synchronize()
    qref, oref = QK.qkv_attention_from_inputs(x["x"], x["w"], H, w.eps)
    _check_q(to_host(q, "bf16"), qref, _terms(x["x"], x["w"]), C,
             f"B={B} N={N} C={C} H={H}")
    assert_close(decode(to_host(out, "bf16"), "bf16"), oref, "bf16",
                 f"qkv B={B} N={N} C={C} H={H}")
