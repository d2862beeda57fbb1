"""sana_linattn_fwd_noalloc: the forward pass with the library's static device
scratch as its workspace, for callers that cannot allocate.

GPU: through the C ABI, two calls in a row - the second on a smaller input -
each bitwise equal to sana_linattn_fwd on a workspace of its own (same
kernels, grids and summation order) and within the oracle tolerance (bf16
max-abs <= 1e-2 and rel-L2 <= 5e-3; fp32 rel-L2 <= 1e-5). CPU: the size limit
and the argument checks reject before any HIP call."""
import ctypes

import numpy as np
import pytest

import oracle.linattn as L
import relu_linear_attention_attn_amd as R
from relu_linear_attention_attn_amd import workloads as W

from gpu_util import assert_close, decode, to_device, to_host, torch

INVALID, WORKSPACE = 1, 3
A = 1 << 20   # placeholder device addresses for calls the host checks reject


def _ws_size(B, N, H, dt):
    n = ctypes.c_size_t(0)
    assert R.lib().sana_linattn_workspace_size(B, N, H, 32, dt, ctypes.byref(n)) == 0
    return n.value


def test_oversize_and_invalid_calls_rejected_on_host():
    lib = R.lib()
    B, N, H = 128, 16384, 70
    assert _ws_size(B, N, H, R.DTYPE_BF16) > R.binding.SCRATCH_BYTES
    assert lib.sana_linattn_fwd_noalloc(A, 2 * A, 3 * A, 4 * A, B, N, H, 32, 1e-6,
                                        R.DTYPE_BF16, None) == WORKSPACE
    assert _ws_size(2, 16384, 70, R.DTYPE_F32) <= R.binding.SCRATCH_BYTES
    f = lib.sana_linattn_fwd_noalloc
    assert f(A, 2 * A, 3 * A, 4 * A, 0, 64, 2, 32, 1e-6, R.DTYPE_BF16, None) == INVALID
    assert f(A, 2 * A, 3 * A, 4 * A, 1, 64, 2, 32, -1.0, R.DTYPE_BF16, None) == INVALID
    assert f(A, 2 * A, 3 * A, None, 1, 64, 2, 32, 1e-6, R.DTYPE_BF16, None) == INVALID
    assert f(A, 2 * A, 3 * A, A + 64, 1, 64, 2, 32, 1e-6, R.DTYPE_BF16, None) == INVALID
    assert f(A + 8, 2 * A, 3 * A, 4 * A, 1, 64, 2, 32, 1e-6, R.DTYPE_BF16, None) == 4
    assert f(A, 2 * A, 3 * A, 4 * A, 1, 64, 2, 16, 1e-6, R.DTYPE_BF16, None) == 2


def _noalloc(dev, w, out):
    t = torch()
    st = t.cuda.current_stream().cuda_stream
    dt = R.DTYPE_BF16 if w.dtype == "bf16" else R.DTYPE_F32
    return R.lib().sana_linattn_fwd_noalloc(dev["q"].data_ptr(), dev["k"].data_ptr(),
                                            dev["v"].data_ptr(), out.data_ptr(), w.B, w.N, w.H,
                                            32, w.eps, dt, st)


def _with_workspace(dev, w):
    t = torch()
    dt = R.DTYPE_BF16 if w.dtype == "bf16" else R.DTYPE_F32
    ws = t.empty(max(_ws_size(w.B, w.N, w.H, dt), 256), dtype=t.uint8, device="cuda")
    out = t.empty_like(dev["q"])
    st = t.cuda.current_stream().cuda_stream
    assert R.lib().sana_linattn_fwd(dev["q"].data_ptr(), dev["k"].data_ptr(),
                                    dev["v"].data_ptr(), out.data_ptr(), w.B, w.N, w.H, 32,
                                    w.eps, dt, ws.data_ptr(), ws.numel(), st) == 0
    return out


CASES = {
    "bf16": [W.WORKLOADS["latent_4096px"], W.custom("na_small", 1, 5000, 6, seed=61)],
    "f32": [W.custom("na_f32_big", 2, 20000, 36, dtype="f32", seed=62),
            W.custom("na_f32_small", 1, 3001, 5, dtype="f32", seed=63)],
    "fused": [W.custom("na_split", 2, 4096, 36, seed=64), W.custom("na_fused", 2, 900, 7, seed=65)],
}


@pytest.mark.gpu
@pytest.mark.parametrize("case", sorted(CASES))
def test_two_calls_match_the_workspace_entry_point(case):
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a ROCm GPU"
    for i, w in enumerate(CASES[case]):
        print(f"\n[case] noalloc {case} call {i}: {w.name} {w.shape} {w.dtype}", flush=True)
        x = W.generate(w)
        dev = {c: to_device(x[c], w.dtype) for c in "qkv"}
        out = t.full_like(dev["q"], float("nan"))
        assert _noalloc(dev, w, out) == 0
        ref_bits = to_host(_with_workspace(dev, w), w.dtype)
        t.cuda.synchronize()
        got_bits = to_host(out, w.dtype)
        assert np.array_equal(got_bits.view(np.uint8), ref_bits.view(np.uint8)), \
            f"{w.name}: noalloc differs from sana_linattn_fwd"
        if w.N * w.B * w.H <= 2_000_000:
            ref = L.linattn_from_inputs(x["q"], x["k"], x["v"], w.eps, w.dtype)
            assert_close(decode(got_bits, w.dtype), ref, w.dtype, f"noalloc {w.name}")
        else:  # large: two heads in full against the oracle
            for b, h in ((0, 0), (w.B - 1, w.H - 1)):
                ref = L.linattn_from_inputs(x["q"][b:b + 1, :, h:h + 1], x["k"][b:b + 1, :, h:h + 1],
                                            x["v"][b:b + 1, :, h:h + 1], w.eps, w.dtype)
                assert_close(decode(got_bits[b:b + 1, :, h:h + 1], w.dtype), ref, w.dtype,
                             f"noalloc {w.name} head ({b}, {h})")
