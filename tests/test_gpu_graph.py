"""The library's launches captured in a HIP graph and replayed.

A captured launch keeps the arguments it was captured with, among them the
per-call tag of the control words through which the last block of a head
pair folds the pair's partials (the fp32 reduction and sana_linattn_kv_state).
Each case captures one call, then replays the graph four times; before each
replay the inputs are overwritten with new values (eager work on the same
stream, then a device synchronisation), and every replay's result must equal,
bit for bit, an eager call on the same inputs with its own workspace (same
kernels, grids and summation order). The eager results are themselves checked
against the oracle by the parity tests."""
import ctypes

import numpy as np
import pytest

import relu_linear_attention_attn_amd as R
from relu_linear_attention_attn_amd import workloads as W

from gpu_util import to_device, to_host, torch

REPLAYS = 4


def _stream():
    return torch().cuda.current_stream().cuda_stream


def _ws(size_fn, *args):
    t = torch()
    n = ctypes.c_size_t(0)
    assert size_fn(*args, ctypes.byref(n)) == 0
    return t.empty(max(n.value, 256), dtype=t.uint8, device="cuda")


def _fwd(dev, w, out, ws, noalloc=False):
    lib = R.lib()
    dt = R.DTYPE_BF16 if w.dtype == "bf16" else R.DTYPE_F32
    ptrs = (dev["q"].data_ptr(), dev["k"].data_ptr(), dev["v"].data_ptr(), out.data_ptr())
    if noalloc:
        return lib.sana_linattn_fwd_noalloc(*ptrs, w.B, w.N, w.H, 32, w.eps, dt, _stream())
    return lib.sana_linattn_fwd(*ptrs, w.B, w.N, w.H, 32, w.eps, dt, ws.data_ptr(), ws.numel(),
                                _stream())


def _kv_state(dev, w, state, ws):
    dt = R.DTYPE_BF16 if w.dtype == "bf16" else R.DTYPE_F32
    return R.lib().sana_linattn_kv_state(dev["k"].data_ptr(), dev["v"].data_ptr(),
                                         state.data_ptr(), w.B, w.N, w.H, 32, dt, ws.data_ptr(),
                                         ws.numel(), _stream())


CASES = {
    # fp32 beyond the fused range: reduction with the fold, then the apply
    "fwd_f32_split": (W.custom("g_f32", 2, 3000, 5, dtype="f32", seed=71), "fwd"),
    "noalloc_f32_split": (W.custom("g_f32_na", 1, 4100, 6, dtype="f32", seed=72), "noalloc"),
    # bf16 state alone: the bf16 reduction with the fold
    "kv_state_bf16": (W.custom("g_kv", 2, 5000, 7, seed=73), "kv"),
    # bf16 split forward (partials straight to the apply, no fold)
    "fwd_bf16_split": (W.custom("g_bf16", 1, 8192, 6, seed=74), "fwd"),
}


@pytest.mark.gpu
@pytest.mark.parametrize("case", sorted(CASES))
def test_graph_replays_match_eager_calls(case):
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a ROCm GPU"
    w, kind = CASES[case]
    dt = R.DTYPE_BF16 if w.dtype == "bf16" else R.DTYPE_F32
    print(f"\n[case] graph {case}: {w.name} {w.shape} {w.dtype}", flush=True)
    lib = R.lib()
    x = W.generate(w)
    dev = {c: to_device(x[c], w.dtype) for c in "qkv"}
    if kind == "kv":
        res = t.empty((w.B, w.H, 32, 33), dtype=t.float32, device="cuda")
        ws = _ws(lib.sana_linattn_workspace_size, w.B, w.N, w.H, 32, dt)
        run = lambda: _kv_state(dev, w, res, ws)  # noqa: E731
    else:
        res = t.empty_like(dev["q"])
        ws = _ws(lib.sana_linattn_workspace_size, w.B, w.N, w.H, 32, dt)
        run = lambda: _fwd(dev, w, res, ws, noalloc=kind == "noalloc")  # noqa: E731
    assert run() == 0  # eager first: device look-ups happen outside the capture
    t.cuda.synchronize()

    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        status = run()
    assert status == 0

    ref_ws = _ws(lib.sana_linattn_workspace_size, w.B, w.N, w.H, 32, dt)
    rng = np.random.default_rng(1000 + sorted(CASES).index(case))
    for r in range(REPLAYS):
        # new inputs for this replay: scaled and shifted copies of the first draw
        for c in "qkv":
            src = t.from_numpy(np.ascontiguousarray(x[c]).view(np.int16)).view(t.bfloat16) \
                if w.dtype == "bf16" else t.from_numpy(np.ascontiguousarray(x[c]))
            a, b = float(rng.uniform(0.5, 2.0)), float(rng.normal(0, 0.5))
            dev[c].copy_((src.float() * a + b).to(dev[c].dtype).cuda())
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        got = res.clone()
        if kind == "kv":
            ref = t.empty_like(res)
            assert _kv_state(dev, w, ref, ref_ws) == 0
        else:
            ref = t.empty_like(res)
            assert _fwd(dev, w, ref, ref_ws) == 0
        t.cuda.synchronize()
        gb = to_host(got, "f32" if kind == "kv" else w.dtype)
        rb = to_host(ref, "f32" if kind == "kv" else w.dtype)
        assert np.array_equal(gb.view(np.uint8), rb.view(np.uint8)), \
            f"{case}: replay {r} differs from the eager call on the same inputs"
