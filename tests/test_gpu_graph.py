"""The library's launches captured in a HIP graph and replayed.

A captured launch keeps the arguments it was captured with, among them the
per-call tag of the control words through which the last block of a head
pair folds the pair's partials (the fp32 reduction and sana_linattn_kv_state).
Each case captures one call through the C ABI, then replays the graph four
times; before each replay the inputs are overwritten with new values (eager
work on the same stream, then a device synchronisation), and every replay's
outputs must equal, bit for bit, an eager call on the same inputs with a
workspace of its own (same kernels, grids and summation order). The eager
results are themselves checked against the oracle by the parity tests."""
import ctypes

import numpy as np
import pytest

import relu_linear_attention_attn_amd as R

from gpu_util import torch

REPLAYS = 4
BF16, F32 = R.DTYPE_BF16, R.DTYPE_F32


def _stream():
    return torch().cuda.current_stream().cuda_stream


def _size(fn, *args):
    n = ctypes.c_size_t(0)
    assert fn(*args, ctypes.byref(n)) == 0
    return max(n.value, 256)


def _p(x):
    return x.data_ptr()


class Case:
    """One entry point: the tensors it reads (rewritten before each replay),
    the tensors it writes (compared), its workspace size and the call."""

    def __init__(self, inputs, outputs, ws_bytes, call):
        self.inputs, self.outputs, self.ws_bytes, self.call = inputs, outputs, ws_bytes, call


def _fwd_case(B, N, H, dt, noalloc=False, variant=None):
    lib = R.lib()
    shape = (B, N, H, 32)
    ws = _size(lib.sana_linattn_workspace_size, B, N, H, 32, dt)

    def call(t, ws_t):
        ptrs = (_p(t["q"]), _p(t["k"]), _p(t["v"]), _p(t["out"]), B, N, H, 32, 1e-6, dt)
        if noalloc:
            return lib.sana_linattn_fwd_noalloc(*ptrs, _stream())
        if variant is not None:
            return lib.sana_linattn_fwd_variant(*ptrs, variant, _p(ws_t), ws_t.numel(), _stream())
        return lib.sana_linattn_fwd(*ptrs, _p(ws_t), ws_t.numel(), _stream())
    return Case({c: (shape, dt) for c in "qkv"}, {"out": (shape, dt)}, ws, call)


def _kv_case(B, N, H, dt):
    lib = R.lib()
    shape = (B, N, H, 32)
    ws = _size(lib.sana_linattn_workspace_size, B, N, H, 32, dt)

    def call(t, ws_t):
        return lib.sana_linattn_kv_state(_p(t["k"]), _p(t["v"]), _p(t["state"]), B, N, H, 32, dt,
                                         _p(ws_t), ws_t.numel(), _stream())
    return Case({c: (shape, dt) for c in "kv"}, {"state": ((B, H, 32, 33), F32)}, ws, call)


def _bwd_case(B, N, H):
    lib = R.lib()
    shape = (B, N, H, 32)
    ws = _size(lib.sana_linattn_bwd_workspace_size, B, N, H, 32, BF16)

    def call(t, ws_t):
        return lib.sana_linattn_bwd(_p(t["q"]), _p(t["k"]), _p(t["v"]), _p(t["g"]), _p(t["dq"]),
                                    _p(t["dk"]), _p(t["dv"]), B, N, H, 32, 1e-6, BF16, _p(ws_t),
                                    ws_t.numel(), _stream())
    return Case({c: (shape, BF16) for c in "qkvg"}, {c: (shape, BF16) for c in ("dq", "dk", "dv")},
                ws, call)


def _bwd_fmap_case(B, N, H, fmap):
    lib = R.lib()
    shape = (B, N, H, 32)
    ws = _size(lib.sana_linattn_bwd_workspace_size, B, N, H, 32, BF16)

    def call(t, ws_t):
        return lib.sana_linattn_bwd_fmap(_p(t["q"]), _p(t["k"]), _p(t["v"]), _p(t["g"]),
                                         _p(t["dq"]), _p(t["dk"]), _p(t["dv"]), B, N, H, 32, 1e-6,
                                         BF16, fmap, _p(ws_t), ws_t.numel(), None, 0, _stream())
    return Case({c: (shape, BF16) for c in "qkvg"}, {c: (shape, BF16) for c in ("dq", "dk", "dv")},
                ws, call)


def _bwd_state_case(B, N, H):
    lib = R.lib()
    shape = (B, N, H, 32)
    ws = _size(lib.sana_linattn_bwd_workspace_size, B, N, H, 32, BF16)

    def call(t, ws_t):
        return lib.sana_linattn_bwd_state(_p(t["q"]), _p(t["k"]), _p(t["v"]), _p(t["g"]),
                                          _p(t["s"]), _p(t["dq"]), _p(t["dk"]), _p(t["dv"]), B, N,
                                          H, 32, 1e-6, BF16, 0, _p(ws_t), ws_t.numel(), None, 0,
                                          _stream())
    inputs = {c: (shape, BF16) for c in "qkvg"}
    inputs["s"] = ((B, H, 32, 33), F32)  # a state; replays only need it fixed per replay
    return Case(inputs, {c: (shape, BF16) for c in ("dq", "dk", "dv")}, ws, call)


def _block_causal_case(B, N, H, L, dt):
    lib = R.lib()
    shape = (B, N, H, 32)
    ws = _size(lib.sana_linattn_block_causal_workspace_size, B, N, H, 32, L, dt)

    def call(t, ws_t):
        return lib.sana_linattn_fwd_block_causal(_p(t["q"]), _p(t["k"]), _p(t["v"]), _p(t["out"]),
                                                 B, N, H, 32, L, 1e-6, dt, _p(ws_t), ws_t.numel(),
                                                 _stream())
    return Case({c: (shape, dt) for c in "qkv"}, {"out": (shape, dt)}, ws, call)


def _causal_case(B, N, H):
    lib = R.lib()
    shape = (B, N, H, 32)
    ws = _size(lib.sana_linattn_causal_workspace_size, B, N, H, 32, BF16)

    def call(t, ws_t):
        return lib.sana_linattn_fwd_causal(_p(t["q"]), _p(t["k"]), _p(t["v"]), _p(t["out"]), B, N,
                                           H, 32, 1e-6, BF16, _p(ws_t), ws_t.numel(), None, 0,
                                           _stream())
    return Case({c: (shape, BF16) for c in "qkv"}, {"out": (shape, BF16)}, ws, call)


def _qkv_case(B, N, C, H):
    lib = R.lib()
    D = H * 32
    ws = _size(lib.sana_linattn_qkv_workspace_size, B, N, C, H, 32)

    def call(t, ws_t):
        return lib.sana_linattn_qkv_fwd(_p(t["x"]), _p(t["w"]), _p(t["q"]), _p(t["out"]), B, N, C,
                                        H, 32, 1e-6, _p(ws_t), ws_t.numel(), None, 0, _stream())
    return Case({"x": ((B, N, C), BF16), "w": ((3 * D, C), BF16)},
                {"q": ((B, N, H, 32), BF16), "out": ((B, N, H, 32), BF16)}, ws, call)


CASES = {
    # fp32 beyond the fused range: the reduction folds, then the apply
    "fwd_f32_split": lambda: _fwd_case(2, 3000, 5, F32),
    "noalloc_f32_split": lambda: _fwd_case(1, 4100, 6, F32, noalloc=True),
    # bf16 state alone: the bf16 reduction with the fold
    "kv_state_bf16": lambda: _kv_case(2, 5000, 7, BF16),
    # bf16 split forward (partials straight to the apply) and fused
    "fwd_bf16_split": lambda: _fwd_case(1, 8192, 6, BF16),
    "fwd_bf16_fused": lambda: _fwd_case(2, 700, 9, BF16, variant=R.VARIANT_FUSED),
    "bwd_bf16": lambda: _bwd_case(1, 3000, 5),
    # the backward with ELU + 1 (the feature-map instantiations of the same passes)
    "bwd_bf16_elu1": lambda: _bwd_fmap_case(1, 3000, 5, 1),
    # the backward from a saved state: the q pass and the k/v pass
    "bwd_bf16_state": lambda: _bwd_state_case(2, 3000, 5),
    # fp32 block-causal: the folding reduction over blocks, the scan, the apply
    "block_causal_f32": lambda: _block_causal_case(2, 2048, 3, 512, F32),
    "qkv_bf16": lambda: _qkv_case(1, 700, 200, 5),
    # token-causal: chunk states, their prefix scan, the chunk-wise apply
    "causal_bf16": lambda: _causal_case(2, 3000, 5),
    # bf16 blocks of 4 tokens: the block-causal entry point on the token-causal kernels
    "block_causal_bf16_small_blocks": lambda: _block_causal_case(1, 2048, 5, 4, BF16),
    # bf16 blocks of 4 tiles: the block-wise chunked apply
    "block_causal_bf16_tile_blocks": lambda: _block_causal_case(2, 2048, 5, 64, BF16),
}


def _fill(x, dtype, rng, scale=1.0):
    """Seeded values (bf16 from fp32 draws) written into tensor x in place."""
    t = torch()
    a = rng.standard_normal(x.numel()).astype(np.float32) * np.float32(scale)
    src = t.from_numpy(a).reshape(x.shape).cuda()
    x.copy_(src.to(x.dtype))


@pytest.mark.gpu
@pytest.mark.parametrize("case", sorted(CASES))
def test_graph_replays_match_eager_calls(case):
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a ROCm GPU"
    print(f"\n[case] graph {case}", flush=True)
    c = CASES[case]()
    tdt = {BF16: t.bfloat16, F32: t.float32}
    rng = np.random.default_rng(2000 + sorted(CASES).index(case))
    scale = {"w": 1.0 / np.sqrt(200.0)}

    def alloc(spec):
        return {n: t.empty(shape, dtype=tdt[dt], device="cuda") for n, (shape, dt) in spec.items()}

    ten = alloc(c.inputs)
    ten.update(alloc(c.outputs))
    for n in c.inputs:
        _fill(ten[n], c.inputs[n][1], rng, scale.get(n, 1.0))
    ws = t.empty(c.ws_bytes, dtype=t.uint8, device="cuda")
    assert c.call(ten, ws) == 0  # eager first: one-time device look-ups outside the capture
    t.cuda.synchronize()

    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        status = c.call(ten, ws)
    assert status == 0

    ref = {n: v for n, v in ten.items() if n in c.inputs}
    ref.update(alloc(c.outputs))
    ref_ws = t.empty(c.ws_bytes, dtype=t.uint8, device="cuda")
    for r in range(REPLAYS):
        for n in c.inputs:
            _fill(ten[n], c.inputs[n][1], rng, scale.get(n, 1.0) * float(rng.uniform(0.5, 2.0)))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        got = {n: ten[n].clone() for n in c.outputs}
        assert c.call(ref, ref_ws) == 0
        t.cuda.synchronize()
        for n in c.outputs:
            a = got[n].view(t.uint8).cpu().numpy()
            b = ref[n].view(t.uint8).cpu().numpy()
            assert np.array_equal(a, b), f"{case}: replay {r} output {n} differs from the eager call"
