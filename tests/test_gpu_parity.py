"""GPU parity: the HIP path against the CPU float64 oracle, element by element,
through the C ABI (ctypes binding), on the same seeded input bits.

Tolerances: bf16 max-abs <= 1e-2 and rel-L2 <= 5e-3; fp32 rel-L2 <= 1e-5 and
max-abs <= 1e-5 * max|ref|. The bf16 output is rounded once from fp32 (a
half-ulp is 2^-9 relative, about 1.1e-3 in rel-L2 for uniform rounding
errors), the fp32 state sum and the hi/lo-split products add less than
1e-5, and max-abs 1e-2 holds while |out| < 4 (the half-ulp is 0.0078 in
[2, 4)), which convex averages of N(0, 1) values keep. fp32 products and sums
round at 2^-24 per operation over at most 2 * 32 + log2 N terms.
"""
import numpy as np
import pytest

import oracle.linattn as L
import relu_linear_attention_attn_amd as R
from relu_linear_attention_attn_amd import workloads as W

from gpu_util import assert_close, decode, metrics, to_device, to_host, torch

pytestmark = pytest.mark.gpu

VARIANTS = {"auto": R.VARIANT_AUTO, "split": R.VARIANT_SPLIT, "fused": R.VARIANT_FUSED}


def variants(dtype):
    """Variants that support dtype (all of them, for both dtypes)."""
    return dict(VARIANTS)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a ROCm GPU"
    R.lib()  # loud failure if the HIP library is missing
    yield


def _inputs(w):
    x = W.generate(w)
    return x, {t: to_device(x[t], w.dtype) for t in "qkv"}


def _run(w, dev, variant=R.VARIANT_AUTO):
    out = R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps, variant=variant)
    torch().cuda.synchronize()
    return decode(to_host(out, w.dtype), w.dtype)


def _oracle(w, x):
    return L.linattn_from_inputs(x["q"], x["k"], x["v"], w.eps, w.dtype)


# ------------------------------------------------------- named workloads

SMALL = ["tiny_f32", "sana06_1024px", "sana16_1024px_b16", "latent_4096px"]


@pytest.mark.parametrize("name", SMALL)
def test_workload_matches_oracle_all_variants(name):
    w = W.WORKLOADS[name]
    print(f"\n[case] workload {name} shape {w.shape} {w.dtype}", flush=True)
    x, dev = _inputs(w)
    ref = _oracle(w, x)
    for vname, var in variants(w.dtype).items():
        got = _run(w, dev, var)
        assert_close(got, ref, w.dtype, f"{name}/{vname}")


def test_tiny_f32_matches_quadratic_form():
    """The fp32 workload is small enough for the explicit n x n form too."""
    w = W.WORKLOADS["tiny_f32"]
    x, dev = _inputs(w)
    f = {t: decode(x[t], "f32") for t in "qkv"}
    ref = L.quadratic_fp64(f["q"], f["k"], f["v"], w.eps)
    assert_close(_run(w, dev), ref, "f32", "tiny_f32 vs quadratic form")


# ----------------------------------------------------------- ragged cases

RAGGED = [
    (1, 1, 1), (1, 2, 2), (2, 15, 3), (1, 16, 1), (3, 17, 5), (1, 100, 2), (2, 257, 3),
    (1, 1000, 7), (2, 4099, 4), (1, 33000, 3),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,N,H", RAGGED)
def test_ragged_shapes(B, N, H, dtype):
    w = W.custom(f"ragged_{B}_{N}_{H}", B, N, H, dtype=dtype, seed=100 + N + H,
                 q=W.Dist("normal", 0.1, 1.0), k=W.Dist("normal", 0.1, 1.0))
    print(f"\n[case] ragged B={B} N={N} H={H} {dtype}", flush=True)
    x, dev = _inputs(w)
    ref = _oracle(w, x)
    for vname, var in variants(dtype).items():
        assert_close(_run(w, dev, var), ref, dtype, f"B={B} N={N} H={H} {dtype} {vname}")


# ------------------------------------- fused kernel at two units per CU


@pytest.mark.parametrize("B,N,H", [(16, 1000, 65), (32, 77, 33), (40, 300, 27), (16, 1024, 64),
                                   (8, 1000, 65), (9, 300, 57), (8, 1024, 64), (4, 1024, 70),
                                   (600, 1, 2), (300, 17, 3)])
def test_fused_block_shapes(B, N, H):
    """The fused kernel's block shape follows the head-pair units per CU
    (MI355X: 256 CUs): 4-wave blocks with one tile in flight from 512 units,
    8-wave blocks with one tile from 256, with two below. Ragged token counts,
    odd head counts (a one-head last pair) and unit counts of exactly 512 and
    256 against the oracle, sequences shorter than a block's waves (N = 1,
    N = 17 over 600 units), and repeat calls bit for bit."""
    w = W.custom(f"fused_{B}_{N}_{H}", B, N, H, seed=300 + N + H,
                 q=W.Dist("normal", 0.1, 1.0), k=W.Dist("normal", 0.1, 1.0))
    print(f"\n[case] fused block shape B={B} N={N} H={H}", flush=True)
    x, dev = _inputs(w)
    ref = _oracle(w, x)
    first = _run(w, dev, R.VARIANT_FUSED)
    assert_close(first, ref, "bf16", f"fused B={B} N={N} H={H}")
    assert np.array_equal(first, _run(w, dev, R.VARIANT_FUSED)), "repeat differs"
    assert_close(_run(w, dev, R.VARIANT_AUTO), ref, "bf16", f"AUTO B={B} N={N} H={H}")


# --------------------------------------------- AUTO's choice by shape


def test_auto_variant_by_shape():
    """AUTO runs the split pair for N > 1024 and for few head pairs at
    N in (512, 1024]; the fused kernel for a tiny call, for N <= 512 and for
    at least CUs / 2 head pairs at N = 1024 (256 CUs on MI355X); each result
    matches the oracle."""
    t = torch()
    for (B, N, H, want) in ((2, 1024, 36, 2), (1, 64, 2, 1), (1, 2048, 4, 2),
                            (16, 1024, 70, 1), (9, 1000, 57, 1), (2, 700, 125, 2),
                            (2, 512, 72, 1)):
        w = W.custom(f"arr_{B}_{N}_{H}", B, N, H, seed=7 + H)
        print(f"\n[case] AUTO B={B} N={N} H={H}", flush=True)
        x, dev = _inputs(w)
        events = [t.cuda.Event(enable_timing=True) for _ in range(3)]
        out, nk = R.forward_profiled(dev["q"], dev["k"], dev["v"], events, eps=w.eps)
        t.cuda.synchronize()
        assert nk == want, (B, N, H, nk)
        assert_close(decode(to_host(out, "bf16"), "bf16"), _oracle(w, x), "bf16",
                     f"AUTO B={B} N={N} H={H}")


# ------------------------------------------------------ state and apply halves


@pytest.mark.parametrize("name", ["sana06_1024px", "latent_4096px"])
def test_kv_state_matches_oracle(name):
    w = W.WORKLOADS[name]
    print(f"\n[case] kv_state {name}", flush=True)
    x, dev = _inputs(w)
    st = R.kv_state(dev["k"], dev["v"])
    torch().cuda.synchronize()
    got = st.cpu().numpy().astype(np.float64)
    ref = L.state_from_inputs(x["k"], x["v"], w.dtype)
    maxabs, rel, refmax = metrics(got, ref)
    print(f"state rel-L2 {rel:.3e} max-abs {maxabs:.3e} max|ref| {refmax:.3e}", flush=True)
    # bf16 x bf16 products are exact in fp32; only the fp32 sums round
    assert rel <= 2e-6 * max(1.0, np.sqrt(w.N / 1024)), rel


def test_apply_from_oracle_state():
    """The apply kernel alone, fed the oracle's state rounded to fp32."""
    w = W.WORKLOADS["sana16_1024px_b16"]
    x, dev = _inputs(w)
    st64 = L.state_from_inputs(x["k"], x["v"], w.dtype)
    st = torch().from_numpy(st64.astype(np.float32)).cuda()
    out = R.apply(dev["q"], st, eps=w.eps)
    torch().cuda.synchronize()
    got = decode(to_host(out, w.dtype), w.dtype)
    # reference from the same fp32-rounded state
    ref = np.empty_like(got)
    st32 = st64.astype(np.float32).astype(np.float64)
    for b in range(w.B):
        ref[b] = L.apply_rows(decode(x["q"][b], w.dtype), st32[b], w.eps)
    assert_close(got, ref, w.dtype, "apply from oracle state")


def test_state_is_additive_over_token_ranges():
    """States of two token halves, summed, equal the state of the whole."""
    w = W.custom("additive", 2, 5000, 6, seed=77)
    x, dev = _inputs(w)
    whole = R.kv_state(dev["k"], dev["v"])
    a = R.kv_state(dev["k"][:, :2000].contiguous(), dev["v"][:, :2000].contiguous())
    b = R.kv_state(dev["k"][:, 2000:].contiguous(), dev["v"][:, 2000:].contiguous())
    torch().cuda.synchronize()
    _, rel, _ = metrics((a + b).cpu().numpy().astype(np.float64),
                        whole.cpu().numpy().astype(np.float64))
    assert rel < 1e-6, rel


# ------------------------------------------------------------- invariants


def test_dead_query_rows_are_exactly_zero():
    """Workload sana16_1024px_b16 makes 2% of Q rows all-negative: phi(q) = 0,
    so those output rows must be exactly 0 (num = 0, den + eps = eps)."""
    w = W.WORKLOADS["sana16_1024px_b16"]
    x, dev = _inputs(w)
    rows = W.masked_rows(w)
    for vname, var in VARIANTS.items():
        out = to_host(R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps, variant=var), "bf16")
        flat = out.reshape(w.B * w.N, -1)
        assert np.all((flat[rows] & 0x7FFF) == 0), vname   # +0 or -0
        live = np.setdiff1d(np.arange(w.B * w.N), rows)[:500]
        assert np.all(np.any((flat[live] & 0x7FFF) != 0, axis=1)), vname


def test_dead_key_tokens_do_not_matter_bitwise():
    """Workload sana06_1024px makes 5% of K rows all-negative: phi(k) = 0, so
    replacing their V rows leaves the output bitwise unchanged."""
    w = W.WORKLOADS["sana06_1024px"]
    x, dev = _inputs(w)
    rows = W.masked_rows(w)
    v2 = x["v"].reshape(w.B * w.N, -1).copy()
    rng = np.random.default_rng(9)
    v2[rows] = W.f32_to_bf16_bits(rng.standard_normal((len(rows), w.D)).astype(np.float32) * 7)
    dv2 = to_device(v2.reshape(w.shape), "bf16")
    for vname, var in VARIANTS.items():
        a = to_host(R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps, variant=var), "bf16")
        b = to_host(R.forward(dev["q"], dev["k"], dv2, eps=w.eps, variant=var), "bf16")
        assert np.array_equal(a, b), vname


@pytest.mark.parametrize("name", ["sana06_1024px", "latent_4096px"])
def test_repeat_calls_are_bitwise_identical(name):
    w = W.WORKLOADS[name]
    x, dev = _inputs(w)
    for vname, var in variants(w.dtype).items():
        a = to_host(R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps, variant=var), w.dtype)
        for _ in range(3):
            b = to_host(R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps, variant=var), w.dtype)
            assert np.array_equal(a, b), vname


def _ordered(u):
    """bf16 bits as sign-magnitude integers: adjacent bf16 values differ by 1."""
    u = u.astype(np.int32)
    return np.where(u & 0x8000, -(u & 0x7FFF), u)


@pytest.mark.parametrize("name", ["sana06_1024px", "latent_4096px"])
@pytest.mark.parametrize("scaled", ["k", "q"])
def test_scaling_by_two_changes_at_most_one_ulp(name, scaled):
    """phi(2x) = 2 phi(x) and doubling is exact in bf16 and fp32. Doubling K
    doubles the state exactly; doubling Q doubles both the numerator and the
    denominator's dot product exactly. Either way the output moves only
    through eps, i.e. by at most one bf16 rounding step, in every variant."""
    w = W.WORKLOADS[name]
    x, dev = _inputs(w)
    two = dict(dev)
    two[scaled] = dev[scaled] * 2
    for vname, var in VARIANTS.items():
        a = to_host(R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps, variant=var), "bf16")
        b = to_host(R.forward(two["q"], two["k"], two["v"], eps=w.eps, variant=var), "bf16")
        assert np.max(np.abs(_ordered(a) - _ordered(b))) <= 1, vname


def test_convex_combination_bound():
    w = W.WORKLOADS["sana06_1024px"]
    x, dev = _inputs(w)
    got = _run(w, dev)
    v = decode(x["v"], "bf16")
    lo = np.minimum(v.min(axis=1, keepdims=True), 0)
    hi = np.maximum(v.max(axis=1, keepdims=True), 0)
    ulp = 2.0 ** -7 * np.maximum(np.abs(got), 2.0 ** -126)  # one bf16 ulp
    assert np.all(got >= lo - ulp) and np.all(got <= hi + ulp)


def test_output_canaries_untouched():
    """Bytes just before and after `out` keep their values."""
    t = torch()
    w = W.custom("canary", 2, 1000, 3, seed=5)
    x, dev = _inputs(w)
    n = w.B * w.N * w.H * w.d
    pad = 4096
    for vname, var in VARIANTS.items():
        buf = t.full((n + 2 * pad,), 12345, dtype=t.int16, device="cuda")
        out = buf[pad:pad + n].view(t.bfloat16).view(w.shape)
        R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps, out=out, variant=var)
        t.cuda.synchronize()
        host = buf.cpu().numpy()
        assert np.all(host[:pad] == 12345) and np.all(host[pad + n:] == 12345), vname


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_workspace_canaries_untouched(dtype):
    """The forward pass and the state reduction write only inside the
    workspace they are given: the bytes just before and after it keep their
    values (the workspace is the exact queried size)."""
    t = torch()
    w = W.custom("ws_canary", 2, 3000, 5, dtype=dtype, seed=6)
    x, dev = _inputs(w)
    dt = R.DTYPE_BF16 if dtype == "bf16" else R.DTYPE_F32
    size = R.workspace_size(w.B, w.N, w.H, dtype=dt)
    pad = 4096
    buf = t.full((size + 2 * pad,), 0xA5, dtype=t.uint8, device="cuda")
    ws = buf[pad:pad + size]
    for vname, var in VARIANTS.items():
        R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps, variant=var, workspace=ws)
    R.kv_state(dev["k"], dev["v"], workspace=ws)
    t.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:pad] == 0xA5) and np.all(host[pad + size:] == 0xA5)


def test_heads_given_as_flat_width():
    """(B, N, D) tensors with heads= are the same memory as (B, N, H, d)."""
    w = W.WORKLOADS["sana06_1024px"]
    x, dev = _inputs(w)
    a = to_host(R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps), "bf16")
    flat = {k: t.view(w.B, w.N, w.D) for k, t in dev.items()}
    b = to_host(R.forward(flat["q"], flat["k"], flat["v"], eps=w.eps, heads=w.H), "bf16")
    assert np.array_equal(a.reshape(-1), b.reshape(-1))


def test_split_equals_kv_state_then_apply_bitwise():
    """The bf16 split forward sums the reduction's partials inside the apply;
    kv_state folds the same partials, in the same order, at the end of the
    reduction. Both routes must give the same bits."""
    for w in (W.WORKLOADS["latent_4096px"], W.custom("odd", 3, 5001, 7, seed=31)):
        x, dev = _inputs(w)
        a = to_host(R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps, variant=R.VARIANT_SPLIT),
                    "bf16")
        st = R.kv_state(dev["k"], dev["v"])
        b = to_host(R.apply(dev["q"], st, eps=w.eps), "bf16")
        assert np.array_equal(a, b), w.name


def test_one_workspace_across_calls_and_shapes():
    """One workspace serves forward and kv_state calls of different shapes in
    turn: stale partials and control words from earlier calls never leak
    into a later result (each call is equal to one on a fresh workspace)."""
    t = torch()
    wa = W.custom("sa", 2, 3000, 6, seed=21)
    wb = W.custom("sb", 1, 5000, 5, seed=22)
    xa, da = _inputs(wa)
    xb, db = _inputs(wb)
    size = max(R.workspace_size(2, 3000, 6), R.workspace_size(1, 5000, 5))
    ws = t.full((size,), 0x7f, dtype=t.uint8, device="cuda")
    ra = to_host(R.forward(da["q"], da["k"], da["v"], variant=R.VARIANT_SPLIT), "bf16")
    rb = to_host(R.forward(db["q"], db["k"], db["v"], variant=R.VARIANT_SPLIT), "bf16")
    sa = R.kv_state(da["k"], da["v"]).cpu().numpy()
    for i in range(4):
        oa = R.forward(da["q"], da["k"], da["v"], workspace=ws, variant=R.VARIANT_SPLIT)
        gs = R.kv_state(da["k"], da["v"], workspace=ws)
        ob = R.forward(db["q"], db["k"], db["v"], workspace=ws, variant=R.VARIANT_SPLIT)
        assert np.array_equal(to_host(oa, "bf16"), ra), f"A call {i}"
        assert np.array_equal(to_host(ob, "bf16"), rb), f"B call {i}"
        assert np.array_equal(gs.cpu().numpy(), sa), f"state call {i}"


def test_errors_enqueue_nothing():
    t = torch()
    w = W.custom("err", 1, 64, 2, seed=1)
    x, dev = _inputs(w)
    out = t.full_like(dev["q"], 3.0)
    L_ = R.lib()
    ws = t.empty(R.workspace_size(1, 64, 2), dtype=t.uint8, device="cuda")
    q, k, v = (dev[c].data_ptr() for c in "qkv")
    st = t.cuda.current_stream().cuda_stream
    assert L_.sana_linattn_fwd(q, k, v, out.data_ptr(), 1, 64, 2, 32, -1.0, 1, ws.data_ptr(),
                               ws.numel(), st) == 1
    assert L_.sana_linattn_fwd(q, k, v, out.data_ptr(), 1, 64, 2, 32, 1e-6, 1, ws.data_ptr(),
                               16, st) == 3
    assert L_.sana_linattn_fwd(q + 2, k, v, out.data_ptr(), 1, 64, 2, 32, 1e-6, 1,
                               ws.data_ptr(), ws.numel(), st) == 4
    t.cuda.synchronize()
    assert bool((out == 3.0).all())


# ------------------------------------------------------------ 1M tokens

def _chunk_edges(N: int, units: int, cus: int = 256):
    """Token offsets where the split kernels' chunks start on this shape, by
    the library's rule for a (head pair, chunk) grid on `cus` one-block-per-CU
    slots: c = slots // units chunks (one round that fills at least 3/4 of the
    slots), each a whole number of 16-token tiles, an even count made odd."""
    c = max(1, cus // units)
    assert 4 * units * c >= 3 * cus, "shape outside the one-round rule"
    tiles = -(-(-(-N // c)) // 16)
    if tiles > 1 and tiles % 2 == 0:
        tiles += 1
    chunk = 16 * tiles
    return list(range(chunk, N, chunk)), chunk


@pytest.mark.timeout(900)
def test_video_1m_tokens():
    """B=1, N=1,048,576, H=36, t(4) heavy-tailed Q and K: heads 0 and 35 (the
    first and last) compared with the oracle on all 1,048,576 rows, element
    by element; every head on sampled rows that include the first and last
    rows and both sides of every chunk boundary of the reduction and the
    apply; and the whole state against the oracle's."""
    w = W.WORKLOADS["video_1m_tokens"]
    x, dev = {}, {}
    for t in "qkv":
        print(f"\n[case] {w.name}: generating {t}", flush=True)
        x[t] = W.generate_tensor(w, t)
        dev[t] = to_device(x[t], "bf16")
    print("[case] running the HIP path", flush=True)
    out = R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps)
    st = R.kv_state(dev["k"], dev["v"])
    torch().cuda.synchronize()
    edges, chunk = _chunk_edges(w.N, w.B * ((w.H + 1) // 2))
    assert chunk == 74928 and len(edges) == 13   # 14 chunks on 256 CUs
    print(f"[case] chunk {chunk} tokens, {len(edges) + 1} chunks", flush=True)
    ref_state = L.state_from_inputs(x["k"], x["v"], "bf16")
    _, srel, _ = metrics(st.cpu().numpy().astype(np.float64), ref_state)
    print(f"state rel-L2 {srel:.3e}", flush=True)
    assert srel < 1e-4
    for h in (0, w.H - 1):
        print(f"[case] head {h}: all {w.N} rows", flush=True)
        got = decode(to_host(out[0, :, h], "bf16"), "bf16")
        ref = L.apply_state(decode(x["q"][0, :, h], "bf16"), ref_state[0, h, :, :w.d],
                            ref_state[0, h, :, w.d], w.eps)
        assert_close(got, ref, "bf16", f"video_1m_tokens head {h}, all rows")
    rng = np.random.default_rng(2024)
    rows = np.unique(np.concatenate([rng.choice(w.N, 4096, replace=False),
                                     [0, 1, 15, 16, 17, w.N - 17, w.N - 1],
                                     *[[e - 1, e, e + 1] for e in edges]]))
    got = decode(to_host(out[0, rows], "bf16"), "bf16")
    ref = L.apply_rows(decode(x["q"][0, rows], "bf16"), ref_state[0], w.eps)
    assert_close(got, ref, "bf16", "video_1m_tokens sampled rows, every head")
