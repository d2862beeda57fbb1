"""GPU parity of the backward pass: dq, dk, dv from the HIP path against the
CPU float64 backward oracle, element by element, on the same seeded bits.

Tolerance, per gradient tensor:

    ||got - ref||_2  <= 5e-3 * ||ref||_2  + 1e-5 * ||scale||_2
    max |got - ref|  <= 1e-2 * max |ref|  + 1e-5 * max |scale|

The first terms cover the bf16 rounding of the stores (2^-9 relative) and are
relative to the tensor's own size, since gradient scales differ by orders of
magnitude between tensors and shapes (dk and dv carry 1/den). The second
terms cover floating-point cancellation: each gradient is a sum of terms
(S dnum + z dden for dq, dS v + dz for dk, phi(k) dS for dv) that can cancel
almost exactly - with one key token out = v s / (s + eps), so dq is O(eps)
while the terms are O(1). The HIP path forms the terms with fp32 factors
split into bf16 hi + lo parts, which keep 16 significant bits, so a
contraction's truncation error is at most 2^-17 times the sum of its terms'
magnitudes (7.6e-6), plus fp32 rounding of the sums: `scale` is those
contractions taken over absolute values, computed below from the decoded
inputs, and 1e-5 covers 2^-17 with the sums' rounding.
"""
import numpy as np
import pytest

import oracle.linattn_bwd as LB
import relu_linear_attention_attn_amd as R
from relu_linear_attention_attn_amd import workloads as W

from gpu_util import decode, metrics, to_device, to_host, torch

pytestmark = pytest.mark.gpu

GRAD_RELL2 = 5e-3
GRAD_MAXABS_REL = 1e-2
GRAD_TERMS = 1e-5


def _term_scales(x, eps):
    """Per element, the magnitude of the terms each gradient sums (the
    backward's contractions with every factor replaced by its absolute
    value; dS and dz by their own term magnitudes)."""
    dec = {t: decode(x[t], "bf16") for t in "qkvg"}
    B, N, H, d = dec["q"].shape
    out = [np.zeros((B, N, H, d)) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            q, k, v, g = (dec[t][b, :, h] for t in "qkvg")
            pq, pk = np.maximum(q, 0), np.maximum(k, 0)
            S, z = pk.T @ v, pk.sum(axis=0)
            den = pq @ z + eps
            out_ = (pq @ S) / den[:, None]
            dnum = np.abs(g) / den[:, None]
            dden = np.abs((g * out_).sum(axis=1)) / den
            out[0][b, :, h] = (dnum @ np.abs(S).T + dden[:, None] * z) * (q > 0)
            dS, dz = pq.T @ dnum, pq.T @ dden
            out[1][b, :, h] = (np.abs(v) @ dS.T + dz) * (k > 0)
            out[2][b, :, h] = pk @ dS
    return out


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a ROCm GPU"
    R.lib()
    yield


def _inputs(w):
    x = W.generate(w, grad=True)
    return x, {t: to_device(x[t], "bf16") for t in "qkvg"}


def _run(w, dev, g=None):
    grads = R.backward(dev["q"], dev["k"], dev["v"], dev["g"] if g is None else g, eps=w.eps)
    torch().cuda.synchronize()
    return [to_host(t, "bf16") for t in grads]


def _check(got_bits, ref, x, eps, what):
    scales = _term_scales(x, eps)
    for name, bits, r, sc in zip(("dq", "dk", "dv"), got_bits, ref, scales):
        got = decode(bits, "bf16")
        maxabs, rel, refmax = metrics(got, r)
        err2 = float(np.linalg.norm((got - r).ravel()))
        ref2 = float(np.linalg.norm(r.ravel()))
        sc2, scmax = float(np.linalg.norm(sc.ravel())), float(np.abs(sc).max())
        msg = (f"{what} {name}: max-abs {maxabs:.3e} (max|ref| {refmax:.3e}, "
               f"max|terms| {scmax:.3e}), rel-L2 {rel:.3e} (||terms||/||ref|| "
               f"{sc2 / max(ref2, 1e-300):.2e})")
        print(msg, flush=True)
        assert np.all(np.isfinite(got)), msg + " (non-finite)"
        assert err2 <= GRAD_RELL2 * ref2 + GRAD_TERMS * sc2, msg
        assert maxabs <= GRAD_MAXABS_REL * refmax + GRAD_TERMS * scmax, msg


@pytest.mark.parametrize("name", ["sana06_1024px", "sana16_1024px_b16", "latent_4096px"])
def test_bwd_matches_oracle(name):
    w = W.WORKLOADS[name]
    print(f"\n[case] bwd workload {name} shape {w.shape}", flush=True)
    x, dev = _inputs(w)
    got = _run(w, dev)
    ref = LB.linattn_bwd_from_inputs(x["q"], x["k"], x["v"], x["g"], w.eps, "bf16")
    _check(got, ref, x, w.eps, name)


def test_bwd_video_1m_tokens_two_heads():
    """The 16 x 65,536-token video shape (B=1, N=1,048,576, H=36): the state
    reduction's (head pair, chunk) grid cuts each of the 18 head pairs into
    14 chunks here, so the q pass's chunked grid and the k/v pass's sum of
    its 14 partials per pair run at their largest. Heads 0 and 35 (the
    first and last pair) compared in full, every token."""
    w = W.WORKLOADS["video_1m_tokens"]
    print(f"\n[case] bwd workload {w.name} shape {w.shape}", flush=True)
    x, dev = _inputs(w)
    grads = R.backward(dev["q"], dev["k"], dev["v"], dev["g"], eps=w.eps)
    torch().cuda.synchronize()
    del dev
    for h in (0, w.H - 1):
        xs = {t: np.ascontiguousarray(x[t][:, :, h:h + 1]) for t in "qkvg"}
        got = [to_host(gr[:, :, h:h + 1].contiguous(), "bf16") for gr in grads]
        ref = LB.linattn_bwd_from_inputs(xs["q"], xs["k"], xs["v"], xs["g"], w.eps, "bf16")
        _check(got, ref, xs, w.eps, f"{w.name} head {h}")


RAGGED = [(1, 1, 1), (1, 2, 2), (2, 15, 3), (1, 16, 1), (3, 17, 5), (1, 100, 2), (2, 257, 3),
          (1, 1000, 7), (2, 4099, 4), (1, 33000, 3)]


@pytest.mark.parametrize("B,N,H", RAGGED)
def test_bwd_ragged_shapes(B, N, H):
    w = W.custom(f"bwd_{B}_{N}_{H}", B, N, H, seed=300 + N + H,
                 q=W.Dist("normal", 0.1, 1.0), k=W.Dist("normal", 0.1, 1.0))
    print(f"\n[case] bwd ragged B={B} N={N} H={H}", flush=True)
    x, dev = _inputs(w)
    ref = LB.linattn_bwd_from_inputs(x["q"], x["k"], x["v"], x["g"], w.eps, "bf16")
    _check(_run(w, dev), ref, x, w.eps, f"B={B} N={N} H={H}")


def test_bwd_dead_rows_are_exactly_zero():
    """All-negative q rows have dq = 0; all-negative k rows have dk = dv = 0
    (phi and its gate are 0 there), bit for bit."""
    wq = W.WORKLOADS["sana16_1024px_b16"]  # 2% of q rows all-negative
    x, dev = _inputs(wq)
    dq = decode(_run(wq, dev)[0], "bf16").reshape(wq.B * wq.N, -1)
    rows = W.masked_rows(wq)
    assert len(rows) > 0 and np.all(dq[rows] == 0)
    wk = W.WORKLOADS["sana06_1024px"]  # 5% of k rows all-negative
    x, dev = _inputs(wk)
    _, dk, dv = (decode(t, "bf16").reshape(wk.B * wk.N, -1) for t in _run(wk, dev))
    rows = W.masked_rows(wk)
    assert len(rows) > 0 and np.all(dk[rows] == 0) and np.all(dv[rows] == 0)


def test_bwd_is_linear_in_dout_bitwise():
    """Every step is linear in g and scaling by 2 is exact in floating point,
    so the gradients for 2 g are exactly twice those for g."""
    w = W.custom("bwd_lin", 2, 3000, 6, seed=41)
    x, dev = _inputs(w)
    a = _run(w, dev)
    b = _run(w, dev, g=dev["g"] * 2)
    for s, t in zip(a, b):
        assert np.array_equal(2 * decode(s, "bf16"), decode(t, "bf16"))


def test_bwd_zero_upstream_gives_zero():
    w = W.custom("bwd_zero", 1, 2000, 5, seed=42)
    x, dev = _inputs(w)
    for t in _run(w, dev, g=torch().zeros_like(dev["g"])):
        assert np.all(decode(t, "bf16") == 0)


def test_bwd_repeat_calls_are_bitwise_identical():
    w = W.custom("bwd_rep", 2, 5000, 7, seed=43)
    x, dev = _inputs(w)
    ws = torch().empty(R.bwd_workspace_size(2, 5000, 7), dtype=torch().uint8, device="cuda")
    runs = []
    for _ in range(3):
        grads = R.backward(dev["q"], dev["k"], dev["v"], dev["g"], eps=w.eps, workspace=ws)
        torch().cuda.synchronize()
        runs.append([to_host(t, "bf16") for t in grads])
    for r in runs[1:]:
        for s, t in zip(runs[0], r):
            assert np.array_equal(s, t)


def test_bwd_profiled_matches_plain():
    w = W.custom("bwd_prof", 1, 4000, 4, seed=44)
    x, dev = _inputs(w)
    a = _run(w, dev)
    ev = [torch().cuda.Event(enable_timing=True) for _ in range(4)]
    grads = R.backward(dev["q"], dev["k"], dev["v"], dev["g"], eps=w.eps, events=ev)
    torch().cuda.synchronize()
    for s, t in zip(a, grads):
        assert np.array_equal(s, to_host(t, "bf16"))
    assert all(ev[i].elapsed_time(ev[i + 1]) > 0 for i in range(3))


@pytest.mark.parametrize("B,N,H", [(1, 1, 1), (2, 257, 3), (2, 5000, 7), (1, 33000, 3),
                                   (16, 1024, 70), (2, 16384, 70)])
def test_bwd_from_saved_state_is_the_recomputing_backward_bitwise(B, N, H):
    """sana_linattn_bwd_state with the state of sana_linattn_kv_state(k, v)
    skips the state reduction and gives sana_linattn_bwd's bits: the fold
    sums the same partials in the same order as the q pass would. Shapes on
    the (head pair, chunk) grid and on balanced ranges (16 x 1024 x 70),
    odd head counts, one token; the event form records its two kernels."""
    w = W.custom(f"bwd_state_{B}_{N}_{H}", B, N, H, seed=500 + N + H,
                 q=W.Dist("normal", 0.1, 1.0), k=W.Dist("normal", 0.1, 1.0))
    print(f"\n[case] bwd from saved state B={B} N={N} H={H}", flush=True)
    x, dev = _inputs(w)
    ref = _run(w, dev)
    state = R.kv_state(dev["k"], dev["v"])
    ev = [torch().cuda.Event(enable_timing=True) for _ in range(3)]
    for events in (None, ev):
        grads = R.backward(dev["q"], dev["k"], dev["v"], dev["g"], eps=w.eps, state=state,
                           events=events)
        torch().cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), ref, grads):
            assert np.array_equal(a, to_host(b, "bf16")), (name, events is not None)
    assert all(ev[i].elapsed_time(ev[i + 1]) > 0 for i in range(2))
