"""GPU parity of the backward pass with the ELU + 1 and cos feature maps
(sana_linattn_bwd_fmap) against the CPU float64 feature-map backward oracle,
element by element, on the same seeded bits.

Tolerance, per gradient tensor, as for the ReLU backward:

    ||got - ref||_2  <= 5e-3 * ||ref||_2  + 1e-5 * ||scale||_2
    max |got - ref|  <= 1e-2 * max |ref|  + 1e-5 * max |scale|

The first terms are the bf16 rounding of the stores (2^-9 relative). The
second cover the sums' cancellation: every factor the kernels multiply is
exact in bf16 or split into bf16 hi + lo parts (16 significant bits, a
truncation of at most 2^-17 of the terms' magnitudes), phi and phi' come
from the hardware's exp, cos and sin instructions (within 2e-6 relative and
4e-7 absolute on these inputs), and fp32 sums round at 2^-24 per step;
`scale` is every contraction taken over absolute values (phi, phi', v, g,
1 / |den|), so 1e-5 of it covers those errors. cos weights can be negative,
so its inputs are checked to keep each row's normaliser at least a third of
the sum of its terms' magnitudes, as in the forward's tests.
"""
import numpy as np
import pytest

import oracle.linattn_bwd_fmap as LBF
import relu_linear_attention_attn_amd as R
from relu_linear_attention_attn_amd import workloads as W

from gpu_util import decode, metrics, to_device, to_host, torch

pytestmark = pytest.mark.gpu

GRAD_RELL2 = 5e-3
GRAD_MAXABS_REL = 1e-2
GRAD_TERMS = 1e-5


def _phi(x, fmap):
    if fmap == "elu1":
        return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    return np.cos(x)


def _dphi(x, fmap):
    if fmap == "elu1":
        return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))
    return -np.sin(x)


def _term_scales(x, eps, fmap):
    """Per element, the magnitude of the terms each gradient sums: the
    backward's contractions with every factor replaced by its absolute value
    (the state by the sum of its terms' magnitudes)."""
    dec = {t: decode(x[t], "bf16") for t in "qkvg"}
    B, N, H, d = dec["q"].shape
    out = [np.zeros((B, N, H, d)) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            q, k, v, g = (dec[t][b, :, h] for t in "qkvg")
            pq, pk = _phi(q, fmap), _phi(k, fmap)
            aq, ak = np.abs(pq), np.abs(pk)
            S, z = ak.T @ np.abs(v), ak.sum(axis=0)
            den = np.abs(pq @ pk.sum(axis=0) + eps)
            outa = (aq @ S) / den[:, None]
            dnum = np.abs(g) / den[:, None]
            dden = (np.abs(g) * outa).sum(axis=1) / den
            out[0][b, :, h] = (dnum @ S.T + dden[:, None] * z) * np.abs(_dphi(q, fmap))
            dS, dz = aq.T @ dnum, aq.T @ dden
            out[1][b, :, h] = (np.abs(v) @ dS.T + dz) * np.abs(_dphi(k, fmap))
            out[2][b, :, h] = ak @ dS
    return out


def _cos_conditioning(x):
    q, k = decode(x["q"], "bf16"), decode(x["k"], "bf16")
    cq, ks = np.cos(q), np.cos(k).sum(axis=1, keepdims=True)
    den = (cq * ks).sum(-1)
    return float((den / (np.abs(cq) * np.abs(ks)).sum(-1)).min())


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a ROCm GPU"
    R.lib()
    yield


def _inputs(w):
    x = W.generate(w, grad=True)
    return x, {t: to_device(x[t], "bf16") for t in "qkvg"}


def _run(w, dev, fmap, g=None, events=None):
    grads = R.backward(dev["q"], dev["k"], dev["v"], dev["g"] if g is None else g, eps=w.eps,
                       fmap=fmap, events=events)
    torch().cuda.synchronize()
    return [to_host(t, "bf16") for t in grads]


def _check(got_bits, ref, x, eps, fmap, what):
    scales = _term_scales(x, eps, fmap)
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


SHAPES = [(1, 1, 1), (1, 2, 2), (2, 15, 3), (1, 16, 1), (3, 17, 5), (1, 100, 2), (2, 257, 3),
          (1, 1000, 7), (2, 4099, 4), (1, 33000, 3), (2, 1024, 36)]


@pytest.mark.parametrize("fmap", ["elu1", "cos"])
@pytest.mark.parametrize("B,N,H", SHAPES)
def test_bwd_fmap_matches_oracle(B, N, H, fmap):
    w = W.custom(f"bwdfm_{B}_{N}_{H}", B, N, H, seed=900 + N + H,
                 q=W.Dist("normal", 0.1, 1.0), k=W.Dist("normal", 0.1, 1.0))
    print(f"\n[case] bwd {fmap} B={B} N={N} H={H}", flush=True)
    x, dev = _inputs(w)
    if fmap == "cos":
        assert _cos_conditioning(x) > 0.3
    ref = LBF.linattn_bwd_fmap_from_inputs(x["q"], x["k"], x["v"], x["g"], w.eps, "bf16", fmap)
    _check(_run(w, dev, fmap), ref, x, w.eps, fmap, f"{fmap} B={B} N={N} H={H}")


def test_bwd_elu1_on_the_4096px_latent():
    """The 2 x 16384 x 70 latent in the benchmark's launch configuration (the
    state reduction's (head pair, chunk) grid), every head in full."""
    w = W.WORKLOADS["latent_4096px"]
    print(f"\n[case] bwd elu1 workload {w.name} shape {w.shape}", flush=True)
    x, dev = _inputs(w)
    got = _run(w, dev, "elu1")
    ref = LBF.linattn_bwd_fmap_from_inputs(x["q"], x["k"], x["v"], x["g"], w.eps, "bf16", "elu1")
    _check(got, ref, x, w.eps, "elu1", w.name)


def test_bwd_fmap_relu_is_the_relu_backward_bitwise():
    w = W.custom("bwdfm_relu", 2, 5000, 7, seed=91)
    x, dev = _inputs(w)
    a = _run(w, dev, "relu")
    grads = [torch().empty_like(dev["q"]) for _ in range(3)]
    ws = torch().empty(R.bwd_workspace_size(2, 5000, 7), dtype=torch().uint8, device="cuda")
    st = R.lib().sana_linattn_bwd_fmap(*[t.data_ptr() for t in (dev["q"], dev["k"], dev["v"],
                                                                dev["g"], *grads)],
                                       2, 5000, 7, 32, w.eps, 1, 0, ws.data_ptr(), ws.numel(),
                                       None, 0, torch().cuda.current_stream().cuda_stream)
    torch().cuda.synchronize()
    assert st == 0
    for s, t in zip(a, grads):
        assert np.array_equal(s, to_host(t, "bf16"))


@pytest.mark.parametrize("fmap", ["elu1", "cos"])
def test_bwd_fmap_linear_repeatable_and_events(fmap):
    """Gradients for 2 g are exactly twice those for g; repeat calls and the
    event form give the same bits."""
    w = W.custom(f"bwdfm_lin_{fmap}", 2, 3000, 6, seed=92)
    x, dev = _inputs(w)
    a = _run(w, dev, fmap)
    b = _run(w, dev, fmap, g=dev["g"] * 2)
    for s, t in zip(a, b):
        assert np.array_equal(2 * decode(s, "bf16"), decode(t, "bf16"))
    assert all(np.array_equal(s, t) for s, t in zip(a, _run(w, dev, fmap)))
    ev = [torch().cuda.Event(enable_timing=True) for _ in range(4)]
    c = _run(w, dev, fmap, events=ev)
    assert all(np.array_equal(s, t) for s, t in zip(a, c))
    assert all(ev[i].elapsed_time(ev[i + 1]) > 0 for i in range(3))


def test_bwd_fmap_rejects_unknown_map():
    w = W.custom("bwdfm_bad", 1, 64, 2, seed=93)
    x, dev = _inputs(w)
    with pytest.raises(ValueError):
        R.backward(dev["q"], dev["k"], dev["v"], dev["g"], fmap="gelu")


@pytest.mark.parametrize("fmap", ["elu1", "cos"])
@pytest.mark.parametrize("B,N,H", [(1, 1, 1), (2, 257, 3), (2, 5000, 7), (16, 1024, 70)])
def test_bwd_fmap_from_saved_state(B, N, H, fmap):
    """kv_state with the map (the folding state reduction) against the oracle's
    state, and the backward from that saved state bitwise as the recomputing
    feature-map backward."""
    import oracle.linattn_feature_maps as FM

    w = W.custom(f"bwdfm_state_{B}_{N}_{H}", B, N, H, seed=950 + N + H,
                 q=W.Dist("normal", 0.1, 1.0), k=W.Dist("normal", 0.1, 1.0))
    print(f"\n[case] bwd {fmap} from saved state B={B} N={N} H={H}", flush=True)
    x, dev = _inputs(w)
    state = R.kv_state(dev["k"], dev["v"], fmap=fmap)
    torch().cuda.synchronize()
    got = state.cpu().numpy().astype(np.float64)
    kd, vd = decode(x["k"], "bf16"), decode(x["v"], "bf16")
    for b in range(B):
        for h in range(H):
            kv, ks = FM.state_head(kd[b, :, h], vd[b, :, h], fmap)
            ref = np.concatenate([kv, ks[:, None]], axis=1)
            ak = np.abs(_phi(kd[b, :, h], fmap))
            scale = np.concatenate([ak.T @ np.abs(vd[b, :, h]), ak.sum(axis=0)[:, None]], axis=1)
            # 1e-5 of the terms (hi + lo products, fp32 sums, exp within 2e-6 relative) plus
            # 1e-6 per token of |v| (cos within 4e-7 absolute, also where cos is near 0)
            absv = np.concatenate([np.abs(vd[b, :, h]).sum(axis=0), [float(N)]])[None, :]
            err = np.abs(got[b, h] - ref)
            assert np.all(err <= 1e-5 * scale + 1e-6 * absv), (b, h, float(err.max()))
    a = _run(w, dev, fmap)
    grads = R.backward(dev["q"], dev["k"], dev["v"], dev["g"], eps=w.eps, fmap=fmap, state=state)
    torch().cuda.synchronize()
    for name, s, t in zip(("dq", "dk", "dv"), a, grads):
        assert np.array_equal(s, to_host(t, "bf16")), name
