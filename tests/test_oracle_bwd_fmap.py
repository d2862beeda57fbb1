"""Pins of the feature-map backward oracle (oracle/linattn_bwd_fmap.py)
against things other than itself: central finite differences of the
feature-map forward oracle's loss, torch float64 autograd through a torch
form of the forward definition, and the ReLU backward oracle. A planted
mistake anywhere in the module must fail at least one pin."""
import numpy as np
import pytest

import oracle.linattn_bwd as LB
import oracle.linattn_bwd_fmap as BF
import oracle.linattn_feature_maps as FM

MAPS = ("relu", "elu1", "cos")


def _inputs(seed, B, N, H, d=32, scale=0.8):
    """q, k away from 0 (ReLU's kink) by at least 0.1, scaled so cos stays
    positive enough that den is far from 0; v and g standard normal."""
    rng = np.random.default_rng(seed)

    def away(shape):
        r = rng.standard_normal(shape)
        return scale * np.sign(r) * (0.1 + np.abs(r))

    q, k = away((B, N, H, d)), away((B, N, H, d))
    v = rng.standard_normal((B, N, H, d))
    g = rng.standard_normal((B, N, H, d))
    return q, k, v, g


def _loss(q, k, v, g, eps, fmap):
    return float((FM.linattn_fmap_fp64(q, k, v, eps, fmap) * g).sum())


def _rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def pin_fd_elementwise():
    """Central differences of sum(g * out), every element of q, k and v."""
    eps, h = 1e-2, 1e-6
    for fmap in MAPS:
        q, k, v, g = _inputs(31, 1, 3, 2, d=6)
        grads = BF.linattn_bwd_fmap_fp64(q, k, v, g, eps, fmap)
        for t, (x, gx) in enumerate(zip((q, k, v), grads)):
            fd = np.empty_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p, args_m = [q, k, v], [q, k, v]
                args_p[t], args_m[t] = xp, xm
                fd[idx] = (_loss(*args_p, g, eps, fmap) - _loss(*args_m, g, eps, fmap)) / (2 * h)
            err = _rel(gx, fd)
            if err > 1e-6:
                return f"{fmap} tensor {'qkv'[t]}: finite differences differ by {err:.2e}"
    return None


def pin_fd_directional():
    """Central differences along random directions, d = 32, several shapes."""
    eps, h = 1e-3, 1e-6
    for fmap in MAPS:
        for seed, (B, N, H) in ((32, (2, 17, 3)), (33, (1, 40, 2)), (34, (1, 1, 2))):
            q, k, v, g = _inputs(seed, B, N, H)
            grads = BF.linattn_bwd_fmap_fp64(q, k, v, g, eps, fmap)
            rng = np.random.default_rng(seed + 100)
            for t in range(3):
                u = rng.standard_normal(q.shape)
                args_p, args_m = [q, k, v], [q, k, v]
                args_p[t] = args_p[t] + h * u
                args_m[t] = args_m[t] - h * u
                fd = (_loss(*args_p, g, eps, fmap) - _loss(*args_m, g, eps, fmap)) / (2 * h)
                an = float((grads[t] * u).sum())
                if abs(fd - an) > 1e-6 * max(1.0, abs(fd)):
                    return f"{fmap} shape {(B, N, H)} tensor {'qkv'[t]}: {an} vs {fd}"
    return None


def pin_torch_autograd():
    """torch float64 autograd through the forward definition written with
    torch operations (the map, the state, the normalised product)."""
    torch = pytest.importorskip("torch")
    eps = 1e-3
    maps = {"relu": torch.relu, "elu1": lambda x: torch.nn.functional.elu(x) + 1.0,
            "cos": torch.cos}
    for fmap in MAPS:
        q, k, v, g = _inputs(35, 2, 23, 3)
        tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
        phi = maps[fmap]
        pq, pk = phi(tq), phi(tk)
        kv = torch.einsum("bnhc,bnhj->bhcj", pk, tv)
        z = pk.sum(dim=1)
        num = torch.einsum("bnhc,bhcj->bnhj", pq, kv)
        den = torch.einsum("bnhc,bhc->bnh", pq, z) + eps
        out = num / den[..., None]
        (out * torch.tensor(g)).sum().backward()
        grads = BF.linattn_bwd_fmap_fp64(q, k, v, g, eps, fmap)
        for t, x in enumerate((tq, tk, tv)):
            err = _rel(grads[t], x.grad.numpy())
            if err > 1e-10:
                return f"{fmap} tensor {'qkv'[t]}: autograd differs by {err:.2e}"
    return None


def pin_relu_is_the_relu_backward():
    eps = 1e-6
    q, k, v, g = _inputs(36, 2, 50, 3)
    a = BF.linattn_bwd_fmap_fp64(q, k, v, g, eps, "relu")
    b = LB.linattn_bwd_fp64(q, k, v, g, eps)
    for t in range(3):
        if _rel(a[t], b[t]) > 1e-13:
            return f"relu tensor {'qkv'[t]} differs from the ReLU backward oracle"
    return None


PINS = [pin_fd_elementwise, pin_fd_directional, pin_torch_autograd,
        pin_relu_is_the_relu_backward]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin_holds(pin):
    msg = pin()
    assert msg is None, msg


def _mut_backward(kind):
    def backward_head_fmap(q, k, v, g, eps, fmap):
        phi, dphi = FM.feature_map(fmap), BF.derivative(fmap)
        pq, pk = phi(q), phi(k)
        kv = pk.T @ v
        ksum = pk.sum(axis=0)
        num = pq @ kv
        den = pq @ ksum + eps
        dnum, dden = LB.output_grads(g, num, den)
        dq = LB.phi_q_grad(dnum, dden, kv, ksum)
        if kind != "dq_ungated":
            dq = dq * dphi(q)
        dkv, dksum = LB.state_grads(pq, dnum, dden)
        dk = LB.phi_k_grad(v, dkv, dksum) * (dphi(q) if kind == "dk_gated_by_q" else dphi(k))
        dv = LB.v_grad(pk if kind != "dv_from_k" else k, dkv)
        return dq, dk, dv
    return backward_head_fmap


MUTANTS = {
    "elu1_derivative_one": ("dphi_elu1", lambda x: np.ones_like(x)),
    "elu1_derivative_shifted": ("dphi_elu1", lambda x: np.where(x > 0, 1.0, np.exp(x) + 1.0)),
    "cos_derivative_sign": ("dphi_cos", lambda x: np.sin(x)),
    "cos_derivative_cos": ("dphi_cos", lambda x: -np.cos(x)),
    "relu_derivative_at_all": ("dphi_relu", lambda x: np.ones_like(x)),
    "dq_ungated": ("backward_head_fmap", _mut_backward("dq_ungated")),
    "dk_gated_by_q": ("backward_head_fmap", _mut_backward("dk_gated_by_q")),
    "dv_from_k": ("backward_head_fmap", _mut_backward("dv_from_k")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(BF, attr, fn)
    if attr.startswith("dphi_"):
        monkeypatch.setitem(BF.DERIVATIVES, attr[len("dphi_"):], fn)
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                msg = pin()
            except Exception as e:  # a crash is a caught mistake too
                msg = f"raised {type(e).__name__}"
            if msg is not None:
                failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"


def test_drivers_agree():
    from relu_linear_attention_attn_amd import workloads as W

    w = W.custom("bwdf_drv", 2, 40, 3, dtype="bf16", seed=19)
    x = W.generate(w, grad=True)
    for fmap in MAPS:
        a = BF.linattn_bwd_fmap_from_inputs(x["q"], x["k"], x["v"], x["g"], w.eps, "bf16", fmap)
        dec = [LB.to_f64(x[t], "bf16") for t in "qkvg"]
        b = BF.linattn_bwd_fmap_fp64(*dec, w.eps, fmap)
        assert all(np.array_equal(s, t) for s, t in zip(a, b))
