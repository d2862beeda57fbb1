"""Pins of the backward oracle (oracle/linattn_bwd.py) against things other
than itself: finite differences of the forward oracle, torch float64
autograd through the explicit n x n quadratic form, and exact homogeneity /
linearity identities. A planted mistake anywhere in the backward oracle must
fail at least one pin."""
import numpy as np
import pytest

import oracle.linattn as L
import oracle.linattn_bwd as LB


def _away_from_kink(rng, shape, lo=0.1):
    """Values whose magnitude is at least lo, so a finite-difference step
    never crosses ReLU's kink at 0."""
    r = rng.standard_normal(shape)
    return np.sign(r) * (lo + np.abs(r))


def _inputs(seed, B, N, H, d=32, kink_free=True):
    rng = np.random.default_rng(seed)
    mk = (lambda s: _away_from_kink(rng, s)) if kink_free else rng.standard_normal
    q, k = mk((B, N, H, d)), mk((B, N, H, d))
    v = rng.standard_normal((B, N, H, d))
    g = rng.standard_normal((B, N, H, d))
    return q, k, v, g


def _loss(q, k, v, g, eps):
    return float((L.linattn_fp64(q, k, v, eps) * g).sum())


def _rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


# ------------------------------------------------------------------ pins


def pin_fd_elementwise():
    """Central differences of sum(g * out), every element of q, k and v."""
    eps, h = 1e-2, 1e-6
    q, k, v, g = _inputs(11, 1, 3, 2)
    grads = LB.linattn_bwd_fp64(q, k, v, g, eps)
    for t, (x, gx) in enumerate(zip((q, k, v), grads)):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[t], args_m[t] = xp, xm
            fd[idx] = (_loss(*args_p, g, eps) - _loss(*args_m, g, eps)) / (2 * h)
        err = _rel(gx, fd)
        if err > 1e-6:
            return f"tensor {'qkv'[t]}: finite differences differ by {err:.2e}"
    return None


def pin_fd_directional():
    """Central differences along random directions, larger shapes."""
    eps, h = 1e-3, 1e-6
    for seed, (B, N, H) in ((12, (2, 17, 3)), (13, (1, 64, 2)), (14, (1, 1, 2))):
        q, k, v, g = _inputs(seed, B, N, H)
        grads = LB.linattn_bwd_fp64(q, k, v, g, eps)
        rng = np.random.default_rng(seed + 100)
        for t in range(3):
            u = rng.standard_normal(q.shape)
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[t] = args_p[t] + h * u
            args_m[t] = args_m[t] - h * u
            fd = (_loss(*args_p, g, eps) - _loss(*args_m, g, eps)) / (2 * h)
            an = float((grads[t] * u).sum())
            if abs(fd - an) > 1e-6 * max(1.0, abs(fd)):
                return f"shape {(B, N, H)} tensor {'qkv'[t]}: {an} vs finite difference {fd}"
    return None


def pin_autograd_quadratic():
    """torch float64 autograd through out = (W V) / (W 1 + eps), W = phi(Q) phi(K)^T
    (the n x n form), with exact zeros and negatives in q and k."""
    torch = pytest.importorskip("torch")
    eps = 1e-2
    q, k, v, g = _inputs(15, 2, 40, 2, kink_free=False)
    q[0, 3, 1, :5] = 0.0  # exact zeros: the derivative there is 0 (reading)
    k[1, 7, 0, 10:20] = 0.0
    q[1, 5, 0, :] = -np.abs(q[1, 5, 0, :])  # a dead query row
    k[0, 9, 1, :] = -np.abs(k[0, 9, 1, :])  # a dead key token
    want = LB.linattn_bwd_fp64(q, k, v, g, eps)
    B, N, H, d = q.shape
    for b in range(B):
        for hh in range(H):
            tq, tk, tv = (torch.tensor(x[b, :, hh], dtype=torch.float64, requires_grad=True)
                          for x in (q, k, v))
            w = torch.relu(tq) @ torch.relu(tk).T
            out = (w @ tv) / (w.sum(dim=1, keepdim=True) + eps)
            (out * torch.tensor(g[b, :, hh])).sum().backward()
            for name, t, ref in zip("qkv", (tq, tk, tv), want):
                err = _rel(ref[b, :, hh], t.grad.numpy())
                if err > 1e-10:
                    return f"d{name} (b={b}, h={hh}) differs from autograd by {err:.2e}"
    return None


def pin_homogeneity():
    """Exact identities (eps large, so they are not trivial):
    sum_c q_ic dq_ic = (g_i . out_i) eps / den_i for every row i;
    sum_{n,c} k_nc dk_nc = sum_i (g_i . out_i) eps / den_i per head;
    sum_{n,c} v_nc dv_nc = sum_i g_i . out_i per head."""
    eps = 0.7
    q, k, v, g = _inputs(16, 2, 33, 3, kink_free=False)
    dq, dk, dv = LB.linattn_bwd_fp64(q, k, v, g, eps)
    B, N, H, d = q.shape
    for b in range(B):
        for h in range(H):
            kv, ksum = L.kv_state(k[b, :, h], v[b, :, h])
            pq = L.phi(q[b, :, h])
            den = pq @ ksum + eps
            out = (pq @ kv) / den[:, None]
            go = (g[b, :, h] * out).sum(axis=1)
            lhs_q = (q[b, :, h] * dq[b, :, h]).sum(axis=1)
            if _rel(lhs_q, go * eps / den) > 1e-11:
                return f"q homogeneity fails at b={b} h={h}"
            lhs_k = float((k[b, :, h] * dk[b, :, h]).sum())
            rhs_k = float((go * eps / den).sum())
            if abs(lhs_k - rhs_k) > 1e-10 * max(1.0, abs(rhs_k)):
                return f"k homogeneity fails at b={b} h={h}: {lhs_k} vs {rhs_k}"
            lhs_v = float((v[b, :, h] * dv[b, :, h]).sum())
            if abs(lhs_v - go.sum()) > 1e-10 * max(1.0, abs(go.sum())):
                return f"v linearity fails at b={b} h={h}"
    return None


def pin_dead_rows():
    """A query row with phi(q_i) = 0 has dq_i = 0 and its g_i reaches no other
    gradient; a key token with phi(k_n) = 0 has dk_n = 0 and dv_n = 0."""
    eps = 1e-3
    q, k, v, g = _inputs(17, 1, 20, 2, kink_free=False)
    q[0, 4] = -np.abs(q[0, 4])
    k[0, 6] = -np.abs(k[0, 6])
    dq, dk, dv = LB.linattn_bwd_fp64(q, k, v, g, eps)
    if np.any(dq[0, 4] != 0) or np.any(dk[0, 6] != 0) or np.any(dv[0, 6] != 0):
        return "dead rows have nonzero gradients"
    g2 = g.copy()
    g2[0, 4] = 5.0 * np.random.default_rng(3).standard_normal(g2[0, 4].shape)
    _, dk2, dv2 = LB.linattn_bwd_fp64(q, k, v, g2, eps)
    if _rel(dk2, dk) > 1e-14 or _rel(dv2, dv) > 1e-14:
        return "a dead query row's upstream gradient changed dk or dv"
    return None


def pin_state_grad():
    """state_grad_head equals the derivative of sum(g * out) with respect to
    the state, by central differences on the state itself."""
    eps, h = 1e-2, 1e-6
    q, k, v, g = _inputs(18, 1, 9, 1)
    kv, ksum = L.kv_state(k[0, :, 0], v[0, :, 0])
    got = LB.state_grad_head(q[0, :, 0], g[0, :, 0], kv, ksum, eps)
    st = np.concatenate([kv, ksum[:, None]], axis=1)

    def loss(s):
        return float((L.apply_state(q[0, :, 0], s[:, :-1], s[:, -1], eps) * g[0, :, 0]).sum())

    fd = np.empty_like(st)
    for idx in np.ndindex(st.shape):
        sp, sm = st.copy(), st.copy()
        sp[idx] += h
        sm[idx] -= h
        fd[idx] = (loss(sp) - loss(sm)) / (2 * h)
    err = _rel(got, fd)
    return None if err < 1e-6 else f"state gradient differs from finite differences by {err:.2e}"


PINS = [pin_fd_elementwise, pin_fd_directional, pin_autograd_quadratic, pin_homogeneity,
        pin_dead_rows, pin_state_grad]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin_holds(pin):
    msg = pin()
    assert msg is None, msg


# --------------------------------------------------- planted mistakes


def _mut_output_grads(kind):
    def f(g, num, den):
        dnum = g / den[:, None]
        dden = -(g * num).sum(axis=1) / (den * den)
        if kind == "no_dden":
            dden = np.zeros_like(dden)
        elif kind == "dden_sign":
            dden = -dden
        elif kind == "dden_one_den":
            dden = dden * den
        elif kind == "dnum_times_den":
            dnum = g * den[:, None]
        return dnum, dden
    return f


def _mut_phi_q_grad(kind):
    def f(dnum, dden, kv, ksum):
        if kind == "no_transpose":
            return dnum @ kv + dden[:, None] * ksum[None, :]
        if kind == "no_ksum":
            return dnum @ kv.T
        raise AssertionError(kind)
    return f


def _mut_state_grads(kind):
    def f(pq, dnum, dden):
        if kind == "transposed":
            return dnum.T @ pq, pq.T @ dden
        if kind == "dksum_from_dnum":
            return pq.T @ dnum, pq.T @ dnum.sum(axis=1)
        if kind == "raw_q":
            return pq.T @ dnum, -pq.T @ dden
        raise AssertionError(kind)
    return f


def _mut_phi_k_grad(kind):
    def f(v, dkv, dksum):
        if kind == "no_transpose":
            return v @ dkv + dksum[None, :]
        if kind == "no_dksum":
            return v @ dkv.T
        raise AssertionError(kind)
    return f


def _mut_v_grad(kind):
    def f(pk, dkv):
        if kind == "transposed":
            return pk @ dkv.T
        if kind == "plus_ksum":
            return pk @ dkv + pk.sum(axis=1, keepdims=True)
        raise AssertionError(kind)
    return f


def _mut_driver(kind):
    def f(q, k, v, g, eps):
        B, N, H, d = q.shape
        dq, dk, dv = (np.empty((B, N, H, d)) for _ in range(3))
        for b in range(B):
            for h in range(H):
                hg = (h + 1) % H if kind == "g_wrong_head" else h
                dq[b, :, h], dk[b, :, h], dv[b, :, h] = LB.backward_head(
                    q[b, :, h], k[b, :, h], v[b, :, h], g[b, :, hg], eps)
        if kind == "dk_dv_swapped":
            dk, dv = dv, dk
        return dq, dk, dv
    return f


MUTANTS = {
    "mask_ge": ("relu_mask", lambda x: (x >= 0).astype(np.float64)),
    "no_mask": ("relu_mask", lambda x: np.ones_like(x)),
    "phi_abs": ("phi", np.abs),
    "no_dden": ("output_grads", _mut_output_grads("no_dden")),
    "dden_sign": ("output_grads", _mut_output_grads("dden_sign")),
    "dden_one_den": ("output_grads", _mut_output_grads("dden_one_den")),
    "dnum_times_den": ("output_grads", _mut_output_grads("dnum_times_den")),
    "phi_q_grad_no_transpose": ("phi_q_grad", _mut_phi_q_grad("no_transpose")),
    "phi_q_grad_no_ksum": ("phi_q_grad", _mut_phi_q_grad("no_ksum")),
    "state_grads_transposed": ("state_grads", _mut_state_grads("transposed")),
    "dksum_from_dnum": ("state_grads", _mut_state_grads("dksum_from_dnum")),
    "dksum_sign": ("state_grads", _mut_state_grads("raw_q")),
    "phi_k_grad_no_transpose": ("phi_k_grad", _mut_phi_k_grad("no_transpose")),
    "phi_k_grad_no_dksum": ("phi_k_grad", _mut_phi_k_grad("no_dksum")),
    "v_grad_transposed": ("v_grad", _mut_v_grad("transposed")),
    "v_grad_plus_ksum": ("v_grad", _mut_v_grad("plus_ksum")),
    "g_wrong_head": ("linattn_bwd_fp64", _mut_driver("g_wrong_head")),
    "dk_dv_swapped": ("linattn_bwd_fp64", _mut_driver("dk_dv_swapped")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(LB, attr, fn)
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
    """The bits-level driver decodes bf16 and matches the float64 driver."""
    from relu_linear_attention_attn_amd import workloads as W

    w = W.custom("bwd_drv", 2, 50, 3, dtype="bf16", seed=9)
    x = W.generate(w)
    rng = np.random.default_rng(4)
    g = W.f32_to_bf16_bits(rng.standard_normal(x["q"].shape).astype(np.float32))
    a = LB.linattn_bwd_from_inputs(x["q"], x["k"], x["v"], g, w.eps, "bf16")
    dec = [L.bf16_bits_to_f64(t) for t in (x["q"], x["k"], x["v"], g)]
    b = LB.linattn_bwd_fp64(*dec, w.eps)
    for s, t in zip(a, b):
        assert np.array_equal(s, t)
