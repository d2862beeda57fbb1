"""Pins for the CPU float64 oracle.

Nothing here re-types the oracle's own formula. Each pin checks the oracle
against something fixed independently: exact rational arithmetic on the
unreordered definition, the explicit n x n form, closed forms, or an
invariant of the mathematics. ``test_planted_mistakes_are_caught`` then plants
plausible mistakes in the oracle and checks that some pin fails for each.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle.linattn as L
from relu_linear_attention_attn_amd import workloads as W

RNG = np.random.default_rng(20240601)


def _rand(shape, rng=RNG, scale=1.0, shift=0.0):
    return rng.standard_normal(shape) * scale + shift


def _rel(a, b):
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


# ------------------------------------------------------------------ pins
# Every pin takes no argument, calls L.linattn_fp64 at call time (so planted
# mistakes are seen) and returns None when it holds, else a message.


def pin_exact_rational():
    """Unreordered definition in exact rational arithmetic on dyadic inputs:
    out_i = sum_j w_ij v_j / (sum_j w_ij + eps), w_ij = phi(q_i).phi(k_j)."""
    rng = np.random.default_rng(7)
    for (B, N, H, d) in [(1, 1, 1, 3), (2, 3, 2, 4), (1, 5, 3, 5), (2, 4, 1, 8)]:
        q, k, v = (rng.integers(-16, 17, size=(B, N, H, d)) / 8.0 for _ in range(3))
        eps = 0.25
        got = L.linattn_fp64(q, k, v, eps)
        fe = Fraction(eps)
        relu = lambda x: max(Fraction(x), Fraction(0))  # noqa: E731
        for b in range(B):
            for h in range(H):
                for i in range(N):
                    w = [sum(relu(q[b, i, h, c]) * relu(k[b, j, h, c]) for c in range(d))
                         for j in range(N)]
                    den = sum(w) + fe
                    for c in range(d):
                        exact = sum(w[j] * Fraction(v[b, j, h, c]) for j in range(N)) / den
                        if abs(got[b, i, h, c] - float(exact)) > 1e-14 * max(1.0, abs(float(exact))):
                            return f"exact mismatch at {(b, i, h, c)}: {got[b, i, h, c]} vs {float(exact)}"
    return None


def pin_quadratic_form():
    """Linear form equals the explicit n x n form phi(Q)phi(K)^T, row-normalised,
    times V (associativity), on the tiny fp32 workload and random tiny shapes."""
    w = W.WORKLOADS["tiny_f32"]
    x = {t: W.generate_tensor(w, t).astype(np.float64) for t in "qkv"}
    cases = [(x["q"], x["k"], x["v"], w.eps)]
    rng = np.random.default_rng(3)
    for n in (1, 2, 3, 17, 64):
        cases.append(tuple(_rand((2, n, 3, 32), rng) for _ in range(3)) + (1e-6,))
    for q, k, v, eps in cases:
        a = L.linattn_fp64(q, k, v, eps)
        b = _quadratic_loops(q, k, v, eps)
        if not np.all(np.isfinite(a)) or _rel(a, b) > 1e-12:
            return f"linear vs quadratic form rel error {_rel(a, b):.3g} at n={q.shape[1]}"
    return None


def _quadratic_loops(q, k, v, eps):
    """n x n weights built by an explicit loop over key tokens (test-local)."""
    B, N, H, d = q.shape
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            pq = np.where(q[b, :, h, :] > 0, q[b, :, h, :], 0.0)
            pk = np.where(k[b, :, h, :] > 0, k[b, :, h, :], 0.0)
            wts = np.zeros((N, N))
            for j in range(N):
                wts[:, j] = (pq * pk[j]).sum(axis=1)
            out[b, :, h, :] = (wts @ v[b, :, h, :]) / (wts.sum(axis=1) + eps)[:, None]
    return out


def _exact_rational_out(q, k, v, eps, b, h, i, c):
    """out[b, i, h, c] of the unreordered definition in exact rational arithmetic."""
    relu = lambda x: max(Fraction(x), Fraction(0))  # noqa: E731
    N, d = q.shape[1], q.shape[3]
    w = [sum(relu(q[b, i, h, e]) * relu(k[b, j, h, e]) for e in range(d)) for j in range(N)]
    return sum(w[j] * Fraction(v[b, j, h, c]) for j in range(N)) / (sum(w) + Fraction(eps))


def pin_quadratic_exact_rational():
    """The explicit n x n form (oracle.linattn.quadratic_fp64) against exact
    rational arithmetic on dyadic inputs; the shapes have n >= 2 and q != k, so
    a transposed weight matrix or a row sum over the key axis changes values."""
    rng = np.random.default_rng(11)
    for (B, N, H, d) in [(1, 2, 1, 3), (2, 3, 2, 4), (1, 5, 3, 5), (1, 7, 1, 8)]:
        q, k, v = (rng.integers(-16, 17, size=(B, N, H, d)) / 8.0 for _ in range(3))
        eps = 0.25
        got = L.quadratic_fp64(q, k, v, eps)
        for b in range(B):
            for h in range(H):
                for i in range(N):
                    for c in range(d):
                        exact = float(_exact_rational_out(q, k, v, eps, b, h, i, c))
                        if abs(got[b, i, h, c] - exact) > 1e-14 * max(1.0, abs(exact)):
                            return (f"quadratic form mismatch at {(b, i, h, c)}: "
                                    f"{got[b, i, h, c]} vs {exact}")
    return None


def pin_quadratic_matches_loops():
    """quadratic_fp64 against the n x n weights built by a loop over key tokens
    (_quadratic_loops), on the tiny fp32 workload and random shapes; with a
    single key token it reduces to v s / (s + eps); dead query rows give 0."""
    w = W.WORKLOADS["tiny_f32"]
    x = {t: W.generate_tensor(w, t).astype(np.float64) for t in "qkv"}
    cases = [(x["q"], x["k"], x["v"], w.eps)]
    rng = np.random.default_rng(13)
    for n in (1, 2, 3, 17, 64):
        cases.append(tuple(_rand((2, n, 3, 32), rng) for _ in range(3)) + (1e-3,))
    for q, k, v, eps in cases:
        a = L.quadratic_fp64(q, k, v, eps)
        b = _quadratic_loops(q, k, v, eps)
        if not np.all(np.isfinite(a)) or _rel(a, b) > 1e-12:
            return f"quadratic form vs loop form rel error {_rel(a, b):.3g} at n={q.shape[1]}"
    d = 32
    q = np.full((1, 1, 1, d), -1.0)
    k = np.full((1, 1, 1, d), -1.0)
    q[0, 0, 0, 3], k[0, 0, 0, 3] = 0.5, 1.0   # s = 0.5 = eps: out = v / 2
    v = _rand((1, 1, 1, d))
    if not np.allclose(L.quadratic_fp64(q, k, v, 0.5), v / 2, rtol=1e-15, atol=0):
        return "quadratic form: N = 1 closed form v s / (s + eps) violated"
    q, k, v = (_rand((1, 20, 2, 32)) for _ in range(3))
    q[:, ::4] = -np.abs(q[:, ::4])
    got = L.quadratic_fp64(q, k, v, 1e-6)
    if np.any(got[:, ::4] != 0) or np.any(np.all(got[:, 1::4] == 0, axis=-1)):
        return "quadratic form: dead query rows not exactly zero (or live rows zero)"
    return None


def pin_single_token():
    """N = 1: out = v * s / (s + eps), s = phi(q).phi(k). Chosen with s = eps so
    that the eps placement matters: out = v / 2."""
    d = 32
    q = np.full((1, 1, 1, d), -1.0)
    k = np.full((1, 1, 1, d), -1.0)
    q[0, 0, 0, 3] = 0.5
    k[0, 0, 0, 3] = 1.0       # s = 0.5
    q[0, 0, 0, 4] = 2.0       # phi(k) is 0 on channel 4: contributes nothing
    v = _rand((1, 1, 1, d))
    got = L.linattn_fp64(q, k, v, 0.5)
    if not np.allclose(got, v / 2, rtol=1e-15, atol=0):
        return "N=1 closed form v*s/(s+eps) violated"
    return None


def pin_constant_inputs():
    """Q = K = 1: out_i = mean_n(v_n) * N d / (N d + eps) for every i."""
    for (N, d, eps) in [(7, 32, 1e-6), (100, 32, 3.0), (5, 4, 0.5)]:
        q = np.ones((1, N, 2, d))
        v = _rand((1, N, 2, d))
        got = L.linattn_fp64(q, q.copy(), v, eps)
        want = v.mean(axis=1, keepdims=True) * (N * d) / (N * d + eps)
        if _rel(got, np.broadcast_to(want, got.shape)) > 1e-14:
            return f"constant-input closed form violated (N={N}, d={d})"
    return None


def pin_one_hot_query():
    """phi(q_i) = e_c: out_i = sum_n phi(k_nc) v_n / (sum_n phi(k_nc) + eps), a
    weighted column mean."""
    N, d, eps = 50, 32, 1e-3
    k = _rand((1, N, 1, d))
    v = _rand((1, N, 1, d))
    q = -np.abs(_rand((1, N, 1, d)))
    for c in range(d):
        q[0, c, 0, c] = 1.0
    got = L.linattn_fp64(q, k, v, eps)
    wk = np.maximum(k[0, :, 0, :], 0)
    for c in range(d):
        want = (wk[:, c:c + 1] * v[0, :, 0, :]).sum(axis=0) / (wk[:, c].sum() + eps)
        if not np.allclose(got[0, c, 0], want, rtol=1e-12, atol=1e-15):
            return f"one-hot query closed form violated on channel {c}"
    return None


def pin_convex_bound():
    """Weights phi(q).phi(k) >= 0: each output column lies in
    [min(0, min_n v), max(0, max_n v)] of its head."""
    q, k, v = (_rand((2, 300, 3, 32), shift=0.1) for _ in range(3))
    got = L.linattn_fp64(q, k, v, 1e-6)
    lo = np.minimum(v.min(axis=1, keepdims=True), 0)
    hi = np.maximum(v.max(axis=1, keepdims=True), 0)
    tol = 1e-12
    if np.any(got < lo - tol) or np.any(got > hi + tol):
        return "output leaves the convex hull of V's columns"
    # and an output that is not a mere copy of V: a strict average
    if np.allclose(got[:, :1], v[:, :1]):
        return "output equals V rows (weights look like the identity)"
    return None


def pin_positive_scaling():
    """phi(cx) = c phi(x) for c > 0: scaling K (or Q) by 2 changes the output only
    through eps, by far less than 1e-9 relative when den >> eps."""
    q, k, v = (_rand((1, 200, 2, 32), shift=0.1) for _ in range(3))
    base = L.linattn_fp64(q, k, v, 1e-6)
    for name, args in (("K", (q, 2 * k, v)), ("Q", (2 * q, k, v))):
        got = L.linattn_fp64(*args, 1e-6)
        if _rel(got, base) > 1e-9:
            return f"scaling {name} by 2 changed the output"
    # scaling V scales the output exactly
    if _rel(L.linattn_fp64(q, k, 2 * v, 1e-6), 2 * base) > 1e-15:
        return "scaling V by 2 did not scale the output"
    return None


def pin_dead_query_rows():
    """phi(q_i) = 0 gives num = 0 and den + eps = eps: out_i = 0 exactly."""
    q, k, v = (_rand((2, 64, 2, 32)) for _ in range(3))
    q[:, ::5] = -np.abs(q[:, ::5])
    got = L.linattn_fp64(q, k, v, 1e-6)
    if np.any(got[:, ::5] != 0):
        return "dead query rows not exactly zero"
    if np.any(np.all(got[:, 1::5] == 0, axis=-1)):
        return "live query rows came out zero"
    return None


def pin_dead_key_tokens():
    """phi(k_n) = 0: token n contributes nothing, so its V row is irrelevant."""
    q, k, v = (_rand((1, 80, 2, 32)) for _ in range(3))
    k[:, 10:30] = -np.abs(k[:, 10:30])
    a = L.linattn_fp64(q, k, v, 1e-6)
    v2 = v.copy()
    v2[:, 10:30] = 1e6 * _rand(v2[:, 10:30].shape)
    b = L.linattn_fp64(q, k, v2, 1e-6)
    if _rel(a, b) > 1e-13:
        return "V rows of dead key tokens changed the output"
    k2 = k.copy()
    k2[:, 10:30] = 0.0
    if _rel(L.linattn_fp64(q, k2, v, 1e-6), a) > 1e-15:
        return "dead key tokens are not equivalent to zero keys"
    return None


def pin_permutation():
    """Jointly permuting (K, V) rows leaves the output unchanged; permuting Q rows
    permutes output rows."""
    q, k, v = (_rand((2, 90, 2, 32)) for _ in range(3))
    a = L.linattn_fp64(q, k, v, 1e-6)
    p = np.random.default_rng(5).permutation(90)
    if _rel(L.linattn_fp64(q, k[:, p], v[:, p], 1e-6), a) > 1e-13:
        return "permuting key/value tokens changed the output"
    if _rel(L.linattn_fp64(q[:, p], k, v, 1e-6), a[:, p]) > 1e-13:
        return "permuting queries did not permute the output"
    return None


def pin_linearity_in_v():
    """out(a V1 + b V2) = a out(V1) + b out(V2)."""
    q, k, v1, v2 = (_rand((1, 70, 2, 32)) for _ in range(4))
    lhs = L.linattn_fp64(q, k, 0.75 * v1 - 2.5 * v2, 1e-6)
    rhs = 0.75 * L.linattn_fp64(q, k, v1, 1e-6) - 2.5 * L.linattn_fp64(q, k, v2, 1e-6)
    if _rel(lhs, rhs) > 1e-13:
        return "output is not linear in V"
    return None


def pin_independence():
    """Heads and batch items do not interact; every head differs from a
    head-summed or batch-summed state."""
    q, k, v = (_rand((3, 40, 4, 32), shift=0.2) for _ in range(3))
    a = L.linattn_fp64(q, k, v, 1e-6)
    k2, v2 = k.copy(), v.copy()
    k2[1] += 3.0
    v2[1] *= -2.0
    k2[:, :, 2] += 1.0
    v2[:, :, 2] *= 5.0
    b = L.linattn_fp64(q, k2, v2, 1e-6)
    same = np.ones((3, 4), bool)
    same[1, :] = False
    same[:, 2] = False
    for bi in range(3):
        for h in range(4):
            eq = np.array_equal(a[bi, :, h], b[bi, :, h])
            if same[bi, h] and not eq:
                return f"(b={bi}, h={h}) changed when another head/batch did"
            if not same[bi, h] and eq:
                return f"(b={bi}, h={h}) did not change with its own inputs"
    return None


def pin_eps_zero_dead_row():
    """eps = 0 and phi(q_i) = 0: 0/0 is NaN (the documented eps rule)."""
    q, k, v = (_rand((1, 8, 1, 32)) for _ in range(3))
    q[0, 0] = -np.abs(q[0, 0])
    with np.errstate(invalid="ignore", divide="ignore"):
        got = L.linattn_fp64(q, k, v, 0.0)
    if not np.all(np.isnan(got[0, 0])) or not np.all(np.isfinite(got[0, 1:])):
        return "eps = 0 rule violated"
    return None


PINS = [
    pin_exact_rational, pin_quadratic_form, pin_quadratic_exact_rational,
    pin_quadratic_matches_loops, pin_single_token, pin_constant_inputs,
    pin_one_hot_query, pin_convex_bound, pin_positive_scaling, pin_dead_query_rows,
    pin_dead_key_tokens, pin_permutation, pin_linearity_in_v, pin_independence,
    pin_eps_zero_dead_row,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin_holds(pin):
    assert pin() is None


# ------------------------------------------------------ planted mistakes


def _mut_kv_state(kind):
    def kv_state(k, v):
        pk = L.phi(k)
        if kind == "k_no_relu":
            pk = k
        if kind == "drop_last_token":
            pk, v = pk[:-1], v[:-1]
        kv = pk.T @ v
        if kind == "kv_transposed":
            kv = kv.T
        ksum = pk.sum(axis=0)
        if kind == "ksum_from_v":
            ksum = v.sum(axis=0)
        if kind == "ksum_sign":
            ksum = -ksum
        return kv, ksum
    return kv_state


def _mut_apply_state(kind):
    def apply_state(q, kv, ksum, eps):
        pq = q if kind == "q_no_relu" else L.phi(q)
        num = pq @ kv
        den = pq @ ksum
        if kind == "no_normaliser":
            return num
        if kind == "eps_as_max":
            return num / np.maximum(den, eps)[:, None]
        if kind == "eps_in_numerator":
            return (num + eps) / (den + eps)[:, None]
        if kind == "wrong_parenthesis":
            return num / den[:, None] + eps
        if kind == "den_from_q_only":
            return num / (pq.sum(axis=1) + eps)[:, None]
        if kind == "normalise_by_column":
            return num / (num.sum(axis=0, keepdims=True) + eps)
        return num / (den + eps)[:, None]
    return apply_state


def _mut_forward(kind):
    def linattn_fp64(q, k, v, eps):
        B, N, H, d = q.shape
        out = np.empty((B, N, H, d))
        for b in range(B):
            for h in range(H):
                hk = (h + 1) % H if kind == "wrong_head" else h
                if kind == "batch_mixed":
                    kk = k[:, :, h, :].reshape(-1, d)
                    vv = v[:, :, h, :].reshape(-1, d)
                else:
                    kk, vv = k[b, :, hk, :], v[b, :, hk, :]
                kv, ksum = L.kv_state(kk, vv)
                qq = q[b, :, h, :]
                if kind == "q_k_swapped":
                    kv, ksum = L.kv_state(qq, vv)
                    qq = k[b, :, h, :]
                out[b, :, h, :] = L.apply_state(qq, kv, ksum, eps)
        return out
    return linattn_fp64


def _mut_quadratic(kind):
    def quadratic_fp64(q, k, v, eps):
        B, N, H, d = q.shape
        out = np.empty((B, N, H, d))
        for b in range(B):
            for h in range(H):
                pk = k[b, :, h, :] if kind == "quad_k_no_relu" else L.phi(k[b, :, h, :])
                w = L.phi(q[b, :, h, :]) @ pk.T
                if kind == "quad_w_transposed":
                    w = w.T
                r = w.sum(axis=0) if kind == "quad_rowsum_axis0" else w.sum(axis=1)
                den = r if kind == "quad_eps_dropped" else r + eps
                num = w @ v[b, :, h, :]
                if kind == "quad_v_from_q":
                    num = w @ q[b, :, h, :]
                out[b, :, h, :] = num / den[:, None]
        return out
    return quadratic_fp64


MUTANTS = {
    "phi_identity": ("phi", lambda x: np.asarray(x, dtype=np.float64)),
    "phi_abs": ("phi", np.abs),
    "phi_leaky": ("phi", lambda x: np.where(x > 0, x, 0.01 * x)),
    "k_no_relu": ("kv_state", _mut_kv_state("k_no_relu")),
    "drop_last_token": ("kv_state", _mut_kv_state("drop_last_token")),
    "kv_transposed": ("kv_state", _mut_kv_state("kv_transposed")),
    "ksum_from_v": ("kv_state", _mut_kv_state("ksum_from_v")),
    "ksum_sign": ("kv_state", _mut_kv_state("ksum_sign")),
    "q_no_relu": ("apply_state", _mut_apply_state("q_no_relu")),
    "no_normaliser": ("apply_state", _mut_apply_state("no_normaliser")),
    "eps_as_max": ("apply_state", _mut_apply_state("eps_as_max")),
    "eps_in_numerator": ("apply_state", _mut_apply_state("eps_in_numerator")),
    "wrong_parenthesis": ("apply_state", _mut_apply_state("wrong_parenthesis")),
    "den_from_q_only": ("apply_state", _mut_apply_state("den_from_q_only")),
    "normalise_by_column": ("apply_state", _mut_apply_state("normalise_by_column")),
    "wrong_head": ("linattn_fp64", _mut_forward("wrong_head")),
    "batch_mixed": ("linattn_fp64", _mut_forward("batch_mixed")),
    "q_k_swapped": ("linattn_fp64", _mut_forward("q_k_swapped")),
    "quad_eps_dropped": ("quadratic_fp64", _mut_quadratic("quad_eps_dropped")),
    "quad_w_transposed": ("quadratic_fp64", _mut_quadratic("quad_w_transposed")),
    "quad_rowsum_axis0": ("quadratic_fp64", _mut_quadratic("quad_rowsum_axis0")),
    "quad_k_no_relu": ("quadratic_fp64", _mut_quadratic("quad_k_no_relu")),
    "quad_v_from_q": ("quadratic_fp64", _mut_quadratic("quad_v_from_q")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(L, attr, fn)
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


# ---------------------------------------------------- decoding and state


def test_bf16_decode_known_bits():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4000, 0xC040, 0x0001, 0x7F7F,
                     0x3E80, 0x4049], dtype=np.uint16)
    want = [0.0, -0.0, 1.0, -1.0, 2.0, -3.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127,
            0.25, 3.140625]
    got = L.bf16_bits_to_f64(bits)
    assert list(got) == want
    assert np.signbit(got[1])


def test_bf16_decode_matches_torch():
    torch = pytest.importorskip("torch")
    bits = np.random.default_rng(1).integers(0, 1 << 16, size=100000, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite values
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(L.bf16_bits_to_f64(bits), t)


def test_state_is_augmented_contraction():
    """state[..., :d] = sum_n phi(k_n) v_n^T and state[..., d] = sum_n phi(k_n),
    accumulated here token by token."""
    k, v = _rand((2, 33, 3, 32)), _rand((2, 33, 3, 32))
    st = L.state_fp64(k, v)
    want = np.zeros_like(st)
    for n in range(33):
        pk = np.maximum(k[:, n], 0)
        want[..., :32] += pk[..., :, None] * v[:, n][..., None, :]
        want[..., 32] += pk
    assert _rel(st, want) < 1e-14


def test_state_size_independent_of_n():
    k, v = _rand((1, 10, 1, 32)), _rand((1, 10, 1, 32))
    k2, v2 = _rand((1, 1000, 1, 32)), _rand((1, 1000, 1, 32))
    assert L.state_fp64(k, v).shape == L.state_fp64(k2, v2).shape == (1, 1, 32, 33)


def test_drivers_agree():
    w = W.custom("drv", 2, 300, 3, dtype="bf16", seed=4)
    x = W.generate(w)
    f = {t: L.to_f64(x[t], "bf16") for t in "qkv"}
    full = L.linattn_fp64(f["q"], f["k"], f["v"], 1e-6)
    assert np.array_equal(L.linattn_from_inputs(x["q"], x["k"], x["v"], 1e-6, "bf16"), full)
    st = L.state_from_inputs(x["k"], x["v"], "bf16", token_block=128)
    assert _rel(st, L.state_fp64(f["k"], f["v"])) < 1e-14
    rows = np.array([0, 7, 299])
    got = L.apply_rows(f["q"][1, rows], st[1], 1e-6)
    assert _rel(got, full[1, rows]) < 1e-13


def test_page_memory_arithmetic():
    """The course notes' memory table is arithmetic on the token counts: an n x n
    fp16 matrix against a d x d one (notes' d = 1536). The oracle's state is
    d x (d+1) per head whatever n is; check the printed figures re-derive."""
    assert 33 <= 4096 ** 2 * 2 / 1e6 < 34                  # ~33 MB
    assert abs(65536 ** 2 * 2 / 1e9 - 8.6) < 0.05          # ~8.6 GB
    assert abs(1536 ** 2 * 2 / 1e6 - 4.7) < 0.05           # ~4.7 MB
    assert 16 * 65536 == 1048576                           # video, 16 frames
    assert W.WORKLOADS["video_1m_tokens"].N == 16 * 65536
