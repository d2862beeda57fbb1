"""Pins of the block-causal oracle (oracle/linattn_block_causal.py) against
things other than itself: the explicit masked n x n form, the non-causal
oracle (one block), token-causal attention (blocks of one token, and single
rows from their definition), the first block alone, and causality (no output depends on later blocks). A planted
mistake anywhere in the oracle must fail at least one pin."""
import numpy as np
import pytest

import oracle.linattn as L
import oracle.linattn_block_causal as BC


def _inputs(seed, B, N, H, d=32):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, N, H, d)) for _ in range(3))
    q += 0.1
    k += 0.1
    return q, k, v


def _rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def pin_masked_form_exact():
    """The masked n x n form itself (masked_quadratic_fp64, the reference of
    the next pin) against exact rational arithmetic on dyadic inputs with a
    non-symmetric 0/1 mask: out_i = sum_n m_in w_in v_n / (sum_n m_in w_in + eps)."""
    from fractions import Fraction

    rng = np.random.default_rng(21)
    B, N, H, d = 1, 6, 2, 4
    q, k, v = (rng.integers(-16, 17, size=(B, N, H, d)) / 8.0 for _ in range(3))
    mask = (rng.random((N, N)) < 0.6).astype(np.float64)
    mask[0] = 0.0          # a query that sees nothing: out = 0
    eps = 0.25
    got = BC.masked_quadratic_fp64(q, k, v, mask, eps)
    relu = lambda x: max(Fraction(x), Fraction(0))  # noqa: E731
    for h in range(H):
        for i in range(N):
            w = [int(mask[i, j]) * sum(relu(q[0, i, h, e]) * relu(k[0, j, h, e]) for e in range(d))
                 for j in range(N)]
            for c in range(d):
                exact = float(sum(w[j] * Fraction(v[0, j, h, c]) for j in range(N))
                              / (sum(w) + Fraction(eps)))
                if abs(got[0, i, h, c] - exact) > 1e-14 * max(1.0, abs(exact)):
                    return f"masked form mismatch at {(i, h, c)}: {got[0, i, h, c]} vs {exact}"
    return None


def pin_masked_quadratic():
    """Against the explicit masked n x n form, including a ragged last block."""
    eps = 1e-3
    for seed, (B, N, H), Lb in ((1, (2, 24, 2), 8), (2, (1, 30, 3), 7), (3, (1, 17, 1), 5),
                                (4, (1, 40, 2), 40)):
        q, k, v = _inputs(seed, B, N, H)
        blk = np.arange(N) // Lb
        mask = (blk[None, :] <= blk[:, None]).astype(np.float64)
        got = BC.block_causal_fp64(q, k, v, Lb, eps)
        want = BC.masked_quadratic_fp64(q, k, v, mask, eps)
        if _rel(got, want) > 1e-12:
            return f"N={N} L={Lb}: differs from the masked quadratic form by {_rel(got, want):.2e}"
    return None


def pin_one_block_is_noncausal():
    eps = 1e-6
    q, k, v = _inputs(5, 2, 50, 3)
    got = BC.block_causal_fp64(q, k, v, 50, eps)
    want = L.linattn_fp64(q, k, v, eps)
    return None if _rel(got, want) < 1e-12 else "one block differs from the non-causal pass"


def pin_token_causal():
    """Blocks of one token: query i sees keys 0..i (lower-triangular mask)."""
    eps = 1e-3
    q, k, v = _inputs(6, 1, 20, 2)
    mask = np.tril(np.ones((20, 20)))
    got = BC.block_causal_fp64(q, k, v, 1, eps)
    want = BC.masked_quadratic_fp64(q, k, v, mask, eps)
    return None if _rel(got, want) < 1e-12 else "L = 1 is not token-causal attention"


def pin_first_block_alone():
    eps = 1e-6
    Lb = 12
    q, k, v = _inputs(7, 2, 60, 2)
    got = BC.block_causal_fp64(q, k, v, Lb, eps)[:, :Lb]
    want = L.linattn_fp64(q[:, :Lb], k[:, :Lb], v[:, :Lb], eps)
    return None if _rel(got, want) < 1e-12 else "the first block does not see exactly itself"


def pin_causality():
    """Changing keys and values after block c leaves blocks 0..c unchanged,
    bit for bit; changing them inside block c changes block c."""
    eps = 1e-6
    Lb = 10
    q, k, v = _inputs(8, 1, 50, 2)
    a = BC.block_causal_fp64(q, k, v, Lb, eps)
    k2, v2 = k.copy(), v.copy()
    k2[:, 30:] += 1.0
    v2[:, 30:] -= 2.0
    b = BC.block_causal_fp64(q, k2, v2, Lb, eps)
    if not np.array_equal(a[:, :30], b[:, :30]):
        return "an output depends on a later block"
    if np.allclose(a[:, 30:40], b[:, 30:40]):
        return "a block does not depend on its own keys"
    return None


def pin_token_causal_rows():
    """Single token-causal rows, each from its definition, against the
    lower-triangular masked form: the first row, rows inside, the last."""
    eps = 1e-3
    q, k, v = _inputs(10, 1, 37, 2)
    mask = np.tril(np.ones((37, 37)))
    want = BC.masked_quadratic_fp64(q, k, v, mask, eps)
    rows = [0, 1, 15, 16, 17, 36]
    for h in range(2):
        got = BC.token_causal_rows(q[0, :, h], k[0, :, h], v[0, :, h], rows, eps)
        if _rel(got, want[0, rows, h]) > 1e-12:
            return f"head {h}: rows differ from the masked form by {_rel(got, want[0, rows, h]):.2e}"
    return None


PINS = [pin_masked_form_exact, pin_masked_quadratic, pin_one_block_is_noncausal,
        pin_token_causal, pin_first_block_alone, pin_causality, pin_token_causal_rows]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin_holds(pin):
    msg = pin()
    assert msg is None, msg


def _mut_masked(kind):
    def masked_quadratic_fp64(q, k, v, mask, eps):
        B, N, H, d = q.shape
        out = np.empty((B, N, H, d))
        for b in range(B):
            for h in range(H):
                w = L.phi(q[b, :, h]) @ L.phi(k[b, :, h]).T
                m = mask.T if kind == "mask_transposed" else mask
                w = w if kind == "mask_ignored" else w * m
                r = w.sum(axis=1)
                if kind == "den_unmasked":
                    r = (L.phi(q[b, :, h]) @ L.phi(k[b, :, h]).T).sum(axis=1)
                out[b, :, h] = (w @ v[b, :, h]) / (r + eps)[:, None]
        return out
    return masked_quadratic_fp64


def _mut_prefix(kind):
    def f(states):
        if kind == "exclusive":
            out = np.cumsum(states, axis=0) - states
            return out
        if kind == "no_prefix":
            return states
        if kind == "reversed":
            return np.cumsum(states[::-1], axis=0)[::-1]
        raise AssertionError(kind)
    return f


def _mut_block_states(kind):
    def f(k, v, Lb):
        n, d = k.shape
        nb = (n + Lb - 1) // Lb
        pk = L.phi(k)
        va = np.concatenate([v, np.ones((n, 1))], axis=1)
        st = np.empty((nb, d, d + 1))
        for c in range(nb):
            lo, hi = c * Lb, (c + 1) * Lb
            if kind == "off_by_one":
                hi = min(hi + 1, n)
            elif kind == "drop_last_token":
                hi = min(hi, n) - 1 if min(hi, n) - 1 > lo else min(hi, n)
            st[c] = pk[lo:hi].T @ va[lo:hi]
        if kind == "no_ones":
            st[:, :, d] = 0.0
        return st
    return f


def _mut_apply(kind):
    def f(q, prefix, Lb, eps):
        n, d = q.shape
        pq = L.phi(q)
        out = np.empty((n, d))
        for c in range(prefix.shape[0]):
            rows = slice(c * Lb, (c + 1) * Lb)
            s = prefix[max(c - 1, 0)] if kind == "previous_block" else prefix[c]
            if kind == "last_prefix":
                s = prefix[-1]
            out[rows] = (pq[rows] @ s[:, :d]) / (pq[rows] @ s[:, d] + eps)[:, None]
        return out
    return f


def _mut_rows(kind):
    def f(q, k, v, rows, eps):
        n, d = q.shape
        out = np.empty((len(rows), d))
        for r, i in enumerate(rows):
            hi = {"sees_next_key": min(i + 2, n), "misses_own_key": i}.get(kind, i + 1)
            pk = L.phi(k[:hi])
            s = pk.T @ np.concatenate([v[:hi], np.ones((hi, 1))], axis=1)
            if kind == "den_without_keys":
                s[:, d] = 0.0
            pq = L.phi(q[i])
            out[r] = (pq @ s[:, :d]) / (pq @ s[:, d] + eps)
        return out
    return f


MUTANTS = {
    "rows_see_next_key": ("token_causal_rows", _mut_rows("sees_next_key")),
    "rows_miss_own_key": ("token_causal_rows", _mut_rows("misses_own_key")),
    "rows_den_without_keys": ("token_causal_rows", _mut_rows("den_without_keys")),
    "exclusive_prefix": ("prefix_states", _mut_prefix("exclusive")),
    "no_prefix": ("prefix_states", _mut_prefix("no_prefix")),
    "reversed_prefix": ("prefix_states", _mut_prefix("reversed")),
    "block_off_by_one": ("block_states", _mut_block_states("off_by_one")),
    "block_drops_token": ("block_states", _mut_block_states("drop_last_token")),
    "no_ones_column": ("block_states", _mut_block_states("no_ones")),
    "previous_block_state": ("apply_prefix", _mut_apply("previous_block")),
    "whole_sequence_state": ("apply_prefix", _mut_apply("last_prefix")),
    "mask_transposed": ("masked_quadratic_fp64", _mut_masked("mask_transposed")),
    "mask_ignored": ("masked_quadratic_fp64", _mut_masked("mask_ignored")),
    "den_unmasked": ("masked_quadratic_fp64", _mut_masked("den_unmasked")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(BC, attr, fn)
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

    w = W.custom("bc_drv", 2, 64, 3, dtype="bf16", seed=9)
    x = W.generate(w)
    a = BC.block_causal_from_inputs(x["q"], x["k"], x["v"], 16, w.eps, "bf16")
    dec = [L.bf16_bits_to_f64(x[t]) for t in "qkv"]
    assert np.array_equal(a, BC.block_causal_fp64(*dec, 16, w.eps))
