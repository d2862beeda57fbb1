"""Pins of the QKV-projection oracle (oracle/linattn_qkv.py) against things
other than itself: a triple loop for the projection, torch's bf16
conversion and exact ties for the rounding, a selection weight that reduces
the whole path to the forward oracle, and the forward oracle's state. A
planted mistake anywhere in the module must fail at least one pin."""
import numpy as np
import pytest

import oracle.linattn as L
import oracle.linattn_qkv as QK


def _rng(seed):
    return np.random.default_rng(seed)


def pin_projection_loops():
    B, N, C, H, d = 2, 3, 5, 2, 4
    r = _rng(1)
    x = r.standard_normal((B, N, C))
    w = r.standard_normal((3 * H * d, C))
    q, k, v = QK.project(x, w, H, d)
    for b in range(B):
        for n in range(N):
            for which, t in enumerate((q, k, v)):
                for h in range(H):
                    for c in range(d):
                        row = which * H * d + h * d + c
                        want = sum(x[b, n, i] * w[row, i] for i in range(C))
                        if abs(t[b, n, h, c] - want) > 1e-12:
                            return f"projection {'qkv'[which]}[{b},{n},{h},{c}]"
    return None


def pin_rounding():
    import torch

    r = _rng(2)
    vals = r.standard_normal(20000).astype(np.float32).astype(np.float64) * 10.0 ** r.integers(-3, 4, 20000)
    vals = vals.astype(np.float32).astype(np.float64)
    want = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    if not np.array_equal(QK.round_bf16(vals), want):
        return "rounding differs from torch's on float32 values"
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 2 + 2.0 ** -7, 0.0])
    if not np.array_equal(QK.round_bf16(ties), np.array([1.0, 1 + 2.0 ** -6, -1.0, 2.0, 0.0])):
        return "ties are not rounded to even"
    return None


def pin_selection_weight():
    """W made of identity rows: q, k, v are column slices of x (bf16 values,
    so the rounding changes nothing) and the path is the forward oracle."""
    B, N, H, d = 2, 50, 3, 32
    D = H * d
    C = 3 * D
    r = _rng(3)
    x = QK.round_bf16(r.standard_normal((B, N, C)) + 0.1)
    perm = r.permutation(C)
    w = np.eye(C)[perm]
    q, out = QK.qkv_attention_fp64(x, w, H, 1e-6, d)
    xs = x[:, :, perm]
    qs, ks, vs = (xs[:, :, i * D:(i + 1) * D].reshape(B, N, H, d) for i in range(3))
    if not np.array_equal(q, qs):
        return "q is not the selected slice"
    want = L.linattn_fp64(qs, ks, vs, 1e-6)
    return None if np.array_equal(out, want) else "selection weight differs from the forward"


def pin_state_of_projection():
    B, N, C, H, d = 1, 40, 24, 2, 32
    r = _rng(4)
    x = r.standard_normal((B, N, C))
    w = r.standard_normal((3 * H * d, C)) / np.sqrt(C)
    q, out = QK.qkv_attention_fp64(x, w, H, 1e-6, d)
    # the projection by hand, rounded with torch, then the forward oracle
    import torch

    y = np.einsum("bnc,oc->bno", x, w)
    y = torch.from_numpy(y).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    D = H * d
    qs, ks, vs = (y[:, :, i * D:(i + 1) * D].reshape(B, N, H, d) for i in range(3))
    want = L.linattn_fp64(qs, ks, vs, 1e-6)
    # torch rounds through float32 (double rounding): agreement up to a rare ulp
    if np.abs(q - qs).max() > 2.0 ** -7 * np.abs(qs).max():
        return "q differs from the hand projection"
    if np.abs(out - want).max() > 1e-2 * np.abs(want).max():
        return "out differs from the hand projection's attention"
    return None


PINS = [pin_projection_loops, pin_rounding, pin_selection_weight, pin_state_of_projection]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin_holds(pin):
    msg = pin()
    assert msg is None, msg


def _project_transposed(x, w, H, d=32):
    B, N, C = x.shape
    D = H * d
    y = x.reshape(B * N, C) @ w.reshape(C, 3 * D)      # reads w in the wrong order
    return tuple(y[:, i * D:(i + 1) * D].reshape(B, N, H, d) for i in range(3))


def _project_qk_swapped(x, w, H, d=32):
    q, k, v = _orig_project(x, w, H, d)
    return k, q, v


def _project_heads_interleaved(x, w, H, d=32):
    B, N, C = x.shape
    D = H * d
    y = (x.reshape(B * N, C) @ w.T).reshape(B * N, 3, d, H).transpose(0, 1, 3, 2)
    return tuple(y[:, i].reshape(B, N, H, d) for i in range(3))


def _round_truncate(a):
    m, e = np.frexp(np.asarray(a, dtype=np.float64))
    return np.ldexp(np.trunc(m * 256.0) / 256.0, e)


def _round_half_up(a):
    m, e = np.frexp(np.asarray(a, dtype=np.float64))
    return np.ldexp(np.floor(m * 256.0 + 0.5) / 256.0, e)


def _round_none(a):
    return np.asarray(a, dtype=np.float64)


_orig_project = QK.project
MUTANTS = {
    "w_transposed": ("project", _project_transposed),
    "q_k_swapped": ("project", _project_qk_swapped),
    "heads_interleaved": ("project", _project_heads_interleaved),
    "round_truncates": ("round_bf16", _round_truncate),
    "round_half_up": ("round_bf16", _round_half_up),
    "no_rounding": ("round_bf16", _round_none),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(QK, attr, fn)
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
