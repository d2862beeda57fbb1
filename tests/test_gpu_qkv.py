"""GPU parity of the QKV projection with the attention state in its
epilogue (sana_linattn_qkv_fwd) against the CPU float64 oracle
(oracle/linattn_qkv.py) on the same seeded bits.

q: the kernel rounds its fp32 projection to bf16, the oracle its float64
one. The fp32 sum of C products is within C 2^-24 sum |x_i w_i| of the
exact one, so each q element must lie within one bf16 ulp of the oracle's
value plus that bound (elements near a rounding boundary, or small results
of large cancelling terms, land on a neighbouring bf16), and at most 0.5% of
elements may differ at all. out: the forward's tolerances (bf16 max-abs <=
1e-2, rel-L2 <= 5e-3), since out is the forward of q, k, v that differ from
the oracle's in such elements only."""
import numpy as np
import pytest

import oracle.linattn_qkv as QK
import relu_linear_attention_attn_amd as R
from relu_linear_attention_attn_amd import workloads as W

from gpu_util import assert_close, decode, to_host, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a ROCm GPU"
    R.lib()
    yield


def _dev(bits):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(t.bfloat16).cuda()


def _check_q(got_bits, ref, terms, C, what):
    """terms: sum_i |x_i w_i| per q element (float64)."""
    got = decode(got_bits, "bf16")
    ref_bits = W.f32_to_bf16_bits(ref.astype(np.float32))   # ref is already a bf16 value
    diff = got_bits != ref_bits
    frac = float(diff.mean()) if diff.size else 0.0
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    bound = ulp + C * 2.0 ** -24 * terms
    worst = float(np.max(np.abs(got - ref) / bound)) if got.size else 0.0
    print(f"{what} q: {frac:.2e} of elements off, worst {worst:.2f} of the bound", flush=True)
    assert frac <= 5e-3 and worst <= 1.0, what


def _terms(x_bits, w_bits, rows=None):
    x = np.abs(decode(x_bits, "bf16"))
    w = np.abs(decode(w_bits if rows is None else w_bits[rows], "bf16"))
    B, N, C = x.shape
    D = w.shape[0] // 3
    return (x.reshape(B * N, C) @ w[:D].T).reshape(B, N, D // 32, 32)


def _run(B, N, C, H, seed):
    w = W.custom(f"qkv_{B}_{N}_{C}_{H}", B, N, H, seed=seed)
    x = W.projection_inputs(w, C)
    q, out = R.forward_qkv(_dev(x["x"]), _dev(x["w"]), H, eps=w.eps)
    torch().cuda.synchronize()
    return w, x, to_host(q, "bf16"), to_host(out, "bf16")


SHAPES = [  # (B, N, C, H): ragged tokens, odd heads, C off the 64-channel step
    (1, 1, 8, 1), (1, 17, 64, 3), (2, 300, 96, 2), (2, 1000, 200, 4), (1, 4099, 512, 5),
    (3, 256, 1152, 36), (1, 600, 2240, 70),
]


@pytest.mark.parametrize("B,N,C,H", SHAPES)
def test_qkv_matches_oracle(B, N, C, H):
    print(f"\n[case] qkv B={B} N={N} C={C} H={H}", flush=True)
    w, x, q, out = _run(B, N, C, H, seed=800 + N + C + H)
    qref, oref = QK.qkv_attention_from_inputs(x["x"], x["w"], H, w.eps)
    _check_q(q, qref, _terms(x["x"], x["w"]), C, f"B={B} N={N} C={C} H={H}")
    assert_close(decode(out, "bf16"), oref, "bf16", f"qkv B={B} N={N} C={C} H={H}")


RAGGED_C = [8 * r for r in range(1, 8)] + [128 + 8 * r for r in range(8)]


@pytest.mark.parametrize("C", RAGGED_C)
def test_qkv_every_channel_residue(C):
    """C over every residue mod 64 (the projection's channel stage), in one
    stage and in three, with a ragged token tile and an odd head count:
    against the oracle, and bit for bit equal to the same inputs with x and W
    padded by zero channels to whole stages (the products of zero channels
    add +0 to every fp32 sum, so the zeroed tail of a ragged stage must act
    exactly like absent channels)."""
    B, N, H = 1, 300, 5
    print(f"\n[case] qkv channel residue C={C}", flush=True)
    w, x, q, out = _run(B, N, C, H, seed=1700 + C)
    qref, oref = QK.qkv_attention_from_inputs(x["x"], x["w"], H, w.eps)
    _check_q(q, qref, _terms(x["x"], x["w"]), C, f"C={C}")
    assert_close(decode(out, "bf16"), oref, "bf16", f"qkv C={C}")
    Cp = -(-C // 64) * 64
    if Cp != C:
        xp = np.zeros(x["x"].shape[:-1] + (Cp,), dtype=np.uint16)
        xp[..., :C] = x["x"]
        wp = np.zeros(x["w"].shape[:-1] + (Cp,), dtype=np.uint16)
        wp[..., :C] = x["w"]
        qp, outp = R.forward_qkv(_dev(xp), _dev(wp), H, eps=w.eps)
        torch().cuda.synchronize()
        assert np.array_equal(q, to_host(qp, "bf16")), f"C={C}: q differs from the padded run"
        assert np.array_equal(out, to_host(outp, "bf16")), f"C={C}: out differs from the padded run"


def test_qkv_latent_4096px_sampled_heads():
    """The 1.6B block at 4096px: x [2, 16384, 2240], 70 heads; heads 0, 33
    and 69 compared in full (the oracle projects only their rows)."""
    B, N, C, H = 2, 16384, 2240, 70
    w, x, q, out = _run(B, N, C, H, seed=4)
    D = H * 32
    for h in (0, 33, 69):
        rows = np.concatenate([np.arange(h * 32, h * 32 + 32) + i * D for i in range(3)])
        qref, oref = QK.qkv_attention_from_inputs(x["x"], x["w"][rows], 1, w.eps)
        sl = (slice(None), slice(None), slice(h, h + 1))
        _check_q(q[sl], qref, _terms(x["x"], x["w"], rows), C, f"4096px head {h}")
        assert_close(decode(out[sl], "bf16"), oref, "bf16", f"4096px head {h}")


def test_qkv_repeat_bitwise_and_events():
    B, N, C, H = 2, 3000, 256, 6
    w = W.custom("qkv_rep", B, N, H, seed=81)
    x = W.projection_inputs(w, C)
    xd, wd = _dev(x["x"]), _dev(x["w"])
    runs = []
    for _ in range(3):
        q, out = R.forward_qkv(xd, wd, H, eps=w.eps)
        runs.append((to_host(q, "bf16"), to_host(out, "bf16")))
    for r in runs[1:]:
        assert np.array_equal(r[0], runs[0][0]) and np.array_equal(r[1], runs[0][1])
    ev = [torch().cuda.Event(enable_timing=True) for _ in range(3)]
    q, out = R.forward_qkv(xd, wd, H, eps=w.eps, events=ev)
    torch().cuda.synchronize()
    assert np.array_equal(to_host(out, "bf16"), runs[0][1])
    assert all(ev[i].elapsed_time(ev[i + 1]) > 0 for i in range(2))


def test_qkv_out_is_the_forward_of_its_q():
    """With a selection weight (rows of the identity) the projection is exact
    (bf16 inputs, one nonzero product per output), so q, k, v are slices of
    x and the whole path must equal sana_linattn_fwd on those slices up to
    the forward's own summation order; q bit for bit."""
    B, N, H = 2, 2000, 4
    D = H * 32
    C = 3 * D
    w = W.custom("qkv_sel", B, N, H, seed=82)
    x = W.projection_inputs(w, C)["x"]
    perm = np.random.default_rng(5).permutation(C)
    eye = np.zeros((C, C), dtype=np.uint16)
    eye[np.arange(C), perm] = 0x3F80                        # bf16 1.0
    q, out = R.forward_qkv(_dev(x), _dev(eye), H, eps=w.eps)
    xs = x[:, :, perm]
    qs, ks, vs = (np.ascontiguousarray(xs[:, :, i * D:(i + 1) * D]).reshape(B, N, H, 32)
                  for i in range(3))
    ref = R.forward(_dev(qs), _dev(ks), _dev(vs), eps=w.eps)
    torch().cuda.synchronize()
    assert np.array_equal(to_host(q, "bf16"), qs)
    assert_close(decode(to_host(out, "bf16"), "bf16"), decode(to_host(ref, "bf16"), "bf16"),
                 "bf16", "selection weight vs the forward")
