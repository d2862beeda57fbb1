"""GPU parity of block-causal attention: the HIP path against the CPU
float64 block-causal oracle, element by element, on the same seeded bits.
Tolerances as for the forward pass: bf16 max-abs <= 1e-2 and rel-L2 <= 5e-3;
fp32 rel-L2 <= 1e-5 and max-abs <= 1e-5 * max|ref|. Blocks of at most 16
tokens take the token-causal bound instead (per element 2^-8 |ref| + 2e-3,
rel-L2 <= 5e-3): a query in an early block averages v over a few keys, so
|out| reaches max |v| and the bf16 rounding of the output alone can exceed
a flat 1e-2 there."""
import numpy as np
import pytest

import oracle.linattn_block_causal as BC
import relu_linear_attention_attn_amd as R
from relu_linear_attention_attn_amd import workloads as W

from gpu_util import assert_close, decode, to_device, to_host, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a ROCm GPU"
    R.lib()
    yield


def _inputs(w):
    x = W.generate(w)
    return x, {t: to_device(x[t], w.dtype) for t in "qkv"}


def _run(w, dev, block):
    out = R.forward_block_causal(dev["q"], dev["k"], dev["v"], block, eps=w.eps)
    torch().cuda.synchronize()
    return to_host(out, w.dtype)


CASES = [  # (B, N, H, block, dtype); bf16 blocks up to 256 tokens take the chunk-wise kernels
    (2, 4096, 6, 1024, "bf16"), (2, 4096, 6, 1024, "f32"), (1, 16384, 36, 1024, "bf16"),
    (3, 5000, 7, 1000, "bf16"), (3, 5000, 7, 1000, "f32"), (2, 160, 3, 16, "bf16"),
    (1, 2048, 5, 2048, "bf16"), (1, 64, 2, 1, "bf16"), (1, 64, 2, 1, "f32"), (2, 96, 1, 32, "bf16"),
    (2, 1000, 3, 2, "bf16"), (1, 4100, 5, 4, "bf16"), (2, 3000, 4, 8, "bf16"),
    (1, 16384, 6, 16, "bf16"), (2, 100, 3, 4, "f32"),
    # bf16 blocks of 2..16 whole tiles: the block-wise chunked apply (512: per block)
    (2, 4096, 6, 32, "bf16"), (1, 4800, 5, 48, "bf16"), (2, 16384, 8, 64, "bf16"),
    (1, 8192, 3, 256, "bf16"), (2, 5120, 5, 512, "bf16"), (3, 64, 7, 32, "bf16"),
    (2, 4096, 6, 64, "f32"),
]


@pytest.mark.parametrize("B,N,H,block,dtype", CASES)
def test_block_causal_matches_oracle(B, N, H, block, dtype):
    w = W.custom(f"bc_{B}_{N}_{H}_{block}", B, N, H, dtype=dtype, seed=500 + N + H + block,
                 q=W.Dist("normal", 0.1, 1.0), k=W.Dist("normal", 0.1, 1.0))
    print(f"\n[case] block-causal B={B} N={N} H={H} block={block} {dtype}", flush=True)
    x, dev = _inputs(w)
    ref = BC.block_causal_from_inputs(x["q"], x["k"], x["v"], block, w.eps, dtype)
    got = decode(_run(w, dev, block), dtype)
    what = f"B={B} N={N} H={H} block={block} {dtype}"
    if dtype == "bf16" and block <= 16:
        from test_gpu_causal import assert_causal_close

        assert_causal_close(got, ref, what)
    else:
        assert_close(got, ref, dtype, what)


@pytest.mark.parametrize("B,N,H", [(1, 64, 2), (2, 3000, 5), (2, 16384, 70)])
def test_unit_blocks_are_the_token_causal_kernels(B, N, H):
    """bf16 blocks of one token: bitwise the token-causal entry point's result."""
    w = W.custom(f"bc1_{B}_{N}_{H}", B, N, H, seed=77 + N)
    x, dev = _inputs(w)
    a = _run(w, dev, 1)
    b = R.forward_causal(dev["q"], dev["k"], dev["v"], eps=w.eps)
    torch().cuda.synchronize()
    assert np.array_equal(a, to_host(b, "bf16"))


def test_one_block_matches_noncausal_forward():
    w = W.WORKLOADS["sana06_1024px"]
    x, dev = _inputs(w)
    a = decode(_run(w, dev, w.N), "bf16")
    b = decode(to_host(R.forward(dev["q"], dev["k"], dev["v"], eps=w.eps,
                                 variant=R.VARIANT_SPLIT), "bf16"), "bf16")
    assert_close(a, b, "bf16", "one block vs the non-causal forward")


def test_outputs_do_not_depend_on_later_blocks():
    """Changing k and v in blocks 3.. leaves blocks 0..2 bitwise unchanged."""
    w = W.custom("bc_causal", 2, 4096, 6, seed=61)
    x, dev = _inputs(w)
    a = _run(w, dev, 512)
    k2, v2 = dev["k"].clone(), dev["v"].clone()
    k2[:, 1536:] = -k2[:, 1536:]
    v2[:, 1536:] = 2 * v2[:, 1536:]
    out = R.forward_block_causal(dev["q"], k2, v2, 512, eps=w.eps)
    torch().cuda.synchronize()
    b = to_host(out, "bf16")
    assert np.array_equal(a[:, :1536], b[:, :1536])
    assert not np.array_equal(a[:, 1536:], b[:, 1536:])


def test_block_causal_repeat_bitwise_and_profiled():
    w = W.custom("bc_rep", 2, 8192, 5, seed=62)
    x, dev = _inputs(w)
    runs = [_run(w, dev, 2048) for _ in range(3)]
    assert all(np.array_equal(runs[0], r) for r in runs[1:])
    ev = [torch().cuda.Event(enable_timing=True) for _ in range(4)]
    out = R.forward_block_causal(dev["q"], dev["k"], dev["v"], 2048, eps=w.eps, events=ev)
    torch().cuda.synchronize()
    assert np.array_equal(to_host(out, "bf16"), runs[0])
    assert all(ev[i].elapsed_time(ev[i + 1]) > 0 for i in range(3))


@pytest.mark.timeout(900)
def test_video_frames_block_causal_sampled_heads():
    """16 frames of 65,536 tokens (the video shape), each frame a block: two
    heads compared in full against the oracle."""
    w = W.WORKLOADS["video_1m_tokens"]
    block = 65536
    print(f"\n[case] block-causal video {w.shape} block={block}", flush=True)
    x, dev = _inputs(w)
    got = _run(w, dev, block)
    for h in (0, w.H - 1):
        sl = (slice(None), slice(None), slice(h, h + 1))
        ref = BC.block_causal_from_inputs(x["q"][sl], x["k"][sl], x["v"][sl], block, w.eps, "bf16")
        assert_close(decode(got[sl], "bf16"), ref, "bf16", f"video head {h}")
