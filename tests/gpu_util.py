"""Helpers shared by the GPU tests: host <-> device copies of raw input bits
and the comparison metrics. No attention arithmetic lives here."""
import numpy as np

import oracle.linattn as L


def torch():
    import torch as _t

    return _t


def gpu_available() -> bool:
    try:
        t = torch()
        return t.cuda.is_available()
    except Exception:
        return False


def to_device(x: np.ndarray, dtype: str):
    """uint16 bf16 bits or float32 values -> contiguous GPU tensor."""
    t = torch()
    if dtype == "bf16":
        return t.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(t.bfloat16).cuda()
    return t.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_host(x, dtype: str) -> np.ndarray:
    """GPU tensor -> uint16 bits (bf16) or float32 values."""
    t = torch()
    x = x.detach()
    if dtype == "bf16":
        return x.view(t.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    return L.to_f64(x, dtype)


def metrics(got: np.ndarray, ref: np.ndarray):
    """(max-abs error, rel-L2 error, max |ref|) in float64."""
    diff = got - ref
    maxabs = float(np.max(np.abs(diff))) if diff.size else 0.0
    nref = float(np.linalg.norm(ref.ravel()))
    rel = float(np.linalg.norm(diff.ravel()) / nref) if nref > 0 else float(np.linalg.norm(diff))
    return maxabs, rel, float(np.max(np.abs(ref))) if ref.size else 0.0


# Acceptance: bf16 in/out with fp32 accumulation: max-abs <= 1e-2 and
# rel-L2 <= 5e-3. fp32: rel-L2 <= 1e-5 and max-abs <= 1e-5 * max|ref|
# (normwise; elementwise relative error is meaningless near 0).
BF16_MAXABS = 1e-2
BF16_RELL2 = 5e-3
F32_REL = 1e-5


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    maxabs, rel, refmax = metrics(got, ref)
    msg = f"{what}: max-abs {maxabs:.3e}, rel-L2 {rel:.3e}, max|ref| {refmax:.3e}"
    print(msg, flush=True)
    assert np.all(np.isfinite(got)), msg + " (non-finite output)"
    if dtype == "bf16":
        assert maxabs <= BF16_MAXABS and rel <= BF16_RELL2, msg
    else:
        assert rel <= F32_REL and maxabs <= F32_REL * max(refmax, 1e-30), msg
    return maxabs, rel
