"""Helpers for the GPU parity tests: move seeded workloads to the device and
compare GPU results with the oracle under the stated tolerance."""
import numpy as np
import torch

# max |x_gpu - x_ref| <= TOL * max |x_ref|, per output tensor (o and final state)
TOL = {"bf16": 2e-2, "fp32": 1e-4}


def to_dev(a, io_dtype=None, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if io_dtype is not None:
        t = t.to(torch.bfloat16 if io_dtype == "bf16" else torch.float32)
    elif dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def inputs_to_dev(p, io_dtype):
    d = dict(q=to_dev(p["q"], io_dtype), k=to_dev(p["k"], io_dtype), v=to_dev(p["v"], io_dtype),
             g=to_dev(p["g"], dtype=torch.float32), beta=to_dev(p["beta"], dtype=torch.float32))
    if p.get("cu_seqlens") is not None:
        d["cu_seqlens"] = to_dev(p["cu_seqlens"], dtype=torch.int32)
    return d


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max()
    return float(np.abs(x - ref).max() / (scale if scale > 0 else 1.0))


def assert_close(x, ref, io_dtype, what=""):
    e = rel_err(x, ref)
    assert np.isfinite(np.asarray(x, dtype=np.float64)).all(), f"{what}: non-finite values"
    assert e <= TOL[io_dtype], f"{what}: max|err|/max|ref| = {e:.3e} > {TOL[io_dtype]:.0e}"
    return e


def host(t):
    return t.detach().float().cpu().numpy()
