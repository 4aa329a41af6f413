"""The allocation-free prefill, kda_chunk_fwd_noalloc, through the C ABI.

Its scratch is a device array inside the library instead of a caller workspace;
otherwise it runs the kernels of kda_chunk_fwd.  Two calls in a row, the second
smaller (so the array still holds the first call's operands), must each give
exactly what kda_chunk_fwd gives on the same inputs, and match the fp64 oracle
within the bf16 contract, max|err| <= 2e-2 * max|ref|.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_08_amd import workloads
from tests.gpu_util import assert_close, host, inputs_to_dev, to_dev

pytestmark = pytest.mark.gpu

kda = pytest.importorskip("gated_delta_rule_08_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kda.load_library()
    yield
    torch.cuda.synchronize()


def _run_both(seed, lens, H):
    """kda_chunk_fwd (caller workspace) and kda_chunk_fwd_noalloc on the same inputs, each
    from the same initial states; returns both outputs and final states and the oracle's."""
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N, T, d = len(lens), int(cu[-1]), 128
    p = workloads.random_problem(rng, T, H, d, d, io_dtype="bf16")
    p["cu_seqlens"] = cu
    s0 = (0.02 * rng.standard_normal((N, H, d, d))).astype(np.float32)
    print(f"noalloc seed={seed} N={N} T={T} H={H}", flush=True)
    dv = inputs_to_dev(p, "bf16")
    st_a = to_dev(s0, dtype=torch.float32)
    st_b = to_dev(s0, dtype=torch.float32)
    o_a = kda.kda_chunk_fwd(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], dv["cu_seqlens"],
                            chunk=64, states=st_a, read_initial=True, write_final=True)
    o_b = torch.full_like(o_a, 7.0)
    kda.kda_chunk_fwd_noalloc(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], dv["cu_seqlens"],
                              o_b, chunk=64, states=st_b, read_initial=True, write_final=True)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], cu, s0=s0)
    return (o_a, st_a), (o_b, st_b), (o_ref, s_ref)


@pytest.mark.parametrize("calls", [
    # few chains (state-only scan + output kernel), then a smaller call of the same kind
    [(71, [300, 64, 129], 4), (72, [70], 4)],
    # many chains (one workgroup per head), then a smaller few-chains call
    [(73, [int(x) for x in np.random.default_rng(5).integers(1, 200, size=40)], 4),
     (74, [65, 3], 2)],
])
def test_noalloc_equals_kda_chunk_fwd_on_two_calls(calls):
    for seed, lens, H in calls:
        (o_a, st_a), (o_b, st_b), (o_ref, s_ref) = _run_both(seed, lens, H)
        assert torch.equal(o_a, o_b), "o differs from kda_chunk_fwd"
        assert torch.equal(st_a, st_b), "final states differ from kda_chunk_fwd"
        assert_close(host(o_b), o_ref, "bf16", "noalloc o")
        assert_close(host(st_b), s_ref, "bf16", "noalloc state")


def test_noalloc_rejects_a_call_beyond_its_scratch():
    """A call that needs more than the static scratch is refused on the host."""
    T, H, d = 4096, 16, 128
    z = torch.zeros((T, H, d), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((T, H, d), device="cuda")
    beta = torch.zeros((T, H), device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    o = torch.full((T, H, d), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kda.KdaError) as e:
        kda.kda_chunk_fwd_noalloc(z, z, z, g, beta, cu, o)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())   # nothing was written
