"""Per-launch timing (kda_launch_timer_begin / kda_launch_timer_end) on the GPU.

The timer is measurement only: the calls it brackets must give the same
results as without it, and it must name the launches in order.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_08_amd import workloads
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu

kda = pytest.importorskip("gated_delta_rule_08_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kda.load_library()
    yield
    torch.cuda.synchronize()


def _inputs(T=512, H=4, d=128, seed=71):
    p = workloads.random_problem(np.random.default_rng(seed), T, H, d, d, io_dtype="bf16")
    dev = lambda a: to_dev(a, "bf16")
    cu = to_dev(np.array([0, T], dtype=np.int32), dtype=torch.int32)
    return (dev(p["q"]), dev(p["k"]), dev(p["v"]), to_dev(p["g"], dtype=torch.float32),
            to_dev(p["beta"], dtype=torch.float32), cu)


def test_forward_launches_are_named_and_timed():
    print("launch timer: forward T=512 H=4", flush=True)
    q, k, v, g, beta, cu = _inputs()
    ref = kda.kda_chunk_fwd(q, k, v, g, beta, cu)
    stream = torch.cuda.current_stream()
    with kda.launch_timer(stream) as lt:
        o = kda.kda_chunk_fwd(q, k, v, g, beta, cu, stream=stream)
    names = [n for n, _ in lt.launches]
    assert names == ["prep_kernel", "scan_out_kernel"]
    assert all(ms > 0.0 for _, ms in lt.launches)
    assert torch.equal(o, ref)                       # the timer changes nothing computed


def test_backward_launches_are_named():
    print("launch timer: backward T=512 H=4", flush=True)
    q, k, v, g, beta, cu = _inputs(seed=72)
    d_o = torch.randn(q.shape, device="cuda").to(torch.bfloat16)
    stream = torch.cuda.current_stream()
    with kda.launch_timer(stream) as lt:
        kda.kda_chunk_bwd(q, k, v, g, beta, cu, d_o, stream=stream)
    assert [n for n, _ in lt.launches] == ["prep_kernel", "scan_pair_kernel", "grad_kernel"]


def test_second_begin_on_a_thread_is_rejected():
    print("launch timer: nested begin", flush=True)
    with kda.launch_timer() as outer:
        with pytest.raises(kda.KdaError):
            with kda.launch_timer():
                pass
    assert outer.launches == []
