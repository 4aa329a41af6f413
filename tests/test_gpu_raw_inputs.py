"""GPU parity of the fused input preparation (raw bf16 projections) against the
fp64 oracle: oracle.prepare_inputs (SiLU + unit length for q and k, sigmoid
write strength, floored log-sigmoid gate) followed by the plain recurrence."""
import math

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_08_amd import workloads
from tests.gpu_util import assert_close, host, to_dev

pytestmark = pytest.mark.gpu

kda = pytest.importorskip("gated_delta_rule_08_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kda.load_library()
    yield
    torch.cuda.synchronize()


def _raw(rng, lead, d, gate):
    """Raw projections in bf16: q, k, v ~ N(0, 1); gate logits ~ N(3, 1) (alpha near 0.95);
    write-strength logits ~ N(0, 1)."""
    bf = workloads.round_to_bf16
    f32 = lambda a: np.asarray(a, dtype=np.float32)
    q = bf(f32(rng.standard_normal(lead + (d,))))
    k = bf(f32(rng.standard_normal(lead + (d,))))
    v = bf(f32(rng.standard_normal(lead + (d,))))
    gshape = lead + (d,) if gate == "channel" else lead
    a = bf(f32(rng.standard_normal(gshape) + 3.0))
    b = bf(f32(rng.standard_normal(lead)))
    return q, k, v, a, b


def _bf(a):
    return to_dev(a, "bf16")


CASES = [("channel", False, -math.inf), ("channel", True, -math.inf), ("scalar", False, -math.inf),
         ("none", False, -math.inf), ("scalar", True, -math.inf), ("channel", False, -0.2)]


@pytest.mark.parametrize("gate,additive,gmin", CASES)
@pytest.mark.parametrize("lengths,H", [([70, 130, 200], 2), ([100, 64, 129, 31], 16)])
def test_prefill_raw(gate, additive, gmin, lengths, H):
    d = 128
    rng = np.random.default_rng(31 + H)
    T = int(sum(lengths))
    q, k, v, a, b = _raw(rng, (T, H), d, gate)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    s0 = (0.02 * rng.standard_normal((len(lengths), H, d, d))).astype(np.float32)
    print(f"raw prefill lengths={lengths} H={H} gate={gate} additive={additive} gate_min={gmin}",
          flush=True)
    states = to_dev(s0, dtype=torch.float32)
    o = kda.kda_chunk_fwd_raw(_bf(q), _bf(k), _bf(v), None if gate == "none" else _bf(a),
                              None if additive else _bf(b), to_dev(cu, dtype=torch.int32),
                              gate_min=gmin, states=states, read_initial=True, write_final=True,
                              gate=gate, additive=additive)
    torch.cuda.synchronize()
    qp, kp, gp, bp = oracle.prepare_inputs(q, k, None if gate == "none" else a,
                                           None if additive else b, gate_min=gmin, gate=gate)
    o_ref, s_ref = oracle.run(qp, kp, v, gp, bp, cu, s0=s0,
                              mode=oracle.MODE_ADDITIVE if additive else oracle.MODE_DELTA)
    assert_close(host(o), o_ref, "bf16", "raw prefill o")
    assert_close(host(states), s_ref, "bf16", "raw prefill state")


@pytest.mark.parametrize("gate,additive,gmin", CASES)
@pytest.mark.parametrize("d", [128, 32])
def test_decode_raw(gate, additive, gmin, d):
    B, H = 6, 3
    rng = np.random.default_rng(41 + d)
    q, k, v, a, b = _raw(rng, (B, H), d, gate)
    pool = (0.3 * rng.standard_normal((B, H, d, d))).astype(np.float32)
    print(f"raw decode d={d} gate={gate} additive={additive} gate_min={gmin}", flush=True)
    states = to_dev(pool, dtype=torch.float32)
    o = kda.kda_decode_step_raw(_bf(q), _bf(k), _bf(v), None if gate == "none" else _bf(a),
                                None if additive else _bf(b), states, gate_min=gmin, gate=gate,
                                additive=additive)
    torch.cuda.synchronize()
    qp, kp, gp, bp = oracle.prepare_inputs(q, k, None if gate == "none" else a,
                                           None if additive else b, gate_min=gmin, gate=gate)
    o_ref, s_ref = oracle.run(qp, kp, v, gp, bp, np.arange(B + 1, dtype=np.int32), s0=pool,
                              mode=oracle.MODE_ADDITIVE if additive else oracle.MODE_DELTA)
    assert_close(host(o), o_ref, "bf16", "raw decode o")
    assert_close(host(states), s_ref, "bf16", "raw decode state")
