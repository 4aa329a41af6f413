"""GPU parity of the variant flags against the fp64 oracle.

The variants are special cases of the same recurrence (engineermaxxing "From
GPT-2 to Kimi K3", ch. 05c: a scalar gate is Gated DeltaNet and alpha = 1 is
DeltaNet; heqinghuang "From GPT2 to Kimi3, Explained", section 07: without the
delta correction the write is additive, u = v, which is linear attention).
The oracle runs the plain recurrence with the scalar gate broadcast over the
key channels, g = 0 for no gate, and its additive mode; the library receives
the compact forms ([T, H] gate, no gate, no beta).
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_08_amd import workloads
from tests.gpu_util import assert_close, host, to_dev

pytestmark = pytest.mark.gpu

kda = pytest.importorskip("gated_delta_rule_08_amd")

VARIANTS = [(gate, additive) for gate in ("channel", "scalar", "none") for additive in (False, True)]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kda.load_library()
    yield
    torch.cuda.synchronize()


def _problem(seed, lengths, H, d, io):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    p = workloads.random_problem(rng, T, H, d, d, io_dtype=io)
    g_scalar = workloads.random_problem(rng, T, H, 1, 1)["g"][..., 0]   # log-sigmoid(N(3, 1))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    s0 = (0.02 * rng.standard_normal((len(lengths), H, d, d))).astype(np.float32)
    return p, g_scalar, cu, s0


def _gates(p, g_scalar, gate):
    """(gate given to the library, per-channel gate given to the oracle)"""
    if gate == "channel":
        return p["g"], p["g"]
    if gate == "scalar":
        return g_scalar, np.repeat(g_scalar[..., None], p["q"].shape[2], axis=2)
    return None, np.zeros_like(p["g"])


def _prefill_case(seed, lengths, H, d, chunk, io, gate, additive):
    p, g_scalar, cu, s0 = _problem(seed, lengths, H, d, io)
    g_lib, g_ref = _gates(p, g_scalar, gate)
    print(f"variant prefill seed={seed} lengths={lengths} H={H} d={d} C={chunk} io={io} "
          f"gate={gate} additive={additive}", flush=True)
    dev = lambda a: to_dev(a, io)
    states = to_dev(s0, dtype=torch.float32)
    o = kda.kda_chunk_fwd(dev(p["q"]), dev(p["k"]), dev(p["v"]),
                          None if g_lib is None else to_dev(g_lib, dtype=torch.float32),
                          None if additive else to_dev(p["beta"], dtype=torch.float32),
                          to_dev(cu, dtype=torch.int32), chunk=chunk, states=states,
                          read_initial=True, write_final=True, gate=gate, additive=additive)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], g_ref, p["beta"], cu, s0=s0,
                              mode=oracle.MODE_ADDITIVE if additive else oracle.MODE_DELTA)
    assert_close(host(o), o_ref, io, f"o ({gate}, additive={additive})")
    assert_close(host(states), s_ref, io, f"state ({gate}, additive={additive})")


@pytest.mark.parametrize("gate,additive", VARIANTS)
def test_prefill_variants_mfma_path(gate, additive):
    """bf16, d = 128, chunk 64 (MFMA path), 3 ragged sequences x 2 heads (state-only scan)."""
    _prefill_case(11, [70, 130, 200], 2, 128, 64, "bf16", gate, additive)


@pytest.mark.parametrize("gate,additive", [("scalar", False), ("none", True)])
def test_prefill_variants_many_chains(gate, additive):
    """64 chains: the single-pass scans carry the variants too."""
    _prefill_case(12, [100, 64, 129, 31], 16, 128, 64, "bf16", gate, additive)


@pytest.mark.parametrize("gate,additive", VARIANTS)
def test_prefill_variants_fp32_path(gate, additive):
    """fp32, d = 32, chunk 16 (fp32 path), 1e-4 contract."""
    _prefill_case(13, [37, 16, 50], 2, 32, 16, "fp32", gate, additive)


@pytest.mark.parametrize("gate,additive", VARIANTS)
@pytest.mark.parametrize("d,io", [(128, "bf16"), (64, "fp32")])
def test_decode_variants(gate, additive, d, io):
    B, H = 6, 3
    rng = np.random.default_rng(21 + d)
    p = workloads.random_problem(rng, B, H, d, d, io_dtype=io)
    g_scalar = workloads.random_problem(rng, B, H, 1, 1)["g"][..., 0]
    pool = (0.3 * rng.standard_normal((B, H, d, d))).astype(np.float32)
    g_lib, g_ref = _gates(p, g_scalar, gate)
    print(f"variant decode d={d} io={io} gate={gate} additive={additive}", flush=True)
    dev = lambda a: to_dev(a, io)
    states = to_dev(pool, dtype=torch.float32)
    o = kda.kda_decode_step(dev(p["q"]), dev(p["k"]), dev(p["v"]),
                            None if g_lib is None else to_dev(g_lib, dtype=torch.float32),
                            None if additive else to_dev(p["beta"], dtype=torch.float32), states,
                            gate=gate, additive=additive)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], g_ref, p["beta"],
                              np.arange(B + 1, dtype=np.int32), s0=pool,
                              mode=oracle.MODE_ADDITIVE if additive else oracle.MODE_DELTA)
    assert_close(host(o), o_ref, io, f"decode o ({gate}, additive={additive})")
    assert_close(host(states), s_ref, io, f"decode state ({gate}, additive={additive})")
