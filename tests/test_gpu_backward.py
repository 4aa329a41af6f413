"""GPU parity of the chunked backward pass (kda_chunk_bwd) with the oracle's
token-by-token reverse-mode gradients.

The pages give no gradient; the oracle's backward is pinned by finite
differences and closed forms (tests/test_oracle_pins.py), and the chunk
algebra the kernels use is checked against it in fp64 on the CPU
(tests/test_chunkform_cpu.py).  Here the GPU result for dq, dk, dv, dg, dbeta
and dL/dS0 must match the oracle within the bf16 contract,
max|err| <= 2e-2 * max|ref| per tensor.
"""
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


def _case(seed, lengths, H, s0=False, d_final=False, wipe=False):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    d = 128
    p = workloads.random_problem(rng, T, H, d, d, io_dtype="bf16")
    if wipe:   # a near-total fade inside a 16-row block: the exact per-element path
        p["g"][5:7] = -45.0
    do = workloads.round_to_bf16(rng.standard_normal((T, H, d)).astype(np.float32))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    N = len(lengths)
    S0 = (0.02 * rng.standard_normal((N, H, d, d))).astype(np.float32) if s0 else None
    dST = (0.1 * rng.standard_normal((N, H, d, d))).astype(np.float32) if d_final else None
    shown = lengths if len(lengths) <= 16 else f"{len(lengths)} sequences, {T} tokens"
    print(f"backward seed={seed} lengths={shown} H={H} s0={s0} d_final={d_final} wipe={wipe}",
          flush=True)
    dev = lambda a: to_dev(a, "bf16")
    out = kda.kda_chunk_bwd(dev(p["q"]), dev(p["k"]), dev(p["v"]),
                            to_dev(p["g"], dtype=torch.float32),
                            to_dev(p["beta"], dtype=torch.float32),
                            to_dev(cu, dtype=torch.int32), dev(do),
                            states=None if S0 is None else to_dev(S0, dtype=torch.float32),
                            read_initial=S0 is not None,
                            d_final=None if dST is None else to_dev(dST, dtype=torch.float32),
                            want_d_initial=True)
    torch.cuda.synchronize()
    ref = oracle.run_bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], do, cu, s0=S0, ds_final=dST)
    errs = {name: assert_close(host(out[name]), ref[name], "bf16", name)
            for name in ("dq", "dk", "dv", "dg", "dbeta")}
    errs["d_initial"] = assert_close(host(out["d_initial"]), ref["ds0"], "bf16", "d_initial")
    print("  max|err|/max|ref|: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)


def test_backward_one_sequence_ragged_tail():
    """4 chunks (the last 8 rows long), 2 heads, zero initial state."""
    _case(41, [200], 2)


def test_backward_packed_with_states():
    """Ragged packed sequences (a one-token one included), initial states and dL/dS_final."""
    _case(42, [70, 130, 1, 64], 2, s0=True, d_final=True)


def test_backward_strong_fade_inside_a_block():
    """A gate spread beyond the split's range inside a block (exact per-element decay)."""
    _case(43, [150], 2, d_final=True, wipe=True)


def test_backward_many_chains():
    """48 (sequence, head) chains of 1-3 chunks."""
    _case(44, [64, 100, 150, 33, 128, 90], 8, s0=True, d_final=True)


def test_backward_zero_length_sequences_and_many_chains():
    """Zero-length sequences between others (their dL/dS0 is dL/dS_final) and 12 x 16 chains."""
    _case(46, [0, 90, 0, 200, 64, 0, 1, 130, 77, 0, 65, 300], 16, s0=True, d_final=True)


def test_backward_chain_lengths_around_the_copy_lookahead():
    """Chains of 6-9 chunks: the reverse pass's copies, dO rows and products start
    several chunks ahead of its carried state, so these lengths end inside each lookahead."""
    _case(47, [330, 420, 449, 520], 2, s0=True, d_final=True)


def test_backward_full_prefill_shape():
    """The prefill workload's shape: one sequence of 4,096 tokens, 16 heads."""
    _case(45, [4096], 16, d_final=True)


def test_backward_long_sequence():
    """One sequence of 16,384 tokens (256 chunks through both passes), 2 heads, slow decay."""
    _case(49, [16384], 2, s0=True, d_final=True)


@pytest.mark.parametrize("N", [384, 450])
def test_backward_sequences_around_the_fused_header_limit(N):
    """384 packed sequences (the most for which the prep builds the sequence header
    itself) and 450 (the header then comes from its own launch), 0-100 tokens each (a
    tenth empty), 2 heads."""
    rng = np.random.default_rng(48)
    lens = rng.integers(1, 101, size=N)
    lens[rng.random(N) < 0.1] = 0
    _case(48, [int(x) for x in lens], 2, s0=True, d_final=True)


def test_backward_empty_is_a_no_op():
    d = 128
    z = torch.zeros((0, 2, d), dtype=torch.bfloat16, device="cuda")
    out = kda.kda_chunk_bwd(z, z, z, torch.zeros((0, 2, d), device="cuda"),
                            torch.zeros((0, 2), device="cuda"),
                            torch.zeros(1, dtype=torch.int32, device="cuda"), z)
    torch.cuda.synchronize()
    assert out["dq"].numel() == 0


VARIANTS = [(gate, additive) for gate in ("channel", "scalar", "none") for additive in (False, True)]


@pytest.mark.parametrize("gate,additive", VARIANTS)
def test_backward_variants(gate, additive):
    """Scalar gate (Gated DeltaNet), no gate (DeltaNet), additive write (gated linear
    attention): the oracle runs the per-channel recurrence with the gate broadcast (its dg
    summed over channels is the scalar gate's gradient), g = 0, or its additive mode."""
    rng = np.random.default_rng(47)
    lengths, H, d = [70, 130, 1], 2, 128
    T = sum(lengths)
    p = workloads.random_problem(rng, T, H, d, d, io_dtype="bf16")
    g_scalar = workloads.random_problem(rng, T, H, 1, 1)["g"][..., 0]
    do = workloads.round_to_bf16(rng.standard_normal((T, H, d)).astype(np.float32))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    S0 = (0.02 * rng.standard_normal((len(lengths), H, d, d))).astype(np.float32)
    dST = (0.1 * rng.standard_normal((len(lengths), H, d, d))).astype(np.float32)
    g_lib = {"channel": p["g"], "scalar": g_scalar, "none": None}[gate]
    g_ref = {"channel": p["g"], "scalar": np.repeat(g_scalar[..., None], d, axis=2),
             "none": np.zeros_like(p["g"])}[gate]
    print(f"backward variant gate={gate} additive={additive}", flush=True)
    dev = lambda a: to_dev(a, "bf16")
    out = kda.kda_chunk_bwd(dev(p["q"]), dev(p["k"]), dev(p["v"]),
                            None if g_lib is None else to_dev(g_lib, dtype=torch.float32),
                            None if additive else to_dev(p["beta"], dtype=torch.float32),
                            to_dev(cu, dtype=torch.int32), dev(do),
                            states=to_dev(S0, dtype=torch.float32), read_initial=True,
                            d_final=to_dev(dST, dtype=torch.float32), want_d_initial=True,
                            gate=gate, additive=additive)
    torch.cuda.synchronize()
    ref = oracle.run_bwd(p["q"], p["k"], p["v"], g_ref, p["beta"], do, cu, s0=S0, ds_final=dST,
                         mode=oracle.MODE_ADDITIVE if additive else oracle.MODE_DELTA)
    for name in ("dq", "dk", "dv"):
        assert_close(host(out[name]), ref[name], "bf16", name)
    assert_close(host(out["d_initial"]), ref["ds0"], "bf16", "d_initial")
    if gate == "channel":
        assert_close(host(out["dg"]), ref["dg"], "bf16", "dg")
    elif gate == "scalar":
        assert_close(host(out["dg"]), ref["dg"].sum(axis=2), "bf16", "dg (scalar)")
    else:
        assert out["dg"] is None
    if additive:
        assert out["dbeta"] is None
    else:
        assert_close(host(out["dbeta"]), ref["dbeta"], "bf16", "dbeta")


RAW_CASES = [("channel", False, -np.inf), ("channel", False, -0.2), ("scalar", False, -0.2),
             ("none", False, -np.inf), ("channel", True, -np.inf), ("scalar", True, -np.inf)]


@pytest.mark.parametrize("gate,additive,gmin", RAW_CASES)
def test_backward_from_raw_projections(gate, additive, gmin):
    """kda_chunk_bwd_raw against the oracle: prepare_inputs, run_bwd, then the chain rule of
    prepare_inputs_bwd (the oracle's own, pinned by central differences)."""
    rng = np.random.default_rng(48)
    lengths, H, d = [70, 130, 1], 2, 128
    T = sum(lengths)
    bf = workloads.round_to_bf16
    f32 = lambda a: np.asarray(a, dtype=np.float32)
    q_raw = bf(f32(rng.standard_normal((T, H, d))))
    k_raw = bf(f32(rng.standard_normal((T, H, d))))
    v = bf(f32(rng.standard_normal((T, H, d))))
    a_raw = bf(f32(rng.standard_normal((T, H, d) if gate == "channel" else (T, H)) + 3.0))
    b_raw = bf(f32(rng.standard_normal((T, H))))
    do = bf(f32(rng.standard_normal((T, H, d))))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    S0 = (0.02 * rng.standard_normal((len(lengths), H, d, d))).astype(np.float32)
    dST = (0.1 * rng.standard_normal((len(lengths), H, d, d))).astype(np.float32)
    print(f"raw backward gate={gate} additive={additive} gate_min={gmin}", flush=True)
    bdev = lambda a: to_dev(a, "bf16")
    out = kda.kda_chunk_bwd_raw(bdev(q_raw), bdev(k_raw), bdev(v),
                                None if gate == "none" else bdev(a_raw),
                                None if additive else bdev(b_raw), to_dev(cu, dtype=torch.int32),
                                bdev(do), gate_min=gmin, states=to_dev(S0, dtype=torch.float32),
                                read_initial=True, d_final=to_dev(dST, dtype=torch.float32),
                                want_d_initial=True, gate=gate, additive=additive)
    torch.cuda.synchronize()
    q, k, g, beta = oracle.prepare_inputs(q_raw, k_raw, None if gate == "none" else a_raw,
                                          None if additive else b_raw, gmin, gate)
    mode = oracle.MODE_ADDITIVE if additive else oracle.MODE_DELTA
    ref = oracle.run_bwd(q, k, v, g, beta, do, cu, s0=S0, ds_final=dST, mode=mode)
    dq_raw, dk_raw, dgl, dbl = oracle.prepare_inputs_bwd(
        q_raw, k_raw, None if gate == "none" else a_raw, None if additive else b_raw, gmin, gate,
        ref["dq"], ref["dk"], ref["dg"], ref["dbeta"])
    assert_close(host(out["dq_raw"]), dq_raw, "bf16", "dq_raw")
    assert_close(host(out["dk_raw"]), dk_raw, "bf16", "dk_raw")
    assert_close(host(out["dv"]), ref["dv"], "bf16", "dv")
    assert_close(host(out["d_initial"]), ref["ds0"], "bf16", "d_initial")
    if gate == "none":
        assert out["dgate_logits"] is None
    else:
        assert_close(host(out["dgate_logits"]), dgl, "bf16", "dgate_logits")
    if additive:
        assert out["dbeta_logits"] is None
    else:
        assert_close(host(out["dbeta_logits"]), dbl, "bf16", "dbeta_logits")


def test_backward_every_sequence_empty_passes_the_state_gradient():
    """total_tokens 0 with sequences given: an empty sequence's final state is its initial
    state, so dL/dS0 = dL/dS_final, and zero when no final-state gradient is given."""
    d, H, N = 128, 2, 3
    z = torch.zeros((0, H, d), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((0, H, d), device="cuda")
    beta = torch.zeros((0, H), device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    s0 = torch.randn((N, H, d, d), device="cuda")
    d_final = torch.randn((N, H, d, d), device="cuda")
    out = kda.kda_chunk_bwd(z, z, z, g, beta, cu, z, states=s0, read_initial=True,
                            d_final=d_final, want_d_initial=True)
    torch.cuda.synchronize()
    assert torch.equal(out["d_initial"], d_final)
    out = kda.kda_chunk_bwd(z, z, z, g, beta, cu, z, want_d_initial=True)
    torch.cuda.synchronize()
    assert not out["d_initial"].any()
