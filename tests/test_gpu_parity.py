"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every comparison is element by element on the same seeded inputs with
max |gpu - oracle| <= tol * max |oracle| for the outputs and the final states,
tol = 2e-2 for bf16 I/O and 1e-4 for the fp32 path.
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


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ decode

def test_decode_c2_full():
    """Decode step at B=256, H=32, d=128, bf16, resident pool (512 MiB)."""
    p = workloads.make_inputs(2)
    _log("decode c2: shapes q%s pool%s" % (p["q"].shape, p["s0"].shape))
    d = inputs_to_dev(p, "bf16")
    states = to_dev(p["s0"], dtype=torch.float32)
    o = kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], states)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.decode(p["q"], p["k"], p["v"], p["g"], p["beta"], p["s0"])
    assert_close(host(o), o_ref, "bf16", "decode o")
    assert_close(host(states), s_ref, "bf16", "decode state")


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_decode_dims_and_slots(d, io):
    rng = np.random.default_rng(d)
    B, H, S = 5, 3, 9
    p = workloads.random_problem(rng, B, H, d, d, io_dtype=io)
    pool = (0.3 * rng.standard_normal((S, H, d, d))).astype(np.float32)
    slots = np.array([7, 0, 4, 2, 8], dtype=np.int32)
    dv = inputs_to_dev(p, io)
    states = to_dev(pool, dtype=torch.float32)
    o = kda.kda_decode_step(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], states,
                            state_slots=to_dev(slots, dtype=torch.int32))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.decode(p["q"], p["k"], p["v"], p["g"], p["beta"], pool[slots])
    assert_close(host(o), o_ref, io, "decode o")
    got = host(states)
    assert_close(got[slots], s_ref, io, "decode state")
    untouched = [s for s in range(S) if s not in slots]
    np.testing.assert_array_equal(got[untouched], pool[untouched])


def test_decode_out_of_range_slot_is_skipped():
    rng = np.random.default_rng(3)
    B, H, d, S = 3, 2, 64, 4
    p = workloads.random_problem(rng, B, H, d, d)
    pool = rng.standard_normal((S, H, d, d)).astype(np.float32)
    states = to_dev(pool, dtype=torch.float32)
    o = torch.full((B, H, d), 123.0, device="cuda")
    dv = inputs_to_dev(p, "fp32")
    kda.kda_decode_step(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], states,
                        state_slots=to_dev(np.array([1, -1, 7], np.int32), dtype=torch.int32), o=o)
    torch.cuda.synchronize()
    oh, sh = host(o), host(states)
    assert np.all(oh[1] == 123.0) and np.all(oh[2] == 123.0)
    np.testing.assert_array_equal(sh[[0, 2, 3]], pool[[0, 2, 3]])
    o_ref, s_ref = oracle.decode(p["q"][:1], p["k"][:1], p["v"][:1], p["g"][:1], p["beta"][:1],
                                 pool[1:2])
    assert_close(oh[:1], o_ref, "fp32", "decode o")
    assert_close(sh[1:2], s_ref, "fp32", "decode state")


def test_decode_sixteen_steps_equal_recurrence():
    rng = np.random.default_rng(4)
    steps, B, H, d = 16, 4, 4, 128
    p = workloads.random_problem(rng, steps * B, H, d, d, io_dtype="bf16")
    pool = (0.02 * rng.standard_normal((B, H, d, d))).astype(np.float32)
    states = to_dev(pool, dtype=torch.float32)
    dv = inputs_to_dev(p, "bf16")
    outs = []
    for t in range(steps):
        sl = slice(t * B, (t + 1) * B)
        outs.append(host(kda.kda_decode_step(dv["q"][sl], dv["k"][sl], dv["v"][sl], dv["g"][sl],
                                             dv["beta"][sl], states)))
    torch.cuda.synchronize()
    # token t of sequence b sits at row t * B + b
    perm = np.array([t * B + b for b in range(B) for t in range(steps)])
    cu = np.arange(0, B * steps + 1, steps, dtype=np.int32)
    o_ref, s_ref = oracle.run(p["q"][perm], p["k"][perm], p["v"][perm], p["g"][perm],
                              p["beta"][perm], cu, s0=pool)
    o_gpu = np.stack(outs).transpose(1, 0, 2, 3).reshape(B * steps, H, d)
    assert_close(o_gpu, o_ref, "bf16", "16-step o")
    assert_close(host(states), s_ref, "bf16", "16-step state")


# ------------------------------------------------------------------ state pool

def test_state_init_load_store_roundtrip():
    rng = np.random.default_rng(5)
    S, H, d = 6, 3, 32
    states = torch.full((S, H, d, d), 7.0, device="cuda")
    kda.kda_state_init(states)
    torch.cuda.synchronize()
    assert float(states.abs().max()) == 0.0
    src = rng.standard_normal((3, H, d, d)).astype(np.float32)
    slots = np.array([4, 1, 5], np.int32)
    kda.kda_state_load(states, to_dev(src, dtype=torch.float32), to_dev(slots, dtype=torch.int32))
    back = kda.kda_state_store(states, to_dev(np.array([5, 4, 0, 1], np.int32), dtype=torch.int32))
    torch.cuda.synchronize()
    b = host(back)
    np.testing.assert_array_equal(b[0], src[2])
    np.testing.assert_array_equal(b[1], src[0])
    np.testing.assert_array_equal(b[2], 0)
    np.testing.assert_array_equal(b[3], src[1])


# ------------------------------------------------------------------ prefill

def _prefill(p, io, chunk, s0=None, slots=None, read=False, write=False, pool_slots=None):
    d = inputs_to_dev(p, io)
    states = None
    if s0 is not None:
        states = to_dev(s0, dtype=torch.float32)
    o = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=chunk,
                          states=states, state_slots=slots, read_initial=read, write_final=write)
    torch.cuda.synchronize()
    return host(o), (host(states) if states is not None else None)


def test_prefill_c0_fp32_path():
    """B=1, H=2, T=64, d=16, chunk=16, fp32: the 1e-4 contract."""
    p = workloads.make_inputs(0)
    cfg = p["config"]
    N, H, d = 1, cfg.num_heads, cfg.dk
    pool = np.zeros((N, H, d, d), np.float32)
    o, s = _prefill(p, "fp32", cfg.chunk, s0=pool, write=True)
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu_seqlens"])
    assert_close(o, o_ref, "fp32", "c0 o")
    assert_close(s, s_ref, "fp32", "c0 state")


@pytest.mark.parametrize("d,chunk", [(16, 16), (16, 64), (32, 32), (64, 16), (64, 64),
                                     (128, 16), (128, 32)])
@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_prefill_fp32_path_varlen(d, chunk, io):
    rng = np.random.default_rng(d * 7 + chunk)
    lens = [1, chunk - 1, chunk, chunk + 1, 0, 3 * chunk + 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    H = 2
    p = workloads.random_problem(rng, int(cu[-1]), H, d, d, io_dtype=io)
    p["cu_seqlens"] = cu
    N = len(lens)
    s0 = (0.05 * rng.standard_normal((N, H, d, d))).astype(np.float32)
    o, s = _prefill(p, io, chunk, s0=s0, read=True, write=True)
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], cu, s0=s0)
    tol_io = "fp32" if io == "fp32" else "bf16"
    assert_close(o, o_ref, tol_io, "o")
    assert_close(s, s_ref, tol_io, "state")


def test_prefill_c1_full():
    """B=1, H=16, T=4096, d=128, chunk=64, bf16 (the measured configuration)."""
    p = workloads.make_inputs(1)
    cfg = p["config"]
    pool = np.zeros((1, cfg.num_heads, 128, 128), np.float32)
    _log("prefill c1: q%s" % (p["q"].shape,))
    o, s = _prefill(p, "bf16", 64, s0=pool, write=True)
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu_seqlens"])
    e_o = assert_close(o, o_ref, "bf16", "c1 o")
    e_s = assert_close(s, s_ref, "bf16", "c1 state")
    _log(f"c1 rel err o={e_o:.2e} state={e_s:.2e}")


@pytest.mark.parametrize("H", [3, 8])
def test_prefill_mfma_ragged_varlen_slots(H):
    """Ragged sequences (empty, one token, a chunk and one row, ...) with state slots;
    H = 3: 24 chains, 16 state columns per scan workgroup; H = 8: 64 chains, 32."""
    rng = np.random.default_rng(11)
    lens = [1, 63, 64, 65, 0, 130, 200, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d, N = 128, len(lens)
    p = workloads.random_problem(rng, int(cu[-1]), H, d, d, io_dtype="bf16")
    p["cu_seqlens"] = cu
    pool = (0.02 * rng.standard_normal((N + 3, H, d, d))).astype(np.float32)
    slots = np.array([9, 0, 3, 10, 1, 5, 7, 2], np.int32)
    d_in = inputs_to_dev(p, "bf16")
    states = to_dev(pool, dtype=torch.float32)
    o = kda.kda_chunk_fwd(d_in["q"], d_in["k"], d_in["v"], d_in["g"], d_in["beta"],
                          d_in["cu_seqlens"], chunk=64, states=states,
                          state_slots=to_dev(slots, dtype=torch.int32), read_initial=True,
                          write_final=True)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], cu, s0=pool[slots])
    assert_close(host(o), o_ref, "bf16", "o")
    got = host(states)
    assert_close(got[slots], s_ref, "bf16", "state")
    untouched = [i for i in range(N + 3) if i not in slots]
    np.testing.assert_array_equal(got[untouched], pool[untouched])


def test_prefill_mfma_many_chains():
    """More than 128 (sequence, head) chains: the throughput layout of the scan
    (one workgroup of 4 waves x 32 columns per head)."""
    rng = np.random.default_rng(15)
    lens = [int(x) for x in rng.integers(1, 200, size=40)]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    H, d, N = 4, 128, len(lens)
    p = workloads.random_problem(rng, int(cu[-1]), H, d, d, io_dtype="bf16")
    p["cu_seqlens"] = cu
    s0 = (0.02 * rng.standard_normal((N, H, d, d))).astype(np.float32)
    o, s = _prefill(p, "bf16", 64, s0=s0, read=True, write=True)
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], cu, s0=s0)
    assert_close(o, o_ref, "bf16", "o")
    assert_close(s, s_ref, "bf16", "state")


@pytest.mark.parametrize("case", ["wipes", "deltanet", "beta0", "scalar_gate", "strong_decay"])
def test_prefill_mfma_special_gates(case):
    """Extreme and degenerate gates, incl. the element-wise path for strong decay."""
    rng = np.random.default_rng(12)
    T, H, d = 300, 2, 128
    p = workloads.random_problem(rng, T, H, d, d, io_dtype="bf16")
    if case == "wipes":
        p["g"][40:44] = -30.0          # several wipes inside one 16-row block
        p["g"][100] = -30.0
    elif case == "deltanet":
        p["g"][:] = 0.0
    elif case == "beta0":
        p["beta"][:] = 0.0
    elif case == "scalar_gate":
        p["g"][:] = p["g"][:, :, :1]
    elif case == "strong_decay":
        p["g"] = np.minimum(p["g"] * 40.0, 0.0).astype(np.float32)
    p["cu_seqlens"] = np.array([0, T], np.int32)
    s0 = (0.5 * rng.standard_normal((1, H, d, d))).astype(np.float32)
    o, s = _prefill(p, "bf16", 64, s0=s0, read=True, write=True)
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu_seqlens"], s0=s0)
    assert_close(o, o_ref, "bf16", f"{case} o")
    assert_close(s, s_ref, "bf16", f"{case} state")


def test_prefill_split_resume_and_decode_continuation():
    """prefill(a||b) == prefill(b) from prefill(a)'s stored state; prefill(T) + decode(T+1)."""
    rng = np.random.default_rng(13)
    T, H, d = 257, 2, 128
    p = workloads.random_problem(rng, T + 1, H, d, d, io_dtype="bf16")
    dv = inputs_to_dev(p, "bf16")
    states = torch.zeros((1, H, d, d), device="cuda")
    cu = lambda a, b: to_dev(np.array([0, b - a], np.int32), dtype=torch.int32)
    sl = lambda a, b: {n: dv[n][a:b].contiguous() for n in ("q", "k", "v", "g", "beta")}
    A, B = sl(0, 100), sl(100, T)
    oa = kda.kda_chunk_fwd(**A, cu_seqlens=cu(0, 100), states=states, write_final=True)
    ob = kda.kda_chunk_fwd(**B, cu_seqlens=cu(100, T), states=states, read_initial=True,
                           write_final=True)
    last = sl(T, T + 1)
    od = kda.kda_decode_step(last["q"], last["k"], last["v"], last["g"], last["beta"], states)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"])
    o_gpu = np.concatenate([host(oa), host(ob), host(od)])
    assert_close(o_gpu, o_ref, "bf16", "split o")
    assert_close(host(states)[0], s_ref[0], "bf16", "split state")


def test_prefill_causality():
    """Perturbing tokens after t leaves o[<= t] unchanged."""
    rng = np.random.default_rng(14)
    T, H, d, t = 200, 2, 128, 90
    p = workloads.random_problem(rng, T, H, d, d, io_dtype="bf16")
    p["cu_seqlens"] = np.array([0, T], np.int32)
    o1, _ = _prefill(p, "bf16", 64)
    p2 = {n: (a.copy() if isinstance(a, np.ndarray) else a) for n, a in p.items()}
    p2["v"][t + 1:] = workloads.round_to_bf16(p2["v"][t + 1:] * -1.5)
    p2["k"][t + 1:] = p2["k"][t + 1:][:, :, ::-1].copy()
    p2["beta"][t + 1:] = 0.9
    o2, _ = _prefill(p2, "bf16", 64)
    np.testing.assert_array_equal(o1[: t + 1], o2[: t + 1])
    assert np.abs(o1[t + 1:] - o2[t + 1:]).max() > 1e-3


# ------------------------------------------------------------------ full-size, whole config

def _full_check(cfg_index, head_group):
    """The whole configuration on the GPU in one call, then every (sequence, head) chain
    against the oracle, streamed over groups of heads so that host memory stays bounded.
    The bar is taken over the whole configuration: max|err| over all chains against
    max|ref| over all chains, for o and for the final states."""
    p = workloads.make_inputs(cfg_index)
    cfg = p["config"]
    cu = p["cu_seqlens"]
    N, H, d = len(cu) - 1, cfg.num_heads, cfg.dk
    _log(f"config {cfg_index}: T={cu[-1]} N={N} H={H} (whole configuration)")
    s0 = p["s0"]
    d_in = inputs_to_dev(p, "bf16")
    states = (to_dev(s0, dtype=torch.float32) if s0 is not None
              else torch.zeros((N, H, d, d), device="cuda"))
    o = kda.kda_chunk_fwd(d_in["q"], d_in["k"], d_in["v"], d_in["g"], d_in["beta"],
                          d_in["cu_seqlens"], chunk=cfg.chunk, states=states,
                          read_initial=s0 is not None, write_final=True)
    torch.cuda.synchronize()
    del d_in
    err = {"o": 0.0, "S": 0.0}
    ref_max = {"o": 0.0, "S": 0.0}
    for h0 in range(0, H, head_group):
        hs = slice(h0, min(H, h0 + head_group))
        o_ref, s_ref = oracle.run(p["q"][:, hs], p["k"][:, hs], p["v"][:, hs], p["g"][:, hs],
                                  p["beta"][:, hs], cu, s0=None if s0 is None else s0[:, hs])
        for name, got, ref in (("o", host(o[:, hs]), o_ref), ("S", host(states[:, hs]), s_ref)):
            assert np.isfinite(got).all(), f"cfg{cfg_index} {name} heads {hs}: non-finite values"
            err[name] = max(err[name], float(np.abs(got - ref).max()))
            ref_max[name] = max(ref_max[name], float(np.abs(ref).max()))
        del o_ref, s_ref
        _log(f"config {cfg_index} heads {hs.start}-{hs.stop - 1}: running max|err| "
             f"o {err['o']:.3e} S {err['S']:.3e}")
    for name in ("o", "S"):
        rel = err[name] / ref_max[name]
        _log(f"config {cfg_index} {name}: max|err|/max|ref| = {rel:.3e} over {N * H} chains")
        assert rel <= 2e-2, f"cfg{cfg_index} {name}: {rel:.3e} > 2e-02"


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_prefill_c3_long_context_full():
    """B=2, H=32, T=65,536, d=128, slow decay: all 64 (sequence, head) chains of 65,536
    tokens (1,024 chunks each) compared with the oracle."""
    _full_check(3, 8)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_prefill_c4_varlen_full():
    """64 packed sequences of 128-8,192 tokens, heads 0-7 per-channel gates, 8-15 scalar
    gates, S0 != 0: all 1,024 chains compared with the oracle."""
    _full_check(4, 8)


def _many_sequences(seed, N, H, max_len):
    """N packed sequences of 0..max_len tokens (a tenth of them empty)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len + 1, size=N)
    lens[rng.random(N) < 0.1] = 0
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    p = workloads.random_problem(rng, int(cu[-1]), H, 128, 128, io_dtype="bf16")
    p["cu_seqlens"] = cu
    s0 = (0.02 * rng.standard_normal((N, H, 128, 128))).astype(np.float32)
    return p, s0, rng


@pytest.mark.parametrize("N", [384, 385, 520])
def test_prefill_sequences_around_the_fused_header_limit(N):
    """384 sequences (the most for which the prep builds the sequence header itself) and
    more (the header then comes from its own launch); every chain is compared (ragged
    lengths, empty sequences, slots)."""
    p, s0, rng = _many_sequences(60 + N, N, 2, 130)
    cu = p["cu_seqlens"]
    _log(f"prefill N={N} T={cu[-1]} H=2 empty={(np.diff(cu) == 0).sum()}")
    pool = (0.02 * rng.standard_normal((N + 7, 2, 128, 128))).astype(np.float32)
    slots = rng.permutation(N + 7)[:N].astype(np.int32)
    pool[slots] = s0
    d_in = inputs_to_dev(p, "bf16")
    states = to_dev(pool, dtype=torch.float32)
    o = kda.kda_chunk_fwd(d_in["q"], d_in["k"], d_in["v"], d_in["g"], d_in["beta"],
                          d_in["cu_seqlens"], chunk=64, states=states,
                          state_slots=to_dev(slots, dtype=torch.int32), read_initial=True,
                          write_final=True)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], cu, s0=s0)
    assert_close(host(o), o_ref, "bf16", "o")
    got = host(states)
    assert_close(got[slots], s_ref, "bf16", "state")
    untouched = np.setdiff1d(np.arange(N + 7), slots)
    np.testing.assert_array_equal(got[untouched], pool[untouched])


@pytest.mark.parametrize("d,chunk,io", [(128, 64, torch.bfloat16), (32, 16, torch.float32)])
def test_prefill_every_sequence_empty(d, chunk, io):
    """total_tokens 0 with sequences given: each ends in the state it starts from (zero
    without one), so a final-state write alone zeroes the sequences' slots and every other
    flag setting leaves the pool as it was."""
    H, N = 2, 3
    z = torch.zeros((0, H, d), dtype=io, device="cuda")
    g = torch.zeros((0, H, d), device="cuda")
    beta = torch.zeros((0, H), device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    pool0 = torch.randn((5, H, d, d), device="cuda")
    for slots, used in [(torch.tensor([4, 0, 2], dtype=torch.int32, device="cuda"), [4, 0, 2]),
                        (None, [0, 1, 2])]:
        for read, write in [(False, True), (True, True), (True, False), (False, False)]:
            pool = pool0.clone()
            kda.kda_chunk_fwd(z, z, z, g, beta, cu, chunk=chunk, states=pool, state_slots=slots,
                              read_initial=read, write_final=write)
            torch.cuda.synchronize()
            want = pool0.clone()
            if write and not read:
                want[used] = 0
            assert torch.equal(pool, want), (slots is None, read, write)


@pytest.mark.parametrize("d,chunk,io", [(128, 64, "bf16"), (32, 16, "fp32")])
def test_prefill_empty_sequences_without_initial_state(d, chunk, io):
    """A final-state write without an initial state: the empty sequences' slots become zero
    (over a pool that held other values), the others hold the recurrence's final state."""
    rng = np.random.default_rng(d + chunk)
    lens, H = [0, chunk + 6, 0], 2
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    p = workloads.random_problem(rng, int(cu[-1]), H, d, d, io_dtype=io)
    p["cu_seqlens"] = cu
    pool = rng.standard_normal((len(lens), H, d, d)).astype(np.float32)
    o, s = _prefill(p, io, chunk, s0=pool, write=True)
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], cu)
    assert not s[0].any() and not s[2].any()
    assert_close(o, o_ref, io, "o")
    assert_close(s, s_ref, io, "state")
