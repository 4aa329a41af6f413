"""GPU parity of the segment decomposition of one sequence (context parallelism).

The state is everything one part of a sequence hands to the next (heqinghuang
"From GPT2 to Kimi3, Explained", section 10; engineermaxxing "From GPT-2 to
Kimi K3", ch. 04f), and every step of the recurrence is affine in it, so a
segment maps its incoming state S to M S + B.  M is the segment run with v = 0
from the identity, B the segment run from the zero state.  The test splits one
sequence into segments, computes every segment's (M, B) with kda_chunk_fwd in
one varlen call each (the segments are the batch), chains the maps with
kda_state_affine, re-runs every segment from its incoming state, and compares
the outputs and the final state with the oracle's single pass over the whole
sequence.  kda_state_affine alone is checked against an fp64 product.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_08_amd import workloads
from tests.gpu_util import assert_close, host, rel_err, to_dev

pytestmark = pytest.mark.gpu

kda = pytest.importorskip("gated_delta_rule_08_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kda.load_library()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("n,H,dk,dv", [(3, 2, 128, 128), (2, 3, 64, 32), (1, 1, 16, 48)])
def test_state_affine_matches_fp64(n, H, dk, dv):
    rng = np.random.default_rng(100 + dk + dv)
    M = rng.standard_normal((n, H, dk, dk)).astype(np.float32) / np.sqrt(dk)
    S = rng.standard_normal((n, H, dk, dv)).astype(np.float32)
    B = rng.standard_normal((n, H, dk, dv)).astype(np.float32)
    print(f"state affine n={n} H={H} dk={dk} dv={dv}", flush=True)
    ref = np.einsum("nhij,nhjc->nhic", M.astype(np.float64), S.astype(np.float64)) + B
    dM, dS, dB = (to_dev(a, dtype=torch.float32) for a in (M, S, B))
    out = kda.kda_state_affine(dM, dS, dB)
    torch.cuda.synchronize()
    assert rel_err(host(out), ref) <= 1e-5
    kda.kda_state_affine(dM, dS, dB, out=dB)          # in place over B
    torch.cuda.synchronize()
    assert rel_err(host(dB), ref) <= 1e-5


def _segment_run(p, bounds, io, s0, chunk):
    """Outputs and final state of the whole sequence, computed segment by segment."""
    P = len(bounds) - 1
    H, dk, dv = p["q"].shape[1], p["q"].shape[2], p["v"].shape[2]
    dev = lambda a: to_dev(a, io)
    q, k, v = dev(p["q"]), dev(p["k"]), dev(p["v"])
    g, beta = to_dev(p["g"], dtype=torch.float32), to_dev(p["beta"], dtype=torch.float32)
    cu = to_dev(np.asarray(bounds, dtype=np.int32), dtype=torch.int32)
    eye = torch.eye(dk, dtype=torch.float32, device="cuda")
    # (M, B) of every segment: the segments are the sequences of one varlen call.
    Ms = eye.expand(P, H, dk, dk).contiguous()
    kda.kda_chunk_fwd(q, k, torch.zeros_like(v), g, beta, cu, chunk=chunk, states=Ms,
                      read_initial=True, write_final=True)
    Bs = torch.zeros((P, H, dk, dv), dtype=torch.float32, device="cuda")
    kda.kda_chunk_fwd(q, k, v, g, beta, cu, chunk=chunk, states=Bs, write_final=True)
    # Exclusive scan of the maps: the incoming state of every segment.
    S_in = torch.empty((P, H, dk, dv), dtype=torch.float32, device="cuda")
    S_in[0] = to_dev(s0, dtype=torch.float32)
    for i in range(P - 1):
        kda.kda_state_affine(Ms[i:i + 1], S_in[i:i + 1], Bs[i:i + 1], out=S_in[i + 1:i + 2])
    states = S_in.clone()
    o = kda.kda_chunk_fwd(q, k, v, g, beta, cu, chunk=chunk, states=states,
                          read_initial=True, write_final=True)
    torch.cuda.synchronize()
    return host(o), host(states[P - 1])


@pytest.mark.parametrize("io,d,chunk,bounds", [
    ("bf16", 128, 64, [0, 256, 512, 768, 1024]),        # MFMA path, chunk-aligned segments
    ("bf16", 128, 64, [0, 200, 530, 531, 777, 1000]),   # ragged, a one-token segment
    ("fp32", 64, 16, [0, 40, 96, 160]),                 # fp32 path, 1e-4 contract
])
def test_segments_compose_to_the_single_pass(io, d, chunk, bounds):
    H = 4 if io == "bf16" else 2
    T = bounds[-1]
    rng = np.random.default_rng(31 + len(bounds))
    p = workloads.random_problem(rng, T, H, d, d, io_dtype=io)
    s0 = (0.02 * rng.standard_normal((H, d, d))).astype(np.float32)
    print(f"segments io={io} d={d} C={chunk} bounds={bounds} H={H}", flush=True)
    o, s = _segment_run(p, bounds, io, s0, chunk)
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"],
                              np.array([0, T], dtype=np.int32), s0=s0[None])
    assert_close(o, o_ref, io, "o (segments)")
    assert_close(s, s_ref[0], io, "final state (segments)")
