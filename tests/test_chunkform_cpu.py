"""The chunkwise-parallel algebra the GPU prefill uses equals the recurrence (CPU).

The pages say the chunked form is a re-ordering of the sequential rule, not an
approximation (engineermaxxing "From GPT-2 to Kimi K3", ch. 04e-04f).  These
tests check that claim for the gated, per-channel form on the fp64 mirror in
tests/chunkform_np.py, against the oracle, for several chunk sizes, ragged
tails, packed sequences, initial states and strong decay.
"""
import numpy as np
import pytest

import oracle
from gated_delta_rule_08_amd import workloads
from tests.chunkform_np import chunk_forward


@pytest.mark.parametrize("C", [1, 2, 16, 64])
@pytest.mark.parametrize("T", [64, 70, 130])
def test_chunk_form_equals_recurrence(C, T):
    rng = np.random.default_rng(100 + C + T)
    p = workloads.random_problem(rng, T, 2, 16, 12)
    s0 = rng.standard_normal((1, 2, 16, 12)) * 0.1
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], s0=s0)
    o, s = chunk_forward(p["q"], p["k"], p["v"], p["g"], p["beta"], C, s0=s0)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(s, s_ref, rtol=1e-10, atol=1e-11)


def test_chunk_form_packed_and_strong_decay():
    rng = np.random.default_rng(7)
    lens = [3, 64, 65, 0, 1, 100]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    p = workloads.random_problem(rng, int(cu[-1]), 3, 8, 8, alpha_mu=-1.0, g_scale=3.0)
    p["g"][10:12] = -30.0   # a wipe inside a chunk
    s0 = rng.standard_normal((len(lens), 3, 8, 8))
    o_ref, s_ref = oracle.run(p["q"], p["k"], p["v"], p["g"], p["beta"], cu, s0=s0)
    o, s = chunk_forward(p["q"], p["k"], p["v"], p["g"], p["beta"], 16, cu, s0=s0)
    np.testing.assert_allclose(o, o_ref, rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(s, s_ref, rtol=1e-9, atol=1e-10)


@pytest.mark.parametrize("C,T", [(16, 16), (16, 70), (64, 130), (4, 9)])
def test_chunk_backward_equals_recurrence_gradients(C, T):
    """The chunked gradient algebra (what the GPU backward computes) equals the
    oracle's token-by-token reverse-mode gradients."""
    from tests.chunkform_np import chunk_backward_head
    rng = np.random.default_rng(300 + C + T)
    H, dk, dv = 2, 16, 12
    p = workloads.random_problem(rng, T, H, dk, dv, alpha_mu=1.0, g_scale=2.0)
    s0 = rng.standard_normal((1, H, dk, dv)) * 0.1
    do = rng.standard_normal((T, H, dv))
    dsf = rng.standard_normal((1, H, dk, dv))
    ref = oracle.run_bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], do, s0=s0, ds_final=dsf)
    for h in range(H):
        dq, dk_, dv_, dg, db, ds0 = chunk_backward_head(
            p["q"][:, h], p["k"][:, h], p["v"][:, h], p["g"][:, h], p["beta"][:, h], C, do[:, h],
            s0[0, h], dsf[0, h])
        for name, x in (("dq", dq), ("dk", dk_), ("dv", dv_), ("dg", dg), ("dbeta", db)):
            np.testing.assert_allclose(x, ref[name][:, h], rtol=1e-8, atol=1e-9, err_msg=name)
        np.testing.assert_allclose(ds0, ref["ds0"][0, h], rtol=1e-8, atol=1e-9)
