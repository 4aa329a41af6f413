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
