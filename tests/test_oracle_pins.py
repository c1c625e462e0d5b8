"""The fp64 oracle pinned to things other than itself (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
import _pins
from _pins import rel, rand_case, sigmoid

TOL = 1e-11
HERE = os.path.dirname(os.path.abspath(__file__))


def run_oracle(q, k, v, log_alpha, beta, g, log_alpha_min, state0):
    return oracle.kda_ref(q, k, v, log_alpha, beta, g, log_alpha_min, state0, nthreads=4)


@pytest.mark.parametrize("name", sorted(_pins.ALL_CHECKS))
def test_oracle_pin(name):
    err = _pins.ALL_CHECKS[name](run_oracle)
    assert err < TOL, f"{name}: rel err {err:.3e}"


def test_golden_hand_examples():
    """Tiny cases worked out by hand in exact arithmetic (tests/golden/hand_examples.json)."""
    with open(os.path.join(HERE, "golden", "hand_examples.json")) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 3
    for c in cases:
        arr = lambda x: np.asarray(x, np.float64)
        T, dk, dv = len(c["k"]), len(c["k"][0]), len(c["v"][0])
        shp = lambda x, d: arr(x).reshape(1, T, 1, d)
        s0 = None if c.get("state0") is None else arr(c["state0"]).reshape(1, 1, dk, dv)
        out, S = oracle.kda_ref(shp(c["q"], dk), shp(c["k"], dk), shp(c["v"], dv), shp(c["log_alpha"], dk),
                                arr(c["beta"]).reshape(1, T, 1), shp(c["g"], dv), c["log_alpha_min"], s0)
        np.testing.assert_allclose(out[0, :, 0], arr(c["out"]), rtol=1e-12, atol=1e-12, err_msg=c["name"])
        np.testing.assert_allclose(S[0, 0], arr(c["state"]), rtol=1e-12, atol=1e-12, err_msg=c["name"])


def _case_long_decay(seed, B, T, H, dk, dv):
    c = rand_case(seed, B=B, T=T, H=H, dk=dk, dv=dv, mu=-4.0)   # slow forgetting: A stays far from 0
    return c


@pytest.mark.parametrize("T1,T2", [(16, 16), (7, 13), (1, 5)])
def test_summary_combine_equals_concatenation(T1, T2):
    """(A2, B2) o (A1, B1) applied to S0 == the run over seg1 || seg2 from S0."""
    c = _case_long_decay(21 + T1, B=1, T=T1 + T2, H=2, dk=8, dv=6)
    _, S = run_oracle(**c)
    ks = lambda n, sl: c[n][:, sl]
    s1, s2 = slice(0, T1), slice(T1, T1 + T2)
    A1, B1 = oracle.kda_summary(ks("k", s1), ks("v", s1), ks("log_alpha", s1), ks("beta", s1), c["log_alpha_min"])
    A2, B2 = oracle.kda_summary(ks("k", s2), ks("v", s2), ks("log_alpha", s2), ks("beta", s2), c["log_alpha_min"])
    assert np.linalg.norm(A1[0, 0] - np.eye(8)) > 1e-3 and np.linalg.norm(A1[0, 0]) > 0.5   # not vacuous
    S_direct = np.einsum("bhik,bhkj->bhij", A2, np.einsum("bhik,bhkj->bhij", A1, c["state0"]) + B1) + B2
    assert rel(S_direct, S) < TOL
    # the oracle's own in-order merge gives the same segment-entry states
    A = np.stack([A1, A2], 1)
    Bz = np.stack([B1, B2], 1)
    seg_in, fin = oracle.kda_combine(A, Bz, c["state0"])
    assert rel(seg_in[:, 0], c["state0"]) == 0.0
    assert rel(seg_in[:, 1], np.einsum("bhik,bhkj->bhij", A1, c["state0"]) + B1) < TOL
    assert rel(fin, S) < TOL


def test_summary_pair_definition():
    """Bz is the run from an empty memory; A is the run of the homogeneous map on I."""
    c = _case_long_decay(31, B=2, T=11, H=2, dk=6, dv=5)
    A, Bz = oracle.kda_summary(c["k"], c["v"], c["log_alpha"], c["beta"], c["log_alpha_min"])
    _, S_zero = run_oracle(**dict(c, state0=None))
    assert rel(Bz, S_zero) < TOL
    # S_end = A S_start + Bz for two unrelated start states
    for s in (c["state0"], np.random.default_rng(5).standard_normal(c["state0"].shape)):
        _, S = run_oracle(**dict(c, state0=s))
        assert rel(np.einsum("bhik,bhkj->bhij", A, s) + Bz, S) < TOL


def test_contraction():
    """beta in [0,1], unit keys, retention <= 1 => every transition has ||A||_2 <= 1."""
    c = rand_case(41, B=3, T=40, H=2, dk=8, dv=4, mu=-3.0)
    A, _ = oracle.kda_summary(c["k"], c["v"], c["log_alpha"], c["beta"], c["log_alpha_min"])
    norms = np.linalg.norm(A.reshape(-1, 8, 8), ord=2, axis=(1, 2))
    assert norms.max() <= 1.0 + 1e-12
    assert norms.min() > 1e-3          # not vacuous


def test_empty_sequence_passes_state_through():
    c = rand_case(51, B=2, T=0, H=2, dk=8, dv=4)
    out, S = run_oracle(**c)
    assert out.shape == (2, 0, 2, 4)
    assert np.array_equal(S, c["state0"])


def test_floor_is_applied_and_idempotent():
    """Values under the floor act exactly as the floor; values above it are untouched."""
    c = rand_case(61, B=1, T=12, H=1, dk=8, dv=4, mu=2.0)
    floor = c["log_alpha_min"]
    assert (c["log_alpha"] < floor).mean() > 0.5
    o1, S1 = run_oracle(**c)
    c2 = dict(c, log_alpha=np.maximum(c["log_alpha"], floor))
    o2, S2 = run_oracle(**c2)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_threads_do_not_change_results():
    c = rand_case(71, B=2, T=30, H=3, dk=16, dv=16, mu=-2.0)
    o1, S1 = oracle.kda_ref(**c, nthreads=1)
    o8, S8 = oracle.kda_ref(**c, nthreads=8)
    assert np.array_equal(o1, o8) and np.array_equal(S1, S8)


def test_generator_is_deterministic_and_shaped():
    from kda_inputs import make_inputs, to_f64
    a = make_inputs(2, 300, 3, 64, 32, io_dtype="bf16", seed=7, alpha_min=0.9, logit_mu=-4.0, threads=1)
    b = make_inputs(2, 300, 3, 64, 32, io_dtype="bf16", seed=7, alpha_min=0.9, logit_mu=-4.0, threads=4)
    for n in ("q", "k", "v", "g", "log_alpha", "beta"):
        assert np.array_equal(getattr(a, n), getattr(b, n)), n
    q = to_f64(a.q, "bf16")
    nrm = np.linalg.norm(q, axis=-1)
    assert np.abs(nrm - 1).max() < 1e-2                     # unit up to bf16 rounding
    assert (a.log_alpha <= 0).all() and (a.beta > 0).all() and (a.beta < 1).all()
    c = make_inputs(2, 300, 3, 64, 32, io_dtype="bf16", seed=8, alpha_min=0.9, threads=1)
    assert not np.array_equal(a.q, c.q)
