"""The pins catch plausible mistakes.

A small numpy version of the recurrence is run through every pin in
``_pins``: unmodified it passes them all; each variant below carries one
plausible mistake (a dropped term, a wrong sign, a wrong side or order) and
must fail at least one pin.  The broken variants live only here, on the CPU.
"""
import numpy as np
import pytest

import _pins

MUTANTS = [
    "decay_on_value_side",     # retention scales value columns instead of key rows
    "read_before_write",       # o taken from the state before this token's write
    "predict_before_decay",    # p = S^T k computed on the undecayed state
    "beta_on_prediction_only", # u = v - beta p
    "error_sign",              # u = beta (v + p)
    "no_key_norm",             # k used unnormalised
    "no_query_norm",           # q used unnormalised
    "floor_ignored",           # lambda = log_alpha, no lower bound
    "floor_as_ceiling",        # lambda = min(log_alpha, floor)
    "gate_dropped",            # out = o
    "gate_on_input",           # out = o * g
    "readout_transposed",      # o = S q (wrong side of S)
    "decay_after_write",       # retention applied after the write
    "state0_ignored",          # initial state treated as zero
]


def make_runner(mut=None):
    def run(q, k, v, log_alpha, beta, g, log_alpha_min, state0):
        B, T, H, dk = k.shape
        dv = v.shape[-1]
        out = np.zeros((B, T, H, dv))
        Sf = np.zeros((B, H, dk, dv))
        for b in range(B):
            for h in range(H):
                S = np.zeros((dk, dv)) if (state0 is None or mut == "state0_ignored") else state0[b, h].copy()
                for t in range(T):
                    la = log_alpha[b, t, h]
                    lam = {"floor_ignored": la, "floor_as_ceiling": np.minimum(la, log_alpha_min)}.get(
                        mut, np.maximum(la, log_alpha_min))
                    a = np.exp(lam)
                    kk, qq = k[b, t, h], q[b, t, h]
                    kh = kk if mut == "no_key_norm" else kk / max(np.linalg.norm(kk), 1e-6)
                    qh = qq if mut == "no_query_norm" else qq / max(np.linalg.norm(qq), 1e-6)
                    Sold = S.copy()
                    if mut == "decay_on_value_side":
                        S = S * a[:dv][None, :] if dk >= dv else S * np.resize(a, dv)[None, :]
                    elif mut != "decay_after_write":
                        S = a[:, None] * S
                    p = (Sold if mut == "predict_before_decay" else S).T @ kh
                    bt = beta[b, t, h]
                    if mut == "beta_on_prediction_only":
                        u = v[b, t, h] - bt * p
                    elif mut == "error_sign":
                        u = bt * (v[b, t, h] + p)
                    else:
                        u = bt * (v[b, t, h] - p)
                    Spre = S
                    S = S + np.outer(kh, u)
                    if mut == "decay_after_write":
                        S = a[:, None] * S
                    if mut == "read_before_write":
                        o = Spre.T @ qh
                    elif mut == "readout_transposed":
                        o = (S @ np.resize(qh, dv))[:dv] if dk == dv else np.resize(S @ np.resize(qh, dv), dv)
                    else:
                        o = S.T @ qh
                    gt = g[b, t, h]
                    out[b, t, h] = {"gate_dropped": o, "gate_on_input": o * gt}.get(mut, o * _pins.sigmoid(gt))
                Sf[b, h] = S
        return out, Sf
    return run


def _errors(run):
    return {name: chk(run) for name, chk in _pins.ALL_CHECKS.items()}


def test_numpy_recurrence_passes_all_pins():
    errs = _errors(make_runner(None))
    assert max(errs.values()) < 1e-10, errs


@pytest.mark.parametrize("mut", MUTANTS)
def test_each_mutant_fails_a_pin(mut):
    errs = _errors(make_runner(mut))
    caught = [n for n, e in errs.items() if not (e < 1e-6)]
    assert caught, f"mutant {mut} passed every pin: {errs}"
