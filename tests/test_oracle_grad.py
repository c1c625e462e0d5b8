"""Pins for the oracle's gradients (the fp64 adjoint of the step recurrence).

The adjoint is checked against the forward recurrence itself by central
finite differences of L = <d_out, out> + <d_state, S_T>: a dropped term, a
wrong sign or a transposed index in any step changes some gradient entry.
Plus exact special cases (zero seeds, beta = 0, T = 0) and linearity.
"""
import numpy as np
import pytest

import oracle

FLOOR = float(np.log(0.9))


def _problem(B, T, H, dk, dv, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g = rng.standard_normal((B, T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    # log-decays well inside (-0.06) or well below (-0.5) the floor, so a
    # finite-difference step never crosses it
    la = np.where(rng.random((B, T, H, dk)) < 0.3, -0.5, -0.03 + 0.02 * rng.standard_normal((B, T, H, dk)))
    s0 = rng.standard_normal((B, H, dk, dv)) * 0.5
    d_out = rng.standard_normal((B, T, H, dv))
    d_state = rng.standard_normal((B, H, dk, dv))
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta, g=g, state0=s0), d_out, d_state


NAMES = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_alpha", "dlog_alpha"), ("beta", "dbeta"), ("g", "dg"),
         ("state0", "dstate0")]


def _loss(x, d_out, d_state):
    out, st = oracle.kda_ref(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["g"], FLOOR, x["state0"],
                             nthreads=1)
    return float(np.sum(out * d_out) + np.sum(st * d_state))


def _grad(x, d_out, d_state):
    return oracle.kda_grad(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["g"], FLOOR, x["state0"],
                           d_out=d_out, d_state=d_state, nthreads=1)


@pytest.mark.parametrize("seed", [1, 2])
def test_grad_matches_directional_finite_differences(seed):
    x, d_out, d_state = _problem(2, 7, 2, 4, 3, seed)
    gr = _grad(x, d_out, d_state)
    rng = np.random.default_rng(100 + seed)
    h = 1e-6
    for name, gname in NAMES:
        for _ in range(3):
            d = rng.standard_normal(x[name].shape)
            xp = dict(x, **{name: x[name] + h * d})
            xm = dict(x, **{name: x[name] - h * d})
            fd = (_loss(xp, d_out, d_state) - _loss(xm, d_out, d_state)) / (2 * h)
            an = float(np.sum(gr[gname] * d))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


def test_grad_every_coordinate_by_finite_differences():
    """Brute force on a tiny problem: each gradient entry against its own
    central difference."""
    x, d_out, d_state = _problem(1, 3, 1, 3, 2, 7)
    gr = _grad(x, d_out, d_state)
    h = 1e-6
    for name, gname in NAMES:
        flat = x[name].reshape(-1)
        for i in range(flat.size):
            e = np.zeros_like(flat)
            e[i] = h
            xp = dict(x, **{name: (flat + e).reshape(x[name].shape)})
            xm = dict(x, **{name: (flat - e).reshape(x[name].shape)})
            fd = (_loss(xp, d_out, d_state) - _loss(xm, d_out, d_state)) / (2 * h)
            an = gr[gname].reshape(-1)[i]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, i, fd, an)


def test_floored_channels_get_no_decay_gradient():
    x, d_out, d_state = _problem(1, 5, 2, 4, 3, 3)
    gr = _grad(x, d_out, d_state)
    floored = x["log_alpha"] <= FLOOR
    assert floored.any()
    assert np.all(gr["dlog_alpha"][floored] == 0.0)
    assert np.any(gr["dlog_alpha"][~floored] != 0.0)


def test_grad_special_cases():
    x, d_out, d_state = _problem(2, 6, 2, 4, 3, 5)
    # zero seeds: zero gradients
    z = _grad(x, np.zeros_like(d_out), np.zeros_like(d_state))
    assert all(np.all(z[g] == 0.0) for _, g in NAMES)
    # linear in the seeds
    g1, g2 = _grad(x, d_out, d_state), _grad(x, 2.5 * d_out, 2.5 * d_state)
    for _, g in NAMES:
        assert np.allclose(g2[g], 2.5 * g1[g], rtol=1e-12, atol=1e-14)
    # beta = 0: no write ever happens, so v cannot matter
    x0 = dict(x, beta=np.zeros_like(x["beta"]))
    assert np.all(_grad(x0, d_out, d_state)["dv"] == 0.0)
    # an empty sequence passes the state seed straight through
    xe = {n: (a[:, :0] if n != "state0" else a) for n, a in x.items()}
    ge = _grad(xe, d_out[:, :0], d_state)
    assert np.array_equal(ge["dstate0"], d_state)


# ---------------------------------------------------------------------------
# Pin strength: a small numpy adjoint, unmodified and with one plausible
# mistake each, run through the directional finite-difference check.  The
# broken variants live only here, on the CPU.

GRAD_MUTANTS = [
    "no_norm_backprop",      # dk = dk^ (normalisation's Jacobian dropped)
    "dp_sign",               # dp = +beta du
    "dkh_misses_prediction", # dk^ without the S' dp term
    "decay_grad_on_prev",    # dlambda from the undecayed state
    "prev_grad_undecayed",   # dS_prev = dS' (retention factor dropped)
    "gate_grad_plain",       # dg = d_out * o (sigmoid' dropped)
    "readout_grad_pre_write",# do flows into the state before the write
    "beta_grad_sign",        # dbeta = du . (p - v)
]


def _numpy_grad(x, d_out, d_state, mut=None):
    q, k, v, la, bt, g, s0 = (x[n] for n in ("q", "k", "v", "log_alpha", "beta", "g", "state0"))
    B, T, H, dk = k.shape
    r = {gn: np.zeros_like(x[n]) for n, gn in NAMES}
    for b in range(B):
        for h in range(H):
            S = s0[b, h].copy()
            hist = []
            for t in range(T):
                hist.append(S.copy())
                S = np.exp(np.maximum(la[b, t, h], FLOOR))[:, None] * S
                kh = k[b, t, h] / max(np.linalg.norm(k[b, t, h]), 1e-6)
                u = bt[b, t, h] * (v[b, t, h] - S.T @ kh)
                S = S + np.outer(kh, u)
            dS = d_state[b, h].copy()
            for t in range(T - 1, -1, -1):
                Sprev = hist[t]
                lam = np.maximum(la[b, t, h], FLOOR)
                D = np.exp(lam)
                Sp = D[:, None] * Sprev
                nk, nq = np.linalg.norm(k[b, t, h]), np.linalg.norm(q[b, t, h])
                kh, qh = k[b, t, h] / nk, q[b, t, h] / nq
                p = Sp.T @ kh
                u = bt[b, t, h] * (v[b, t, h] - p)
                St = Sp + np.outer(kh, u)
                o = St.T @ qh
                sg = 1.0 / (1.0 + np.exp(-g[b, t, h]))
                dy = d_out[b, t, h]
                do = dy * sg
                r["dg"][b, t, h] = dy * o if mut == "gate_grad_plain" else dy * o * sg * (1 - sg)
                dqh = St @ do
                if mut != "readout_grad_pre_write":
                    dS = dS + np.outer(qh, do)
                du = dS.T @ kh
                r["dbeta"][b, t, h] = du @ ((p - v[b, t, h]) if mut == "beta_grad_sign" else (v[b, t, h] - p))
                r["dv"][b, t, h] = bt[b, t, h] * du
                dp = (1 if mut == "dp_sign" else -1) * bt[b, t, h] * du
                dkh = dS @ u + (0 if mut == "dkh_misses_prediction" else Sp @ dp)
                dSp = dS + np.outer(kh, dp)
                if mut == "readout_grad_pre_write":
                    dSp = dSp + np.outer(qh, do)
                dl = np.sum((Sprev if mut == "decay_grad_on_prev" else Sp) * dSp, axis=1)
                r["dlog_alpha"][b, t, h] = np.where(la[b, t, h] > FLOOR, dl, 0.0)
                dS = dSp if mut == "prev_grad_undecayed" else D[:, None] * dSp
                for xh, n_, dxh, key in ((kh, nk, dkh, "dk"), (qh, nq, dqh, "dq")):
                    r[key][b, t, h] = dxh if mut == "no_norm_backprop" else (dxh - xh * (xh @ dxh)) / n_
            r["dstate0"][b, h] = dS
    return r


def _fd_ok(grad_fn, seed=11):
    x, d_out, d_state = _problem(1, 5, 2, 4, 3, seed)
    gr = grad_fn(x, d_out, d_state)
    rng = np.random.default_rng(200 + seed)
    h = 1e-6
    for name, gname in NAMES:
        for _ in range(2):
            d = rng.standard_normal(x[name].shape)
            fd = (_loss(dict(x, **{name: x[name] + h * d}), d_out, d_state)
                  - _loss(dict(x, **{name: x[name] - h * d}), d_out, d_state)) / (2 * h)
            if abs(fd - float(np.sum(gr[gname] * d))) > 1e-6 * max(1.0, abs(fd)):
                return False
    return True


def test_numpy_adjoint_agrees_with_oracle_and_passes():
    x, d_out, d_state = _problem(2, 6, 2, 4, 3, 13)
    a, b = _numpy_grad(x, d_out, d_state), _grad(x, d_out, d_state)
    for _, g in NAMES:
        assert np.allclose(a[g], b[g], rtol=1e-10, atol=1e-12), g
    assert _fd_ok(_numpy_grad)


@pytest.mark.parametrize("mut", GRAD_MUTANTS)
def test_finite_difference_pin_catches(mut):
    assert not _fd_ok(lambda x, do, ds: _numpy_grad(x, do, ds, mut))
