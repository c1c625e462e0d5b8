"""The chunk-parallel form the HIP kernels evaluate equals the step recurrence.

The pages describe the two-stage chunk method only in words
[zuoshipin.com/article/18261 §四, FlashKDA paragraph: per-chunk "update
cards" (forget gate, q/k normalisation, decay, intra-chunk correction matrix)
are prepared in parallel; only the state hand-off and the read-out run in
order].  The algebra below is this repository's derivation of that method
from the recurrence; this fp64 numpy version checks
it against the oracle before any kernel relies on it.  It is test code, not
part of the library, and shares nothing with the kernels.

Per chunk of C tokens, gamma = inclusive cumulative sum of the floored
log-retention over the chunk, per key channel:

    Qt = q^ e^gamma   Kt = k^ e^gamma   Kh = k^ e^-gamma   Ke = k^ e^(gamma_C - gamma)
    L  = strict_lower(Kt Kh^T)          P = lower_incl(Qt Kh^T)
    T  = (I + diag(beta) L)^-1          Wk = T diag(beta) Kt     Wv = T diag(beta) V
    -- ordered hand-off --
    U  = Wv - Wk S        O = Qt S + P U        S <- diag(e^gamma_C) S + Ke^T U
"""
import numpy as np
import pytest

import oracle
from _pins import rand_case, rel, sigmoid


def chunk_form(q, k, v, log_alpha, beta, g, log_alpha_min, state0, C):
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    nch = -(-T // C)
    Tp = nch * C
    pad = lambda x: np.concatenate([x, np.zeros((B, Tp - T) + x.shape[2:])], 1)
    lam = np.maximum(log_alpha, log_alpha_min)
    # padded tokens: beta = 0, lambda = 0, q = k = v = 0 -> exact identity steps
    q, k, v, g, lam, beta = map(pad, (q, k, v, g, lam, beta))
    kh = k / np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), 1e-6)
    qh = q / np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), 1e-6)
    out = np.zeros((B, Tp, H, dv))
    Sf = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if state0 is None else state0[b, h].copy()
            for n in range(nch):
                sl = slice(n * C, (n + 1) * C)
                gam = np.cumsum(lam[b, sl, h], axis=0)                   # [C, dk]
                Qt = qh[b, sl, h] * np.exp(gam)
                Kt = kh[b, sl, h] * np.exp(gam)
                Kh = kh[b, sl, h] * np.exp(-gam)
                Ke = kh[b, sl, h] * np.exp(gam[-1] - gam)
                L = np.tril(Kt @ Kh.T, -1)
                P = np.tril(Qt @ Kh.T, 0)
                bt = beta[b, sl, h]
                Tm = np.linalg.inv(np.eye(C) + bt[:, None] * L)
                Wk = Tm @ (bt[:, None] * Kt)
                Wv = Tm @ (bt[:, None] * v[b, sl, h])
                U = Wv - Wk @ S
                O = Qt @ S + P @ U
                S = np.exp(gam[-1])[:, None] * S + Ke.T @ U
                out[b, sl, h] = O * sigmoid(g[b, sl, h])
            Sf[b, h] = S
    return out[:, :T], Sf


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("T", [64, 150, 5])
def test_chunk_form_matches_recurrence(C, T):
    c = rand_case(100 + C + T, B=2, T=T, H=2, dk=16, dv=8, mu=-2.0)
    o_ref, S_ref = oracle.kda_ref(**c)
    o, S = chunk_form(**c, C=C)
    assert rel(o, o_ref) < 1e-12
    assert rel(S, S_ref) < 1e-12


def test_chunk_form_at_the_floor():
    """Every step at the retention floor (the largest e^-gamma the floor allows)."""
    c = rand_case(7, B=1, T=128, H=1, dk=32, dv=16, mu=3.0)
    assert (c["log_alpha"] < c["log_alpha_min"]).mean() > 0.9
    o_ref, S_ref = oracle.kda_ref(**c)
    o, S = chunk_form(**c, C=64)
    assert rel(o, o_ref) < 1e-11 and rel(S, S_ref) < 1e-11


def test_floor_bounds_the_decay_folding():
    """With the floor, e^{-gamma} over a 64-token chunk stays below e^{64 |log 0.9|} ~ 848."""
    assert np.exp(-64 * np.log(0.9)) < 850.0
    assert np.exp(-64 * np.log(0.9)) * 1.0 < np.finfo(np.float32).max
