"""Checks that pin a KDA recurrence implementation to what the pages and the
mathematics fix, independent of any implementation.

Every check takes a ``run`` callable with the oracle's calling convention

    run(q, k, v, log_alpha, beta, g, log_alpha_min, state0) -> (out, state)

(fp64 numpy arrays, token-major [B,T,H,d]; state [B,H,dk,dv]) and returns the
largest relative error it found.  ``test_oracle_pins`` applies them to the C
oracle; ``test_pin_strength`` applies them to deliberately broken variants to
show that each plausible mistake fails at least one of them.

What each check pins, and where it comes from on the pages:

* closed_form_t1 -- one token from an empty memory: the write stores
  beta * k^ v^T, and the gated read returns beta (q^.k^) v * sigmoid(g).
  Pins the write strength, the normalisation and the output gate
  [devpress.csdn.net K3 article §二 (write the corrected error);
  zuoshipin.com/article/18261 §二 (full-rank output gate)].
* pure_decay -- beta = 0 turns writing off, so the memory only fades, row by
  row per key channel, with the per-step floor: S_T = diag(exp(sum lambda)) S_0.
  Pins the channel-wise retention and its lower bound [zuoshipin §二;
  devpress §二, channel-wise retention paragraph].
* orthonormal_retrieval -- no forgetting, full-strength writes and orthonormal
  keys: every stored value is read back exactly through its key.  Pins the
  delta rule's "replace what the key used to return" [devpress §二].
* read_after_write -- a full-strength write (beta = 1) followed by a read
  with the same key returns exactly the value just written, whatever the
  history and the retention.  Pins the order decay -> predict -> write -> read.
* unrolled_product -- for T <= 16 the state is rebuilt from explicit d_k x d_k
  per-token transition matrices as a sum of products (no step loop).
* segment_combine / resume -- the context-parallel pair (A, Bz) composes to the
  run over the concatenation, and a run resumed from a saved state equals the
  uninterrupted run [zuoshipin §三, context-parallel paragraph; devpress §十四,
  state checkpoints at reusable boundaries].
* linearity / column_permutation / qk_scale -- (v, S_0) -> (o, S_T) is linear;
  value channels never mix; q and k enter only through their directions.
* contraction -- each per-token transition has spectral norm <= 1, so every
  segment transition A has ||A||_2 <= 1.
"""
from __future__ import annotations

import numpy as np

LOG09 = float(np.float32(np.log(0.9)))


def softplus(x):
    return np.logaddexp(0.0, x)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    d = np.linalg.norm((a - b).ravel())
    n = np.linalg.norm(b.ravel())
    return float(d / n) if n > 0 else float(d)


def rand_case(seed, B=1, T=8, H=1, dk=8, dv=8, mu=0.0, unit=False, s0=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, dk)) * r.uniform(0.5, 3.0, (B, T, H, 1))
    k = r.standard_normal((B, T, H, dk)) * r.uniform(0.5, 3.0, (B, T, H, 1))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, dv))
    g = r.standard_normal((B, T, H, dv))
    la = -softplus(r.standard_normal((B, T, H, dk)) + mu)
    beta = r.uniform(0.0, 1.0, (B, T, H))
    S0 = r.standard_normal((B, H, dk, dv)) if s0 else None
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta, g=g, log_alpha_min=LOG09, state0=S0)


def _unit(x):
    return x / np.maximum(np.linalg.norm(x, axis=-1, keepdims=True), 1e-6)


def closed_form_t1(run, seed=11, dk=8, dv=6):
    c = rand_case(seed, B=2, T=1, H=3, dk=dk, dv=dv, s0=False)
    out, S = run(**c)
    kh, qh = _unit(c["k"][:, 0]), _unit(c["q"][:, 0])               # [B,H,dk]
    b = c["beta"][:, 0]                                             # [B,H]
    S_exp = b[..., None, None] * kh[..., :, None] * c["v"][:, 0][..., None, :]
    o_exp = (b * np.sum(qh * kh, -1))[..., None] * c["v"][:, 0]
    out_exp = o_exp * sigmoid(c["g"][:, 0])
    return max(rel(S, S_exp), rel(out[:, 0], out_exp))


def pure_decay(run, seed=12, T=20, dk=8, dv=5):
    c = rand_case(seed, B=1, T=T, H=2, dk=dk, dv=dv, mu=1.0)       # many channels under the floor
    c["beta"][:] = 0.0
    out, S = run(**c)
    lam = np.maximum(c["log_alpha"], c["log_alpha_min"])            # [B,T,H,dk]
    cum = np.cumsum(lam, axis=1)
    St = np.exp(cum)[..., None] * c["state0"][:, None]              # [B,T,H,dk,dv]
    o = np.einsum("bthkv,bthk->bthv", St, _unit(c["q"]))
    return max(rel(S, St[:, -1]), rel(out, o * sigmoid(c["g"])))


def orthonormal_retrieval(run, seed=13, dk=8, dv=4, T=6):
    r = np.random.default_rng(seed)
    Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    c = rand_case(seed, B=1, T=T, H=1, dk=dk, dv=dv)
    c["k"][0, :, 0] = Qm[:T] * r.uniform(0.5, 2.0, (T, 1))
    c["log_alpha"][:] = 0.0
    c["beta"][:] = 1.0
    _, S = run(**c)
    kh = _unit(c["k"][0, :, 0])
    got = kh @ S[0, 0]                                              # row j = S^T k_j
    return rel(got, c["v"][0, :, 0])


def read_after_write(run, seed=14, T=24, dk=8, dv=6):
    c = rand_case(seed, B=1, T=T, H=2, dk=dk, dv=dv, mu=-1.0)
    r = np.random.default_rng(seed + 1)
    pick = np.sort(r.choice(np.arange(2, T), size=6, replace=False))
    c["beta"][:, pick] = 1.0
    c["q"][:, pick] = c["k"][:, pick] * 2.5
    out, _ = run(**c)
    exp = c["v"][:, pick] * sigmoid(c["g"][:, pick])
    return rel(out[:, pick], exp)


def unrolled_product(run, seed=15, T=16, dk=6, dv=5):
    c = rand_case(seed, B=1, T=T, H=2, dk=dk, dv=dv, mu=-1.0)
    out, S = run(**c)
    lam = np.maximum(c["log_alpha"], c["log_alpha_min"])
    kh, qh = _unit(c["k"]), _unit(c["q"])
    err = 0.0
    for h in range(2):
        Ms = []
        for t in range(T):
            kk = kh[0, t, h]
            Ms.append((np.eye(dk) - c["beta"][0, t, h] * np.outer(kk, kk)) @ np.diag(np.exp(lam[0, t, h])))
        for t in range(T):
            # S_t = (M_t ... M_1) S_0 + sum_{i<=t} (M_t ... M_{i+1}) beta_i k_i v_i^T
            P = np.eye(dk)
            St = np.zeros((dk, dv))
            for i in range(t, -1, -1):
                St += P @ (c["beta"][0, i, h] * np.outer(kh[0, i, h], c["v"][0, i, h]))
                P = P @ Ms[i]
            St += P @ c["state0"][0, h]
            o = St.T @ qh[0, t, h] * sigmoid(c["g"][0, t, h])
            err = max(err, rel(out[0, t, h], o))
        err = max(err, rel(S[0, h], St))
    return err


def resume(run, seed=16, T1=9, T2=7, dk=8, dv=6):
    c = rand_case(seed, B=2, T=T1 + T2, H=2, dk=dk, dv=dv, mu=-4.0)
    out, S = run(**c)
    a = {n: (x[:, :T1] if n not in ("state0", "log_alpha_min") else x) for n, x in c.items()}
    b = {n: (x[:, T1:] if n not in ("state0", "log_alpha_min") else x) for n, x in c.items()}
    out1, S1 = run(**a)
    b["state0"] = S1
    out2, S2 = run(**b)
    return max(rel(np.concatenate([out1, out2], 1), out), rel(S2, S))


def linearity(run, seed=17, T=12, dk=8, dv=6):
    c1 = rand_case(seed, B=1, T=T, H=2, dk=dk, dv=dv, mu=-1.0)
    c2 = dict(c1)
    r = np.random.default_rng(seed + 1)
    c2["v"] = r.standard_normal(c1["v"].shape)
    c2["state0"] = r.standard_normal(c1["state0"].shape)
    c1["g"][:] = 0.0   # gate sigmoid(0) = 1/2 is a constant factor
    c2["g"] = c1["g"]
    a, b = 1.7, -0.6
    c3 = dict(c1)
    c3["v"] = a * c1["v"] + b * c2["v"]
    c3["state0"] = a * c1["state0"] + b * c2["state0"]
    o1, S1 = run(**c1)
    o2, S2 = run(**c2)
    o3, S3 = run(**c3)
    return max(rel(o3, a * o1 + b * o2), rel(S3, a * S1 + b * S2))


def column_permutation(run, seed=18, T=10, dk=8, dv=7):
    c = rand_case(seed, B=1, T=T, H=1, dk=dk, dv=dv, mu=-1.0)
    perm = np.random.default_rng(seed).permutation(dv)
    o, S = run(**c)
    cp = dict(c)
    cp["v"], cp["g"], cp["state0"] = c["v"][..., perm], c["g"][..., perm], c["state0"][..., perm]
    op, Sp = run(**cp)
    return max(rel(op, o[..., perm]), rel(Sp, S[..., perm]))


def qk_scale(run, seed=19, T=10, dk=8, dv=6):
    c = rand_case(seed, B=1, T=T, H=2, dk=dk, dv=dv, mu=-1.0)
    o, S = run(**c)
    cs = dict(c)
    r = np.random.default_rng(seed)
    cs["q"] = c["q"] * r.uniform(0.1, 10.0, c["q"].shape[:-1] + (1,))
    cs["k"] = c["k"] * r.uniform(0.1, 10.0, c["k"].shape[:-1] + (1,))
    os_, Ss = run(**cs)
    return max(rel(os_, o), rel(Ss, S))


ALL_CHECKS = dict(closed_form_t1=closed_form_t1, pure_decay=pure_decay,
                  orthonormal_retrieval=orthonormal_retrieval, read_after_write=read_after_write,
                  unrolled_product=unrolled_product, resume=resume, linearity=linearity,
                  column_permutation=column_permutation, qk_scale=qk_scale)
