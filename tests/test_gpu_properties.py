"""The pages' properties and the method's edge cases, run on the HIP path
(needs an MI355X).

Each case feeds prefill (kda_chunk_prepare + kda_chunk_scan) and the decode
step (kda_decode_step, one token at a time) inputs that the generic
workloads never produce, and checks the GPU result twice:

* against the fp64 oracle on the same, already rounded inputs (relative L2
  per (batch row, head) slice: 1e-4 for fp32 I/O, 2e-2 for bf16 I/O with the
  fp32 state), and
* where the mathematics fixes the answer by itself, against that closed form
  (so a mistake shared by the oracle and the kernels would still fail).

The cases, and where they come from:
* pure decay -- beta = 0 switches the corrective write off, so the memory only
  fades row by row with the floored per-channel retention
  [zuoshipin.com/article/18261 §二; devpress.csdn.net K3 article §二,
  channel-wise retention];
* orthonormal retrieval -- no forgetting (alpha = 1), full-strength writes
  (beta = 1) and d_k orthonormal keys: each stored value comes back exactly
  through its key, whatever the initial memory [devpress §二: predict, take
  the error, write the correction];
* read after write -- beta = 1 and a query along the token's own key return
  exactly the value just written, for any history and retention (the order
  decay -> predict -> write -> read);
* non-unit and zero q/k -- per-token scales from 0.1 to 10, an all-zero key
  row, an all-zero query row, and rows below the 1e-6 normaliser floor (the
  epsilon branch) [zuoshipin §四, FlashKDA paragraph: q/k normalisation];
* the lowest floor the library accepts, log_alpha_min = -80/64 = -1.25, with
  most channels floored, forward and backward [zuoshipin §二: the lower bound
  keeps the parallel form inside bf16 range];
* NaN log-decay -- the maximum with the floor returns the floor, on both sides.
"""
import sys

import numpy as np
import pytest

import oracle
from kda_inputs import f32_to_bf16_bits, to_f64

torch = pytest.importorskip("torch")
import gated_delta_rule_91_amd as kda

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda"
LOG09 = float(np.float32(np.log(0.9)))


def note(*a):
    print(*a, file=sys.stderr, flush=True)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b.ravel())
    d = np.linalg.norm((a - b).ravel())
    return float(d / n) if n > 0 else float(d)


def slice_err(gpu, ref, token_major):
    """max relative L2 over (b, h) slices of [B,T,H,d] (token_major) or [B,H,dk,dv]."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    if token_major:
        gpu, ref = gpu.transpose(0, 2, 1, 3), ref.transpose(0, 2, 1, 3)
    return max(rel(gpu[b, h], ref[b, h]) for b in range(ref.shape[0]) for h in range(ref.shape[1]))


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def unit(x):
    return x / np.maximum(np.linalg.norm(x, axis=-1, keepdims=True), 1e-6)


class Case:
    """Inputs of one case: fp64 values exactly representable in the I/O dtype
    (what both sides see), the device tensors made from them, and runners."""

    def __init__(self, io, q, k, v, g, log_alpha, beta, floor, state0=None):
        self.io, self.floor = io, float(floor)

        def rnd(x):
            if io == "bf16":
                bits = f32_to_bf16_bits(np.asarray(x, np.float64).astype(np.float32))
                return bits, to_f64(bits, "bf16")
            a = np.asarray(x, np.float64).astype(np.float32)
            return a, a.astype(np.float64)

        def dev_io(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
            return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)

        (qs, self.q), (ks, self.k), (vs, self.v), (gs, self.g) = rnd(q), rnd(k), rnd(v), rnd(g)
        self.log_alpha = np.asarray(log_alpha, np.float32)
        self.beta = np.asarray(beta, np.float32)
        self.state0 = None if state0 is None else np.asarray(state0, np.float32)
        self.d = dict(q=dev_io(qs), k=dev_io(ks), v=dev_io(vs), g=dev_io(gs),
                      log_alpha=torch.from_numpy(np.ascontiguousarray(self.log_alpha)).to(DEV),
                      beta=torch.from_numpy(np.ascontiguousarray(self.beta)).to(DEV),
                      state0=None if state0 is None else torch.from_numpy(self.state0).to(DEV))

    def oracle(self):
        return oracle.kda_ref(self.q, self.k, self.v, self.log_alpha, self.beta, self.g, self.floor, self.state0)

    def prefill(self):
        d = self.d
        out, st = kda.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["g"], self.floor,
                              state_in=d["state0"])
        torch.cuda.synchronize()
        return host(out), host(st)

    def decode(self):
        """T decode steps from state0 (zeros if none); returns (out [B,T,H,dv], state)."""
        d = self.d
        B, T, H, dk = d["q"].shape
        dv = d["v"].shape[-1]
        sm = {n: d[n].transpose(0, 1).contiguous() for n in ("q", "k", "v", "g", "log_alpha", "beta")}
        state = d["state0"].clone() if d["state0"] is not None else torch.zeros(B, H, dk, dv, device=DEV)
        outs = [kda.decode_step(sm["q"][t], sm["k"][t], sm["v"][t], sm["log_alpha"][t], sm["beta"][t],
                                sm["g"][t], state, self.floor) for t in range(T)]
        torch.cuda.synchronize()
        out = torch.stack(outs, 1) if outs else torch.empty(B, 0, H, dv, device=DEV)
        return host(out), host(state)


def host(x):
    return x.float().cpu().numpy().astype(np.float64)


def check_vs_oracle(case, out, st, what):
    o_ref, s_ref = case.oracle()
    eo, es = slice_err(out, o_ref, True), slice_err(st, s_ref, False)
    note(f"  {what} vs oracle: out {eo:.2e} state {es:.2e}")
    assert eo <= TOL[case.io] and es <= TOL[case.io], (what, eo, es)
    return o_ref, s_ref


MODES = ("prefill", "decode")
SHAPES = [("f32", 64), ("f32", 128), ("bf16", 128), ("bf16", 64)]


def run(case, mode):
    return case.prefill() if mode == "prefill" else case.decode()


# ----------------------------------------------------------------- pure decay
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("io,d", SHAPES)
def test_pure_decay(io, d, mode):
    """beta = 0: S_T = diag(exp(sum_t max(log_alpha_t, floor))) S_0 on a random
    S_0, and o_t = (S_t^T q^_t) sigmoid(g_t); about half of the channels sit
    under the floor."""
    B, T, H = 2, 200, 3
    r = np.random.default_rng(1000 + d)
    q = r.standard_normal((B, T, H, d))
    k = r.standard_normal((B, T, H, d))
    v = r.standard_normal((B, T, H, d))
    g = r.standard_normal((B, T, H, d))
    la = -np.logaddexp(0.0, r.standard_normal((B, T, H, d)) + 1.0)
    s0 = r.standard_normal((B, H, d, d)) / np.sqrt(d)
    c = Case(io, q, k, v, g, la, np.zeros((B, T, H)), LOG09, s0)
    note(f"[pure decay] {mode} {io} d={d}")
    out, st = run(c, mode)
    check_vs_oracle(c, out, st, mode)
    lam = np.maximum(c.log_alpha.astype(np.float64), c.floor)
    cum = np.cumsum(lam, axis=1)                                    # [B,T,H,dk]
    St = np.exp(cum)[..., None] * c.state0.astype(np.float64)[:, None]   # [B,T,H,dk,dv]
    o = np.einsum("bthkv,bthk->bthv", St, unit(c.q)) * sigmoid(c.g)
    es, eo = slice_err(st, St[:, -1], False), slice_err(out, o, True)
    note(f"  vs closed form: out {eo:.2e} state {es:.2e}")
    assert es <= TOL[io] and eo <= TOL[io]


# ------------------------------------------------------- orthonormal retrieval
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("io,d", SHAPES)
def test_orthonormal_retrieval(io, d, mode):
    """alpha = 1, beta = 1, the d keys of a random orthonormal basis (each
    token's key scaled by 0.5..2 to exercise the normaliser), a random S_0:
    afterwards S^T k^_j = v_j for every j.  The closed form holds exactly for
    exactly orthonormal keys, so it is checked at the fp32 bound on fp32 I/O;
    bf16 keys are orthonormal only to their rounding, so there the HIP path
    is held to the oracle on the same keys."""
    B, H = 1, 2
    T = d
    r = np.random.default_rng(2000 + d)
    k = np.empty((B, T, H, d))
    for h in range(H):
        Qm, _ = np.linalg.qr(r.standard_normal((d, d)))
        k[0, :, h] = Qm * r.uniform(0.5, 2.0, (T, 1))
    q = r.standard_normal((B, T, H, d))
    v = r.standard_normal((B, T, H, d))
    g = r.standard_normal((B, T, H, d))
    s0 = r.standard_normal((B, H, d, d)) / np.sqrt(d)
    c = Case(io, q, k, v, g, np.zeros((B, T, H, d)), np.ones((B, T, H)), LOG09, s0)
    note(f"[orthonormal retrieval] {mode} {io} d={d}")
    out, st = run(c, mode)
    check_vs_oracle(c, out, st, mode)
    kh = unit(c.k)
    got = np.einsum("btk,bkv->btv", kh[0].transpose(1, 0, 2), st[0])   # [H,T,dv]: S_h^T k^_j
    err = rel(got, c.v[0].transpose(1, 0, 2))
    note(f"  retrieval vs the stored values: {err:.2e}")
    if io == "f32":
        assert err <= TOL["f32"]


# ---------------------------------------------------------- read after write
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("io,d", SHAPES)
def test_read_after_write(io, d, mode):
    """At scattered tokens beta = 1 and q = c k (c in {0.5, 2, 4}, exact in
    bf16): out_t = v_t * sigmoid(g_t) exactly, whatever came before (random
    beta, retention and initial memory elsewhere, a ragged last chunk)."""
    B, T, H = 2, 300, 2
    r = np.random.default_rng(3000 + d)
    q = r.standard_normal((B, T, H, d))
    k = r.standard_normal((B, T, H, d)) * r.uniform(0.3, 3.0, (B, T, H, 1))
    v = r.standard_normal((B, T, H, d))
    g = r.standard_normal((B, T, H, d))
    la = -np.logaddexp(0.0, r.standard_normal((B, T, H, d)) - 1.0)
    beta = r.uniform(0.0, 1.0, (B, T, H))
    pick = np.sort(r.choice(np.arange(1, T), size=24, replace=False))
    beta[:, pick] = 1.0
    q[:, pick] = k[:, pick] * r.choice([0.5, 2.0, 4.0], size=(1, len(pick), 1, 1))
    s0 = r.standard_normal((B, H, d, d)) / np.sqrt(d)
    c = Case(io, q, k, v, g, la, beta, LOG09, s0)
    note(f"[read after write] {mode} {io} d={d} ({len(pick)} tokens)")
    out, st = run(c, mode)
    check_vs_oracle(c, out, st, mode)
    exp = c.v[:, pick] * sigmoid(c.g[:, pick])
    err = rel(out[:, pick], exp)
    note(f"  o_t vs v_t sigmoid(g_t): {err:.2e}")
    assert err <= TOL[io]


# ------------------------------------------------------ non-unit and zero q/k
def _nonunit_case(io, d, T, seed, floor=LOG09, mu=-1.0):
    B, H = 2, 3
    r = np.random.default_rng(seed)
    scale = lambda: np.exp(r.uniform(np.log(0.1), np.log(10.0), (B, T, H, 1)))
    q = r.standard_normal((B, T, H, d)) * scale()
    k = r.standard_normal((B, T, H, d)) * scale()
    k[0, 5, 1] = 0.0                                   # all-zero key: nothing written
    q[0, 9, 0] = 0.0                                   # all-zero query: output 0
    k[1, 13, 2] = r.standard_normal(d) * 1e-9          # |k| ~ 1e-8 < 1e-6: k^ = k / 1e-6
    q[1, 17, 1] = r.standard_normal(d) * 1e-9          # the same for a query
    k[1, T - 1, 0] = 0.0                               # the last (ragged) token too
    v = r.standard_normal((B, T, H, d))
    g = r.standard_normal((B, T, H, d))
    la = -np.logaddexp(0.0, r.standard_normal((B, T, H, d)) + mu)
    beta = r.uniform(0.0, 1.0, (B, T, H))
    s0 = r.standard_normal((B, H, d, d)) / np.sqrt(d)
    return Case(io, q, k, v, g, la, beta, floor, s0)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("io,d", SHAPES)
def test_nonunit_and_zero_qk(io, d, mode):
    c = _nonunit_case(io, d, 150, 4000 + d)
    note(f"[non-unit and zero q/k] {mode} {io} d={d}")
    out, st = run(c, mode)
    o_ref, _ = check_vs_oracle(c, out, st, mode)
    assert np.all(out[0, 9, 0] == 0.0)                  # a zero query reads nothing
    # the epsilon branch: a key below the floor writes beta (k / 1e-6) u^T, a
    # small but nonzero amount -- the oracle's value at that token differs
    # from the unit-key value, and the GPU follows the oracle
    assert np.isfinite(out).all() and np.isfinite(st).all()


# -------------------------------------------------------------- lowest floor
LOWEST_FLOOR = -80.0 / 64.0   # -1.25, exactly representable


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("io,d", SHAPES)
def test_lowest_floor_mostly_floored(io, d, mode):
    """log_alpha_min = -1.25 (the lowest the library accepts): a chunk's
    decay then spans e^{-80}, and ~90% of the channels sit on the floor."""
    B, T, H = 2, 200, 3
    r = np.random.default_rng(5000 + d)
    q = r.standard_normal((B, T, H, d))
    k = r.standard_normal((B, T, H, d)) * r.uniform(0.5, 2.0, (B, T, H, 1))
    v = r.standard_normal((B, T, H, d))
    g = r.standard_normal((B, T, H, d))
    la = -np.logaddexp(0.0, r.standard_normal((B, T, H, d)) + 2.5)
    beta = r.uniform(0.0, 1.0, (B, T, H))
    s0 = r.standard_normal((B, H, d, d)) / np.sqrt(d)
    c = Case(io, q, k, v, g, la, beta, LOWEST_FLOOR, s0)
    frac = float(np.mean(c.log_alpha <= LOWEST_FLOOR))
    note(f"[floor -1.25] {mode} {io} d={d}: {frac:.0%} of channels floored")
    assert frac > 0.8
    out, st = run(c, mode)
    check_vs_oracle(c, out, st, mode)
    assert np.isfinite(out).all() and np.isfinite(st).all()


def test_lowest_floor_long_bf16_prefill():
    """The same floor over 1,000 tokens (16 chunk hand-offs) at d = 128."""
    B, T, H, d = 1, 1000, 4, 128
    r = np.random.default_rng(5100)
    c = Case("bf16", r.standard_normal((B, T, H, d)), r.standard_normal((B, T, H, d)),
             r.standard_normal((B, T, H, d)), r.standard_normal((B, T, H, d)),
             -np.logaddexp(0.0, r.standard_normal((B, T, H, d)) + 2.5), r.uniform(0.0, 1.0, (B, T, H)),
             LOWEST_FLOOR)
    note("[floor -1.25] long bf16 prefill")
    out, st = c.prefill()
    check_vs_oracle(c, out, st, "prefill")


@pytest.mark.parametrize("io,d", [("f32", 64), ("bf16", 128), ("f32", 128)])
def test_lowest_floor_backward(io, d):
    """Backward at the lowest floor with non-unit q/k: every gradient against
    the fp64 adjoint, and dlog_alpha exactly zero wherever the floor binds."""
    B, T, H = 1, 150, 2
    r = np.random.default_rng(5200 + d)
    c = Case(io, r.standard_normal((B, T, H, d)) * r.uniform(0.2, 5.0, (B, T, H, 1)),
             r.standard_normal((B, T, H, d)) * r.uniform(0.2, 5.0, (B, T, H, 1)),
             r.standard_normal((B, T, H, d)), r.standard_normal((B, T, H, d)),
             -np.logaddexp(0.0, r.standard_normal((B, T, H, d)) + 2.5), r.uniform(0.0, 1.0, (B, T, H)),
             LOWEST_FLOOR, r.standard_normal((B, H, d, d)) / np.sqrt(d))
    d_out64 = r.standard_normal((B, T, H, d))
    d_state = r.standard_normal((B, H, d, d)).astype(np.float32)
    if io == "bf16":
        bits = f32_to_bf16_bits(d_out64.astype(np.float32))
        d_out_dev = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
        d_out64 = to_f64(bits, "bf16")
    else:
        d_out_dev = torch.from_numpy(d_out64.astype(np.float32)).to(DEV)
        d_out64 = d_out64.astype(np.float32).astype(np.float64)
    note(f"[floor -1.25] backward {io} d={d}")
    dd = c.d
    gr = kda.backward(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"], dd["g"], c.floor,
                      state_in=dd["state0"], d_out=d_out_dev, d_state=torch.from_numpy(d_state).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.kda_grad(c.q, c.k, c.v, c.log_alpha, c.beta, c.g, c.floor, c.state0, d_out=d_out64,
                          d_state=d_state)
    for n in ("dq", "dk", "dv", "dg", "dlog_alpha"):
        e = slice_err(host(gr[n]), ref[n], True)
        note(f"  {n} {e:.2e}")
        assert e <= TOL[io], (n, e)
    e = rel(host(gr["dbeta"]), ref["dbeta"])
    es = slice_err(host(gr["dstate0"]), ref["dstate0"], False)
    note(f"  dbeta {e:.2e} dstate0 {es:.2e}")
    assert e <= TOL[io] and es <= TOL[io]
    floored = c.log_alpha <= LOWEST_FLOOR
    assert np.all(host(gr["dlog_alpha"])[floored] == 0.0)


# ------------------------------------------------------------ NaN log-decay
@pytest.mark.parametrize("mode", MODES)
def test_nan_log_alpha_acts_as_the_floor(mode):
    """max(NaN, floor) is the floor on the HIP path and in the oracle: NaN
    entries of log_alpha give bit-identical results to the floor itself."""
    B, T, H, d = 1, 130, 2, 128
    r = np.random.default_rng(6000)
    base = [r.standard_normal((B, T, H, d)) for _ in range(4)]
    la = -np.logaddexp(0.0, r.standard_normal((B, T, H, d)) - 2.0)
    beta = r.uniform(0.0, 1.0, (B, T, H))
    mask = r.uniform(size=la.shape) < 0.05
    la_nan, la_floor = la.copy(), la.copy()
    la_nan[mask] = np.nan
    la_floor[mask] = LOG09
    c1 = Case("bf16", *base, la_nan, beta, LOG09)
    c2 = Case("bf16", *base, la_floor, beta, LOG09)
    note(f"[NaN log_alpha] {mode}: {mask.sum()} NaN entries")
    o1, s1 = run(c1, mode)
    o2, s2 = run(c2, mode)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    check_vs_oracle(c1, o1, s1, mode)
