"""kda_backward (HIP) vs the fp64 oracle adjoint, element by element (needs an
MI355X).

Same inputs on both sides (bf16 -> fp64 is exact).  Error measure: relative
L2 per (batch row, head) slice of every gradient; the largest must stay
within 1e-4 for fp32 inputs and 2e-2 for bf16 inputs (there dq, dk, dv and dg
are rounded to bf16 on output, half an ulp = 2e-3 relative).  q and k are
scaled by 0.5 and 2 (exact in both dtypes) so the normalisation's 1/|x|
factor is exercised, and one key row is zero (the 1e-6 normaliser branch).
"""
import sys

import numpy as np
import pytest

import oracle
from kda_inputs import f32_to_bf16_bits, make_inputs, to_f64

torch = pytest.importorskip("torch")
import gated_delta_rule_91_amd as kda

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda"
TOKEN_GRADS = ("dq", "dk", "dv", "dg", "dlog_alpha", "dbeta")


def note(*a):
    print(*a, file=sys.stderr, flush=True)


def slice_err(gpu, ref, token_major=True):
    """max rel-L2 over (b, h) slices of [B,T,H,...] (or [B,H,...] states)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    if token_major:
        gpu, ref = np.moveaxis(gpu, 2, 1), np.moveaxis(ref, 2, 1)
    B, H = ref.shape[:2]
    worst = 0.0
    for b in range(B):
        for h in range(H):
            d = np.linalg.norm((gpu[b, h] - ref[b, h]).ravel())
            n = np.linalg.norm(ref[b, h].ravel())
            worst = max(worst, d / n if n > 0 else d)
    return worst


def _io(a64, io_dtype):
    """(array in the I/O dtype's storage, its exact fp64 value)."""
    if io_dtype == "bf16":
        bits = f32_to_bf16_bits(a64.astype(np.float32))
        return bits, to_f64(bits, "bf16")
    a = a64.astype(np.float32)
    return a, a.astype(np.float64)


def _dev(a, io_dtype):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _case(B, T, H, d, io_dtype, seed, *, state0=True, d_out=True, d_state=True, zero_key=True, alpha_min=0.9):
    inp = make_inputs(B, T, H, d, d, io_dtype=io_dtype, seed=seed, alpha_min=alpha_min, logit_mu=-1.0,
                      with_state0=state0)
    f = lambda a: to_f64(a, io_dtype)
    q64, k64 = f(inp.q) * 0.5, f(inp.k) * 2.0
    if zero_key and T > 5:
        k64[0, 5, 0, :] = 0.0
    rng = np.random.default_rng(seed + 1000)
    q_io, q64 = _io(q64, io_dtype)
    k_io, k64 = _io(k64, io_dtype)
    do_io, do64 = _io(rng.standard_normal((B, T, H, d)), io_dtype) if d_out else (None, None)
    ds = rng.standard_normal((B, H, d, d)).astype(np.float32) if d_state else None
    ref = oracle.kda_grad(q64, k64, f(inp.v), inp.log_alpha, inp.beta, f(inp.g), inp.log_alpha_min, inp.state0,
                          d_out=do64, d_state=ds)
    t = dict(q=_dev(q_io, io_dtype), k=_dev(k_io, io_dtype), v=_dev(inp.v, io_dtype), g=_dev(inp.g, io_dtype),
             log_alpha=_dev(inp.log_alpha, "f32"), beta=_dev(inp.beta, "f32"))
    note(f"[backward] B={B} T={T} H={H} d={d} {io_dtype} seed={seed} state0={state0} d_out={d_out} "
         f"d_state={d_state}")
    gr = kda.backward(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["g"], inp.log_alpha_min,
                      state_in=None if inp.state0 is None else _dev(inp.state0, "f32"),
                      d_out=None if do_io is None else _dev(do_io, io_dtype),
                      d_state=None if ds is None else _dev(ds, "f32"))
    torch.cuda.synchronize()
    return gr, ref


def _check(gr, ref, io_dtype):
    errs = {n: slice_err(gr[n].float().cpu().numpy(), ref[n]) for n in TOKEN_GRADS}
    errs["dstate0"] = slice_err(gr["dstate0"].cpu().numpy(), ref["dstate0"], token_major=False)
    note("  rel-L2 " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[io_dtype], (n, e)


@pytest.mark.parametrize("T", [130, 64, 1])
def test_f32_d64_backward_vs_oracle(T):
    gr, ref = _case(2, T, 3, 64, "f32", seed=500 + T)
    _check(gr, ref, "f32")


def test_f32_d128_backward_vs_oracle():
    gr, ref = _case(1, 200, 2, 128, "f32", seed=611)
    _check(gr, ref, "f32")


@pytest.mark.parametrize("B,T,H,d", [(2, 130, 3, 64), (1, 300, 4, 128)])
def test_bf16_backward_vs_oracle(B, T, H, d):
    gr, ref = _case(B, T, H, d, "bf16", seed=700 + T)
    _check(gr, ref, "bf16")


def test_backward_without_optional_inputs():
    """No initial state and no output gradient: only the final-state seed
    drives the gradients (q and g then get exactly zero)."""
    gr, ref = _case(1, 100, 2, 64, "f32", seed=801, state0=False, d_out=False)
    _check(gr, ref, "f32")
    assert torch.count_nonzero(gr["dq"]).item() == 0 and torch.count_nonzero(gr["dg"]).item() == 0


def test_backward_without_state_seed():
    gr, ref = _case(2, 70, 2, 64, "bf16", seed=802, d_state=False)
    _check(gr, ref, "bf16")


def test_backward_empty_sequence_passes_state_seed_through():
    ds = torch.randn(2, 3, 64, 64, device=DEV)
    e = torch.empty(2, 0, 3, 64, device=DEV)
    gr = kda.backward(e, e, e, e, torch.empty(2, 0, 3, device=DEV), e, -0.1, d_state=ds)
    torch.cuda.synchronize()
    assert torch.equal(gr["dstate0"], ds)


def test_bf16_backward_full_medium_workload_sampled_heads():
    """The medium prefill workload at full size (B=4, T=4096, H=16, d=128,
    bf16), in the same launch configuration the benchmark times; the oracle
    adjoint runs on three sampled (row, head) pairs (heads are independent)."""
    from kda_inputs import workload
    inp = workload(1)
    B, T, H, d = inp.q.shape[0], inp.q.shape[1], inp.q.shape[2], inp.q.shape[3]
    rng = np.random.default_rng(4242)
    do_io, do64 = _io(rng.standard_normal((B, T, H, d)), "bf16")
    ds = rng.standard_normal((B, H, d, d)).astype(np.float32)
    dev = kda.to_device(inp)
    note(f"[backward] full medium workload B={B} T={T} H={H} d={d} bf16")
    gr = kda.backward(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["g"], inp.log_alpha_min,
                      d_out=_dev(do_io, "bf16"), d_state=_dev(ds, "f32"))
    torch.cuda.synchronize()
    f = lambda a: to_f64(a, "bf16")
    for b, h in [(0, 0), (2, 7), (3, 15)]:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        ref = oracle.kda_grad(f(inp.q[sl]), f(inp.k[sl]), f(inp.v[sl]), inp.log_alpha[sl], inp.beta[sl], f(inp.g[sl]),
                              inp.log_alpha_min, None, d_out=do64[sl], d_state=ds[b:b + 1, h:h + 1])
        errs = {n: slice_err(gr[n][sl].float().cpu().numpy(), ref[n]) for n in TOKEN_GRADS}
        errs["dstate0"] = slice_err(gr["dstate0"][b:b + 1, h:h + 1].cpu().numpy(), ref["dstate0"], token_major=False)
        note(f"  (b={b}, h={h}) " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
        for n, e in errs.items():
            assert e <= TOL["bf16"], (b, h, n, e)


def test_backward_floored_channels_and_long_sequence():
    """fp32, 1,000 tokens (16 chunks, a ragged tail): the gradients stay within
    the fp32 bound over many chunk hand-offs, and dlog_alpha is exactly zero
    wherever the retention floor binds (log_alpha <= floor)."""
    B, T, H, d = 1, 1000, 2, 64
    inp = make_inputs(B, T, H, d, d, io_dtype="f32", seed=901, alpha_min=0.95, logit_mu=-3.0, with_state0=True)
    floored = inp.log_alpha <= inp.log_alpha_min
    assert floored.any() and (~floored).any()
    f = lambda a: to_f64(a, "f32")
    rng = np.random.default_rng(902)
    do = rng.standard_normal((B, T, H, d)).astype(np.float32)
    ds = rng.standard_normal((B, H, d, d)).astype(np.float32)
    ref = oracle.kda_grad(f(inp.q), f(inp.k), f(inp.v), inp.log_alpha, inp.beta, f(inp.g), inp.log_alpha_min,
                          inp.state0, d_out=do.astype(np.float64), d_state=ds)
    dev = kda.to_device(inp)
    note(f"[backward] B={B} T={T} H={H} d={d} f32, {floored.mean():.0%} of decays floored")
    gr = kda.backward(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["g"], inp.log_alpha_min,
                      state_in=dev["state0"], d_out=_dev(do, "f32"), d_state=_dev(ds, "f32"))
    torch.cuda.synchronize()
    _check(gr, ref, "f32")
    dla = gr["dlog_alpha"].cpu().numpy()
    assert np.all(dla[floored] == 0.0)
    assert np.count_nonzero(dla[~floored]) > 0.9 * (~floored).sum()


@pytest.mark.parametrize("B,T,H,d,io", [(2, 300, 3, 128, "bf16"), (1, 777, 2, 64, "f32"), (3, 64, 2, 128, "f32"),
                                        (1, 4096, 16, 128, "bf16")])
def test_backward_after_prefill_equals_backward(B, T, H, d, io):
    """kda_prefill_for_backward + kda_backward_after_prefill give what
    kda_chunk_prepare + kda_chunk_scan and kda_backward give, bit for bit:
    the same kernels run, the backward half just reuses the forward's cards,
    chunk states and output.  A second backward call on the same workspace
    with another d_out reuses them again."""
    inp = make_inputs(B, T, H, d, d, io_dtype=io, seed=7700 + T, alpha_min=0.9, logit_mu=-1.0, with_state0=True)
    t = kda.to_device(inp)
    note(f"[backward after prefill] B={B} T={T} H={H} d={d} {io}")
    args = (t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["g"])
    gen = torch.Generator(device=DEV).manual_seed(T)
    dout = torch.randn(t["g"].shape, device=DEV, generator=gen).to(t["g"].dtype)
    dout2 = torch.randn(t["g"].shape, device=DEV, generator=gen).to(t["g"].dtype)
    dst = torch.randn((B, H, d, d), device=DEV, generator=gen)
    r_out, r_st = kda.prefill(*args, inp.log_alpha_min, state_in=t["state0"])
    out, st, ws = kda.prefill_for_backward(*args, inp.log_alpha_min, state_in=t["state0"])
    torch.cuda.synchronize()
    assert torch.equal(out, r_out) and torch.equal(st, r_st)
    for do, ds in ((dout, dst), (dout2, None)):
        ref = kda.backward(*args, inp.log_alpha_min, state_in=t["state0"], d_out=do, d_state=ds)
        got = kda.backward_after_prefill(*args, out, ws, inp.log_alpha_min, d_out=do, d_state=ds)
        torch.cuda.synchronize()
        for name in ref:
            assert torch.equal(got[name], ref[name]), name


def test_prefill_for_backward_in_place_state_and_empty_sequence():
    """state_out may be state_in (the workspace keeps the entering state for
    the backward half); with no tokens the call only passes the state through."""
    inp = make_inputs(2, 200, 3, 64, 64, io_dtype="bf16", seed=7791, alpha_min=0.9, logit_mu=-1.0,
                      with_state0=True)
    t = kda.to_device(inp)
    note("[backward after prefill] B=2 T=200 H=3 d=64 bf16, state in place; T=0")
    args = (t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["g"])
    r_out, r_st = kda.prefill(*args, inp.log_alpha_min, state_in=t["state0"])
    ref = kda.backward(*args, inp.log_alpha_min, state_in=t["state0"], d_out=torch.ones_like(t["g"]))
    s = t["state0"].clone()
    out, st, ws = kda.prefill_for_backward(*args, inp.log_alpha_min, state_in=s, state_out=s)
    torch.cuda.synchronize()
    assert st.data_ptr() == s.data_ptr()
    assert torch.equal(out, r_out) and torch.equal(st, r_st)
    got = kda.backward_after_prefill(*args, out, ws, inp.log_alpha_min, d_out=torch.ones_like(t["g"]))
    torch.cuda.synchronize()
    for name in ref:
        assert torch.equal(got[name], ref[name]), name
    empty = [x[:, :0].contiguous() for x in args]
    out, st, _ = kda.prefill_for_backward(*empty, inp.log_alpha_min, state_in=t["state0"])
    torch.cuda.synchronize()
    assert out.numel() == 0 and torch.equal(st, t["state0"])


@pytest.mark.parametrize("B,T,H,d,io", [(2, 300, 3, 128, "bf16"), (1, 200, 2, 64, "f32")])
def test_prefill_autograd_matches_backward(B, T, H, d, io):
    """prefill_autograd under torch.autograd: the forward equals prefill, and
    the gradients loss.backward() leaves equal kda_backward's bit for bit,
    for a loss on both outputs (state_in a leaf that needs its gradient) and
    for a loss on the output alone (no state_in, the final state unused, so
    its gradient arrives as None)."""
    inp = make_inputs(B, T, H, d, d, io_dtype=io, seed=7800 + T, alpha_min=0.9, logit_mu=-1.0, with_state0=True)
    t = kda.to_device(inp)
    names = ("q", "k", "v", "log_alpha", "beta", "g")
    grad_of = {"q": "dq", "k": "dk", "v": "dv", "log_alpha": "dlog_alpha", "beta": "dbeta", "g": "dg"}
    gen = torch.Generator(device=DEV).manual_seed(T + 1)
    w_out = torch.randn(t["g"].shape, device=DEV, generator=gen)
    w_st = torch.randn((B, H, d, d), device=DEV, generator=gen)
    for with_state in (True, False):
        note(f"[autograd] B={B} T={T} H={H} d={d} {io}, loss on {'out and state' if with_state else 'out'}")
        leaves = {n: t[n].clone().requires_grad_() for n in names}
        s0 = t["state0"].clone().requires_grad_() if with_state else None
        out, st = kda.prefill_autograd(*(leaves[n] for n in names), inp.log_alpha_min, state_in=s0)
        plain = tuple(t[n] for n in names)
        state_ref = t["state0"] if with_state else None
        r_out, r_st = kda.prefill(*plain, inp.log_alpha_min, state_in=state_ref)
        torch.cuda.synchronize()
        assert torch.equal(out.detach(), r_out) and torch.equal(st.detach(), r_st)
        loss = (out.float() * w_out).sum()
        if with_state:
            loss = loss + (st * w_st).sum()
        loss.backward()
        ref = kda.backward(*plain, inp.log_alpha_min, state_in=state_ref, d_out=w_out.to(t["g"].dtype),
                           d_state=w_st if with_state else None, want_dstate=with_state)
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(leaves[n].grad, ref[grad_of[n]]), (n, with_state)
        if with_state:
            assert torch.equal(s0.grad, ref["dstate0"])
