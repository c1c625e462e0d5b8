"""Packed variable-length batches (kda_varlen_prepare + kda_varlen_scan) on the
GPU: bit-identical to prefill run on each sequence alone (the same per-chunk
arithmetic), and within tolerance of the fp64 oracle per sequence.  Lengths
include 0, 1, exact chunk multiples and ragged tails; one batch has more than
256 sequences (the chunk-offset scan carries across blocks)."""
import sys

import numpy as np
import pytest

import oracle
from kda_inputs import make_inputs, to_f64

torch = pytest.importorskip("torch")
import gated_delta_rule_91_amd as kda

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}


def note(*a):
    print(*a, file=sys.stderr, flush=True)


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    n = np.linalg.norm(b.ravel())
    return np.linalg.norm((a - b).ravel()) / n if n > 0 else np.linalg.norm(a.ravel())


def _packed(lengths, H, d, io, seed):
    T = int(sum(lengths))
    inp = make_inputs(1, T, H, d, d, io_dtype=io, seed=seed, alpha_min=0.9, logit_mu=-1.0)
    dev = kda.to_device(inp)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    s0 = torch.randn(len(lengths), H, d, d, device="cuda", generator=torch.Generator("cuda").manual_seed(seed)) * 0.1
    return inp, dev, cu, s0


@pytest.mark.parametrize("io,d", [("bf16", 128), ("f32", 64)])
def test_varlen_matches_per_sequence_prefill_exactly(io, d):
    lengths = [0, 1, 63, 64, 65, 200, 130, 7]
    H = 3
    note(f"[varlen] exact vs per-sequence prefill, {io} d={d} lengths={lengths}")
    inp, dev, cu, s0 = _packed(lengths, H, d, io, seed=31)
    cu_t = torch.from_numpy(cu).cuda()
    out, st = kda.varlen_prefill(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["g"],
                                 inp.log_alpha_min, cu_t, state_in=s0)
    torch.cuda.synchronize()
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        sl = lambda x: x[:, a:b].contiguous()
        o1, st1 = kda.prefill(sl(dev["q"]), sl(dev["k"]), sl(dev["v"]), sl(dev["log_alpha"]), sl(dev["beta"]),
                              sl(dev["g"]), inp.log_alpha_min, state_in=s0[s:s + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(out[:, a:b], o1), s
        assert torch.equal(st[s:s + 1], st1), s


def test_varlen_bf16_vs_oracle():
    rng = np.random.default_rng(5)
    lengths = [int(x) for x in rng.integers(0, 300, size=12)] + [0, 64, 1]
    H, d = 2, 128
    note(f"[varlen] oracle parity bf16 d={d} lengths={lengths}")
    inp, dev, cu, s0 = _packed(lengths, H, d, "bf16", seed=77)
    out, st = kda.varlen_prefill(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["g"],
                                 inp.log_alpha_min, torch.from_numpy(cu).cuda(), state_in=s0)
    torch.cuda.synchronize()
    out_h, st_h, s0_h = out.float().cpu().numpy(), st.cpu().numpy(), s0.cpu().numpy().astype(np.float64)
    f = lambda x: to_f64(x, "bf16")
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        sl = (slice(None), slice(a, b))
        o_ref, s_ref = oracle.kda_ref(f(inp.q[sl]), f(inp.k[sl]), f(inp.v[sl]), inp.log_alpha[sl], inp.beta[sl],
                                      f(inp.g[sl]), inp.log_alpha_min, s0_h[s:s + 1])
        if b > a:
            assert _rel(out_h[:, a:b], o_ref) <= TOL["bf16"], s
        assert _rel(st_h[s:s + 1], s_ref) <= TOL["bf16"], s


def test_varlen_many_sequences():
    rng = np.random.default_rng(9)
    lengths = [int(x) for x in rng.integers(0, 140, size=300)]
    H, d = 2, 64
    note(f"[varlen] {len(lengths)} sequences, {sum(lengths)} tokens, f32 d={d}")
    inp, dev, cu, s0 = _packed(lengths, H, d, "f32", seed=123)
    cu_t = torch.from_numpy(cu).cuda()
    out, st = kda.varlen_prefill(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["g"],
                                 inp.log_alpha_min, cu_t, state_in=s0)
    torch.cuda.synchronize()
    for s in list(range(0, 300, 37)) + [299]:
        a, b = int(cu[s]), int(cu[s + 1])
        sl = lambda x: x[:, a:b].contiguous()
        o1, st1 = kda.prefill(sl(dev["q"]), sl(dev["k"]), sl(dev["v"]), sl(dev["log_alpha"]), sl(dev["beta"]),
                              sl(dev["g"]), inp.log_alpha_min, state_in=s0[s:s + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(out[:, a:b], o1), s
        assert torch.equal(st[s:s + 1], st1), s


def test_varlen_state_in_place():
    """state_out may be the same buffer as state_in (resume in place)."""
    lengths = [70, 0, 129, 5]
    H, d = 2, 64
    inp, dev, cu, s0 = _packed(lengths, H, d, "bf16", seed=55)
    cu_t = torch.from_numpy(cu).cuda()
    out_ref, st_ref = kda.varlen_prefill(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["g"],
                                         inp.log_alpha_min, cu_t, state_in=s0)
    st = s0.clone()
    ws = kda.varlen_prepare(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], inp.log_alpha_min, cu_t)
    out, _ = kda.varlen_scan(ws, dev["g"], inp.log_alpha_min, cu_t, state_in=st, state_out=st)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    assert torch.equal(st, st_ref)


def test_varlen_benchmark_configuration_sampled_vs_oracle():
    """The packed batch the benchmark times: the long workload's 65,536 tokens
    x 32 heads (d=128, bf16) cut into the seeded log-uniform length mix, in the
    same launch configuration; the oracle runs on sampled (sequence, head)
    pairs, each from an empty state."""
    from kda_inputs import varlen_lengths, workload
    inp = workload(2)
    T = inp.q.shape[1]
    lens = varlen_lengths(T)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    note(f"[varlen] benchmark configuration: {len(lens)} sequences, {T} tokens x 32 heads")
    dev = kda.to_device(inp)
    out, st = kda.varlen_prefill(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["g"],
                                 inp.log_alpha_min, torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    f = lambda x: to_f64(x, "bf16")
    longest = int(np.argmax(lens))
    for s, h in [(0, 0), (longest, 17), (len(lens) - 1, 31), (len(lens) // 2, 5)]:
        a, b = int(cu[s]), int(cu[s + 1])
        sl = (slice(None), slice(a, b), slice(h, h + 1))
        o_ref, s_ref = oracle.kda_ref(f(inp.q[sl]), f(inp.k[sl]), f(inp.v[sl]), inp.log_alpha[sl], inp.beta[sl],
                                      f(inp.g[sl]), inp.log_alpha_min)
        eo = _rel(out[sl].float().cpu().numpy(), o_ref)
        es = _rel(st[s:s + 1, h:h + 1].cpu().numpy(), s_ref)
        note(f"  sequence {s} ({b - a} tokens), head {h}: rel-L2 out {eo:.2e} state {es:.2e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"], (s, h, eo, es)


def test_varlen_overlapping_offsets_stay_inside_the_workspace():
    """Offsets that go back (sequences 0, 2 and 4 all cover tokens 0..255)
    need 12 chunks where the workspace holds ceil(256/64) + 5 = 9: the plan
    clamps the chunk offsets, so the last copy keeps one chunk and no access
    leaves the workspace.  The complete copies equal an ordinary prefill."""
    H, d, T = 2, 128, 256
    note("[varlen] overlapping offsets, 12 chunks for a 9-chunk workspace")
    inp = make_inputs(1, T, H, d, d, io_dtype="bf16", seed=47, alpha_min=0.9, logit_mu=-1.0)
    dev = kda.to_device(inp)
    cu = torch.tensor([0, 256, 0, 256, 0, 256], dtype=torch.int32, device="cuda")
    out, st = kda.varlen_prefill(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["g"],
                                 inp.log_alpha_min, cu)
    o1, st1 = kda.prefill(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["g"], inp.log_alpha_min)
    first = lambda x: x[:, :64].contiguous()
    _, st64 = kda.prefill(*(first(dev[n]) for n in ("q", "k", "v", "log_alpha", "beta", "g")), inp.log_alpha_min)
    torch.cuda.synchronize()
    assert torch.equal(out, o1)
    assert torch.equal(st[0:1], st1) and torch.equal(st[2:3], st1)
    assert torch.equal(st[4:5], st64)   # the clamped copy: its first chunk only
    assert not st[1].any() and not st[3].any()   # empty sequences from a zero state


GRADS = ("dq", "dk", "dv", "dg", "dlog_alpha", "dbeta")


def _varlen_grads(lengths, H, d, io, seed):
    inp, dev, cu, s0 = _packed(lengths, H, d, io, seed)
    gen = torch.Generator(device="cuda").manual_seed(seed + 1)
    dout = torch.randn(dev["g"].shape, device="cuda", generator=gen).to(dev["g"].dtype)
    dst = torch.randn((len(lengths), H, d, d), device="cuda", generator=gen)
    args = (dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], dev["g"])
    gr = kda.varlen_backward(*args, inp.log_alpha_min, torch.from_numpy(cu).cuda(), state_in=s0, d_out=dout,
                             d_state=dst)
    torch.cuda.synchronize()
    return inp, dev, cu, s0, dout, dst, args, gr


@pytest.mark.parametrize("io,d,lengths", [
    ("bf16", 128, [0, 1, 63, 64, 65, 200, 130, 7]),
    ("f32", 64, [5, 0, 130, 64, 1, 300]),
    ("bf16", 64, [777, 2, 0]),
])
def test_varlen_backward_equals_per_sequence_backward(io, d, lengths):
    """kda_varlen_backward: all sequences' chunks in one launch per kernel,
    bit-identical to kda_backward on each sequence alone (its slice of the
    packed arrays, its own state and state gradient); an empty sequence
    passes its state gradient through."""
    H = 3
    note(f"[varlen backward] exact vs per-sequence backward, {io} d={d} lengths={lengths}")
    inp, dev, cu, s0, dout, dst, args, gr = _varlen_grads(lengths, H, d, io, seed=41 + d)
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        sl = lambda x: x[:, a:b].contiguous()
        ref = kda.backward(*(sl(x) for x in args), inp.log_alpha_min, state_in=s0[s:s + 1].contiguous(),
                           d_out=sl(dout), d_state=dst[s:s + 1].contiguous())
        torch.cuda.synchronize()
        for n in GRADS:
            assert torch.equal(gr[n][:, a:b], ref[n]), (s, n)
        assert torch.equal(gr["dstate0"][s:s + 1], ref["dstate0"]), s


def test_varlen_backward_vs_oracle():
    """The same call against the fp64 adjoint of the step recurrence, run on
    every sequence of the packing alone and packed back.  The measure is the
    relative L2 per (row, head) slice of each gradient as the call returns it
    (the packed [1, T, H, d] arrays) and per (sequence, head) for the state
    gradients; a slice of one or two tokens would measure single bf16
    roundings, not the method."""
    rng = np.random.default_rng(9)
    lengths = [int(x) for x in rng.integers(0, 260, size=6)] + [0, 64, 1]
    H, d = 2, 128
    note(f"[varlen backward] oracle parity bf16 d={d} lengths={lengths}")
    inp, dev, cu, s0, dout, dst, args, gr = _varlen_grads(lengths, H, d, "bf16", seed=83)
    f = lambda x: to_f64(x, "bf16")
    do64 = dout.float().cpu().numpy().astype(np.float64)
    ds64, s064 = dst.cpu().numpy().astype(np.float64), s0.cpu().numpy().astype(np.float64)
    packed = {n: np.zeros(gr[n].shape) for n in GRADS}
    ds0 = gr["dstate0"].cpu().numpy()
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        sl = (slice(None), slice(a, b))
        ref = oracle.kda_grad(f(inp.q[sl]), f(inp.k[sl]), f(inp.v[sl]), inp.log_alpha[sl], inp.beta[sl],
                              f(inp.g[sl]), inp.log_alpha_min, s064[s:s + 1], d_out=do64[sl], d_state=ds64[s:s + 1])
        for n in GRADS:
            packed[n][sl] = ref[n]
        for h in range(H):
            e = _rel(ds0[s, h], ref["dstate0"][0, h])
            assert e <= TOL["bf16"], ("dstate0", s, h, e)
    for n in GRADS:
        got = gr[n].float().cpu().numpy()
        for h in range(H):
            e = _rel(got[:, :, h], packed[n][:, :, h])
            note(f"  {n} head {h}: {e:.2e}")
            assert e <= TOL["bf16"], (n, h, e)


def test_varlen_backward_medium_packing_equals_per_sequence():
    """A training-sized packing: 16,384 tokens x 16 heads at d = 128 bf16 in
    sequences of 64..4,096 tokens, bit-identical to per-sequence backward."""
    rng = np.random.default_rng(13)
    lengths, left = [], 16384
    while left > 0:
        n = min(left, int(np.exp(rng.uniform(np.log(64), np.log(4096)))))
        lengths.append(n)
        left -= n
    H, d = 16, 128
    note(f"[varlen backward] {len(lengths)} sequences, {sum(lengths)} tokens x {H} heads bf16")
    inp, dev, cu, s0, dout, dst, args, gr = _varlen_grads(lengths, H, d, "bf16", seed=97)
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        sl = lambda x: x[:, a:b].contiguous()
        ref = kda.backward(*(sl(x) for x in args), inp.log_alpha_min, state_in=s0[s:s + 1].contiguous(),
                           d_out=sl(dout), d_state=dst[s:s + 1].contiguous())
        torch.cuda.synchronize()
        for n in GRADS:
            assert torch.equal(gr[n][:, a:b], ref[n]), (s, n)
        assert torch.equal(gr["dstate0"][s:s + 1], ref["dstate0"]), s


def test_varlen_backward_no_tokens_passes_state_gradients_through():
    H, d = 2, 64
    note("[varlen backward] three empty sequences")
    e = torch.empty(1, 0, H, d, device="cuda")
    dst = torch.randn(3, H, d, d, device="cuda")
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    gr = kda.varlen_backward(e, e, e, e, torch.empty(1, 0, H, device="cuda"), e, -0.1, cu, d_state=dst)
    torch.cuda.synchronize()
    assert torch.equal(gr["dstate0"], dst)


@pytest.mark.parametrize("io,d,lengths", [("bf16", 128, [0, 1, 63, 64, 65, 200, 130, 7]), ("f32", 64, [300, 5, 0, 64])])
def test_varlen_split_pair_and_autograd_equal_varlen_backward(io, d, lengths):
    """kda_varlen_prefill_for_backward + kda_varlen_backward_after_prefill, and
    prefill_autograd with cu_seqlens under loss.backward(), give what
    varlen_prefill and kda_varlen_backward give, bit for bit."""
    H = 3
    note(f"[varlen split pair] {io} d={d} lengths={lengths}")
    inp, dev, cu, s0, dout, dst, args, ref = _varlen_grads(lengths, H, d, io, seed=61 + d)
    cu_t = torch.from_numpy(cu).cuda()
    r_out, r_st = kda.varlen_prefill(*args, inp.log_alpha_min, cu_t, state_in=s0)
    out, st, ws = kda.varlen_prefill_for_backward(*args, inp.log_alpha_min, cu_t, state_in=s0)
    torch.cuda.synchronize()
    assert torch.equal(out, r_out) and torch.equal(st, r_st)
    got = kda.varlen_backward_after_prefill(*args, out, ws, inp.log_alpha_min, cu_t, d_out=dout, d_state=dst)
    torch.cuda.synchronize()
    for n in ref:
        assert torch.equal(got[n], ref[n]), n
    names = ("q", "k", "v", "log_alpha", "beta", "g")
    leaves = [x.clone().requires_grad_() for x in args]
    s0l = s0.clone().requires_grad_()
    o, s = kda.prefill_autograd(*leaves, inp.log_alpha_min, state_in=s0l, cu_seqlens=cu_t)
    ((o.float() * dout.float()).sum() + (s * dst).sum()).backward()
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), r_out) and torch.equal(s.detach(), r_st)
    grad_of = {"q": "dq", "k": "dk", "v": "dv", "log_alpha": "dlog_alpha", "beta": "dbeta", "g": "dg"}
    for n, x in zip(names, leaves):
        assert torch.equal(x.grad, ref[grad_of[n]]), n
    assert torch.equal(s0l.grad, ref["dstate0"])


def test_varlen_backward_overlapping_offsets_stay_inside_the_workspace():
    """The backward over offsets that go back (as in the forward test above:
    12 chunks for a workspace that holds 9): every kernel takes the clamped
    chunk offsets, so no access leaves the arrays or the workspace.  The
    complete copies (sequences 0 and 2, the same state seed) write identical
    values, so token rows past the first chunk equal an ordinary backward;
    each sequence's state gradient is its own."""
    H, d, T = 2, 128, 256
    note("[varlen backward] overlapping offsets, 12 chunks for a 9-chunk workspace")
    inp = make_inputs(1, T, H, d, d, io_dtype="bf16", seed=48, alpha_min=0.9, logit_mu=-1.0)
    dev = kda.to_device(inp)
    args = tuple(dev[n] for n in ("q", "k", "v", "log_alpha", "beta", "g"))
    cu = torch.tensor([0, 256, 0, 256, 0, 256], dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(3)
    dout = torch.randn(dev["g"].shape, device="cuda", generator=gen).to(torch.bfloat16)
    dst = torch.randn((5, H, d, d), device="cuda", generator=gen)
    dst[2] = dst[0]
    gr = kda.varlen_backward(*args, inp.log_alpha_min, cu, d_out=dout, d_state=dst)
    full = kda.backward(*args, inp.log_alpha_min, d_out=dout, d_state=dst[0:1].contiguous())
    first = lambda x: x[:, :64].contiguous()
    one = kda.backward(*(first(x) for x in args), inp.log_alpha_min, d_out=first(dout),
                       d_state=dst[4:5].contiguous())
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(gr[n][:, 64:], full[n][:, 64:]), n
    assert torch.equal(gr["dstate0"][0:1], full["dstate0"]) and torch.equal(gr["dstate0"][2:3], full["dstate0"])
    assert torch.equal(gr["dstate0"][4:5], one["dstate0"])   # the clamped copy: its first chunk only
    assert torch.equal(gr["dstate0"][1], dst[1]) and torch.equal(gr["dstate0"][3], dst[3])   # empty sequences


def test_second_calls_with_other_offsets_stay_inside_the_workspace():
    """kda_varlen_scan and kda_varlen_backward_after_prefill read back the chunk
    offsets the first call wrote, clamped to the workspace and to each
    sequence's length: called with other cu_seqlens than the first call's
    (sequences longer and shorter than the offsets say), they give wrong
    values (finite in the per-sequence states and state gradients, which
    every call writes; token rows the clamped chunks do not cover are not
    written), with every access inside the arrays and the workspace, and the
    right cu_seqlens still give the right result after."""
    H, d, T = 2, 128, 300
    note("[varlen] second calls with other offsets than the first")
    inp = make_inputs(1, T, H, d, d, io_dtype="bf16", seed=49, alpha_min=0.9, logit_mu=-1.0)
    dev = kda.to_device(inp)
    args = tuple(dev[n] for n in ("q", "k", "v", "log_alpha", "beta", "g"))
    cu_a = torch.tensor([0, 100, 300], dtype=torch.int32, device="cuda")
    cu_b = torch.tensor([0, 250, 300], dtype=torch.int32, device="cuda")
    ws = kda.varlen_prepare(*args[:5], inp.log_alpha_min, cu_a)
    out, st = kda.varlen_scan(ws, dev["g"], inp.log_alpha_min, cu_b)
    torch.cuda.synchronize()
    assert torch.isfinite(st).all()
    ref_out, ref_st = kda.varlen_prefill(*args, inp.log_alpha_min, cu_a)
    out2, st2 = kda.varlen_scan(ws, dev["g"], inp.log_alpha_min, cu_a)
    torch.cuda.synchronize()
    assert torch.equal(out2, ref_out) and torch.equal(st2, ref_st)
    o, s, wsb = kda.varlen_prefill_for_backward(*args, inp.log_alpha_min, cu_a)
    dout = torch.ones_like(dev["g"])
    gr = kda.varlen_backward_after_prefill(*args, o, wsb, inp.log_alpha_min, cu_b, d_out=dout,
                                           d_state=torch.ones_like(s))
    torch.cuda.synchronize()
    assert torch.isfinite(gr["dstate0"]).all()
    ref = kda.varlen_backward(*args, inp.log_alpha_min, cu_a, d_out=dout)
    got = kda.varlen_backward_after_prefill(*args, o, wsb, inp.log_alpha_min, cu_a, d_out=dout)
    torch.cuda.synchronize()
    for n in ref:
        assert torch.equal(got[n], ref[n]), n
