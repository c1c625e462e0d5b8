"""The serving path under HIP graph capture (needs an MI355X), through the C
ABI.  A serving loop captures its launches once and replays them: decode
steps, the two-call prefill with a preallocated workspace, the
allocation-free prefill and the two-stream pipelined prefill are each
captured into a graph and replayed several times, with the program's own
eager work and synchronisations between the replays.  The library records
nothing but kernel launches (no memset, copy or allocation), so every
replay must equal the eager result bit for bit; one replay is also checked
against the fp64 oracle.
"""
import sys

import numpy as np
import pytest

import oracle
from kda_inputs import make_inputs, to_f64

torch = pytest.importorskip("torch")
import gated_delta_rule_91_amd as kda

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
REPLAYS = 4


def note(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_err(gpu, ref, token_major):
    """max relative L2 over (b, h) slices; token_major: [B,T,H,d], else [B,H,...]."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    if token_major:
        gpu, ref = np.moveaxis(gpu, 2, 1), np.moveaxis(ref, 2, 1)
    worst = 0.0
    for b in range(ref.shape[0]):
        for h in range(ref.shape[1]):
            n = np.linalg.norm(ref[b, h].ravel())
            worst = max(worst, np.linalg.norm((gpu[b, h] - ref[b, h]).ravel()) / n)
    return worst


def host(x):
    return x.float().cpu().numpy().astype(np.float64)


def oracle_of(inp):
    f = lambda a: to_f64(a, inp.io_dtype)
    return oracle.kda_ref(f(inp.q), f(inp.k), f(inp.v), inp.log_alpha, inp.beta, f(inp.g), inp.log_alpha_min,
                          inp.state0)


def replay_and_check(graph, reset, results, expected, label):
    """Replay `graph` REPLAYS times; before each, `reset()` restores the
    inputs the graph updates in place; after each, every tensor in `results`
    must equal its eager counterpart.  Eager work of the program's own runs
    between the replays."""
    for r in range(REPLAYS):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(results, expected):
            assert torch.equal(got, want), (label, r)
        side = torch.randn(1 << 20, device="cuda")
        assert torch.isfinite(side.sum()).item()


@pytest.mark.parametrize("io,d", [("bf16", 128), ("f32", 64)])
def test_decode_steps_in_a_graph(io, d):
    N, T, H = 8, 24, 4
    note(f"[graph] decode N={N} H={H} d={d} {io}, {T} steps in one graph")
    inp = make_inputs(N, T, H, d, d, io_dtype=io, seed=950 + d, alpha_min=0.9, logit_mu=-2.0, with_state0=True)
    dd = kda.to_device(inp)
    sm = {n: dd[n].transpose(0, 1).contiguous() for n in ("q", "k", "v", "g", "log_alpha", "beta")}
    floor = inp.log_alpha_min

    def steps(state, outs):
        for t in range(T):
            kda.decode_step(sm["q"][t], sm["k"][t], sm["v"][t], sm["log_alpha"][t], sm["beta"][t], sm["g"][t],
                            state, floor, out=outs[t])

    st_ref = dd["state0"].clone()
    out_ref = torch.empty((T, N, H, d), dtype=dd["g"].dtype, device="cuda")
    steps(st_ref, out_ref)
    torch.cuda.synchronize()

    state = dd["state0"].clone()
    outs = torch.empty_like(out_ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps(state, outs)

    def reset():
        state.copy_(dd["state0"])
        outs.zero_()

    replay_and_check(graph, reset, (state, outs), (st_ref, out_ref), "decode")
    o_ref, s_ref = oracle_of(inp)
    eo = rel_err(host(outs.transpose(0, 1)), o_ref, True)
    es = rel_err(host(state), s_ref, False)
    note(f"  replay vs oracle: out {eo:.2e} state {es:.2e}")
    assert eo <= TOL[io] and es <= TOL[io]


@pytest.mark.parametrize("io,d,T", [("bf16", 128, 1000), ("f32", 64, 333)])
def test_prefill_in_a_graph(io, d, T):
    B, H = 2, 4
    note(f"[graph] prefill B={B} T={T} H={H} d={d} {io}: two calls, and allocation-free")
    inp = make_inputs(B, T, H, d, d, io_dtype=io, seed=960 + T, alpha_min=0.9, logit_mu=-2.0, with_state0=True)
    dd = kda.to_device(inp)
    floor = inp.log_alpha_min
    args = (dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"])
    p = kda.problem(B, T, H, d, d, kda.KDA_BF16 if io == "bf16" else kda.KDA_F32, floor)
    ws = torch.empty(kda.workspace_size(p), dtype=torch.uint8, device="cuda")

    ref_out, ref_st = kda.prefill(*args, dd["g"], floor, state_in=dd["state0"])
    torch.cuda.synchronize()

    # the two calls, with the state carried in place (state_out == state_in)
    out = torch.empty_like(dd["g"])
    st = dd["state0"].clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.chunk_prepare(*args, floor, workspace=ws)
        kda.chunk_scan(ws, dd["g"], floor, state_in=st, out=out, state_out=st)

    def reset():
        st.copy_(dd["state0"])
        out.zero_()

    replay_and_check(graph, reset, (out, st), (ref_out, ref_st), "prefill")

    # the allocation-free prefill (warmed up eagerly first: its scratch
    # address is looked up on the first call on a device)
    out2 = torch.empty_like(dd["g"])
    st2 = torch.empty_like(ref_st)
    kda.prefill_noalloc(*args, dd["g"], floor, state_in=dd["state0"], out=out2, state_out=st2)
    torch.cuda.synchronize()
    graph2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph2):
        kda.prefill_noalloc(*args, dd["g"], floor, state_in=dd["state0"], out=out2, state_out=st2)

    def reset2():
        out2.zero_()
        st2.zero_()

    replay_and_check(graph2, reset2, (out2, st2), (ref_out, ref_st), "prefill_noalloc")

    o_ref, s_ref = oracle_of(inp)
    eo, es = rel_err(host(out2), o_ref, True), rel_err(host(st2), s_ref, False)
    note(f"  replay vs oracle: out {eo:.2e} state {es:.2e}")
    assert eo <= TOL[io] and es <= TOL[io]


def test_pipelined_prefill_in_a_graph():
    """The two-stream prefill: its second stream joins the capture through
    the events the call records, and the call joins it back before
    returning, so the whole range pipeline is one graph."""
    B, T, H, d = 1, 3000, 8, 128
    note(f"[graph] pipelined prefill B={B} T={T} H={H} d={d} bf16, ranges of 7 chunks")
    inp = make_inputs(B, T, H, d, d, io_dtype="bf16", seed=971, alpha_min=0.9, logit_mu=-2.0, with_state0=True)
    dd = kda.to_device(inp)
    floor = inp.log_alpha_min
    args = (dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"], dd["g"], floor)
    ref_out, ref_st = kda.prefill(*args[:5], dd["g"], floor, state_in=dd["state0"])
    torch.cuda.synchronize()
    p = kda.problem(B, T, H, d, d, kda.KDA_BF16, floor)
    ws = torch.empty(kda.pipelined_workspace_size(p, 7), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dd["g"])
    st = torch.empty_like(ref_st)
    aux = torch.cuda.Stream()
    kda.prefill_pipelined(*args, state_in=dd["state0"], out=out, state_out=st, range_chunks=7, workspace=ws,
                          aux_stream=aux)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(st, ref_st)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.prefill_pipelined(*args, state_in=dd["state0"], out=out, state_out=st, range_chunks=7, workspace=ws,
                              aux_stream=aux)

    def reset():
        out.zero_()
        st.zero_()

    replay_and_check(graph, reset, (out, st), (ref_out, ref_st), "prefill_pipelined")
