"""HIP path vs the fp64 oracle, element by element (needs an MI355X).

Every call goes through the C ABI (the ctypes binding passes device pointers
and the current stream).  The oracle sees the same, already rounded inputs
(bf16 -> fp64 is exact), so input quantisation is not charged to the
kernels.  Error measure: relative L2 per (batch row, head) slice, separately
for the outputs [T, d_v] and the final state [d_k, d_v]; the largest slice
error must stay within 1e-4 for fp32 inputs and 2e-2 for bf16 inputs with the
fp32 state.
"""
import sys

import numpy as np
import pytest

import oracle
from kda_inputs import make_inputs, to_f64, workload

torch = pytest.importorskip("torch")
import gated_delta_rule_91_amd as kda

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda"


def note(*a):
    print(*a, file=sys.stderr, flush=True)


def slice_err(gpu, ref, kind):
    """max rel-L2 over (b, h) slices; kind 'out' = [B,T,H,d], 'state' = [B,H,dk,dv]."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    if kind == "out":
        gpu, ref = gpu.transpose(0, 2, 1, 3), ref.transpose(0, 2, 1, 3)
    B, H = ref.shape[:2]
    worst = 0.0
    for b in range(B):
        for h in range(H):
            d = np.linalg.norm((gpu[b, h] - ref[b, h]).ravel())
            n = np.linalg.norm(ref[b, h].ravel())
            worst = max(worst, d / n if n > 0 else d)
    return worst


def token_worst(gpu, ref):
    """Largest per-token error of [B,T,H,d] outputs, relative to the RMS token
    norm of its (b, h) slice.  A slice-wide relative L2 over 65,536 tokens
    would hide one wrong token row (about 0.4% of the slice norm); here one
    fully wrong row scores about 1.4."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.linalg.norm(gpu - ref, axis=-1)           # [B,T,H]
    rms = np.sqrt(np.mean(np.sum(ref * ref, axis=-1), axis=1, keepdims=True))   # [B,1,H]
    return float(np.max(err / np.maximum(rms, 1e-300)))


# bound on token_worst for bf16 I/O: the slice error is ~5e-3 and the
# largest of 65,536 per-token errors a few times that; a wrong row or a
# localised error of a tenth of a token's norm exceeds it
TOKEN_TOL_BF16 = 0.1


def host(x):
    return x.float().cpu().numpy().astype(np.float64)


def oracle_run(inp, heads=None, state0="inp", T=None):
    f = lambda a: to_f64(a, inp.io_dtype)
    sel = (slice(None), slice(None) if T is None else slice(0, T), heads if heads is not None else slice(None))
    s0 = inp.state0 if state0 == "inp" else state0
    if s0 is not None and heads is not None:
        s0 = s0[:, heads]
    return oracle.kda_ref(f(inp.q[sel]), f(inp.k[sel]), f(inp.v[sel]), inp.log_alpha[sel], inp.beta[sel],
                          f(inp.g[sel]), inp.log_alpha_min, s0)


def gpu_prefill(d, floor, state_in="d"):
    s0 = d["state0"] if state_in == "d" else state_in
    out, st = kda.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["g"], floor, state_in=s0)
    torch.cuda.synchronize()
    return out, st


@pytest.mark.parametrize("T", [256, 1, 63, 65, 200])
def test_f32_prefill_vs_oracle(T):
    note(f"[f32 prefill] T={T}")
    if T == 256:
        inp = workload(0)                                  # the 256-token, d=64 fp32 workload
    else:
        inp = make_inputs(2, T, 3, 64, 64, io_dtype="f32", seed=100 + T, alpha_min=0.9, logit_mu=-1.0,
                          with_state0=True)
    d = kda.to_device(inp)
    out, st = gpu_prefill(d, inp.log_alpha_min)
    o_ref, s_ref = oracle_run(inp)
    eo, es = slice_err(host(out), o_ref, "out"), slice_err(host(st), s_ref, "state")
    note(f"  rel-L2 out {eo:.2e} state {es:.2e}")
    assert eo <= TOL["f32"] and es <= TOL["f32"]


# (128, 777, 5): ragged, heads not a multiple of the 8 XCDs; (64, 130, 64):
# 128 (row, head) chains, so the hand-off runs two 16-column slices per
# workgroup at d = 64; (128, 70, 64): four slices per workgroup at d = 128
@pytest.mark.parametrize("dk,T,H,mu", [(128, 777, 5, -4.0), (64, 300, 3, 0.0), (128, 64, 9, 0.0), (64, 130, 64, -4.0),
                                       (128, 70, 64, -4.0)])
def test_bf16_prefill_vs_oracle(dk, T, H, mu):
    note(f"[bf16 prefill] dk={dk} T={T} H={H}")
    inp = make_inputs(2, T, H, dk, dk, io_dtype="bf16", seed=7 + T, alpha_min=0.9, logit_mu=mu, with_state0=True)
    d = kda.to_device(inp)
    out, st = gpu_prefill(d, inp.log_alpha_min)
    o_ref, s_ref = oracle_run(inp)
    eo, es = slice_err(host(out), o_ref, "out"), slice_err(host(st), s_ref, "state")
    note(f"  rel-L2 out {eo:.2e} state {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


# fp32 at d = 128 runs a two-deep operand ring: 8 (row, head) chains give one
# 16-column slice per workgroup (odd and even chunk counts, full and ragged
# last chunk), 64 chains two slices, 256 chains four
@pytest.mark.parametrize("B,T,H", [(2, 100, 32), (1, 300, 8), (1, 256, 8), (1, 129, 8), (4, 200, 64)])
def test_f32_d128_prefill_vs_oracle(B, T, H):
    note(f"[f32 prefill] dk=128 B={B} T={T} H={H}")
    inp = make_inputs(B, T, H, 128, 128, io_dtype="f32", seed=23 + T, alpha_min=0.9, logit_mu=-2.0,
                      with_state0=True)
    d = kda.to_device(inp)
    out, st = gpu_prefill(d, inp.log_alpha_min)
    o_ref, s_ref = oracle_run(inp)
    eo, es = slice_err(host(out), o_ref, "out"), slice_err(host(st), s_ref, "state")
    note(f"  rel-L2 out {eo:.2e} state {es:.2e}")
    assert eo <= TOL["f32"] and es <= TOL["f32"]


def test_f32_d64_four_slices_vs_oracle():
    """fp32 at d = 64 with 256 (row, head) chains: four 16-column slices per
    workgroup in the hand-off (its three-deep operand ring), ragged tail."""
    note("[f32 prefill] dk=64 B=4 T=70 H=64")
    inp = make_inputs(4, 70, 64, 64, 64, io_dtype="f32", seed=29, alpha_min=0.9, logit_mu=-2.0, with_state0=True)
    d = kda.to_device(inp)
    out, st = gpu_prefill(d, inp.log_alpha_min)
    o_ref, s_ref = oracle_run(inp)
    eo, es = slice_err(host(out), o_ref, "out"), slice_err(host(st), s_ref, "state")
    note(f"  rel-L2 out {eo:.2e} state {es:.2e}")
    assert eo <= TOL["f32"] and es <= TOL["f32"]


def test_medium_prefill_full_vs_oracle():
    """B=4, T=4096, H=16, d=128, bf16; every (b, h) slice checked."""
    note("[bf16 prefill] B=4 T=4096 H=16 d=128")
    inp = workload(1)
    d = kda.to_device(inp)
    out, st = gpu_prefill(d, inp.log_alpha_min)
    o_ref, s_ref = oracle_run(inp)
    eo, es = slice_err(host(out), o_ref, "out"), slice_err(host(st), s_ref, "state")
    note(f"  rel-L2 out {eo:.2e} state {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.timeout(600)
def test_long_prefill_sampled_heads_vs_oracle():
    """B=1, T=65536, H=32, d=128 bf16 at full size; the oracle checks 2 heads end to end."""
    note("[bf16 prefill] B=1 T=65536 H=32 d=128")
    inp = workload(2)
    d = kda.to_device(inp)
    out, st = gpu_prefill(d, inp.log_alpha_min)
    heads = [0, 31]
    o_ref, s_ref = oracle_run(inp, heads=heads)
    eo = slice_err(host(out[:, :, heads]), o_ref, "out")
    es = slice_err(host(st[:, heads]), s_ref, "state")
    et = token_worst(host(out[:, :, heads]), o_ref)
    note(f"  rel-L2 out {eo:.2e} state {es:.2e}; worst token {et:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    assert et <= TOKEN_TOL_BF16
    assert torch.isfinite(out).all() and torch.isfinite(st).all()


def test_prefix_cache_resume_at_benchmark_size():
    """B=1, T=65536, H=32, d=128 bf16 (one 16-column slice per workgroup, as
    the benchmark launches it): checkpoints every 64 chunks equal the
    plain scan's outputs and final state, and prefilling the rest from the
    checkpoints after 32,768 and 61,440 tokens reproduces outputs and final
    state bit for bit."""
    note("[checkpoints] B=1 T=65536 H=32 d=128, every 64 chunks")
    inp = workload(2)
    d = kda.to_device(inp)
    floor = inp.log_alpha_min
    T = d["q"].shape[1]
    ws = kda.chunk_prepare(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], floor)
    out, st = kda.chunk_scan(ws, d["g"], floor)
    out_c, st_c, ck = kda.chunk_scan_checkpoints(ws, d["g"], floor, 64)
    torch.cuda.synchronize()
    assert ck.shape[2] == 17
    assert torch.equal(out_c, out) and torch.equal(st_c, st) and torch.equal(ck[:, :, 16], st)
    assert not ck[:, :, 0].any()
    # the checkpoint contents against the oracle's state after the same prefix
    h = 3
    for j in (8, 15):
        _, s_ref = oracle_run(inp, heads=[h], T=4096 * j)
        e = slice_err(host(ck[:, h:h + 1, j]), s_ref, "state")
        note(f"  checkpoint {j} (head {h}) vs oracle: {e:.2e}")
        assert e <= TOL["bf16"], j
    for j in (8, 15):
        t = 4096 * j
        rest = {n: d[n][:, t:] for n in ("q", "k", "v", "log_alpha", "beta", "g")}
        o_r, s_r = kda.prefill(rest["q"], rest["k"], rest["v"], rest["log_alpha"], rest["beta"], rest["g"], floor,
                               state_in=ck[:, :, j].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o_r, out[:, t:]), j
        assert torch.equal(s_r, st), j


@pytest.mark.timeout(900)
def test_segmented_1m_prefill_sampled_head_vs_oracle():
    """T = 1,048,576, H=8, d=128 as 16 segments of 65,536: prepare -> summarize ->
    combine -> scan; one head checked against the unsegmented oracle over all 1M tokens."""
    note("[segmented prefill] T=1048576 H=8 16 segments")
    inp = workload(3)
    d = kda.to_device(inp)
    out, st = kda.segmented_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["g"], inp.log_alpha_min,
                                    n_seg=16)
    torch.cuda.synchronize()
    heads = [5]
    o_ref, s_ref = oracle_run(inp, heads=heads)
    eo = slice_err(host(out[:, :, heads]), o_ref, "out")
    es = slice_err(host(st[:, heads]), s_ref, "state")
    et = token_worst(host(out[:, :, heads]), o_ref)
    note(f"  rel-L2 out {eo:.2e} state {es:.2e}; worst token {et:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    assert et <= TOKEN_TOL_BF16


# With 2 rows x 4 segments the summary sees 8H (segment, head) pairs, each
# with 16 column tiles of the augmented state.  At d = 128 in bf16: H = 3
# (24 pairs) runs the summaries with two 16-column slices per workgroup
# (four waves share a slice), H = 4 and H = 8 one whole slice per wave, H =
# 16 two slices per wave (and four slices per workgroup in the recompute)
@pytest.mark.parametrize("io,H", [("f32", 3), ("bf16", 3), ("bf16", 4), ("bf16", 8), ("bf16", 16)])
def test_summarize_and_combine_vs_oracle(io, H):
    note(f"[summary/combine] {io} H={H}")
    n_seg, Ts, dk = 4, 96, 64 if io == "f32" else 128
    inp = make_inputs(2, n_seg * Ts, H, dk, dk, io_dtype=io, seed=41, alpha_min=0.9, logit_mu=-4.0, with_state0=True)
    d = kda.to_device(inp)
    out, fin = kda.segmented_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["g"], inp.log_alpha_min,
                                     n_seg=n_seg, state_in=d["state0"])
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_run(inp)
    eo, es = slice_err(host(out), o_ref, "out"), slice_err(host(fin), s_ref, "state")
    note(f"  segmented vs oracle: out {eo:.2e} state {es:.2e}")
    assert eo <= TOL[io] and es <= TOL[io]
    # the summary pair itself, against the oracle's
    f = lambda a: to_f64(a, io)
    seg = lambda a: a.reshape((2 * n_seg, Ts) + a.shape[2:])
    ws = kda.chunk_prepare(*(seg(d[n]) for n in ("q", "k", "v", "log_alpha", "beta")), inp.log_alpha_min)
    A, Bz = kda.segment_summarize(ws, 2 * n_seg, Ts, H, dk, d["q"].dtype, inp.log_alpha_min)
    torch.cuda.synchronize()
    A_ref, B_ref = oracle.kda_summary(seg(f(inp.k)), seg(f(inp.v)), seg(inp.log_alpha), seg(inp.beta),
                                      inp.log_alpha_min)
    ea, eb = slice_err(host(A), A_ref, "state"), slice_err(host(Bz), B_ref, "state")
    note(f"  summary A {ea:.2e} Bz {eb:.2e}")
    assert ea <= TOL[io] and eb <= TOL[io]
    # the merge alone is fp32 on both sides' inputs: feed it the GPU pairs
    seg_in, fin2 = kda.segment_combine(A.view(2, n_seg, H, dk, dk), Bz.view(2, n_seg, H, dk, dk), d["state0"])
    torch.cuda.synchronize()
    si_ref, f_ref = oracle.kda_combine(host(A).reshape(2, n_seg, H, dk, dk), host(Bz).reshape(2, n_seg, H, dk, dk),
                                       inp.state0)
    assert slice_err(host(seg_in).reshape(-1, H, dk, dk), si_ref.reshape(-1, H, dk, dk), "state") < 1e-5
    assert slice_err(host(fin2), f_ref, "state") < 1e-5


# Segments shorter than a chunk, one full chunk, a ragged tail and none at
# all, on both per-wave summary layouts (8 rows x H=4: one slice per wave;
# 8 rows x H=16: two).  An empty segment is the identity map.
@pytest.mark.parametrize("H", [4, 16])
@pytest.mark.parametrize("Ts", [0, 1, 40, 64, 161])
def test_summary_lengths_vs_oracle(H, Ts):
    note(f"[summary lengths] rows=8 H={H} T={Ts}")
    inp = make_inputs(8, Ts, H, 128, 128, io_dtype="bf16", seed=43, alpha_min=0.9, logit_mu=-4.0)
    d = kda.to_device(inp)
    ws = kda.chunk_prepare(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], inp.log_alpha_min)
    A, Bz = kda.segment_summarize(ws, 8, Ts, H, 128, torch.bfloat16, inp.log_alpha_min)
    torch.cuda.synchronize()
    if Ts == 0:
        eye = torch.eye(128, device=DEV).expand(8, H, 128, 128)
        assert torch.equal(A, eye) and not torch.any(Bz)
        return
    f = lambda a: to_f64(a, "bf16")
    A_ref, B_ref = oracle.kda_summary(f(inp.k), f(inp.v), inp.log_alpha, inp.beta, inp.log_alpha_min)
    ea, eb = slice_err(host(A), A_ref, "state"), slice_err(host(Bz), B_ref, "state")
    note(f"  summary A {ea:.2e} Bz {eb:.2e}")
    assert ea <= TOL["bf16"] and eb <= TOL["bf16"]


def _decode_all(d, floor, T):
    """T decode steps; inputs re-laid out step-major so each step's slice is contiguous."""
    sm = {n: d[n].transpose(0, 1).contiguous() for n in ("q", "k", "v", "g", "log_alpha", "beta")}
    state = d["state0"].clone()
    outs = []
    for t in range(T):
        outs.append(kda.decode_step(sm["q"][t], sm["k"][t], sm["v"][t], sm["log_alpha"][t], sm["beta"][t],
                                    sm["g"][t], state, floor))
    torch.cuda.synchronize()
    return torch.stack(outs, 1), state


def test_decode_batched_vs_oracle():
    """256 sequences x 32 heads, d=128, 64 steps, bf16; oracle on 3 sequences x 32 heads."""
    note("[decode] N=256 H=32 d=128 64 steps")
    inp = workload(4)
    d = kda.to_device(inp)
    out, st = _decode_all(d, inp.log_alpha_min, 64)
    rows = [0, 77, 255]
    sub = lambda a: a[rows]
    f = lambda a: to_f64(a, "bf16")
    o_ref, s_ref = oracle.kda_ref(f(sub(inp.q)), f(sub(inp.k)), f(sub(inp.v)), sub(inp.log_alpha), sub(inp.beta),
                                  f(sub(inp.g)), inp.log_alpha_min, sub(inp.state0))
    eo = slice_err(host(out[rows]), o_ref, "out")
    es = slice_err(host(st[rows]), s_ref, "state")
    note(f"  rel-L2 out {eo:.2e} state {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_decode_f32_vs_oracle_and_prefill():
    note("[decode] f32 d=64 and d=128")
    for dk in (64, 128):
        inp = make_inputs(3, 40, 5, dk, dk, io_dtype="f32", seed=9 + dk, alpha_min=0.9, logit_mu=-2.0,
                          with_state0=True)
        d = kda.to_device(inp)
        out, st = _decode_all(d, inp.log_alpha_min, 40)
        o_ref, s_ref = oracle_run(inp)
        eo, es = slice_err(host(out), o_ref, "out"), slice_err(host(st), s_ref, "state")
        note(f"  dk={dk} decode vs oracle: out {eo:.2e} state {es:.2e}")
        assert eo <= TOL["f32"] and es <= TOL["f32"]
        # T decode steps == prefill over the same T tokens
        out_p, st_p = gpu_prefill(d, inp.log_alpha_min)
        assert slice_err(host(out), host(out_p), "out") <= TOL["f32"]
        assert slice_err(host(st), host(st_p), "state") <= TOL["f32"]


def test_resume_in_place_equals_uninterrupted():
    """run(T1) then run(T2 | S_T1) with state_out aliasing state_in == run(T1 + T2) (oracle)."""
    note("[resume] bf16")
    inp = make_inputs(2, 320, 4, 128, 128, io_dtype="bf16", seed=5, alpha_min=0.9, logit_mu=-4.0, with_state0=True)
    d = kda.to_device(inp)
    T1 = 130
    part = lambda sl: {n: (d[n][:, sl].contiguous() if n != "state0" else d[n]) for n in d}
    a, b = part(slice(0, T1)), part(slice(T1, None))
    o1, S = gpu_prefill(a, inp.log_alpha_min)
    ws = kda.chunk_prepare(b["q"], b["k"], b["v"], b["log_alpha"], b["beta"], inp.log_alpha_min)
    o2, S2 = kda.chunk_scan(ws, b["g"], inp.log_alpha_min, state_in=S, state_out=S)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S.data_ptr()
    o_ref, s_ref = oracle_run(inp)
    eo = slice_err(np.concatenate([host(o1), host(o2)], 1), o_ref, "out")
    es = slice_err(host(S), s_ref, "state")
    note(f"  rel-L2 out {eo:.2e} state {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_empty_sequence_and_batch():
    note("[edge] T=0, B=0")
    inp = make_inputs(2, 0, 3, 128, 128, io_dtype="bf16", seed=1, alpha_min=0.9, with_state0=True)
    d = kda.to_device(inp)
    out, st = gpu_prefill(d, inp.log_alpha_min)
    assert out.shape == (2, 0, 3, 128)
    assert torch.equal(st, d["state0"])
    out0, st0 = gpu_prefill(d, inp.log_alpha_min, state_in=None)
    assert torch.count_nonzero(st0) == 0
    e = make_inputs(0, 64, 3, 128, 128, io_dtype="bf16", seed=1, alpha_min=0.9)
    de = kda.to_device(e)
    o, s = gpu_prefill(de, e.log_alpha_min, state_in=None)
    assert o.shape == (0, 64, 3, 128) and s.shape == (0, 3, 128, 128)


def test_bitwise_deterministic():
    note("[determinism]")
    inp = make_inputs(1, 1000, 4, 128, 128, io_dtype="bf16", seed=3, alpha_min=0.9, logit_mu=-4.0)
    d = kda.to_device(inp)
    o1, s1 = gpu_prefill(d, inp.log_alpha_min)
    o2, s2 = gpu_prefill(d, inp.log_alpha_min)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("T,every,io", [(300, 2, "bf16"), (256, 4, "bf16"), (130, 1, "bf16"), (64, 3, "bf16"),
                                       (300, 2, "f32"), (200, 1, "f32")])
def test_scan_checkpoints_match_prefix_runs(T, every, io):
    """Prefix-cache checkpoints: entry j holds the oracle's state after the
    first 64*every*j tokens (to the I/O dtype's bound), is bit-identical to
    the final state of a prefill over that prefix, the last entry is the final
    state, and resuming from a checkpoint reproduces the rest of the outputs
    exactly."""
    note(f"[checkpoints] T={T} every={every} {io}")
    inp = make_inputs(2, T, 3, 64, 64, io_dtype=io, seed=300 + T, alpha_min=0.9, logit_mu=-1.0,
                      with_state0=True)
    d = kda.to_device(inp)
    ws = kda.chunk_prepare(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], inp.log_alpha_min)
    out, st, ck = kda.chunk_scan_checkpoints(ws, d["g"], inp.log_alpha_min, every, state_in=d["state0"])
    torch.cuda.synchronize()
    J = ck.shape[2] - 1
    assert J == ((T + 63) // 64 + every - 1) // every
    assert torch.equal(ck[:, :, J], st)
    assert torch.equal(ck[:, :, 0], d["state0"])
    sl = lambda x, a, b: x[:, a:b].contiguous()
    for j in range(J + 1):
        t = min(64 * every * j, T)
        _, s_ref = oracle_run(inp, T=t)
        e = slice_err(host(ck[:, :, j]), s_ref, "state")
        note(f"  checkpoint {j} (after {t} tokens) vs oracle: {e:.2e}")
        assert e <= TOL[io], j
    for j in range(1, J):
        t = 64 * every * j
        _, st_j = kda.prefill(sl(d["q"], 0, t), sl(d["k"], 0, t), sl(d["v"], 0, t), sl(d["log_alpha"], 0, t),
                              sl(d["beta"], 0, t), sl(d["g"], 0, t), inp.log_alpha_min, state_in=d["state0"])
        torch.cuda.synchronize()
        assert torch.equal(ck[:, :, j], st_j), j
        o_rest, st_rest = kda.prefill(sl(d["q"], t, T), sl(d["k"], t, T), sl(d["v"], t, T),
                                      sl(d["log_alpha"], t, T), sl(d["beta"], t, T), sl(d["g"], t, T),
                                      inp.log_alpha_min, state_in=ck[:, :, j].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o_rest, out[:, t:]), j
        assert torch.equal(st_rest, st), j


@pytest.mark.parametrize("every", [2 ** 31 - 1, 2 ** 31 - 1000, 5])
def test_checkpoints_every_beyond_chunk_count(every):
    """`every` at or past the chunk count (up to INT32_MAX) gives two entries:
    the entering state and the final state."""
    note(f"[checkpoints] every={every}")
    inp = make_inputs(1, 300, 2, 64, 64, io_dtype="bf16", seed=77, alpha_min=0.9, logit_mu=-1.0, with_state0=True)
    d = kda.to_device(inp)
    ws = kda.chunk_prepare(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], inp.log_alpha_min)
    out, st, ck = kda.chunk_scan_checkpoints(ws, d["g"], inp.log_alpha_min, every, state_in=d["state0"])
    out2, st2 = kda.chunk_scan(ws, d["g"], inp.log_alpha_min, state_in=d["state0"])
    torch.cuda.synchronize()
    assert ck.shape[2] == 2
    assert torch.equal(ck[:, :, 0], d["state0"]) and torch.equal(ck[:, :, 1], st)
    assert torch.equal(out, out2) and torch.equal(st, st2)
