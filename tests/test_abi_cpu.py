"""The C ABI library: builds, loads, exports what include/kda.h declares, and
rejects bad arguments synchronously -- all without a GPU."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_91_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
FAKE = 0x10000            # aligned, never dereferenced: validation fails first
MISALIGNED = 0x10008


def _have_gpu():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_91_amd import build
        build.build()
    return kda.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) == 22, names
    assert sorted(kda.EXPORTS) == names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, text in kda.STATUS.items():
        assert L.kda_status_string(code).decode() == text
    assert L.kda_status_string(99).decode() == "unknown status"


def _p(**kw):
    base = dict(batch=2, seqlen=200, heads=3, dk=128, dv=128, io_dtype=kda.KDA_BF16, log_alpha_min=-0.10536)
    base.update(kw)
    return kda.problem(**base)


def test_workspace_size(L):
    p = _p()
    card = 74240          # 3*64*128 + 64*64 + 64*128 bf16 elements, + 128 fp32, rounded to 256 B
    assert L.kda_workspace_size(ctypes.byref(p)) == 2 * 3 * 4 * card
    pf = _p(io_dtype=kda.KDA_F32, dk=64, dv=64)
    assert L.kda_workspace_size(ctypes.byref(pf)) == 2 * 3 * 4 * 82176
    for bad in (_p(dk=96, dv=96), _p(dk=64, dv=128), _p(chunk=32), _p(heads=0), _p(seqlen=-1),
                _p(log_alpha_min=0.0), _p(log_alpha_min=-2.0), _p(log_alpha_min=float("nan")),
                _p(io_dtype=7)):
        assert L.kda_workspace_size(ctypes.byref(bad)) == 0
    assert L.kda_workspace_size(None) == 0


def test_prepare_argument_errors(L):
    p = _p()
    ws = L.kda_workspace_size(ctypes.byref(p))
    call = lambda pr=p, q=FAKE, k=FAKE, v=FAKE, la=FAKE, b=FAKE, w=FAKE, n=ws: L.kda_chunk_prepare(
        ctypes.byref(pr) if pr is not None else None, q, k, v, la, b, w, n, None)
    assert call(pr=None) == 1
    assert call(q=None) == 1
    assert call(k=MISALIGNED) == 1
    assert call(w=None) == 1
    assert call(n=ws - 1) == 3
    assert call(pr=_p(dk=96, dv=96)) == 2
    assert call(pr=_p(chunk=128)) == 2
    assert call(pr=_p(log_alpha_min=0.5)) == 1
    # empty problems need no pointers and touch no device
    assert call(pr=_p(seqlen=0), q=None, k=None, v=None, la=None, b=None, w=None, n=0) == 0
    assert call(pr=_p(batch=0), q=None, k=None, v=None, la=None, b=None, w=None, n=0) == 0


def test_scan_summarize_combine_decode_argument_errors(L):
    p = _p()
    ws = L.kda_workspace_size(ctypes.byref(p))
    ck = lambda every=2, c=FAKE: L.kda_chunk_scan_checkpoints(ctypes.byref(p), FAKE, ws, FAKE, None, FAKE, None,
                                                              every, c, None)
    assert ck(every=0) == 1
    assert ck(c=None) == 1
    assert ck(c=MISALIGNED) == 1
    assert L.kda_chunk_scan(ctypes.byref(p), FAKE, ws, None, None, FAKE, None, None) == 1
    assert L.kda_chunk_scan(ctypes.byref(p), FAKE, ws, FAKE, MISALIGNED, FAKE, None, None) == 1
    assert L.kda_chunk_scan(ctypes.byref(p), FAKE, ws - 256, FAKE, None, FAKE, None, None) == 3
    assert L.kda_segment_summarize(ctypes.byref(p), FAKE, ws, None, FAKE, None) == 1
    assert L.kda_segment_summarize(ctypes.byref(_p(dk=64, dv=128)), FAKE, ws, FAKE, FAKE, None) == 2
    assert L.kda_segment_combine(1, 4, 2, 128, 128, None, FAKE, None, FAKE, None, None) == 1
    assert L.kda_segment_combine(1, 4, 2, 96, 96, FAKE, FAKE, None, FAKE, None, None) == 2
    assert L.kda_segment_combine(-1, 4, 2, 128, 128, FAKE, FAKE, None, FAKE, None, None) == 1
    assert L.kda_segment_combine(0, 4, 2, 128, 128, None, None, None, None, None, None) == 0
    dec = lambda **kw: L.kda_decode_step(*[kw.get(n, d) for n, d in [
        ("N", 4), ("H", 2), ("dk", 128), ("dv", 128), ("io", kda.KDA_BF16), ("fl", -0.1), ("q", FAKE),
        ("k", FAKE), ("v", FAKE), ("la", FAKE), ("b", FAKE), ("g", FAKE), ("s", FAKE), ("o", FAKE),
        ("st", None)]])
    assert dec(q=None) == 1
    assert dec(s=MISALIGNED) == 1
    assert dec(dk=64) == 2
    assert dec(io=3) == 1
    assert dec(fl=1.0) == 1
    assert dec(N=0, q=None, k=None, v=None, la=None, b=None, g=None, s=None, o=None) == 0


def _bwd(L, pr, ws, **kw):
    names = ["q", "k", "v", "la", "b", "g", "s0", "do", "ds", "dq", "dk", "dv", "dla", "db", "dg", "ds0", "w"]
    vals = {n: FAKE for n in names}
    vals.update(s0=None, do=FAKE, ds=None, ds0=FAKE)
    vals.update(kw)
    n = kw.get("n", ws)
    return L.kda_backward(ctypes.byref(pr) if pr is not None else None, *[vals[x] for x in names], n, None)


def test_backward_workspace_and_argument_errors(L):
    p = _p()
    ws = L.kda_backward_workspace_size(ctypes.byref(p))
    # forward cards, reverse-pass cards (4 x 64x128 + 64x128 bf16 + 128 fp32),
    # the forward output, and fp32 states: the one entering every chunk plus
    # the final one, and the gradient of the state leaving every chunk
    chunks = 2 * 3 * 4
    assert ws == chunks * 74240 + chunks * 82432 + 2 * 200 * 3 * 128 * 2 + (2 * chunks + 2 * 3) * 128 * 128 * 4
    assert L.kda_backward_workspace_size(ctypes.byref(_p(seqlen=0))) == 0
    assert L.kda_backward_workspace_size(ctypes.byref(_p(dk=96, dv=96))) == 0
    assert _bwd(L, None, ws) == 1
    assert _bwd(L, p, ws, q=None) == 1
    assert _bwd(L, p, ws, dla=None) == 1
    assert _bwd(L, p, ws, dg=MISALIGNED) == 1
    assert _bwd(L, p, ws, do=MISALIGNED) == 1
    assert _bwd(L, p, ws, w=None) == 1
    assert _bwd(L, p, ws, n=ws - 1) == 3
    assert _bwd(L, _p(dk=64, dv=128), ws) == 2
    assert _bwd(L, _p(log_alpha_min=0.5), ws) == 1
    # nothing to do: no rows, or no tokens and no state gradient wanted
    none = {n: None for n in ["q", "k", "v", "la", "b", "g", "dq", "dk", "dv", "dla", "db", "dg", "w"]}
    assert _bwd(L, _p(batch=0), 0, ds0=None, **none) == 0
    assert _bwd(L, _p(seqlen=0), 0, ds0=None, **none) == 0


def test_varlen_workspace_and_argument_errors(L):
    p = _p(batch=1, seqlen=1000)
    # chunk offsets (11 int64 -> 256 B), the sequence of each of at most ceil(1000/64) + 10 = 26
    # chunks (4 B each -> 256 B), then 26 chunks of cards per head
    assert L.kda_varlen_workspace_size(ctypes.byref(p), 10) == 256 + 256 + (16 + 10) * 3 * 74240
    assert L.kda_varlen_workspace_size(ctypes.byref(_p()), 10) == 0          # batch must be 1
    assert L.kda_varlen_workspace_size(ctypes.byref(p), -1) == 0
    ws = L.kda_varlen_workspace_size(ctypes.byref(p), 10)
    prep = lambda pr=p, ns=10, cu=FAKE, w=FAKE, n=ws, q=FAKE: L.kda_varlen_prepare(
        ctypes.byref(pr), ns, cu, q, FAKE, FAKE, FAKE, FAKE, w, n, None)
    assert prep(cu=None) == 1
    assert prep(cu=FAKE + 2) == 1       # int32 offsets need 4-byte alignment
    assert prep(q=MISALIGNED) == 1
    assert prep(n=ws - 1) == 3
    assert prep(pr=_p(batch=2, seqlen=1000)) == 1
    assert prep(pr=_p(batch=1, seqlen=1000, dk=96, dv=96)) == 2
    assert prep(ns=0, cu=None, w=None, n=0) == 0
    scan = lambda ns=10, cu=FAKE, g=FAKE, si=None, so=None: L.kda_varlen_scan(
        ctypes.byref(p), ns, cu, FAKE, ws, g, si, FAKE, so, None)
    assert scan(cu=None) == 1
    assert scan(g=None) == 1
    assert scan(si=MISALIGNED) == 1
    assert scan(ns=0, cu=None) == 0


def _vbwd(L, pr, ns, ws, **kw):
    names = ["cu", "q", "k", "v", "la", "b", "g", "s0", "do", "ds", "dq", "dk", "dv", "dla", "db", "dg", "ds0", "w"]
    vals = {n: FAKE for n in names}
    vals.update(s0=None, ds=None)
    vals.update(kw)
    n = kw.get("n", ws)
    return L.kda_varlen_backward(ctypes.byref(pr), ns, *[vals[x] for x in names], n, None)


def test_varlen_backward_workspace_and_argument_errors(L):
    p = _p(batch=1, seqlen=1000)
    up = lambda x: (x + 255) // 256 * 256
    # chunk offsets, the sequence of each of at most ceil(1000/64) + 10 = 26
    # chunks, then per chunk-head (26 x 3): forward card, reverse card, the
    # forward output, and two fp32 states (entering, gradient leaving)
    c = (16 + 10) * 3
    want = (up(11 * 8) + up(26 * 4) + up(c * 74240) + up(c * 82432) + up(1000 * 3 * 128 * 2)
            + 2 * up(c * 128 * 128 * 4))
    ws = L.kda_varlen_backward_workspace_size(ctypes.byref(p), 10)
    assert ws == want
    assert L.kda_varlen_backward_workspace_size(ctypes.byref(_p()), 10) == 0        # batch must be 1
    assert L.kda_varlen_backward_workspace_size(ctypes.byref(p), 0) == 0
    assert L.kda_varlen_backward_workspace_size(ctypes.byref(_p(batch=1, seqlen=0)), 3) == 0
    assert _vbwd(L, p, 10, ws, cu=None) == 1
    assert _vbwd(L, p, 10, ws, cu=FAKE + 2) == 1      # int32 offsets need 4-byte alignment
    assert _vbwd(L, p, 10, ws, q=MISALIGNED) == 1
    assert _vbwd(L, p, 10, ws, dla=None) == 1
    assert _vbwd(L, p, 10, ws, s0=MISALIGNED) == 1
    assert _vbwd(L, p, 10, ws, w=None) == 1
    assert _vbwd(L, p, 10, ws, n=ws - 1) == 3
    assert _vbwd(L, _p(batch=2, seqlen=1000), 10, ws) == 1
    assert _vbwd(L, _p(batch=1, seqlen=1000, dk=96, dv=96), 10, ws) == 2
    assert _vbwd(L, p, -1, ws) == 1
    # nothing to do: no sequences, or no tokens and no state gradient wanted
    none = {n: None for n in ["q", "k", "v", "la", "b", "g", "dq", "dk", "dv", "dla", "db", "dg", "w", "ds0"]}
    assert _vbwd(L, p, 0, 0, cu=None, w=None, ds0=None) == 0
    assert _vbwd(L, _p(batch=1, seqlen=0), 3, 0, **none) == 0


def test_varlen_split_pair_argument_errors(L):
    p = _p(batch=1, seqlen=1000)
    ws = L.kda_varlen_backward_workspace_size(ctypes.byref(p), 10)
    fwd = lambda pr=p, ns=10, cu=FAKE, q=FAKE, o=FAKE, w=FAKE, n=ws, so=None: L.kda_varlen_prefill_for_backward(
        ctypes.byref(pr), ns, cu, q, FAKE, FAKE, FAKE, FAKE, FAKE, None, o, so, w, n, None)
    assert fwd(cu=None) == 1
    assert fwd(q=None) == 1
    assert fwd(o=None) == 1
    assert fwd(w=None) == 1
    assert fwd(n=ws - 1) == 3
    assert fwd(pr=_p(batch=2, seqlen=1000)) == 1
    assert fwd(ns=0, cu=None, w=None, n=0) == 0
    assert fwd(pr=_p(batch=1, seqlen=0), q=None, o=None, w=None, n=0) == 0    # no tokens, no state_out
    names = ["cu", "q", "k", "v", "la", "b", "g", "o", "do", "ds", "dq", "dk", "dv", "dla", "db", "dg", "ds0", "w"]

    def bwd(pr=p, ns=10, n=ws, **kw):
        vals = {x: FAKE for x in names}
        vals.update(ds=None, ds0=None)
        vals.update(kw)
        return L.kda_varlen_backward_after_prefill(ctypes.byref(pr), ns, *[vals[x] for x in names], n, None)

    assert bwd(cu=None) == 1
    assert bwd(o=None) == 1
    assert bwd(dq=MISALIGNED) == 1
    assert bwd(n=ws - 1) == 3
    assert bwd(ns=0, cu=None, w=None, n=0) == 0


@pytest.mark.skipif(_have_gpu(), reason="only meaningful where no HIP device exists")
def test_valid_call_without_device_reports_hip_error(L):
    p = _p()
    ws = L.kda_workspace_size(ctypes.byref(p))
    assert L.kda_chunk_prepare(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == 4
    assert L.kda_decode_step(4, 2, 128, 128, 1, -0.1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 4
    assert _bwd(L, p, L.kda_backward_workspace_size(ctypes.byref(p))) == 4


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(kda, "LIB_PATH", "/nonexistent/libkda.so")
    monkeypatch.setattr(kda, "_lib", None)
    with pytest.raises(ImportError):
        kda.lib()


def test_beta_needs_only_natural_alignment(L):
    p = _p()
    ws = L.kda_workspace_size(ctypes.byref(p))
    # 4-byte aligned beta passes validation (then fails only for lack of a device / or is a real call)
    if not _have_gpu():
        assert L.kda_chunk_prepare(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE, ws, None) == 4
    assert L.kda_chunk_prepare(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE + 2, FAKE, ws, None) == 1


def _prefill_args(B=2, T=70, H=3, d=64, io="bfloat16"):
    import torch
    dt = getattr(torch, io)
    return dict(q=torch.zeros(B, T, H, d, dtype=dt), k=torch.zeros(B, T, H, d, dtype=dt),
                v=torch.zeros(B, T, H, d, dtype=dt), log_alpha=torch.zeros(B, T, H, d),
                beta=torch.zeros(B, T, H), g=torch.zeros(B, T, H, d, dtype=dt))


@pytest.mark.parametrize("bad,err", [
    (dict(k=("shape", (2, 70, 3, 32))), ValueError),
    (dict(v=("shape", (2, 69, 3, 64))), ValueError),
    (dict(log_alpha=("dtype", "bfloat16")), TypeError),
    (dict(beta=("shape", (2, 70))), ValueError),
    (dict(k=("dtype", "float32")), TypeError),
])
def test_binding_rejects_mismatched_prefill_inputs(L, bad, err):
    """Every extent the kernels read is implied by q and v: a tensor that does
    not match them is refused before any pointer reaches the library."""
    import torch
    a = _prefill_args()
    (name, (kind, val)), = bad.items()
    a[name] = torch.zeros(val, dtype=a[name].dtype) if kind == "shape" else a[name].to(getattr(torch, val))
    with pytest.raises(err, match=name):
        kda.chunk_prepare(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], -0.1)
    with pytest.raises(err, match=name):
        kda.backward(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["g"], -0.1)


def test_binding_rejects_mismatched_scan_decode_combine_args(L):
    import torch
    a = _prefill_args()
    ws = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="state_in"):
        kda.chunk_scan(ws, a["g"], -0.1, state_in=torch.zeros(2, 3, 64, 32))
    with pytest.raises(ValueError, match="out"):
        kda.chunk_scan(ws, a["g"], -0.1, out=torch.zeros(2, 70, 3, 32, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="workspace"):
        kda.chunk_scan(torch.zeros(4, dtype=torch.float32), a["g"], -0.1)
    N, H, d = 5, 3, 64
    q = torch.zeros(N, H, d, dtype=torch.bfloat16)
    st = torch.zeros(N, H, d, d)
    with pytest.raises(ValueError, match="state"):
        kda.decode_step(q, q, q, torch.zeros(N, H, d), torch.zeros(N, H), q, torch.zeros(N, H, d, 32), -0.1)
    with pytest.raises(TypeError, match="log_alpha"):
        kda.decode_step(q, q, q, torch.zeros(N, H, d, dtype=torch.bfloat16), torch.zeros(N, H), q, st, -0.1)
    with pytest.raises(ValueError, match="zero_state"):
        kda.segment_combine(torch.zeros(1, 4, H, d, d), torch.zeros(1, 3, H, d, d))
    with pytest.raises(TypeError, match="cu_seqlens"):
        kda.varlen_prepare(*(_prefill_args(B=1)[n] for n in ("q", "k", "v", "log_alpha", "beta")), -0.1,
                           torch.zeros(3, dtype=torch.int64))


@pytest.mark.skipif(_have_gpu(), reason="only meaningful where no HIP device exists")
def test_checkpoint_every_accepts_the_whole_int32_range(L):
    """every up to INT32_MAX is valid (values above the chunk count act as the
    chunk count); with no device the call gets past validation to the HIP
    error, and every < 1 is an invalid argument."""
    p = _p()
    ws = L.kda_workspace_size(ctypes.byref(p))
    ck = lambda every: L.kda_chunk_scan_checkpoints(ctypes.byref(p), FAKE, ws, FAKE, None, FAKE, None, every,
                                                    FAKE, None)
    for every in (1, 4, 5, 2 ** 31 - 1024, 2 ** 31 - 1):
        assert ck(every) == 4, every
    for every in (0, -1, -(2 ** 31)):
        assert ck(every) == 1, every


def test_binding_checks_checkpoint_every():
    """The binding refuses an `every` the C int32 argument cannot carry (ctypes
    would truncate 2**32 + 1 to 1 and size the checkpoint tensor wrongly)."""
    import torch
    g = torch.zeros(1, 200, 2, 64, dtype=torch.bfloat16)
    ws = torch.zeros(16, dtype=torch.uint8)
    for every in (0, -3, 2 ** 31, 2 ** 32 + 1, 1.5):
        with pytest.raises(ValueError, match="every"):
            kda.chunk_scan_checkpoints(ws, g, -0.1, every)


def test_prefill_noalloc_rejects_what_its_scratch_cannot_hold(L):
    """kda_prefill_noalloc needs the cards of one chunk for every (row, head)
    to fit its fixed scratch area beside the carried state; larger batches
    are refused before any launch, and bad pointers as for prefill."""
    card = 74240
    assert kda.NOALLOC_SCRATCH_BYTES // card == 903
    call = lambda pr, so=None, q=FAKE: L.kda_prefill_noalloc(ctypes.byref(pr), q, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                            None, FAKE, so, None)
    assert call(_p(batch=904, heads=1)) == 3
    assert call(_p(batch=1, heads=904), so=FAKE) == 3
    assert call(_p(), q=None) == 1
    assert call(_p(), q=MISALIGNED) == 1
    assert call(_p(log_alpha_min=0.5)) == 1
    assert call(_p(dk=64, dv=128)) == 2
    if not _have_gpu():   # valid arguments get past validation to the (missing) device
        assert call(_p(batch=903, heads=1), so=FAKE) == 4
        assert call(_p()) == 4


def test_pipelined_workspace_and_argument_errors(L):
    """kda_prefill_pipelined: the workspace is the carried state plus one
    range's cards, twice when the sequence spans several ranges; bad ranges,
    pointers and workspaces are refused before any launch."""
    card, state = 74240, 2 * 3 * 128 * 128 * 4            # _p(): B=2, H=3, T=200 -> 4 chunks
    size = lambda pr, rc: L.kda_pipelined_workspace_size(ctypes.byref(pr), rc)
    assert size(_p(), 1) == state + 2 * ((1 * 6 * card + 255) // 256 * 256)
    assert size(_p(), 3) == state + 2 * 3 * 6 * card
    assert size(_p(), 4) == state + 4 * 6 * card           # one range: one buffer
    assert size(_p(), 2 ** 31 - 1) == state + 4 * 6 * card
    assert size(_p(seqlen=0), 8) == state
    assert size(_p(), 0) == 0 and size(_p(), -5) == 0
    assert size(_p(dk=96, dv=96), 4) == 0
    ws = size(_p(), 2)
    call = lambda pr=_p(), rc=2, w=FAKE, n=ws, q=FAKE, so=None: L.kda_prefill_pipelined(
        ctypes.byref(pr), q, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, so, rc, w, n, None, None)
    assert call(rc=0) == 1
    assert call(rc=-1) == 1
    assert call(q=None) == 1
    assert call(q=MISALIGNED) == 1
    assert call(w=None) == 1
    assert call(w=MISALIGNED) == 1
    assert call(n=ws - 1) == 3
    assert call(pr=_p(log_alpha_min=0.5)) == 1
    assert call(pr=_p(dk=64, dv=128)) == 2
    assert call(pr=_p(batch=0), w=None, n=0) == 0
    if not _have_gpu():   # valid arguments get past validation to the (missing) device
        assert call() == 4
        assert call(pr=_p(seqlen=0), w=None, n=size(_p(seqlen=0), 2), so=FAKE) == 4


def test_binding_checks_range_chunks():
    for rc in (0, -1, 2 ** 31, 1.5):
        with pytest.raises(ValueError, match="range_chunks"):
            kda._range_chunks(rc)


def test_prefill_for_backward_and_backward_after_prefill_argument_errors(L):
    """The split training pair takes a kda_backward workspace; the backward
    half also needs the forward output.  Bad arguments are refused before
    any launch."""
    p = _p()
    ws = L.kda_backward_workspace_size(ctypes.byref(p))
    fwd = lambda pr=p, q=FAKE, o=FAKE, w=FAKE, n=ws, si=None, so=None: L.kda_prefill_for_backward(
        ctypes.byref(pr), q, FAKE, FAKE, FAKE, FAKE, FAKE, si, o, so, w, n, None)
    assert fwd(q=None) == 1
    assert fwd(o=None) == 1
    assert fwd(o=MISALIGNED) == 1
    assert fwd(w=None) == 1
    assert fwd(si=MISALIGNED) == 1
    assert fwd(n=ws - 1) == 3
    assert fwd(pr=_p(dk=64, dv=128)) == 2
    assert fwd(pr=_p(batch=0), q=None, o=None, w=None, n=0) == 0
    assert fwd(pr=_p(seqlen=0), q=None, o=None, w=None, n=0) == 0        # no state_out: nothing to do
    bwd = lambda pr=p, o=FAKE, w=FAKE, n=ws, dq=FAKE, dsi=None: L.kda_backward_after_prefill(
        ctypes.byref(pr), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, o, None, None, dq, FAKE, FAKE, FAKE, FAKE, FAKE,
        dsi, w, n, None)
    assert bwd(o=None) == 1
    assert bwd(o=MISALIGNED) == 1
    assert bwd(dq=None) == 1
    assert bwd(w=None) == 1
    assert bwd(n=ws - 1) == 3
    assert bwd(pr=_p(log_alpha_min=0.5)) == 1
    assert bwd(pr=_p(seqlen=0), o=None, w=None, n=0, dq=None) == 0      # no d_state_in: nothing to do
    if not _have_gpu():   # valid arguments get past validation to the (missing) device
        assert fwd() == 4
        assert bwd() == 4
