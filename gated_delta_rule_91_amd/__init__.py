"""MI355X-native KDA (Kimi Delta Attention) token mixer.

A thin Python binding over the C ABI of ``libkda.so`` (``include/kda.h``).
Every step of the mixer runs in the library's HIP kernels; this module only
checks tensor dtypes/shapes, passes device pointers and the current HIP
stream, and allocates the update-card workspace with PyTorch.  There is no
CPU or PyTorch fallback: if the library is missing, every call raises.

Entry points (same names as the C ABI, minus the ``kda_`` prefix):
    workspace_size, chunk_prepare, chunk_scan, chunk_scan_checkpoints, segment_summarize,
    segment_combine, decode_step, backward_workspace_size, backward,
    varlen_workspace_size, varlen_prepare, varlen_scan, prefill_for_backward,
    backward_after_prefill, pipelined_workspace_size, varlen_backward_workspace_size,
    varlen_backward, varlen_prefill_for_backward, varlen_backward_after_prefill
Conveniences built from them: prefill, segmented_prefill, varlen_prefill, and
prefill_autograd (a torch.autograd.Function over the split training pair).
prefill_pipelined calls kda_prefill_pipelined (chunk ranges, the next range's
cards prepared on a second stream during the current range's scan);
prefill_noalloc calls kda_prefill_noalloc, which needs no workspace.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
# another build of the library to load instead (the sanitizer tests set it)
LIB_PATH = os.environ.get("KDA_LIB") or os.path.join(_PKG, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape or dtype", 3: "workspace too small",
          4: "HIP runtime error"}
EXPORTS = ("kda_workspace_size", "kda_chunk_prepare", "kda_chunk_scan", "kda_chunk_scan_checkpoints",
           "kda_segment_summarize",
           "kda_segment_combine", "kda_decode_step", "kda_backward_workspace_size", "kda_backward",
           "kda_varlen_workspace_size", "kda_varlen_prepare", "kda_varlen_scan",
           "kda_prefill_for_backward", "kda_backward_after_prefill", "kda_pipelined_workspace_size",
           "kda_prefill_pipelined", "kda_prefill_noalloc", "kda_varlen_backward_workspace_size",
           "kda_varlen_backward", "kda_varlen_prefill_for_backward", "kda_varlen_backward_after_prefill",
           "kda_status_string")
# bytes of kda_prefill_noalloc's fixed per-GPU scratch area (KDA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


class KdaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({code})")
        self.code = code


class KdaProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("heads", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("log_alpha_min", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkda.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m gated_delta_rule_91_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        PP = ctypes.POINTER(KdaProblem)
        L.kda_workspace_size.argtypes = [PP]
        L.kda_workspace_size.restype = SZ
        L.kda_chunk_prepare.argtypes = [PP, P, P, P, P, P, P, SZ, P]
        L.kda_chunk_scan.argtypes = [PP, P, SZ, P, P, P, P, P]
        L.kda_chunk_scan_checkpoints.argtypes = [PP, P, SZ, P, P, P, P, I32, P, P]
        L.kda_segment_summarize.argtypes = [PP, P, SZ, P, P, P]
        L.kda_segment_combine.argtypes = [I64, I32, I32, I32, I32, P, P, P, P, P, P]
        L.kda_decode_step.argtypes = [I64, I32, I32, I32, I32, F32, P, P, P, P, P, P, P, P, P]
        L.kda_backward_workspace_size.argtypes = [PP]
        L.kda_backward_workspace_size.restype = SZ
        L.kda_backward.argtypes = [PP] + [P] * 16 + [P, SZ, P]
        L.kda_varlen_workspace_size.argtypes = [PP, I64]
        L.kda_varlen_workspace_size.restype = SZ
        L.kda_varlen_prepare.argtypes = [PP, I64, P, P, P, P, P, P, P, SZ, P]
        L.kda_varlen_scan.argtypes = [PP, I64, P, P, SZ, P, P, P, P, P]
        L.kda_prefill_for_backward.argtypes = [PP] + [P] * 10 + [SZ, P]
        L.kda_backward_after_prefill.argtypes = [PP] + [P] * 17 + [SZ, P]
        L.kda_pipelined_workspace_size.argtypes = [PP, I32]
        L.kda_pipelined_workspace_size.restype = SZ
        L.kda_prefill_pipelined.argtypes = [PP, P, P, P, P, P, P, P, P, P, I32, P, SZ, P, P]
        L.kda_prefill_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P, P, P]
        L.kda_varlen_backward_workspace_size.argtypes = [PP, I64]
        L.kda_varlen_backward_workspace_size.restype = SZ
        L.kda_varlen_backward.argtypes = [PP, I64] + [P] * 17 + [P, SZ, P]
        L.kda_varlen_prefill_for_backward.argtypes = [PP, I64] + [P] * 10 + [P, SZ, P]
        L.kda_varlen_backward_after_prefill.argtypes = [PP, I64] + [P] * 17 + [P, SZ, P]
        for f in EXPORTS[1:-1]:
            if not f.endswith("workspace_size"):
                getattr(L, f).restype = I32
        L.kda_status_string.argtypes = [I32]
        L.kda_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(fn: str, code: int):
    if code != 0:
        raise KdaError(fn, code)


def _torch():
    import torch
    return torch


def _io_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.bfloat16:
        return KDA_BF16
    if dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"q/k/v/g must be bfloat16 or float32, got {dtype}")


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if not x.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not x.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return x.data_ptr()


def _stream(stream=None, device=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _expect(name: str, x, shape, dtype, device):
    """Shape, dtype and device of an argument, checked before any pointer is
    taken: the kernels trust every extent the problem implies."""
    if x is None:
        return
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {tuple(shape)}")
    if x.dtype != dtype:
        raise TypeError(f"{name} has dtype {x.dtype}, expected {dtype}")
    if x.device != device:
        raise ValueError(f"{name} is on {x.device}, expected {device}")


def _expect_workspace(ws, device):
    torch = _torch()
    if ws.dtype != torch.uint8 or ws.dim() != 1:
        raise TypeError("the workspace must be a 1-D uint8 tensor")
    if ws.device != device:
        raise ValueError(f"the workspace is on {ws.device}, expected {device}")


def _expect_prefill_inputs(q, k, v, log_alpha, beta):
    """q, k, log_alpha [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H]; q/k/v share a dtype."""
    torch = _torch()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be [B, T, H, d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _io_code(q.dtype)
    _expect("k", k, (B, T, H, dk), q.dtype, q.device)
    _expect("v", v, (B, T, H, dv), q.dtype, q.device)
    _expect("log_alpha", log_alpha, (B, T, H, dk), torch.float32, q.device)
    _expect("beta", beta, (B, T, H), torch.float32, q.device)


def problem(batch: int, seqlen: int, heads: int, dk: int, dv: int, io_dtype: int, log_alpha_min: float,
            chunk: int = 64) -> KdaProblem:
    return KdaProblem(batch, seqlen, heads, dk, dv, chunk, io_dtype, float(log_alpha_min))


def _problem_of(q, v, log_alpha_min, chunk=64) -> KdaProblem:
    B, T, H, dk = q.shape
    return problem(B, T, H, dk, v.shape[-1], _io_code(q.dtype), log_alpha_min, chunk)


def workspace_size(p: KdaProblem) -> int:
    n = lib().kda_workspace_size(ctypes.byref(p))
    if n == 0 and p.batch * p.heads * p.seqlen > 0:
        raise KdaError("kda_workspace_size", 2)
    return n


def chunk_prepare(q, k, v, log_alpha, beta, log_alpha_min: float, workspace=None, stream=None):
    """Stage 1: update cards for every chunk.  Returns the workspace (uint8 tensor)."""
    torch = _torch()
    _expect_prefill_inputs(q, k, v, log_alpha, beta)
    p = _problem_of(q, v, log_alpha_min)
    nbytes = workspace_size(p)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _expect_workspace(workspace, q.device)
    _check("kda_chunk_prepare", lib().kda_chunk_prepare(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(workspace),
        workspace.numel(), _stream(stream, q.device)))
    return workspace


def chunk_scan(workspace, g, log_alpha_min: float, state_in=None, out=None, state_out=None,
               want_state: bool = True, stream=None):
    """Stage 2: ordered hand-off + gated read-out.  Returns (out, state_out)."""
    torch = _torch()
    B, T, H, dv = g.shape
    p = problem(B, T, H, dv, dv, _io_code(g.dtype), log_alpha_min)
    _expect_workspace(workspace, g.device)
    _expect("state_in", state_in, (B, H, dv, dv), torch.float32, g.device)
    _expect("out", out, g.shape, g.dtype, g.device)
    _expect("state_out", state_out, (B, H, dv, dv), torch.float32, g.device)
    if out is None:
        out = torch.empty_like(g)
    if state_out is None and want_state:
        state_out = torch.empty((B, H, dv, dv), dtype=torch.float32, device=g.device)
    _check("kda_chunk_scan", lib().kda_chunk_scan(
        ctypes.byref(p), _ptr(workspace), workspace.numel(), _ptr(g), _ptr(state_in), _ptr(out),
        _ptr(state_out), _stream(stream, g.device)))
    return out, state_out


def chunk_scan_checkpoints(workspace, g, log_alpha_min: float, every: int, state_in=None, out=None,
                           state_out=None, stream=None):
    """Stage 2 plus prefix-cache checkpoints.  Returns (out, state_out, checkpoints
    [B, H, J+1, dk, dv]) with J = ceil(ceil(T/64) / every): entry j < J is the state
    after 64*every*j tokens, entry J the final state."""
    torch = _torch()
    if not isinstance(every, int) or not 1 <= every <= 2 ** 31 - 1:
        raise ValueError(f"every must be an int in [1, 2**31 - 1], got {every!r}")
    B, T, H, dv = g.shape
    p = problem(B, T, H, dv, dv, _io_code(g.dtype), log_alpha_min)
    nc = (T + 63) // 64
    every = min(every, max(nc, 1))   # the library clamps the same way; the slots are unchanged
    J = (nc + every - 1) // every
    _expect_workspace(workspace, g.device)
    _expect("state_in", state_in, (B, H, dv, dv), torch.float32, g.device)
    _expect("out", out, g.shape, g.dtype, g.device)
    _expect("state_out", state_out, (B, H, dv, dv), torch.float32, g.device)
    if out is None:
        out = torch.empty_like(g)
    if state_out is None:
        state_out = torch.empty((B, H, dv, dv), dtype=torch.float32, device=g.device)
    ck = torch.empty((B, H, J + 1, dv, dv), dtype=torch.float32, device=g.device)
    _check("kda_chunk_scan_checkpoints", lib().kda_chunk_scan_checkpoints(
        ctypes.byref(p), _ptr(workspace), workspace.numel(), _ptr(g), _ptr(state_in), _ptr(out), _ptr(state_out),
        int(every), _ptr(ck), _stream(stream, g.device)))
    return out, state_out, ck


def segment_summarize(workspace, batch: int, seqlen: int, heads: int, dk: int, io_dtype, log_alpha_min: float,
                      stream=None):
    """(transition [B,H,dk,dk], zero_state [B,H,dk,dv]) of each (row, head) from its cards."""
    torch = _torch()
    p = problem(batch, seqlen, heads, dk, dk, _io_code(io_dtype), log_alpha_min)
    _expect_workspace(workspace, workspace.device)
    A = torch.empty((batch, heads, dk, dk), dtype=torch.float32, device=workspace.device)
    Bz = torch.empty((batch, heads, dk, dk), dtype=torch.float32, device=workspace.device)
    _check("kda_segment_summarize", lib().kda_segment_summarize(
        ctypes.byref(p), _ptr(workspace), workspace.numel(), _ptr(A), _ptr(Bz), _stream(stream, workspace.device)))
    return A, Bz


def segment_combine(transition, zero_state, state_init=None, stream=None):
    """In-order merge.  transition [B,n,H,dk,dk], zero_state [B,n,H,dk,dv] ->
    (state entering each segment [B,n,H,dk,dv], final state [B,H,dk,dv])."""
    torch = _torch()
    if transition.dim() != 5 or zero_state.dim() != 5:
        raise ValueError("transition and zero_state must be [B, n_seg, H, dk, d]")
    B, n, H, dk, _ = transition.shape
    dv = zero_state.shape[-1]
    dev = transition.device
    _expect("transition", transition, (B, n, H, dk, dk), torch.float32, dev)
    _expect("zero_state", zero_state, (B, n, H, dk, dv), torch.float32, dev)
    _expect("state_init", state_init, (B, H, dk, dv), torch.float32, dev)
    seg_in = torch.empty_like(zero_state)
    fin = torch.empty((B, H, dk, dv), dtype=torch.float32, device=zero_state.device)
    _check("kda_segment_combine", lib().kda_segment_combine(
        B, n, H, dk, dv, _ptr(transition), _ptr(zero_state), _ptr(state_init), _ptr(seg_in), _ptr(fin),
        _stream(stream, dev)))
    return seg_in, fin


def decode_step(q, k, v, log_alpha, beta, g, state, log_alpha_min: float, out=None, stream=None):
    """One token per sequence: q,k,log_alpha [N,H,dk]; v,g [N,H,dv]; beta [N,H];
    state [N,H,dk,dv] fp32 updated in place.  Returns out [N,H,dv]."""
    torch = _torch()
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q and v must be [N, H, d]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev, io = q.device, q.dtype
    _io_code(io)
    _expect("k", k, (N, H, dk), io, dev)
    _expect("v", v, (N, H, dv), io, dev)
    _expect("log_alpha", log_alpha, (N, H, dk), torch.float32, dev)
    _expect("beta", beta, (N, H), torch.float32, dev)
    _expect("g", g, (N, H, dv), io, dev)
    _expect("state", state, (N, H, dk, dv), torch.float32, dev)
    _expect("out", out, (N, H, dv), io, dev)
    if out is None:
        out = torch.empty_like(g)
    _check("kda_decode_step", lib().kda_decode_step(
        N, H, dk, dv, _io_code(q.dtype), float(log_alpha_min), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
        _ptr(beta), _ptr(g), _ptr(state), _ptr(out), _stream(stream, dev)))
    return out


def backward_workspace_size(p: KdaProblem) -> int:
    n = lib().kda_backward_workspace_size(ctypes.byref(p))
    if n == 0 and p.batch * p.heads * p.seqlen > 0:
        raise KdaError("kda_backward_workspace_size", 2)
    return n


def backward(q, k, v, log_alpha, beta, g, log_alpha_min: float, state_in=None, d_out=None, d_state=None,
             want_dstate: bool = True, workspace=None, stream=None) -> dict:
    """Gradients of <d_out, out> + <d_state, final state> with respect to every
    input of prefill.  Returns a dict with dq, dk, dv, dg (dtype of q), dlog_alpha,
    dbeta (fp32) and dstate0 ([B,H,dk,dv] fp32, None unless want_dstate)."""
    torch = _torch()
    _expect_prefill_inputs(q, k, v, log_alpha, beta)
    p = _problem_of(q, v, log_alpha_min)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _expect("g", g, (B, T, H, dv), q.dtype, q.device)
    _expect("state_in", state_in, (B, H, dk, dv), torch.float32, q.device)
    _expect("d_out", d_out, (B, T, H, dv), q.dtype, q.device)
    _expect("d_state", d_state, (B, H, dk, dv), torch.float32, q.device)
    nbytes = backward_workspace_size(p)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _expect_workspace(workspace, q.device)
    r = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v), dg=torch.empty_like(g),
             dlog_alpha=torch.empty_like(log_alpha), dbeta=torch.empty_like(beta))
    r["dstate0"] = torch.empty((B, H, dk, v.shape[-1]), dtype=torch.float32, device=q.device) if want_dstate \
        else None
    _check("kda_backward", lib().kda_backward(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(g), _ptr(state_in),
        _ptr(d_out), _ptr(d_state), _ptr(r["dq"]), _ptr(r["dk"]), _ptr(r["dv"]), _ptr(r["dlog_alpha"]),
        _ptr(r["dbeta"]), _ptr(r["dg"]), _ptr(r["dstate0"]), _ptr(workspace), workspace.numel(),
        _stream(stream, q.device)))
    return r


def prefill_for_backward(q, k, v, log_alpha, beta, g, log_alpha_min: float, state_in=None, out=None,
                         state_out=None, want_state: bool = True, workspace=None, stream=None):
    """Prefill that leaves its cards and chunk states in a backward workspace
    (kda_prefill_for_backward).  Returns (out, state_out, workspace); pass
    out and workspace to backward_after_prefill with the same inputs."""
    torch = _torch()
    _expect_prefill_inputs(q, k, v, log_alpha, beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _expect("g", g, (B, T, H, dv), q.dtype, q.device)
    _expect("state_in", state_in, (B, H, dk, dv), torch.float32, q.device)
    _expect("out", out, (B, T, H, dv), q.dtype, q.device)
    _expect("state_out", state_out, (B, H, dk, dv), torch.float32, q.device)
    p = _problem_of(q, v, log_alpha_min)
    nbytes = backward_workspace_size(p)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _expect_workspace(workspace, q.device)
    if out is None:
        out = torch.empty_like(g)
    if state_out is None and want_state:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    _check("kda_prefill_for_backward", lib().kda_prefill_for_backward(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(g), _ptr(state_in),
        _ptr(out), _ptr(state_out), _ptr(workspace), workspace.numel(), _stream(stream, q.device)))
    return out, state_out, workspace


def backward_after_prefill(q, k, v, log_alpha, beta, g, out, workspace, log_alpha_min: float, d_out=None,
                           d_state=None, want_dstate: bool = True, stream=None) -> dict:
    """backward() without its forward pass: out and workspace come from
    prefill_for_backward on the same inputs.  Returns the same dict."""
    torch = _torch()
    _expect_prefill_inputs(q, k, v, log_alpha, beta)
    p = _problem_of(q, v, log_alpha_min)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _expect("g", g, (B, T, H, dv), q.dtype, q.device)
    _expect("out", out, (B, T, H, dv), q.dtype, q.device)
    _expect("d_out", d_out, (B, T, H, dv), q.dtype, q.device)
    _expect("d_state", d_state, (B, H, dk, dv), torch.float32, q.device)
    _expect_workspace(workspace, q.device)
    r = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v), dg=torch.empty_like(g),
             dlog_alpha=torch.empty_like(log_alpha), dbeta=torch.empty_like(beta))
    r["dstate0"] = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if want_dstate else None
    _check("kda_backward_after_prefill", lib().kda_backward_after_prefill(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(g), _ptr(out),
        _ptr(d_out), _ptr(d_state), _ptr(r["dq"]), _ptr(r["dk"]), _ptr(r["dv"]), _ptr(r["dlog_alpha"]),
        _ptr(r["dbeta"]), _ptr(r["dg"]), _ptr(r["dstate0"]), _ptr(workspace), workspace.numel(),
        _stream(stream, q.device)))
    return r


_PREFILL_FUNCTION = None


def _prefill_function():
    """The torch.autograd.Function over the split training pair, created on
    first use (torch is imported lazily)."""
    global _PREFILL_FUNCTION
    if _PREFILL_FUNCTION is None:
        torch = _torch()

        class PrefillFunction(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, log_alpha, beta, g, state_in, log_alpha_min, cu_seqlens):
                if cu_seqlens is None:
                    out, state, ws = prefill_for_backward(q, k, v, log_alpha, beta, g, log_alpha_min,
                                                          state_in=state_in)
                else:
                    out, state, ws = varlen_prefill_for_backward(q, k, v, log_alpha, beta, g, log_alpha_min,
                                                                 cu_seqlens, state_in=state_in)
                ctx.save_for_backward(q, k, v, log_alpha, beta, g, out)
                ctx.cu_seqlens = cu_seqlens
                ctx.workspace = ws
                ctx.log_alpha_min = log_alpha_min
                ctx.has_state_in = state_in is not None
                ctx.set_materialize_grads(False)
                return out, state

            @staticmethod
            def backward(ctx, d_out, d_state):
                q, k, v, log_alpha, beta, g, out = ctx.saved_tensors
                kw = dict(d_out=None if d_out is None else d_out.contiguous(),
                          d_state=None if d_state is None else d_state.contiguous(),
                          want_dstate=ctx.has_state_in and ctx.needs_input_grad[6])
                if ctx.cu_seqlens is None:
                    r = backward_after_prefill(q, k, v, log_alpha, beta, g, out, ctx.workspace, ctx.log_alpha_min,
                                               **kw)
                else:
                    r = varlen_backward_after_prefill(q, k, v, log_alpha, beta, g, out, ctx.workspace,
                                                      ctx.log_alpha_min, ctx.cu_seqlens, **kw)
                return r["dq"], r["dk"], r["dv"], r["dlog_alpha"], r["dbeta"], r["dg"], r["dstate0"], None, None

        _PREFILL_FUNCTION = PrefillFunction
    return _PREFILL_FUNCTION


def prefill_autograd(q, k, v, log_alpha, beta, g, log_alpha_min: float, state_in=None, cu_seqlens=None):
    """Differentiable prefill for training: returns (out, final state) like
    prefill(), or like varlen_prefill() for a packed batch when cu_seqlens is
    given, and loss.backward() then fills the gradients of q, k, v,
    log_alpha, beta, g and state_in.  The forward pass is
    kda_prefill_for_backward (kda_varlen_prefill_for_backward), whose
    workspace (cards and chunk states) is held until the backward pass,
    kda_backward_after_prefill (kda_varlen_backward_after_prefill); the state
    gradient is taken only when state_in is given and needs one, and an
    output the loss does not use contributes nothing."""
    return _prefill_function().apply(q, k, v, log_alpha, beta, g, state_in, float(log_alpha_min), cu_seqlens)


def varlen_workspace_size(p: KdaProblem, n_seq: int) -> int:
    n = lib().kda_varlen_workspace_size(ctypes.byref(p), n_seq)
    if n == 0 and n_seq > 0:
        raise KdaError("kda_varlen_workspace_size", 2)
    return n


def _cu(cu_seqlens, device):
    torch = _torch()
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise TypeError("cu_seqlens must be a non-empty 1-D int32 tensor")
    if cu_seqlens.device != device:
        raise ValueError(f"cu_seqlens is on {cu_seqlens.device}, expected {device}")
    return cu_seqlens.numel() - 1


def varlen_prepare(q, k, v, log_alpha, beta, log_alpha_min: float, cu_seqlens, workspace=None, stream=None):
    """Stage 1 for a packed batch: q, k, v, log_alpha [1, T, H, d], beta [1, T, H];
    cu_seqlens int32 [n_seq+1] on the device.  Returns the workspace."""
    torch = _torch()
    _expect_prefill_inputs(q, k, v, log_alpha, beta)
    p = _problem_of(q, v, log_alpha_min)
    n_seq = _cu(cu_seqlens, q.device)
    nbytes = varlen_workspace_size(p, n_seq)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _expect_workspace(workspace, q.device)
    _check("kda_varlen_prepare", lib().kda_varlen_prepare(
        ctypes.byref(p), n_seq, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
        _ptr(workspace), workspace.numel(), _stream(stream, q.device)))
    return workspace


def varlen_scan(workspace, g, log_alpha_min: float, cu_seqlens, state_in=None, out=None, state_out=None,
                want_state: bool = True, stream=None):
    """Stage 2 for a packed batch.  Returns (out [1, T, H, dv], state_out [n_seq, H, dk, dv])."""
    torch = _torch()
    B, T, H, dv = g.shape
    p = problem(B, T, H, dv, dv, _io_code(g.dtype), log_alpha_min)
    n_seq = _cu(cu_seqlens, g.device)
    _expect_workspace(workspace, g.device)
    _expect("state_in", state_in, (n_seq, H, dv, dv), torch.float32, g.device)
    _expect("out", out, g.shape, g.dtype, g.device)
    _expect("state_out", state_out, (n_seq, H, dv, dv), torch.float32, g.device)
    if out is None:
        out = torch.empty_like(g)
    if state_out is None and want_state:
        state_out = torch.empty((n_seq, H, dv, dv), dtype=torch.float32, device=g.device)
    _check("kda_varlen_scan", lib().kda_varlen_scan(
        ctypes.byref(p), n_seq, _ptr(cu_seqlens), _ptr(workspace), workspace.numel(), _ptr(g), _ptr(state_in),
        _ptr(out), _ptr(state_out), _stream(stream, g.device)))
    return out, state_out


def varlen_prefill(q, k, v, log_alpha, beta, g, log_alpha_min: float, cu_seqlens, state_in=None, workspace=None,
                   stream=None):
    """Chunked prefill of a packed variable-length batch.  Returns (out, final states [n_seq, H, dk, dv])."""
    ws = varlen_prepare(q, k, v, log_alpha, beta, log_alpha_min, cu_seqlens, workspace=workspace, stream=stream)
    return varlen_scan(ws, g, log_alpha_min, cu_seqlens, state_in=state_in, stream=stream)


def varlen_backward_workspace_size(p: KdaProblem, n_seq: int) -> int:
    return lib().kda_varlen_backward_workspace_size(ctypes.byref(p), n_seq)


def varlen_backward(q, k, v, log_alpha, beta, g, log_alpha_min: float, cu_seqlens, state_in=None, d_out=None,
                    d_state=None, want_dstate: bool = True, workspace=None, stream=None) -> dict:
    """Gradients of a packed batch (kda_varlen_backward): the token arrays are
    [1, T, H, d] as for varlen_prefill, state_in and d_state [n_seq, H, dk, dv].
    Returns the dict of backward(), with dstate0 [n_seq, H, dk, dv]."""
    torch = _torch()
    _expect_prefill_inputs(q, k, v, log_alpha, beta)
    p = _problem_of(q, v, log_alpha_min)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    n_seq = _cu(cu_seqlens, q.device)
    _expect("g", g, (B, T, H, dv), q.dtype, q.device)
    _expect("state_in", state_in, (n_seq, H, dk, dv), torch.float32, q.device)
    _expect("d_out", d_out, (B, T, H, dv), q.dtype, q.device)
    _expect("d_state", d_state, (n_seq, H, dk, dv), torch.float32, q.device)
    nbytes = varlen_backward_workspace_size(p, n_seq)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _expect_workspace(workspace, q.device)
    r = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v), dg=torch.empty_like(g),
             dlog_alpha=torch.empty_like(log_alpha), dbeta=torch.empty_like(beta))
    r["dstate0"] = torch.empty((n_seq, H, dk, dv), dtype=torch.float32, device=q.device) if want_dstate else None
    _check("kda_varlen_backward", lib().kda_varlen_backward(
        ctypes.byref(p), n_seq, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(g),
        _ptr(state_in), _ptr(d_out), _ptr(d_state), _ptr(r["dq"]), _ptr(r["dk"]), _ptr(r["dv"]),
        _ptr(r["dlog_alpha"]), _ptr(r["dbeta"]), _ptr(r["dg"]), _ptr(r["dstate0"]), _ptr(workspace),
        workspace.numel(), _stream(stream, q.device)))
    return r


def varlen_prefill_for_backward(q, k, v, log_alpha, beta, g, log_alpha_min: float, cu_seqlens, state_in=None,
                                out=None, state_out=None, want_state: bool = True, workspace=None, stream=None):
    """varlen_prefill whose cards and chunk states stay in a varlen backward
    workspace (kda_varlen_prefill_for_backward).  Returns (out, state_out,
    workspace); pass out and workspace to varlen_backward_after_prefill."""
    torch = _torch()
    _expect_prefill_inputs(q, k, v, log_alpha, beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    n_seq = _cu(cu_seqlens, q.device)
    _expect("g", g, (B, T, H, dv), q.dtype, q.device)
    _expect("state_in", state_in, (n_seq, H, dk, dv), torch.float32, q.device)
    _expect("out", out, (B, T, H, dv), q.dtype, q.device)
    _expect("state_out", state_out, (n_seq, H, dk, dv), torch.float32, q.device)
    p = _problem_of(q, v, log_alpha_min)
    nbytes = varlen_backward_workspace_size(p, n_seq)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _expect_workspace(workspace, q.device)
    if out is None:
        out = torch.empty_like(g)
    if state_out is None and want_state:
        state_out = torch.empty((n_seq, H, dk, dv), dtype=torch.float32, device=q.device)
    _check("kda_varlen_prefill_for_backward", lib().kda_varlen_prefill_for_backward(
        ctypes.byref(p), n_seq, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(g),
        _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(workspace), workspace.numel(), _stream(stream, q.device)))
    return out, state_out, workspace


def varlen_backward_after_prefill(q, k, v, log_alpha, beta, g, out, workspace, log_alpha_min: float, cu_seqlens,
                                  d_out=None, d_state=None, want_dstate: bool = True, stream=None) -> dict:
    """varlen_backward without its forward pass: out and workspace come from
    varlen_prefill_for_backward on the same inputs.  Returns the same dict."""
    torch = _torch()
    _expect_prefill_inputs(q, k, v, log_alpha, beta)
    p = _problem_of(q, v, log_alpha_min)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    n_seq = _cu(cu_seqlens, q.device)
    _expect("g", g, (B, T, H, dv), q.dtype, q.device)
    _expect("out", out, (B, T, H, dv), q.dtype, q.device)
    _expect("d_out", d_out, (B, T, H, dv), q.dtype, q.device)
    _expect("d_state", d_state, (n_seq, H, dk, dv), torch.float32, q.device)
    _expect_workspace(workspace, q.device)
    r = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v), dg=torch.empty_like(g),
             dlog_alpha=torch.empty_like(log_alpha), dbeta=torch.empty_like(beta))
    r["dstate0"] = torch.empty((n_seq, H, dk, dv), dtype=torch.float32, device=q.device) if want_dstate else None
    _check("kda_varlen_backward_after_prefill", lib().kda_varlen_backward_after_prefill(
        ctypes.byref(p), n_seq, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(g),
        _ptr(out), _ptr(d_out), _ptr(d_state), _ptr(r["dq"]), _ptr(r["dk"]), _ptr(r["dv"]), _ptr(r["dlog_alpha"]),
        _ptr(r["dbeta"]), _ptr(r["dg"]), _ptr(r["dstate0"]), _ptr(workspace), workspace.numel(),
        _stream(stream, q.device)))
    return r


def prefill(q, k, v, log_alpha, beta, g, log_alpha_min: float, state_in=None, workspace=None, stream=None):
    """Chunked prefill: prepare + scan.  Returns (out, final state)."""
    ws = chunk_prepare(q, k, v, log_alpha, beta, log_alpha_min, workspace=workspace, stream=stream)
    return chunk_scan(ws, g, log_alpha_min, state_in=state_in, stream=stream)


def pipelined_workspace_size(p: KdaProblem, range_chunks: int) -> int:
    n = lib().kda_pipelined_workspace_size(ctypes.byref(p), _range_chunks(range_chunks))
    if n == 0 and p.batch * p.heads > 0:
        raise KdaError("kda_pipelined_workspace_size", 2)
    return n


def _range_chunks(range_chunks) -> int:
    if not isinstance(range_chunks, int) or not 1 <= range_chunks <= 2 ** 31 - 1:
        raise ValueError(f"range_chunks must be an int in [1, 2**31 - 1], got {range_chunks!r}")
    return range_chunks


_AUX_STREAMS = {}


def _aux_stream(device):
    """A second stream per device (default priority) for the pipelined prefill."""
    torch = _torch()
    idx = torch.device(device).index
    idx = torch.cuda.current_device() if idx is None else idx
    if idx not in _AUX_STREAMS:
        _AUX_STREAMS[idx] = torch.cuda.Stream(device=idx)
    return _AUX_STREAMS[idx]


def prefill_pipelined(q, k, v, log_alpha, beta, g, log_alpha_min: float, state_in=None, out=None, state_out=None,
                      want_state: bool = True, range_chunks: int = 256, workspace=None, stream=None,
                      aux_stream=None):
    """Chunked prefill in ranges of range_chunks chunks through
    kda_prefill_pipelined: the next range's cards are prepared on aux_stream
    (a cached second stream unless given) while the current range is scanned
    on `stream`.  The workspace holds two ranges' cards and the carried state
    (allocated here unless given).  Returns (out, state_out)."""
    torch = _torch()
    _expect_prefill_inputs(q, k, v, log_alpha, beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _expect("g", g, (B, T, H, dv), q.dtype, q.device)
    _expect("state_in", state_in, (B, H, dk, dv), torch.float32, q.device)
    _expect("out", out, (B, T, H, dv), q.dtype, q.device)
    _expect("state_out", state_out, (B, H, dk, dv), torch.float32, q.device)
    p = _problem_of(q, v, log_alpha_min)
    rc = _range_chunks(range_chunks)
    need = pipelined_workspace_size(p, rc)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _expect_workspace(workspace, q.device)
    if out is None:
        out = torch.empty_like(g)
    if state_out is None and want_state:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    aux = aux_stream if aux_stream is not None else _aux_stream(q.device)
    _check("kda_prefill_pipelined", lib().kda_prefill_pipelined(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(g), _ptr(state_in),
        _ptr(out), _ptr(state_out), rc, _ptr(workspace), workspace.numel(), _stream(stream, q.device),
        aux.cuda_stream))
    return out, state_out


def prefill_noalloc(q, k, v, log_alpha, beta, g, log_alpha_min: float, state_in=None, out=None, state_out=None,
                    want_state: bool = True, stream=None):
    """Chunked prefill through kda_prefill_noalloc: the library takes no
    workspace and allocates nothing (the update cards go to its fixed per-GPU
    scratch area).  out and state_out are allocated here unless given.
    Returns (out, state_out)."""
    torch = _torch()
    _expect_prefill_inputs(q, k, v, log_alpha, beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _expect("g", g, (B, T, H, dv), q.dtype, q.device)
    _expect("state_in", state_in, (B, H, dk, dv), torch.float32, q.device)
    _expect("out", out, (B, T, H, dv), q.dtype, q.device)
    _expect("state_out", state_out, (B, H, dk, dv), torch.float32, q.device)
    p = _problem_of(q, v, log_alpha_min)
    if out is None:
        out = torch.empty_like(g)
    if state_out is None and want_state:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    _check("kda_prefill_noalloc", lib().kda_prefill_noalloc(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(g), _ptr(state_in),
        _ptr(out), _ptr(state_out), _stream(stream, q.device)))
    return out, state_out


def segmented_prefill(q, k, v, log_alpha, beta, g, log_alpha_min: float, n_seg: int, state_in=None,
                      workspace=None, stream=None):
    """Context-parallel prefill on one GPU: the sequence [B, n_seg*Ts, H, d] is
    treated as n_seg segments (extra batch rows), each summarised from its
    cards, the summaries merged in order, and every segment's outputs computed
    from its exact entering state.  Returns (out, final state)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if T % n_seg:
        raise ValueError("sequence length must split into n_seg equal segments")
    Ts = T // n_seg
    seg = lambda x: x.view((B * n_seg, Ts) + tuple(x.shape[2:]))
    ws = chunk_prepare(seg(q), seg(k), seg(v), seg(log_alpha), seg(beta), log_alpha_min, workspace=workspace,
                       stream=stream)
    A, Bz = segment_summarize(ws, B * n_seg, Ts, H, dk, q.dtype, log_alpha_min, stream=stream)
    seg_in, fin = segment_combine(A.view(B, n_seg, H, dk, dk), Bz.view(B, n_seg, H, dk, dv), state_in,
                                  stream=stream)
    out, _ = chunk_scan(ws, seg(g), log_alpha_min, state_in=seg_in.view(B * n_seg, H, dk, dv),
                        want_state=False, stream=stream)
    return out.view(B, T, H, dv), fin


def to_device(inp, device="cuda"):
    """Upload a kda_inputs.KdaInputs workload (bf16 bit patterns reinterpreted, no rounding)."""
    import numpy as np
    torch = _torch()

    def io(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(a).to(device)

    d = dict(q=io(inp.q), k=io(inp.k), v=io(inp.v), g=io(inp.g),
             log_alpha=torch.from_numpy(inp.log_alpha).to(device), beta=torch.from_numpy(inp.beta).to(device))
    d["state0"] = None if inp.state0 is None else torch.from_numpy(inp.state0).to(device)
    return d
