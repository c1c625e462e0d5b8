"""fp64 CPU oracle for the KDA token mixer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the HIP library and is
never on the product path.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, pthreads), which
states what each step follows on the pages.  This file only marshals numpy
arrays through ctypes and builds the C library with gcc.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
# another build of kda_oracle.c to load instead (the sanitizer tests set it)
_LIB_OVERRIDE = os.environ.get("KDA_ORACLE_LIB")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (portable x86-64 code: no -march=native)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-pthread",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_native(dst_dir: str) -> str:
    """Compile the same source with -march=native into dst_dir (for timing the
    oracle on the host it runs on; the checks use the portable build)."""
    out = os.path.join(dst_dir, "libkda_oracle_native.so")
    subprocess.check_call(["gcc", "-O3", "-march=native", "-std=c11", "-fPIC", "-shared", "-pthread",
                           _SRC, "-o", out, "-lm"])
    return out


def use_library(path: str) -> None:
    """Load the oracle from `path` (a build of kda_oracle.c) for later calls."""
    global _lib
    _lib = _declare(ctypes.CDLL(path))


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            _lib = _declare(ctypes.CDLL(_LIB_OVERRIDE))
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _declare(lib):
    """Argument and result types of the oracle's C functions."""
    P = ctypes.c_void_p
    I64, I32, F64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.kda_oracle_ref.argtypes = [I64, I64, I32, I32, I32, P, P, P, P, P, P, F64, P, P, P, I32]
    lib.kda_oracle_ref.restype = I32
    lib.kda_oracle_summary.argtypes = [I64, I64, I32, I32, I32, P, P, P, P, F64, P, P, I32]
    lib.kda_oracle_summary.restype = I32
    lib.kda_oracle_combine.argtypes = [I64, I32, I32, I32, I32, P, P, P, P, P]
    lib.kda_oracle_combine.restype = I32
    lib.kda_oracle_grad.argtypes = [I64, I64, I32, I32, I32, P, P, P, P, P, P, F64, P, P, P,
                                    P, P, P, P, P, P, P, I32]
    lib.kda_oracle_grad.restype = I32
    return lib


def _c(a: Optional[np.ndarray]) -> Optional[np.ndarray]:
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def host_threads() -> int:
    """Threads this process may use on the host: the CPU share given to it
    (OMP_NUM_THREADS when set), else the CPUs in its affinity mask."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def kda_ref(q, k, v, log_alpha, beta, g, log_alpha_min: float, state0=None,
            nthreads: Optional[int] = None, want_out: bool = True) -> Tuple[Optional[np.ndarray], np.ndarray]:
    """Step-by-step recurrence in fp64.

    q, k, log_alpha: [B,T,H,dk]; v, g: [B,T,H,dv]; beta: [B,T,H];
    state0: [B,H,dk,dv] or None (zeros).  Returns (out [B,T,H,dv] or None,
    final state [B,H,dk,dv]).
    """
    q, k, v, la, bt, g, s0 = map(_c, (q, k, v, log_alpha, beta, g, state0))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    out = np.zeros((B, T, H, dv)) if want_out else None
    st = np.zeros((B, H, dk, dv))
    rc = _load().kda_oracle_ref(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(la), _p(bt), _p(g),
                                float(log_alpha_min), _p(s0), _p(out), _p(st),
                                nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kda_oracle_ref failed ({rc})")
    return out, st


def kda_summary(k, v, log_alpha, beta, log_alpha_min: float,
                nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Segment pair (A [B,H,dk,dk], Bz [B,H,dk,dv]) with S_end = A S_start + Bz."""
    k, v, la, bt = map(_c, (k, v, log_alpha, beta))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    A = np.zeros((B, H, dk, dk))
    Bz = np.zeros((B, H, dk, dv))
    rc = _load().kda_oracle_summary(B, T, H, dk, dv, _p(k), _p(v), _p(la), _p(bt),
                                    float(log_alpha_min), _p(A), _p(Bz), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kda_oracle_summary failed ({rc})")
    return A, Bz


def kda_combine(A, Bz, state_init=None) -> Tuple[np.ndarray, np.ndarray]:
    """In-order merge.  A [B,n,H,dk,dk], Bz [B,n,H,dk,dv] -> (state entering
    each segment [B,n,H,dk,dv], final state [B,H,dk,dv])."""
    A, Bz, s0 = map(_c, (A, Bz, state_init))
    B, n, H, dk, _ = A.shape
    dv = Bz.shape[-1]
    seg_in = np.zeros((B, n, H, dk, dv))
    fin = np.zeros((B, H, dk, dv))
    rc = _load().kda_oracle_combine(B, n, H, dk, dv, _p(A), _p(Bz), _p(s0), _p(seg_in), _p(fin))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_combine failed ({rc})")
    return seg_in, fin


def kda_grad(q, k, v, log_alpha, beta, g, log_alpha_min: float, state0=None, d_out=None, d_state=None,
             nthreads: Optional[int] = None) -> dict:
    """Gradients of <d_out, out> + <d_state, final state> (fp64 adjoint of the
    step recurrence).  Returns a dict with dq, dk, dv, dlog_alpha, dbeta, dg
    (shapes of the inputs) and dstate0 [B,H,dk,dv]."""
    q, k, v, la, bt, g, s0, do, ds = map(_c, (q, k, v, log_alpha, beta, g, state0, d_out, d_state))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    r = {n: np.zeros(x.shape) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dlog_alpha", la), ("dbeta", bt),
                                          ("dg", g))}
    r["dstate0"] = np.zeros((B, H, dk, dv))
    rc = _load().kda_oracle_grad(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(la), _p(bt), _p(g),
                                 float(log_alpha_min), _p(s0), _p(do), _p(ds),
                                 _p(r["dq"]), _p(r["dk"]), _p(r["dv"]), _p(r["dlog_alpha"]), _p(r["dbeta"]),
                                 _p(r["dg"]), _p(r["dstate0"]), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kda_oracle_grad failed ({rc})")
    return r
