"""Seeded synthetic inputs for the KDA token-mixer workloads.

This module is shared by the tests, the benchmark and the smoke check. It
holds only random draws, the input distributions and dtype rounding; none of
the mixer's own arithmetic lives here (no retention floor, no cumulative
decay, no delta-rule step, no output gate).

Distributions (the pages give no numeric workload; these are the workload
recipes this repository uses):

* q, k ~ N(0, 1), then L2-normalised per (token, head) in fp64, then rounded
  to the I/O dtype.  The kernels normalise again; on these inputs that only
  undoes the rounding of the norm.
* v, g ~ N(0, 1), rounded to the I/O dtype.
* beta = sigmoid(N(0, 1)) in fp64, stored fp32 (the write strength).
* log_alpha = -softplus(N(mu, 1)) in fp64, stored fp32 (per key channel).
  mu = 0 for the small and medium prefill shapes, mu = -4 for the long ones.
  The retention floor is NOT applied here: the mixer applies it.
* state0 (decode only) ~ N(0, 1) / sqrt(d_k), fp32.

Random numbers come from numpy's Philox counter generator, one independent
stream per (tensor, batch row, block of tokens), keyed from the workload seed
with ``SeedSequence(seed, spawn_key=...)``.  The same seed therefore gives the
same bytes whatever the thread count, and a large workload is generated in
parallel on the host.

bf16 values are carried as their uint16 bit patterns (round to nearest even
from fp32); ``to_f64`` widens either dtype exactly.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# tensor ids used in the Philox spawn keys
_T_Q, _T_K, _T_V, _T_BETA, _T_ALPHA, _T_G, _T_S0 = range(7)
_TOKENS_PER_BLOCK = 256


@dataclass
class KdaInputs:
    """One synthetic KDA workload.  Arrays are token-major ``[B, T, H, d]``."""

    q: np.ndarray            # uint16 (bf16 bits) or float32, [B,T,H,dk]
    k: np.ndarray            # same
    v: np.ndarray            # [B,T,H,dv]
    g: np.ndarray            # [B,T,H,dv]
    log_alpha: np.ndarray    # float32 [B,T,H,dk]; <= 0; floor not applied
    beta: np.ndarray         # float32 [B,T,H]
    io_dtype: str            # "bf16" or "f32"
    log_alpha_min: float     # float32 value of log(alpha_min)
    chunk: int = 64
    state0: Optional[np.ndarray] = None   # float32 [B,H,dk,dv] or None (zeros)
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        B, T, H, dk = self.q.shape
        return B, T, H, dk, self.v.shape[-1]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray, io_dtype: str) -> np.ndarray:
    """Exact widening of an I/O-dtype array (bf16 bits or float32) to float64."""
    if io_dtype == "bf16" and a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def log_alpha_floor(alpha_min: float) -> float:
    """The float32 value of log(alpha_min), shared by every consumer."""
    return float(np.float32(math.log(alpha_min)))


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def make_inputs(B: int, T: int, H: int, dk: int, dv: int, *, io_dtype: str, seed: int,
                alpha_min: float, logit_mu: float = 0.0, with_state0: bool = False,
                chunk: int = 64, threads: Optional[int] = None) -> KdaInputs:
    """Draw one workload.  Deterministic in ``seed`` (and the shape)."""
    if io_dtype not in ("bf16", "f32"):
        raise ValueError("io_dtype must be 'bf16' or 'f32'")
    io_np = np.uint16 if io_dtype == "bf16" else np.float32
    q = np.empty((B, T, H, dk), io_np)
    k = np.empty((B, T, H, dk), io_np)
    v = np.empty((B, T, H, dv), io_np)
    g = np.empty((B, T, H, dv), io_np)
    la = np.empty((B, T, H, dk), np.float32)
    beta = np.empty((B, T, H), np.float32)

    def store(dst, x64):
        if io_dtype == "bf16":
            dst[...] = f32_to_bf16_bits(x64.astype(np.float32))
        else:
            dst[...] = x64.astype(np.float32)

    def unit(x32):
        x = x32.astype(np.float64)
        return x / np.linalg.norm(x, axis=-1, keepdims=True)

    def block(bb: int, blk: int):
        t0 = blk * _TOKENS_PER_BLOCK
        t1 = min(T, t0 + _TOKENS_PER_BLOCK)
        n = t1 - t0
        sl = (bb, slice(t0, t1))
        store(q[sl], unit(_rng(seed, _T_Q, bb, blk).standard_normal((n, H, dk), dtype=np.float32)))
        store(k[sl], unit(_rng(seed, _T_K, bb, blk).standard_normal((n, H, dk), dtype=np.float32)))
        store(v[sl], _rng(seed, _T_V, bb, blk).standard_normal((n, H, dv), dtype=np.float32).astype(np.float64))
        xb = _rng(seed, _T_BETA, bb, blk).standard_normal((n, H), dtype=np.float32).astype(np.float64)
        beta[sl] = _sigmoid(xb).astype(np.float32)
        xa = _rng(seed, _T_ALPHA, bb, blk).standard_normal((n, H, dk), dtype=np.float32).astype(np.float64)
        la[sl] = (-_softplus(xa + logit_mu)).astype(np.float32)
        store(g[sl], _rng(seed, _T_G, bb, blk).standard_normal((n, H, dv), dtype=np.float32).astype(np.float64))

    jobs = [(bb, blk) for bb in range(B) for blk in range((T + _TOKENS_PER_BLOCK - 1) // _TOKENS_PER_BLOCK)]
    nthr = threads or min(16, os.cpu_count() or 1)
    if len(jobs) <= 1 or nthr <= 1:
        for j in jobs:
            block(*j)
    else:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(lambda j: block(*j), jobs))

    state0 = None
    if with_state0:
        state0 = np.empty((B, H, dk, dv), np.float32)
        for bb in range(B):
            state0[bb] = (_rng(seed, _T_S0, bb).standard_normal((H, dk, dv), dtype=np.float32)
                          / np.float32(math.sqrt(dk)))
    return KdaInputs(q=q, k=k, v=v, g=g, log_alpha=la, beta=beta, io_dtype=io_dtype,
                     log_alpha_min=log_alpha_floor(alpha_min), chunk=chunk, state0=state0,
                     meta=dict(B=B, T=T, H=H, dk=dk, dv=dv, seed=seed, alpha_min=alpha_min,
                               logit_mu=logit_mu))


# The five workload shapes (small parity case, medium prefill, 64K long
# prefill, 1M-token segmented prefill, batched decode).  ``T`` for the decode
# workload is the number of consecutive decode steps.
WORKLOADS = {
    0: dict(name="kda-prefill B1 T256 H1 d64 f32", B=1, T=256, H=1, dk=64, dv=64, io_dtype="f32",
            alpha_min=0.9, logit_mu=0.0, seed=0),
    1: dict(name="kda-prefill B4 T4096 H16 d128 bf16", B=4, T=4096, H=16, dk=128, dv=128, io_dtype="bf16",
            alpha_min=0.95, logit_mu=0.0, seed=1),
    2: dict(name="kda-prefill B1 T65536 H32 d128 bf16", B=1, T=65536, H=32, dk=128, dv=128, io_dtype="bf16",
            alpha_min=0.9, logit_mu=-4.0, seed=2),
    3: dict(name="kda-segmented-prefill B1 T1048576 H8 d128 bf16 16x65536", B=1, T=1048576, H=8, dk=128,
            dv=128, io_dtype="bf16", alpha_min=0.9, logit_mu=-4.0, seed=3, n_seg=16),
    4: dict(name="kda-decode N256 H32 d128 bf16 64 steps", B=256, T=64, H=32, dk=128, dv=128, io_dtype="bf16",
            alpha_min=0.9, logit_mu=-4.0, seed=4, with_state0=True),
}


def varlen_lengths(total: int, seed: int = 2024, lo: int = 64, hi: int = 8192) -> list:
    """Sequence lengths of a packed batch: log-uniform between lo and hi tokens
    (seeded), the last one taking the remainder, summing to `total` -- short
    and long requests mixed as in serving."""
    rng = np.random.default_rng(seed)
    lens = []
    while sum(lens) < total:
        lens.append(int(min(total - sum(lens), round(float(np.exp(rng.uniform(np.log(lo), np.log(hi))))))))
    return lens


def workload(i: int, **override) -> KdaInputs:
    """Inputs of workload ``i``; keyword overrides (e.g. a shorter ``T``) keep the recipe."""
    w = dict(WORKLOADS[i])
    w.update(override)
    w.pop("name")
    w.pop("n_seg", None)
    return make_inputs(w.pop("B"), w.pop("T"), w.pop("H"), w.pop("dk"), w.pop("dv"), **w)
