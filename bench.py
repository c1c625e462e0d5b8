"""KDA benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-segmented] [--no-backward]
                    [--no-varlen] [--no-pipelined] [--no-cpu-baseline]

A step is one chunked prefill (update-card preparation + ordered hand-off
with the gated read-out) of the long-prefill workload: B=1, T=65,536, H=32,
d_k=d_v=128, bf16 q/k/v/g/out, fp32 gates and state, chunk 64, synthetic
inputs (kda_inputs, seed 2), resident in HBM before timing starts.  `value`
is prefill tokens/s (sequence tokens; all 32 heads).

Also reported on the same JSON line:
  * per-kernel average durations from HIP events recorded on the launch
    stream inside the timed region, and the roofline of the dominant kernel
    (algorithmic bytes per launch / its average duration, against 8 TB/s);
  * the whole path against the HBM and bf16-MFMA peaks and against the
    attainable roofline min(MFMA peak, HBM peak x arithmetic intensity);
  * the batched decode workload (256 sequences x 32 heads, d=128, 64 steps,
    fp32 state updated in place): GB/s and fraction of HBM peak, with a
    plain device copy and a large bf16 GEMM timed in the same job as the
    achievable HBM and MFMA references;
  * the segmented (context-parallel) prefill of 1,048,576 tokens x 8 heads as
    16 segments: per-call times of prepare, segment summaries, in-order
    combine and the per-segment recompute;
  * the same hand-off emitting prefix-cache checkpoints every 64 chunks
    (kda_chunk_scan_checkpoints), beside the plain scan, and the last 4,096
    tokens prefilled again from the checkpoint cached before them (the
    prefix-cache use: prepare + scan with state_in);
  * the same step through kda_prefill_pipelined: chunk ranges of 128 or 256
    chunks, each range's prepare on a second stream overlapping the previous
    range's scan, with two ranges' cards instead of the whole sequence's;
  * packed variable-length prefill: the long workload's 65,536 tokens x 32
    heads re-cut into sequences of a seeded length mix (kda_varlen_prepare +
    kda_varlen_scan), tokens/s beside the uniform step;
  * the backward pass (gradients of every prefill input and of the initial
    state) on the medium prefill workload B=4, T=4,096, H=16, d=128 bf16:
    ms per call and token-heads/s, beside the forward on the same inputs;
    and the split pair for training, a prefill that keeps its cards and
    chunk states (kda_prefill_for_backward) and the backward without its
    forward pass (kda_backward_after_prefill);
  * cpu_baseline: the fp64 oracle (its source compiled -march=native for the
    host) timed over the whole long workload on the CPU share given to the
    job, with the host's CPU count and model.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 MFMA, TFLOP/s
C = 64
D = 128
# algorithmic bytes per token-head (bf16 I/O, fp32 log-decay and beta):
PATH_BYTES = 4 * D * 2 + D * 4 + 4 + D * 2          # q,k,v,g in; log_alpha, beta in; out -> 1,796
CARD_BYTES = 74240 // C    # update card per token-head (bf16, d=128; meaningful bytes, 1 KB padding excluded) -> 1,160
PREP_BYTES = 3 * D * 2 + D * 4 + 4 + CARD_BYTES       # q,k,v,log_alpha,beta in; card out -> 2,444
SCAN_BYTES = CARD_BYTES + D * 2 + D * 2               # card, g in; out -> 1,672
# the card parts a segment summary reads: Wk, Ke^T, Wv (C x d bf16 each) and e^gamma_C (d fp32) -> 776
SUMMARY_CARD_BYTES = (3 * C * D * 2 + D * 4) // C
# algorithmic FLOPs per token-head of the chunk method (triangular C x C products at half):
FLOP_TOK = 6 * D * D + C * (3 * D + 2 * D) + C * C / 3
# decode: per (sequence, head) the fp32 state is read and written once, plus the token's inputs/outputs
DEC_BYTES = 2 * D * D * 4 + (2 * D * 2 + D * 4 + 4 + D * 2 + D * 2) + D * 2


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_rule_91_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def traffic_for(kernel: str, src: str, tokens_heads: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(p)).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("src_hash") != src:
        return None
    return rec["bytes_per_token_head"] * tokens_heads


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-segmented", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-pipelined", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-only", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run one plain device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures the KDA path on one GPU only (--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import gated_delta_rule_91_amd as kda
    from kda_inputs import WORKLOADS, workload

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    result = {}
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 18   # float32 elements
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": n * 4, "calib_copy_bytes_written": n * 4}), flush=True)
        return

    # ------------------------------------------------------------------ prefill
    W = WORKLOADS[2]
    B, T, H = W["B"], W["T"], W["H"]
    if not args.decode_only:
        t0 = time.time()
        inp = workload(2)
        log(f"[bench] generated prefill inputs in {time.time() - t0:.1f}s")
        d = kda.to_device(inp, dev)
        floor = inp.log_alpha_min
        del inp
        p = kda.problem(B, T, H, D, D, kda.KDA_BF16, floor)
        ws = torch.empty(kda.workspace_size(p), dtype=torch.uint8, device=dev)
        out = torch.empty_like(d["g"])
        st = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream()

        def step(evs=None):
            if evs is not None:
                evs[0].record(stream)
            kda.chunk_prepare(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], floor, workspace=ws)
            if evs is not None:
                evs[1].record(stream)
            kda.chunk_scan(ws, d["g"], floor, state_in=None, out=out, state_out=st)
            if evs is not None:
                evs[2].record(stream)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        prep_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
        scan_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
        ms = wall * 1e3 / args.steps
        th = B * T * H
        log(f"[bench] prefill {ms:.3f} ms/step (prepare {prep_ms:.3f} ms, scan {scan_ms:.3f} ms)")
        shash = {"kda_prepare_kernel": src_hash("kda_prepare.hip", "kda_common.hpp"),
                 "kda_scan_kernel": src_hash("kda_scan.hip", "kda_common.hpp")}
        kern = {"kda_prepare_kernel": (prep_ms, PREP_BYTES), "kda_scan_kernel": (scan_ms, SCAN_BYTES)}
        dom = max(kern, key=lambda k: kern[k][0])
        dms, dbytes = kern[dom]
        achieved = dbytes * th / (dms * 1e-3) / 1e9
        result.update(
            metric="KDA prefill tokens/s + % MFMA peak @T=64K,H=32,d=128; decode GB/s % HBM",
            value=B * T / (ms * 1e-3), unit="tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
            ms_per_step=ms, higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16",
            data="synthetic (seeded; q,k unit-normalised, v,g N(0,1), beta=sigmoid(N(0,1)), "
                 "log_alpha=-softplus(N(-4,1)) floored at log 0.9)",
            config={"workload": W["name"], "batch": B, "seq_len": T, "heads": H, "d_k": D, "d_v": D,
                    "chunk": C, "state": "fp32", "parallelism": "single GPU"},
            roofline={"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes_per_token_head": dbytes,
                      "avg_launch_ms": dms, "traffic": traffic_for(dom, shash[dom], th),
                      # the whole step against the same peaks: the path's algorithmic
                      # bytes (1,796 per token-head) and FLOPs over ms_per_step
                      "path_frac": PATH_BYTES * th / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "path_mfma_frac_bf16": FLOP_TOK * th / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                      "path_mfma_frac_ceiling": min(1.0, FLOP_TOK / PATH_BYTES * HBM_PEAK_GBS / 1e3
                                                    / MFMA_BF16_PEAK_TFLOPS)},
            kernels_ms={"kda_prepare_kernel": prep_ms, "kda_scan_kernel": scan_ms},
            path={"algorithmic_bytes_per_token_head": PATH_BYTES,
                  "hbm_GBps": PATH_BYTES * th / (ms * 1e-3) / 1e9,
                  "hbm_frac": PATH_BYTES * th / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "flop_per_token_head": FLOP_TOK,
                  "mfma_TFLOPs": FLOP_TOK * th / (ms * 1e-3) / 1e12,
                  "mfma_frac_bf16": FLOP_TOK * th / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                  "roofline_ceiling_mfma_frac": min(1.0, FLOP_TOK / PATH_BYTES * HBM_PEAK_GBS / 1e3
                                                    / MFMA_BF16_PEAK_TFLOPS),
                  # achieved FLOP rate against the attainable one, min(MFMA peak, HBM peak x intensity)
                  "attainable_roofline_frac": FLOP_TOK * th / (ms * 1e-3) / 1e12
                  / min(MFMA_BF16_PEAK_TFLOPS, FLOP_TOK / PATH_BYTES * HBM_PEAK_GBS / 1e3)},
        )
        # the same hand-off emitting prefix-cache checkpoints every 64 chunks (4,096 tokens)
        every = 64
        ckpt_ms = 0.0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        kda.chunk_scan_checkpoints(ws, d["g"], floor, every, out=out, state_out=st)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            _, _, ck = kda.chunk_scan_checkpoints(ws, d["g"], floor, every, out=out, state_out=st)
        e1.record()
        torch.cuda.synchronize()
        ckpt_ms = e0.elapsed_time(e1) / 5
        log(f"[bench] scan with checkpoints every {every} chunks {ckpt_ms:.3f} ms ({ck.shape[2]} per head)")
        result["checkpoints"] = {"every_chunks": every, "per_head": int(ck.shape[2]), "scan_ms": ckpt_ms,
                                 "plain_scan_ms": scan_ms}
        # prefix cache in use: the last 4,096 tokens prefilled again from the
        # checkpoint cached after the first 61,440 (prepare + scan with state_in)
        new_t = every * C
        j = (T - new_t) // new_t
        sl = {n: d[n][:, T - new_t:] for n in ("q", "k", "v", "log_alpha", "beta", "g")}
        s_cached = ck[:, :, j].contiguous()
        ws_r = torch.empty(kda.workspace_size(kda.problem(B, new_t, H, D, D, kda.KDA_BF16, floor)),
                           dtype=torch.uint8, device=dev)
        out_r = torch.empty_like(sl["g"])
        st_r = torch.empty_like(st)

        def resume():
            kda.chunk_prepare(sl["q"], sl["k"], sl["v"], sl["log_alpha"], sl["beta"], floor, workspace=ws_r)
            kda.chunk_scan(ws_r, sl["g"], floor, state_in=s_cached, out=out_r, state_out=st_r)

        resume()
        torch.cuda.synchronize()
        same = bool(torch.equal(out_r, out[:, T - new_t:]) and torch.equal(st_r, st))
        e0.record()
        for _ in range(10):
            resume()
        e1.record()
        torch.cuda.synchronize()
        res_ms = e0.elapsed_time(e1) / 10
        log(f"[bench] resume: {new_t} new tokens from the cached state after {T - new_t} in {res_ms:.3f} ms "
            f"(identical to the uninterrupted run: {same})")
        result["resume"] = {"workload": f"kda-prefill B1 T{new_t} H{H} d{D} bf16 resumed from the checkpoint after "
                                        f"{T - new_t} tokens",
                            "ms": res_ms, "tokens_per_s": B * new_t / (res_ms * 1e-3),
                            "identical_to_uninterrupted": same}
        del ck, sl, s_cached, ws_r, out_r, st_r
        # the same step as chunk ranges, each range's prepare on a second
        # stream overlapping the previous range's scan (two ranges' cards)
        if not args.no_pipelined:
            pipe = {}
            out_p = torch.empty_like(out)
            st_p = torch.empty_like(st)
            for rc in (128, 256):
                ws_p = torch.empty(kda.pipelined_workspace_size(p, rc), dtype=torch.uint8, device=dev)

                def pstep():
                    kda.prefill_pipelined(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["g"], floor,
                                          out=out_p, state_out=st_p, range_chunks=rc, workspace=ws_p)

                pstep()
                torch.cuda.synchronize()
                same = bool(torch.equal(out_p, out) and torch.equal(st_p, st))
                e0.record(stream)
                for _ in range(10):
                    pstep()
                e1.record(stream)
                torch.cuda.synchronize()
                pms = e0.elapsed_time(e1) / 10
                log(f"[bench] pipelined, ranges of {rc} chunks: {pms:.3f} ms (identical to the step: {same})")
                pipe[str(rc)] = {"ms": pms, "workspace_bytes": ws_p.numel(), "identical_to_step": same}
                del ws_p
            result["pipelined"] = {"workload": W["name"], "step_ms": ms, "card_workspace_bytes": ws.numel(),
                                   "by_range_chunks": pipe}
            del out_p, st_p
        del d, ws, out, st
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------ decode
    if not args.no_decode:
        Wd = WORKLOADS[4]
        inp = workload(4)
        dd = kda.to_device(inp, dev)
        N, Td = Wd["B"], Wd["T"]
        sm = {n: dd[n].transpose(0, 1).contiguous() for n in ("q", "k", "v", "g", "log_alpha", "beta")}
        state = dd["state0"].clone()
        outd = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev)
        floor_d = inp.log_alpha_min

        def dstep(t):
            kda.decode_step(sm["q"][t], sm["k"][t], sm["v"][t], sm["log_alpha"][t], sm["beta"][t], sm["g"][t],
                            state, floor_d, out=outd)

        for t in range(Td):
            dstep(t)
        torch.cuda.synchronize()
        reps = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for t in range(Td):
                dstep(t)
        e1.record()
        torch.cuda.synchronize()
        per_step_ms = e0.elapsed_time(e1) / (reps * Td)
        gbs = DEC_BYTES * N * H / (per_step_ms * 1e-3) / 1e9
        log(f"[bench] decode {per_step_ms * 1e3:.1f} us/step, {gbs:.0f} GB/s")
        result["decode"] = {"workload": Wd["name"], "us_per_step": per_step_ms * 1e3, "GBps": gbs,
                            "hbm_frac": gbs / HBM_PEAK_GBS, "bytes_per_step": DEC_BYTES * N * H,
                            "tokens_per_s": N / (per_step_ms * 1e-3)}
        # a serving loop at a small batch (the first 8 sequences): the steps
        # launched one by one from the host, and the same steps captured once
        # in a HIP graph and replayed (the library records kernel launches
        # only); both from the same state must give the same bits
        Ns = 8
        small = {n: sm[n][:, :Ns].contiguous() for n in sm}
        st_e, st_g = dd["state0"][:Ns].clone(), dd["state0"][:Ns].clone()
        out_e = torch.empty((Td, Ns, H, D), dtype=torch.bfloat16, device=dev)
        out_g = torch.empty_like(out_e)

        def sloop(st, outs):
            for t in range(Td):
                kda.decode_step(small["q"][t], small["k"][t], small["v"][t], small["log_alpha"][t],
                                small["beta"][t], small["g"][t], st, floor_d, out=outs[t])

        sloop(st_e, out_e)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            sloop(st_g, out_g)
        st_e.copy_(dd["state0"][:Ns])
        st_g.copy_(dd["state0"][:Ns])
        sloop(st_e, out_e)
        graph.replay()
        torch.cuda.synchronize()
        same_g = torch.equal(st_e, st_g) and torch.equal(out_e, out_g)
        e0.record()
        for _ in range(reps):
            sloop(st_e, out_e)
        e1.record()
        torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) * 1e3 / (reps * Td)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) * 1e3 / (reps * Td)
        log(f"[bench] decode of {Ns} sequences: {eager_us:.1f} us/step launched from the host, "
            f"{graph_us:.1f} us/step replayed from a graph (identical: {same_g})")
        result["decode"]["small_batch_graph"] = {
            "workload": f"kda-decode N{Ns} H{H} d{D} bf16 {Td} steps", "eager_us_per_step": eager_us,
            "graph_us_per_step": graph_us, "identical": same_g}
        del graph, small, st_e, st_g, out_e, out_g
        # achievable-bandwidth reference in the same job: a plain device copy
        x = torch.empty(1 << 29, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            y.copy_(x)
        e1.record()
        torch.cuda.synchronize()
        result["hbm_copy_GBps"] = 2 * x.numel() * 4 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del x, y
        # achievable-MFMA reference in the same job: a large bf16 GEMM (library)
        n = 8192
        a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        b2 = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        c2 = a @ b2
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            c2 = a @ b2
        e1.record()
        torch.cuda.synchronize()
        result["mfma_gemm_bf16_TFLOPs"] = 2 * n ** 3 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e12
        del a, b2, c2, dd, sm, state
        torch.cuda.empty_cache()

    # --------------------------------------------------------- segmented prefill
    if not args.no_segmented and not args.decode_only:
        Ws = WORKLOADS[3]
        t0 = time.time()
        inp = workload(3)
        log(f"[bench] generated segmented inputs in {time.time() - t0:.1f}s")
        ds = kda.to_device(inp, dev)
        floor_s = inp.log_alpha_min
        del inp
        Bs, Ts_all, Hs, nseg = Ws["B"], Ws["T"], Ws["H"], Ws["n_seg"]
        Ts = Ts_all // nseg
        seg = lambda x: x.view((Bs * nseg, Ts) + tuple(x.shape[2:]))
        ps = kda.problem(Bs * nseg, Ts, Hs, D, D, kda.KDA_BF16, floor_s)
        wss = torch.empty(kda.workspace_size(ps), dtype=torch.uint8, device=dev)
        outs = torch.empty((Bs * nseg, Ts, Hs, D), dtype=torch.bfloat16, device=dev)

        def sstep(ev=None):
            rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
            rec(0)
            kda.chunk_prepare(seg(ds["q"]), seg(ds["k"]), seg(ds["v"]), seg(ds["log_alpha"]), seg(ds["beta"]),
                              floor_s, workspace=wss)
            rec(1)
            A, Bz = kda.segment_summarize(wss, Bs * nseg, Ts, Hs, D, torch.bfloat16, floor_s)
            rec(2)
            seg_in, fin = kda.segment_combine(A.view(Bs, nseg, Hs, D, D), Bz.view(Bs, nseg, Hs, D, D), None)
            rec(3)
            kda.chunk_scan(wss, seg(ds["g"]), floor_s, state_in=seg_in.view(Bs * nseg, Hs, D, D), out=outs,
                           want_state=False)
            rec(4)

        sstep()
        torch.cuda.synchronize()
        reps = 3
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(reps)]
        for r in range(reps):
            sstep(evs[r])
        torch.cuda.synchronize()
        part = lambda i: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / reps
        total = sum(e[0].elapsed_time(e[4]) for e in evs) / reps
        ths = Bs * Ts_all * Hs
        names = ("prepare", "summarize", "combine", "scan")
        times = {nm: part(i) for i, nm in enumerate(names)}
        log(f"[bench] segmented {total:.3f} ms (" + ", ".join(f"{k} {v:.3f}" for k, v in times.items()) + ")")
        result["segmented"] = {
            "workload": Ws["name"], "ms": total, "tokens_per_s": Bs * Ts_all / (total * 1e-3),
            "ms_per_call": times,
            # algorithmic bytes: prepare and scan as in the prefill; the
            # summaries read Wk, Ke^T, Wv and e^gamma_C of the cards (776 B
            # per token-head) and write 2 d^2 fp32 per segment-head
            "GBps": {"prepare": PREP_BYTES * ths / (times["prepare"] * 1e-3) / 1e9,
                     "summarize": (SUMMARY_CARD_BYTES * ths + 2 * D * D * 4 * Bs * nseg * Hs)
                     / (times["summarize"] * 1e-3) / 1e9,
                     "scan": SCAN_BYTES * ths / (times["scan"] * 1e-3) / 1e9},
        }
        del ds, wss, outs
        torch.cuda.empty_cache()

    # ------------------------------------------------- packed variable-length
    if not args.no_varlen and not args.decode_only:
        import numpy as np
        inp = workload(2)
        dl = kda.to_device(inp, dev)
        from kda_inputs import varlen_lengths
        lens = varlen_lengths(T)   # log-uniform 64..8,192 tokens, seeded
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
        pv = kda.problem(1, T, H, D, D, kda.KDA_BF16, inp.log_alpha_min)
        wsv = torch.empty(kda.varlen_workspace_size(pv, len(lens)), dtype=torch.uint8, device=dev)
        outv = torch.empty_like(dl["g"])

        def vstep():
            kda.varlen_prepare(dl["q"], dl["k"], dl["v"], dl["log_alpha"], dl["beta"], inp.log_alpha_min, cu,
                               workspace=wsv)
            kda.varlen_scan(wsv, dl["g"], inp.log_alpha_min, cu, out=outv, want_state=True)

        vstep()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            vstep()
        e1.record()
        torch.cuda.synchronize()
        vms = e0.elapsed_time(e1) / reps
        log(f"[bench] varlen {vms:.3f} ms for {len(lens)} sequences ({min(lens)}..{max(lens)} tokens)")
        result["varlen"] = {"workload": f"kda-varlen-prefill {len(lens)} sequences, {T} packed tokens, H{H} d{D} bf16",
                            "ms": vms, "tokens_per_s": T / (vms * 1e-3), "n_seq": len(lens),
                            "min_len": min(lens), "max_len": max(lens),
                            "GBps": PATH_BYTES * T * H / (vms * 1e-3) / 1e9}
        del dl, wsv, outv
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- backward
    if not args.no_backward and not args.decode_only:
        Wb = WORKLOADS[1]
        inp = workload(1)
        db = kda.to_device(inp, dev)
        floor_b = inp.log_alpha_min
        Bb, Tb, Hb = Wb["B"], Wb["T"], Wb["H"]
        gen = torch.Generator(device=dev).manual_seed(11)
        d_out = torch.randn((Bb, Tb, Hb, D), device=dev, generator=gen).to(torch.bfloat16)
        d_state = torch.randn((Bb, Hb, D, D), device=dev, generator=gen)
        pb = kda.problem(Bb, Tb, Hb, D, D, kda.KDA_BF16, floor_b)
        wsb = torch.empty(kda.backward_workspace_size(pb), dtype=torch.uint8, device=dev)

        def bstep():
            return kda.backward(db["q"], db["k"], db["v"], db["log_alpha"], db["beta"], db["g"], floor_b,
                                d_out=d_out, d_state=d_state, workspace=wsb)

        def fstep():
            return kda.prefill(db["q"], db["k"], db["v"], db["log_alpha"], db["beta"], db["g"], floor_b)

        bstep(); fstep()
        torch.cuda.synchronize()
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        reps = 10
        e0.record()
        for _ in range(reps):
            bstep()
        e1.record()
        for _ in range(reps):
            fstep()
        e2.record()
        torch.cuda.synchronize()
        bms, fms = e0.elapsed_time(e1) / reps, e1.elapsed_time(e2) / reps
        th = Bb * Tb * Hb
        # algorithmic bytes per token-head: q,k,v,g,d_out in (bf16), log_alpha,
        # beta in (fp32); dq,dk,dv,dg out (bf16), dlog_alpha, dbeta out (fp32)
        bwd_bytes = 5 * D * 2 + D * 4 + 4 + 4 * D * 2 + D * 4 + 4
        # gradient-kernel products per token-head: five C x d x d (with a state), nine C x C x d
        bwd_flop = 5 * 2 * D * D + 9 * 2 * C * D
        log(f"[bench] backward {bms:.3f} ms, forward {fms:.3f} ms on {Wb['name']}")
        # the split pair: a prefill that keeps its cards and chunk states in
        # the backward workspace, then the backward without its forward pass
        fwd_out = torch.empty_like(db["g"])

        def fkeep():
            kda.prefill_for_backward(db["q"], db["k"], db["v"], db["log_alpha"], db["beta"], db["g"], floor_b,
                                     out=fwd_out, workspace=wsb)

        def bafter():
            return kda.backward_after_prefill(db["q"], db["k"], db["v"], db["log_alpha"], db["beta"], db["g"],
                                              fwd_out, wsb, floor_b, d_out=d_out, d_state=d_state)

        ref = bstep()
        fkeep()
        got = bafter()
        torch.cuda.synchronize()
        same = all(torch.equal(got[n], ref[n]) for n in ref)
        e0.record()
        for _ in range(reps):
            fkeep()
        e1.record()
        for _ in range(reps):
            bafter()
        e2.record()
        torch.cuda.synchronize()
        kms, ams = e0.elapsed_time(e1) / reps, e1.elapsed_time(e2) / reps
        log(f"[bench] prefill keeping the forward {kms:.3f} ms, backward after it {ams:.3f} ms "
            f"(identical to the backward: {same})")
        result["backward"] = {"workload": Wb["name"], "ms": bms, "forward_ms": fms, "ratio_to_forward": bms / fms,
                              "token_heads_per_s": th / (bms * 1e-3), "GBps": bwd_bytes * th / (bms * 1e-3) / 1e9,
                              "bytes_per_token_head": bwd_bytes, "grad_flop_per_token_head": bwd_flop,
                              "grad_TFLOPs_over_whole_call": bwd_flop * th / (bms * 1e-3) / 1e12,
                              "after_prefill": {"prefill_for_backward_ms": kms, "ms": ams,
                                                "ratio_to_forward": ams / fms, "identical_to_backward": same}}
        # the same 16,384 tokens x 16 heads as one packed row of sequences with
        # log-uniform lengths of 64..4,096 tokens (seeded), through
        # kda_varlen_backward; its gradients must equal kda_backward's on each
        # sequence alone (checked on the first and the last)
        rngv = np.random.default_rng(23)
        Tp, lens = Bb * Tb, []
        while sum(lens) < Tp:
            lens.append(min(Tp - sum(lens), int(np.exp(rngv.uniform(np.log(64), np.log(4096))))))
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
        pk = {n: db[n].reshape((1, Tp) + tuple(db[n].shape[2:])) for n in ("q", "k", "v", "log_alpha", "beta", "g")}
        d_out_p = d_out.reshape(1, Tp, Hb, D)
        d_state_p = torch.randn((len(lens), Hb, D, D), device=dev, generator=gen)
        pvl = kda.problem(1, Tp, Hb, D, D, kda.KDA_BF16, floor_b)
        wsv = torch.empty(kda.varlen_backward_workspace_size(pvl, len(lens)), dtype=torch.uint8, device=dev)

        def vstep():
            return kda.varlen_backward(pk["q"], pk["k"], pk["v"], pk["log_alpha"], pk["beta"], pk["g"], floor_b, cu,
                                       d_out=d_out_p, d_state=d_state_p, workspace=wsv)

        gv = vstep()
        torch.cuda.synchronize()
        same_v = True
        for s in (0, len(lens) - 1):
            a0, a1 = int(sum(lens[:s])), int(sum(lens[:s + 1]))
            one = {n: pk[n][:, a0:a1].contiguous() for n in pk}
            rv = kda.backward(one["q"], one["k"], one["v"], one["log_alpha"], one["beta"], one["g"], floor_b,
                              d_out=d_out_p[:, a0:a1].contiguous(), d_state=d_state_p[s:s + 1].contiguous())
            torch.cuda.synchronize()
            same_v = same_v and all(torch.equal(gv[n][:, a0:a1], rv[n]) for n in rv if n != "dstate0") and \
                torch.equal(gv["dstate0"][s:s + 1], rv["dstate0"])
        e0.record()
        for _ in range(reps):
            vstep()
        e1.record()
        torch.cuda.synchronize()
        vms = e0.elapsed_time(e1) / reps
        log(f"[bench] packed backward of {len(lens)} sequences ({min(lens)}..{max(lens)} tokens): {vms:.3f} ms "
            f"(identical to per-sequence backward: {same_v})")
        result["backward"]["varlen"] = {
            "workload": f"kda-varlen-backward {len(lens)} sequences, {Tp} packed tokens, H{Hb} d{D} bf16",
            "ms": vms, "n_seq": len(lens), "min_len": min(lens), "max_len": max(lens),
            "identical_to_per_sequence": same_v}
        del pk, d_out_p, d_state_p, wsv, gv
        del db, wsb, d_out, d_state, fwd_out, ref, got
        torch.cuda.empty_cache()

    # ------------------------------------------------------------- cpu baseline
    if not args.no_cpu_baseline and not args.decode_only:
        import tempfile
        import oracle
        from kda_inputs import to_f64
        # the unmodified oracle source, compiled for this host's CPU; the
        # thread count is the CPU share this job was given
        try:
            oracle.use_library(oracle.build_native(tempfile.mkdtemp(prefix="kda_oracle_")))
            build = "gcc -O3 -march=native"
        except Exception as e:   # no compiler on the host: the portable build the checks use
            build = f"gcc -O3 (portable build; native build failed: {type(e).__name__})"
        sample = workload(2)
        f = lambda a: to_f64(a, "bf16")
        args_o = (f(sample.q), f(sample.k), f(sample.v), sample.log_alpha, sample.beta, f(sample.g),
                  sample.log_alpha_min)
        del sample
        nthr = oracle.host_threads()
        t0 = time.perf_counter()
        oracle.kda_ref(*args_o, nthreads=nthr)
        dt = time.perf_counter() - t0
        del args_o
        try:
            affinity = len(os.sched_getaffinity(0))
        except (AttributeError, OSError):
            affinity = None
        result["cpu_baseline"] = {
            "value": B * T / dt, "unit": "tokens/s", "cores": nthr, "kind": "oracle",
            "sample": f"the whole workload: fp64 step recurrence over all {H} heads x {T} tokens ({dt:.1f} s)",
            "threads_used": nthr, "host_cpus": os.cpu_count(), "affinity_cpus": affinity,
            "threads_rule": "OMP_NUM_THREADS (the CPU share given to the job) if set, else the affinity mask",
            "cpu_model": cpu_model(), "build": build}
        log(f"[bench] oracle {dt:.1f}s on {nthr} threads ({cpu_model()}, {build})")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
