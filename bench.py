#!/usr/bin/env python3
"""Benchmark of libkda on one MI355X: KDA chunked forward tokens/s at H=96,
d=128 (with its fraction of the bf16 matrix-core peak and of HBM bandwidth)
and decode GB/s (fraction of HBM peak).

One step = one pass of the whole hot path over one batch of synthetic input:
  * kda_fwd_chunked over the long-context workload (1 x 1,048,576 tokens,
    H=96, dk=dv=128, bf16 inputs, fp32 state and output), then
  * 64 kda_decode_step calls over the decode workload (256 sequences x 96
    heads, fp32 state 1.61 GB updated in place, fresh bf16 tokens per step).
Inputs are generated on the device before timing (seeded, synthetic) and are
resident in HBM when the timed region starts.  Each leg is timed with HIP
events recorded on the stream the kernels are launched on.

Prints ONE JSON line.  ``value`` is the forward throughput (tokens/s, a token
being one position across all 96 heads).

After the timed steps (outside them), ``kcp_share`` reports one GPU's share of
the same sequence under 8-way head sharding -- 12 heads, 1 x 1,048,576 tokens
-- through kda_fwd_chunked (direct form: 24 workgroups) and through
kda_fwd_chunked_kcp (segment-transition form with the automatic segment
length), each the mean of 3 launches after one warm-up, and ``layer`` times
the layer operations around the core (short convolution -> Swish -> L2 on q,
RMSNorm -> sigmoid gate on o) on the same resident tensors, and ``bwd`` times
the backward on the 4 x 4096-token, 32-head prefill workload.

Profiling helpers (not part of a timed run):
  --no-kcp-share / --only-kcp-share   skip, or run only, the 12-head comparison;
  --no-layer / --only-layer           skip, or run only, the layer operations;
  --no-bwd / --only-bwd               skip, or run only, the backward;
  --copy-probe          after the timed steps, run a plain 2 GiB device copy so
                        that a hardware-counter run of this same command can
                        scale FETCH_SIZE / WRITE_SIZE against known bytes;
  --pmc-summary F W     turn two rocprofv3 --pmc CSV files (FETCH_SIZE run,
                        WRITE_SIZE run) into the traffic summary text that the
                        forward line's roofline.traffic is read from;
  --trace-spans CSV     from a rocprofv3 --kernel-trace CSV, the wall-clock span
                        of each forward call (first start to last end of its
                        kernels, which overlap across two streams).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E peak, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix-core peak, TFLOP/s
CHUNK = 32                   # chunk length of the bf16 forward kernels
# The bf16 forward transposes b, then runs in blocks of chunks, each block a
# plan kernel, the chunk-record pass and the state pass; the roofline is taken
# over the whole forward call (every launch of these kernels).
FWD_KERNELS = ("chunk_prep_bf16_kernel<128>", "chunk_state_bf16_kernel<128, 4, 2, false, true, false>",
               "split_plan_kernel", "b_transpose_kernel")
FWD_KERNEL = "split forward: " + " + ".join(FWD_KERNELS[:2]) + " (per block of chunks)"
# the two-pass forward's kernel source and the headers its kernels include
FWD_SOURCES = [os.path.join(ROOT, "delta_rule_linear_kda_amd", "csrc", f)
               for f in ("kda_split_bf16.hip", "kda_chunk_common.h", "kda_device.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "split_fwd_bf16_T1048576_H96_d128.traffic.txt")
COPY_PROBE_BYTES = 2 << 30


def falg_per_token_head(dk: int, dv: int, C: int = CHUNK) -> float:
    """Algorithmic flops per token-head of the chunked form with C-token chunks:
    6 dk dv (W S, Qbar S, Kend^T U) + (3C - 1) dk (A, P, W) + 2C dv (U0, P U)
    + C^2 / 3 (the triangular inverse)."""
    return 6 * dk * dv + (3 * C - 1) * dk + 2 * C * dv + C * C / 3.0


def fwd_bytes_per_token_head(dk: int, dv: int, in_bytes: int = 2) -> int:
    """Compulsory HBM bytes per token-head: q, k, a (dk each), v, gate (dv
    each), b (1) in the input dtype, plus the fp32 output row."""
    return in_bytes * (3 * dk + 2 * dv + 1) + 4 * dv


def decode_bytes_per_step(N: int, H: int, dk: int, dv: int, in_bytes: int = 2) -> int:
    """Per decode step: the fp32 state read and written once, the token
    inputs read once, the fp32 output written once."""
    return N * H * (2 * 4 * dk * dv + in_bytes * (3 * dk + 2 * dv + 1) + 4 * dv)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_time(w, lens, heads, t_lim=None, nthreads=None, step=None):
    """Oracle (fp64 token recurrence) time over the sequences `lens` of
    workload w restricted to `heads` (first t_lim tokens of each sequence, in
    8192-token slices with the state carried; decode: one step over every
    sequence).  Input generation is outside the timed region.  Returns
    (seconds, token-heads processed)."""
    import numpy as np

    import oracle
    import synth

    nthreads = nthreads or oracle.threads()
    cu = np.concatenate([[0], np.cumsum(w.seq_lens())]).astype(np.int64)
    dt, done = 0.0, 0
    every = list(heads) == list(range(w.heads))

    def rows(name, t0, t1, st=0):
        """tokens [t0, t1) of `heads` as fp64 [n, len(heads), L] (b: [n, len(heads)])"""
        if every:  # contiguous rows: one generator call
            L = synth.token_row_len(w, name)
            arr = synth.host_normal(synth.key(w.seed, name, st), (t1 - t0) * w.heads, L,
                                    dtype=w.dtype, std=w.std_of(name), base=t0 * w.heads * L)
            arr = synth.to_f64(arr)
            return arr.reshape(t1 - t0, w.heads) if name == "b" else \
                arr.reshape(t1 - t0, w.heads, L)
        return np.stack([synth.to_f64(synth.host_head_slice(w, name, t0, t1, h, step=st))
                         for h in heads], axis=1)

    if step is not None:  # decode: one token per sequence per step, the state carried
        N = w.num_seqs
        if every:
            st = synth.host_state(w, N).astype(np.float64)
        else:
            st = np.stack([np.stack([synth.host_state_item(w, n, h) for h in heads])
                           for n in range(N)]).astype(np.float64)
        for s_ in step:
            x = {n: rows(n, 0, N, s_) for n in synth.TOKEN_TENSORS}
            t0 = time.perf_counter()
            oracle.decode_step(*(x[n] for n in synth.TOKEN_TENSORS), st, nthreads=nthreads)
            dt += time.perf_counter() - t0
            done += N * len(heads)
        return dt, done
    for n in lens:
        L = int(cu[n + 1] - cu[n])
        L = L if t_lim is None else min(L, t_lim)
        state = None
        if w.s0_std is not None:
            state = np.stack([synth.host_state_item(w, n, h) for h in heads])[None].astype(
                np.float64)
        for s0 in range(0, L, 8192):
            s1 = min(L, s0 + 8192)
            x = {nm: rows(nm, int(cu[n]) + s0, int(cu[n]) + s1) for nm in synth.TOKEN_TENSORS}
            t0 = time.perf_counter()
            _, state = oracle.fwd(x["q"], x["k"], x["v"], x["a"], x["b"], x["gate"],
                                  np.array([0, s1 - s0]), state, nthreads=nthreads)
            dt += time.perf_counter() - t0
            done += (s1 - s0) * len(heads)
    return dt, done


def cpu_baseline() -> dict:
    """The fp64 oracle timed on this host's cores, per workload, on all cores
    (<= 16 threads: the host share of one GPU) and on one core, each over a
    bounded sample whose token-heads are stated; tokens/s counts positions
    across all of a workload's heads (token-heads/s divided by H).  The
    headline `value` is the long-context workload's all-core rate."""
    import oracle
    import synth

    threads = oracle.threads()
    W = synth.WORKLOADS
    plan = {  # workload -> (sequences, heads, tokens per sequence or None, decode steps)
        0: (list(range(W[0].num_seqs)), list(range(W[0].heads)), None, None),
        1: (list(range(W[1].num_seqs)), list(range(W[1].heads)), None, None),
        2: (list(range(W[2].num_seqs)), list(range(0, W[2].heads, 12)), None, None),
        3: ([0], list(range(W[3].heads)), 32768, None),
        4: (None, list(range(W[4].heads)), None, list(range(W[4].decode_steps))),
    }
    one_core = {0: ([0], [0], None, None), 1: ([0], [0], 4096, None), 2: ([0], [0], 8192, None),
                3: ([0], [0], 16384, None), 4: (None, list(range(16)), None, [0])}
    per = {}
    for i, w in W.items():
        row = {"workload": w.name}
        for label, spec, nt in (("all_cores", plan[i], threads), ("one_core", one_core[i], 1)):
            seqs, heads, t_lim, steps = spec
            if steps is not None:
                dt, done = _oracle_time(w, None, heads, nthreads=nt, step=steps)
            else:
                dt, done = _oracle_time(w, seqs, heads, t_lim, nthreads=nt)
            row[label] = {"tokens_per_s": done / w.heads / dt, "token_heads": done,
                          "seconds": dt, "threads": nt}
        per[str(i)] = row
    head = per["3"]["all_cores"]
    return {"value": head["tokens_per_s"], "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 token recurrence over tokens [0, 32768) of the 1x1048576-token "
                      f"workload, all 96 heads (d=128), in 8192-token slices with the state "
                      f"carried, {threads} threads, {head['seconds']:.1f} s of oracle time",
            "nproc": os.cpu_count(), "cpu_model": _cpu_model(), "per_config": per}


def fwd_config_leg(i: int, stream, reps: int = 25, warmup: int = 3) -> dict:
    """kda_fwd_chunked on workload i (device-generated inputs and initial
    states, resident before timing): `warmup` untimed calls, then `reps`
    calls each bracketed by HIP events on the launch stream; the median."""
    import torch

    import delta_rule_linear_kda_amd as kda
    import synth

    w = synth.WORKLOADS[i]
    lens = w.seq_lens()
    T, H = int(sum(lens)), w.heads
    x = {n: synth.device_tokens(w, n, T) for n in synth.TOKEN_TENSORS}
    s0 = synth.device_state(w, w.num_seqs)
    cu = torch.tensor(w.cu_seqlens(), dtype=torch.int32, device="cuda")
    o = torch.empty((T, H, w.dv), dtype=torch.float32, device="cuda")
    sf = torch.empty((w.num_seqs, H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    ws_bytes = kda.fwd_workspace_bytes(w.num_seqs, T, H, w.dk, w.dv)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    args = tuple(x[n] for n in ("q", "k", "v", "a", "b", "gate"))

    def call():
        kda.fwd_chunked(*args, cu, s0, out=o, final_state=sf, workspace=ws, stream=stream)

    for _ in range(warmup):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    med = ms[len(ms) // 2]
    th = T * H
    nbytes = fwd_bytes_per_token_head(w.dk, w.dv) * th + 4 * w.num_seqs * H * w.dk * w.dv * (
        2 if s0 is not None else 1)
    gbs = nbytes / (med * 1e-3) / 1e9
    out = {"workload": w.name, "tokens": T, "heads": H, "reps": reps, "ms_median": med,
           "ms_min": ms[0], "ms_max": ms[-1], "tokens_per_s": T / (med * 1e-3),
           "GB_per_s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
           "frac_bf16_mfma_alg": falg_per_token_head(w.dk, w.dv) * th / (med * 1e-3) / 1e12
           / BF16_PEAK_TFLOPS,
           "frac_bf16_mfma_alg_c64": falg_per_token_head(w.dk, w.dv, 64) * th / (med * 1e-3)
           / 1e12 / BF16_PEAK_TFLOPS,
           "form": "two-pass" if ws_bytes > 0 else "fused", "workspace_bytes": ws_bytes}
    del x, o, sf, ws
    torch.cuda.empty_cache()
    return out


def kcp_share(T: int, stream, reps: int = 3) -> dict:
    """Direct vs segment-transition form on 12 heads x 1 x T tokens."""
    import torch

    import delta_rule_linear_kda_amd as kda
    import synth

    H = 12
    w = synth.custom_workload(synth.WORKLOADS[3], heads=H)
    x = {n: synth.device_tokens(w, n, T) for n in synth.TOKEN_TENSORS}
    args = tuple(x[n] for n in ("q", "k", "v", "a", "b", "gate"))
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    o = torch.empty((T, H, w.dv), dtype=torch.float32, device="cuda")
    sf = torch.empty((1, H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    ws_bytes = kda.kcp_workspace_bytes(1, T, H, w.dk, w.dv, 0)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def timed(fn) -> float:
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    direct = timed(lambda: kda.fwd_chunked(*args, cu, None, out=o, final_state=sf, stream=stream))
    seg = timed(lambda: kda.fwd_chunked_kcp(*args, cu, None, out=o, final_state=sf,
                                            workspace=ws, stream=stream))
    return {"workload": f"kda_fwd_bf16_T{T}_H{H}_d128 (one GPU's share under 8-way head "
                        f"sharding)", "direct_ms": direct, "segment_form_ms": seg,
            "segment_form_tokens_per_s": T / (seg * 1e-3), "speedup": direct / seg,
            "workspace_bytes": ws_bytes}


def cp_share(xin: dict, stream, T: int = 1 << 17, reps: int = 3) -> dict:
    """One GPU's share of the long-context workload under 8-way sequence
    splitting (context parallelism): the first T/8 = 131,072 tokens x 96
    heads of the resident tensors, as the segment it would own.  Times the
    two per-GPU kernels of that split: the segment's [S_loc | M] transition
    and the forward from the composed start state (here zero)."""
    import torch

    import delta_rule_linear_kda_amd as kda

    x = {n: xin[n][:T] for n in ("q", "k", "v", "a", "b", "gate")}
    H, dk, dv = x["q"].shape[1], x["q"].shape[2], x["v"].shape[2]
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    o = torch.empty((T, H, dv), dtype=torch.float32, device="cuda")
    sf = torch.empty((1, H, dk, dv), dtype=torch.float32, device="cuda")
    tr = torch.empty((1, H, dk, dv + dk), dtype=torch.float32, device="cuda")

    def timed(fn) -> float:
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    fwd = timed(lambda: kda.fwd_chunked(x["q"], x["k"], x["v"], x["a"], x["b"], x["gate"], cu,
                                        None, out=o, final_state=sf, stream=stream))
    trans = timed(lambda: kda.segment_transition(x["k"], x["v"], x["a"], x["b"], cu, out=tr,
                                                 stream=stream))
    return {"workload": f"kda_fwd_bf16_T{T}_H{H}_d128 (one GPU's segment under 8-way sequence "
                        f"splitting)", "forward_ms": fwd, "transition_ms": trans,
            "forward_tokens_per_s": T / (fwd * 1e-3)}


def layer_ops(q, gate, o, stream, reps: int = 5) -> dict:
    """The layer operations around the core on the resident long-context
    tensors: the short convolution -> Swish -> L2 front on q (width 4,
    synthetic weights) and the RMSNorm -> sigmoid gate back on o (in place).
    Algorithmic bytes: front 2 x 2 B per element (bf16 in and out), back
    4 + 2 + 4 B per element (fp32 o read and written, bf16 gate read)."""
    import torch

    import delta_rule_linear_kda_amd as kda

    T, H, d = q.shape
    wt = torch.full((H, d, 4), 0.25, dtype=torch.float32, device=q.device)
    nw = torch.ones(o.shape[2], dtype=torch.float32, device=q.device)
    cu = torch.tensor([0, T], dtype=torch.int32, device=q.device)
    y = torch.empty_like(q)

    def timed(fn) -> float:
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_f = timed(lambda: kda.shortconv_swish_l2(q, wt, cu, out=y, stream=stream))
    ms_b = timed(lambda: kda.rmsnorm_gate(o, gate, nw, 1e-6, out=o, stream=stream))
    bf, bb = 4.0 * q.numel(), 10.0 * o.numel()
    return {"workload": f"{T} tokens x {H} heads x d={d}, bf16 q and gate, fp32 o",
            "shortconv_swish_l2": {"ms": ms_f, "GB_per_s": bf / ms_f / 1e6,
                                   "frac_hbm": bf / ms_f / 1e6 / HBM_PEAK_GBS},
            "rmsnorm_gate": {"ms": ms_b, "GB_per_s": bb / ms_b / 1e6,
                             "frac_hbm": bb / ms_b / 1e6 / HBM_PEAK_GBS}}


def fused_norm_leg(xin: dict, cu, o, sf, fwd_ms: float, norm_ms: float, stream,
                   reps: int = 3) -> dict:
    """The forward with the head-wise RMSNorm -> sigmoid gate applied in its
    output stage (kda_fwd_chunked_rmsnorm_gate) on the resident long-context
    tensors, against the forward followed by the separate norm pass."""
    import torch

    import delta_rule_linear_kda_amd as kda

    T, H, dk = xin["q"].shape
    dv = xin["v"].shape[2]
    nw = torch.ones(dv, dtype=torch.float32, device=o.device)
    ws = torch.empty(max(kda.fwd_workspace_bytes(1, T, H, dk, dv), 1), dtype=torch.uint8,
                     device=o.device)
    args = tuple(xin[n] for n in ("q", "k", "v", "a", "b", "gate"))

    def call():
        kda.fwd_chunked_rmsnorm_gate(*args, cu, None, nw, 1e-6, out=o, final_state=sf,
                                     workspace=ws, stream=stream)

    call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"ms": ms, "forward_then_norm_pass_ms": fwd_ms + norm_ms,
            "saved_ms": fwd_ms + norm_ms - ms}


def backward(stream, reps: int = 3) -> dict:
    """kda_bwd_chunked on the training-shaped prefill workload (4 x 4096
    tokens, 32 heads, d = 128, bf16 inputs, zero initial state, fp32 dy):
    the forward recomputation with states every 64 tokens, the adjoint
    recurrence and the reduction over column slices, one call each."""
    import torch

    import delta_rule_linear_kda_amd as kda
    import synth

    w = synth.WORKLOADS[1]
    T, H = sum(w.seq_lens()), w.heads
    x = {n: synth.device_tokens(w, n, T) for n in synth.TOKEN_TENSORS}
    args = tuple(x[n] for n in ("q", "k", "v", "a", "b", "gate"))
    cu = torch.tensor(w.cu_seqlens(), dtype=torch.int32, device="cuda")
    dy = torch.empty((T, H, w.dv), dtype=torch.float32, device="cuda")
    synth.device_normal(dy.view(-1, w.dv), synth.key(w.seed, "o", 1))
    ws = torch.empty(kda.bwd_workspace_bytes(w.num_seqs, T, H, w.dk, w.dv), dtype=torch.uint8,
                     device="cuda")

    def timed(fn) -> float:
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    fwd_ms = timed(lambda: kda.fwd_chunked(*args, cu, None, stream=stream))
    bwd_ms = timed(lambda: kda.bwd_chunked(*args, cu, None, dy, None, workspace=ws,
                                           stream=stream))
    return {"workload": f"kda_bwd_bf16_{w.num_seqs}x{T // w.num_seqs}_H{H}_d{w.dk}",
            "ms": bwd_ms, "tokens_per_s": T / (bwd_ms * 1e-3), "fwd_ms": fwd_ms,
            "bwd_over_fwd": bwd_ms / fwd_ms, "workspace_bytes": ws.numel()}


def _sha256(paths: list) -> str:
    """sha256 of C/HIP sources' code: comments removed and whitespace
    collapsed, so that editing a comment does not invalidate counters taken
    on unchanged code."""
    import hashlib
    import re

    text = ""
    for path in paths:
        with open(path) as f:
            text += f.read() + "\n"
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


def read_traffic() -> dict | None:
    """HBM bytes per forward launch from the committed counter summary, or
    None when it is absent or was taken on a different kernel source."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_code_sha256") != _sha256(FWD_SOURCES):
            return None
        return {"fetch": float(kv["fetch_bytes_per_launch"]),
                "write": float(kv["write_bytes_per_launch"])}
    except (OSError, KeyError, ValueError):
        return None


def pmc_summary(fetch_csv: str, write_csv: str) -> str:
    """Summarise a FETCH_SIZE run and a WRITE_SIZE run of ``bench.py --steps 1
    --warmup 0 --copy-probe`` (rocprofv3 --pmc, csv output).  Each counter is
    calibrated on the plain copy of COPY_PROBE_BYTES (it reads and writes
    exactly that many bytes), then summed over every dispatch of the forward's
    kernels: the run makes exactly one forward call."""
    import csv

    def per_dispatch(path: str, counter: str) -> dict:
        acc: dict = {}
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                d = acc.setdefault(r["Kernel_Name"], {})
                d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        return {k: list(v.values()) for k, v in acc.items()}

    fetch = per_dispatch(fetch_csv, "FETCH_SIZE")
    write = per_dispatch(write_csv, "WRITE_SIZE")

    def pick(d: dict, word: str) -> tuple:
        hits = [(k, v) for k, v in d.items() if word in k]
        if len(hits) != 1:
            raise SystemExit(f"expected one kernel matching {word!r}, got {[h[0] for h in hits]}")
        return hits[0]

    # The probe's device-to-device copy is the runtime's copy kernel; its
    # largest dispatch is the probe (others are small staging copies).
    _, cfl = pick(fetch, "copyBuffer")
    _, cwl = pick(write, "copyBuffer")
    cf, cw = max(cfl), max(cwl)
    f_scale = COPY_PROBE_BYTES / (cf * 1024.0)
    w_scale = COPY_PROBE_BYTES / (cw * 1024.0)
    lines = [
        "# HBM traffic of one forward call (every dispatch of its kernels)",
        "# workload: 1 x 1048576 tokens, H=96, dk=dv=128, bf16 inputs, fp32 o, final state",
        f"copy_probe_bytes: {COPY_PROBE_BYTES}",
        f"copy_fetch_kib: {cf:.1f}",
        f"copy_write_kib: {cw:.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
    ]
    fb = wb = 0.0
    for kn in FWD_KERNELS:
        name, kfl = pick(fetch, kn)
        _, kwl = pick(write, kn)
        kf, kw = sum(kfl) * 1024.0 * f_scale, sum(kwl) * 1024.0 * w_scale
        fb, wb = fb + kf, wb + kw
        lines += [f"# {name[:100]}: {len(kfl)} dispatches",
                  f"fetch_bytes[{kn}]: {kf:.0f}", f"write_bytes[{kn}]: {kw:.0f}"]
    lines += [
        f"fetch_bytes_per_launch: {fb:.0f}",
        f"write_bytes_per_launch: {wb:.0f}",
        f"kernel_code_sha256: {_sha256(FWD_SOURCES)}",
    ]
    return "\n".join(lines) + "\n"


def util_summary(pmc_csv: str) -> str:
    """Per-kernel utilization from one rocprofv3 --pmc run of GRBM_GUI_ACTIVE,
    SQ_ACTIVE_INST_VALU, SQ_VALU_MFMA_BUSY_CYCLES, SQ_ACTIVE_INST_LDS,
    SQ_LDS_BANK_CONFLICT, SQ_INSTS_VALU, SQ_INSTS_MFMA (csv output), as
    rocprofv3 defines the derived metrics, GRBM_GUI_ACTIVE taken per XCD (the
    csv sums its 8 instances): VALUBusy = SQ_ACTIVE_INST_VALU / CUs /
    GRBM_GUI_ACTIVE, MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x
    GRBM_GUI_ACTIVE), LDSinst and LDSconf likewise per CU."""
    import collections
    import csv

    agg = collections.defaultdict(lambda: collections.defaultdict(float))
    dur = collections.defaultdict(float)
    seen = collections.defaultdict(set)
    with open(pmc_csv, newline="") as f:
        for r in csv.DictReader(f):
            k = r["Kernel_Name"].replace("void ", "").replace("kda::(anonymous namespace)::", "")
            k = k.replace("(anonymous namespace)::", "").split("(")[0]
            agg[k][r["Counter_Name"]] += float(r["Counter_Value"])
            if r["Dispatch_Id"] not in seen[k]:
                seen[k].add(r["Dispatch_Id"])
                dur[k] += (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    cu, simd = 256, 1024
    lines = []
    for k, c in agg.items():
        g = c["GRBM_GUI_ACTIVE"] / 8
        if g == 0:
            continue
        n = len(seen[k])
        lines.append(
            f"{k[:60]:<60} n={n:4d} dur={dur[k] * 1e3 / n:8.3f}ms "
            f"clk={g / n / (dur[k] / n) / 1e9:5.2f}GHz "
            f"VALUBusy={100 * c['SQ_ACTIVE_INST_VALU'] / cu / g:5.1f}% "
            f"MfmaUtil={100 * c['SQ_VALU_MFMA_BUSY_CYCLES'] / (g * simd):5.1f}% "
            f"LDSinst={100 * c['SQ_ACTIVE_INST_LDS'] / cu / g:5.1f}% "
            f"LDSconf={100 * c['SQ_LDS_BANK_CONFLICT'] / cu / g:5.1f}% "
            f"VALUinsts/MFMA={c['SQ_INSTS_VALU'] / max(1, c['SQ_INSTS_MFMA']):7.1f}")
    return "\n".join(lines) + "\n"


def kernel_stats(stats_csv: str) -> str:
    """The kernel table of a rocprofv3 --kernel-trace --stats csv: calls,
    average / min / max duration (us), share of the total."""
    import csv

    lines = [f"{'kernel':<78} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
    with open(stats_csv, newline="") as f:
        for r in csv.DictReader(f):
            k = r["Name"].replace("void ", "").replace("kda::(anonymous namespace)::", "")
            k = k.replace("(anonymous namespace)::", "").split("(")[0]
            lines.append(f"{k[:78]:<78} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                         f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f} "
                         f"{float(r['Percentage']):6.2f}")
    return "\n".join(lines) + "\n"


def trace_spans(trace_csv: str) -> str:
    """Per forward call: first start to last end of its kernels' dispatches
    (calls are separated by the decode launches that follow each forward)."""
    import csv

    rows = []
    with open(trace_csv, newline="") as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    calls, cur = [], None
    for st, en, name in rows:
        if any(k in name for k in FWD_KERNELS):
            if cur is None:
                cur = [st, en, 0]
            cur[0], cur[1], cur[2] = min(cur[0], st), max(cur[1], en), cur[2] + 1
        elif "decode_kernel" in name and cur is not None:
            calls.append(cur)
            cur = None
    if cur is not None:
        calls.append(cur)
    lines = [f"forward call {i}: {c[2]} dispatches, span {(c[1] - c[0]) / 1e6:.3f} ms"
             for i, c in enumerate(calls)]
    return "\n".join(lines) + "\n"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--tokens", type=int, default=1 << 20, help="forward sequence length")
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kcp-share", action="store_true")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip timing the layer operations around the core")
    ap.add_argument("--only-layer", action="store_true",
                    help="time only the layer operations around the core")
    ap.add_argument("--no-bwd", action="store_true", help="skip timing the backward")
    ap.add_argument("--only-bwd", action="store_true", help="time only the backward")
    ap.add_argument("--only-kcp-share", action="store_true",
                    help="run only the 12-head direct vs segment-form comparison")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload forward legs (4 x 4096 x 32, varlen 16 x 96)")
    ap.add_argument("--only-configs", action="store_true",
                    help="time only the per-workload forward legs")
    ap.add_argument("--only-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--trace-spans", metavar="TRACE_CSV")
    ap.add_argument("--util-summary", metavar="PMC_CSV")
    ap.add_argument("--kernel-stats", metavar="STATS_CSV")
    args = ap.parse_args()

    if args.trace_spans:
        sys.stdout.write(trace_spans(args.trace_spans))
        return 0
    if args.util_summary:
        sys.stdout.write(util_summary(args.util_summary))
        return 0
    if args.kernel_stats:
        sys.stdout.write(kernel_stats(args.kernel_stats))
        return 0
    if args.pmc_summary:
        sys.stdout.write(pmc_summary(*args.pmc_summary))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the KDA hot path shards over heads and "
              "sequences with no communication, so --gpus N > 1 is not run here.",
              file=sys.stderr)
        return 2

    import torch

    import delta_rule_linear_kda_amd as kda
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.only_kcp_share:
        print(json.dumps({"kcp_share": kcp_share(args.tokens, stream)}), flush=True)
        return 0
    if args.only_bwd:
        print(json.dumps({"bwd": backward(stream)}), flush=True)
        return 0
    if args.only_configs:
        print(json.dumps({"fwd_configs": {str(i): fwd_config_leg(i, stream) for i in (1, 2)}}),
              flush=True)
        return 0
    if args.only_cpu_baseline:
        print(json.dumps({"cpu_baseline": cpu_baseline()}), flush=True)
        return 0
    if args.only_layer:
        wl = synth.WORKLOADS[3]
        q = synth.device_tokens(wl, "q", args.tokens)
        g = synth.device_tokens(wl, "gate", args.tokens)
        o = torch.empty((args.tokens, wl.heads, wl.dv), dtype=torch.float32, device=dev)
        synth.device_normal(o.view(-1, wl.dv), synth.key(wl.seed, "o"))
        print(json.dumps({"layer": layer_ops(q, g, o, stream)}), flush=True)
        return 0

    # ---- forward workload: 1 x T tokens, H=96, d=128, bf16 ----------------
    wf = synth.WORKLOADS[3]
    T, H, dk, dv = args.tokens, wf.heads, wf.dk, wf.dv
    xin = {n: synth.device_tokens(wf, n, T) for n in synth.TOKEN_TENSORS}
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    o = torch.empty((T, H, dv), dtype=torch.float32, device=dev)
    sf = torch.empty((1, H, dk, dv), dtype=torch.float32, device=dev)

    # ---- decode workload: 256 x 96 heads, 64 steps of pre-staged tokens -----
    wd = synth.WORKLOADS[4]
    N, D = wd.num_seqs, args.decode_steps
    state = synth.device_state(wd, N)
    dec_in = [{n: synth.device_tokens(wd, n, N, step=s) for n in synth.TOKEN_TENSORS}
              for s in range(D)]
    o_dec = torch.empty((N, wd.heads, wd.dv), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def fwd():
        kda.fwd_chunked(xin["q"], xin["k"], xin["v"], xin["a"], xin["b"], xin["gate"], cu, None,
                        out=o, final_state=sf, stream=stream)

    def decode_pass():
        for s in range(D):
            x = dec_in[s]
            kda.decode_step(x["q"], x["k"], x["v"], x["a"], x["b"], x["gate"], state, out=o_dec,
                            stream=stream)

    for _ in range(args.warmup):
        fwd()
        decode_pass()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        fwd()
        ev[s][1].record(stream)
        decode_pass()
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    if args.copy_probe:
        n = COPY_PROBE_BYTES // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    fwd_ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    dec_ms = sorted(e[1].elapsed_time(e[2]) for e in ev)
    fwd_avg = fwd_ms[len(fwd_ms) // 2]  # medians over the timed steps
    dec_avg = dec_ms[len(dec_ms) // 2]
    ms_step = wall * 1e3 / args.steps

    th = T * H
    falg = falg_per_token_head(dk, dv)
    flops = falg * th
    fbytes = fwd_bytes_per_token_head(dk, dv) * th + 4 * H * dk * dv  # + final state (S0 = 0: none read)
    fwd_tps = T / (fwd_avg * 1e-3)
    fwd_gbs = fbytes / (fwd_avg * 1e-3) / 1e9
    dbytes = decode_bytes_per_step(N, wd.heads, wd.dk, wd.dv)
    dec_step_ms = dec_avg / D
    dec_gbs = dbytes / (dec_step_ms * 1e-3) / 1e9

    out = {
        "metric": "KDA fwd tokens/s at H=96,d=128 (% bf16 MFMA peak); decode GB/s (% HBM)",
        "value": fwd_tps,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller, generated on device)",
        "config": {"workload": f"kda_fwd_bf16_T{T}_H96_d128 + kda_decode_bf16_N256_H96_d128 "
                               f"x{D} steps", "fwd_tokens": T, "heads": H, "dk": dk, "dv": dv,
                   "chunk": CHUNK, "decode_seqs": N, "decode_steps": D},
        "fwd": {"ms": fwd_avg, "ms_min": fwd_ms[0], "ms_max": fwd_ms[-1],
                "tokens_per_s": fwd_tps, "GB_per_s": fwd_gbs,
                "frac_hbm": fwd_gbs / HBM_PEAK_GBS,
                "TFLOP_per_s_alg": flops / (fwd_avg * 1e-3) / 1e12,
                "frac_bf16_mfma_alg": flops / (fwd_avg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                "frac_bf16_mfma_alg_c64": falg_per_token_head(dk, dv, 64) * th / (fwd_avg * 1e-3)
                / 1e12 / BF16_PEAK_TFLOPS,
                "falg_per_token_head": falg, "bytes_per_token_head": fwd_bytes_per_token_head(dk, dv)},
        "decode": {"ms_per_step": dec_step_ms, "GB_per_s": dec_gbs,
                   "frac_hbm": dec_gbs / HBM_PEAK_GBS,
                   "tokens_per_s": N / (dec_step_ms * 1e-3)},
        "roofline": {"bound": "hbm", "achieved": fwd_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": fwd_gbs / HBM_PEAK_GBS, "traffic": None, "kernel": FWD_KERNEL},
    }
    tr = read_traffic() if T == 1 << 20 else None
    if tr is not None:
        out["roofline"]["traffic"] = tr["fetch"] + tr["write"]
        out["roofline"]["traffic_fetch"] = tr["fetch"]
        out["roofline"]["traffic_write"] = tr["write"]
    if not args.no_layer:
        out["layer"] = layer_ops(xin["q"], xin["gate"], o, stream)
        out["layer"]["fwd_rmsnorm_gate"] = fused_norm_leg(
            xin, cu, o, sf, fwd_avg, out["layer"]["rmsnorm_gate"]["ms"], stream)
    if not args.no_kcp_share:
        out["cp_share"] = cp_share(xin, stream)
    if not args.no_kcp_share or not args.no_bwd or not args.no_configs:
        del xin, o, dec_in
        torch.cuda.empty_cache()
    if not args.no_configs:
        out["fwd_configs"] = {str(i): fwd_config_leg(i, stream) for i in (1, 2)}
    if not args.no_bwd:
        out["bwd"] = backward(stream)
    if not args.no_kcp_share:
        torch.cuda.empty_cache()
        out["kcp_share"] = kcp_share(T, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
