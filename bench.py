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
CHUNK = 64


def falg_per_token_head(dk: int, dv: int, C: int = CHUNK) -> float:
    """Algorithmic flops per token-head of the chunked form (64-token chunks):
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


def cpu_baseline(seconds_hint: float = 20.0) -> dict:
    """The fp64 oracle timed on this host's cores over a bounded sample of the
    forward workload (its first 16384 tokens, all 96 heads)."""
    import numpy as np

    import oracle
    import synth
    from tests import kda_cases as kc

    w = synth.WORKLOADS[3]
    T = 16384
    x = {n: kc.f64(kc.host_tokens(w, n, T)) for n in synth.TOKEN_TENSORS}
    threads = oracle.threads()
    t0 = time.perf_counter()
    oracle.fwd(x["q"], x["k"], x["v"], x["a"], x["b"], x["gate"], np.array([0, T]),
               nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 token recurrence over tokens [0, {T}) of the 1x1048576-token "
                      f"workload, all 96 heads (d=128), {dt:.1f} s wall"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--tokens", type=int, default=1 << 20, help="forward sequence length")
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the KDA hot path shards over heads and "
              "sequences with no communication, so --gpus N > 1 is not run here.",
              file=sys.stderr)
        return 2

    import torch

    import delta_rule_linear_kda_amd as kda
    import synth
    from tests import kda_cases as kc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ---- forward workload: 1 x T tokens, H=96, d=128, bf16 ----------------
    wf = synth.WORKLOADS[3]
    T, H, dk, dv = args.tokens, wf.heads, wf.dk, wf.dv
    xin = {n: kc.device_tokens(wf, n, T) for n in synth.TOKEN_TENSORS}
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    o = torch.empty((T, H, dv), dtype=torch.float32, device=dev)
    sf = torch.empty((1, H, dk, dv), dtype=torch.float32, device=dev)

    # ---- decode workload: 256 x 96 heads, 64 steps of pre-staged tokens -----
    wd = synth.WORKLOADS[4]
    N, D = wd.num_seqs, args.decode_steps
    state = kc.device_state(wd, N)
    dec_in = [{n: kc.device_tokens(wd, n, N, step=s) for n in synth.TOKEN_TENSORS}
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
    fwd_ms = [e[0].elapsed_time(e[1]) for e in ev]
    dec_ms = [e[1].elapsed_time(e[2]) for e in ev]
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    ms_step = wall * 1e3 / args.steps

    th = T * H
    flops = falg_per_token_head(dk, dv) * th
    fbytes = fwd_bytes_per_token_head(dk, dv) * th + 2 * 4 * H * dk * dv * 0  # S0 = 0: no state read
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
        "fwd": {"ms": fwd_avg, "tokens_per_s": fwd_tps, "GB_per_s": fwd_gbs,
                "frac_hbm": fwd_gbs / HBM_PEAK_GBS,
                "TFLOP_per_s_alg": flops / (fwd_avg * 1e-3) / 1e12,
                "frac_bf16_mfma_alg": flops / (fwd_avg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "decode": {"ms_per_step": dec_step_ms, "GB_per_s": dec_gbs,
                   "frac_hbm": dec_gbs / HBM_PEAK_GBS,
                   "tokens_per_s": N / (dec_step_ms * 1e-3)},
        "roofline": {"bound": "hbm", "achieved": fwd_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": fwd_gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "chunk_fwd_kernel<bf16, dk=128>"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
