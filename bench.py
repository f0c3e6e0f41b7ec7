"""Benchmark: KDA chunked prefill tokens/s and decode-step state GB/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--profile]

One step = one chunked prefill (chunk prep + chunked recurrence) of the
single-sequence workload T=8192, H=32, d_k=d_v=128, bf16 I/O, fp32 state, with
seeded synthetic inputs resident in HBM.  Four copies of the inputs are rotated
so a step never finds its inputs in the 256 MB MALL.  Before the W warm-up
steps, untimed calls run until --ramp-ms of GPU time has passed, because the
shader clock rises over the first ~25 ms of load.  K back-to-back steps are
timed between device synchronisations, with two HIP events on the launch stream
around them giving the average call duration behind the roofline figure; a
separate loop with events around each call gives the per-call spread.  In
the same run the decode step is timed on 256 sequences x 32 heads (512 MiB
fp32 state, advanced in place), one pipelined prefill of a single 2^20-token
sequence with 16 heads and one packed batch of 64 sequences (about 1M tokens,
32 heads) are timed as secondary figures, and the fp64 oracle is
timed on the host cores on the full prefill workload (repeated to ~10 s of CPU
work).

Prints one JSON line (rank 0, N = 1).
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA chunked-prefill tokens/s and decode-step state HBM GB/s on 1 MI355X"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6       # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk
D = 128
PREFILL_T, PREFILL_H = 8192, 32
DECODE_N, DECODE_H = 256, 32


def prefill_algorithmic_bytes(T, H, d, n_seqs=1):
    """q, k, v, g (4 x 2d B), beta (2 B) in, o (2d B) out per token-head, plus the
    fp32 state read and written once per (sequence, head)."""
    return (10 * d + 2) * T * H + 2 * 4 * d * d * n_seqs * H


def prefill_executed_flops(T, H, d, C=64):
    """MFMA work per token-head as executed (full tiles): 6 d^2 + 10 C d + C^2 / 3."""
    return (6 * d * d + 10 * C * d + C * C / 3) * T * H


def decode_state_bytes(n, h, d):
    return 2 * 4 * d * d * n * h


def decode_token_bytes(n, h, d):
    return (10 * d + 2) * n * h


def source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "linear_attention_recurrence_06_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(kind: str):
    """HBM bytes per call from the committed rocprofv3 counter summary, or None
    when it is missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash() or kind not in t:
        return None
    return t[kind].get("hbm_bytes_per_call")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--ramp-ms", type=float, default=80.0,
                    help="untimed prefill calls before the warm-up steps until this much GPU "
                         "time has passed (the shader clock rises over the first ~25 ms of load)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="short run for profilers: the clock ramp, few steps, no CPU baseline, one 1 GiB "
                         "device copy as a traffic calibration")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(heads and sequences shard across GPUs with no exchange, so one GPU's "
              "throughput is the per-GPU figure)", file=sys.stderr)
        sys.exit(2)
    if args.profile:
        args.steps, args.warmup, args.decode_steps = 5, 2, 10
        args.no_cpu_baseline = True

    import numpy as np
    import torch

    import linear_attention_recurrence_06_amd as kda
    from kda_inputs import CONFIGS, make_config_decode, make_config_prefill

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    kda.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    # ------------------------------------------------------------------ prefill
    base = make_config_prefill(1, device=dev)
    T, H = PREFILL_T, PREFILL_H
    sets = [base] + [{k: (v.clone() if torch.is_tensor(v) else v) for k, v in base.items()}
                     for _ in range(3)]
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    dims = kda.make_dims(T, 1, H, D, D, 0)
    ws = torch.empty(kda.kda_prefill_workspace_bytes(dims), dtype=torch.uint8, device=dev)

    def prefill(i):
        s = sets[i % len(sets)]
        kda.kda_chunk_prefill(s["q"], s["k"], s["v"], s["g"], s["beta"], s["initial_state"],
                              None, out, fin, workspace=ws, stream=stream)

    # clock ramp: untimed calls until ramp_ms of GPU time has passed
    ramp_s, r_i = 0.0, 0
    while ramp_s * 1e3 < args.ramp_ms:
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0.record(stream)
        for _ in range(10):
            prefill(r_i)
            r_i += 1
        r1.record(stream)
        torch.cuda.synchronize(dev)
        ramp_s += r0.elapsed_time(r1) * 1e-3
    for i in range(args.warmup):
        prefill(i)
    # timed region: K back-to-back calls bracketed by two events on the
    # launch stream (per-call events inside it would serialise the calls)
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    e_start.record(stream)
    for i in range(args.steps):
        prefill(i)
    e_end.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    call_avg_s = e_start.elapsed_time(e_end) * 1e-3 / args.steps
    tokens_per_s = T / (wall / args.steps)
    # per-call spread, in a separate loop with events around each call
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        prefill(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize(dev)
    call_ms = [a.elapsed_time(b) for a, b in ev]
    p_bytes = prefill_algorithmic_bytes(T, H, D)
    p_achieved = p_bytes / call_avg_s / 1e9
    p_traffic = counter_traffic("prefill")

    # checkpointed prefill (intermediate states every `interval` chunks)
    ckpt = {}
    for interval in (16, 1):
        n_ck = kda.kda_checkpoint_count(dims, None, interval)
        ck_buf = torch.empty((n_ck, H, D, D), dtype=torch.float32, device=dev)
        reps = max(3, args.steps // 4)
        for i in range(2):
            kda.kda_chunk_prefill_checkpoints(
                sets[i]["q"], sets[i]["k"], sets[i]["v"], sets[i]["g"], sets[i]["beta"],
                sets[i]["initial_state"], None, out, fin, checkpoint_interval=interval,
                checkpoints=ck_buf, workspace=ws, stream=stream)
        ck_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(reps)]
        for i in range(reps):
            s_ = sets[i % len(sets)]
            ck_ev[i][0].record(stream)
            kda.kda_chunk_prefill_checkpoints(
                s_["q"], s_["k"], s_["v"], s_["g"], s_["beta"], s_["initial_state"], None, out,
                fin, checkpoint_interval=interval, checkpoints=ck_buf, workspace=ws,
                stream=stream)
            ck_ev[i][1].record(stream)
        torch.cuda.synchronize(dev)
        ck_us = float(np.median([a.elapsed_time(b) for a, b in ck_ev])) * 1e3
        ckpt[f"every_{interval}_chunks"] = {
            "checkpoints": n_ck, "bytes_written": n_ck * H * D * D * 4,
            "median_call_us": ck_us,
            "overhead_vs_plain_median": ck_us / (float(np.median(call_ms)) * 1e3) - 1.0}
        del ck_buf

    # per-head (scalar) gate: g [T, H], same workload otherwise
    from kda_inputs import make_prefill as _mk
    sg_in = _mk([T], H, D, "bf16", g_scale=0.5, s0_std=0.02, seed=1, device=dev, scalar_gate=True)
    for i in range(2):
        kda.kda_chunk_prefill(sg_in["q"], sg_in["k"], sg_in["v"], sg_in["g"], sg_in["beta"],
                              sg_in["initial_state"], None, out, fin, workspace=ws, stream=stream)
    sg_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(max(3, args.steps // 4))]
    for a_, b_ in sg_ev:
        a_.record(stream)
        kda.kda_chunk_prefill(sg_in["q"], sg_in["k"], sg_in["v"], sg_in["g"], sg_in["beta"],
                              sg_in["initial_state"], None, out, fin, workspace=ws, stream=stream)
        b_.record(stream)
    torch.cuda.synchronize(dev)
    sg_us = float(np.median([a_.elapsed_time(b_) for a_, b_ in sg_ev])) * 1e3
    del sg_in

    def median_call_us(fn, reps):
        for _ in range(2):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a_, b_ in evs:
            a_.record(stream)
            fn()
            b_.record(stream)
        torch.cuda.synchronize(dev)
        return float(np.median([a_.elapsed_time(b_) for a_, b_ in evs])) * 1e3

    # output gate fused into the output write: out = o * sigmoid(z), z [T, H, d_v]
    from kda_inputs import make_out_gate
    z_pf = make_out_gate((T, H, D), "bf16", seed=2, device=dev)
    og_us = median_call_us(
        lambda: kda.kda_chunk_prefill_ex(base["q"], base["k"], base["v"], base["g"],
                                         base["beta"], base["initial_state"], None, out, fin,
                                         out_gate_z=z_pf, workspace=ws, stream=stream),
        max(3, args.steps // 4))
    del z_pf

    # front end: raw q, k, v through a width-4 convolution with SiLU, g from a
    # rank-64 projection (g not read)
    from kda_inputs import make_front_end
    fe_in = make_front_end(T, 1, H, D, "bf16", width=4, rank=64, bias_std=0.3, seed=4,
                           device=dev)
    fe_state_out = torch.empty_like(fe_in["conv_state"])
    fe_us = median_call_us(
        lambda: kda.kda_chunk_prefill_ex(base["q"], base["k"], base["v"], None, base["beta"],
                                         base["initial_state"], None, out, fin,
                                         conv_weight=fe_in["conv_weight"], conv_silu=True,
                                         conv_state_in=fe_in["conv_state"],
                                         conv_state_out=fe_state_out, gate_a=fe_in["gate_a"],
                                         gate_b=fe_in["gate_b"], gate_bias=fe_in["gate_bias"],
                                         workspace=ws, stream=stream),
        max(3, args.steps // 4))
    fe_bytes = p_bytes - 2 * D * T * H + 2 * 64 * T + 2 * H * D * 64


    # ------------------------------------------------------------------ decode
    dw = make_config_decode(3, device=dev, steps=args.decode_steps)
    state = dw["state"]
    dout = torch.empty((DECODE_N, DECODE_H, D), dtype=torch.bfloat16, device=dev)

    def decode(s):
        kda.kda_decode_step(dw["q"][s], dw["k"][s], dw["v"][s], dw["g"][s], dw["beta"][s],
                            state, dout, stream=stream)

    for s in range(min(3, args.decode_steps)):
        decode(s)
    torch.cuda.synchronize(dev)
    d_start, d_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t1 = time.perf_counter()
    d_start.record(stream)
    for s in range(args.decode_steps):
        decode(s)
    d_end.record(stream)
    torch.cuda.synchronize(dev)
    d_wall = time.perf_counter() - t1
    d_avg_s = d_start.elapsed_time(d_end) * 1e-3 / args.decode_steps
    # per-step spread, in a separate loop with events around each step
    n_spread = min(20, args.decode_steps)
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_spread)]
    for s in range(n_spread):
        dev_ev[s][0].record(stream)
        decode(s)
        dev_ev[s][1].record(stream)
    torch.cuda.synchronize(dev)
    d_ms = [a.elapsed_time(b) for a, b in dev_ev]
    sb = decode_state_bytes(DECODE_N, DECODE_H, D)
    tb = decode_token_bytes(DECODE_N, DECODE_H, D)
    d_traffic = counter_traffic("decode")

    # decode with the output gate per value channel (z [N, H, d_v])
    z_dec = make_out_gate((DECODE_N, DECODE_H, D), "bf16", seed=3, device=dev)
    og_dec_us = median_call_us(
        lambda: kda.kda_decode_step_ex(dw["q"][0], dw["k"][0], dw["v"][0], dw["g"][0],
                                       dw["beta"][0], state, dout, out_gate_z=z_dec,
                                       stream=stream),
        max(10, args.decode_steps // 4))
    del z_dec

    # decode with the front end (width-4 convolution state advanced in place,
    # rank-64 gate)
    fe_dec = make_front_end(DECODE_N, DECODE_N, DECODE_H, D, "bf16", width=4, rank=64,
                            bias_std=0.3, seed=5, device=dev)
    fe_dec_us = median_call_us(
        lambda: kda.kda_decode_step_ex(dw["q"][0], dw["k"][0], dw["v"][0], None, dw["beta"][0],
                                       state, dout, conv_weight=fe_dec["conv_weight"],
                                       conv_silu=True, conv_state=fe_dec["conv_state"],
                                       gate_a=fe_dec["gate_a"], gate_b=fe_dec["gate_b"],
                                       gate_bias=fe_dec["gate_bias"], stream=stream),
        max(10, args.decode_steps // 4))
    del fe_dec

    # one long sequence: 2^20 tokens x 16 heads, which the library pipelines over
    # two streams (chunk prep of later segments beside the recurrence of earlier
    # ones, since 16 heads x 8 column tiles leave half the CUs to the prep)
    long_in = make_config_prefill(4, device=dev)
    LT, LH = long_in["q"].shape[0], long_in["q"].shape[1]
    l_dims = kda.make_dims(LT, 1, LH, D, D, 0)
    l_ws = torch.empty(kda.kda_prefill_workspace_bytes(l_dims), dtype=torch.uint8, device=dev)
    l_out = torch.empty((LT, LH, D), dtype=torch.bfloat16, device=dev)
    l_fin = torch.empty((1, LH, D, D), dtype=torch.float32, device=dev)
    long_us = median_call_us(
        lambda: kda.kda_chunk_prefill(long_in["q"], long_in["k"], long_in["v"], long_in["g"],
                                      long_in["beta"], long_in["initial_state"], None, l_out,
                                      l_fin, workspace=l_ws, stream=stream),
        2 if args.profile else 4)
    long_segs = kda.kda_prefill_pipeline_segments(l_dims)
    long_bytes = prefill_algorithmic_bytes(LT, LH, D)
    del long_in, l_ws, l_out, l_fin

    # 64 packed sequences of 1,024..32,768 tokens (about 1M tokens), 32 heads,
    # each from its own initial state, final states for every sequence
    var_in = make_config_prefill(2, device=dev)
    VT, VH = var_in["q"].shape[0], var_in["q"].shape[1]
    VN = var_in["cu_seqlens"].numel() - 1
    v_dims = kda.make_dims(VT, VN, VH, D, D, 0)
    v_ws = torch.empty(kda.kda_prefill_workspace_bytes(v_dims), dtype=torch.uint8, device=dev)
    v_out = torch.empty((VT, VH, D), dtype=torch.bfloat16, device=dev)
    v_fin = torch.empty((VN, VH, D, D), dtype=torch.float32, device=dev)
    var_us = median_call_us(
        lambda: kda.kda_chunk_prefill(var_in["q"], var_in["k"], var_in["v"], var_in["g"],
                                      var_in["beta"], var_in["initial_state"],
                                      var_in["cu_seqlens"], v_out, v_fin, workspace=v_ws,
                                      stream=stream),
        2 if args.profile else 4)
    var_bytes = prefill_algorithmic_bytes(VT, VH, D, n_seqs=VN)
    del var_in, v_ws, v_out, v_fin

    # plain 1 GiB device-to-device copy: the practical HBM ceiling on this machine
    # (and, in --profile runs, the known-size transfer that scales the counters)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copy_ms = []
    for i in range(1 if args.profile else 4):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize(dev)
        copy_ms.append(c0.elapsed_time(c1))
    copy_GBps = 2 * (1 << 30) / (min(copy_ms[1:] or copy_ms) * 1e-3) / 1e9
    del src, dst

    # ------------------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import kda_oracle
        kda_oracle.build(force=False)
        host = lambda t: t.detach().float().cpu().numpy()
        hq, hk, hv, hg, hb = (host(base[x]) for x in ("q", "k", "v", "g", "beta"))
        hs0 = host(base["initial_state"])
        threads = kda_oracle.default_threads()
        reps, spent = 0, 0.0
        while spent < 10.0 and reps < 50:
            c0 = time.perf_counter()
            kda_oracle.prefill(hq, hk, hv, hg, hb, initial_state=hs0, threads=threads)
            spent += time.perf_counter() - c0
            reps += 1
        cpu_model = ""
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        cpu_model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        cpu = {"value": T * reps / spent, "unit": "tokens/s", "cores": threads,
               "kind": "oracle", "token_heads_per_s": T * H * reps / spent,
               "cpu_model": cpu_model,
               "sample": f"the full prefill workload (T=8192, all 32 heads, fp64 "
                         f"token-by-token recurrence) run {reps} times, {spent:.1f} s, "
                         f"one (sequence, head) chain per thread"}

    cfg = CONFIGS[1]
    res = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k unit-norm N(0,1), v N(0,1), beta sigmoid(N(0,1)), "
                "g -softplus(N(0,1))*0.5, S0 N(0,0.02^2))",
        "config": {"workload": cfg.name, "seq_len": T, "num_seqs": 1, "heads": H,
                   "d_k": D, "d_v": D, "chunk": 64, "io": "bf16", "state": "fp32"},
        "roofline": {
            "kernel": "kda_chunk_prefill call (chunk_index + prep + recur kernels)",
            "bound": "hbm",
            "achieved": p_achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": p_achieved / HBM_PEAK_GBPS,
            "traffic": p_traffic,
            "algorithmic_bytes_per_call": p_bytes,
            "avg_call_us": call_avg_s * 1e6,
            "median_call_us": float(np.median(call_ms)) * 1e3,
            "min_call_us": float(np.min(call_ms)) * 1e3,
            "practical_hbm_GBps": copy_GBps,
            "frac_of_practical": p_achieved / copy_GBps,
            "mfma_view_tflops": prefill_executed_flops(T, H, D) / call_avg_s / 1e12,
            "mfma_view_frac": prefill_executed_flops(T, H, D) / call_avg_s / 1e12 / BF16_PEAK_TFLOPS,
        },
        "cpu_baseline": cpu,
        "prefill_checkpoints": ckpt,
        "prefill_scalar_gate": {"g": "[T, H] (one decay per token and head)",
                                "median_call_us": sg_us, "tokens_per_s": T / (sg_us * 1e-6),
                                "algorithmic_bytes_per_call": p_bytes - 2 * (D - 1) * T * H},
        "prefill_output_gate": {"z": "[T, H, d_v] (one gate per value channel)",
                                "median_call_us": og_us, "tokens_per_s": T / (og_us * 1e-6),
                                "overhead_vs_plain_median":
                                    og_us / (float(np.median(call_ms)) * 1e3) - 1.0,
                                "algorithmic_bytes_per_call": p_bytes + T * H * D * 2},
        "prefill_varlen": {
            "workload": f"{VN} packed sequences, {VT} tokens, H={VH} d={D} bf16 (varlen prefill)",
            "median_call_ms": var_us / 1e3,
            "tokens_per_s": VT / (var_us * 1e-6),
            "algorithmic_bytes_per_call": var_bytes,
            "achieved_GBps": var_bytes / (var_us * 1e-6) / 1e9,
        },
        "prefill_long": {
            "workload": f"one sequence T={LT} H={LH} d={D} bf16 (million-token prefill)",
            "pipeline_segments": long_segs,
            "median_call_ms": long_us / 1e3,
            "tokens_per_s": LT / (long_us * 1e-6),
            "algorithmic_bytes_per_call": long_bytes,
            "achieved_GBps": long_bytes / (long_us * 1e-6) / 1e9,
        },
        "prefill_front_end": {"front_end": "raw q, k, v through a width-4 causal "
                                            "convolution + SiLU; g = -softplus(a b^T + bias), "
                                            "rank 64 (no g read)",
                              "median_call_us": fe_us, "tokens_per_s": T / (fe_us * 1e-6),
                              "overhead_vs_plain_median":
                                  fe_us / (float(np.median(call_ms)) * 1e3) - 1.0,
                              "algorithmic_bytes_per_call": fe_bytes},
        "decode": {
            "workload": CONFIGS[3].name.replace(", 100 steps", ""),
            "steps": args.decode_steps,
            "us_per_step": d_wall * 1e6 / args.decode_steps,
            "tokens_per_s": DECODE_N * args.decode_steps / d_wall,
            "state_GBps": sb / d_avg_s / 1e9,
            "roofline": {
                "kernel": "decode_kernel<bf16,128>",
                "bound": "hbm",
                "achieved": (sb + tb) / d_avg_s / 1e9,
                "peak": HBM_PEAK_GBPS,
                "unit": "GB/s",
                "frac": (sb + tb) / d_avg_s / 1e9 / HBM_PEAK_GBPS,
                "traffic": d_traffic,
                "algorithmic_bytes_per_call": sb + tb,
                "avg_call_us": d_avg_s * 1e6,
                "median_call_us": float(np.median(d_ms)) * 1e3,
                "total_ms": d_avg_s * 1e3 * args.decode_steps,
                "practical_hbm_GBps": copy_GBps,
                "frac_of_practical": (sb + tb) / d_avg_s / 1e9 / copy_GBps,
            },
            "front_end": {"median_call_us": fe_dec_us,
                          "note": "width-4 convolution state advanced in place, rank-64 gate"},
            "output_gate": {"z": "[N, H, d_v]", "median_call_us": og_dec_us,
                            "algorithmic_bytes_per_call": sb + tb + DECODE_N * DECODE_H * D * 2,
                            "achieved_GBps": (sb + tb + DECODE_N * DECODE_H * D * 2)
                            / (og_dec_us * 1e-6) / 1e9},
        },
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
