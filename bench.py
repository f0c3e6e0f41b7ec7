"""Benchmark: KDA chunked-prefill tokens/s and decode-step state GB/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--profile]

One step = one kda_chunk_prefill call over the packed varlen batch: 64
sequences with lengths drawn uniformly in [1024, 32768] (1,007,721 tokens with
its seed), H=32, d_k=d_v=128, bf16 I/O, fp32 per-sequence initial and final
states; seeded synthetic inputs resident in HBM (33 GB of q, k, v, g per call,
far past the 256 MB MALL).  Its 2,048 (sequence, head) chains take the fused
kernel (chain order + one persistent kernel); the single-sequence workloads
below take the segmented path (two passes of the same kernel around a scan of
the segments' state maps).  This is the largest single-GPU workload.  Untimed calls run first until --ramp-ms of GPU
time has passed (the shader clock rises over the first ~25 ms of load), then
W warm-up steps, then K back-to-back steps timed between device
synchronisations, with two HIP events on the launch stream around them giving
the average call duration behind the roofline figure; a separate loop with
events around each call gives the per-call spread.

Secondary figures in the same run, each with its own roofline object:
* the 8,192-token single-sequence prefill (H=32; 8 chains per head in each
  segmented pass), four input copies rotated so a call never finds its inputs
  in the MALL, plus its checkpoint, per-head gate, output-gate and front-end
  variants (these take the preparation and recurrence kernels);
* the 2^20-token single-sequence prefill (H=16; 16 chains per head in each
  segmented pass, 17 segments);
* the decode step on 256 sequences x 32 heads (512 MiB fp32 state advanced in
  place), plus its output-gate and front-end variants.

CPU baseline: the fp64 oracle timed on the host's cores on bounded samples of
the same workloads (the varlen batch on 2 seeded heads of all 64 sequences;
the first 131,072 tokens of 2 seeded heads of the million-token sequence),
with labelled extrapolations to the whole workloads.

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
DECODE_N, DECODE_H = 256, 32


def prefill_algorithmic_bytes(T, H, d, n_seqs=1):
    """q, k, v, g (4 x 2d B), beta (2 B) in, o (2d B) out per token-head, plus the
    fp32 state read and written once per (sequence, head)."""
    return (10 * d + 2) * T * H + 2 * 4 * d * d * n_seqs * H


def prefill_executed_flops(T, H, d, C=64):
    """MFMA work per token-head as executed by the preparation and recurrence
    kernels (full tiles): 6 d^2 + 10 C d + C^2 / 3."""
    return (6 * d * d + 10 * C * d + C * C / 3) * T * H


def fused_executed_flops(T, H, d, C=16):
    """bf16 MFMA work per token-head as executed by the fused kernel (16-token
    sub-chunks): X = Ke S and Qe S 4 d^2, the state update 2 d^2, T Diag(beta) Y
    and M u 2 C d each, the diagonal A, A^T, M^T 6 C d, the K'^T selector
    products 4 C d (the inverse's fp32 products, 16 C^2, are not counted)."""
    return (6 * d * d + 14 * C * d) * T * H


def segmented_executed_flops(T, H, d, P, C=16):
    """bf16 MFMA work of the segmented prefill of one T-token sequence with P
    chains per head: every token-head runs the fused kernel with its outputs
    (6 d^2 + 14 C d), and those of segments 1..P-1 are first run for their
    maps (Ke S, the state update and T Diag(beta) Y for the b and the M tiles,
    8 d^2 + 4 C d, and the A, A^T and selector products once, 8 C d).  The
    segments as the kernel places them: of n chunks, P of l = ceil(7 n /
    (7 P + 8)) after a first segment of n - P l; the scan's fp32 products are
    not counted."""
    n = (T + 63) // 64
    l = (7 * n + 7 * P + 7) // (7 * P + 8)
    a = max(0, n - P * l)
    mapped = max(0, min(n, a + (P - 1) * l) - a) * 64
    return (6 * d * d + 14 * C * d) * T * H + (8 * d * d + 12 * C * d) * min(mapped, T) * H


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


def roofline(kernel, alg_bytes, avg_s, traffic, copy_GBps, flops=None, **extra):
    """The HBM roofline object of one workload: algorithmic bytes per call over
    the event-timed average call duration."""
    achieved = alg_bytes / avg_s / 1e9
    r = {"kernel": kernel, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
         "algorithmic_bytes_per_call": alg_bytes, "avg_call_us": avg_s * 1e6,
         "practical_hbm_GBps": copy_GBps, "frac_of_practical": achieved / copy_GBps}
    if flops is not None:
        r["mfma_view_tflops"] = flops / avg_s / 1e12
        r["mfma_view_frac"] = flops / avg_s / 1e12 / BF16_PEAK_TFLOPS
    r.update(extra)
    return r


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--ramp-ms", type=float, default=80.0,
                    help="untimed calls before the warm-up steps until this much GPU time has "
                         "passed (the shader clock rises over the first ~25 ms of load)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="short run for profilers: the clock ramp, few steps, no CPU baseline, "
                         "one 1 GiB device copy as a traffic calibration")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(heads and sequences shard across GPUs with no exchange, so one GPU's "
              "throughput is the per-GPU figure)", file=sys.stderr)
        sys.exit(2)
    if args.profile:
        args.steps, args.warmup, args.decode_steps = 3, 1, 10
        args.no_cpu_baseline = True

    import numpy as np
    import torch

    import linear_attention_recurrence_06_amd as kda
    from kda_inputs import (CONFIGS, make_config_decode, make_config_prefill, make_front_end,
                            make_out_gate, make_prefill, seeded_heads)

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    kda.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def ramp(fn):
        """Untimed calls until ramp_ms of GPU time has passed."""
        spent = 0.0
        while spent < args.ramp_ms:
            a, b = ev(), ev()
            a.record(stream)
            for _ in range(4):
                fn()
            b.record(stream)
            torch.cuda.synchronize(dev)
            spent += a.elapsed_time(b)

    def timed(fn, steps, warmup):
        """K back-to-back calls between synchronisations, two events around
        them; then the per-call spread from events around each call.  Returns
        (wall seconds per step, event average seconds per call, per-call ms)."""
        for i in range(warmup):
            fn(i)
        e0, e1 = ev(), ev()
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        wall = (time.perf_counter() - t0) / steps
        avg = e0.elapsed_time(e1) * 1e-3 / steps
        evs = [(ev(), ev()) for _ in range(steps)]
        for i in range(steps):
            evs[i][0].record(stream)
            fn(i)
            evs[i][1].record(stream)
        torch.cuda.synchronize(dev)
        return wall, avg, [a.elapsed_time(b) for a, b in evs]

    def median_call_us(fn, reps):
        for _ in range(2):
            fn()
        evs = [(ev(), ev()) for _ in range(reps)]
        for a_, b_ in evs:
            a_.record(stream)
            fn()
            b_.record(stream)
        torch.cuda.synchronize(dev)
        return float(np.median([a_.elapsed_time(b_) for a_, b_ in evs])) * 1e3

    host = lambda t: t.detach().float().cpu().numpy()
    secondary_steps = max(3, args.steps // 2)

    # ------------------------------------------------------------ headline: varlen
    var_in = make_config_prefill(2, device=dev)
    VT, VH = var_in["q"].shape[0], var_in["q"].shape[1]
    VN = var_in["cu_seqlens"].numel() - 1
    v_dims = kda.make_dims(VT, VN, VH, D, D, 0)
    # the workspace the call's path uses (the fused kernel: its index areas)
    v_ws = torch.empty(kda.kda_prefill_path_workspace_bytes(v_dims, True), dtype=torch.uint8,
                       device=dev)
    v_out = torch.empty((VT, VH, D), dtype=torch.bfloat16, device=dev)
    v_fin = torch.empty((VN, VH, D, D), dtype=torch.float32, device=dev)

    def varlen(_i=0):
        kda.kda_chunk_prefill(var_in["q"], var_in["k"], var_in["v"], var_in["g"],
                              var_in["beta"], var_in["initial_state"], var_in["cu_seqlens"],
                              v_out, v_fin, workspace=v_ws, stream=stream)

    ramp(varlen)
    v_wall, v_avg, v_ms = timed(varlen, args.steps, args.warmup)
    v_bytes = prefill_algorithmic_bytes(VT, VH, D, n_seqs=VN)
    v_lens = var_in["lens"]
    # oracle inputs: 2 seeded heads of every sequence (copied before freeing)
    v_heads = seeded_heads(VH, 2, 102)
    v_host = None
    if not args.no_cpu_baseline:
        v_host = {x: host(var_in[x][:, v_heads].contiguous()) for x in ("q", "k", "v", "g", "beta")}
        v_host["s0"] = host(var_in["initial_state"][:, v_heads].contiguous())
        v_host["cu"] = var_in["cu_seqlens"].cpu().numpy()
    del var_in, v_ws, v_out, v_fin
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ single sequence, T=8192
    base = make_config_prefill(1, device=dev)
    T, H = base["q"].shape[0], base["q"].shape[1]
    sets = [base] + [{k: (v.clone() if torch.is_tensor(v) else v) for k, v in base.items()}
                     for _ in range(3)]
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    dims = kda.make_dims(T, 1, H, D, D, 0)
    # (the full workspace: the option variants below take the two-kernel path)
    ws = torch.empty(kda.kda_prefill_workspace_bytes(dims), dtype=torch.uint8, device=dev)
    single_path, single_segs = kda.kda_prefill_path(dims)

    def single(i=0):
        s = sets[i % len(sets)]
        kda.kda_chunk_prefill(s["q"], s["k"], s["v"], s["g"], s["beta"], s["initial_state"],
                              None, out, fin, workspace=ws, stream=stream)

    ramp(lambda: single(0))
    s_wall, s_avg, s_ms = timed(single, max(args.steps, 20), args.warmup)
    s_bytes = prefill_algorithmic_bytes(T, H, D)
    s_med_us = float(np.median(s_ms)) * 1e3
    # the option variants below take the two-kernel path: their overheads are
    # against the plain call on that path
    saved_path = os.environ.get("KDA_PREFILL_PATH")
    os.environ["KDA_PREFILL_PATH"] = "split"
    try:
        split_med_us = median_call_us(lambda: single(0), secondary_steps)
    finally:
        if saved_path is None:
            del os.environ["KDA_PREFILL_PATH"]
        else:
            os.environ["KDA_PREFILL_PATH"] = saved_path

    # checkpointed prefill (intermediate states every `interval` chunks)
    ckpt = {}
    for interval in (16, 1):
        n_ck = kda.kda_checkpoint_count(dims, None, interval)
        ck_buf = torch.empty((n_ck, H, D, D), dtype=torch.float32, device=dev)
        it = iter(range(1 << 30))

        def ck_call():
            s_ = sets[next(it) % len(sets)]
            kda.kda_chunk_prefill_checkpoints(
                s_["q"], s_["k"], s_["v"], s_["g"], s_["beta"], s_["initial_state"], None, out,
                fin, checkpoint_interval=interval, checkpoints=ck_buf, workspace=ws,
                stream=stream)
        ck_us = median_call_us(ck_call, secondary_steps)
        ckpt[f"every_{interval}_chunks"] = {
            "checkpoints": n_ck, "bytes_written": n_ck * H * D * D * 4,
            "median_call_us": ck_us, "overhead_vs_plain_two_kernel_median": ck_us / split_med_us - 1.0}
        del ck_buf

    # per-head (scalar) gate: g [T, H], same workload otherwise
    sg_in = make_prefill([T], H, D, "bf16", g_scale=0.5, s0_std=0.02, seed=1, device=dev,
                         scalar_gate=True)
    sg_us = median_call_us(
        lambda: kda.kda_chunk_prefill(sg_in["q"], sg_in["k"], sg_in["v"], sg_in["g"],
                                      sg_in["beta"], sg_in["initial_state"], None, out, fin,
                                      workspace=ws, stream=stream), secondary_steps)
    del sg_in

    # output gate fused into the output write: out = o * sigmoid(z), z [T, H, d_v]
    z_pf = make_out_gate((T, H, D), "bf16", seed=2, device=dev)
    og_us = median_call_us(
        lambda: kda.kda_chunk_prefill_ex(base["q"], base["k"], base["v"], base["g"],
                                         base["beta"], base["initial_state"], None, out, fin,
                                         out_gate_z=z_pf, workspace=ws, stream=stream),
        secondary_steps)
    del z_pf

    # front end: raw q, k, v through a width-4 convolution with SiLU, g from a
    # rank-64 projection (g not read)
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
        secondary_steps)
    fe_bytes = s_bytes - 2 * D * T * H + 2 * 64 * T + 2 * H * D * 64
    del fe_in, fe_state_out
    s_host = None
    if not args.no_cpu_baseline:
        s_host = {x: host(base[x]) for x in ("q", "k", "v", "g", "beta")}
        s_host["s0"] = host(base["initial_state"])
    del sets, base, out, fin, ws
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ decode
    dw = make_config_decode(3, device=dev, steps=args.decode_steps)
    state = dw["state"]
    dout = torch.empty((DECODE_N, DECODE_H, D), dtype=torch.bfloat16, device=dev)

    def decode(s):
        kda.kda_decode_step(dw["q"][s], dw["k"][s], dw["v"][s], dw["g"][s], dw["beta"][s],
                            state, dout, stream=stream)

    for s in range(min(3, args.decode_steps)):
        decode(s)
    torch.cuda.synchronize(dev)
    d0, d1 = ev(), ev()
    t1 = time.perf_counter()
    d0.record(stream)
    for s in range(args.decode_steps):
        decode(s)
    d1.record(stream)
    torch.cuda.synchronize(dev)
    d_wall = time.perf_counter() - t1
    d_avg_s = d0.elapsed_time(d1) * 1e-3 / args.decode_steps
    n_spread = min(20, args.decode_steps)
    dev_ev = [(ev(), ev()) for _ in range(n_spread)]
    for s in range(n_spread):
        dev_ev[s][0].record(stream)
        decode(s)
        dev_ev[s][1].record(stream)
    torch.cuda.synchronize(dev)
    d_ms = [a.elapsed_time(b) for a, b in dev_ev]
    sb = decode_state_bytes(DECODE_N, DECODE_H, D)
    tb = decode_token_bytes(DECODE_N, DECODE_H, D)

    z_dec = make_out_gate((DECODE_N, DECODE_H, D), "bf16", seed=3, device=dev)
    og_dec_us = median_call_us(
        lambda: kda.kda_decode_step_ex(dw["q"][0], dw["k"][0], dw["v"][0], dw["g"][0],
                                       dw["beta"][0], state, dout, out_gate_z=z_dec,
                                       stream=stream),
        max(10, args.decode_steps // 4))
    del z_dec
    fe_dec = make_front_end(DECODE_N, DECODE_N, DECODE_H, D, "bf16", width=4, rank=64,
                            bias_std=0.3, seed=5, device=dev)
    fe_dec_us = median_call_us(
        lambda: kda.kda_decode_step_ex(dw["q"][0], dw["k"][0], dw["v"][0], None, dw["beta"][0],
                                       state, dout, conv_weight=fe_dec["conv_weight"],
                                       conv_silu=True, conv_state=fe_dec["conv_state"],
                                       gate_a=fe_dec["gate_a"], gate_b=fe_dec["gate_b"],
                                       gate_bias=fe_dec["gate_bias"], stream=stream),
        max(10, args.decode_steps // 4))
    del fe_dec, dw, state, dout
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ one sequence, T=2^20
    long_in = make_config_prefill(4, device=dev)
    LT, LH = long_in["q"].shape[0], long_in["q"].shape[1]
    l_dims = kda.make_dims(LT, 1, LH, D, D, 0)
    # (segmented: the index areas and the segments' state maps)
    l_ws = torch.empty(kda.kda_prefill_path_workspace_bytes(l_dims), dtype=torch.uint8,
                       device=dev)
    l_out = torch.empty((LT, LH, D), dtype=torch.bfloat16, device=dev)
    l_fin = torch.empty((1, LH, D, D), dtype=torch.float32, device=dev)

    def long_call(_i=0):
        kda.kda_chunk_prefill(long_in["q"], long_in["k"], long_in["v"], long_in["g"],
                              long_in["beta"], long_in["initial_state"], None, l_out, l_fin,
                              workspace=l_ws, stream=stream)

    l_wall, l_avg, l_ms = timed(long_call, 2 if args.profile else 4, 1)
    long_path, long_segs = kda.kda_prefill_path(l_dims)
    l_bytes = prefill_algorithmic_bytes(LT, LH, D)
    l_heads = seeded_heads(LH, 2, 104)
    L_SAMPLE = 131072
    l_host = None
    if not args.no_cpu_baseline:
        l_host = {x: host(long_in[x][:L_SAMPLE, l_heads].contiguous())
                  for x in ("q", "k", "v", "g", "beta")}
        l_host["s0"] = host(long_in["initial_state"][:, l_heads].contiguous())
    del long_in, l_ws, l_out, l_fin
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ practical HBM ceiling
    # plain 1 GiB device-to-device copy (and, in --profile runs, the known-size
    # transfer that scales the counters)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copy_ms = []
    for i in range(1 if args.profile else 4):
        c0, c1 = ev(), ev()
        c0.record(stream)
        dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize(dev)
        copy_ms.append(c0.elapsed_time(c1))
    copy_GBps = 2 * (1 << 30) / (min(copy_ms[1:] or copy_ms) * 1e-3) / 1e9
    del src, dst

    # ------------------------------------------------------------ CPU baseline (oracle)
    cpu = cpu_single = cpu_long = None
    if not args.no_cpu_baseline:
        from oracle import kda_oracle
        kda_oracle.build(force=False)
        threads = kda_oracle.default_threads()
        model = cpu_model()

        def run_oracle(h, n_seqs, cu, min_s, max_reps):
            reps, spent = 0, 0.0
            while spent < min_s and reps < max_reps:
                c0 = time.perf_counter()
                kda_oracle.prefill(h["q"], h["k"], h["v"], h["g"], h["beta"], cu_seqlens=cu,
                                   initial_state=h["s0"], n_seqs=n_seqs, threads=threads)
                spent += time.perf_counter() - c0
                reps += 1
            return reps, spent

        # varlen: 2 seeded heads of all 64 sequences (128 chains over the threads)
        reps, spent = run_oracle(v_host, VN, v_host["cu"], 8.0, 10)
        th_s = VT * len(v_heads) * reps / spent
        cpu = {"value": th_s / VH, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "token_heads_per_s": th_s, "cpu_model": model,
               "sample": f"the varlen workload on {len(v_heads)} seeded heads (of {VH}) of all "
                         f"{VN} sequences ({VT * len(v_heads):,} token-heads, fp64 token-by-token "
                         f"recurrence, one (sequence, head) chain per thread), run {reps} times "
                         f"in {spent:.1f} s; value = token-heads/s / {VH} heads, i.e. the "
                         f"whole-workload tokens/s these cores would reach (an extrapolation "
                         f"over heads: chains are independent)",
               "extrapolated_whole_workload_s": VT * VH / th_s}
        # single sequence: all 32 heads (32 chains)
        reps, spent = run_oracle(s_host, 1, None, 4.0, 20)
        th_s1 = T * H * reps / spent
        cpu_single = {"value": th_s1 / H, "unit": "tokens/s", "cores": threads,
                      "kind": "oracle", "token_heads_per_s": th_s1,
                      "sample": f"the whole T={T} workload (all {H} heads) run {reps} times, "
                                f"{spent:.1f} s"}
        # one long sequence: the first 131,072 tokens of 2 seeded heads (2 chains,
        # so 2 threads work)
        reps, spent = run_oracle(l_host, 1, None, 2.0, 5)
        th_l = L_SAMPLE * len(l_heads) * reps / spent
        per_core = th_l / len(l_heads)
        cpu_long = {"value": per_core * threads / LH, "unit": "tokens/s",
                    "cores": len(l_heads), "kind": "oracle",
                    "token_heads_per_s": th_l, "token_heads_per_s_per_core": per_core,
                    "sample": f"the first {L_SAMPLE:,} tokens of {len(l_heads)} seeded heads "
                              f"(2 chains on 2 threads), run {reps} times in {spent:.1f} s; "
                              f"value = per-core rate x {threads} cores / {LH} heads "
                              f"(extrapolated: a single sequence has only {LH} chains)",
                    "extrapolated_whole_workload_s": LT * LH / per_core / min(threads, LH)}

    p_traffic = counter_traffic("prefill_varlen")
    res = {
        "metric": METRIC,
        "value": VT / v_wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": v_wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k unit-norm N(0,1), v N(0,1), beta sigmoid(N(0,1)), "
                "g -softplus(N(0,1))*0.5, S0 N(0,0.02^2) per sequence)",
        "config": {"workload": f"varlen prefill: {VN} packed sequences U[1024,32768] "
                               f"({VT:,} tokens), H={VH}, d_k=d_v={D}, bf16 I/O, fp32 state",
                   "num_seqs": VN, "total_tokens": VT, "min_len": min(v_lens),
                   "max_len": max(v_lens), "heads": VH, "d_k": D, "d_v": D, "chunk": 64,
                   "io": "bf16", "state": "fp32"},
        "roofline": roofline("kda_chunk_prefill call (chain_order_kernel + fused_ws_kernel<128>)",
                             v_bytes, v_avg, p_traffic, copy_GBps,
                             flops=fused_executed_flops(VT, VH, D),
                             median_call_ms=float(np.median(v_ms)),
                             min_call_ms=float(np.min(v_ms))),
        "cpu_baseline": cpu,
        "prefill_single": {
            "workload": CONFIGS[1].name,
            "path": {0: "split", 1: "pipelined", 2: "fused", 3: "segmented"}.get(single_path, "?"),
            "segments": single_segs,
            "tokens_per_s": T / s_wall,
            "ms_per_step": s_wall * 1e3,
            "roofline": roofline("kda_chunk_prefill call", s_bytes, s_avg,
                                 counter_traffic("prefill_single"), copy_GBps,
                                 flops=(segmented_executed_flops(T, H, D, single_segs)
                                        if single_path == 3 else prefill_executed_flops(T, H, D)),
                                 median_call_us=s_med_us,
                                 min_call_us=float(np.min(s_ms)) * 1e3),
            "cpu_baseline": cpu_single,
            "plain_two_kernel_median_call_us": split_med_us,
            "checkpoints": ckpt,
            "scalar_gate": {"g": "[T, H] (one decay per token and head)",
                            "median_call_us": sg_us, "tokens_per_s": T / (sg_us * 1e-6),
                            "algorithmic_bytes_per_call": s_bytes - 2 * (D - 1) * T * H},
            "output_gate": {"z": "[T, H, d_v] (one gate per value channel)",
                            "median_call_us": og_us, "tokens_per_s": T / (og_us * 1e-6),
                            "overhead_vs_plain_two_kernel_median": og_us / split_med_us - 1.0,
                            "algorithmic_bytes_per_call": s_bytes + T * H * D * 2},
            "front_end": {"front_end": "raw q, k, v through a width-4 causal convolution + "
                                       "SiLU; g = -softplus(a b^T + bias), rank 64 (no g read)",
                          "median_call_us": fe_us, "tokens_per_s": T / (fe_us * 1e-6),
                          "overhead_vs_plain_two_kernel_median": fe_us / split_med_us - 1.0,
                          "algorithmic_bytes_per_call": fe_bytes},
        },
        "prefill_long": {
            "workload": CONFIGS[4].name,
            "path": {0: "split", 1: "pipelined", 2: "fused", 3: "segmented"}.get(long_path, "?"),
            "segments": long_segs,
            "tokens_per_s": LT / l_avg,
            "roofline": roofline("kda_chunk_prefill call", l_bytes, l_avg,
                                 counter_traffic("prefill_long"), copy_GBps,
                                 flops=(segmented_executed_flops(LT, LH, D, long_segs) if long_path == 3
                                        else prefill_executed_flops(LT, LH, D)),
                                 median_call_ms=float(np.median(l_ms))),
            "cpu_baseline": cpu_long,
        },
        "decode": {
            "workload": CONFIGS[3].name.replace(", 100 steps", ""),
            "steps": args.decode_steps,
            "us_per_step": d_wall * 1e6 / args.decode_steps,
            "tokens_per_s": DECODE_N * args.decode_steps / d_wall,
            "state_GBps": sb / d_avg_s / 1e9,
            "roofline": roofline("decode_kernel<bf16,128>", sb + tb, d_avg_s,
                                 counter_traffic("decode"), copy_GBps,
                                 median_call_us=float(np.median(d_ms)) * 1e3,
                                 total_ms=d_avg_s * 1e3 * args.decode_steps),
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
