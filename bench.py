#!/usr/bin/env python3
"""Chunked KDA forward benchmark on one MI355X.

One step = one full forward (kda_fwd: intra-chunk kernel + state-chain
kernel) over the safe-gate workload B=2, T=8192, H=32, K=V=128 (lower_bound
-5, fp32 initial and final state), inputs resident in HBM.  Prints one JSON
line: tokens/s with the median / min / max step, the sustained rate of the
steps that run on after the timed ones (the clocks ramp up over the first
tens of milliseconds of load), the dominant kernel's
roofline from HIP events recorded around each stage on the launch stream
(algorithmic bytes: the kernel's own share of the method's minimum HBM bytes
per token-head), the path's fraction of the HBM and bf16 MFMA peaks, counter
figures from the committed rocprofv3 summaries when they match the current
source, and the fp64 CPU oracle timed on this host's cores.
"""
import argparse
import hashlib
import json
import os
import re
import glob
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunk_kda fwd tokens/s (H=32,K=V=128,T=8192) + % bf16 MFMA peak, 1 MI355X"
HBM_PEAK_GBPS = 8000.0
# MI355X published fp32 vector peak: 256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2 (packed fp32) x 2.4 GHz.
FP32_VALU_PEAK_TFLOPS = 157.3
BF16_PEAK_TFLOPS = 2516.6
# Method work per token-head (dense 64-token tiles): 5 x 2*64*128 for Akk, Aqk,
# w, u, Aqk.U plus 3 x 2*128*128 for W.S, Q.S, K^T.U.
FLOP_PER_TOKEN_HEAD = 5 * 2 * 64 * 128 + 3 * 2 * 128 * 128
BLOCK_BYTES = 76800  # per (v-head, chunk) intermediates written by the intra kernel


def kernel_source_hash(name="kda_fwd.hip"):
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "gated_delta_rule_act_amd", "csrc", name), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def profile_figure(name, kernel, workload_name, key):
    """A figure from a committed rocprofv3 summary (profiles/<name>_<kernel>_<workload>.md),
    if that summary was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{name}_{kernel}_{workload_name}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"source_sha:\s*([0-9a-f]+)", txt)
    m_b = re.search(key + r":\s*([0-9.eE+-]+)", txt)
    if not m_src or not m_b or m_src.group(1) != kernel_source_hash():
        return None
    return float(m_b.group(1))


def profiled_bwd_traffic(workload_name):
    """Counted HBM bytes of one backward call (every kernel's FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy's readings) from the committed backward
    counter summary, if taken on the current backward source; else None."""
    path = os.path.join(ROOT, "profiles", f"counters_backward_{workload_name}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"bwd_source_sha:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_call:\s*([0-9.eE+-]+)", txt)
    if not m_src or not m_b or m_src.group(1) != kernel_source_hash("kda_bwd.hip"):
        return None
    return float(m_b.group(1))


def profiled_traffic(kernel, workload_name):
    """Counted HBM bytes per launch (FETCH_SIZE and WRITE_SIZE passes scaled by a
    plain copy's readings) from the committed summary; None if stale or absent."""
    return profile_figure("traffic", kernel, workload_name, "hbm_bytes_per_launch")


def kernel_names(inp, nseg):
    """The kernels a chunked forward of this workload runs: the intra kernel, and
    the state pass's kernel as the library picks it (32-column slices on the
    split chain/helper kernel when a 64-column launch would not take fewer
    rounds of 256 workgroups weighted by its 1.85 x step time, else 64-column
    slices on the 4-wave kernel)."""
    jobs = inp.N * inp.Hv * nseg
    narrow_rounds = (jobs * 4 + 255) // 256
    wide_rounds = (jobs * 2 + 255) // 256
    narrow = wide_rounds * 185 >= narrow_rounds * 100
    return {"intra": "kda_intra_kernel", "state": "kda_state_split_kernel" if narrow else "kda_state_kernel"}


def bytes_model(inp):
    """Algorithmic HBM bytes: the method's minimum per token-head (q, k per qk-head
    and v, g, out at 256 B each, beta 2 B; states once per (sequence, v-head)),
    split into each kernel's own share -- the intra kernel reads q, k, g and
    beta (770 B per token-head with one qk-head per v-head), the state kernel
    reads v and the initial state and writes out and the final state (512 B
    per token-head plus the states).  The per-chunk workspace the intra kernel
    writes and the state kernel reads is an overhead of the two-kernel
    dataflow, reported beside these, never inside them."""
    B, T, Hqk, Hv, K, V = inp.B, inp.T, inp.Hqk, inp.Hv, inp.K, inp.V
    nchunks = B * ((T + 63) // 64) if inp.cu_seqlens is None else sum(
        (int(inp.cu_seqlens[n + 1] - inp.cu_seqlens[n]) + 63) // 64 for n in range(inp.N))
    tok = B * T
    st = {0: 0, 1: 4, 2: 2}
    h0 = inp.N * Hv * V * K * st[inp.init_state_dtype]
    hT = inp.N * Hv * V * K * st[inp.final_state_dtype]
    intra = tok * Hqk * K * 2 * 2 + tok * Hv * K * 2 + tok * Hv * 2
    state = tok * Hv * V * 2 + tok * Hv * V * 2 + h0 + hT
    return {"intra": intra, "state": state, "path": intra + state, "workspace": nchunks * Hv * BLOCK_BYTES,
            "token_heads": tok * Hv}


def host_info():
    """CPU model and thread count of this host, and the GPU clock levels as the
    driver's sysfs files list them (the current level is marked with *).  Read
    from files: no program is started once the GPU is in use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    clocks = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        for clk in ("sclk", "mclk", "fclk"):
            try:
                with open(os.path.join(dev, f"pp_dpm_{clk}")) as f:
                    cur = [l.strip() for l in f if "*" in l]
                if cur:
                    clocks[f"{os.path.basename(os.path.dirname(dev))}.{clk}"] = cur[0]
            except OSError:
                pass
    return {"cpu_model": model, "cpu_threads": os.cpu_count(), "gpu_clocks": clocks or None}


def cpu_baseline(inp, out_gpu, state_gpu, budget_s=30.0):
    """Time the fp64 oracle on this host (all cores) on the same inputs; also
    report the GPU result's parity against it."""
    import numpy as np
    import oracle
    from tests import gpu_util as U

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    build = oracle.native_build_description()
    # calibrate on one head to keep the run bounded (10-30 s of CPU work)
    t0 = time.perf_counter()
    U.oracle_pair(inp, 0, 0, inp.initial_state_f64())
    one = time.perf_counter() - t0
    est_full = one * inp.N * inp.Hv / max(1, threads)
    heads = inp.Hv
    if est_full > budget_s:
        heads = max(threads, int(inp.Hv * budget_s / est_full) // threads * threads)
        heads = min(heads, inp.Hv)
    sub = inp
    if heads < inp.Hv:
        G = inp.Hv // inp.Hqk
        hq = max(1, heads // G)
        heads = hq * G
        import dataclasses
        sub = dataclasses.replace(inp, q=np.ascontiguousarray(inp.q[:, :, :hq]), k=np.ascontiguousarray(inp.k[:, :, :hq]),
                                  v=np.ascontiguousarray(inp.v[:, :, :heads]), g=np.ascontiguousarray(inp.g[:, :, :heads]),
                                  beta=np.ascontiguousarray(inp.beta[:, :, :heads]),
                                  A_log=None if inp.A_log is None else inp.A_log[:heads],
                                  dt_bias=None if inp.dt_bias is None else inp.dt_bias[:heads],
                                  initial_state=None if inp.initial_state is None else
                                  np.ascontiguousarray(inp.initial_state[:, :heads]))
    t0 = time.perf_counter()
    o_ref, s_ref = U.run_oracle(sub, nthreads=threads)
    dt = time.perf_counter() - t0
    tokens_per_s = inp.B * inp.T * (heads / inp.Hv) / dt
    og = U.as_f64(out_gpu[:, :, :heads])
    e = U.errors(og, o_ref, U.as_f64(state_gpu[:, :heads]), s_ref)
    cpu = {"value": tokens_per_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{inp.name}: all {inp.B * inp.T} tokens of {heads} of {inp.Hv} v-heads "
                     f"(fp64 token recurrence, {dt:.1f} s; tokens/s scaled to all heads)",
           "seconds": dt, "build": build}
    parity = {"out_max_abs": e["out_max_abs"], "out_rel_rms": e["out_rel_rms"], "state_rel": e["state_rel"],
              "heads_checked": heads, "tol_out_max_abs": U.OUT_MAX_ABS, "tol_state_rel": U.STATE_REL}
    return cpu, parity


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--sustain-steps", type=int, default=200,
                    help="untimed-for-value steps after the timed region, for the sustained rate")
    ap.add_argument("--workload", type=int, default=None,
                    help="workload index (chunked: 1-5, the bench line is 3; recurrent: 1-2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--segments", type=int, default=0,
                    help="time segments per state chain (0: the library decides, 1: none)")
    ap.add_argument("--mode", choices=("chunked", "recurrent", "backward"), default="chunked",
                    help="chunked: the headline forward; recurrent: the token-recurrent entry on a decode workload")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="instead of the forward, run N plain 1 GiB device copies (traffic counter scale)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: the path runs on exactly one GPU (asked for {args.gpus}); "
              "sharding across GPUs is not built", file=sys.stderr)
        sys.exit(2)

    if not args.no_cpu_baseline and not args.copy_calibration:
        # the oracle for the CPU baseline, compiled for this host's CPU before
        # anything touches the GPU (no program is started after that)
        import oracle
        oracle.use_native_build()

    import torch
    from gated_delta_rule_act_amd import kda, workloads as W
    from tests import gpu_util as U

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.copy_calibration):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_copy": {"read": 1 << 30, "write": 1 << 30},
                          "copies": args.copy_calibration}))
        return

    if args.mode == "recurrent":
        return run_recurrent(args, dev)
    if args.mode == "backward":
        return run_backward(args, dev)

    t_gen = time.perf_counter()
    inp = W.workload(3 if args.workload is None else args.workload)
    d = U.to_device(inp)
    fdt = U.final_dtype_of(inp)
    out = torch.empty((inp.B, inp.T, inp.Hv, inp.V), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((inp.N, inp.Hv, inp.V, inp.K), dtype=fdt, device=dev)
    p = kda.make_params(B=inp.B, T=inp.T, H_qk=inp.Hqk, H_v=inp.Hv, num_seqs=inp.N, scale=inp.scale,
                        lower_bound=inp.lower_bound, gate_mode=inp.gate_mode,
                        init_state_dtype=inp.init_state_dtype, final_state_dtype=inp.final_state_dtype,
                        segments=args.segments)
    ws = torch.empty(kda.workspace_size(p), dtype=torch.uint8, device=dev)
    nseg = kda.segments_of(p, packed=inp.cu_seqlens is not None)
    print(f"[bench] workload {inp.name} ready in {time.perf_counter() - t_gen:.1f} s; "
          f"workspace {ws.numel() / 2**30:.2f} GiB", file=sys.stderr, flush=True)

    def step(stage=None):
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"], inp.scale, inp.lower_bound,
                inp.gate_mode, initial_state=d["h0"], cu_seqlens=d["cu_seqlens"], out=out, final_state=fs,
                final_state_dtype=fdt, workspace=ws, stage=stage, segments=args.segments)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` full forwards, an event after each
    evt = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evt[0].record()
    for i in range(args.steps):
        step()
        evt[i + 1].record()
    torch.cuda.synchronize()
    ms_per_step = evt[0].elapsed_time(evt[-1]) / args.steps
    step_ms = [evt[i].elapsed_time(evt[i + 1]) for i in range(args.steps)]

    # Sustained rate, after the timed region (not part of `value`): the GPU
    # raises its clocks over the first tens of milliseconds of load (workload 3:
    # about 595 us per step at first, 521 us after some 35 steps, and back to
    # the start after an idle of 0.1 s), so a short window right after a few
    # warm-up steps measures part of that ramp.  This loop runs on from the
    # timed one with no idle in between.
    sus = [torch.cuda.Event(enable_timing=True) for _ in range(args.sustain_steps + 1)]
    sus[0].record()
    for i in range(args.sustain_steps):
        step()
        sus[i + 1].record()
    torch.cuda.synchronize()
    sus_ms = [sus[i].elapsed_time(sus[i + 1]) for i in range(args.sustain_steps)]
    sus_tail = sus_ms[len(sus_ms) // 2:]  # the second half, past the ramp

    # per-kernel durations: events around each stage on the launch stream,
    # right after the sustained loop (so at the clocks of continuous load)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e in evs:
        e[0].record()
        step("intra")
        e[1].record()
        step("state")
        e[2].record()
    torch.cuda.synchronize()
    t_intra = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    t_state = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps

    tokens = inp.B * inp.T
    value = tokens / (ms_per_step * 1e-3)
    bm = bytes_model(inp)
    kern = {"intra": t_intra, "state": t_state}
    dom = max(kern, key=kern.get)
    names = kernel_names(inp, nseg)
    kname = names[dom]
    achieved = bm[dom] / (kern[dom] * 1e-3) / 1e9
    traffic = profiled_traffic(kname, inp.name)
    path_gbps = bm["path"] / (ms_per_step * 1e-3) / 1e9
    mfma_tflops = FLOP_PER_TOKEN_HEAD * tokens * inp.Hv / (ms_per_step * 1e-3) / 1e12
    counters = {}
    for k in ("intra", "state"):
        for fig in ("mfma_busy_pct", "valu_busy_pct", "wait_pct"):
            v = profile_figure("counters", names[k], inp.name, fig)
            if v is not None:
                counters[f"{names[k]}.{fig}"] = v

    rec = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded numpy PCG64 draws of the workload's shapes and distributions)",
        "config": {"workload": inp.name, "B": inp.B, "T": inp.T, "H_qk": inp.Hqk, "H_v": inp.Hv, "K": inp.K,
                   "V": inp.V, "gate": ["softplus", "safe_sigmoid", "pregated"][inp.gate_mode],
                   "lower_bound": inp.lower_bound, "chunk": 64, "sub_chunk": 16,
                   "initial_state": ["none", "fp32", "bf16"][inp.init_state_dtype],
                   "final_state": ["none", "fp32", "bf16"][inp.final_state_dtype],
                   "packed": inp.cu_seqlens is not None, "state_segments": nseg},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": bm[dom],
                     "algorithmic_bytes_per_token_head": bm[dom] / bm["token_heads"],
                     "convention": "the kernel's own share of the method minimum (intra: q, k, g, beta; "
                                   "state: v, out, states); the per-chunk workspace is overhead",
                     "workspace_bytes_per_launch": bm["workspace"],
                     "traffic_over_algorithmic": None if traffic is None else traffic / bm[dom],
                     "avg_launch_ms": kern[dom]},
        "kernels_ms": {names["intra"]: t_intra, names["state"]: t_state},
        "step_ms": {"mean": ms_per_step, "median": statistics.median(step_ms), "min": min(step_ms),
                    "max": max(step_ms)},
        "sustained": None if not sus_tail else {
            "steps": args.sustain_steps, "ms_per_step_median": statistics.median(sus_tail),
            "ms_per_step_mean": statistics.mean(sus_tail), "min": min(sus_tail), "max": max(sus_tail),
            "tokens_per_s": tokens / (statistics.median(sus_tail) * 1e-3),
            "note": "steps run on right after the timed region; figures over the second half of them"},
        "path": {"min_bytes_per_step": bm["path"], "min_bytes_per_token_head": bm["path"] / bm["token_heads"],
                 "achieved_GBps": path_gbps, "hbm_frac": path_gbps / HBM_PEAK_GBPS,
                 "mfma_algorithmic_TFLOPs": mfma_tflops,
                 "mfma_pct_bf16_peak": 100.0 * mfma_tflops / BF16_PEAK_TFLOPS,
                 "flop_per_token_head": FLOP_PER_TOKEN_HEAD,
                 "workspace_round_trip_bytes": 2 * bm["workspace"]},
        "counters_rocprof": counters or None,
        "conditions": {**host_info(),
                       "cache": "inputs resident in HBM and warm from the previous step; the working set "
                                "(inputs, outputs, workspace) is larger than the 256 MB Infinity Cache; "
                                "no flush between steps"},
        "kernel_source_sha": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu, parity = cpu_baseline(inp, out, fs)
        rec["cpu_baseline"] = cpu
        rec["parity"] = parity
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


def run_recurrent(args, dev):
    """The token-recurrent entry: one launch per step.  A decode step is
    HBM-bound on the state (read and written once per (sequence, head)); with
    many tokens per sequence the per-token state arithmetic (7 flops per state
    element: decay, S k, the delta write, S q) outweighs the bytes, and the
    roofline is taken against the fp32 vector peak instead."""
    import torch
    from gated_delta_rule_act_amd import kda, workloads as W
    from tests import gpu_util as U

    inp = W.recurrent_workload(1 if args.workload is None else args.workload)
    d = U.to_device(inp)
    out = torch.empty((inp.B, inp.T, inp.Hv, inp.V), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((inp.N, inp.Hv, inp.V, inp.K), dtype=torch.float32, device=dev)

    def step():
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"], inp.scale, inp.lower_bound,
                inp.gate_mode, initial_state=d["h0"], out=out, final_state=fs, recurrent=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    # sustained rate: five times as many steps as the chunked forward's (a decode
    # step is about a tenth as long), run on after the timed ones in blocks of
    # 100 with an event per block; figures over the second half of the blocks
    nblk = args.sustain_steps * 5 // 100
    sus = [torch.cuda.Event(enable_timing=True) for _ in range(nblk + 1)]
    sus[0].record()
    for b in range(nblk):
        for _ in range(100):
            step()
        sus[b + 1].record()
    torch.cuda.synchronize()
    sus_tail = [sus[b].elapsed_time(sus[b + 1]) / 100 for b in range(nblk)][nblk // 2:]
    tok = inp.B * inp.T
    st = {0: 0, 1: 4, 2: 2}
    # algorithmic bytes: q, k per (token, qk-head); v, g, beta, out per (token, v-head);
    # the state read and written once per (sequence, v-head); dt_bias and A_log
    nbytes = (tok * inp.Hqk * inp.K * 2 * 2 + tok * inp.Hv * (inp.K * 2 + inp.V * 2 + 2 + inp.V * 2)
              + inp.N * inp.Hv * inp.V * inp.K * (st[inp.init_state_dtype] + st[inp.final_state_dtype])
              + inp.Hv * (inp.K + 1) * 4)
    flops = 7 * inp.K * inp.V * tok * inp.Hv
    if flops / (FP32_VALU_PEAK_TFLOPS * 1e12) > nbytes / (HBM_PEAK_GBPS * 1e9):
        roof = {"bound": "alu", "kernel": "kda_recurrent_kernel", "achieved": flops / (ms * 1e-3) / 1e12,
                "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "kernel": "kda_recurrent_kernel", "achieved": nbytes / (ms * 1e-3) / 1e9,
                "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    roof.update({"frac": roof["achieved"] / roof["peak"], "traffic": profiled_traffic("kda_recurrent_kernel", inp.name),
                 "algorithmic_bytes_per_launch": nbytes,
                 "algorithmic_flops_per_launch": flops, "avg_launch_ms": ms})
    rec = {
        "metric": "fused_recurrent_kda tokens/s (fp32 state in and out), 1 MI355X",
        "value": tok / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded numpy PCG64 draws of the workload's shapes and distributions)",
        "config": {"workload": inp.name, "B": inp.B, "T": inp.T, "H_qk": inp.Hqk, "H_v": inp.Hv, "K": inp.K,
                   "V": inp.V, "gate": ["softplus", "safe_sigmoid", "pregated"][inp.gate_mode],
                   "lower_bound": inp.lower_bound, "initial_state": "fp32", "final_state": "fp32"},
        "roofline": roof,
        "sustained": None if not sus_tail else {
            "steps": nblk * 100, "ms_per_step_median": statistics.median(sus_tail), "min": min(sus_tail),
            "max": max(sus_tail), "tokens_per_s": tok / (statistics.median(sus_tail) * 1e-3),
            "achieved_GBps": nbytes / (statistics.median(sus_tail) * 1e-3) / 1e9,
            "note": "blocks of 100 steps run on right after the timed ones; per-step figures of the second half"},
        "kernel_source_sha": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
        # the whole workload, repeated until at least 5 s of oracle time
        reps, t0 = 0, time.perf_counter()
        while True:
            o_ref, s_ref = U.run_oracle(inp, nthreads=threads)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 5.0:
                break
        e = U.errors(U.as_f64(out), o_ref, U.as_f64(fs), s_ref)
        rec["cpu_baseline"] = {"value": tok * reps / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"{inp.name}: the whole workload, {reps} times ({dt:.2f} s)", "seconds": dt}
        rec["parity"] = {"out_max_abs": e["out_max_abs"], "out_rel_rms": e["out_rel_rms"],
                         "state_rel": e["state_rel"], "tol_out_max_abs": U.OUT_MAX_ABS, "tol_state_rel": U.STATE_REL}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


def run_backward(args, dev):
    """The backward (kda_bwd) on a chunked workload: one call per step, which
    recomputes the forward quantities it needs and writes every gradient."""
    import numpy as np
    import torch
    import oracle
    from gated_delta_rule_act_amd import kda, workloads as W
    from tests import gpu_util as U

    inp = W.workload(3 if args.workload is None else args.workload)
    d = U.to_device(inp)
    d_out, dhT = W.make_grads(inp, seed=1000 + (3 if args.workload is None else args.workload))
    dev_dout = U.bf16_dev(d_out)
    dev_dhT = torch.from_numpy(dhT).to(dev)
    nseg = kda.segments_of(kda.make_params(B=inp.B, T=inp.T, H_qk=inp.Hqk, H_v=inp.Hv, num_seqs=inp.N,
                                           scale=inp.scale, lower_bound=inp.lower_bound, gate_mode=inp.gate_mode,
                                           flags=inp.flags, segments=args.segments),
                           packed=inp.cu_seqlens is not None)
    res = {}

    def step():
        res.update(kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"], inp.scale, dev_dout,
                           lower_bound=inp.lower_bound, gate_mode=inp.gate_mode, initial_state=d["h0"],
                           d_final_state=dev_dhT, cu_seqlens=d["cu_seqlens"], segments=args.segments))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    # sustained rate: steps run on after the timed ones (a quarter as many as the
    # forward's, each step being about eight times longer), second half
    ns = args.sustain_steps // 4
    sus = [torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)]
    sus[0].record()
    for i in range(ns):
        step()
        sus[i + 1].record()
    torch.cuda.synchronize()
    sus_tail = [sus[i].elapsed_time(sus[i + 1]) for i in range(ns)][ns // 2:]
    tok = inp.B * inp.T
    # the method's contractions for the gradients: the forward's 180,224 flop per
    # token-head recomputed, plus twice that for the reverse products
    flops = 3 * FLOP_PER_TOKEN_HEAD * tok * inp.Hv
    rec = {
        "metric": "chunk_kda bwd tokens/s (all input gradients), 1 MI355X",
        "value": tok / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded numpy PCG64 draws of the workload's shapes and distributions)",
        "config": {"workload": inp.name, "B": inp.B, "T": inp.T, "H_qk": inp.Hqk, "H_v": inp.Hv, "K": inp.K,
                   "V": inp.V, "gate": ["softplus", "safe_sigmoid", "pregated"][inp.gate_mode],
                   "state_segments": nseg},
        "roofline": {"bound": "alu", "kernel": "kda_bwd (all launches)",
                     "achieved": flops / (ms * 1e-3) / 1e12, "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / (ms * 1e-3) / 1e12 / FP32_VALU_PEAK_TFLOPS,
                     "traffic": profiled_bwd_traffic(inp.name),
                     "algorithmic_flops_per_launch": flops, "avg_launch_ms": ms},
        "sustained": None if not sus_tail else {
            "steps": ns, "ms_per_step_median": statistics.median(sus_tail), "min": min(sus_tail),
            "max": max(sus_tail), "tokens_per_s": tok / (statistics.median(sus_tail) * 1e-3),
            "note": "steps run on right after the timed ones; figures over the second half of them"},
        "kernel_source_sha": kernel_source_hash(),
        "bwd_kernel_source_sha": kernel_source_hash("kda_bwd.hip"),
    }
    if not args.no_cpu_baseline:
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
        # a bounded sample: the first sequence's first G v-heads (one q/k head), whole length
        G = inp.Hv // inp.Hqk
        nh = max(G, 2 if G == 1 else G)
        hs, hqs = slice(0, nh), slice(0, max(1, nh // G))
        f = oracle.bf16_to_f64
        sl = lambda a, hh: np.ascontiguousarray(a[:1, :, hh])
        t0 = time.perf_counter()
        ref = oracle.bwd(f(sl(inp.q, hqs)), f(sl(inp.k, hqs)), f(sl(inp.v, hs)), f(sl(inp.g, hs)),
                         f(np.ascontiguousarray(inp.beta[:1, :, hs])),
                         None if inp.A_log is None else inp.A_log[hs],
                         None if inp.dt_bias is None else inp.dt_bias[hs], f(sl(d_out, hs)),
                         dhT[:1, hs].astype(np.float64), scale=inp.scale, lower_bound=inp.lower_bound,
                         gate_mode=inp.gate_mode, flags=inp.flags,
                         initial_state=None if inp.initial_state is None else inp.initial_state_f64()[:1, hs],
                         nthreads=threads)
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": inp.T * nh / inp.Hv / dt, "unit": "tokens/s", "cores": threads,
                               "kind": "oracle", "seconds": dt,
                               "sample": f"{inp.name}: sequence 0, v-heads 0-{nh - 1} with their q/k heads, all "
                                         f"{inp.T} tokens ({dt:.2f} s); tokens/s scaled to all {inp.Hv} heads"}
        errs = {}
        for n, sel in (("dq", hqs), ("dk", hqs), ("dv", hs), ("dg", hs), ("dbeta", hs), ("dh0", hs)):
            a = res[n][:1, :, sel].double().cpu().numpy() if n != "dh0" else res[n][:1, sel].double().cpu().numpy()
            b = ref[n]
            errs[n] = float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
        rec["parity"] = {"sampled_rel_fro": errs, "tol": 1e-3}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
