#!/usr/bin/env python3
"""Benchmark of the RoPE + attention hot path on one MI355X.

One step = one pass of the path over one batch of the sliding-window GQA
prefill workload, the largest of the prefill workloads by work (B=2,
S=16384, H_q=32, H_kv=8, d_h=128, causal with window W=4096, bf16, RoPE base
10000):
  1. RoPE of K into the rotated-key buffer (apex_rope_qk, elementwise launch);
  2. attention with RoPE of Q fused into its tile loads (apex_attn_prefill,
     apply_rope=2).
Throughput is mask-adjusted: 4 * B * H_q * d_h FLOPs per visible (query, key)
pair (RoPE and softmax are not credited). Inputs are seeded N(0,1) draws
already resident in HBM when the timed region starts.

Timing. The steps are timed with nothing but a synchronize on both sides
(and one event pair around the whole loop); no event is recorded between
them. A kernel's average launch duration, which its roofline block divides
into, comes from a second timed region: the same launch repeated back to back
on the launch stream with one HIP event pair around the loop.

The same line carries, each with its own roofline block: the causal GQA
prefill (B=4, S=2048), the long local-window prefill (B=1, S=65536, W=512)
and the split-K decode (B=64, Sk=32768, H_q=128, H_kv=8) in HBM GB/s; the
tiny fp32 prefill (B=1, S=128) for information; the prefix, YaRN and MLA
prefill and the RMSNorm workloads; and the fp64 CPU oracle timed on a bounded
sample of the headline workload (a baseline, not a target).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
HEADLINE = "window_prefill_s16384_w4096"
ROOFLINE_PREFILLS = ("gqa_prefill_s2048", "local_prefill_s65536_w512")
DECODE = "gqa_decode_sk32768"
TINY = "tiny_prefill_f32"
MLA_DECODE = "mla_global_decode_sk32768"
RMSNORMS = ("rmsnorm_b4_s2048_d7168", "rmsnorm_b64_s2048_d512")
OTHERS = ("prefix_prefill_s2048_p512", "prefix_local_prefill_s16384_w4096_p1024",
          "yarn_local_prefill_s32768_w4096_s4", "mla_global_prefill_s16384")
PREFILL_KERNEL = "prefill_bf16_kernel<128, 128, 128>"
DECODE_KERNEL = "decode_split_kernel<128, 128, 128>"
KERNEL_SOURCES = {
    PREFILL_KERNEL: ("transformer_attention_amd/csrc/prefill_kernel.hpp",
                     "transformer_attention_amd/csrc/device_common.hpp"),
    DECODE_KERNEL: ("transformer_attention_amd/csrc/decode_kernel.hpp",
                    "transformer_attention_amd/csrc/device_common.hpp"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def n_visible(S, causal, W, P=0):
    """Visible (query, key) pairs of one (b, h): key j visible to query i iff
    j <= i and, with a window, i - j < W (Part 2, §10.2); with a prefix of P
    positions, rows i < P see exactly the keys j < P (Part 2, §11.1)."""
    if not causal:
        return S * S
    P = min(P, S)
    if W == 0 or W >= S:
        rest = S * (S + 1) // 2 - P * (P + 1) // 2     # rows P .. S-1 see i + 1 keys
    else:
        def upto(n):  # sum over rows i < n of min(i + 1, W)
            m = min(n, W)
            return m * (m + 1) // 2 + max(0, n - W) * W
        rest = upto(S) - upto(P)
    return P * P + rest


def prefill_flops(w):
    """2 FLOPs per multiply-add of q.k (d_h + d_r wide; d_r = 0 outside MLA)
    and of p.v (d_h wide), per visible pair and query head."""
    width = 2 * w["d"] + w.get("d_r", 0)
    return 2 * width * w["B"] * w["Hq"] * n_visible(w["S"], w["causal"], w["W"],
                                                    w.get("prefix", 0))


def prefill_bytes(w):
    """Algorithmic HBM bytes of the attention launch: q, k, v read once, o written once."""
    e = 2 if w["dtype"] == "bf16" else 4
    dqk, dv = w["d"] + w.get("d_r", 0), w["d"]
    return e * w["S"] * w["B"] * (w["Hq"] * (dqk + dv) + w["Hkv"] * (dqk + dv))


def decode_bytes(w):
    """Algorithmic bytes of one decode call: the K and V caches read once, q
    read, o written, the new key and value read (keys d_h + d_r wide for MLA)."""
    B, Sk, Hq, Hkv, d = w["B"], w["Sk"], w["Hq"], w["Hkv"], w["d"]
    dk = d + w.get("d_r", 0)
    return 2 * ((B * Hkv * Sk + B * Hq + B * Hkv) * (dk + d))


def rmsnorm_bytes(w):
    """Algorithmic bytes of one RMSNorm call: x read once, y written once, gamma read."""
    e = 2 if w["dtype"] == "bf16" else 4
    return e * w["d"] * (2 * w["B"] * w["S"] + 1)


def sources_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)


def load_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` at `workload` from the committed
    rocprofv3 counter summary, or None when there is none or the kernel's
    sources changed since the counters were taken."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel") != kernel or t.get("source_sha") != sources_sha(KERNEL_SOURCES[kernel]):
        return None
    return t.get("hbm_bytes_per_launch")


SETTLE_S = 0.3  # untimed work before the warm-up steps of each timed workload


def settle(torch, fn):
    """Run fn untimed for about SETTLE_S seconds of wall time, so the GPU's
    clocks have left their idle state before the warm-up steps; a few
    milliseconds of work at the start of a run measure ~20% slow otherwise."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
    return n


def timed_loop(torch, fn, n):
    """Mean duration (ms) of n back-to-back calls of fn, from one event pair
    around the loop on the current (launch) stream, and the wall time per
    call between synchronizes on both sides."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / n * 1e3
    return e0.elapsed_time(e1) / n, wall


def time_prefill(taa, torch, name, steps, warmup):
    """Step time (RoPE of K + attention) over `steps` timed steps, then the
    attention launch alone and the RoPE launch alone, each over `steps`
    back-to-back launches."""
    import apex_inputs
    w = apex_inputs.WORKLOADS[name]
    q, k, v = apex_inputs.workload_inputs(name, device="cuda")
    kr, o = torch.empty_like(k), torch.empty_like(q)
    ys = w.get("yarn_s", 1.0)
    kw = dict(causal=w["causal"], W=w["W"], m0=w["m0"], base=w["base"], prefix=w.get("prefix", 0),
              yarn_s=ys)
    mla = w["kind"] == "mla_prefill"
    if mla:  # the MLA call rotates the key rope parts and runs the attention in one call
        o = torch.empty(q.shape[:3] + (w["d"],), dtype=q.dtype, device=q.device)

    def rope():
        taa.apex_rope_qk(None, k, k_out=kr, m0=w["m0"], base=w["base"], yarn_s=ys)

    def attn():
        if mla:
            taa.apex_attn_prefill_mla(q, k, v, o, kr, apply_rope=1, **kw)
        else:
            taa.apex_attn_prefill(q, kr, v, o, None, apply_rope=2, **kw)

    def step():
        if not mla:
            rope()
        attn()

    settle(torch, step)
    for _ in range(warmup):
        step()
    ev_ms, wall_ms = timed_loop(torch, step, steps)
    attn_ms, _ = timed_loop(torch, attn, steps)
    rope_ms = None if mla else timed_loop(torch, rope, steps)[0]
    del q, k, v, kr, o
    return w, wall_ms, ev_ms, attn_ms, rope_ms


def prefill_roofline(w, attn_ms, kernel, name):
    flops = prefill_flops(w)
    tf = flops / (attn_ms * 1e-3) / 1e12
    return {"kernel": kernel, "bound": "mfma", "achieved": round(tf, 1),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "traffic": load_traffic(name, kernel), "launch_ms_mean": round(attn_ms, 4),
            "algorithmic_flops": flops, "algorithmic_bytes": prefill_bytes(w)}


def prefill_entry(taa, torch, name, steps, warmup, roofline):
    log("timing %s: %d warmup + %d steps" % (name, warmup, steps))
    w, ms, ev_ms, attn_ms, rope_ms = time_prefill(taa, torch, name, steps, warmup)
    flops = prefill_flops(w)
    tf = flops / (ms * 1e-3) / 1e12
    log("  step %.4f ms (events %.4f; attention %.4f ms, rope_k %s) -> %.1f TFLOP/s"
        % (ms, ev_ms, attn_ms, "%.4f ms" % rope_ms if rope_ms is not None else "-", tf))
    e = {"ms_per_step": round(ms, 4), "steps": steps, "tflops": round(tf, 1),
         "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
         "attention_ms": round(attn_ms, 4),
         "attention_tflops": round(flops / (attn_ms * 1e-3) / 1e12, 1),
         "rope_k_ms": round(rope_ms, 4) if rope_ms is not None else None,
         "mask_adjusted_flops": flops}
    if w["kind"] == "mla_prefill":
        e["note"] = "one apex_attn_prefill_mla call: attention_ms includes its key RoPE launch"
    if roofline:
        e["roofline"] = prefill_roofline(w, attn_ms, PREFILL_KERNEL, name)
    return w, ms, e


def time_rmsnorm(taa, torch, name, steps, warmup):
    import apex_inputs
    w = apex_inputs.WORKLOADS[name]
    x, g = apex_inputs.workload_inputs(name, device="cuda")
    y = torch.empty_like(x)

    def call():
        taa.apex_rmsnorm(x, g, y, eps=w["eps"])

    settle(torch, call)
    for _ in range(warmup):
        call()
    mean, _ = timed_loop(torch, call, steps)
    del x, g, y
    return w, mean


def time_decode(taa, torch, steps, warmup, name):
    import apex_inputs
    w = apex_inputs.WORKLOADS[name]
    q, kc, vc, kn, vn = apex_inputs.workload_inputs(name, device="cuda")
    B, Hq = q.shape[:2]
    Hkv, Sk, d = kc.shape[1], kc.shape[2], w["d"]
    o = torch.empty(B, Hq, 1, d, dtype=q.dtype, device="cuda")
    ws = torch.empty(taa.apex_attn_decode_workspace_bytes(B, Hq, Hkv, Sk, d), dtype=torch.uint8,
                     device="cuda")
    fn = taa.apex_attn_decode_mla if w["kind"] == "mla_decode" else taa.apex_attn_decode

    def call():
        fn(q, kc, vc, kn, vn, o, m=w["m"], W=w["W"], base=w["base"], workspace=ws)

    settle(torch, call)
    for _ in range(warmup):
        call()
    mean, wall = timed_loop(torch, call, steps)
    del q, kc, vc, kn, vn, o, ws
    return w, mean, wall


def decode_entry(taa, torch, name, steps, warmup, roofline):
    log("timing %s: %d warmup + %d calls" % (name, warmup, steps))
    w, mean, wall = time_decode(taa, torch, steps, warmup, name)
    b = decode_bytes(w)
    gbs = b / (mean * 1e-3) / 1e9
    log("  decode %.4f ms (wall %.4f) -> %.1f GB/s" % (mean, wall, gbs))
    e = {"metric": "decode HBM GB/s (algorithmic bytes)", "value": round(gbs, 1), "unit": "GB/s",
         "ms_per_call": round(mean, 4), "steps": steps, "algorithmic_bytes": b,
         "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
         "note": ("whole call, events around the back-to-back calls; at this shape the split "
                  "pass merges its two key ranges itself, so it is the call's only launch")}
    if roofline:
        e["roofline"] = {"kernel": DECODE_KERNEL, "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": load_traffic(name, DECODE_KERNEL),
                         "launch_ms_mean": round(mean, 4), "algorithmic_bytes": b}
    return e


def cpu_baseline(w, budget_s):
    """Time the fp64 oracle on a bounded sample of the workload: every row of
    batch element 0's first KV group (G query heads x S rows, drawn on the
    host from the workload's seeds), whole passes repeated until about
    budget_s seconds have been spent."""
    import numpy as np

    import apex_inputs
    import oracle
    threads = oracle.default_threads()
    S, Hq, Hkv, d = w["S"], w["Hq"], w["Hkv"], w["d"]
    G = Hq // Hkv
    q, k, v = apex_inputs.prefill_inputs(1, S, Hq, Hkv, d, w["dtype"], seed=w["seed"],
                                         device="cpu")
    rows = np.arange(G * S, dtype=np.int64)
    flops = 4 * d * G * n_visible(S, w["causal"], w["W"])
    kw = dict(causal=w["causal"], W=w["W"], m0=w["m0"], base=w["base"], nthreads=threads,
              rows=rows)
    passes, t = 0, 0.0
    while passes == 0 or t < budget_s:
        t0 = time.perf_counter()
        oracle.prefill(q, k, v, **kw)
        t += time.perf_counter() - t0
        passes += 1
    return {"value": round(passes * flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d whole pass(es) over batch element 0, query heads 0-%d (KV head 0) x "
                      "%d rows of %s (inputs drawn on the host from its seeds), %.1f s, "
                      "%.4g GFLOP mask-adjusted per pass" % (passes, G - 1, S, HEADLINE, t,
                                                             flops / 1e9)}


# ------------------------------------------------------- counter summaries --
def copy_calibration(torch):
    """A plain elementwise copy of known size (read 1 GiB, write 1 GiB), run for
    scaling the rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes."""
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_kernel": "neg", "read_bytes": 4 * n, "write_bytes": 4 * n,
                      "launches": 5}))


def _pmc_per_dispatch(csv_path, kernel_substr, counter=None):
    """Mean counter value per dispatch of the kernels whose name contains
    kernel_substr, from a rocprofv3 --pmc ... --output-format csv file."""
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if kernel_substr in r["Kernel_Name"]
            and (counter is None or r["Counter_Name"] == counter)]
    if not vals:
        raise ValueError("no %s dispatches in %s" % (kernel_substr, csv_path))
    return sum(vals) / len(vals), len(vals)


def _csv(d):
    return os.path.join(d, "p_counter_collection.csv")


def traffic_summary(workload, kernel, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """Write `kernel`'s HBM traffic per launch at `workload`, from FETCH_SIZE and
    WRITE_SIZE runs scaled by what the same counters read for the calibration
    copy (read 1 GiB, write 1 GiB), into profiles/ next to the source hash."""
    import apex_inputs
    w = apex_inputs.WORKLOADS[workload]
    fetch, nf = _pmc_per_dispatch(_csv(fetch_dir), kernel)
    write, nw = _pmc_per_dispatch(_csv(write_dir), kernel)
    cf, _ = _pmc_per_dispatch(_csv(copy_fetch_dir), "neg_kernel")
    cw, _ = _pmc_per_dispatch(_csv(copy_write_dir), "neg_kernel")
    known_kib = (1 << 30) / 1024.0
    fetch_scale, write_scale = known_kib / cf, known_kib / cw
    alg = decode_bytes(w) if "decode" in w["kind"] else prefill_bytes(w)
    out = {
        "kernel": kernel, "workload": workload,
        "fetch_kib_per_dispatch_raw": round(fetch, 1), "write_kib_per_dispatch_raw": round(write, 1),
        "dispatches": [nf, nw],
        "copy_calibration": {"known_kib_read": known_kib, "fetch_kib": round(cf, 1),
                             "known_kib_written": known_kib, "write_kib": round(cw, 1),
                             "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4)},
        "hbm_read_bytes_per_launch": int(fetch * fetch_scale * 1024),
        "hbm_write_bytes_per_launch": int(write * write_scale * 1024),
        "hbm_bytes_per_launch": int((fetch * fetch_scale + write * write_scale) * 1024),
        "algorithmic_bytes_per_launch": alg,
        "source_sha": sources_sha(KERNEL_SOURCES[kernel]),
    }
    os.makedirs(os.path.dirname(traffic_file(workload)), exist_ok=True)
    with open(traffic_file(workload), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE",
                 "SQ_BUSY_CYCLES")


def mfma_summary(workload, pmc_dir, trace_dir):
    """Matrix-core use of the prefill kernel at `workload` from one rocprofv3
    --pmc run of MFMA_COUNTERS (averaged per dispatch) and the kernel's average
    duration from a --kernel-trace run of the same command. Printed as JSON."""
    import csv
    import apex_inputs
    w = apex_inputs.WORKLOADS[workload]
    vals = {c: _pmc_per_dispatch(_csv(pmc_dir), PREFILL_KERNEL, c) for c in MFMA_COUNTERS}
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
            for r in csv.DictReader(open(os.path.join(trace_dir, "t_kernel_trace.csv")))
            if PREFILL_KERNEL in r["Kernel_Name"]]
    out = {"kernel": PREFILL_KERNEL, "workload": workload,
           "per_dispatch": {c: v[0] for c, v in vals.items()},
           "dispatches": {c: v[1] for c, v in vals.items()},
           "kernel_us_mean": sum(durs) / len(durs), "trace_dispatches": len(durs),
           "mask_adjusted_flops": prefill_flops(w), "source_sha": sources_sha(
               KERNEL_SOURCES[PREFILL_KERNEL])}
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--only", metavar="WORKLOAD",
                    help="time only this prefill or decode workload (for profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run the counter-calibration copy kernel and exit")
    ap.add_argument("--traffic-summary", nargs=6,
                    metavar=("WORKLOAD", "KERNEL", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc output dirs -> profiles/traffic_<WORKLOAD>.json")
    ap.add_argument("--mfma-summary", nargs=3, metavar=("WORKLOAD", "PMC_DIR", "TRACE_DIR"),
                    help="rocprofv3 MFMA counter + kernel trace dirs -> JSON on stdout")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.mfma_summary:
        mfma_summary(*args.mfma_summary)
        return

    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    from transformer_attention_amd import build as hipbuild
    if not os.path.exists(hipbuild.LIB):
        hipbuild.build()
    import transformer_attention_amd as taa
    taa.lib()

    if args.only:
        import apex_inputs
        if apex_inputs.WORKLOADS[args.only]["kind"] in ("decode", "mla_decode"):
            e = decode_entry(taa, torch, args.only, args.steps, args.warmup, False)
        else:
            e = prefill_entry(taa, torch, args.only, args.steps, args.warmup, False)[2]
        print(json.dumps({"workload": args.only, **e}), flush=True)
        return

    w, ms_step, head = prefill_entry(taa, torch, HEADLINE, args.steps, args.warmup, True)
    flops = prefill_flops(w)
    value = flops / (ms_step * 1e-3) / 1e12

    workloads = {}
    for name in ROOFLINE_PREFILLS:
        workloads[name] = prefill_entry(taa, torch, name, args.steps, args.warmup, True)[2]
        torch.cuda.empty_cache()
    workloads[DECODE] = decode_entry(taa, torch, DECODE, args.steps, args.warmup, True)
    torch.cuda.empty_cache()
    tw, tms, tiny = prefill_entry(taa, torch, TINY, args.steps, args.warmup, False)
    tf = prefill_flops(tw) / (tms * 1e-3) / 1e12
    workloads[TINY] = {"us_per_step": round(tms * 1e3, 2), "steps": args.steps,
                       "tflops": round(tf, 4), "frac_of_fp32_peak": round(tf / PEAK_F32_TFLOPS, 6),
                       "attention_us": round(tiny["attention_ms"] * 1e3, 2),
                       "note": "fp32, launch-latency bound; for information only"}
    workloads[MLA_DECODE] = decode_entry(taa, torch, MLA_DECODE, args.steps, args.warmup, False)
    torch.cuda.empty_cache()
    for name in OTHERS:
        workloads[name] = prefill_entry(taa, torch, name, args.steps, args.warmup, False)[2]
        torch.cuda.empty_cache()
    norms = {}
    for name in RMSNORMS:
        log("timing %s: %d warmup + %d calls" % (name, args.warmup, args.steps))
        rw, rms_mean = time_rmsnorm(taa, torch, name, args.steps, args.warmup)
        rb = rmsnorm_bytes(rw)
        gbs = rb / (rms_mean * 1e-3) / 1e9
        norms[name] = {"ms_per_call": round(rms_mean, 4), "algorithmic_bytes": rb,
                       "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                       "note": "events around the back-to-back calls only"}
    torch.cuda.empty_cache()

    line = {
        "metric": "attention TFLOP/s (mask-adjusted) + % bf16 MFMA peak; decode HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "B": w["B"], "S": w["S"], "H_q": w["Hq"],
                   "H_kv": w["Hkv"], "d_h": w["d"], "causal": w["causal"], "W": w["W"],
                   "rope_base": w["base"], "mask_adjusted_flops": flops},
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": head["roofline"],
        "attention_ms": head["attention_ms"],
        "rope_k_ms": head["rope_k_ms"],
        "timing": ("steps: wall clock between synchronizes; launch_ms_mean: HIP events around "
                   "the launch repeated back to back, on the launch stream"),
        "workloads": workloads,
        "rmsnorm": norms,
    }
    if args.cpu_budget > 0:
        log("timing the CPU oracle (budget %.0f s)" % args.cpu_budget)
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
