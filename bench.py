#!/usr/bin/env python3
"""Benchmark of the RoPE + attention hot path on one MI355X.

One step = one pass of the path over one batch of the GQA causal prefill
workload (B=4, S=2048, H_q=32, H_kv=8, d_h=128, bf16, RoPE base 10000):
  1. RoPE of K into the rotated-key buffer (apex_rope_qk, elementwise launch);
  2. attention with RoPE of Q fused into its tile loads (apex_attn_prefill,
     apply_rope=2).
Throughput is mask-adjusted: 4 * B * H_q * d_h FLOPs per visible (query, key)
pair (RoPE and softmax are not credited). Inputs are seeded N(0,1) draws
already resident in HBM when the timed region starts.

The line also carries the split-K decode workload (B=64, Sk=32768, H_q=128,
H_kv=8) in HBM GB/s, the window / long-context prefill workloads, the
roofline of the dominant kernel, and the fp64 CPU oracle timed on a bounded
sample of the same workload (a baseline, not a target).

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
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
HEADLINE = "gqa_prefill_s2048"
DECODE = "gqa_decode_sk32768"
MLA_DECODE = "mla_global_decode_sk32768"
RMSNORMS = ("rmsnorm_b4_s2048_d7168", "rmsnorm_b64_s2048_d512")
OTHERS = ("window_prefill_s16384_w4096", "local_prefill_s65536_w512",
          "prefix_prefill_s2048_p512", "prefix_local_prefill_s16384_w4096_p1024",
          "yarn_local_prefill_s32768_w4096_s4", "mla_global_prefill_s16384")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_bf16_gqa_s2048_traffic.json")
PREFILL_SOURCES = ("transformer_attention_amd/csrc/prefill_kernel.hpp",
                   "transformer_attention_amd/csrc/device_common.hpp")


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


def load_traffic():
    """HBM bytes per launch of the prefill kernel from the committed rocprofv3
    counter summary, or None when the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != sources_sha(PREFILL_SOURCES):
        return None
    return t.get("hbm_bytes_per_launch")


SETTLE_S = 0.3  # untimed work before the warm-up steps of each timed workload
EVENT_EVERY = 8  # per-launch events on one step in EVENT_EVERY (see time_prefill)


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


def time_prefill(taa, torch, name, steps, warmup):
    import apex_inputs
    w = apex_inputs.WORKLOADS[name]
    q, k, v = apex_inputs.workload_inputs(name, device="cuda")
    kr, o = torch.empty_like(k), torch.empty_like(q)
    ys = w.get("yarn_s", 1.0)
    kw = dict(causal=w["causal"], W=w["W"], m0=w["m0"], base=w["base"], prefix=w.get("prefix", 0),
              yarn_s=ys)

    if w["kind"] == "mla_prefill":
        # the MLA call rotates the key rope parts and runs the attention in one call
        o = torch.empty(q.shape[:3] + (w["d"],), dtype=q.dtype, device=q.device)

    # Per-launch HIP events go on a sample of the timed steps only: each
    # record costs about 3.5 us of GPU time, so recording around both launches
    # of every step would slow the very steps whose wall time is reported.
    # Step i records around its RoPE launch when i % every == every // 2,
    # around its attention launch when i % every == 0 (every step of a short run).
    every = EVENT_EVERY if steps >= 2 * EVENT_EVERY else 1

    def step(i=-1, ev=None):
        samp_attn = ev is not None and i % every == 0
        samp_rope = ev is not None and i % every == every // 2
        if samp_rope:
            ev[0].record()
        if w["kind"] != "mla_prefill":
            taa.apex_rope_qk(None, k, k_out=kr, m0=w["m0"], base=w["base"], yarn_s=ys)
        if samp_rope or samp_attn:
            ev[1].record()
        if w["kind"] == "mla_prefill":
            taa.apex_attn_prefill_mla(q, k, v, o, kr, apply_rope=1, **kw)
        else:
            taa.apex_attn_prefill(q, kr, v, o, None, apply_rope=2, **kw)
        if samp_attn:
            ev[2].record()

    settle(torch, step)
    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    attn = [evs[i][1].elapsed_time(evs[i][2]) for i in range(0, steps, every)]
    ropes = [evs[i][0].elapsed_time(evs[i][1]) for i in range(every // 2, steps, every)]
    rope_ms = sum(ropes) / len(ropes)
    attn_ms = sum(attn) / len(attn)
    attn_min = min(attn)
    del q, k, v, kr, o
    return w, wall * 1e3, rope_ms, attn_ms, attn_min


def time_calls(torch, fn, steps):
    """Mean duration of `steps` back-to-back calls of fn, from one pair of
    events around the whole loop, plus the per-call durations of a sample of
    the calls (events around one call in EVENT_EVERY; every call of a short
    run), all on the launch stream. Events around every call would add their
    own ~3.5 us to short kernels."""
    every = EVENT_EVERY if steps >= 2 * EVENT_EVERY else 1
    ev = lambda: torch.cuda.Event(enable_timing=True)
    e0, e1 = ev(), ev()
    samples = [(ev(), ev()) for _ in range(0, steps, every)]
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        if i % every == 0:
            samples[i // every][0].record()
        fn()
        if i % every == 0:
            samples[i // every][1].record()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, sorted(a.elapsed_time(b) for a, b in samples)


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
    mean, ms = time_calls(torch, call, steps)
    del x, g, y
    return w, mean, ms[0]


def time_decode(taa, torch, steps, warmup, name=DECODE):
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
    mean, ms = time_calls(torch, call, steps)
    del q, kc, vc, kn, vn, o, ws
    return w, mean, ms[len(ms) // 2], ms[0]


def cpu_baseline(w, budget_s):
    """Time the fp64 oracle over the whole workload (every batch element, head
    and row, drawn on the host from the same seeds), repeating whole passes
    until about budget_s seconds have been spent."""
    import apex_inputs
    import oracle
    threads = oracle.default_threads()
    B, S, Hq, Hkv, d = w["B"], w["S"], w["Hq"], w["Hkv"], w["d"]
    q, k, v = apex_inputs.prefill_inputs(B, S, Hq, Hkv, d, w["dtype"], seed=w["seed"],
                                         device="cpu")
    flops = 4 * d * B * Hq * n_visible(S, w["causal"], w["W"])
    kw = dict(causal=w["causal"], W=w["W"], m0=w["m0"], base=w["base"], nthreads=threads)
    passes, t = 0, 0.0
    while passes == 0 or t < budget_s:
        t0 = time.perf_counter()
        oracle.prefill(q, k, v, **kw)
        t += time.perf_counter() - t0
        passes += 1
    return {"value": round(passes * flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d whole pass(es) over %s (B=%d x %d heads x %d rows, drawn on the "
                      "host), %.1f s, %.4g GFLOP mask-adjusted per pass"
                      % (passes, HEADLINE, B, Hq, S, t, flops / 1e9)}


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


def _pmc_per_dispatch(csv_path, kernel_substr):
    """Mean counter value (KiB) per dispatch of the kernels whose name contains
    kernel_substr, from a rocprofv3 --pmc ... --output-format csv file."""
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if kernel_substr in r["Kernel_Name"]]
    if not vals:
        raise ValueError("no %s dispatches in %s" % (kernel_substr, csv_path))
    return sum(vals) / len(vals), len(vals)


def pmc_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """Write the prefill kernel's HBM traffic per launch, from FETCH_SIZE and
    WRITE_SIZE runs scaled by what the same counters read for the calibration
    copy (read 1 GiB, write 1 GiB), into profiles/ next to the source hash."""
    f = lambda d: os.path.join(d, "p_counter_collection.csv")
    kname = "prefill_bf16_kernel<128, 128, 128>"
    fetch, nf = _pmc_per_dispatch(f(fetch_dir), kname)
    write, nw = _pmc_per_dispatch(f(write_dir), kname)
    cf, _ = _pmc_per_dispatch(f(copy_fetch_dir), "neg_kernel")
    cw, _ = _pmc_per_dispatch(f(copy_write_dir), "neg_kernel")
    known_kib = (1 << 30) / 1024.0
    fetch_scale, write_scale = known_kib / cf, known_kib / cw
    out = {
        "kernel": kname, "workload": HEADLINE,
        "fetch_kib_per_dispatch_raw": round(fetch, 1), "write_kib_per_dispatch_raw": round(write, 1),
        "dispatches": [nf, nw],
        "copy_calibration": {"known_kib_read": known_kib, "fetch_kib": round(cf, 1),
                             "known_kib_written": known_kib, "write_kib": round(cw, 1),
                             "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4)},
        "hbm_read_bytes_per_launch": int(fetch * fetch_scale * 1024),
        "hbm_write_bytes_per_launch": int(write * write_scale * 1024),
        "hbm_bytes_per_launch": int((fetch * fetch_scale + write * write_scale) * 1024),
        "algorithmic_bytes_per_launch": prefill_bytes(__import__("apex_inputs").WORKLOADS[HEADLINE]),
        "source_sha": sources_sha(PREFILL_SOURCES),
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline prefill (for profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run the counter-calibration copy kernel and exit")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc output dirs -> the prefill traffic summary in profiles/")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
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

    log("timing %s: %d warmup + %d steps" % (HEADLINE, args.warmup, args.steps))
    w, ms_step, rope_ms, attn_ms, attn_min = time_prefill(taa, torch, HEADLINE, args.steps,
                                                         args.warmup)
    flops = prefill_flops(w)
    value = flops / (ms_step * 1e-3) / 1e12
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    log("step %.4f ms (rope_k %.4f ms, attention %.4f ms) -> %.1f TFLOP/s"
        % (ms_step, rope_ms, attn_ms, value))

    extra = {}
    if not args.headline_only:
        dsteps = max(5, args.steps // 10)
        log("timing %s: %d warmup + %d calls" % (DECODE, args.warmup, dsteps))
        dw, d_mean, d_med, d_min = time_decode(taa, torch, dsteps, args.warmup)
        dbytes = decode_bytes(dw)
        gbs = dbytes / (d_mean * 1e-3) / 1e9
        log("decode %.4f ms -> %.1f GB/s" % (d_mean, gbs))
        extra["decode"] = {
            "workload": DECODE, "metric": "decode HBM GB/s (algorithmic bytes)",
            "value": round(gbs, 1), "unit": "GB/s", "ms_per_call": round(d_mean, 4),
            "ms_median": round(d_med, 4), "ms_min": round(d_min, 4),
            "algorithmic_bytes": dbytes, "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "note": ("whole call: split-K pass + combine pass; mean from events around the "
                     "timed calls, median/min from per-call events on a sample of them")}
        torch.cuda.empty_cache()
        log("timing %s: %d warmup + %d calls" % (MLA_DECODE, args.warmup, dsteps))
        mw, m_mean, m_med, m_min = time_decode(taa, torch, dsteps, args.warmup, MLA_DECODE)
        mbytes = decode_bytes(mw)
        mgbs = mbytes / (m_mean * 1e-3) / 1e9
        log("mla decode %.4f ms -> %.1f GB/s" % (m_mean, mgbs))
        extra["decode_mla"] = {
            "workload": MLA_DECODE, "value": round(mgbs, 1), "unit": "GB/s",
            "ms_per_call": round(m_mean, 4), "ms_median": round(m_med, 4),
            "ms_min": round(m_min, 4), "algorithmic_bytes": mbytes,
            "frac_of_hbm_peak": round(mgbs / PEAK_HBM_GBS, 4)}
        torch.cuda.empty_cache()
        others = {}
        for name in OTHERS:
            log("timing %s" % name)
            ow, oms, orope, oattn, _ = time_prefill(taa, torch, name, max(3, args.steps // 25),
                                                    3)
            of = prefill_flops(ow)
            others[name] = {"ms_per_step": round(oms, 4), "rope_k_ms": round(orope, 4),
                            "attention_ms": round(oattn, 4),
                            "tflops": round(of / (oms * 1e-3) / 1e12, 1),
                            "attention_tflops": round(of / (oattn * 1e-3) / 1e12, 1),
                            "frac_of_bf16_peak": round(of / (oms * 1e-3) / 1e12
                                                       / PEAK_BF16_TFLOPS, 4)}
            if ow["kind"] == "mla_prefill":
                others[name]["note"] = ("one apex_attn_prefill_mla call: attention_ms includes "
                                        "its key RoPE launch")
        extra["other_workloads"] = others
        torch.cuda.empty_cache()
        norms = {}
        for name in RMSNORMS:
            log("timing %s" % name)
            rw, rms_mean, rms_min = time_rmsnorm(taa, torch, name, max(10, args.steps // 5), 3)
            rb = rmsnorm_bytes(rw)
            norms[name] = {"ms_per_call": round(rms_mean, 4),
                           "ms_min_event_bracketed": round(rms_min, 4),
                           "algorithmic_bytes": rb,
                           "gbs": round(rb / (rms_mean * 1e-3) / 1e9, 1),
                           "frac_of_hbm_peak": round(rb / (rms_mean * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                                     4),
                           "note": ("mean from events around the whole timed loop; the minimum "
                                    "comes from events around single calls, which add about "
                                    "2 us each")}
        extra["rmsnorm"] = norms
        torch.cuda.empty_cache()

    line = {
        "metric": "attention TFLOP/s (mask-adjusted) + % bf16 MFMA peak; decode HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "event_sample": "per-launch events on 1 step in %d" % EVENT_EVERY,
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
        "roofline": {"kernel": "prefill_bf16_kernel<128, 128, 128>", "bound": "mfma",
                     "achieved": round(attn_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": load_traffic(), "launch_ms_mean": round(attn_ms, 4),
                     "launch_ms_min": round(attn_min, 4),
                     "algorithmic_bytes": prefill_bytes(w)},
        "rope_k_ms": round(rope_ms, 4),
    }
    line.update(extra)
    if args.cpu_budget > 0:
        log("timing the CPU oracle (budget %.0f s)" % args.cpu_budget)
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
