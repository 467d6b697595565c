"""Host-side arithmetic of bench.py: visible-pair counts and algorithmic bytes."""
import subprocess
import sys

import pytest

import bench
import oracle


@pytest.mark.parametrize("S", [1, 2, 7, 64, 100])
@pytest.mark.parametrize("W", [0, 1, 3, 64, 99, 100, 1000])
@pytest.mark.parametrize("causal", [0, 1])
def test_n_visible_matches_the_mask(S, W, causal):
    if W and not causal:
        return
    brute = sum(oracle.visible(i, j, causal, W) for i in range(S) for j in range(S))
    assert bench.n_visible(S, causal, W) == brute


@pytest.mark.parametrize("S", [1, 7, 64, 100])
@pytest.mark.parametrize("W", [0, 1, 3, 64])
@pytest.mark.parametrize("P", [1, 5, 63, 100, 150])
def test_n_visible_with_prefix_matches_the_mask(S, W, P):
    brute = sum(oracle.visible(i, j, 1, W, P) for i in range(S) for j in range(S))
    assert bench.n_visible(S, 1, W, P) == brute


def test_workload_counts():
    import apex_inputs
    w = apex_inputs.WORKLOADS
    assert bench.n_visible(2048, 1, 0) == 2098176
    assert bench.n_visible(16384, 1, 4096) == 58722304
    assert bench.n_visible(65536, 1, 512) == 33423616
    assert bench.prefill_flops(w["gqa_prefill_s2048"]) == 137506062336
    assert bench.decode_bytes(w["gqa_decode_sk32768"]) == 8594391040
    # MLA decode: 192-wide keys, 128-wide values
    assert bench.decode_bytes(w["mla_global_decode_sk32768"]) == \
        2 * (64 * 8 * 32768 + 64 * 128 + 64 * 8) * (192 + 128)
    # MLA: q.k over 128 + 64 dims, p.v over 128 -> 2 * 320 FLOPs per pair and head
    assert bench.prefill_flops(w["mla_global_prefill_s16384"]) == 640 * 64 * (16384 * 16385 // 2)
    assert bench.prefill_bytes(w["mla_global_prefill_s16384"]) == 2 * 16384 * 72 * 320
    assert bench.rmsnorm_bytes(w["rmsnorm_b4_s2048_d7168"]) == 2 * 7168 * (2 * 4 * 2048 + 1)


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_headline_is_the_largest_prefill_by_work():
    # the line's value is quoted on the prefill workload with the most
    # mask-adjusted FLOPs among the benchmark's prefill configurations
    import apex_inputs
    w = apex_inputs.WORKLOADS
    cands = (bench.HEADLINE,) + bench.ROOFLINE_PREFILLS + (bench.TINY,)
    assert max(cands, key=lambda n: bench.prefill_flops(w[n])) == bench.HEADLINE
    assert bench.prefill_flops(w[bench.HEADLINE]) == 4 * 128 * 2 * 32 * 58722304


def test_cpu_baseline_sample_counts_its_rows():
    # the sample is one KV group of batch element 0: G heads x all S rows
    import apex_inputs
    w = apex_inputs.WORKLOADS[bench.HEADLINE]
    G = w["Hq"] // w["Hkv"]
    whole = bench.prefill_flops(w)
    assert 4 * w["d"] * G * bench.n_visible(w["S"], w["causal"], w["W"]) * w["B"] * w["Hkv"] \
        == whole


def test_prefill_roofline_block_carries_the_contract_fields():
    import apex_inputs
    w = apex_inputs.WORKLOADS[bench.HEADLINE]
    r = bench.prefill_roofline(w, 1.6, bench.PREFILL_KERNEL, bench.HEADLINE)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2516.6
    assert r["achieved"] == round(bench.prefill_flops(w) / 1.6e-3 / 1e12, 1)
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-4
    assert r["algorithmic_bytes"] == bench.prefill_bytes(w)


@pytest.mark.parametrize("workload,kernel", [
    ("window_prefill_s16384_w4096", "PREFILL_KERNEL"),
    ("gqa_prefill_s2048", "PREFILL_KERNEL"),
    ("local_prefill_s65536_w512", "PREFILL_KERNEL"),
    ("gqa_decode_sk32768", "DECODE_KERNEL"),
])
def test_committed_traffic_matches_the_kernel_sources(workload, kernel):
    # the counter-derived HBM bytes under profiles/ were taken with the kernel
    # sources as they are now (else the bench reports traffic as null)
    t = bench.load_traffic(workload, getattr(bench, kernel))
    assert t is not None and t > 0


def test_cpu_baseline_block_fields():
    import apex_inputs
    w = dict(apex_inputs.WORKLOADS[bench.HEADLINE], S=256, W=64)
    c = bench.cpu_baseline(w, 0.0)
    assert c["kind"] == "oracle" and c["unit"] == "TFLOP/s" and c["cores"] >= 1
    assert c["value"] > 0 and "1 whole pass" in c["sample"]
