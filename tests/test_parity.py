"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Inputs are seeded N(0,1) draws (apex_inputs) made on the GPU; the oracle gets
exact CPU copies of the same inputs. Bars (per element):
  fp32 workloads: max |gpu - oracle| <= 1e-4
  bf16 workloads: max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <= 2e-3
Small shapes are compared on every output element. Every benchmark workload
(tiny fp32 prefill, GQA causal prefill S=2048, window prefill S=16384 W=4096,
local prefill S=65536 W=512, GQA decode Sk=32768, and the prefix, YaRN and MLA
prefills and the MLA decode) is run at full size in the launch configuration
the benchmark times and compared on every output element, streamed one KV
group of (batch element, heads) at a time so the fp64 reference never holds a
whole output; the larger ones are split into parts so that each test stays
under a minute on the host cores. Samplers of tile-edge, first/last and random
rows run beside some of them as quicker checks.
"""
import math
import sys

import numpy as np
import pytest
import torch

import apex_inputs
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(max_abs=1e-4, mean_abs=1e-4), "bf16": dict(max_abs=2e-2, mean_abs=2e-3)}


def _say(*a):
    print("[parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def taa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_attention_amd as t
    t.lib()  # raises if the HIP library is not built
    return t


def _check(got, ref, dtype, what):
    got = got.detach().to("cpu", torch.float64).numpy().reshape(ref.shape)
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    _say("%s: max_abs %.3g mean_abs %.3g (%d values)" % (what, mx, mean, err.size))
    assert np.all(np.isfinite(got)), what
    assert mx <= TOL[dtype]["max_abs"], (what, mx)
    assert mean <= TOL[dtype]["mean_abs"], (what, mean)
    return mx, mean


def _rows(B, Hq, S, n_random, seed):
    rng = np.random.default_rng(seed)
    iset = [i for i in (0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 255, 256, 511, 512, 513, 1023,
                        1024, 1025,
                        S // 2, S - 65, S - 64, S - 33, S - 32, S - 2, S - 1) if 0 <= i < S]
    rows = set()
    for b in sorted({0, B - 1}):
        for h in sorted({0, Hq - 1, int(rng.integers(Hq))}):
            for i in iset:
                rows.add((b * Hq + h) * S + i)
    rows.update(int(x) for x in rng.integers(0, B * Hq * S, size=n_random))
    return np.array(sorted(rows), dtype=np.int64)


# ---------------------------------------------------------------- RoPE ----
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("m0", [0, 1000, 65535 - 40, 10 ** 6])
def test_rope_matches_oracle(taa, dtype, d, m0):
    _say("rope", dtype, d, m0)
    q, k, _ = apex_inputs.prefill_inputs(2, 41, 3, 2, d, dtype, seed=11, device="cuda")
    q0, k0 = q.cpu(), k.cpu()
    taa.apex_rope_qk(q, k, m0=m0)
    torch.cuda.synchronize()
    for got, src in ((q, q0), (k, k0)):
        x = src.double().numpy()
        ref = np.empty_like(x)
        for b in range(x.shape[0]):
            for h in range(x.shape[1]):
                for s in range(x.shape[2]):
                    ref[b, h, s] = oracle.rope_row(x[b, h, s], m0 + s)
        g = got.cpu().double().numpy()
        if dtype == "f32":
            assert np.max(np.abs(g - ref)) <= 1e-5
        else:  # one bf16 rounding of the rotated value
            assert np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("s,m0", [(4.0, 30000), (40.0, 0), (64.0, 10 ** 6)])
def test_rope_yarn_matches_oracle(taa, dtype, d, s, m0):
    # s = 40 and 64 put some frequencies in YaRN's interpolated band
    _say("rope yarn", dtype, d, s, m0)
    q, k, _ = apex_inputs.prefill_inputs(1, 37, 2, 1, d, dtype, seed=13, device="cuda")
    q0 = q.cpu()
    taa.apex_rope_qk(q, None, m0=m0, yarn_s=s)
    torch.cuda.synchronize()
    x = q0.double().numpy()
    ref = np.empty_like(x)
    for h in range(x.shape[1]):
        for r in range(x.shape[2]):
            ref[0, h, r] = oracle.rope_row(x[0, h, r], m0 + r, yarn_s=s)
    g = q.cpu().double().numpy()
    if dtype == "f32":
        assert np.max(np.abs(g - ref)) <= 1e-5
    else:
        assert np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)


# -------------------------------------------------------------- prefill ----
PREFILL_CASES = [
    # B, S, Hq, Hkv, d, causal, W, m0, dtype, apply_rope
    (1, 1, 2, 1, 128, 1, 0, 0, "bf16", 1),
    (1, 2, 4, 2, 64, 1, 0, 0, "bf16", 1),
    (2, 3, 4, 4, 128, 1, 0, 7, "bf16", 1),
    (1, 17, 8, 2, 128, 1, 5, 0, "bf16", 1),
    (1, 64, 16, 1, 128, 1, 0, 1000, "bf16", 1),
    (2, 65, 8, 1, 64, 1, 2, 0, "bf16", 1),
    (1, 129, 4, 4, 128, 0, 0, 0, "bf16", 1),
    (1, 300, 32, 8, 128, 1, 64, 1000, "bf16", 1),
    (1, 513, 8, 8, 64, 1, 1, 0, "bf16", 1),
    (1, 1000, 12, 4, 128, 1, 0, 0, "bf16", 1),
    (1, 777, 6, 1, 128, 0, 0, 0, "bf16", 1),
    (2, 700, 32, 8, 128, 1, 0, 0, "bf16", 0),
    (1, 640, 64, 8, 128, 1, 128, 0, "bf16", 1),
    # d_h = 128 with heads packed 4 to a workgroup: S = 1 and 2, non-causal,
    # W = 1, G = 16, positions near 65535
    (1, 1, 4, 1, 128, 1, 0, 0, "bf16", 1),
    (1, 2, 8, 1, 128, 1, 0, 3, "bf16", 1),
    (1, 129, 4, 1, 128, 0, 0, 0, "bf16", 1),
    (3, 333, 12, 3, 128, 1, 1, 0, "bf16", 1),
    (1, 100, 32, 2, 128, 1, 0, 0, "bf16", 1),
    (2, 96, 16, 4, 128, 0, 0, 0, "bf16", 0),
    (1, 1000, 64, 4, 128, 1, 0, 0, "bf16", 1),
    (1, 577, 8, 1, 128, 1, 200, 65535 - 600, "bf16", 1),
    (1, 128, 4, 2, 64, 1, 0, 0, "f32", 1),
    (1, 77, 4, 1, 128, 1, 9, 5, "f32", 1),
    (2, 33, 2, 2, 64, 0, 0, 0, "f32", 1),
    (1, 300, 8, 2, 128, 1, 0, 0, "f32", 0),
    # many batch elements of a short sequence: the flat work-item index of the
    # bf16 prefill and the batch grid dimension of the fp32 one
    (1500, 3, 8, 2, 128, 1, 0, 0, "bf16", 1),
    (700, 5, 4, 4, 64, 1, 2, 11, "bf16", 1),
    (1200, 2, 4, 1, 64, 1, 0, 0, "f32", 1),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_small(taa, case):
    B, S, Hq, Hkv, d, causal, W, m0, dtype, rope = case
    _say("prefill", case)
    q, k, v = apex_inputs.prefill_inputs(B, S, Hq, Hkv, d, dtype, seed=S + Hq, device="cuda")
    o = torch.empty_like(q)
    kr = torch.empty_like(k)
    taa.apex_attn_prefill(q, k, v, o, kr, causal=causal, W=W, m0=m0, apply_rope=rope)
    torch.cuda.synchronize()
    ref = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), causal=causal, W=W, m0=m0, apply_rope=rope)
    _check(o, ref, dtype, "prefill %s" % (case,))


PREFIX_CASES = [
    # B, S, Hq, Hkv, d, W, prefix, dtype -- prefix-bidirectional regime
    (1, 100, 4, 2, 128, 0, 37, "bf16"),
    (1, 300, 8, 2, 128, 0, 129, "bf16"),     # the prefix ends inside a key tile
    (1, 300, 8, 8, 64, 0, 300, "bf16"),      # all prefix: bidirectional attention
    (2, 513, 16, 4, 128, 64, 200, "bf16"),   # window after the prefix, ragged tail
    (1, 257, 4, 1, 128, 16, 1, "bf16"),      # P = 1: the causal mask
    (1, 1000, 32, 8, 128, 300, 520, "bf16"),
    (1, 640, 64, 8, 128, 128, 64, "bf16"),
    (1, 500, 16, 2, 128, 50, 77, "bf16"),
    (1, 70, 4, 1, 128, 0, 70, "bf16"),
    (1, 130, 4, 2, 64, 0, 45, "f32"),
    (1, 77, 4, 1, 128, 9, 20, "f32"),
]


@pytest.mark.parametrize("case", PREFIX_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_prefix(taa, case):
    B, S, Hq, Hkv, d, W, P, dtype = case
    _say("prefill prefix", case)
    q, k, v = apex_inputs.prefill_inputs(B, S, Hq, Hkv, d, dtype, seed=S + P, device="cuda")
    o = torch.empty_like(q)
    kr = torch.empty_like(k)
    taa.apex_attn_prefill(q, k, v, o, kr, causal=1, W=W, prefix=P, apply_rope=1)
    torch.cuda.synchronize()
    ref = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), causal=1, W=W, prefix=P)
    _check(o, ref, dtype, "prefill prefix %s" % (case,))


YARN_CASES = [
    # B, S, Hq, Hkv, d, W, m0, yarn_s, apply_rope, dtype
    (1, 300, 8, 2, 128, 0, 5000, 4.0, 1, "bf16"),
    (2, 129, 4, 1, 64, 50, 100000, 64.0, 1, "bf16"),
    (1, 200, 8, 8, 128, 0, 0, 8.0, 0, "bf16"),   # temperature only: q, k given rotated
    (1, 77, 4, 2, 64, 0, 30000, 40.0, 1, "f32"),
]


@pytest.mark.parametrize("case", YARN_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_yarn(taa, case):
    B, S, Hq, Hkv, d, W, m0, ys, rope, dtype = case
    _say("prefill yarn", case)
    q, k, v = apex_inputs.prefill_inputs(B, S, Hq, Hkv, d, dtype, seed=S + 3, device="cuda")
    o = torch.empty_like(q)
    kr = torch.empty_like(k)
    taa.apex_attn_prefill(q, k, v, o, kr, causal=1, W=W, m0=m0, apply_rope=rope, yarn_s=ys)
    torch.cuda.synchronize()
    ref = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), causal=1, W=W, m0=m0, apply_rope=rope,
                         yarn_s=ys)
    _check(o, ref, dtype, "prefill yarn %s" % (case,))


# Scores built to move the running row max: every query's dim 0 is A and key
# j's dim 0 is c * (j // 64), so in log2 units q.k / sqrt(d_h) steps by `jump`
# from one 64-key tile to the next (past the kernels' lazy-rescale headroom of
# 8 when |jump| > 8); the other dims carry a small noise. Inputs are given
# rotated (apply_rope = 0) so the designed scores are the scores.
GROW_CASES = [
    # B, S, Hq, Hkv, d, W, jump, dtype
    (1, 300, 4, 2, 128, 0, 9.0, "bf16"),     # the max moves on every tile
    (1, 300, 4, 2, 128, 100, 9.0, "bf16"),   # ... inside a window that spans tiles
    (1, 200, 4, 1, 64, 0, 9.0, "bf16"),
    (1, 300, 4, 2, 128, 0, -9.0, "bf16"),    # falling scores: the first tile holds the max
    (1, 300, 8, 2, 128, 0, 30.0, "bf16"),    # jumps far past the headroom
    (1, 300, 4, 2, 128, 0, 9.0, "f32"),
    (1, 300, 8, 2, 128, 0, 9.0, "bf16"),     # 4 heads per workgroup: rising,
    (1, 300, 16, 2, 128, 100, 9.0, "bf16"),  # ... in a window,
    (1, 300, 8, 2, 128, 0, -9.0, "bf16"),    # ... falling,
    (1, 300, 32, 4, 128, 0, 30.0, "bf16"),   # ... far past the headroom
]


@pytest.mark.parametrize("case", GROW_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_running_max_moves(taa, case):
    B, S, Hq, Hkv, d, W, jump, dtype = case
    _say("prefill running max", case)
    q, k, v = apex_inputs.prefill_inputs(B, S, Hq, Hkv, d, dtype, seed=77, device="cuda")
    A = 8.0
    c = jump * math.sqrt(d) / (A * math.log2(math.e))
    q, k = q * 0.05, k * 0.05
    q[..., 0] = A
    k[..., 0] = (c * (torch.arange(S, device="cuda") // 64).float()).to(k.dtype)
    o = torch.empty_like(q)
    taa.apex_attn_prefill(q, k, v, o, None, causal=1, W=W, apply_rope=0)
    torch.cuda.synchronize()
    ref = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), causal=1, W=W, apply_rope=0)
    _check(o, ref, dtype, "prefill running max %s" % (case,))


def test_k_rope_out_holds_rotated_keys_and_may_alias_k(taa):
    B, S, Hq, Hkv, d = 1, 200, 8, 2, 128
    q, k, v = apex_inputs.prefill_inputs(B, S, Hq, Hkv, d, "bf16", seed=5, device="cuda")
    o1, kr = torch.empty_like(q), torch.empty_like(k)
    taa.apex_attn_prefill(q, k, v, o1, kr, W=50, m0=3)
    k2 = k.clone()
    taa.apex_rope_qk(k2, None, m0=3)  # rotates its first argument only
    torch.cuda.synchronize()
    assert torch.equal(kr, k2)  # same kernel, same bits
    o2 = torch.empty_like(q)
    k3 = k.clone()
    taa.apex_attn_prefill(q, k3, v, o2, k3, W=50, m0=3)  # rotate in place
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(k3, kr)


def test_fused_rope_agrees_with_prerotated_inputs(taa):
    B, S, Hq, Hkv, d = 1, 333, 16, 4, 128
    q, k, v = apex_inputs.prefill_inputs(B, S, Hq, Hkv, d, "bf16", seed=6, device="cuda")
    o_fused, kr = torch.empty_like(q), torch.empty_like(k)
    taa.apex_attn_prefill(q, k, v, o_fused, kr, m0=40000)
    qr, kr2 = q.clone(), k.clone()
    taa.apex_rope_qk(qr, kr2, m0=40000)
    o_pre = torch.empty_like(q)
    taa.apex_attn_prefill(qr, kr2, v, o_pre, None, m0=40000, apply_rope=0)
    torch.cuda.synchronize()
    ref = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), m0=40000)
    _check(o_fused, ref, "bf16", "fused RoPE")
    _check(o_pre, ref, "bf16", "pre-rotated")


# ------------------------------------------------------------------ MLA ----
MLA_CASES = [
    # B, S, Hq, Hkv, causal, W, prefix, m0, yarn_s, apply_rope -- d_h 128, d_r 64
    (1, 1, 2, 1, 1, 0, 0, 0, 1.0, 1),
    (1, 3, 4, 4, 1, 0, 0, 9, 1.0, 1),
    (1, 65, 8, 2, 1, 0, 0, 0, 1.0, 1),
    (2, 300, 16, 4, 1, 0, 0, 1000, 1.0, 1),
    (1, 513, 8, 8, 0, 0, 0, 0, 1.0, 1),        # no mask, ragged tail
    (1, 700, 32, 8, 1, 128, 0, 0, 1.0, 1),     # a window, tile skipping
    (1, 640, 64, 8, 1, 0, 200, 0, 1.0, 1),     # prefix-bidirectional
    (1, 257, 8, 2, 1, 0, 0, 20000, 8.0, 1),    # YaRN frequencies over d_r, temperature
    (1, 200, 8, 2, 1, 0, 0, 0, 1.0, 0),        # q, k given rotated
]


@pytest.mark.parametrize("case", MLA_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_mla(taa, case):
    B, S, Hq, Hkv, causal, W, P, m0, ys, rope = case
    _say("prefill mla", case)
    q, k, v = apex_inputs.mla_prefill_inputs(B, S, Hq, Hkv, 128, 64, "bf16", seed=S + Hq + 1,
                                             device="cuda")
    o = torch.empty(B, Hq, S, 128, dtype=torch.bfloat16, device="cuda")
    kr = torch.empty_like(k)
    taa.apex_attn_prefill_mla(q, k, v, o, kr, causal=causal, W=W, prefix=P, m0=m0,
                              apply_rope=rope, yarn_s=ys)
    torch.cuda.synchronize()
    ref = oracle.prefill_mla(q.cpu(), k.cpu(), v.cpu(), 64, causal=causal, W=W, prefix=P, m0=m0,
                             apply_rope=rope, yarn_s=ys)
    _check(o, ref, "bf16", "prefill mla %s" % (case,))


def test_mla_rope_buffer_rotates_only_the_rope_part(taa):
    B, S, Hq, Hkv = 1, 130, 4, 2
    q, k, v = apex_inputs.mla_prefill_inputs(B, S, Hq, Hkv, 128, 64, "bf16", seed=12,
                                             device="cuda")
    o1 = torch.empty(B, Hq, S, 128, dtype=torch.bfloat16, device="cuda")
    kr = torch.empty_like(k)
    taa.apex_attn_prefill_mla(q, k, v, o1, kr, m0=77)
    torch.cuda.synchronize()
    assert torch.equal(kr[..., :128], k[..., :128])  # content part copied bit for bit
    kr_rope = kr[..., 128:].double().cpu().numpy()
    k_rope = k[..., 128:].double().cpu().numpy()
    for h in range(Hkv):
        for s_ in range(S):
            want = oracle.rope_row(k_rope[0, h, s_], 77 + s_)
            assert np.all(np.abs(kr_rope[0, h, s_] - want) <= np.abs(want) * 2.0 ** -8 + 1e-6)
    o2 = torch.empty_like(o1)
    k2 = k.clone()
    taa.apex_attn_prefill_mla(q, k2, v, o2, k2, m0=77)  # in place: only the rope part moves
    torch.cuda.synchronize()
    assert torch.equal(k2, kr) and torch.equal(o1, o2)


# ------------------------------------------------------ full workloads ----
def _run_prefill_workload(taa, name, n_random):
    w = apex_inputs.WORKLOADS[name]
    _say("workload", name, w)
    q, k, v = apex_inputs.workload_inputs(name, device="cuda")
    o, kr = torch.empty_like(q), torch.empty_like(k)
    P, ys = w.get("prefix", 0), w.get("yarn_s", 1.0)
    taa.apex_attn_prefill(q, k, v, o, kr, causal=w["causal"], W=w["W"], m0=w["m0"],
                          base=w["base"], apply_rope=1, prefix=P, yarn_s=ys)
    torch.cuda.synchronize()
    B, Hq, S, d = q.shape
    if n_random is None:
        ref = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), causal=w["causal"], W=w["W"],
                             m0=w["m0"], base=w["base"], prefix=P, yarn_s=ys)
        return _check(o, ref, w["dtype"], name)
    rows = _rows(B, Hq, S, n_random, seed=w["seed"])
    ref = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), causal=w["causal"], W=w["W"], m0=w["m0"],
                         base=w["base"], rows=rows, prefix=P, yarn_s=ys)
    got = o.reshape(-1, d)[torch.from_numpy(rows).to(o.device)]
    return _check(got, ref, w["dtype"], "%s (%d sampled rows)" % (name, rows.size))


class _Stats:
    """Running max-abs and mean-abs of |gpu - oracle| over streamed chunks."""

    def __init__(self):
        self.mx, self.sum, self.n = 0.0, 0.0, 0

    def add(self, got, ref, what):
        got = got.detach().to("cpu", torch.float64).numpy().reshape(ref.shape)
        assert np.all(np.isfinite(got)), what
        err = np.abs(got - ref)
        self.mx = max(self.mx, float(err.max()))
        self.sum += float(err.sum())
        self.n += err.size

    def check(self, dtype, what):
        mean = self.sum / self.n
        _say("%s: max_abs %.3g mean_abs %.3g (all %d values)" % (what, self.mx, mean, self.n))
        assert self.mx <= TOL[dtype]["max_abs"], (what, self.mx)
        assert mean <= TOL[dtype]["mean_abs"], (what, mean)


def _run_prefill_workload_full(taa, name, part=0, nparts=1):
    """Every output row of the (b, KV group) chunks in part `part` of `nparts`
    (chunks dealt round-robin), each chunk's reference computed on its own."""
    w = apex_inputs.WORKLOADS[name]
    _say("workload", name, "part %d/%d" % (part + 1, nparts), w)
    q, k, v = apex_inputs.workload_inputs(name, device="cuda")
    B, Hq, S, _ = q.shape
    mla = w["kind"] == "mla_prefill"
    o = torch.empty(B, Hq, S, v.shape[3], dtype=q.dtype, device="cuda")
    kr = torch.empty_like(k)
    P, ys = w.get("prefix", 0), w.get("yarn_s", 1.0)
    if mla:
        taa.apex_attn_prefill_mla(q, k, v, o, kr, causal=w["causal"], W=w["W"], m0=w["m0"],
                                  base=w["base"])
    else:
        taa.apex_attn_prefill(q, k, v, o, kr, causal=w["causal"], W=w["W"], m0=w["m0"],
                              base=w["base"], apply_rope=1, prefix=P, yarn_s=ys)
    torch.cuda.synchronize()
    Hkv = k.shape[1]
    G = Hq // Hkv
    chunks = [(b, g) for b in range(B) for g in range(Hkv)][part::nparts]
    stats = _Stats()
    for b, g in chunks:
        qc, kc, vc = (x[b:b + 1].cpu() for x in (q, k, v))
        heads = range(g * G, (g + 1) * G)
        rows = np.array([h * S + i for h in heads for i in range(S)], dtype=np.int64)
        if mla:
            ref = oracle.prefill_mla(qc, kc, vc, w["d_r"], causal=w["causal"], W=w["W"],
                                     m0=w["m0"], base=w["base"], rows=rows)
        else:
            ref = oracle.prefill(qc, kc, vc, causal=w["causal"], W=w["W"], m0=w["m0"],
                                 base=w["base"], rows=rows, prefix=P, yarn_s=ys)
        stats.add(o[b, g * G:(g + 1) * G], ref, "%s b %d group %d" % (name, b, g))
    stats.check(w["dtype"], "%s part %d/%d (%d chunks of %d heads x %d rows)"
                % (name, part + 1, nparts, len(chunks), G, S))


def test_workload_tiny_prefill_f32(taa):
    _run_prefill_workload_full(taa, "tiny_prefill_f32")


def test_workload_gqa_prefill_s2048(taa):
    _run_prefill_workload_full(taa, "gqa_prefill_s2048")


def test_workload_gqa_prefill_s2048_sampled_tile_edges(taa):
    _run_prefill_workload(taa, "gqa_prefill_s2048", 3000)


@pytest.mark.parametrize("part", range(4))
def test_workload_window_prefill_s16384_w4096(taa, part):
    _run_prefill_workload_full(taa, "window_prefill_s16384_w4096", part, 4)


@pytest.mark.parametrize("part", range(4))
def test_workload_local_prefill_s65536_w512(taa, part):
    _run_prefill_workload_full(taa, "local_prefill_s65536_w512", part, 4)


@pytest.mark.parametrize("part", range(4))
def test_workload_yarn_local_prefill_s32768_w4096_s4(taa, part):
    _run_prefill_workload_full(taa, "yarn_local_prefill_s32768_w4096_s4", part, 4)


def test_workload_yarn_local_prefill_s32768_w4096_s4_sampled(taa):
    _run_prefill_workload(taa, "yarn_local_prefill_s32768_w4096_s4", 2000)


def test_workload_prefix_prefill_s2048_p512(taa):
    _run_prefill_workload_full(taa, "prefix_prefill_s2048_p512")


@pytest.mark.parametrize("part", range(4))
def test_workload_prefix_local_prefill_s16384_w4096_p1024(taa, part):
    _run_prefill_workload_full(taa, "prefix_local_prefill_s16384_w4096_p1024", part, 4)


def test_workload_prefix_local_prefill_s16384_w4096_p1024_sampled(taa):
    _run_prefill_workload(taa, "prefix_local_prefill_s16384_w4096_p1024", 1500)


@pytest.mark.parametrize("part", range(8))
def test_workload_mla_global_prefill_s16384(taa, part):
    _run_prefill_workload_full(taa, "mla_global_prefill_s16384", part, 8)


def test_workload_mla_global_prefill_s16384_sampled(taa):
    name = "mla_global_prefill_s16384"
    w = apex_inputs.WORKLOADS[name]
    _say("workload", name, w)
    q, k, v = apex_inputs.workload_inputs(name, device="cuda")
    B, Hq, S, _ = q.shape
    o = torch.empty(B, Hq, S, w["d"], dtype=q.dtype, device="cuda")
    kr = torch.empty_like(k)
    taa.apex_attn_prefill_mla(q, k, v, o, kr, causal=w["causal"], W=w["W"], m0=w["m0"],
                              base=w["base"])
    torch.cuda.synchronize()
    rows = _rows(B, Hq, S, 1500, seed=w["seed"])
    ref = oracle.prefill_mla(q.cpu(), k.cpu(), v.cpu(), w["d_r"], causal=w["causal"], W=w["W"],
                             m0=w["m0"], base=w["base"], rows=rows)
    got = o.reshape(-1, w["d"])[torch.from_numpy(rows).to(o.device)]
    _check(got, ref, w["dtype"], "%s (%d sampled rows)" % (name, rows.size))


# ------------------------------------------ offsets past 2 GiB per head ----
BIG_S = 12_000_000  # one head of 256-byte rows spans 3.07 GB; rows past 2**23 lie beyond 2**31 bytes


def test_prefill_rows_beyond_2_gib_in_one_head(taa):
    # The prefill addresses a head's rows through 32-bit buffer offsets, which
    # must stay unsigned up to the 4 GiB the boundary accepts; RoPE runs at
    # positions up to 12e6. With a 64-key window a row depends only on the 64
    # rows up to it, so the oracle runs on short slices around rows on both
    # sides of byte offset 2**31 (m0 = the slice's first row).
    S, W, d = BIG_S, 64, 128
    _say("prefill beyond 2 GiB per head", S, W)
    q, k, v = apex_inputs.prefill_inputs(1, S, 1, 1, d, "bf16", seed=91, device="cuda")
    o, kr = torch.empty_like(q), torch.empty_like(k)
    taa.apex_attn_prefill(q, k, v, o, kr, causal=1, W=W, apply_rope=1)
    torch.cuda.synchronize()
    stats = _Stats()
    for c in (100, 4_000_000, (1 << 23) - 1, 1 << 23, (1 << 23) + 1, 10_000_000, S - 1):
        lo, hi = max(0, c - 255), min(S, c + 129)
        ref = oracle.prefill(q[:, :, lo:hi].cpu(), k[:, :, lo:hi].cpu(), v[:, :, lo:hi].cpu(),
                             causal=1, W=W, m0=lo)
        first = 0 if lo == 0 else W - 1  # rows whose whole window lies in the slice
        stats.add(o[:, :, lo + first:hi], ref[:, :, first:], "rows %d..%d" % (lo + first, hi - 1))
        # the rotated keys written out at these positions
        x = k[0, 0, c].cpu().double().numpy()
        want = oracle.rope_row(x, c)
        got = kr[0, 0, c].cpu().double().numpy()
        assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -8 + 1e-6), c
    stats.check("bf16", "prefill S=%d W=%d around byte offset 2**31" % (S, W))


def test_prefill_mla_rows_beyond_2_gib_in_one_head(taa):
    # MLA key rows are 384 bytes, so one head of 8e6 rows spans 3.07 GB and rows
    # past 5,592,405 lie beyond byte offset 2**31; windowed, checked on slices.
    S, W = 8_000_000, 64
    _say("mla prefill beyond 2 GiB per head", S, W)
    q, k, v = apex_inputs.mla_prefill_inputs(1, S, 1, 1, 128, 64, "bf16", seed=93, device="cuda")
    o = torch.empty(1, 1, S, 128, dtype=q.dtype, device="cuda")
    kr = torch.empty_like(k)
    taa.apex_attn_prefill_mla(q, k, v, o, kr, causal=1, W=W)
    torch.cuda.synchronize()
    edge = (1 << 31) // 384
    stats = _Stats()
    for c in (100, 3_000_000, edge - 1, edge, edge + 1, S - 1):
        lo, hi = max(0, c - 255), min(S, c + 129)
        ref = oracle.prefill_mla(q[:, :, lo:hi].cpu(), k[:, :, lo:hi].cpu(), v[:, :, lo:hi].cpu(),
                                 64, causal=1, W=W, m0=lo)
        first = 0 if lo == 0 else W - 1
        stats.add(o[:, :, lo + first:hi], ref[:, :, first:], "rows %d..%d" % (lo + first, hi - 1))
        x = k[0, 0, c].cpu().double().numpy()
        got = kr[0, 0, c].cpu().double().numpy()
        assert np.array_equal(got[:128], x[:128]), c  # the content part is copied
        want = oracle.rope_row(x[128:], c)
        assert np.all(np.abs(got[128:] - want) <= np.abs(want) * 2.0 ** -8 + 1e-6), c
    stats.check("bf16", "mla prefill S=%d W=%d around byte offset 2**31" % (S, W))


def test_prefill_f32_rows_beyond_2_gib_in_one_head(taa):
    # The fp32 path: one head of 12e6 rows of 64 floats (3.07 GB).
    S, W, d = BIG_S, 64, 64
    _say("f32 prefill beyond 2 GiB per head", S, W)
    q, k, v = apex_inputs.prefill_inputs(1, S, 1, 1, d, "f32", seed=94, device="cuda")
    o, kr = torch.empty_like(q), torch.empty_like(k)
    taa.apex_attn_prefill(q, k, v, o, kr, causal=1, W=W, apply_rope=1)
    torch.cuda.synchronize()
    stats = _Stats()
    for c in (100, (1 << 23) - 1, 1 << 23, (1 << 23) + 1, S - 1):
        lo, hi = max(0, c - 255), min(S, c + 129)
        ref = oracle.prefill(q[:, :, lo:hi].cpu(), k[:, :, lo:hi].cpu(), v[:, :, lo:hi].cpu(),
                             causal=1, W=W, m0=lo)
        first = 0 if lo == 0 else W - 1
        stats.add(o[:, :, lo + first:hi], ref[:, :, first:], "rows %d..%d" % (lo + first, hi - 1))
    stats.check("f32", "f32 prefill S=%d W=%d around byte offset 2**31" % (S, W))


@pytest.mark.parametrize("m", [(1 << 23) + 10, BIG_S - 1])
def test_decode_slots_beyond_2_gib_in_one_head(taa, m):
    # A cache of 12e6 slots per (b, KV head); with a 64-slot window the visible
    # slots m-63 .. m straddle byte offset 2**31 (m = 2**23 + 10) or lie past it.
    # Without RoPE (inputs taken as already rotated) positions drop out of the
    # arithmetic, so the oracle runs on the visible slice alone.
    Sk, W, d, Hq = BIG_S, 64, 128, 16
    _say("decode beyond 2 GiB per head", Sk, W, m)
    q, kc, vc, kn, vn = apex_inputs.decode_inputs(1, Sk, Hq, 1, d, "bf16", seed=92,
                                                  device="cuda")
    lo = m - W + 1
    kc0, vc0 = kc[:, :, lo:m + 1].cpu(), vc[:, :, lo:m + 1].cpu()
    o = torch.empty_like(q)
    ws = torch.empty(taa.apex_attn_decode_workspace_bytes(1, Hq, 1, Sk, d), dtype=torch.uint8,
                     device="cuda")
    taa.apex_attn_decode(q, kc, vc, kn, vn, o, m=m, W=W, apply_rope=0, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.decode(q.cpu(), kc0, vc0, kn.cpu(), vn.cpu(), m=W - 1, W=W, apply_rope=False)
    _check(o, ref, "bf16", "decode Sk=%d W=%d m=%d" % (Sk, W, m))
    assert torch.equal(kc[:, :, m], kn[:, :, 0]) and torch.equal(vc[:, :, m], vn[:, :, 0])
    assert torch.equal(kc[:, :, lo:m].cpu(), kc0[:, :, :-1])  # the other visible slots untouched


# --------------------------------------------------------------- decode ----
DECODE_CASES = [
    # B, Sk, Hq, Hkv, d, W, m, with_new, apply_rope
    (1, 1, 16, 1, 128, 0, 0, True, 1),
    (2, 5, 4, 1, 128, 0, 4, True, 1),
    (1, 33, 16, 1, 64, 0, 20, True, 1),
    (2, 100, 32, 2, 128, 7, 99, True, 1),
    (1, 1000, 8, 8, 128, 64, 999, False, 0),
    (1, 5000, 64, 2, 128, 0, 4321, True, 1),
    (3, 4096, 12, 4, 64, 100, 4095, True, 1),
    (2, 20000, 16, 1, 128, 0, 19999, True, 1),
    # many batch elements of a short cache (the batch grid dimension)
    (2000, 40, 16, 2, 128, 0, 39, True, 1),
    (3000, 64, 8, 8, 64, 16, 50, True, 1),
]


def _decode_inputs(B, Sk, Hq, Hkv, d, seed):
    return apex_inputs.decode_inputs(B, Sk, Hq, Hkv, d, "bf16", seed=seed, device="cuda")


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_small(taa, case):
    B, Sk, Hq, Hkv, d, W, m, with_new, rope = case
    _say("decode", case)
    q, kc, vc, kn, vn = _decode_inputs(B, Sk, Hq, Hkv, d, seed=Sk + Hq)
    if not with_new:
        kn = vn = None
    kc0, vc0 = kc.cpu(), vc.cpu()
    o = torch.empty_like(q)
    ws = torch.empty(taa.apex_attn_decode_workspace_bytes(B, Hq, Hkv, Sk, d), dtype=torch.uint8,
                     device="cuda")
    taa.apex_attn_decode(q, kc, vc, kn, vn, o, m=m, W=W, apply_rope=rope, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.decode(q.cpu(), kc0, vc0, kn.cpu() if with_new else None,
                        vn.cpu() if with_new else None, m=m, W=W, apply_rope=rope)
    _check(o, ref, "bf16", "decode %s" % (case,))
    kc1, vc1 = kc.cpu(), vc.cpu()
    other = torch.ones(Sk, dtype=torch.bool)
    other[m] = False
    assert torch.equal(kc1[:, :, other], kc0[:, :, other])  # only slot m may change
    assert torch.equal(vc1[:, :, other], vc0[:, :, other])
    if with_new:
        assert torch.equal(vc1[:, :, m], vn.cpu()[:, :, 0])
        x = kn.cpu().double().numpy()[:, :, 0]
        want = np.array([[oracle.rope_row(x[b, h], m) if rope else x[b, h] for h in range(Hkv)]
                         for b in range(B)])
        got = kc1[:, :, m].double().numpy()
        assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -8 + 1e-6)


@pytest.mark.parametrize("ys", [4.0, 64.0])
def test_decode_yarn(taa, ys):
    B, Sk, Hq, Hkv, d, m = 2, 3000, 16, 2, 128, 2999
    _say("decode yarn", ys)
    q, kc, vc, kn, vn = _decode_inputs(B, Sk, Hq, Hkv, d, seed=17)
    kc0, vc0 = kc.cpu(), vc.cpu()
    o = torch.empty_like(q)
    ws = torch.empty(taa.apex_attn_decode_workspace_bytes(B, Hq, Hkv, Sk, d), dtype=torch.uint8,
                     device="cuda")
    taa.apex_attn_decode(q, kc, vc, kn, vn, o, m=m, workspace=ws, yarn_s=ys)
    torch.cuda.synchronize()
    ref = oracle.decode(q.cpu(), kc0, vc0, kn.cpu(), vn.cpu(), m=m, yarn_s=ys)
    _check(o, ref, "bf16", "decode yarn %s" % ys)


# Cached keys whose scores step by `jump` (log2 units) every 32 slots, so the
# running max of every split part moves and the parts' maxima differ widely
# before the log-sum-exp combine; q and the cache are given rotated.
@pytest.mark.parametrize("jump", [9.0, -9.0, 30.0])
def test_decode_running_max_moves(taa, jump):
    B, Sk, Hq, Hkv, d = 2, 9000, 16, 2, 128
    _say("decode running max", jump)
    q, kc, vc, _, _ = _decode_inputs(B, Sk, Hq, Hkv, d, seed=91)
    A = 8.0
    c = jump * math.sqrt(d) / (A * math.log2(math.e))
    q, kc = q * 0.05, kc * 0.05
    q[..., 0] = A
    steps = (torch.arange(Sk, device="cuda") // 32).float()
    kc[..., 0] = (c * (steps - steps.max() / 2) / 10).to(kc.dtype)  # ramps over the cache
    o = torch.empty_like(q)
    ws = torch.empty(taa.apex_attn_decode_workspace_bytes(B, Hq, Hkv, Sk, d), dtype=torch.uint8,
                     device="cuda")
    taa.apex_attn_decode(q, kc, vc, None, None, o, m=Sk - 1, apply_rope=0, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.decode(q.cpu(), kc.cpu(), vc.cpu(), None, None, m=Sk - 1, apply_rope=0)
    _check(o, ref, "bf16", "decode running max %s" % jump)


def test_decode_repeat_is_idempotent(taa):
    B, Sk, Hq, Hkv, d = 2, 3000, 32, 2, 128
    q, kc, vc, kn, vn = _decode_inputs(B, Sk, Hq, Hkv, d, seed=77)
    ws = torch.empty(taa.apex_attn_decode_workspace_bytes(B, Hq, Hkv, Sk, d), dtype=torch.uint8,
                     device="cuda")
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    taa.apex_attn_decode(q, kc, vc, kn, vn, o1, m=Sk - 1, workspace=ws)
    taa.apex_attn_decode(q, kc, vc, kn, vn, o2, m=Sk - 1, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("Sk,fused", [(1500, True), (6000, False)])
def test_decode_workspace_use_follows_the_split(taa, Sk, fused):
    # With the keys of a (b, KV head) in two parts (one workgroup) the split
    # pass merges them itself and leaves the workspace untouched; with more
    # parts the partials go through the workspace to the combine kernel.
    # Either way the output matches the oracle.
    B, Hq, Hkv, d = 1, 16, 1, 128
    q, kc, vc, kn, vn = _decode_inputs(B, Sk, Hq, Hkv, d, seed=91)
    kc0, vc0 = kc.cpu(), vc.cpu()
    ws = torch.full((taa.apex_attn_decode_workspace_bytes(B, Hq, Hkv, Sk, d),), 0x5A,
                    dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    taa.apex_attn_decode(q, kc, vc, kn, vn, o, m=Sk - 1, workspace=ws)
    torch.cuda.synchronize()
    untouched = bool((ws == 0x5A).all().item())
    assert untouched == fused
    ref = oracle.decode(q.cpu(), kc0, vc0, kn.cpu(), vn.cpu(), m=Sk - 1)
    _check(o, ref, "bf16", "decode Sk=%d, merged in the split pass: %s" % (Sk, fused))


def test_decode_equals_last_prefill_row(taa):
    B, S, Hq, Hkv, d = 1, 1500, 32, 2, 128
    q, k, v = apex_inputs.prefill_inputs(B, S, Hq, Hkv, d, "bf16", seed=8, device="cuda")
    o, kr = torch.empty_like(q), torch.empty_like(k)
    taa.apex_attn_prefill(q, k, v, o, kr)
    kc, vc = kr.clone(), v.clone()
    kc[:, :, S - 1].zero_()  # slot m comes from k_new / v_new
    vc[:, :, S - 1].zero_()
    od = torch.empty(B, Hq, 1, d, dtype=q.dtype, device=q.device)
    ws = torch.empty(taa.apex_attn_decode_workspace_bytes(B, Hq, Hkv, S, d), dtype=torch.uint8,
                     device="cuda")
    taa.apex_attn_decode(q[:, :, S - 1:].contiguous(), kc, vc, k[:, :, S - 1:].contiguous(),
                         v[:, :, S - 1:].contiguous(), od, m=S - 1, workspace=ws)
    torch.cuda.synchronize()
    diff = (od[:, :, 0].float() - o[:, :, S - 1].float()).abs().max().item()
    _say("decode vs prefill last row: max_abs %.3g" % diff)
    assert diff <= 2e-2


def test_workload_gqa_decode_sk32768(taa):
    name = "gqa_decode_sk32768"
    w = apex_inputs.WORKLOADS[name]
    _say("workload", name, w)
    q, kc, vc, kn, vn = apex_inputs.workload_inputs(name, device="cuda")
    B, Hq, _, d = q.shape
    Hkv, Sk = kc.shape[1], kc.shape[2]
    o = torch.empty_like(q)
    ws = torch.empty(taa.apex_attn_decode_workspace_bytes(B, Hq, Hkv, Sk, d), dtype=torch.uint8,
                     device="cuda")
    taa.apex_attn_decode(q, kc, vc, kn, vn, o, m=w["m"], W=w["W"], base=w["base"], workspace=ws)
    torch.cuda.synchronize()
    # Every batch element, all heads. The call writes only slot m of the
    # caches, and with k_new / v_new given the oracle takes slot m from them,
    # so the caches read back after the call are the inputs it needs.
    stats = _Stats()
    for b in range(B):
        ref = oracle.decode(q[b:b + 1].cpu(), kc[b:b + 1].cpu(), vc[b:b + 1].cpu(),
                            kn[b:b + 1].cpu(), vn[b:b + 1].cpu(), m=w["m"], W=w["W"],
                            base=w["base"])
        stats.add(o[b:b + 1], ref, "%s batch %d" % (name, b))
    stats.check("bf16", "%s (all %d batch elements x %d heads)" % (name, B, Hq))


# ----------------------------------------------------------- MLA decode ----
MLA_DECODE_CASES = [
    # B, Sk, Hq, Hkv, W, m, with_new, apply_rope, yarn_s -- d_h 128, d_r 64
    (1, 1, 16, 1, 0, 0, True, 1, 1.0),
    (2, 40, 8, 2, 0, 39, True, 1, 1.0),
    (1, 1000, 32, 8, 100, 999, False, 0, 1.0),
    (2, 5000, 64, 4, 0, 3210, True, 1, 1.0),
    (1, 3000, 16, 2, 0, 2999, True, 1, 8.0),
]


@pytest.mark.parametrize("case", MLA_DECODE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_mla(taa, case):
    B, Sk, Hq, Hkv, W, m, with_new, rope, ys = case
    _say("decode mla", case)
    q, kc, vc, kn, vn = apex_inputs.mla_decode_inputs(B, Sk, Hq, Hkv, 128, 64, "bf16",
                                                      seed=Sk + Hq + 2, device="cuda")
    if not with_new:
        kn = vn = None
    kc0, vc0 = kc.cpu(), vc.cpu()
    o = torch.empty(B, Hq, 1, 128, dtype=q.dtype, device="cuda")
    ws = torch.empty(taa.apex_attn_decode_workspace_bytes(B, Hq, Hkv, Sk, 128),
                     dtype=torch.uint8, device="cuda")
    taa.apex_attn_decode_mla(q, kc, vc, kn, vn, o, m=m, W=W, apply_rope=rope, workspace=ws,
                             yarn_s=ys)
    torch.cuda.synchronize()
    ref = oracle.decode_mla(q.cpu(), kc0, vc0, kn.cpu() if with_new else None,
                            vn.cpu() if with_new else None, m=m, d_r=64, W=W, apply_rope=rope,
                            yarn_s=ys)
    _check(o, ref, "bf16", "decode mla %s" % (case,))
    kc1, vc1 = kc.cpu(), vc.cpu()
    other = torch.ones(Sk, dtype=torch.bool)
    other[m] = False
    assert torch.equal(kc1[:, :, other], kc0[:, :, other])  # only slot m may change
    assert torch.equal(vc1[:, :, other], vc0[:, :, other])
    if with_new:
        assert torch.equal(vc1[:, :, m], vn.cpu()[:, :, 0])
        x = kn.cpu().double().numpy()[:, :, 0]
        got = kc1[:, :, m].double().numpy()
        assert np.array_equal(got[..., :128], x[..., :128])  # content part stored as given
        want = np.array([[oracle.rope_row(x[b, h, 128:], m, yarn_s=ys) if rope else x[b, h, 128:]
                          for h in range(Hkv)] for b in range(B)])
        assert np.all(np.abs(got[..., 128:] - want) <= np.abs(want) * 2.0 ** -8 + 1e-6)


def test_decode_mla_equals_last_mla_prefill_row(taa):
    B, S, Hq, Hkv = 1, 1200, 32, 4
    q, k, v = apex_inputs.mla_prefill_inputs(B, S, Hq, Hkv, 128, 64, "bf16", seed=14,
                                             device="cuda")
    o = torch.empty(B, Hq, S, 128, dtype=q.dtype, device="cuda")
    kr = torch.empty_like(k)
    taa.apex_attn_prefill_mla(q, k, v, o, kr)
    kc, vc = kr.clone(), v.clone()
    kc[:, :, S - 1].zero_()  # slot m comes from k_new / v_new
    vc[:, :, S - 1].zero_()
    od = torch.empty(B, Hq, 1, 128, dtype=q.dtype, device=q.device)
    ws = torch.empty(taa.apex_attn_decode_workspace_bytes(B, Hq, Hkv, S, 128), dtype=torch.uint8,
                     device="cuda")
    taa.apex_attn_decode_mla(q[:, :, S - 1:].contiguous(), kc, vc, k[:, :, S - 1:].contiguous(),
                             v[:, :, S - 1:].contiguous(), od, m=S - 1, workspace=ws)
    torch.cuda.synchronize()
    diff = (od[:, :, 0].float() - o[:, :, S - 1].float()).abs().max().item()
    _say("mla decode vs prefill last row: max_abs %.3g" % diff)
    assert diff <= 2e-2


def test_workload_mla_global_decode_sk32768(taa):
    name = "mla_global_decode_sk32768"
    w = apex_inputs.WORKLOADS[name]
    _say("workload", name, w)
    q, kc, vc, kn, vn = apex_inputs.workload_inputs(name, device="cuda")
    B, Hq = q.shape[:2]
    Hkv, Sk = kc.shape[1], kc.shape[2]
    o = torch.empty(B, Hq, 1, w["d"], dtype=q.dtype, device="cuda")
    ws = torch.empty(taa.apex_attn_decode_workspace_bytes(B, Hq, Hkv, Sk, w["d"]),
                     dtype=torch.uint8, device="cuda")
    taa.apex_attn_decode_mla(q, kc, vc, kn, vn, o, m=w["m"], W=w["W"], base=w["base"],
                             workspace=ws)
    torch.cuda.synchronize()
    # Every batch element, all heads; as for the GQA decode, the caches read back
    # after the call differ from the inputs only in slot m, which the oracle
    # takes from k_new / v_new.
    stats = _Stats()
    for b in range(B):
        ref = oracle.decode_mla(q[b:b + 1].cpu(), kc[b:b + 1].cpu(), vc[b:b + 1].cpu(),
                                kn[b:b + 1].cpu(), vn[b:b + 1].cpu(), m=w["m"], d_r=w["d_r"],
                                W=w["W"], base=w["base"])
        stats.add(o[b:b + 1], ref, "%s batch %d" % (name, b))
    stats.check("bf16", "%s (all %d batch elements x %d heads)" % (name, B, Hq))


# -------------------------------------------------------------- RMSNorm ----
def _check_rmsnorm(got, ref, dtype, what):
    got = got.detach().to("cpu", torch.float64).numpy().reshape(ref.shape)
    err = np.abs(got - ref)
    if dtype == "bf16":
        # one rounding of y to bf16 (relative 2^-9) on top of fp32 arithmetic
        bound = np.abs(ref) * 2.0 ** -8 + 1e-30
        mean_rel = float(err.sum() / max(np.abs(ref).sum(), 1e-30))
        _say("%s: max rel %.3g mean rel %.3g" % (what, float((err / (np.abs(ref) + 1e-30)).max()),
                                                 mean_rel))
        assert mean_rel <= 2.0 ** -9, (what, mean_rel)  # rounding alone averages ~2^-10
    else:
        bound = np.abs(ref) * 2e-6 + 1e-6
        _say("%s: max abs %.3g" % (what, float(err.max())))
    assert np.all(np.isfinite(got)), what
    assert np.all(err <= bound), (what, float((err - bound).max()))


RMSNORM_CASES = [
    # rows, d, dtype, eps, in_place
    (1, 8, "bf16", 1e-6, False),
    (3, 520, "bf16", 1e-6, False),     # chunks not a multiple of the wave
    (257, 4096, "bf16", 1e-6, True),
    (100, 7168, "bf16", 1e-6, False),
    (5, 8192, "bf16", 0.0, False),
    (20000, 64, "bf16", 1e-6, False),  # more rows than resident waves: grid-stride
    (64, 512, "f32", 1e-6, False),
    (33, 1000, "f32", 0.25, True),
    (7, 8192, "f32", 1e-6, False),
]


@pytest.mark.parametrize("case", RMSNORM_CASES, ids=lambda c: "-".join(map(str, c)))
def test_rmsnorm(taa, case):
    rows, d, dtype, eps, in_place = case
    _say("rmsnorm", case)
    x, g = apex_inputs.rmsnorm_inputs(1, rows, d, dtype, seed=rows + d, device="cuda")
    x0 = x.cpu()
    y = taa.apex_rmsnorm(x, g, x if in_place else None, eps=eps)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(x0, g.cpu(), eps=eps)
    _check_rmsnorm(y, ref, dtype, "rmsnorm %s" % (case,))


def test_rmsnorm_zero_rows_with_eps(taa):
    x = torch.zeros(4, 256, dtype=torch.bfloat16, device="cuda")
    g = torch.ones(256, dtype=torch.bfloat16, device="cuda")
    y = taa.apex_rmsnorm(x, g, eps=1e-6)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0


@pytest.mark.parametrize("name", ["rmsnorm_b4_s2048_d7168", "rmsnorm_b64_s2048_d512"])
def test_workload_rmsnorm(taa, name):
    w = apex_inputs.WORKLOADS[name]
    _say("workload", name, w)
    x, g = apex_inputs.workload_inputs(name, device="cuda")
    y = taa.apex_rmsnorm(x, g, eps=w["eps"])
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(x.cpu(), g.cpu(), eps=w["eps"])
    _check_rmsnorm(y, ref, w["dtype"], name)


def test_rmsnorm_beyond_2g_elements(taa):
    # 300,000 rows of 8192 bf16 features: 2.46e9 elements (4.9 GB), rows from
    # 262,144 on starting past element 2**31.
    rows, d = 300_000, 8192
    _say("rmsnorm beyond 2**31 elements", rows, d)
    x, g = apex_inputs.rmsnorm_inputs(1, rows, d, "bf16", seed=95, device="cuda")
    y = taa.apex_rmsnorm(x, g, eps=1e-6)
    torch.cuda.synchronize()
    pick = torch.tensor([0, 1, (1 << 18) - 1, 1 << 18, (1 << 18) + 1, 280_001, rows - 1])
    ref = oracle.rmsnorm(x[0, pick.cuda()].cpu(), g.cpu(), eps=1e-6)
    _check_rmsnorm(y[0, pick.cuda()], ref, "bf16", "rmsnorm rows %s of %d" % (pick.tolist(), rows))


def test_calls_on_concurrent_streams_match_serial_calls(taa):
    # Every entry point only enqueues work on the stream it is given and keeps
    # no state between calls (the decode's partials live in the caller's
    # workspace), so calls on different streams may overlap freely.
    dev = torch.device("cuda")
    q, k, v = apex_inputs.prefill_inputs(2, 700, 16, 4, 128, "bf16", seed=31, device=dev)
    qd, kc, vc, kn, vn = apex_inputs.decode_inputs(8, 9000, 32, 2, 128, "bf16", seed=32,
                                                   device=dev)
    x, g = apex_inputs.rmsnorm_inputs(4, 3000, 4096, "bf16", seed=33, device=dev)
    ws = torch.empty(taa.apex_attn_decode_workspace_bytes(8, 32, 2, 9000, 128),
                     dtype=torch.uint8, device=dev)

    def run(streams):
        o, kr = torch.empty_like(q), torch.empty_like(k)
        od = torch.empty_like(qd)
        kc1, vc1 = kc.clone(), vc.clone()
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        taa.apex_attn_prefill(q, k, v, o, kr, causal=1, W=300, stream=streams[0])
        taa.apex_attn_decode(qd, kc1, vc1, kn, vn, od, m=8999, workspace=ws, stream=streams[1])
        taa.apex_rmsnorm(x, g, y, stream=streams[2])
        torch.cuda.synchronize()
        return o, kr, od, kc1, y

    serial = run([torch.cuda.current_stream()] * 3)
    side = [torch.cuda.Stream(device=dev) for _ in range(3)]  # default priority
    for _ in range(3):
        together = run(side)
        for a, b in zip(serial, together):
            assert torch.equal(a, b)


def test_calls_replay_from_a_hip_graph(taa):
    # Every entry point only enqueues kernels on the caller's stream and
    # allocates nothing, so a sequence of calls can be captured once and
    # replayed; each replay must reproduce the eager results bit for bit.
    B, S, Hq, Hkv, d = 1, 300, 8, 2, 128
    q, k, v = apex_inputs.prefill_inputs(B, S, Hq, Hkv, d, "bf16", seed=21, device="cuda")
    kr, o = torch.empty_like(k), torch.empty_like(q)
    Sk = 2048
    dq, kc, vc, kn, vn = _decode_inputs(2, Sk, 16, 2, d, seed=22)
    od = torch.empty_like(dq)
    ws = torch.empty(taa.apex_attn_decode_workspace_bytes(2, 16, 2, Sk, d), dtype=torch.uint8,
                     device="cuda")
    x = torch.randn(64, 512, device="cuda").to(torch.bfloat16)
    gam = torch.ones(512, device="cuda").to(torch.bfloat16)
    y = torch.empty_like(x)

    def calls():
        taa.apex_rope_qk(None, k, k_out=kr, m0=5)
        taa.apex_attn_prefill(q, kr, v, o, None, causal=1, W=100, m0=5, apply_rope=2)
        taa.apex_attn_decode(dq, kc, vc, None, None, od, m=Sk - 1, workspace=ws)
        taa.apex_rmsnorm(x, gam, y)

    calls()
    torch.cuda.synchronize()
    want = [t.clone() for t in (kr, o, od, y)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (kr, o, od, y):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip((kr, o, od, y), want):
            assert torch.equal(got, ref), rep
        calls()  # eager work between the replays
        torch.cuda.synchronize()
