"""Pins of the fp64 CPU oracle against what the pages and mathematics fix.

Sources (APEX-1 Mathematical Reference):
  Part 1 §4.2-§4.6  RoPE rotation, frequencies, compact form, relative-position
                    property, worked example at d_h = 4, position 3.
  Part 2 §6.2-§6.4  scaled dot-product attention, the 1/sqrt(d_h) argument and
                    the worked 2x3 example.
  Part 2 §8.2, §8.4 GQA head mapping and its H_q = 4, H_kv = 2 example.
  Part 2 §10.2      window mask formula;  §11.3 mask visual.

Each pin is chosen so that a plausible slip in the oracle (dropped scale, wrong
sign or pairing of the rotation, wrong exponent in theta_i, wrong KV-head index,
an off-by-one in the window, a transposed operand) fails at least one test.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest
import torch

import apex_inputs
import oracle
from oracle import pyref

RNG = np.random.default_rng(1234)


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


# --------------------------------------------------------------------------
# Scaled dot-product attention: worked example (Part 2, §6.4)
# --------------------------------------------------------------------------
def _sdpa_example_via_decode(g):
    Q, K, V = np.array(g["Q"], float), np.array(g["K"], float), np.array(g["V"], float)
    rows = []
    for qrow in Q:
        o = oracle.decode(_f32(qrow.reshape(1, 1, 1, 2)), _f32(K.reshape(1, 1, 3, 2)),
                          _f32(V.reshape(1, 1, 3, 2)), None, None, m=2, apply_rope=False)
        rows.append(o.reshape(2))
    return np.array(rows)


def test_sdpa_worked_example_closed_form(golden_dir):
    g = _golden(golden_dir, "sdpa_worked_example.json")
    out = _sdpa_example_via_decode(g)
    e = math.exp(1.0 / math.sqrt(2.0))
    # Row 0 weights (e, 1, e)/(1+2e) on V rows (1,2),(3,4),(5,6): exactly (3, 4).
    assert np.allclose(out[0], [3.0, 4.0], rtol=0, atol=1e-12)
    # Row 1 weights (1, e, e)/(1+2e): ((1+8e), (2+10e)) / (1+2e).
    assert np.allclose(out[1], [(1 + 8 * e) / (1 + 2 * e), (2 + 10 * e) / (1 + 2 * e)],
                       rtol=0, atol=1e-12)


def test_sdpa_worked_example_printed_values(golden_dir):
    g = _golden(golden_dir, "sdpa_worked_example.json")
    tol = 10.0 ** (-g["printed_decimals"])  # the page truncates/rounds to 3 decimals
    out = _sdpa_example_via_decode(g)
    assert np.max(np.abs(out - np.array(g["output"]))) <= tol
    py = pyref.sdpa(g["Q"], g["K"], g["V"])
    assert np.max(np.abs(np.array(py) - out)) <= 1e-12
    for r, qrow in enumerate(g["Q"]):
        _, p = pyref.sdpa_row(qrow, g["K"], g["V"])
        assert np.max(np.abs(np.array(p) - np.array(g["weights"][r]))) <= tol / 2
        assert abs(sum(p) - 1.0) <= 1e-12


def test_sdpa_scale_is_one_over_sqrt_dh(golden_dir):
    # A dropped or squared scale changes the example's row 1; pin it directly.
    g = _golden(golden_dir, "sdpa_worked_example.json")
    for r, qrow in enumerate(g["Q"]):
        scores = [sum(a * b for a, b in zip(qrow, k)) / math.sqrt(g["d_h"]) for k in g["K"]]
        assert np.allclose(scores, g["scaled_scores"][r], atol=5e-4)
        assert np.allclose(np.exp(scores), g["exp_scores"][r], atol=5e-4)


# --------------------------------------------------------------------------
# RoPE: worked example (Part 1, §4.6) and the rotation's properties
# --------------------------------------------------------------------------
def test_rope_theta_formula(golden_dir):
    g = _golden(golden_dir, "rope_worked_example.json")
    assert np.allclose(oracle.theta(g["d_h"], g["base"]), g["theta"], rtol=1e-12)
    assert np.allclose(pyref.theta(g["d_h"], g["base"]), g["theta"], rtol=1e-12)
    # d_h = 128: theta_0 = 1, theta_last = base^(-(d_h-2)/d_h), strictly decreasing.
    th = oracle.theta(128, 10000.0)
    assert th[0] == 1.0 and np.all(np.diff(th) < 0)
    assert math.isclose(th[-1], 10000.0 ** (-126 / 128), rel_tol=1e-12)


def test_rope_worked_example(golden_dir):
    g = _golden(golden_dir, "rope_worked_example.json")
    out = oracle.rope_row(g["q"], g["m"], g["base"])
    assert np.max(np.abs(out - np.array(g["q_rotated"]))) <= 5e-4
    assert np.max(np.abs(np.array(pyref.rope(g["q"], g["m"], g["base"])) - out)) <= 1e-15
    # cos/sin columns of the example: rotate the unit vectors (1,0) of each pair.
    cs = oracle.rope_row([1.0, 0.0, 1.0, 0.0], g["m"], g["base"])
    assert np.allclose([cs[0], cs[0], cs[2], cs[2]], g["cos"], atol=5e-4)
    assert np.allclose([cs[1], cs[1], cs[3], cs[3]], g["sin"], atol=5e-4)
    # The page's norm figure is a slip; the norms are equal (sqrt(1.38)).
    assert math.isclose(np.linalg.norm(out), math.sqrt(1.38), rel_tol=1e-12)


def test_rope_equals_complex_rotation():
    # Pair (x_2i, x_2i+1) as the complex number x_2i + i x_2i+1, multiplied by
    # exp(i p theta_i): the closed form of a 2-D rotation by p theta_i.
    for d in (4, 8, 64, 128):
        theta = 10000.0 ** (-np.arange(0, d, 2, dtype=np.float64) / d)
        for p in (0, 1, 7, 2047, 65535, 10 ** 6):
            x = RNG.standard_normal(d)
            z = (x[0::2] + 1j * x[1::2]) * np.exp(1j * p * theta)
            ref = np.empty(d)
            ref[0::2], ref[1::2] = z.real, z.imag
            got = oracle.rope_row(x, p)
            assert np.max(np.abs(got - ref)) <= 1e-9 * max(1.0, p * 1e-3), (d, p)


def test_rope_preserves_every_pair_norm():
    for p in (0, 3, 127, 32767, 65535, 10 ** 6):
        x = RNG.standard_normal(128)
        y = oracle.rope_row(x, p)
        nx = np.hypot(x[0::2], x[1::2])
        ny = np.hypot(y[0::2], y[1::2])
        assert np.allclose(nx, ny, rtol=1e-12, atol=0)


def test_rope_relative_position_property():
    # <R(q,m), R(k,n)> depends on m - n only (Part 1, §4.5).
    for _ in range(20):
        q, k = RNG.standard_normal(64), RNG.standard_normal(64)
        m, n, t = (int(x) for x in RNG.integers(0, 50000, size=3))
        a = np.dot(oracle.rope_row(q, m), oracle.rope_row(k, n))
        b = np.dot(oracle.rope_row(q, m + t), oracle.rope_row(k, n + t))
        c = np.dot(q, oracle.rope_row(k, n - m))
        scale = np.linalg.norm(q) * np.linalg.norm(k)
        assert abs(a - b) <= 1e-9 * scale
        assert abs(a - c) <= 1e-9 * scale


def test_rope_group_laws():
    x = RNG.standard_normal(128)
    assert np.array_equal(oracle.rope_row(x, 0), x)
    for a, b in ((3, 5), (1000, 24), (65535, 1)):
        ab = oracle.rope_row(oracle.rope_row(x, a), b)
        assert np.allclose(ab, oracle.rope_row(x, a + b), rtol=0, atol=1e-10)
        assert np.allclose(oracle.rope_row(oracle.rope_row(x, a), -a), x, rtol=0, atol=1e-10)


def test_rope_pairs_are_adjacent_not_halves():
    # rotate-half on adjacent pairs (Part 1, §4.4): [x0,x1,x2,x3] -> [-x1,x0,-x3,x2].
    # Rotating e_0 must only touch components 0 and 1.
    e0 = np.zeros(8)
    e0[0] = 1.0
    y = oracle.rope_row(e0, 1)
    assert y[1] == pytest.approx(math.sin(1.0), abs=1e-15)
    assert np.all(y[2:] == 0.0)


# --------------------------------------------------------------------------
# Attention definition, GQA, masks
# --------------------------------------------------------------------------
def _rand(shape, dtype=np.float32):
    return _f32(RNG.standard_normal(shape))


def _dense_mask(S, causal, W):
    """Mask built literally from Part 2, §10.2: 1 iff 0 <= i-j < W and j <= i."""
    m = np.zeros((S, S), bool)
    for i in range(S):
        for j in range(S):
            if not causal:
                m[i, j] = True
            elif W == 0:
                m[i, j] = j <= i
            else:
                m[i, j] = (0 <= i - j < W) and j <= i
    return m


def _torch_reference(q, k, v, causal, W, m0, base, apply_rope):
    """torch's scaled_dot_product_attention in float64 on the CPU, with the
    dense mask above, KV heads repeated per the GQA map and RoPE applied as a
    complex multiplication. A library routine, independent of the oracle."""
    q, k, v = (torch.from_numpy(np.asarray(x, np.float64)) for x in (q, k, v))
    B, Hq, S, d = q.shape
    G = Hq // k.shape[1]
    if apply_rope:
        pos = torch.arange(S, dtype=torch.float64) + m0
        theta = base ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
        rot = torch.polar(torch.ones(S, d // 2, dtype=torch.float64), pos[:, None] * theta)

        def r(x):
            z = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous()) * rot
            return torch.view_as_real(z).reshape(x.shape)
        q, k = r(q), r(k)
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    mask = torch.from_numpy(_dense_mask(S, causal, W))
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask).numpy()


@pytest.mark.parametrize("S,Hq,Hkv,d,causal,W,m0", [
    (1, 2, 1, 8, 1, 0, 0),
    (17, 4, 2, 16, 1, 0, 0),
    (33, 4, 1, 8, 1, 5, 1000),
    (40, 2, 2, 64, 1, 1, 7),
    (29, 8, 2, 32, 0, 0, 3),
    (64, 4, 2, 16, 1, 64, 0),
])
def test_prefill_matches_torch_sdpa_float64(S, Hq, Hkv, d, causal, W, m0):
    q, k, v = _rand((2, Hq, S, d)), _rand((2, Hkv, S, d)), _rand((2, Hkv, S, d))
    for apply_rope in (False, True):
        got = oracle.prefill(q, k, v, causal=causal, W=W, m0=m0, apply_rope=apply_rope)
        ref = _torch_reference(q, k, v, causal, W, m0, 10000.0, apply_rope)
        assert np.max(np.abs(got - ref)) <= 1e-10


def test_gqa_page_example_mapping():
    # H_q = 4, H_kv = 2: Q0, Q1 -> KV0 and Q2, Q3 -> KV1 (Part 2, §8.4).
    S, d = 12, 16
    q, k, v = _rand((1, 4, S, d)), _rand((1, 2, S, d)), _rand((1, 2, S, d))
    got = oracle.prefill(q, k, v)
    assignment = [0, 0, 1, 1]
    k4, v4 = _f32(k[:, assignment]), _f32(v[:, assignment])
    mha = oracle.prefill(q, k4, v4)  # H_kv = H_q: plain multi-head attention
    assert np.array_equal(got, mha)
    wrong = oracle.prefill(q, _f32(k[:, [0, 1, 0, 1]]), _f32(v[:, [0, 1, 0, 1]]))
    assert np.max(np.abs(wrong[:, 1] - got[:, 1])) > 1e-3


def test_gqa_with_hkv_equal_hq_is_independent_heads():
    S, d, H = 10, 8, 3
    q, k, v = _rand((1, H, S, d)), _rand((1, H, S, d)), _rand((1, H, S, d))
    got = oracle.prefill(q, k, v, W=4)
    for h in range(H):
        one = oracle.prefill(_f32(q[:, h:h + 1]), _f32(k[:, h:h + 1]), _f32(v[:, h:h + 1]), W=4)
        assert np.array_equal(got[:, h:h + 1], one)


@pytest.mark.parametrize("S", [1, 2, 5, 17, 40])
@pytest.mark.parametrize("W", [0, 1, 2, 4, 5, "S"])
@pytest.mark.parametrize("causal", [0, 1])
def test_mask_matches_dense_formula(S, W, causal):
    W = S if W == "S" else W
    if W > 0 and not causal:
        return
    q, k, v = _rand((1, 1, S, 8)), _rand((1, 1, S, 8)), _rand((1, 1, S, 8))
    _, p = oracle.prefill(q, k, v, causal=causal, W=W, probs=True)
    assert np.array_equal(p[0, 0] > 0, _dense_mask(S, causal, W))
    assert np.allclose(p[0, 0].sum(-1), 1.0, rtol=0, atol=1e-12)
    for i in range(S):
        for j in range(S):
            assert oracle.visible(i, j, causal, W) == bool(_dense_mask(S, causal, W)[i, j])


def test_mask_matches_page_visual(golden_dir):
    g = _golden(golden_dir, "mask_visual.json")
    S = g["S"]
    q, k, v = _rand((1, 1, S, 8)), _rand((1, 1, S, 8)), _rand((1, 1, S, 8))
    _, pg = oracle.prefill(q, k, v, causal=1, W=0, probs=True)
    for row, want in g["global_causal_rows"].items():
        assert list((pg[0, 0, int(row)] > 0).astype(int)) == want
    _, pl = oracle.prefill(q, k, v, causal=1, W=g["local_window"], probs=True)
    for row, want in g["local_window_rows"].items():
        assert list((pl[0, 0, int(row)] > 0).astype(int)) == want


# --------------------------------------------------------------------------
# Special cases with closed forms
# --------------------------------------------------------------------------
def test_single_key_returns_its_value():
    q, k, v = _rand((2, 4, 1, 16)), _rand((2, 2, 1, 16)), _rand((2, 2, 1, 16))
    out = oracle.prefill(q, k, v)
    assert np.array_equal(out, np.repeat(v.astype(np.float64), 2, axis=1))


def test_window_one_returns_own_value():
    q, k, v = _rand((1, 4, 23, 16)), _rand((1, 2, 23, 16)), _rand((1, 2, 23, 16))
    out = oracle.prefill(q, k, v, causal=1, W=1, m0=77)
    assert np.array_equal(out, np.repeat(v.astype(np.float64), 2, axis=1))


@pytest.mark.parametrize("W", [0, 1, 3, 8])
def test_zero_query_gives_running_mean(W):
    # q = 0 makes every visible score 0: uniform weights, so row i is the mean
    # of the visible values (a windowed running mean, via prefix sums).
    S, d = 31, 8
    q = np.zeros((1, 2, S, d), np.float32)
    k, v = _rand((1, 1, S, d)), _rand((1, 1, S, d))
    out = oracle.prefill(q, k, v, causal=1, W=W)
    csum = np.concatenate([np.zeros((1, d)), np.cumsum(v[0, 0].astype(np.float64), 0)])
    for i in range(S):
        lo = 0 if W == 0 else max(0, i - W + 1)
        mean = (csum[i + 1] - csum[lo]) / (i + 1 - lo)
        assert np.allclose(out[0, 0, i], mean, rtol=0, atol=1e-12)
        assert np.allclose(out[0, 1, i], mean, rtol=0, atol=1e-12)


def test_equal_keys_give_running_mean():
    S, d = 19, 8
    q, v = _rand((1, 1, S, d)), _rand((1, 1, S, d))
    k = np.repeat(_rand((1, 1, 1, d)), S, axis=2)
    out = oracle.prefill(q, _f32(k), v, causal=1, apply_rope=False)
    csum = np.cumsum(v[0, 0].astype(np.float64), 0)
    for i in range(S):
        assert np.allclose(out[0, 0, i], csum[i] / (i + 1), rtol=0, atol=1e-12)


def test_window_wider_than_sequence_is_causal():
    q, k, v = _rand((1, 2, 20, 8)), _rand((1, 1, 20, 8)), _rand((1, 1, 20, 8))
    a = oracle.prefill(q, k, v, causal=1, W=0)
    for W in (20, 21, 1000):
        assert np.array_equal(a, oracle.prefill(q, k, v, causal=1, W=W))


# --------------------------------------------------------------------------
# C oracle vs its pure-Python twin; decode vs prefill; inputs
# --------------------------------------------------------------------------
@pytest.mark.parametrize("S,Hq,Hkv,d,causal,W,m0", [
    (1, 1, 1, 4, 1, 0, 0), (3, 2, 1, 4, 1, 2, 0), (7, 2, 2, 8, 0, 0, 5),
    (7, 4, 2, 8, 1, 5, 1000), (6, 2, 1, 4, 1, 1, 3),
])
def test_c_oracle_matches_python_twin(S, Hq, Hkv, d, causal, W, m0):
    q, k, v = _rand((2, Hq, S, d)), _rand((2, Hkv, S, d)), _rand((2, Hkv, S, d))
    got = oracle.prefill(q, k, v, causal=causal, W=W, m0=m0)
    ref = np.array(pyref.prefill(q.astype(float).tolist(), k.astype(float).tolist(),
                                 v.astype(float).tolist(), causal, W, m0))
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("Sk,m,W,with_new", [(9, 8, 0, True), (9, 4, 0, True), (12, 11, 3, False),
                                             (5, 0, 0, True)])
def test_c_decode_matches_python_twin(Sk, m, W, with_new):
    B, Hq, Hkv, d = 2, 4, 2, 8
    q, kc, vc = _rand((B, Hq, 1, d)), _rand((B, Hkv, Sk, d)), _rand((B, Hkv, Sk, d))
    kn, vn = (_rand((B, Hkv, 1, d)), _rand((B, Hkv, 1, d))) if with_new else (None, None)
    got = oracle.decode(q, kc, vc, kn, vn, m=m, W=W)
    ref = pyref.decode(q[:, :, 0].astype(float).tolist(), kc.astype(float).tolist(),
                       vc.astype(float).tolist(),
                       kn[:, :, 0].astype(float).tolist() if with_new else None,
                       vn[:, :, 0].astype(float).tolist() if with_new else None, m, W)
    assert np.max(np.abs(got[:, :, 0] - np.array(ref))) <= 1e-12


def test_decode_equals_last_prefill_row():
    B, Hq, Hkv, S, d = 1, 4, 2, 24, 16
    q, k, v = _rand((B, Hq, S, d)), _rand((B, Hkv, S, d)), _rand((B, Hkv, S, d))
    for W in (0, 5):
        pre = oracle.prefill(q, k, v, causal=1, W=W, apply_rope=False)
        dec = oracle.decode(_f32(q[:, :, S - 1:]), k, v, None, None, m=S - 1, W=W,
                            apply_rope=False)
        assert np.array_equal(dec[:, :, 0], pre[:, :, S - 1])
    # With RoPE: the cache holds rotated keys (rounded to fp32 when stored), the
    # new key arrives raw and is rotated at m.
    krot = np.stack([[[oracle.rope_row(k[0, h, j], j) for j in range(S)] for h in range(Hkv)]])
    pre = oracle.prefill(q, k, v, causal=1, apply_rope=True)
    dec = oracle.decode(_f32(q[:, :, S - 1:]), _f32(krot), v, _f32(k[:, :, S - 1:]),
                        _f32(v[:, :, S - 1:]), m=S - 1, apply_rope=True)
    assert np.max(np.abs(dec[:, :, 0] - pre[:, :, S - 1])) <= 1e-5


def test_decode_uses_new_key_value_at_slot_m():
    B, Hq, Hkv, Sk, d = 1, 2, 1, 6, 8
    q, kc, vc = _rand((B, Hq, 1, d)), _rand((B, Hkv, Sk, d)), _rand((B, Hkv, Sk, d))
    kn, vn = _rand((B, Hkv, 1, d)), _rand((B, Hkv, 1, d))
    m = 3
    got = oracle.decode(q, kc, vc, kn, vn, m=m, apply_rope=False)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, m], vc2[:, :, m] = kn[:, :, 0], vn[:, :, 0]
    assert np.array_equal(got, oracle.decode(q, kc2, vc2, None, None, m=m, apply_rope=False))


def test_bf16_inputs_are_widened_exactly():
    q, k, v = apex_inputs.prefill_inputs(1, 9, 2, 1, 8, "bf16", seed=9)
    a = oracle.prefill(q, k, v, W=3)
    b = oracle.prefill(q.float(), k.float(), v.float(), W=3)
    assert np.array_equal(a, b)


def test_input_scores_have_unit_variance():
    # q_i, k_i ~ N(0,1) => Var(q.k) = d_h; after 1/sqrt(d_h) the variance is 1
    # (Part 2, §6.3). Checks the generated inputs, bf16-rounded.
    q, k, _ = apex_inputs.prefill_inputs(1, 512, 4, 4, 128, "bf16", seed=3)
    s = (q.double() @ k.double().transpose(-1, -2)) / math.sqrt(128)
    assert abs(float(s.var()) - 1.0) < 0.05
    assert abs(float(q.double().mean())) < 0.01 and abs(float(q.double().std()) - 1) < 0.01


def test_oracle_rejects_bad_arguments():
    q, k, v = _rand((1, 3, 4, 8)), _rand((1, 2, 4, 8)), _rand((1, 2, 4, 8))
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v)  # H_q % H_kv != 0
    q, k, v = _rand((1, 2, 4, 8)), _rand((1, 2, 4, 8)), _rand((1, 2, 4, 8))
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, causal=0, W=2)
    with pytest.raises(ValueError):
        oracle.decode(_rand((1, 2, 1, 8)), k, v, None, None, m=4)  # m >= Sk


def test_rows_subset_matches_full():
    q, k, v = _rand((2, 4, 37, 16)), _rand((2, 2, 37, 16)), _rand((2, 2, 37, 16))
    full = oracle.prefill(q, k, v, W=9, m0=11)
    rows = np.array([0, 5, 36, 37 * 3 + 2, 37 * 7 + 36, 37 * 4])
    sub = oracle.prefill(q, k, v, W=9, m0=11, rows=rows)
    assert np.array_equal(sub, full.reshape(-1, 16)[rows])
    full_d = oracle.decode(_rand((2, 4, 1, 16)), k, v, None, None, m=30, W=0)
    assert full_d.shape == (2, 4, 1, 16)


# --------------------------------------------------------------------------
# Prefix-bidirectional regime (Part 2, §11.1; picture in §11.3)
# --------------------------------------------------------------------------
def test_prefix_mask_matches_page_visual(golden_dir):
    # Both grids of the picture: prefix P = 4 with full causal rows after it
    # (global layer), and with a window of 4 after it (local layer).
    g = _golden(golden_dir, "mask_visual.json")
    S, P = g["S"], g["prefix"]
    q, k, v = _rand((1, 1, S, 8)), _rand((1, 1, S, 8)), _rand((1, 1, S, 8))
    _, pg = oracle.prefill(q, k, v, causal=1, W=0, prefix=P, probs=True)
    _, pl = oracle.prefill(q, k, v, causal=1, W=g["local_window"], prefix=P, probs=True)
    for probs in (pg, pl):
        for row, want in g["prefix_rows"].items():
            assert list((probs[0, 0, int(row)] > 0).astype(int)) == want
    for row, want in g["global_causal_rows"].items():
        assert list((pg[0, 0, int(row)] > 0).astype(int)) == want
    for row, want in g["local_window_rows"].items():
        assert list((pl[0, 0, int(row)] > 0).astype(int)) == want
    # rows 1 and 2 of the prefix, which the picture elides, follow rows 0 and 3
    for row in (1, 2):
        assert list((pg[0, 0, row] > 0).astype(int)) == g["prefix_rows"]["0"]


@pytest.mark.parametrize("S", [1, 5, 17, 40])
@pytest.mark.parametrize("P", [0, 1, 3, 16, 39, 40, 55])
@pytest.mark.parametrize("W", [0, 1, 4])
def test_prefix_mask_matches_dense_regimes(S, P, W):
    # A dense S x S mask assembled block by block from the three regimes of
    # the table: prefix rows see the whole prefix block, the other rows see the
    # causal lower triangle, cut to a band of width W on local layers.
    dense = np.zeros((S, S), dtype=bool)
    Pc = min(P, S)
    dense[:Pc, :Pc] = True
    tri = np.tril(np.ones((S, S), dtype=bool))
    band = tri & ~np.tril(np.ones((S, S), dtype=bool), -W) if W else tri
    dense[Pc:, :] = band[Pc:, :]
    for i in range(S):
        for j in range(S):
            assert oracle.visible(i, j, 1, W, P) == dense[i, j], (i, j)
    q, k, v = _rand((1, 1, S, 4)), _rand((1, 1, S, 4)), _rand((1, 1, S, 4))
    _, pr = oracle.prefill(q, k, v, causal=1, W=W, prefix=P, probs=True)
    assert np.array_equal(pr[0, 0] > 0, dense)


def test_prefix_zero_is_causal_and_prefix_past_end_is_bidirectional():
    S, d = 23, 8
    q, k, v = _rand((2, 4, S, d)), _rand((2, 2, S, d)), _rand((2, 2, S, d))
    for W in (0, 5):
        assert np.array_equal(oracle.prefill(q, k, v, causal=1, W=W, prefix=0),
                              oracle.prefill(q, k, v, causal=1, W=W))
    full = oracle.prefill(q, k, v, causal=0)
    for P in (S, S + 7):
        assert np.max(np.abs(oracle.prefill(q, k, v, causal=1, prefix=P) - full)) <= 1e-12


@pytest.mark.parametrize("W", [0, 3])
def test_prefix_rows_zero_query_give_prefix_mean_rest_unchanged(W):
    # q = 0: every prefix row is the mean of v over [0, P); rows past the
    # prefix are those of the plain causal / window mask.
    S, d, P = 29, 8, 11
    q = np.zeros((1, 2, S, d), np.float32)
    k, v = _rand((1, 1, S, d)), _rand((1, 1, S, d))
    out = oracle.prefill(q, k, v, causal=1, W=W, prefix=P)
    mean = v[0, 0, :P].astype(np.float64).mean(0)
    assert np.allclose(out[0, :, :P], mean, rtol=0, atol=1e-12)
    q2 = _rand((1, 2, S, d))
    a = oracle.prefill(q2, k, v, causal=1, W=W, prefix=P)
    b = oracle.prefill(q2, k, v, causal=1, W=W)
    assert np.array_equal(a[0, :, P:], b[0, :, P:])


@pytest.mark.parametrize("S,P,W", [(9, 4, 0), (9, 4, 4), (7, 7, 0), (12, 5, 2)])
def test_prefix_c_oracle_matches_python_twin(S, P, W):
    q, k, v = _rand((1, 2, S, 6)), _rand((1, 1, S, 6)), _rand((1, 1, S, 6))
    got = oracle.prefill(q, k, v, causal=1, W=W, prefix=P, m0=3)
    ref = np.array(pyref.prefill(q.astype(float).tolist(), k.astype(float).tolist(),
                                 v.astype(float).tolist(), True, W, 3, P=P))
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_prefix_needs_the_causal_mask():
    q, k, v = _rand((1, 1, 4, 4)), _rand((1, 1, 4, 4)), _rand((1, 1, 4, 4))
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, causal=0, prefix=2)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, causal=1, prefix=-1)


# --------------------------------------------------------------------------
# RMSNorm (Part 1, §3)
# --------------------------------------------------------------------------
def test_rmsnorm_worked_example(golden_dir):
    g = _golden(golden_dir, "rmsnorm_worked_example.json")
    x = np.array([g["x"]], np.float32)
    out = oracle.rmsnorm(x, np.array(g["gamma"], np.float32), eps=g["eps"])[0]
    # the printed steps, to the printed precision
    assert abs(float(np.mean(x.astype(np.float64) ** 2)) - g["mean_of_squares"]) == 0
    assert abs(math.sqrt(g["mean_of_squares"] + g["eps"]) - g["rms_printed"]) < 5e-5
    assert np.max(np.abs(out - np.array(g["output_printed"]))) < 5e-5
    # and the exact value behind them
    exact = np.array(g["x"]) / math.sqrt(1.875 + 1e-6)
    assert np.max(np.abs(out - exact)) < 1e-15


@pytest.mark.parametrize("d", [1, 4, 64, 7168])
def test_rmsnorm_output_mean_square_closed_form(d):
    # with gamma = 1, mean(y^2) = mean(x^2) / (mean(x^2) + eps): the page's
    # "mean(output^2) ~ 1" check made exact
    x = _rand((5, d))
    for eps in (1e-6, 0.5):
        y = oracle.rmsnorm(x, np.ones(d, np.float32), eps=eps)
        msq = (x.astype(np.float64) ** 2).mean(-1)
        assert np.allclose((y ** 2).mean(-1), msq / (msq + eps), rtol=1e-12, atol=0)


def test_rmsnorm_scale_invariance_and_gamma():
    x = _rand((7, 96))
    g = _rand((96,))
    y1 = oracle.rmsnorm(x, np.ones(96, np.float32), eps=0.0)
    for c in (0.25, 4.0, 1024.0):  # powers of two: c * x is exact in fp32
        yc = oracle.rmsnorm((x * c).astype(np.float32), np.ones(96, np.float32), eps=0.0)
        assert np.max(np.abs(yc - y1)) <= 1e-12
    yg = oracle.rmsnorm(x, g, eps=0.0)
    assert np.max(np.abs(yg - y1 * g.astype(np.float64))) <= 1e-12


def test_rmsnorm_zero_row_and_bf16_widening():
    x = np.zeros((2, 16), np.float32)
    assert np.array_equal(oracle.rmsnorm(x, np.ones(16, np.float32)), np.zeros((2, 16)))
    t = torch.randn(3, 40).to(torch.bfloat16)
    gt = torch.randn(40).to(torch.bfloat16)
    a = oracle.rmsnorm(t, gt, eps=1e-6)
    b = oracle.rmsnorm(t.float().numpy(), gt.float().numpy(), eps=1e-6)
    assert np.array_equal(a, b)


def test_rmsnorm_c_oracle_matches_python_twin():
    x, g = _rand((6, 33)), _rand((33,))
    got = oracle.rmsnorm(x, g, eps=1e-3)
    ref = np.array(pyref.rmsnorm(x.astype(float).tolist(), g.astype(float).tolist(), 1e-3))
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_rmsnorm_rejects():
    with pytest.raises(ValueError):
        oracle.rmsnorm(_rand((2, 8)), _rand((7,)))
    with pytest.raises(ValueError):
        oracle.rmsnorm(_rand((2, 8)), _rand((8,)), eps=-1.0)


# --------------------------------------------------------------------------
# YaRN (Part 1, §5)
# --------------------------------------------------------------------------
def test_yarn_worked_example(golden_dir):
    g = _golden(golden_dir, "rope_yarn_worked_example.json")
    s = g["s"]
    by_i = {p["i"]: p for p in g["pairs"]}
    for p in g["pairs"]:
        assert abs(2 * math.pi / p["theta"] - p["wavelength_printed"]) < 0.5
    assert oracle.yarn_theta(by_i[0]["theta"], s) == by_i[0]["theta_yarn_printed"]  # high: kept
    assert abs(oracle.yarn_theta(by_i[15]["theta"], s) - by_i[15]["theta_yarn_printed"]) < 1e-18
    # mid band with t = (628 - 1) / 31 ~ 20.2 clamped to 1: theta / s
    lam = 2 * math.pi / by_i[8]["theta"]
    assert abs((lam - 1) / (s - 1) - by_i[8]["t_unclamped_printed"]) < 0.05
    assert oracle.yarn_theta(by_i[8]["theta"], s) == pytest.approx(by_i[8]["theta"] / s, rel=1e-15)
    assert abs(oracle.yarn_attn_factor(s) - g["attn_factor_printed"]) < 5e-4
    assert oracle.yarn_attn_factor(s) == pytest.approx(0.1 * math.log(32) + 1, rel=1e-15)


@pytest.mark.parametrize("s", [1.0, 4.0, 8.0, 32.0, 64.0, 1000.0])
def test_yarn_regimes(s):
    # the regime table: wavelength below 32 keeps theta, above s divides it
    # by s, and between the two the divisor lies in [1, s]; s = 1 changes nothing
    for th in np.geomspace(1e-7, 4.0, 400):
        lam = 2 * math.pi / th
        got = oracle.yarn_theta(th, s)
        if s == 1.0 or lam < 32:
            assert got == th
        elif lam > s:
            assert got == pytest.approx(th / s, rel=1e-15)
        else:
            assert th / s * (1 - 1e-15) <= got <= th * (1 + 1e-15)
    assert oracle.yarn_attn_factor(1.0) == 1.0


def test_yarn_mid_band_interpolation_formula():
    # s = 64: wavelengths 32 .. 64 are interpolated with t = (lambda - 1) / 63
    s = 64.0
    for lam in (32.0, 40.0, 63.9):
        th = 2 * math.pi / lam
        t = (lam - 1) / (s - 1)
        assert oracle.yarn_theta(th, s) == pytest.approx(th / (t * s + 1 - t), rel=1e-14)


@pytest.mark.parametrize("s", [33.0, 64.0, 100.0, 1000.0, 65536.0])
def test_yarn_mid_band_closed_form(s):
    # With beta_slow = 1 the unclamped t = (lambda - 1) / (s - 1) makes the
    # divisor t s + 1 - t = 1 + t (s - 1) equal to lambda itself, so across the
    # band 32 <= lambda <= s the frequency becomes theta / lambda
    # = theta^2 / (2 pi): a closed form that does not restate the interpolation
    # (Part 1, §5.4, with the §5.3 defaults).
    lams = np.concatenate([[32.0, 40.0, s - 0.1, s], np.geomspace(32.0, s, 200)])
    for lam in lams[lams <= s]:
        th = 2 * math.pi / lam
        assert oracle.yarn_theta(th, s) == pytest.approx(th * th / (2 * math.pi), rel=1e-13)


@pytest.mark.parametrize("s", [64.0, 1000.0])
def test_yarn_band_edges(s):
    # continuity where the band meets the low-frequency regime (lambda = beta_slow s):
    # both sides give theta / s there
    for eps in (1e-9, 1e-6, 1e-3):
        lo, hi = 2 * math.pi / (s - eps), 2 * math.pi / (s + eps)
        # a continuous theta' / theta moves by about eps / s^2 over a step of eps
        assert abs(oracle.yarn_theta(lo, s) / lo - 1 / s) <= 2 * eps / s ** 2 + 1e-15
        assert oracle.yarn_theta(hi, s) / hi == pytest.approx(1 / s, rel=1e-15)
    # at the high-frequency edge (lambda = beta_fast = 32) the table's regimes
    # meet with a jump whenever s > 32: just below it theta is kept, at it the
    # divisor is already lambda = 32
    below, at = 2 * math.pi / (32 - 1e-9), 2 * math.pi / 32
    assert oracle.yarn_theta(below, s) == below
    assert oracle.yarn_theta(at, s) / at == pytest.approx(1 / 32, rel=1e-13)
    # theta' / theta never increases with the wavelength inside the band
    lams = np.geomspace(32.0, s, 300)
    ratio = [oracle.yarn_theta(2 * math.pi / l, s) * l / (2 * math.pi) for l in lams]
    assert all(b <= a * (1 + 1e-15) for a, b in zip(ratio, ratio[1:]))
    assert ratio[0] == pytest.approx(1 / 32, rel=1e-13) and ratio[-1] == pytest.approx(1 / s)


@pytest.mark.parametrize("s", [4.0, 64.0])
def test_yarn_prefill_matches_torch_sdpa(s):
    # RoPE with the YaRN frequencies as a complex rotation, then torch's SDPA
    # with the scores multiplied by the temperature
    S, Hq, Hkv, d = 21, 4, 2, 64
    q, k, v = _rand((1, Hq, S, d)), _rand((1, Hkv, S, d)), _rand((1, Hkv, S, d))
    got = oracle.prefill(q, k, v, causal=1, W=0, m0=5000, yarn_s=s)
    qt, kt, vt = (torch.from_numpy(np.asarray(x, np.float64)) for x in (q, k, v))
    th = torch.from_numpy(oracle.theta(d, 10000.0, s))
    pos = torch.arange(S, dtype=torch.float64) + 5000
    rot = torch.polar(torch.ones(S, d // 2, dtype=torch.float64), pos[:, None] * th)

    def r(x):
        z = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous()) * rot
        return torch.view_as_real(z).reshape(x.shape)
    qt, kt = r(qt), r(kt).repeat_interleave(Hq // Hkv, dim=1)
    vt = vt.repeat_interleave(Hq // Hkv, dim=1)
    mask = torch.from_numpy(_dense_mask(S, 1, 0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=(0.1 * math.log(s) + 1) / math.sqrt(d)).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-10


def test_yarn_c_oracle_matches_python_twin():
    S, d = 9, 8
    q, k, v = _rand((1, 2, S, d)), _rand((1, 1, S, d)), _rand((1, 1, S, d))
    for s in (2.0, 40.0):
        got = oracle.prefill(q, k, v, causal=1, m0=100, base=10.0, yarn_s=s)
        ref = np.array(pyref.prefill(q.astype(float).tolist(), k.astype(float).tolist(),
                                     v.astype(float).tolist(), True, 0, 100, 10.0, True, 0, s))
        assert np.max(np.abs(got - ref)) <= 1e-12


def test_yarn_rejects_scale_below_one():
    q, k, v = _rand((1, 1, 4, 4)), _rand((1, 1, 4, 4)), _rand((1, 1, 4, 4))
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, yarn_s=0.5)
    with pytest.raises(ValueError):
        oracle.theta(8, 10000.0, 0.0)


# --------------------------------------------------------------------------
# MLA attention with decoupled RoPE (Part 2, §9.3)
# --------------------------------------------------------------------------
def _torch_mla_reference(q, k, v, d_r, m0, base, W=0):
    """torch SDPA in float64 on [content | RoPE(rope part)] rows, RoPE of the
    rope part as a complex rotation with d_r-dimensional frequencies, scale
    1 / sqrt(d_h + d_r)."""
    q, k, v = (torch.from_numpy(np.asarray(x, np.float64)) for x in (q, k, v))
    B, Hq, S, dqk = q.shape
    G = Hq // k.shape[1]
    dh = dqk - d_r
    pos = torch.arange(S, dtype=torch.float64) + m0
    theta = base ** (-torch.arange(0, d_r, 2, dtype=torch.float64) / d_r)
    rot = torch.polar(torch.ones(S, d_r // 2, dtype=torch.float64), pos[:, None] * theta)

    def r(x):
        xr = x[..., dh:]
        z = torch.view_as_complex(xr.reshape(*xr.shape[:-1], d_r // 2, 2).contiguous()) * rot
        return torch.cat([x[..., :dh], torch.view_as_real(z).reshape(xr.shape)], -1)
    q, k = r(q), r(k).repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    mask = torch.from_numpy(_dense_mask(S, 1, W))
    return torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=mask, scale=1.0 / math.sqrt(dqk)).numpy()


@pytest.mark.parametrize("S,Hq,Hkv,d_h,d_r,W,m0", [
    (1, 2, 1, 8, 4, 0, 0),
    (19, 4, 2, 16, 8, 0, 100),
    (33, 4, 1, 32, 16, 7, 5000),
    (24, 2, 2, 128, 64, 0, 3),
])
def test_mla_matches_torch_sdpa(S, Hq, Hkv, d_h, d_r, W, m0):
    q = _rand((1, Hq, S, d_h + d_r))
    k = _rand((1, Hkv, S, d_h + d_r))
    v = _rand((1, Hkv, S, d_h))
    got = oracle.prefill_mla(q, k, v, d_r, causal=1, W=W, m0=m0)
    ref = _torch_mla_reference(q, k, v, d_r, m0, 10000.0, W)
    assert np.max(np.abs(got - ref)) <= 1e-10


def test_mla_rope_touches_only_the_rope_part():
    # rotating the whole row instead of the last d_r would change the result;
    # with a zero rope part the positions drop out entirely
    S, d_h, d_r = 17, 16, 8
    q, k, v = _rand((1, 2, S, d_h + d_r)), _rand((1, 1, S, d_h + d_r)), _rand((1, 1, S, d_h))
    q[..., d_h:] = 0
    k[..., d_h:] = 0
    a = oracle.prefill_mla(q, k, v, d_r, m0=0)
    b = oracle.prefill_mla(q, k, v, d_r, m0=12345)
    assert np.max(np.abs(a - b)) <= 1e-13
    # and then the result is plain attention on the content part, scaled by
    # 1 / sqrt(d_h + d_r): the same as content scaled by sqrt(d_h / (d_h + d_r))
    qs = (q[..., :d_h].astype(np.float64) * math.sqrt(d_h / (d_h + d_r)))
    ref = _torch_reference(qs, k[..., :d_h], v, 1, 0, 0, 10000.0, False)
    assert np.max(np.abs(a - ref)) <= 1e-10


def test_mla_scores_depend_on_relative_position_only():
    S, d_h, d_r = 21, 16, 16
    q, k, v = _rand((1, 2, S, d_h + d_r)), _rand((1, 1, S, d_h + d_r)), _rand((1, 1, S, d_h))
    a = oracle.prefill_mla(q, k, v, d_r, m0=0)
    b = oracle.prefill_mla(q, k, v, d_r, m0=777)
    assert np.max(np.abs(a - b)) <= 1e-9


def test_mla_c_oracle_matches_python_twin():
    S, d_h, d_r = 8, 6, 4
    q, k, v = _rand((1, 2, S, d_h + d_r)), _rand((1, 1, S, d_h + d_r)), _rand((1, 1, S, d_h))
    got = oracle.prefill_mla(q, k, v, d_r, causal=1, W=3, m0=11, prefix=2, yarn_s=2.0)
    ref = np.array(pyref.prefill_mla(q.astype(float).tolist(), k.astype(float).tolist(),
                                     v.astype(float).tolist(), d_r, True, 3, 11, 10000.0, 2, 2.0))
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_mla_decode_equals_last_mla_prefill_row():
    # the decode of the query at m = S - 1 against a cache of the S keys is the
    # last row of the prefill, itself pinned to torch's SDPA above
    B, Hq, Hkv, S, d_h, d_r = 1, 4, 2, 20, 16, 8
    q = _rand((B, Hq, S, d_h + d_r))
    k, v = _rand((B, Hkv, S, d_h + d_r)), _rand((B, Hkv, S, d_h))
    for W in (0, 6):
        pre = oracle.prefill_mla(q, k, v, d_r, causal=1, W=W, apply_rope=False)
        dec = oracle.decode_mla(_f32(q[:, :, S - 1:]), k, v, None, None, m=S - 1, d_r=d_r, W=W,
                                apply_rope=False)
        assert np.array_equal(dec[:, :, 0], pre[:, :, S - 1])
    # with RoPE: the cache holds [content | rotated rope part] keys, the new
    # key arrives raw and only its rope part turns at m
    krot = k.astype(np.float64).copy()
    for h in range(Hkv):
        for j in range(S):
            krot[0, h, j, d_h:] = oracle.rope_row(k[0, h, j, d_h:], j)
    pre = _torch_mla_reference(q, k, v, d_r, 0, 10000.0)
    dec = oracle.decode_mla(_f32(q[:, :, S - 1:]), _f32(krot), v, _f32(k[:, :, S - 1:]),
                            _f32(v[:, :, S - 1:]), m=S - 1, d_r=d_r)
    assert np.max(np.abs(dec[:, :, 0] - pre[:, :, S - 1])) <= 1e-5


def test_mla_decode_uses_new_key_value_at_slot_m():
    B, Hq, Hkv, Sk, d_h, d_r = 1, 2, 1, 7, 8, 4
    q = _rand((B, Hq, 1, d_h + d_r))
    kc, vc = _rand((B, Hkv, Sk, d_h + d_r)), _rand((B, Hkv, Sk, d_h))
    kn, vn = _rand((B, Hkv, 1, d_h + d_r)), _rand((B, Hkv, 1, d_h))
    m = 4
    got = oracle.decode_mla(q, kc, vc, kn, vn, m=m, d_r=d_r, apply_rope=False)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, m], vc2[:, :, m] = kn[:, :, 0], vn[:, :, 0]
    assert np.array_equal(got, oracle.decode_mla(q, kc2, vc2, None, None, m=m, d_r=d_r,
                                                 apply_rope=False))
