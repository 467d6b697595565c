"""Pure-Python fp64 twin of the C oracle, for tiny sizes.

TEST INFRASTRUCTURE: only the test suite uses it. Nested lists and the ``math``
module, no arrays, so that every step can be read against the pages:

* RoPE (APEX-1 Mathematical Reference, Part 1, §4.2-§4.4): pair (2i, 2i+1) is
  rotated by m*theta_i with theta_i = b^(-2i/d_h).
* Scaled dot-product attention (Part 2, §6.2): softmax(q.k / sqrt(d_h)) v.
* GQA (Part 2, §8.2): query head h reads KV head floor(h / G), G = H_q / H_kv.
* Window mask (Part 2, §10.2): key j visible to query i iff 0 <= i - j < W and
  j <= i; W = 0 means no window.
"""
import math


def yarn(th, s, beta_fast=32.0, beta_slow=1.0):
    """YaRN frequency by wavelength regime (Part 1, §5.3-5.4), t clamped to [0, 1]."""
    if s == 1:
        return th
    lam = 2 * math.pi / th
    if lam < beta_fast:
        return th
    if lam > beta_slow * s:
        return th / s
    t = min(1.0, max(0.0, (lam / beta_slow - 1) / (s - 1)))
    return th / (t * s + (1 - t))


def theta(d_h, base=10000.0, s=1.0):
    return [yarn(base ** (-2.0 * i / d_h), s) for i in range(d_h // 2)]


def rope(x, pos, base=10000.0, s=1.0):
    d_h = len(x)
    y = list(x)
    for i, th in enumerate(theta(d_h, base, s)):
        c, s = math.cos(pos * th), math.sin(pos * th)
        a, b = x[2 * i], x[2 * i + 1]
        y[2 * i] = a * c - b * s
        y[2 * i + 1] = a * s + b * c
    return y


def visible(i, j, causal, W, P=0):
    if not causal:
        return True
    if i < P:  # prefix-bidirectional regime
        return j < P
    return j <= i and (W == 0 or i - j < W)


def sdpa_row(q, keys, vals, factor=1.0):
    """softmax(factor * q.k_j / sqrt(d)) weighted sum of v_j, plus the weights."""
    d = len(q)
    scores = [factor * sum(a * b for a, b in zip(q, k)) / math.sqrt(d) for k in keys]
    mx = max(scores)
    w = [math.exp(s - mx) for s in scores]
    tot = sum(w)
    p = [x / tot for x in w]
    out = [sum(p[j] * vals[j][t] for j in range(len(vals))) for t in range(len(vals[0]))]
    return out, p


def sdpa(Q, K, V):
    """Unmasked attention of every row of Q against all rows of K, V."""
    return [sdpa_row(q, K, V)[0] for q in Q]


def prefill(q, k, v, causal=True, W=0, m0=0, base=10000.0, apply_rope=True, P=0, s=1.0):
    """q[B][Hq][S][d], k and v [B][Hkv][S][d] -> o[B][Hq][S][d]."""
    B, Hq, S = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    out = []
    for b in range(B):
        heads = []
        for h in range(Hq):
            kvh = h // G
            keys = [rope(k[b][kvh][j], m0 + j, base, s) if apply_rope else k[b][kvh][j]
                    for j in range(S)]
            rows = []
            for i in range(S):
                qi = rope(q[b][h][i], m0 + i, base, s) if apply_rope else q[b][h][i]
                js = [j for j in range(S) if visible(i, j, causal, W, P)]
                o, _ = sdpa_row(qi, [keys[j] for j in js], [v[b][kvh][j] for j in js],
                                0.1 * math.log(s) + 1.0)
                rows.append(o)
            heads.append(rows)
        out.append(heads)
    return out


def decode(q, k_cache, v_cache, k_new, v_new, m, W=0, base=10000.0, apply_rope=True):
    """q[B][Hq][d] at position m; caches [B][Hkv][Sk][d] hold rotated keys;
    k_new, v_new [B][Hkv][d] (or None) occupy slot m. -> o[B][Hq][d]."""
    B, Hq = len(q), len(q[0])
    Hkv = len(k_cache[0])
    G = Hq // Hkv
    out = []
    for b in range(B):
        heads = []
        for h in range(Hq):
            kvh = h // G
            qi = rope(q[b][h], m, base) if apply_rope else q[b][h]
            keys, vals = [], []
            for j in range(m + 1):
                if not visible(m, j, True, W):
                    continue
                if j == m and k_new is not None:
                    kj = rope(k_new[b][kvh], m, base) if apply_rope else k_new[b][kvh]
                else:
                    kj = k_cache[b][kvh][j]
                vj = v_new[b][kvh] if (j == m and v_new is not None) else v_cache[b][kvh][j]
                keys.append(kj)
                vals.append(vj)
            heads.append(sdpa_row(qi, keys, vals)[0])
        out.append(heads)
    return out


def rmsnorm(x, gamma, eps=1e-6):
    """x [rows][d], gamma [d] -> rows divided by sqrt(mean of squares + eps), times gamma."""
    out = []
    for row in x:
        rms = math.sqrt(sum(v * v for v in row) / len(row) + eps)
        out.append([v / rms * g for v, g in zip(row, gamma)])
    return out


def prefill_mla(q, k, v, d_r, causal=True, W=0, m0=0, base=10000.0, P=0, s=1.0):
    """MLA with decoupled RoPE: q, k rows [content | rope(d_r)], v rows of d_h."""
    B, Hq, S = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    dqk = len(q[0][0][0])
    dh = dqk - d_r

    def rot(x, pos):
        return list(x[:dh]) + rope(x[dh:], pos, base, s)
    out = []
    for b in range(B):
        heads = []
        for h in range(Hq):
            kvh = h // G
            keys = [rot(k[b][kvh][j], m0 + j) for j in range(S)]
            rows = []
            for i in range(S):
                qi = rot(q[b][h][i], m0 + i)
                js = [j for j in range(S) if visible(i, j, causal, W, P)]
                # sdpa_row scales by 1/sqrt(len(q)) = 1/sqrt(d_h + d_r)
                o, _ = sdpa_row(qi, [keys[j] for j in js], [v[b][kvh][j] for j in js],
                                0.1 * math.log(s) + 1.0)
                rows.append(o)
            heads.append(rows)
        out.append(heads)
    return out
