"""fp64 CPU oracle for RoPE + GQA / causal / sliding-window attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code with
the GPU library (``transformer_attention_amd``) and never imports it.

``apex_oracle.c`` holds the definition (see its header for the passages of the
APEX-1 Mathematical Reference it follows); ``pyref.py`` is a pure-Python twin
for tiny sizes. This module only marshals numpy arrays into the C library.
"""
import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "apex_oracle.c")
_LIB_PATH = os.path.join(_DIR, "libapex_oracle.so")
_lib = None

F32, BF16 = 0, 1


def build(force=True):
    """Compile the C oracle with gcc into oracle/libapex_oracle.so."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC",
                           "-pthread", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        L.apex_oracle_theta.argtypes = [i32, dbl, dbl, vp]
        L.apex_oracle_rope_row.argtypes = [vp, vp, i32, i64, dbl, dbl]
        L.apex_oracle_rope_row.restype = None
        L.apex_oracle_yarn_theta.argtypes = [dbl, dbl]
        L.apex_oracle_yarn_theta.restype = dbl
        L.apex_oracle_yarn_attn_factor.argtypes = [dbl]
        L.apex_oracle_yarn_attn_factor.restype = dbl
        L.apex_oracle_visible.argtypes = [i64, i64, i32, i64, i64]
        L.apex_oracle_prefill.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                          i64, i64, dbl, dbl, i32, i64, vp, vp, vp, i32]
        L.apex_oracle_rmsnorm.argtypes = [vp, vp, i32, i64, i32, dbl, vp, i32]
        L.apex_oracle_prefill_mla.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                              i32, i64, i64, dbl, dbl, i32, i64, vp, vp, vp, i32]
        L.apex_oracle_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                         i64, dbl, dbl, i32, i64, vp, vp, i32]
        L.apex_oracle_decode_mla.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                             i32, i32, i64, dbl, dbl, i32, i64, vp, vp, i32]
        _lib = L
    return _lib


def default_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _as_input(x):
    """Return (contiguous array, dtype code). float32 arrays pass as is; bf16
    values arrive as their uint16 bit patterns (dtype code BF16)."""
    if hasattr(x, "detach"):  # a torch CPU tensor
        import torch
        t = x.detach().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16), BF16
        if t.dtype == torch.float32:
            return t.numpy(), F32
        raise TypeError("oracle inputs are float32 or bfloat16, got %s" % t.dtype)
    a = np.ascontiguousarray(x)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    if a.dtype == np.float64:  # convenience for hand-written cases: must be exact in fp32
        f = a.astype(np.float32)
        if not np.array_equal(f.astype(np.float64), a):
            raise ValueError("float64 oracle input is not exactly representable in fp32")
        return f, F32
    raise TypeError("unsupported oracle input dtype %s" % a.dtype)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def theta(d_h, base=10000.0, yarn_s=1.0):
    out = np.empty(d_h // 2, np.float64)
    if lib().apex_oracle_theta(d_h, base, float(yarn_s), _ptr(out)) != 0:
        raise ValueError("bad theta arguments")
    return out


def yarn_theta(theta_i, s):
    """One RoPE frequency after YaRN at scale factor s (Part 1, §5.3-5.4)."""
    return float(lib().apex_oracle_yarn_theta(float(theta_i), float(s)))


def yarn_attn_factor(s):
    """The YaRN attention temperature 0.1 ln(s) + 1 (Part 1, §5.5)."""
    return float(lib().apex_oracle_yarn_attn_factor(float(s)))


def rope_row(x, pos, base=10000.0, yarn_s=1.0):
    x = np.ascontiguousarray(x, np.float64)
    y = np.empty_like(x)
    lib().apex_oracle_rope_row(_ptr(x), _ptr(y), x.shape[-1], int(pos), float(base),
                               float(yarn_s))
    return y


def visible(i, j, causal, W, prefix=0):
    return bool(lib().apex_oracle_visible(i, j, int(causal), int(W), int(prefix)))


def prefill(q, k, v, causal=True, W=0, m0=0, base=10000.0, apply_rope=True,
            rows=None, probs=False, nthreads=None, prefix=0, yarn_s=1.0):
    """q [B,Hq,S,d]; k, v [B,Hkv,S,d] (float32, or bf16 bits as uint16 / torch bf16).

    prefix: P of the prefix-bidirectional regime (rows i < P see keys j < P).
    yarn_s: YaRN scale factor (1 = plain RoPE and unscaled scores).
    rows: optional flat row indices (b*Hq+h)*S+i. Returns fp64 [len(rows), d]
    (or [B,Hq,S,d] when rows is None), and the [.., S] softmax weights if probs."""
    qa, dt = _as_input(q)
    ka, dk = _as_input(k)
    va, dv = _as_input(v)
    if not (dt == dk == dv):
        raise TypeError("q, k, v must share a dtype")
    B, Hq, S, d = qa.shape
    Hkv = ka.shape[1]
    if ka.shape != (B, Hkv, S, d) or va.shape != ka.shape:
        raise ValueError("shape mismatch")
    if rows is None:
        nrows, rarr = B * Hq * S, None
    else:
        rarr = np.ascontiguousarray(rows, np.int64)
        nrows = rarr.size
    out = np.empty((nrows, d), np.float64)
    pr = np.empty((nrows, S), np.float64) if probs else None
    rc = lib().apex_oracle_prefill(_ptr(qa), _ptr(ka), _ptr(va), dt, B, S, Hq, Hkv, d,
                                   int(causal), int(W), int(prefix), int(m0), float(base),
                                   float(yarn_s), int(apply_rope),
                                   nrows, _ptr(rarr), _ptr(out), _ptr(pr),
                                   nthreads or default_threads())
    if rc != 0:
        raise ValueError("apex_oracle_prefill rejected its arguments")
    if rows is None:
        out = out.reshape(B, Hq, S, d)
        if probs:
            pr = pr.reshape(B, Hq, S, S)
    return (out, pr) if probs else out


def decode(q, k_cache, v_cache, k_new, v_new, m, W=0, base=10000.0, apply_rope=True,
           rows=None, nthreads=None, yarn_s=1.0):
    """q [B,Hq,1,d] at position m; caches [B,Hkv,Sk,d]; k_new, v_new [B,Hkv,1,d] or None.

    rows: optional flat b*Hq+h. Returns fp64 [len(rows), d] or [B,Hq,1,d]."""
    qa, dt = _as_input(q)
    kc, _ = _as_input(k_cache)
    vc, _ = _as_input(v_cache)
    kn = _as_input(k_new)[0] if k_new is not None else None
    vn = _as_input(v_new)[0] if v_new is not None else None
    B, Hq, _, d = qa.shape
    Hkv, Sk = kc.shape[1], kc.shape[2]
    if rows is None:
        nrows, rarr = B * Hq, None
    else:
        rarr = np.ascontiguousarray(rows, np.int64)
        nrows = rarr.size
    out = np.empty((nrows, d), np.float64)
    rc = lib().apex_oracle_decode(_ptr(qa), _ptr(kc), _ptr(vc), _ptr(kn), _ptr(vn), dt,
                                  B, Sk, Hq, Hkv, d, int(W), int(m), float(base),
                                  float(yarn_s), int(apply_rope), nrows, _ptr(rarr), _ptr(out),
                                  nthreads or default_threads())
    if rc != 0:
        raise ValueError("apex_oracle_decode rejected its arguments")
    return out.reshape(B, Hq, 1, d) if rows is None else out



def decode_mla(q, k_cache, v_cache, k_new, v_new, m, d_r, W=0, base=10000.0, apply_rope=True,
               rows=None, nthreads=None, yarn_s=1.0):
    """MLA decode: q [B,Hq,1,d_h+d_r] at position m; k_cache [B,Hkv,Sk,d_h+d_r],
    v_cache [B,Hkv,Sk,d_h]; k_new [B,Hkv,1,d_h+d_r], v_new [B,Hkv,1,d_h] or None.
    RoPE on the last d_r dims of q and k_new. Returns fp64 [len(rows), d_h] or
    [B,Hq,1,d_h]."""
    qa, dt = _as_input(q)
    kc, _ = _as_input(k_cache)
    vc, _ = _as_input(v_cache)
    kn = _as_input(k_new)[0] if k_new is not None else None
    vn = _as_input(v_new)[0] if v_new is not None else None
    B, Hq, _, dqk = qa.shape
    Hkv, Sk, d_h = kc.shape[1], kc.shape[2], vc.shape[3]
    if dqk != d_h + d_r or kc.shape[3] != dqk:
        raise ValueError("shape mismatch")
    if rows is None:
        nrows, rarr = B * Hq, None
    else:
        rarr = np.ascontiguousarray(rows, np.int64)
        nrows = rarr.size
    out = np.empty((nrows, d_h), np.float64)
    rc = lib().apex_oracle_decode_mla(_ptr(qa), _ptr(kc), _ptr(vc), _ptr(kn), _ptr(vn), dt,
                                      B, Sk, Hq, Hkv, d_h, int(d_r), int(W), int(m), float(base),
                                      float(yarn_s), int(apply_rope), nrows, _ptr(rarr),
                                      _ptr(out), nthreads or default_threads())
    if rc != 0:
        raise ValueError("apex_oracle_decode_mla rejected its arguments")
    return out.reshape(B, Hq, 1, d_h) if rows is None else out


def rmsnorm(x, gamma, eps=1e-6, nthreads=None):
    """RMSNorm over the last dimension: x [..., d], gamma [d] (float32, or bf16
    bits / torch bf16, both the same dtype). Returns fp64 of x's shape."""
    xa, dt = _as_input(x)
    ga, dg = _as_input(gamma)
    if dt != dg:
        raise TypeError("x and gamma must share a dtype")
    d = xa.shape[-1]
    if ga.shape != (d,):
        raise ValueError("gamma must have shape [d]")
    rows = xa.size // d
    out = np.empty(xa.shape, np.float64)
    if lib().apex_oracle_rmsnorm(_ptr(xa), _ptr(ga), dt, rows, d, float(eps), _ptr(out),
                                 nthreads or default_threads()) != 0:
        raise ValueError("apex_oracle_rmsnorm rejected its arguments")
    return out


def prefill_mla(q, k, v, d_r, causal=True, W=0, m0=0, base=10000.0, apply_rope=True,
                rows=None, probs=False, nthreads=None, prefix=0, yarn_s=1.0):
    """MLA attention with decoupled RoPE: q [B,Hq,S,d_h+d_r], k [B,Hkv,S,d_h+d_r]
    ([content | rope] rows, RoPE on the last d_r), v [B,Hkv,S,d_h]. Returns fp64
    [B,Hq,S,d_h] (or [len(rows), d_h]), and the softmax weights if probs."""
    qa, dt = _as_input(q)
    ka, dk = _as_input(k)
    va, dv_ = _as_input(v)
    if not (dt == dk == dv_):
        raise TypeError("q, k, v must share a dtype")
    B, Hq, S, dqk = qa.shape
    Hkv, d_h = ka.shape[1], va.shape[3]
    if ka.shape != (B, Hkv, S, dqk) or va.shape != (B, Hkv, S, d_h) or dqk != d_h + d_r:
        raise ValueError("shape mismatch")
    if rows is None:
        nrows, rarr = B * Hq * S, None
    else:
        rarr = np.ascontiguousarray(rows, np.int64)
        nrows = rarr.size
    out = np.empty((nrows, d_h), np.float64)
    pr = np.empty((nrows, S), np.float64) if probs else None
    rc = lib().apex_oracle_prefill_mla(_ptr(qa), _ptr(ka), _ptr(va), dt, B, S, Hq, Hkv, d_h,
                                       int(d_r), int(causal), int(W), int(prefix), int(m0),
                                       float(base), float(yarn_s), int(apply_rope), nrows,
                                       _ptr(rarr), _ptr(out), _ptr(pr),
                                       nthreads or default_threads())
    if rc != 0:
        raise ValueError("apex_oracle_prefill_mla rejected its arguments")
    if rows is None:
        out = out.reshape(B, Hq, S, d_h)
        if probs:
            pr = pr.reshape(B, Hq, S, S)
    return (out, pr) if probs else out
