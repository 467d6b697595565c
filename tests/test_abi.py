"""The C ABI library loads, exports every symbol include/apex_attn.h declares,
and rejects every invalid argument with the documented status before touching
the GPU (these calls return before any HIP call, so they run on the CPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "apex_attn.h")

EINVAL, EUNSUP, EWS = -1, -2, -3
P = 0x10000  # a non-null pointer value; never dereferenced on these paths


@pytest.fixture(scope="module")
def L():
    import transformer_attention_amd as taa
    if not os.path.exists(taa.lib_path()):
        from transformer_attention_amd import build
        build.build()
    return taa.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|size_t|const char\*)\s+(apex_\w+)\(", text, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == ["apex_attn_decode", "apex_attn_decode_mla",
                                    "apex_attn_decode_noalloc",
                                    "apex_attn_decode_workspace_bytes", "apex_attn_prefill",
                                    "apex_attn_prefill_mla", "apex_rmsnorm", "apex_rope_qk",
                                    "apex_strerror"]


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
        assert isinstance(getattr(L, name), ctypes._CFuncPtr)


def test_strerror_covers_every_status(L):
    for s in (0, -1, -2, -3, -4, 7):
        assert L.apex_strerror(s)
    assert L.apex_strerror(-3).decode().startswith("decode workspace")


def _rope(L, q=P, k=P, qo=P, ko=P, B=1, S=8, Hq=2, Hkv=1, d=64, m0=0, base=1e4, yarn=1.0,
          dtype=1):
    return L.apex_rope_qk(q, k, qo, ko, B, S, Hq, Hkv, d, m0, base, yarn, dtype, None)


def test_rope_rejects(L):
    assert _rope(L, q=None) == EINVAL           # q given without q_out and vice versa
    assert _rope(L, qo=None) == EINVAL
    assert _rope(L, k=None) == EINVAL
    assert _rope(L, ko=None) == EINVAL
    assert _rope(L, q=None, qo=None, k=None, ko=None) == EINVAL
    assert _rope(L, B=0) == EINVAL
    assert _rope(L, S=0) == EINVAL
    assert _rope(L, Hq=0) == EINVAL
    assert _rope(L, Hkv=0) == EINVAL
    assert _rope(L, m0=-1) == EINVAL
    assert _rope(L, base=0.0) == EINVAL
    assert _rope(L, base=-5.0) == EINVAL
    assert _rope(L, yarn=0.5) == EINVAL
    assert _rope(L, yarn=float("nan")) == EINVAL
    assert _rope(L, yarn=float("inf")) == EINVAL
    assert _rope(L, dtype=7) == EINVAL
    assert _rope(L, d=63) == EINVAL
    assert _rope(L, d=96) == EUNSUP
    assert _rope(L, d=256) == EUNSUP
    # an absent pair does not need its head count
    assert _rope(L, k=None, ko=None, Hkv=0, d=96) == EUNSUP
    assert _rope(L, q=None, qo=None, Hq=0, d=96) == EUNSUP


def _prefill(L, q=P, k=P, v=P, o=P, kr=P, B=1, S=8, Hq=4, Hkv=2, d=128, causal=1, W=0, prefix=0,
             m0=0, base=1e4, yarn=1.0, rope=1, dtype=1):
    return L.apex_attn_prefill(q, k, v, o, kr, B, S, Hq, Hkv, d, causal, W, prefix, m0, base, yarn,
                               rope, dtype, None)


def test_prefill_rejects(L):
    for kw in (dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(kr=None)):
        assert _prefill(L, **kw) == EINVAL, kw
    assert _prefill(L, Hq=3, Hkv=2) == EINVAL      # H_q % H_kv != 0
    assert _prefill(L, B=0) == EINVAL
    assert _prefill(L, S=0) == EINVAL
    assert _prefill(L, Hkv=0) == EINVAL
    assert _prefill(L, W=-1) == EINVAL
    assert _prefill(L, causal=0, W=4) == EINVAL     # a window needs the causal mask
    assert _prefill(L, prefix=-1) == EINVAL
    assert _prefill(L, causal=0, prefix=3) == EINVAL  # so does a bidirectional prefix
    assert _prefill(L, causal=2) == EINVAL
    assert _prefill(L, m0=-3) == EINVAL
    assert _prefill(L, base=0.0) == EINVAL
    assert _prefill(L, yarn=0.99) == EINVAL
    assert _prefill(L, yarn=0.5, rope=0) == EINVAL  # the temperature needs s >= 1 too
    assert _prefill(L, rope=3) == EINVAL
    assert _prefill(L, rope=-1) == EINVAL
    assert _prefill(L, dtype=2) == EINVAL
    assert _prefill(L, d=7) == EINVAL
    assert _prefill(L, d=32) == EUNSUP
    assert _prefill(L, d=80) == EUNSUP


def test_prefill_rejects_rows_beyond_32_bit_offsets(L):
    # one head's rows are addressed with 32-bit byte offsets; checked before
    # anything is launched, so the dummy pointers are never touched
    assert _prefill(L, S=1 << 24, B=1, Hq=1, Hkv=1) == EUNSUP             # bf16, d_h 128
    assert _prefill(L, S=1 << 24, d=64, dtype=0, Hq=1, Hkv=1) == EUNSUP  # fp32, d_h 64
    assert _mla(L, S=(1 << 32) // 384 + 1, Hq=1, Hkv=1) == EUNSUP


def test_prefill_rope_modes_and_rope_buffer(L):
    # k_rope_out is needed only when apply_rope = 1; other checks still apply.
    assert _prefill(L, kr=None, rope=0, Hq=3, Hkv=2) == EINVAL
    assert _prefill(L, kr=None, rope=0, base=0.0, d=96) == EUNSUP  # base unused without RoPE
    assert _prefill(L, kr=None, rope=2, d=96) == EUNSUP            # q-only RoPE: no buffer
    assert _prefill(L, kr=None, rope=2, base=0.0) == EINVAL


def _mla(L, q=P, k=P, v=P, o=P, kr=P, B=1, S=8, Hq=4, Hkv=2, d=128, dr=64, causal=1, W=0,
         prefix=0, m0=0, base=1e4, yarn=1.0, rope=1, dtype=1):
    return L.apex_attn_prefill_mla(q, k, v, o, kr, B, S, Hq, Hkv, d, dr, causal, W, prefix, m0,
                                   base, yarn, rope, dtype, None)


def test_prefill_mla_rejects(L):
    for kw in (dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(kr=None)):
        assert _mla(L, **kw) == EINVAL, kw
    assert _mla(L, kr=None, rope=2, d=64) == EUNSUP   # no RoPE buffer needed
    assert _mla(L, Hq=3, Hkv=2) == EINVAL
    assert _mla(L, B=0) == EINVAL
    assert _mla(L, S=0) == EINVAL
    assert _mla(L, causal=0, W=4) == EINVAL
    assert _mla(L, causal=0, prefix=2) == EINVAL
    assert _mla(L, m0=-1) == EINVAL
    assert _mla(L, base=-1.0) == EINVAL
    assert _mla(L, yarn=0.0) == EINVAL
    assert _mla(L, rope=3) == EINVAL
    assert _mla(L, dtype=2) == EINVAL
    assert _mla(L, d=127) == EINVAL
    assert _mla(L, dr=0) == EINVAL
    assert _mla(L, dr=63) == EINVAL
    assert _mla(L, d=64) == EUNSUP      # built for d_h = 128, d_r = 64
    assert _mla(L, dr=32) == EUNSUP
    assert _mla(L, dtype=0) == EUNSUP   # and for bf16


def test_decode_workspace_bytes(L):
    f = L.apex_attn_decode_workspace_bytes
    assert f(0, 8, 8, 16, 64) == 0
    assert f(1, 3, 2, 16, 64) == 0
    assert f(1, 8, 8, 0, 64) == 0
    n = f(64, 128, 8, 32768, 128)
    # partial results: per (b, h, part) d_h + 2 fp32; parts come in whole
    # workgroups of 2 waves, one part per wave
    assert n > 0 and n % (64 * 128 * 130 * 4) == 0 and (n // (64 * 128 * 130 * 4)) % 2 == 0
    assert f(1, 8, 8, 16, 64) > 0


def _decode(L, q=P, kc=P, vc=P, kn=P, vn=P, o=P, B=2, Sk=64, Hq=16, Hkv=1, d=128, W=0, m=63,
            base=1e4, yarn=1.0, rope=1, ws=P, wsb=None, dtype=1):
    if wsb is None:
        wsb = L.apex_attn_decode_workspace_bytes(B, Hq, Hkv, Sk, d) if Hkv > 0 else 0
    return L.apex_attn_decode(q, kc, vc, kn, vn, o, B, Sk, Hq, Hkv, d, W, m, base, yarn, rope, ws,
                              wsb, dtype, None)


def test_decode_rejects(L):
    for kw in (dict(q=None), dict(kc=None), dict(vc=None), dict(o=None)):
        assert _decode(L, **kw) == EINVAL, kw
    assert _decode(L, kn=None) == EINVAL   # exactly one of k_new / v_new
    assert _decode(L, vn=None) == EINVAL
    assert _decode(L, Hq=12, Hkv=8) == EINVAL
    assert _decode(L, B=0) == EINVAL
    assert _decode(L, Sk=0, wsb=1 << 20) == EINVAL
    assert _decode(L, W=-2) == EINVAL
    assert _decode(L, m=-1) == EINVAL
    assert _decode(L, m=64) == EINVAL       # m >= Sk
    assert _decode(L, base=-1.0) == EINVAL
    assert _decode(L, yarn=0.0) == EINVAL
    assert _decode(L, rope=3) == EINVAL
    assert _decode(L, dtype=5) == EINVAL
    assert _decode(L, d=9) == EINVAL
    assert _decode(L, d=96) == EUNSUP
    assert _decode(L, dtype=0) == EUNSUP    # decode is built for bf16 caches
    assert _decode(L, ws=None) == EWS
    assert _decode(L, wsb=16) == EWS


def _decode_noalloc(L, q=P, kc=P, vc=P, kn=P, vn=P, o=P, B=2, Sk=64, Hq=16, Hkv=1, d=128, W=0,
                    m=63, base=1e4, yarn=1.0, rope=1, dtype=1):
    return L.apex_attn_decode_noalloc(q, kc, vc, kn, vn, o, B, Sk, Hq, Hkv, d, W, m, base, yarn,
                                      rope, dtype, None)


def test_decode_noalloc_rejects(L):
    for kw in (dict(q=None), dict(kc=None), dict(vc=None), dict(o=None)):
        assert _decode_noalloc(L, **kw) == EINVAL, kw
    assert _decode_noalloc(L, kn=None) == EINVAL
    assert _decode_noalloc(L, Hq=12, Hkv=8) == EINVAL
    assert _decode_noalloc(L, B=0) == EINVAL
    assert _decode_noalloc(L, W=-1) == EINVAL
    assert _decode_noalloc(L, m=64) == EINVAL
    assert _decode_noalloc(L, base=0.0) == EINVAL
    assert _decode_noalloc(L, yarn=0.5) == EINVAL
    assert _decode_noalloc(L, rope=2) == EINVAL
    assert _decode_noalloc(L, dtype=4) == EINVAL
    assert _decode_noalloc(L, d=9) == EINVAL
    assert _decode_noalloc(L, d=96) == EUNSUP
    assert _decode_noalloc(L, dtype=0) == EUNSUP
    for name in ("q", "kc", "vc", "kn", "vn", "o"):
        assert _decode_noalloc(L, **{name: P + 8}) == EINVAL, name
    # partial results beyond the 16 MiB scratch are refused before any launch
    ws = L.apex_attn_decode_workspace_bytes
    assert ws(64, 128, 8, 32768, 128) <= 16 << 20   # the decode workload fits
    assert ws(128, 256, 8, 32768, 128) > 16 << 20
    assert _decode_noalloc(L, B=128, Sk=32768, Hq=256, Hkv=8, m=100) == EWS


def _decode_mla(L, q=P, kc=P, vc=P, kn=P, vn=P, o=P, B=2, Sk=64, Hq=16, Hkv=1, d=128, dr=64,
                W=0, m=63, base=1e4, yarn=1.0, rope=1, ws=P, wsb=None, dtype=1):
    if wsb is None:
        wsb = L.apex_attn_decode_workspace_bytes(B, Hq, Hkv, Sk, d) if Hkv > 0 else 0
    return L.apex_attn_decode_mla(q, kc, vc, kn, vn, o, B, Sk, Hq, Hkv, d, dr, W, m, base, yarn,
                                  rope, ws, wsb, dtype, None)


def test_decode_mla_rejects(L):
    for kw in (dict(q=None), dict(kc=None), dict(vc=None), dict(o=None)):
        assert _decode_mla(L, **kw) == EINVAL, kw
    assert _decode_mla(L, kn=None) == EINVAL
    assert _decode_mla(L, Hq=12, Hkv=8) == EINVAL
    assert _decode_mla(L, B=0) == EINVAL
    assert _decode_mla(L, W=-1) == EINVAL
    assert _decode_mla(L, m=64) == EINVAL
    assert _decode_mla(L, base=0.0) == EINVAL
    assert _decode_mla(L, yarn=0.5) == EINVAL
    assert _decode_mla(L, rope=2) == EINVAL
    assert _decode_mla(L, dtype=4) == EINVAL
    assert _decode_mla(L, d=127) == EINVAL
    assert _decode_mla(L, dr=1) == EINVAL
    assert _decode_mla(L, d=64) == EUNSUP     # built for d_h = 128, d_r = 64, bf16
    assert _decode_mla(L, dr=32) == EUNSUP
    assert _decode_mla(L, dtype=0) == EUNSUP
    assert _decode_mla(L, ws=None) == EWS
    assert _decode_mla(L, wsb=64) == EWS


def _rms(L, x=P, g=P, y=P, rows=4, d=64, eps=1e-6, dtype=1):
    return L.apex_rmsnorm(x, g, y, rows, d, eps, dtype, None)


def test_rmsnorm_rejects(L):
    for kw in (dict(x=None), dict(g=None), dict(y=None)):
        assert _rms(L, **kw) == EINVAL, kw
    assert _rms(L, rows=0) == EINVAL
    assert _rms(L, d=0) == EINVAL
    assert _rms(L, eps=-1e-6) == EINVAL
    assert _rms(L, eps=float("inf")) == EINVAL
    assert _rms(L, eps=float("nan")) == EINVAL
    assert _rms(L, dtype=3) == EINVAL
    assert _rms(L, d=12) == EUNSUP      # not a multiple of 8
    assert _rms(L, d=8200) == EUNSUP    # wider than the kernels hold in registers


def test_binding_refuses_cpu_tensors():
    import torch
    import transformer_attention_amd as taa
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        taa.apex_rope_qk(q, None)


def test_misaligned_pointers_are_rejected(L):
    # every buffer is moved in 16-byte pieces, so each pointer argument must
    # sit on that grid; checked before anything is launched
    off = P + 8
    for name in ("q", "k", "qo", "ko"):
        assert _rope(L, **{name: off}) == EINVAL, name
    for name in ("q", "k", "v", "o", "kr"):
        assert _prefill(L, **{name: off}) == EINVAL, name
        assert _mla(L, **{name: off}) == EINVAL, name
    # k_rope_out is not checked when apply_rope != 1 (d_h 96 stops the call later)
    assert _prefill(L, kr=off, rope=2, d=96) == EUNSUP
    for name in ("q", "kc", "vc", "kn", "vn", "o", "ws"):
        assert _decode(L, **{name: off}) == EINVAL, name
        assert _decode_mla(L, **{name: off}) == EINVAL, name
    for name in ("x", "g", "y"):
        assert _rms(L, **{name: off}) == EINVAL, name


def test_binding_checks_shapes_before_any_pointer():
    # the C entry points take sizes once and touch every buffer to the extent
    # they imply, so the binding refuses tensors that do not match the call
    import torch
    import transformer_attention_amd as taa
    bf = torch.bfloat16
    q = torch.zeros(1, 4, 8, 64, dtype=bf)
    k = torch.zeros(1, 2, 8, 64, dtype=bf)
    o = torch.zeros(1, 4, 8, 64, dtype=bf)
    bad = [
        dict(k=torch.zeros(1, 2, 9, 64, dtype=bf)),               # S differs from q's
        dict(v=torch.zeros(1, 2, 8, 32, dtype=bf)),               # d differs
        dict(o=torch.zeros(1, 2, 8, 64, dtype=bf)),               # o with H_kv heads
        dict(k_rope_out=torch.zeros(1, 4, 8, 64, dtype=bf)),      # rotated k with H_q heads
        dict(v=torch.zeros(1, 2, 8, 64, dtype=torch.float32)),    # dtype differs
        dict(k=torch.zeros(2, 8, 64, dtype=bf)),                  # not [B, H, S, d]
    ]
    for change in bad:
        args = dict(q=q, k=k, v=k.clone(), o=o, k_rope_out=None)
        args.update(change)
        with pytest.raises(ValueError, match="apex_attn_prefill"):
            taa.apex_attn_prefill(**args)
    with pytest.raises(ValueError, match="device tensors"):  # consistent: reaches the device check
        taa.apex_attn_prefill(q, k, k.clone(), o, k.clone())

    qd = torch.zeros(2, 16, 1, 64, dtype=bf)
    kc = torch.zeros(2, 1, 100, 64, dtype=bf)
    kn = torch.zeros(2, 1, 1, 64, dtype=bf)
    od = torch.zeros(2, 16, 1, 64, dtype=bf)
    for fn in (taa.apex_attn_decode, taa.apex_attn_decode_noalloc):
        with pytest.raises(ValueError, match="v_cache"):
            fn(qd, kc, torch.zeros(2, 1, 99, 64, dtype=bf), kn, kn.clone(), od, m=99)
        with pytest.raises(ValueError, match="k_new"):
            fn(qd, kc, kc.clone(), torch.zeros(2, 2, 1, 64, dtype=bf), kn, od, m=99)
        with pytest.raises(ValueError, match="o has shape"):
            fn(qd, kc, kc.clone(), kn, kn.clone(), torch.zeros(2, 16, 1, 32, dtype=bf), m=99)
    x = torch.zeros(3, 64, dtype=bf)
    with pytest.raises(ValueError, match="gamma"):
        taa.apex_rmsnorm(x, torch.ones(32, dtype=bf))
    with pytest.raises(ValueError, match="y has shape"):
        taa.apex_rmsnorm(x, torch.ones(64, dtype=bf), torch.zeros(3, 32, dtype=bf))
    with pytest.raises(ValueError, match="k_out"):
        taa.apex_rope_qk(q, k, None, torch.zeros(1, 2, 8, 32, dtype=bf))
    mq = torch.zeros(1, 4, 8, 192, dtype=bf)
    mk = torch.zeros(1, 2, 8, 192, dtype=bf)
    with pytest.raises(ValueError, match="o has shape"):
        taa.apex_attn_prefill_mla(mq, mk, torch.zeros(1, 2, 8, 128, dtype=bf),
                                  torch.zeros(1, 4, 8, 192, dtype=bf))
