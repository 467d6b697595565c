"""Seeded synthetic inputs for the RoPE + attention path.

This module holds no arithmetic of the method: it only names the workloads and
draws their inputs. Both the GPU path's tests and the oracle's tests take their
inputs from here; nothing here imports either side.

Inputs are i.i.d. N(0, 1), the distribution the APEX-1 Mathematical Reference
uses to argue for the 1/sqrt(d_h) scale (Part 2, §6.3), drawn in fp32 with
torch's generator on the target device and rounded to bf16 (round to nearest
even) for the bf16 workloads. Each tensor has its own generator seeded with
seed * 16 + tensor index, and is drawn batch element by batch element, so a
large cache never needs a full fp32 copy.
"""
import torch

# The workloads: name -> sizes. Symbols follow the pages' notation table
# (Part 1, §1): B batch, S sequence, H_q / H_kv query / KV heads, d_h head
# size, d_r the RoPE part of an MLA head, W window (0 = none), prefix P of the
# bidirectional prefix (absent = 0), yarn_s the YaRN scale factor (absent = 1),
# m0 position of row 0, base the RoPE base.
WORKLOADS = {
    "tiny_prefill_f32": dict(kind="prefill", B=1, S=128, Hq=4, Hkv=2, d=64, causal=1, W=0,
                             m0=0, base=10000.0, dtype="f32", seed=1),
    "gqa_prefill_s2048": dict(kind="prefill", B=4, S=2048, Hq=32, Hkv=8, d=128, causal=1, W=0,
                              m0=0, base=10000.0, dtype="bf16", seed=2),
    "window_prefill_s16384_w4096": dict(kind="prefill", B=2, S=16384, Hq=32, Hkv=8, d=128,
                                        causal=1, W=4096, m0=0, base=10000.0, dtype="bf16",
                                        seed=3),
    "local_prefill_s65536_w512": dict(kind="prefill", B=1, S=65536, Hq=64, Hkv=8, d=128,
                                      causal=1, W=512, m0=0, base=10000.0, dtype="bf16", seed=4),
    # prefix-bidirectional regime (Part 2, §11.1): rows < prefix see the whole prefix
    "prefix_prefill_s2048_p512": dict(kind="prefill", B=4, S=2048, Hq=32, Hkv=8, d=128, causal=1,
                                      W=0, prefix=512, m0=0, base=10000.0, dtype="bf16", seed=6),
    "prefix_local_prefill_s16384_w4096_p1024": dict(kind="prefill", B=2, S=16384, Hq=32, Hkv=8,
                                                    d=128, causal=1, W=4096, prefix=1024, m0=0,
                                                    base=10000.0, dtype="bf16", seed=7),
    # YaRN (Part 1, §5): an 8K-trained model run at 32K positions, s = 4
    "yarn_local_prefill_s32768_w4096_s4": dict(kind="prefill", B=1, S=32768, Hq=32, Hkv=8, d=128,
                                               causal=1, W=4096, yarn_s=4.0, m0=0, base=10000.0,
                                               dtype="bf16", seed=10),
    # MLA global layer (Part 2, §9.3, §11.2): [content d_h | rope d_r] queries and keys,
    # full causal attention over the whole sequence
    "mla_global_prefill_s16384": dict(kind="mla_prefill", B=1, S=16384, Hq=64, Hkv=8, d=128,
                                      d_r=64, causal=1, W=0, m0=0, base=10000.0, dtype="bf16",
                                      seed=11),
    # RMSNorm over d_model features (Part 1, §3); the pages' widths run 512 .. 7168
    "rmsnorm_b4_s2048_d7168": dict(kind="rmsnorm", B=4, S=2048, d=7168, eps=1e-6, dtype="bf16",
                                   seed=8),
    "rmsnorm_b64_s2048_d512": dict(kind="rmsnorm", B=64, S=2048, d=512, eps=1e-6, dtype="bf16",
                                   seed=9),
    "gqa_decode_sk32768": dict(kind="decode", B=64, Sk=32768, Hq=128, Hkv=8, d=128, W=0,
                               m=32767, base=10000.0, dtype="bf16", seed=5),
    # MLA global-layer decode: the same batch and cache length with [content | rope] keys
    "mla_global_decode_sk32768": dict(kind="mla_decode", B=64, Sk=32768, Hq=128, Hkv=8, d=128,
                                      d_r=64, W=0, m=32767, base=10000.0, dtype="bf16", seed=13),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def normal(shape, seed, dtype, device, chunk_dim0=True):
    """N(0,1) tensor of `shape`, fp32 draws rounded to `dtype`, drawn along
    dim 0 one slice at a time from one generator seeded with `seed`."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(shape, dtype=dtype, device=device)
    if not chunk_dim0 or len(shape) == 0 or shape[0] == 0:
        out.copy_(torch.randn(shape, generator=g, device=device, dtype=torch.float32))
        return out
    for i in range(shape[0]):
        out[i].copy_(torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32))
    return out


def prefill_inputs(B, S, Hq, Hkv, d, dtype="bf16", seed=0, device="cpu"):
    """(q [B,Hq,S,d], k [B,Hkv,S,d], v [B,Hkv,S,d])."""
    dt = TORCH_DTYPE[dtype] if isinstance(dtype, str) else dtype
    q = normal((B, Hq, S, d), seed * 16 + 0, dt, device)
    k = normal((B, Hkv, S, d), seed * 16 + 1, dt, device)
    v = normal((B, Hkv, S, d), seed * 16 + 2, dt, device)
    return q, k, v


def mla_prefill_inputs(B, S, Hq, Hkv, d, d_r, dtype="bf16", seed=0, device="cpu"):
    """(q [B,Hq,S,d+d_r], k [B,Hkv,S,d+d_r], v [B,Hkv,S,d]): [content | rope] rows."""
    dt = TORCH_DTYPE[dtype] if isinstance(dtype, str) else dtype
    q = normal((B, Hq, S, d + d_r), seed * 16 + 0, dt, device)
    k = normal((B, Hkv, S, d + d_r), seed * 16 + 1, dt, device)
    v = normal((B, Hkv, S, d), seed * 16 + 2, dt, device)
    return q, k, v


def decode_inputs(B, Sk, Hq, Hkv, d, dtype="bf16", seed=0, device="cpu"):
    """(q [B,Hq,1,d], k_cache, v_cache [B,Hkv,Sk,d], k_new, v_new [B,Hkv,1,d]).

    The cache entries stand for keys that were stored after rotation; an
    N(0,1) draw has the same distribution before and after a rotation."""
    dt = TORCH_DTYPE[dtype] if isinstance(dtype, str) else dtype
    q = normal((B, Hq, 1, d), seed * 16 + 0, dt, device)
    k_new = normal((B, Hkv, 1, d), seed * 16 + 1, dt, device)
    v_new = normal((B, Hkv, 1, d), seed * 16 + 2, dt, device)
    k_cache = normal((B, Hkv, Sk, d), seed * 16 + 3, dt, device)
    v_cache = normal((B, Hkv, Sk, d), seed * 16 + 4, dt, device)
    return q, k_cache, v_cache, k_new, v_new


def mla_decode_inputs(B, Sk, Hq, Hkv, d, d_r, dtype="bf16", seed=0, device="cpu"):
    """(q [B,Hq,1,d+d_r], k_cache [B,Hkv,Sk,d+d_r], v_cache [B,Hkv,Sk,d],
    k_new [B,Hkv,1,d+d_r], v_new [B,Hkv,1,d]): [content | rope] keys."""
    dt = TORCH_DTYPE[dtype] if isinstance(dtype, str) else dtype
    q = normal((B, Hq, 1, d + d_r), seed * 16 + 0, dt, device)
    k_new = normal((B, Hkv, 1, d + d_r), seed * 16 + 1, dt, device)
    v_new = normal((B, Hkv, 1, d), seed * 16 + 2, dt, device)
    k_cache = normal((B, Hkv, Sk, d + d_r), seed * 16 + 3, dt, device)
    v_cache = normal((B, Hkv, Sk, d), seed * 16 + 4, dt, device)
    return q, k_cache, v_cache, k_new, v_new


def rmsnorm_inputs(B, S, d, dtype="bf16", seed=0, device="cpu"):
    """(x [B,S,d] ~ N(0,1), gamma [d] ~ 1 + 0.1 N(0,1)): gamma away from its
    initial all-ones value so that the scale is exercised."""
    dt = TORCH_DTYPE[dtype] if isinstance(dtype, str) else dtype
    x = normal((B, S, d), seed * 16 + 0, dt, device)
    g = normal((d,), seed * 16 + 1, torch.float32, device, chunk_dim0=False)
    return x, (1.0 + 0.1 * g).to(dt)


def workload_inputs(name, device="cpu"):
    w = WORKLOADS[name]
    if w["kind"] == "rmsnorm":
        return rmsnorm_inputs(w["B"], w["S"], w["d"], w["dtype"], w["seed"], device)
    if w["kind"] == "mla_prefill":
        return mla_prefill_inputs(w["B"], w["S"], w["Hq"], w["Hkv"], w["d"], w["d_r"], w["dtype"],
                                  w["seed"], device)
    if w["kind"] == "mla_decode":
        return mla_decode_inputs(w["B"], w["Sk"], w["Hq"], w["Hkv"], w["d"], w["d_r"], w["dtype"],
                                 w["seed"], device)
    if w["kind"] == "prefill":
        return prefill_inputs(w["B"], w["S"], w["Hq"], w["Hkv"], w["d"], w["dtype"], w["seed"],
                              device)
    return decode_inputs(w["B"], w["Sk"], w["Hq"], w["Hkv"], w["d"], w["dtype"], w["seed"],
                         device)
