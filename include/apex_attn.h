/*
 * apex_attn.h -- C ABI of the MI355X (gfx950) RoPE + attention library.
 *
 * The operations follow the APEX-1 Mathematical Reference:
 *   - Rotary position embedding (Part 1, §4.2 "Core Idea", §4.3 "Frequency
 *     Formula", §4.4 "Compact Form"): the pair (x_2i, x_2i+1) of a head vector
 *     at position p is rotated by the angle p*theta_i, theta_i = b^(-2i/d_h):
 *       x'_2i   = x_2i cos(p theta_i) - x_2i+1 sin(p theta_i)
 *       x'_2i+1 = x_2i sin(p theta_i) + x_2i+1 cos(p theta_i)
 *   - Scaled dot-product attention (Part 2, §6.2):
 *       Attention(Q, K, V) = softmax(Q K^T / sqrt(d_h)) V
 *   - Grouped-query attention (Part 2, §8.2): G = H_q / H_kv and query head h
 *     reads KV head floor(h / G).
 *   - Causal and sliding-window masks (Part 2, §10.2): key j is visible to
 *     query i iff j <= i and, when W > 0, i - j < W (W keys including i).
 *
 * Conventions shared by every call:
 *   - Tensors are contiguous row-major [B, H, S, d_h] (Part 1, §1 "Tensor
 *     Shape Convention"): element (b, h, s, t) sits at ((b*H + h)*S + s)*d_h + t.
 *   - dtype: APEX_F32 (fp32 storage and math) or APEX_BF16 (bf16 storage,
 *     fp32 softmax and accumulation, bf16 output rounded to nearest even).
 *   - Every pointer is a device pointer owned by the caller, 16-byte aligned
 *     (the kernels move every buffer in 16-byte pieces; a pointer that is not
 *     is APEX_EINVAL).
 *     The library never allocates, frees or synchronizes; it keeps no mutable
 *     global state and is reentrant.
 *   - stream is a hipStream_t (NULL = the null stream). Every call only
 *     enqueues work on it and returns; results are ready when the stream is.
 *   - Every call checks all of its arguments before enqueueing anything. On a
 *     bad argument it returns a negative apex_status and enqueues nothing.
 *     A failed kernel launch returns APEX_EHIP. No C++ exception crosses the ABI.
 *   - Supported head sizes: d_h = 64 or 128 (other even sizes return
 *     APEX_EUNSUPPORTED, odd sizes APEX_EINVAL).
 */
#ifndef APEX_ATTN_H
#define APEX_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  APEX_OK = 0,
  APEX_EINVAL = -1,        /* a size, pointer, flag or position is invalid   */
  APEX_EUNSUPPORTED = -2,  /* valid by the definition, not built (d_h, dtype) */
  APEX_EWORKSPACE = -3,    /* decode workspace missing or too small          */
  APEX_EHIP = -4           /* the HIP runtime reported a launch error        */
} apex_status;

enum { APEX_F32 = 0, APEX_BF16 = 1 };

/*
 * apex_rope_qk -- rotate Q and/or K (Part 1, §4.2-§4.4).
 *   q: [B, H_q, S, d_h] read; q_out: [B, H_q, S, d_h] receives RoPE(q).
 *   k: [B, H_kv, S, d_h] read; k_out: [B, H_kv, S, d_h] receives RoPE(k).
 *   Row s of every head sits at position m0 + s. Each pair (q, q_out) and
 *   (k, k_out) is either both NULL or both given, at least one pair is given,
 *   and an output may equal its own input (in-place rotation) but must not
 *   overlap any other buffer.
 *   base: the RoPE base b (> 0), 10000 on the pages.
 *   yarn_s: YaRN scale factor s >= 1 (Part 1, §5.3-5.4); 1 = plain RoPE.
 *     Each frequency theta_i is replaced by its YaRN value with the pages'
 *     defaults beta_fast = 32, beta_slow = 1: kept when its wavelength
 *     2 pi / theta_i is below 32, divided by s when the wavelength exceeds s,
 *     otherwise divided by t s + 1 - t, t = (wavelength - 1) / (s - 1)
 *     clamped to [0, 1].
 * Angles are formed in fp64 and reduced to one turn before the fp32 sine and
 * cosine, so large positions keep full fp32 accuracy.
 * Errors: APEX_EINVAL for B or S < 1, H_q < 1 when q is given, H_kv < 1 when
 * k is given, a half-given pair, no pair, m0 < 0, base <= 0, yarn_s < 1 or
 * not finite, an unknown dtype; APEX_EUNSUPPORTED for d_h not 64 or 128.
 */
int apex_rope_qk(const void* q, const void* k, void* q_out, void* k_out, int B, int S,
                 int H_q, int H_kv, int d_h, int64_t m0, double base, double yarn_s,
                 int dtype, void* stream);

/*
 * apex_attn_prefill -- o = softmax(RoPE(q) RoPE(k)^T / sqrt(d_h)) v with GQA
 * and the causal / window / prefix-bidirectional masks (Part 2, §6.2, §8.2,
 * §10.2, §11.1).
 *   q: [B, H_q, S, d_h]   (read only)
 *   k: [B, H_kv, S, d_h]  (read only)
 *   v: [B, H_kv, S, d_h]  (read only)
 *   o: [B, H_q, S, d_h]   output; must not overlap any input.
 *   causal: 1 = key j visible to query i only if j <= i; 0 = all visible.
 *   W: window width (> 0 requires causal = 1); 0 = no window.
 *   prefix: P >= 0 (> 0 requires causal = 1). Rows i < P form the
 *     bidirectional prefix: each sees exactly the keys j < P. Rows i >= P keep
 *     the causal mask and the window. 0 = no prefix.
 *   m0: position of row 0 (>= 0). The mask depends on row indices only.
 *   base, yarn_s: the RoPE base and YaRN scale factor as for apex_rope_qk.
 *     With yarn_s > 1 the scores are also multiplied by the YaRN attention
 *     temperature 0.1 ln(yarn_s) + 1 (Part 1, §5.5), whatever apply_rope.
 *   apply_rope:
 *     1 = q and k are raw: k is rotated once into k_rope_out (one elementwise
 *         launch), then the attention launch rotates q while its tiles load
 *         and reads the rotated keys from k_rope_out;
 *     2 = q is raw and k already holds rotated keys (for example a cache
 *         filled by an earlier call): only the attention launch runs, rotating
 *         q as it loads; k_rope_out is ignored;
 *     0 = q and k both hold rotated values; k_rope_out is ignored.
 *   k_rope_out: [B, H_kv, S, d_h] receives RoPE(k) when apply_rope = 1 (the
 *     values a KV cache stores). It may equal k (in-place rotation) but must
 *     not overlap q, v or o.
 * Precision with APEX_BF16: the matrix-core operands are bf16 -- the rotated
 * keys, the rotated queries already multiplied by log2(e)/sqrt(d_h) (times the
 * YaRN temperature), and the probabilities -- each rounded to nearest even
 * once; scores, the softmax and the output sums are fp32.
 * Errors: APEX_EINVAL for H_q % H_kv != 0, sizes < 1, W < 0, W > 0 with
 * causal = 0, prefix < 0, prefix > 0 with causal = 0, m0 < 0, apply_rope not
 * 0/1/2, base <= 0 with apply_rope, yarn_s < 1 or not finite, a NULL
 * required pointer, an unknown dtype; APEX_EUNSUPPORTED for d_h not 64 or 128,
 * and for S * d_h * (element bytes) of 4 GiB or more (one head's rows are
 * addressed with 32-bit byte offsets: S up to 16.7 million bf16 rows of 128).
 */
int apex_attn_prefill(const void* q, const void* k, const void* v, void* o,
                      void* k_rope_out, int B, int S, int H_q, int H_kv, int d_h,
                      int causal, int W, int prefix, int64_t m0, double base,
                      double yarn_s, int apply_rope, int dtype, void* stream);

/*
 * apex_attn_prefill_mla -- the attention core of multi-head latent attention
 * with decoupled RoPE (Part 2, §9.3; used by the global layers, §11.2). Each
 * query and key row is the concatenation [content (d_h) | rope (d_r)]; only
 * the last d_r dims carry position, rotated as in apex_rope_qk with the
 * frequencies of a d_r-wide head (theta_i = b^(-2i/d_r)). Values and outputs
 * are d_h wide:
 *   o = softmax(q' k'^T / sqrt(d_h + d_r)) v,  x' = [x_content | RoPE(x_rope)]
 * (the pages leave the scale open; the score is a dot product over all
 * d_h + d_r dims, and its variance is what the 1/sqrt(width) of §6.2 undoes).
 *   q: [B, H_q, S, d_h + d_r]   (read only)
 *   k: [B, H_kv, S, d_h + d_r]  (read only; query head h reads KV head
 *      floor(h / G) as in apex_attn_prefill, rope part included)
 *   v: [B, H_kv, S, d_h]        (read only)
 *   o: [B, H_q, S, d_h]         output; must not overlap any input.
 *   k_rope_out: [B, H_kv, S, d_h + d_r] receives k' when apply_rope = 1 (the
 *     content part copied, the rope part rotated). It may equal k (then only
 *     the rope part is rewritten) but must not overlap q, v or o.
 *   causal, W, prefix, m0, base, yarn_s, apply_rope, dtype, stream: as for
 *   apex_attn_prefill (the YaRN frequencies follow d_r).
 * Built for bf16 with d_h = 128, d_r = 64.
 * Errors: as apex_attn_prefill, with d_h and d_r each even and >= 2
 * (APEX_EINVAL otherwise); APEX_EUNSUPPORTED for any other (d_h, d_r) or fp32,
 * and for S * (d_h + d_r) * 2 bytes of 4 GiB or more.
 */
int apex_attn_prefill_mla(const void* q, const void* k, const void* v, void* o,
                          void* k_rope_out, int B, int S, int H_q, int H_kv, int d_h,
                          int d_r, int causal, int W, int prefix, int64_t m0, double base,
                          double yarn_s, int apply_rope, int dtype, void* stream);

/*
 * apex_rmsnorm -- y = x / sqrt(mean(x^2) + eps) * gamma over each row of d
 * features (Part 1, §3.2; the norm in front of attention, §3.5).
 *   x: [rows, d] row-major (read only unless y == x).
 *   gamma: [d] scale.
 *   y: [rows, d] output; may equal x (in place) but must not partly overlap it.
 *   All three in `dtype`; bf16 is computed in fp32 and y rounded once.
 *   eps: >= 0 and finite (1e-6 on the pages).
 * Errors: APEX_EINVAL for a NULL pointer, rows or d < 1, eps < 0 or not
 * finite, an unknown dtype; APEX_EUNSUPPORTED for d not a multiple of 8 or
 * d > 8192.
 */
int apex_rmsnorm(const void* x, const void* gamma, void* y, int64_t rows, int d, double eps,
                 int dtype, void* stream);

/*
 * apex_attn_decode_workspace_bytes -- bytes of scratch apex_attn_decode needs
 * for these sizes (the split-K partial results: per query head and split, a
 * running max, a sum and d_h fp32 accumulators). Returns 0 for invalid sizes.
 */
size_t apex_attn_decode_workspace_bytes(int B, int H_q, int H_kv, int Sk, int d_h);

/*
 * apex_attn_decode -- one query token per (b, h) at position m against a
 * cache of Sk slots (Part 2, §6.2 with S_q = 1, §7.4 "KV Cache Problem",
 * §8.2 GQA, §10.2 window).
 *   q: [B, H_q, 1, d_h] raw query of the new token (rotated at m if apply_rope).
 *   k_cache, v_cache: [B, H_kv, Sk, d_h]; slot j holds position j, keys
 *     stored already rotated. Visible slots: j <= m and (W == 0 or m - j < W).
 *   k_new, v_new: [B, H_kv, 1, d_h] key and value of the new token, or both
 *     NULL. When given, the rotated k_new (raw when apply_rope = 0) and v_new
 *     are written into slot m of the caches and used for slot m in this call.
 *   o: [B, H_q, 1, d_h] output.
 *   base, yarn_s: as for apex_attn_prefill (YaRN frequencies for q and k_new,
 *     the temperature on the scores when yarn_s > 1).
 *   workspace: device scratch of workspace_bytes >= the value returned by
 *     apex_attn_decode_workspace_bytes for the same sizes. Always required;
 *     left untouched when the keys of a (b, KV head) are split in two parts
 *     only (the two waves of one workgroup then merge them directly).
 * Errors: APEX_EINVAL for H_q % H_kv != 0, sizes < 1, W < 0, m < 0 or
 * m >= Sk, exactly one of k_new / v_new given, base <= 0 with apply_rope,
 * yarn_s < 1 or not finite, a NULL required pointer, an unknown dtype;
 * APEX_EUNSUPPORTED for d_h not 64 or 128 or dtype fp32; APEX_EWORKSPACE when
 * workspace is NULL or too small.
 */
int apex_attn_decode(const void* q, void* k_cache, void* v_cache,
                     const void* k_new, const void* v_new, void* o,
                     int B, int Sk, int H_q, int H_kv, int d_h, int W, int64_t m,
                     double base, double yarn_s, int apply_rope, void* workspace,
                     size_t workspace_bytes, int dtype, void* stream);

/* Bytes of the library's own decode scratch per GPU (apex_attn_decode_noalloc). */
#define APEX_DECODE_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * apex_attn_decode_noalloc -- apex_attn_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, results and errors as
 * apex_attn_decode, without the workspace: the split-K partial results go to
 * a scratch array inside the library, APEX_DECODE_SCRATCH_BYTES (16 MiB) on
 * each GPU it runs on, held until the process ends. The call allocates
 * nothing; its first call on a device looks up that device's scratch address.
 *   Sizes whose apex_attn_decode_workspace_bytes exceeds
 *   APEX_DECODE_SCRATCH_BYTES return APEX_EWORKSPACE (the decode workload,
 *   B = 64, H_q = 128, H_kv = 8, Sk = 32768, d_h = 128, needs 8.5 MB).
 *   Nothing in the scratch has to start at zero: every partial result the
 *   merge reads is written by the same call. Every call on one GPU shares
 *   that GPU's scratch, so calls that overlap on one GPU (on different
 *   streams, or from different threads) race on it; calls in one stream's
 *   order do not. Errors: as apex_attn_decode, plus APEX_EHIP when the
 *   scratch address cannot be obtained.
 */
int apex_attn_decode_noalloc(const void* q, void* k_cache, void* v_cache,
                             const void* k_new, const void* v_new, void* o,
                             int B, int Sk, int H_q, int H_kv, int d_h, int W, int64_t m,
                             double base, double yarn_s, int apply_rope, int dtype,
                             void* stream);

/*
 * apex_attn_decode_mla -- apex_attn_decode for MLA with decoupled RoPE
 * (Part 2, §9.3): query and cached key rows are [content (d_h) | rope (d_r)],
 * value rows and the output d_h wide; scores scaled by 1 / sqrt(d_h + d_r)
 * (the reading taken for apex_attn_prefill_mla).
 *   q: [B, H_q, 1, d_h + d_r] raw query; its rope part is rotated at m when
 *     apply_rope = 1 (frequencies of a d_r-wide head, YaRN as for
 *     apex_rope_qk), the content part is used as is.
 *   k_cache: [B, H_kv, Sk, d_h + d_r], rope parts stored already rotated.
 *   v_cache: [B, H_kv, Sk, d_h].
 *   k_new: [B, H_kv, 1, d_h + d_r], v_new: [B, H_kv, 1, d_h], or both NULL;
 *     when given they go to slot m as in apex_attn_decode (k_new's rope part
 *     rotated first when apply_rope = 1).
 *   o: [B, H_q, 1, d_h] output.
 *   workspace: at least apex_attn_decode_workspace_bytes(B, H_q, H_kv, Sk, d_h)
 *     bytes (the partial results are d_h wide).
 *   W, m, base, yarn_s, apply_rope, dtype, stream: as for apex_attn_decode.
 * Built for bf16 with d_h = 128, d_r = 64.
 * Errors: as apex_attn_decode, with d_h and d_r each even and >= 2
 * (APEX_EINVAL otherwise); APEX_EUNSUPPORTED for any other (d_h, d_r) or fp32.
 */
int apex_attn_decode_mla(const void* q, void* k_cache, void* v_cache,
                         const void* k_new, const void* v_new, void* o,
                         int B, int Sk, int H_q, int H_kv, int d_h, int d_r, int W,
                         int64_t m, double base, double yarn_s, int apply_rope,
                         void* workspace, size_t workspace_bytes, int dtype, void* stream);

/* apex_strerror -- static text for a status code; never NULL. */
const char* apex_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* APEX_ATTN_H */
