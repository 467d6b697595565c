// apex_attn.hip -- host side of the C ABI declared in include/apex_attn.h:
// argument checks, launch geometry and kernel launches. All work is enqueued
// on the caller's stream; nothing here allocates, frees or synchronizes.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "apex_attn.h"
#include "decode_kernel.hpp"
#include "prefill_f32_kernel.hpp"
#include "prefill_kernel.hpp"
#include "rmsnorm_kernel.hpp"
#include "rope_kernel.hpp"

namespace {

constexpr double kLog2e = 1.4426950408889634074;

bool head_size_ok(int d_h) { return d_h == 64 || d_h == 128; }

// The kernels move every buffer in 16-byte pieces; a pointer off that grid is
// rejected (NULL passes, its own check decides).
bool aligned16(std::initializer_list<const void*> ptrs) {
  for (const void* ptr : ptrs)
    if ((uintptr_t)ptr & 15u) return false;
  return true;
}

// A YaRN scale factor: >= 1 and finite (1 = plain RoPE).
bool yarn_ok(double s) { return s >= 1.0 && s <= 1e30; }

// The YaRN attention temperature 0.1 ln(s) + 1 (Part 1, §5.5); 1 for s = 1.
double yarn_attn_factor(double s) { return 0.1 * log(s) + 1.0; }

int check_dims(int d_h, int dtype) {
  if (d_h < 2 || (d_h & 1)) return APEX_EINVAL;
  if (dtype != APEX_F32 && dtype != APEX_BF16) return APEX_EINVAL;
  if (!head_size_ok(d_h)) return APEX_EUNSUPPORTED;
  return APEX_OK;
}

int launch_status() {
  return hipGetLastError() == hipSuccess ? APEX_OK : APEX_EHIP;
}

// RoPE over rows of row_len elements whose last d_h turn (row_len = d_h for
// the standard layers).
int launch_rope(const void* src, void* dst, long long n_bh, int S, int d_h, int row_len,
                int64_t m0, double base, double yarn_s, int dtype, hipStream_t st) {
  apex::RopeParams p{src, dst, n_bh, S, d_h, row_len, (long long)m0,
                     apex::make_rope_turns(d_h, base, yarn_s)};
  const long long work = n_bh * ((S + apex::kRopeRows - 1) / apex::kRopeRows) * (row_len / 8);
  long long blocks = (work + apex::kRopeThreads - 1) / apex::kRopeThreads;
  if (blocks > 65535LL * 16) blocks = 65535LL * 16;
  if (blocks < 1) blocks = 1;
  if (dtype == APEX_BF16)
    hipLaunchKernelGGL(apex::rope_kernel<uint16_t>, dim3((unsigned)blocks), dim3(apex::kRopeThreads),
                       0, st, p);
  else
    hipLaunchKernelGGL(apex::rope_kernel<float>, dim3((unsigned)blocks), dim3(apex::kRopeThreads), 0,
                       st, p);
  return launch_status();
}

// Largest power of two that divides G, capped at the waves of a workgroup.
int head_pack(int G) {
  int gp = 1;
  while (gp < apex::kPfWaves && G % (gp * 2) == 0) gp *= 2;
  return gp;
}

// Split-K geometry of the decode: workgroups per (b, KV head, head block).
int decode_splits(int B, int Hkv, int n_hb, int Sk) {
  const long long groups = (long long)B * Hkv * n_hb;
  long long want = (512 + groups - 1) / groups;         // about one wave per SIMD
  const long long cap = (Sk + 2047) / 2048;             // >= 1024 keys per wave
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  return (int)want;
}

// Workgroups of an RMSNorm launch: every wave is resident from the start
// and takes the same number of rows (grid-stride), so no second, partly
// filled round of workgroups trails the first.
template <typename K>
long long rmsnorm_blocks(K kernel, long long rows) {
  const long long waves_per_block = apex::kRmsThreads / 64;
  int dev = 0, n_cu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, apex::kRmsThreads, 0) !=
          hipSuccess ||
      n_cu < 1 || per_cu < 1) {
    (void)hipGetLastError();
    n_cu = 256;
    per_cu = 4;
  }
  const long long resident = (long long)n_cu * per_cu * waves_per_block;
  const long long rows_per_wave = (rows + resident - 1) / resident;
  const long long waves = (rows + rows_per_wave - 1) / rows_per_wave;
  return (waves + waves_per_block - 1) / waves_per_block;
}

template <typename T, int NC>
void launch_rmsnorm_nc(const apex::RmsNormParams& p, hipStream_t st) {
  const long long blocks = rmsnorm_blocks(apex::rmsnorm_kernel<T, NC>, p.rows);
  hipLaunchKernelGGL((apex::rmsnorm_kernel<T, NC>), dim3((unsigned)blocks),
                     dim3(apex::kRmsThreads), 0, st, p);
}

template <typename T>
int launch_rmsnorm(const apex::RmsNormParams& p, int nc, hipStream_t st) {
  switch (nc) {
    case 1: launch_rmsnorm_nc<T, 1>(p, st); break;
    case 2: launch_rmsnorm_nc<T, 2>(p, st); break;
    case 4: launch_rmsnorm_nc<T, 4>(p, st); break;
    case 8: launch_rmsnorm_nc<T, 8>(p, st); break;
    case 16: launch_rmsnorm_nc<T, 16>(p, st); break;
    default: return APEX_EUNSUPPORTED;
  }
  return launch_status();
}

// Split pass + combine of a decode whose arguments have been checked: q and
// keys DQK wide with RoPE on their last DR dims, values and output DV wide.
template <int DQK, int DV, int DR>
int launch_decode(const void* q, void* k_cache, void* v_cache, const void* k_new,
                  const void* v_new, void* o, int B, int Sk, int H_q, int H_kv, int W, int64_t m,
                  double base, double yarn_s, int apply_rope, void* workspace, hipStream_t st) {
  (void)hipGetLastError();
  const int G = H_q / H_kv;
  const int n_hb = (G + apex::kDecHeads - 1) / apex::kDecHeads;
  const int n_split = decode_splits(B, H_kv, n_hb, Sk);
  const int n_parts = n_split * apex::kDecWaves;
  const long long key_lo = W > 0 ? (m - W + 1 > 0 ? m - W + 1 : 0) : 0;
  const long long n_keys = m - key_lo + 1;
  long long kpp = (n_keys + n_parts - 1) / n_parts;
  kpp = (kpp + apex::kDecBN - 1) / apex::kDecBN * apex::kDecBN;

  apex::DecodeParams p{};
  p.q = (const uint16_t*)q;
  p.kc = (uint16_t*)k_cache;
  p.vc = (uint16_t*)v_cache;
  p.kn = (const uint16_t*)k_new;
  p.vn = (const uint16_t*)v_new;
  p.ws_o = (float*)workspace;
  p.ws_ml = p.ws_o + (size_t)B * H_q * n_parts * DV;
  p.Sk = Sk; p.Hq = H_q; p.Hkv = H_kv; p.G = G;
  p.m = m; p.apply_rope = apply_rope;
  if (apply_rope) p.turns = apex::make_rope_turns(DR, base, yarn_s);
  p.n_hb = n_hb; p.n_parts = n_parts;
  p.o = (uint16_t*)o;
  p.fuse = n_split == 1;
  p.key_lo = (int)key_lo;
  p.keys_per_part = (int)kpp;
  // scores are q.k over all DQK dims
  p.sc = (float)(kLog2e * yarn_attn_factor(yarn_s) / sqrt((double)DQK));
  const dim3 grid(n_split, H_kv * n_hb, B);
  hipLaunchKernelGGL((apex::decode_split_kernel<DQK, DV, DR>), grid, dim3(apex::kDecThreads), 0,
                     st, p);
  const int rc = launch_status();
  if (rc != APEX_OK || p.fuse) return rc;
  apex::CombineParams c{p.ws_o, p.ws_ml, (uint16_t*)o, B * H_q, n_parts};
  hipLaunchKernelGGL(apex::decode_combine_kernel<DV>, dim3((B * H_q + 3) / 4), dim3(256), 0, st,
                     c);
  return launch_status();
}

// Scratch of apex_attn_decode_noalloc: the split-K partial results live in
// this file-scope device array instead of a caller workspace. Each GPU the
// library runs on holds its own copy at its own address until the process
// ends. In host code `scratch` is only a stand-in symbol, never a device
// address: the address comes from hipGetSymbolAddress, once per device with
// that device current, and only that address reaches kernels.
static __device__ __align__(256) unsigned char scratch[APEX_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the device that owns `st` (the current device for
// the null stream), looked up on the first call for that device.
int scratch_address(hipStream_t st, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return APEX_EHIP;
  int dev = cur;
  if (st != nullptr && hipStreamGetDevice(st, &dev) != hipSuccess) return APEX_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return APEX_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return APEX_EHIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return APEX_EHIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return APEX_OK;
}

}  // namespace

extern "C" {

const char* apex_strerror(int status) {
  switch (status) {
    case APEX_OK: return "ok";
    case APEX_EINVAL: return "invalid argument";
    case APEX_EUNSUPPORTED: return "unsupported head size or dtype";
    case APEX_EWORKSPACE: return "decode workspace missing or too small";
    case APEX_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int apex_rope_qk(const void* q, const void* k, void* q_out, void* k_out, int B, int S, int H_q,
                 int H_kv, int d_h, int64_t m0, double base, double yarn_s, int dtype,
                 void* stream) {
  if ((q == nullptr) != (q_out == nullptr) || (k == nullptr) != (k_out == nullptr) || (!q && !k))
    return APEX_EINVAL;
  if (!aligned16({q, k, q_out, k_out})) return APEX_EINVAL;
  if (B < 1 || S < 1 || (q && H_q < 1) || (k && H_kv < 1) || m0 < 0 || !(base > 0.0) ||
      !yarn_ok(yarn_s))
    return APEX_EINVAL;
  const int dc = check_dims(d_h, dtype);
  if (dc != APEX_OK) return dc;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  int rc = APEX_OK;
  if (q) rc = launch_rope(q, q_out, (long long)B * H_q, S, d_h, d_h, m0, base, yarn_s, dtype, st);
  if (rc == APEX_OK && k)
    rc = launch_rope(k, k_out, (long long)B * H_kv, S, d_h, d_h, m0, base, yarn_s, dtype, st);
  return rc;
}

int apex_attn_prefill(const void* q, const void* k, const void* v, void* o, void* k_rope_out,
                      int B, int S, int H_q, int H_kv, int d_h, int causal, int W, int prefix,
                      int64_t m0, double base, double yarn_s, int apply_rope, int dtype,
                      void* stream) {
  if (!q || !k || !v || !o || (apply_rope == 1 && !k_rope_out)) return APEX_EINVAL;
  if (!aligned16({q, k, v, o, apply_rope == 1 ? k_rope_out : nullptr})) return APEX_EINVAL;
  if (B < 1 || S < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0) return APEX_EINVAL;
  if (W < 0 || (W > 0 && !causal) || (causal != 0 && causal != 1)) return APEX_EINVAL;
  if (prefix < 0 || (prefix > 0 && !causal)) return APEX_EINVAL;
  if (m0 < 0 || apply_rope < 0 || apply_rope > 2 || (apply_rope && !(base > 0.0)) ||
      !yarn_ok(yarn_s))
    return APEX_EINVAL;
  const int dc = check_dims(d_h, dtype);
  if (dc != APEX_OK) return dc;
  // the attention kernels address one head's rows with 32-bit byte offsets
  if ((long long)S * d_h * (dtype == APEX_BF16 ? 2 : 4) > 0xffffffffLL) return APEX_EUNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();

  const void* kr = k;
  if (apply_rope == 1) {
    const int rc = launch_rope(k, k_rope_out, (long long)B * H_kv, S, d_h, d_h, m0, base, yarn_s,
                               dtype, st);
    if (rc != APEX_OK) return rc;
    kr = k_rope_out;
  }
  const int G = H_q / H_kv;
  if (dtype == APEX_BF16) {
    apex::PrefillParams p{};
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)kr;
    p.v = (const uint16_t*)v;
    p.o = (uint16_t*)o;
    p.S = S; p.Hq = H_q; p.Hkv = H_kv; p.G = G;
    p.causal = causal; p.W = W; p.P = prefix < S ? prefix : S;
    p.m0 = m0; p.apply_rope = apply_rope != 0;
    if (apply_rope) p.turns = apex::make_rope_turns(d_h, base, yarn_s);
    p.g_pack = head_pack(G);
    p.bm = apex::kPfRows / p.g_pack;
    p.n_pos_tiles = (S + p.bm - 1) / p.bm;
    p.n_head_packs = G / p.g_pack;
    p.n_groups = B * H_kv * p.n_head_packs;
    p.sc = (float)(kLog2e * yarn_attn_factor(yarn_s) / sqrt((double)d_h));
    const long long blocks = (long long)p.n_pos_tiles * p.n_groups;
    if (blocks > 0x7fffffffLL) return APEX_EUNSUPPORTED;
    if (d_h == 128)
      hipLaunchKernelGGL((apex::prefill_bf16_kernel<128, 128, 128>), dim3((unsigned)blocks),
                         dim3(apex::kPfThreads), 0, st, p);
    else
      hipLaunchKernelGGL((apex::prefill_bf16_kernel<64, 64, 64>), dim3((unsigned)blocks),
                         dim3(apex::kPfThreads), 0, st, p);
  } else {
    apex::PrefillF32Params p{};
    p.q = (const float*)q;
    p.k = (const float*)kr;
    p.v = (const float*)v;
    p.o = (float*)o;
    p.S = S; p.Hq = H_q; p.Hkv = H_kv; p.G = G;
    p.causal = causal; p.W = W; p.P = prefix < S ? prefix : S;
    p.m0 = m0; p.apply_rope = apply_rope != 0;
    if (apply_rope) p.turns = apex::make_rope_turns(d_h, base, yarn_s);
    p.scale = (float)(yarn_attn_factor(yarn_s) / sqrt((double)d_h));
    if (B > 65535 || H_q > 65535) return APEX_EUNSUPPORTED;
    const dim3 grid((S + apex::kF32Rows - 1) / apex::kF32Rows, H_q, B);
    if (d_h == 128)
      hipLaunchKernelGGL(apex::prefill_f32_kernel<128>, grid, dim3(apex::kF32Threads), 0, st, p);
    else
      hipLaunchKernelGGL(apex::prefill_f32_kernel<64>, grid, dim3(apex::kF32Threads), 0, st, p);
  }
  return launch_status();
}

int apex_attn_prefill_mla(const void* q, const void* k, const void* v, void* o,
                          void* k_rope_out, int B, int S, int H_q, int H_kv, int d_h, int d_r,
                          int causal, int W, int prefix, int64_t m0, double base, double yarn_s,
                          int apply_rope, int dtype, void* stream) {
  if (!q || !k || !v || !o || (apply_rope == 1 && !k_rope_out)) return APEX_EINVAL;
  if (!aligned16({q, k, v, o, apply_rope == 1 ? k_rope_out : nullptr})) return APEX_EINVAL;
  if (B < 1 || S < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0) return APEX_EINVAL;
  if (d_h < 2 || (d_h & 1) || d_r < 2 || (d_r & 1)) return APEX_EINVAL;
  if (W < 0 || (W > 0 && !causal) || (causal != 0 && causal != 1)) return APEX_EINVAL;
  if (prefix < 0 || (prefix > 0 && !causal)) return APEX_EINVAL;
  if (m0 < 0 || apply_rope < 0 || apply_rope > 2 || (apply_rope && !(base > 0.0)) ||
      !yarn_ok(yarn_s))
    return APEX_EINVAL;
  if (dtype != APEX_F32 && dtype != APEX_BF16) return APEX_EINVAL;
  if (dtype != APEX_BF16 || d_h != 128 || d_r != 64) return APEX_EUNSUPPORTED;
  // the attention kernel addresses one head's rows with 32-bit byte offsets
  if ((long long)S * (d_h + d_r) * 2 > 0xffffffffLL) return APEX_EUNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();

  const int dqk = d_h + d_r;
  const void* kr = k;
  if (apply_rope == 1) {
    const int rc = launch_rope(k, k_rope_out, (long long)B * H_kv, S, d_r, dqk, m0, base, yarn_s,
                               dtype, st);
    if (rc != APEX_OK) return rc;
    kr = k_rope_out;
  }
  const int G = H_q / H_kv;
  apex::PrefillParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)kr;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.S = S; p.Hq = H_q; p.Hkv = H_kv; p.G = G;
  p.causal = causal; p.W = W; p.P = prefix < S ? prefix : S;
  p.m0 = m0; p.apply_rope = apply_rope != 0;
  if (apply_rope) p.turns = apex::make_rope_turns(d_r, base, yarn_s);
  p.g_pack = head_pack(G);
  p.bm = apex::kPfRows / p.g_pack;
  p.n_pos_tiles = (S + p.bm - 1) / p.bm;
  p.n_head_packs = G / p.g_pack;
  p.n_groups = B * H_kv * p.n_head_packs;
  // scores are q.k over the whole [content | rope] width
  p.sc = (float)(kLog2e * yarn_attn_factor(yarn_s) / sqrt((double)dqk));
  const long long blocks = (long long)p.n_pos_tiles * p.n_groups;
  if (blocks > 0x7fffffffLL) return APEX_EUNSUPPORTED;
  hipLaunchKernelGGL((apex::prefill_bf16_kernel<192, 128, 64>), dim3((unsigned)blocks),
                     dim3(apex::kPfThreads), 0, st, p);
  return launch_status();
}

int apex_rmsnorm(const void* x, const void* gamma, void* y, int64_t rows, int d, double eps,
                 int dtype, void* stream) {
  if (!x || !gamma || !y || rows < 1 || d < 1 || !(eps >= 0.0) || !(eps <= 1e30)) return APEX_EINVAL;
  if (!aligned16({x, gamma, y})) return APEX_EINVAL;
  if (dtype != APEX_F32 && dtype != APEX_BF16) return APEX_EINVAL;
  if (d % 8 != 0 || d > 8192) return APEX_EUNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  const int need = (d / 8 + 63) / 64;  // 16-byte chunks per lane
  int nc = 1;
  while (nc < need) nc *= 2;
  apex::RmsNormParams p{x, gamma, y, (long long)rows, d, (float)eps};
  return dtype == APEX_BF16 ? launch_rmsnorm<uint16_t>(p, nc, st) : launch_rmsnorm<float>(p, nc, st);
}

size_t apex_attn_decode_workspace_bytes(int B, int H_q, int H_kv, int Sk, int d_h) {
  if (B < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || Sk < 1 || d_h < 2) return 0;
  const int G = H_q / H_kv;
  const int n_hb = (G + apex::kDecHeads - 1) / apex::kDecHeads;
  const int n_parts = decode_splits(B, H_kv, n_hb, Sk) * apex::kDecWaves;
  return (size_t)B * H_q * n_parts * (size_t)(d_h + 2) * sizeof(float);
}

int apex_attn_decode(const void* q, void* k_cache, void* v_cache, const void* k_new,
                     const void* v_new, void* o, int B, int Sk, int H_q, int H_kv, int d_h, int W,
                     int64_t m, double base, double yarn_s, int apply_rope, void* workspace,
                     size_t workspace_bytes, int dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !o || ((k_new == nullptr) != (v_new == nullptr)))
    return APEX_EINVAL;
  if (!aligned16({q, k_cache, v_cache, k_new, v_new, o, workspace})) return APEX_EINVAL;
  if (B < 1 || Sk < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || W < 0) return APEX_EINVAL;
  if (m < 0 || m >= Sk || (apply_rope != 0 && apply_rope != 1) || (apply_rope && !(base > 0.0)) ||
      !yarn_ok(yarn_s))
    return APEX_EINVAL;
  const int dc = check_dims(d_h, dtype);
  if (dc != APEX_OK) return dc;
  if (dtype != APEX_BF16) return APEX_EUNSUPPORTED;
  const size_t need = apex_attn_decode_workspace_bytes(B, H_q, H_kv, Sk, d_h);
  if (!workspace || workspace_bytes < need) return APEX_EWORKSPACE;
  if (B > 65535) return APEX_EUNSUPPORTED;
  if (d_h == 128)
    return launch_decode<128, 128, 128>(q, k_cache, v_cache, k_new, v_new, o, B, Sk, H_q, H_kv,
                                        W, m, base, yarn_s, apply_rope, workspace,
                                        (hipStream_t)stream);
  return launch_decode<64, 64, 64>(q, k_cache, v_cache, k_new, v_new, o, B, Sk, H_q, H_kv, W, m,
                                   base, yarn_s, apply_rope, workspace, (hipStream_t)stream);
}

int apex_attn_decode_noalloc(const void* q, void* k_cache, void* v_cache, const void* k_new,
                             const void* v_new, void* o, int B, int Sk, int H_q, int H_kv,
                             int d_h, int W, int64_t m, double base, double yarn_s,
                             int apply_rope, int dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !o || ((k_new == nullptr) != (v_new == nullptr)))
    return APEX_EINVAL;
  if (!aligned16({q, k_cache, v_cache, k_new, v_new, o})) return APEX_EINVAL;
  if (B < 1 || Sk < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || W < 0) return APEX_EINVAL;
  if (m < 0 || m >= Sk || (apply_rope != 0 && apply_rope != 1) || (apply_rope && !(base > 0.0)) ||
      !yarn_ok(yarn_s))
    return APEX_EINVAL;
  const int dc = check_dims(d_h, dtype);
  if (dc != APEX_OK) return dc;
  if (dtype != APEX_BF16) return APEX_EUNSUPPORTED;
  if (apex_attn_decode_workspace_bytes(B, H_q, H_kv, Sk, d_h) > APEX_DECODE_SCRATCH_BYTES)
    return APEX_EWORKSPACE;
  if (B > 65535) return APEX_EUNSUPPORTED;
  void* ws = nullptr;
  const int rc = scratch_address((hipStream_t)stream, &ws);
  if (rc != APEX_OK) return rc;
  if (d_h == 128)
    return launch_decode<128, 128, 128>(q, k_cache, v_cache, k_new, v_new, o, B, Sk, H_q, H_kv,
                                        W, m, base, yarn_s, apply_rope, ws, (hipStream_t)stream);
  return launch_decode<64, 64, 64>(q, k_cache, v_cache, k_new, v_new, o, B, Sk, H_q, H_kv, W, m,
                                   base, yarn_s, apply_rope, ws, (hipStream_t)stream);
}

int apex_attn_decode_mla(const void* q, void* k_cache, void* v_cache, const void* k_new,
                         const void* v_new, void* o, int B, int Sk, int H_q, int H_kv, int d_h,
                         int d_r, int W, int64_t m, double base, double yarn_s, int apply_rope,
                         void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !o || ((k_new == nullptr) != (v_new == nullptr)))
    return APEX_EINVAL;
  if (!aligned16({q, k_cache, v_cache, k_new, v_new, o, workspace})) return APEX_EINVAL;
  if (B < 1 || Sk < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || W < 0) return APEX_EINVAL;
  if (d_h < 2 || (d_h & 1) || d_r < 2 || (d_r & 1)) return APEX_EINVAL;
  if (m < 0 || m >= Sk || (apply_rope != 0 && apply_rope != 1) || (apply_rope && !(base > 0.0)) ||
      !yarn_ok(yarn_s))
    return APEX_EINVAL;
  if (dtype != APEX_F32 && dtype != APEX_BF16) return APEX_EINVAL;
  if (dtype != APEX_BF16 || d_h != 128 || d_r != 64) return APEX_EUNSUPPORTED;
  const size_t need = apex_attn_decode_workspace_bytes(B, H_q, H_kv, Sk, d_h);
  if (!workspace || workspace_bytes < need) return APEX_EWORKSPACE;
  if (B > 65535) return APEX_EUNSUPPORTED;
  return launch_decode<192, 128, 64>(q, k_cache, v_cache, k_new, v_new, o, B, Sk, H_q, H_kv, W,
                                     m, base, yarn_s, apply_rope, workspace, (hipStream_t)stream);
}

}  // extern "C"
