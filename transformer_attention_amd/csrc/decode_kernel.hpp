// decode_kernel.hpp -- split-K attention of one new query token per (b, h)
// against a long bf16 KV cache (APEX-1 Mathematical Reference, Part 2, §6.2
// with S_q = 1; §7.4 "KV Cache Problem"; §8.2 GQA; §10.2 window), the new
// query and key rotated at position m (Part 1, §4.2).
//
// The pass is HBM-bound (about 16 FLOP per cache byte), so the design goal is
// to read every cache byte once, with coalesced 16-byte loads and many bytes
// in flight:
//   - one wave streams a contiguous slice ("part") of the visible slots of one
//     (b, KV head) for up to 16 query heads of its GQA group at once: the
//     heads are the N dimension of v_mfma_f32_16x16x32_bf16, so the G heads
//     share one read of K and V;
//   - S^T = K Q^T: K rows go from HBM straight into the A operand (lane l
//     loads 16 contiguous bytes of key l%16); Q^T stays in registers;
//   - O^T += V^T P^T: each wave stages its 32-key V tile in its own LDS slice
//     and reads it back transposed with ds_read_b64_tr_b16;
//   - loads run two 32-key iterations ahead of the compute (two register
//     buffers, so 32 KB per wave are in flight);
//   - each part ends with its fp32 (running max, sum, unnormalised output) in
//     the workspace; the combine kernel merges the parts of a query head with
//     the log-sum-exp rule and writes the bf16 output.
// When the new token's key/value are given, the wave whose part holds slot m
// uses them from registers for slot m (so no wave reads slot m from memory in
// this call) and writes them into the cache.
//
// DQK is the width of q and of the cached keys, DV that of the cached values
// and the output, and RoPE turns the last DR dims of q and of the new key:
// DQK = DV = DR = d_h for the standard layers, [content d_h | rope d_r] keys
// (DQK = d_h + d_r, DV = d_h, DR = d_r) for MLA with decoupled RoPE (Part 2,
// §9.3).
#pragma once
#include "device_common.hpp"

namespace apex {

// Two waves per workgroup and, for the workloads here, one split: about one
// wave per SIMD, each streaming one long contiguous slice of its (b, KV head)
// (measured: 7.0 TB/s, against 6.85 with twice as many waves and 6.6 with
// four times as many over shorter slices).
constexpr int kDecWaves = 2;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kDecBN = 32;    // keys per wave iteration
constexpr int kDecVPad = 16;  // bf16 pad per LDS V row
constexpr int kDecHeads = 16; // query heads per wave (MFMA N)

struct DecodeParams {
  const uint16_t* q;   // [B, Hq, 1, DQK]
  uint16_t* kc;        // [B, Hkv, Sk, DQK]
  uint16_t* vc;        // [B, Hkv, Sk, DV]
  const uint16_t* kn;  // [B, Hkv, 1, DQK] or null
  const uint16_t* vn;  // [B, Hkv, 1, DV] or null
  float* ws_o;         // [B*Hq, n_parts, DV]
  float* ws_ml;        // [B*Hq, n_parts, 2]
  uint16_t* o;         // [B, Hq, 1, DV]: written here when fuse is set
  int fuse;            // one split: the two waves merge their parts themselves
  int Sk, Hq, Hkv, G;
  long long m;
  RopeTurns turns;     // theta_i / (2 pi) of the DR / 2 rotated pairs (YaRN applied)
  int apply_rope;
  int n_hb;            // ceil(G / 16)
  int n_parts;         // parts per (b, KV head, head block) = gridDim.x * kDecWaves
  int key_lo;          // first visible slot
  int keys_per_part;   // multiple of kDecBN
  float sc;            // log2(e) / sqrt(DQK), times the YaRN temperature
};

template <int DQK, int DV, int DR>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecodeParams p) {
  static_assert(DQK % 32 == 0 && DV % 16 == 0 && (DQK - DR) % 32 == 0 && DV <= DQK, "widths");
  constexpr int KK = DQK / 32;          // 16x16x32 steps over the q.k width
  constexpr int KR = (DQK - DR) / 32;   // first step of the RoPE part
  constexpr int DB = DV / 16;           // 16-row blocks of O^T
  constexpr int VS = DV + kDecVPad;
  constexpr int VCH = kDecBN * DV / 8 / 64;  // 16-byte V chunks per lane per tile
  constexpr int VCPR = DV / 8;               // 16-byte chunks per V row
  __shared__ __attribute__((aligned(16))) uint16_t vlds[kDecWaves][kDecBN * VS];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int part = blockIdx.x * kDecWaves + wave;
  const int kvh = blockIdx.y / p.n_hb;
  const int hb = blockIdx.y % p.n_hb;
  const int b = blockIdx.z;
  const int hg = hb * kDecHeads + l16;  // head within the GQA group
  const bool head_ok = hg < p.G;
  const int head = kvh * p.G + hg;
  const long long m = p.m;

  const int part_lo = p.key_lo + part * p.keys_per_part;
  const int part_hi = (int)min((long long)part_lo + p.keys_per_part - 1, m);
  const size_t kv_row0 = ((size_t)b * p.Hkv + kvh) * p.Sk;
  uint16_t* kcb = p.kc + kv_row0 * DQK;
  uint16_t* vcb = p.vc + kv_row0 * DV;

  // ---- Q^T operand: head l16, dims 32kk + 8g4 .. +7, rotated at m ----
  u32x4 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; kk++) {
    const int d0 = 32 * kk + 8 * g4;
    u32x4 w = u32x4{0, 0, 0, 0};
    if (head_ok) w = *(const u32x4*)(p.q + ((size_t)b * p.Hq + head) * DQK + d0);
    if (kk >= KR && p.apply_rope) {
#pragma unroll
      for (int e = 0; e < 4; e++) {
        float c, s;
        rope_cs_accurate(m, p.turns.v[(d0 - (DQK - DR)) / 2 + e], c, s);
        const float x0 = bf16_lo(w[e]), x1 = bf16_hi(w[e]);
        w[e] = pack_bf16x2(x0 * c - x1 * s, x0 * s + x1 * c);
      }
    }
    qf[kk] = w;
  }

  // ---- the new token: rotated key in the A-operand slice of this lane ----
  const bool has_new = p.kn != nullptr && part_lo <= m && m <= part_hi;
  u32x4 knew[KK];
  if (has_new) {
    const size_t nrow = (size_t)b * p.Hkv + kvh;
#pragma unroll
    for (int kk = 0; kk < KK; kk++) {
      const int d0 = 32 * kk + 8 * g4;
      u32x4 w = *(const u32x4*)(p.kn + nrow * DQK + d0);
      if (kk >= KR && p.apply_rope) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
          float c, s;
          rope_cs_accurate(m, p.turns.v[(d0 - (DQK - DR)) / 2 + e], c, s);
          const float x0 = bf16_lo(w[e]), x1 = bf16_hi(w[e]);
          w[e] = pack_bf16x2(x0 * c - x1 * s, x0 * s + x1 * c);
        }
      }
      knew[kk] = w;
      if (l16 == 0) *(u32x4*)(kcb + (size_t)m * DQK + d0) = w;  // store into slot m
      if (l16 == 1 && d0 < DV)
        *(u32x4*)(vcb + (size_t)m * DV + d0) = *(const u32x4*)(p.vn + nrow * DV + d0);
    }
  }

  // Two register buffers of loads in flight: the keys/values of iteration
  // it + 2 are requested as soon as iteration it has taken its own out of
  // the buffer they share (32 KB per wave in flight).
  u32x4 kA[2][KK], vA[VCH], kB[2][KK], vB[VCH];
  // Cache lines are read once, so the loads are marked non-temporal; the
  // exception is measured: the 384-byte [content | rope] key rows of MLA read
  // 1.5% faster as plain loads (their values stay non-temporal).
  auto load_k = [](const u32x4* ptr) {
    return DQK == DV ? __builtin_nontemporal_load(ptr) : *ptr;
  };
  auto load = [&](int base, u32x4 (&kreg)[2][KK], u32x4 (&vreg)[VCH]) {
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      const int key = base + kb * 16 + l16;
#pragma unroll
      for (int kk = 0; kk < KK; kk++)
        kreg[kb][kk] = key <= part_hi ? load_k((const u32x4*)(kcb + (size_t)key * DQK + 32 * kk + 8 * g4))
                                      : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int c = 0; c < VCH; c++) {
      const int ci = lane + 64 * c;
      const int key = base + ci / VCPR;
      const int col = (ci % VCPR) * 8;
      vreg[c] = key <= part_hi ? __builtin_nontemporal_load((const u32x4*)(vcb + (size_t)key * DV + col))
                               : u32x4{0, 0, 0, 0};
    }
  };

  f32x4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; db++) oacc[db] = f32x4{};
  float m_run = kNegInf, l_run = 0.0f;

  const int n_it = part_hi >= part_lo ? (part_hi - part_lo) / kDecBN + 1 : 0;
  if (n_it > 0) load(part_lo, kA, vA);
  if (n_it > 1) load(part_lo + kDecBN, kB, vB);
  auto iteration = [&](int it, u32x4 (&kreg)[2][KK], u32x4 (&vreg)[VCH]) {
    const int base = part_lo + it * kDecBN;
    u32x4 kcur[2][KK], vcur[VCH];
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int kk = 0; kk < KK; kk++) kcur[kb][kk] = kreg[kb][kk];
#pragma unroll
    for (int c = 0; c < VCH; c++) vcur[c] = vreg[c];
    if (it + 2 < n_it) load(base + 2 * kDecBN, kreg, vreg);

    if (has_new && base <= m && m < base + kDecBN) {  // slot m from registers
      const int km = (int)(m - base);
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
        if (kb * 16 + l16 == km) {
#pragma unroll
          for (int kk = 0; kk < KK; kk++) kcur[kb][kk] = knew[kk];
        }
#pragma unroll
      for (int c = 0; c < VCH; c++) {
        const int ci = lane + 64 * c;
        if (ci / VCPR == km)
          vcur[c] = *(const u32x4*)(p.vn + ((size_t)b * p.Hkv + kvh) * DV + (ci % VCPR) * 8);
      }
    }

    // stage V in this wave's LDS slice
    uint16_t* vw = vlds[wave];
#pragma unroll
    for (int c = 0; c < VCH; c++) {
      const int ci = lane + 64 * c;
      *(u32x4*)(vw + (ci / VCPR) * VS + (ci % VCPR) * 8) = vcur[c];
    }

    // S^T = K Q^T: key 16kb + 4g4 + r, head l16
    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      sacc[kb] = f32x4{};
#pragma unroll
      for (int kk = 0; kk < KK; kk++) sacc[kb] = mfma16(kcur[kb][kk], qf[kk], sacc[kb]);
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        if (base + kb * 16 + 4 * g4 + r > part_hi) sacc[kb][r] = kNegInf;
        mx = fmaxf(mx, sacc[kb][r]);
      }
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m_run, mx * p.sc);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], p.sc, -m_use));
        sacc[kb][r] = e;
        lsum += e;
      }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DB; db++) oacc[db] *= alpha;
    // P^T operand: k-index 8g4+e <-> key 4g4+e (e < 4) and 16+4g4+(e-4) (e >= 4)
    const u32x4 pk = {pack_bf16x2(sacc[0][0], sacc[0][1]), pack_bf16x2(sacc[0][2], sacc[0][3]),
                      pack_bf16x2(sacc[1][0], sacc[1][1]), pack_bf16x2(sacc[1][2], sacc[1][3])};

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T += V^T P^T: d = 16db + 4g4 + r, head l16
#pragma unroll
    for (int db = 0; db < DB; db++) {
      const uint16_t* vp = vw + (4 * g4 + (l16 >> 2)) * VS + 16 * db + 4 * (l16 & 3);
      const u32x2 lo = lds_read_tr16(vp);
      const u32x2 hi = lds_read_tr16(vp + 16 * VS);
      oacc[db] = mfma16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pk, oacc[db]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  int it = 0;
  for (; it + 1 < n_it; it += 2) {
    iteration(it, kA, vA);
    iteration(it + 1, kB, vB);
  }
  if (it < n_it) iteration(it, kA, vA);

  // ---- partial result of this part ----
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (p.fuse) {
    // With one split the workgroup's two waves hold the only two parts of
    // their heads: they merge them by the log-sum-exp rule through LDS (each
    // wave's own V slice, free after its last tile), and each writes the
    // bf16 output of half of the dims. Lane layout as in O^T: dims
    // 16db + 4g4 + r of head l16.
    static_assert(kDecWaves == 2, "two parts per workgroup");
    static_assert((DB * 64 * 4 + 2 * 64) * 4 <= kDecBN * VS * 2, "partials fit a V slice");
    float* const mine = (float*)vlds[wave];
    const float* const other = (const float*)vlds[wave ^ 1];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int db = 0; db < DB; db++) *(f32x4*)(mine + (db * 64 + lane) * 4) = oacc[db];
    mine[DB * 256 + lane] = m_run;
    mine[DB * 256 + 64 + lane] = l_tot;
    __syncthreads();
    const float m_o = other[DB * 256 + lane], l_o = other[DB * 256 + 64 + lane];
    const float M = fmaxf(m_run, m_o);
    const float w_me = m_run == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m_run - M);
    const float w_o = m_o == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m_o - M);
    const float inv = 1.0f / (w_me * l_tot + w_o * l_o);
    if (head_ok) {
      uint16_t* const orow = p.o + ((size_t)b * p.Hq + head) * DV;
#pragma unroll
      for (int db = 0; db < DB; db++)
        if ((db < DB / 2) == (wave == 0)) {
          const f32x4 oo = *(const f32x4*)(other + (db * 64 + lane) * 4);
          u32x2 w;
          w[0] = pack_bf16x2((w_me * oacc[db][0] + w_o * oo[0]) * inv,
                             (w_me * oacc[db][1] + w_o * oo[1]) * inv);
          w[1] = pack_bf16x2((w_me * oacc[db][2] + w_o * oo[2]) * inv,
                             (w_me * oacc[db][3] + w_o * oo[3]) * inv);
          *(u32x2*)(orow + 16 * db + 4 * g4) = w;
        }
    }
    return;
  }
  if (head_ok) {
    const size_t rec = ((size_t)b * p.Hq + head) * p.n_parts + part;
#pragma unroll
    for (int db = 0; db < DB; db++)
      *(f32x4*)(p.ws_o + rec * DV + 16 * db + 4 * g4) = oacc[db];
    if (g4 == 0) {
      p.ws_ml[rec * 2 + 0] = m_run;
      p.ws_ml[rec * 2 + 1] = l_tot;
    }
  }
}

struct CombineParams {
  const float* ws_o;
  const float* ws_ml;
  uint16_t* o;  // [B*Hq, D]
  int n_rows;   // B * Hq
  int n_parts;
};

// Merge the parts of one query head: M = max m_s, L = sum l_s 2^(m_s - M),
// O = sum 2^(m_s - M) o_s / L  (m_s in log2 units). One wave per head.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int rowi = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rowi >= p.n_rows) return;
  const float* ml = p.ws_ml + (size_t)rowi * p.n_parts * 2;
  const float* wo = p.ws_o + (size_t)rowi * p.n_parts * D;
  float M = kNegInf;
  for (int s = 0; s < p.n_parts; s++) M = fmaxf(M, ml[2 * s]);
  float L = 0.0f;
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) acc[i] = 0.0f;
  for (int s = 0; s < p.n_parts; s++) {
    const float ms = ml[2 * s];
    if (ms == kNegInf) continue;  // an empty part
    const float w = __builtin_amdgcn_exp2f(ms - M);
    L += w * ml[2 * s + 1];
#pragma unroll
    for (int i = 0; i < PER; i++) acc[i] += w * wo[(size_t)s * D + lane * PER + i];
  }
  const float inv = 1.0f / L;
  uint16_t* orow = p.o + (size_t)rowi * D + lane * PER;
  if (PER == 2) {
    *(uint32_t*)orow = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  } else {
#pragma unroll
    for (int i = 0; i < PER; i++) orow[i] = f32_to_bf16(acc[i] * inv);
  }
}

}  // namespace apex
