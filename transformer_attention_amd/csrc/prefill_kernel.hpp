// prefill_kernel.hpp -- flash-style attention prefill for gfx950 in bf16:
//   O = softmax(Q K^T / sqrt(d_h)) V with GQA, causal and window masks
// (APEX-1 Mathematical Reference, Part 2, §6.2 "Formula", §8.2 GQA head map,
// §10.2 window mask), Q rotated by RoPE (Part 1, §4.2) as its tile loads.
//
// Work decomposition
//   One workgroup = 8 waves = 256 query rows that all read the same KV head:
//   g_pack query heads of one GQA group x (256 / g_pack) consecutive positions.
//   Each wave owns 32 rows (one head, 32 positions). K/V tiles of 64 keys are
//   staged once in LDS and reused by all 8 waves, i.e. by all g_pack heads.
//   Tiles are visited only inside the rows' visible key range; per wave a
//   tile is skipped, computed without a mask, or masked element by element.
//   Workgroups are numbered longest-first (latest positions first) and the
//   (batch, KV head) group varies fastest, so one group's workgroups land on
//   one XCD (workgroup i runs on XCD i mod 8) and share its L2.
//
// Register layout (the transposed product)
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims read from
//   LDS, B = Q^T held in registers for the whole loop. The accumulator puts
//   one query row per lane (row l%32) and 16 keys per lane, so the row max
//   needs one exchange with lane l^32 and the row sum none until the end.
//   The same registers, rounded to bf16, are exactly the B operand of
//   O^T += V^T P^T (keys as the contraction), and V^T comes from LDS through
//   the transposing ds_read_b64_tr_b16. O^T keeps one query row per lane.
//
// Online softmax (fp32): scores are scaled by log2(e)/sqrt(d_h) so exp2 can
// be used; a running max m and sum l per row; O and l are rescaled by
// exp2(m_old - m_new) when the max grows.
#pragma once
#include "device_common.hpp"

namespace apex {

constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kPfRows = kPfWaves * 32;  // query rows per workgroup
constexpr int kPfBN = 64;               // keys per K/V tile
constexpr int kPfKPad = 8;              // bf16 pad per K row in LDS (16 B)
constexpr int kPfVPad = 32;             // bf16 pad per V row in LDS (64 B)

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;  // already rotated
  const uint16_t* v;
  uint16_t* o;
  int S, Hq, Hkv, G;
  int causal, W;
  long long m0;
  double base;
  int apply_rope;     // rotate q while it loads
  int g_pack;         // query heads per workgroup (divides G, <= 8)
  int bm;             // positions per workgroup = kPfRows / g_pack
  int n_pos_tiles;    // ceil(S / bm)
  int n_head_packs;   // G / g_pack
  int n_groups;       // B * Hkv * n_head_packs
  float sc;           // log2(e) / sqrt(d_h)
};

enum TileClass { kSkip = 0, kFull = 1, kPartial = 2 };

// Classify keys [j0, j0 + kPfBN) against rows [r0, r0 + 32) (Part 2, §10.2).
__device__ __forceinline__ int classify_tile(int j0, int r0, int S, int causal, int W) {
  const int j1 = j0 + kPfBN - 1;
  if (!causal) return j1 < S ? kFull : kPartial;
  if (j0 > r0 + 31) return kSkip;                  // every key after every row
  if (W > 0 && j1 <= r0 - W) return kSkip;         // every key outside every window
  const bool below = j1 <= r0;                     // j <= i for all pairs
  const bool inside = W == 0 || j0 >= r0 + 32 - W; // i - j < W for all pairs
  return (below && inside && j1 < S) ? kFull : kPartial;
}

template <int D>
__global__ __launch_bounds__(kPfThreads, 1) void prefill_bf16_kernel(PrefillParams p) {
  static_assert(D == 64 || D == 128, "head size");
  constexpr int KS = D + kPfKPad;   // LDS row strides (elements)
  constexpr int VS = D + kPfVPad;
  constexpr int KK = D / 16;        // MFMA steps over the head dimension
  constexpr int DB = D / 32;        // 32-wide blocks of the head dimension
  constexpr int CHUNKS = kPfBN * D / 8;            // 16-byte chunks per tile
  constexpr int REP = CHUNKS / kPfThreads;         // chunks per thread per tile
  static_assert(REP >= 1 && CHUNKS % kPfThreads == 0, "tile split");

  __shared__ __attribute__((aligned(16))) uint16_t ks[2][kPfBN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][kPfBN * VS];
  __shared__ double turns_lds[D / 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  // ---- which rows this workgroup and wave own ----
  const int flat = blockIdx.x;
  const int pos_tile = p.n_pos_tiles - 1 - flat / p.n_groups;
  const int grp = flat % p.n_groups;
  const int hp = grp % p.n_head_packs;
  const int kvh = (grp / p.n_head_packs) % p.Hkv;
  const int b = grp / (p.n_head_packs * p.Hkv);
  const int pos_blocks = p.bm >> 5;
  const int head = kvh * p.G + hp * p.g_pack + wave / pos_blocks;
  const int p0 = pos_tile * p.bm;
  const int pw = p0 + (wave % pos_blocks) * 32;
  const int row = pw + r32;  // this lane's query row

  if (p.apply_rope) {
    if (tid < D / 2) turns_lds[tid] = rope_turns(tid, D, p.base);
    __syncthreads();
  }

  // ---- Q^T operand: lane holds row `row`, dims 16kk + 8g .. +7 ----
  u32x4 qf[KK];
  {
    const uint16_t* qrow = p.q + (((size_t)b * p.Hq + head) * p.S + row) * D;
#pragma unroll
    for (int kk = 0; kk < KK; kk++) {
      const int d0 = 16 * kk + 8 * g;
      u32x4 w = row < p.S ? *(const u32x4*)(qrow + d0) : u32x4{0, 0, 0, 0};
      if (p.apply_rope) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
          float c, s;
          rope_cs_fast(p.m0 + row, turns_lds[d0 / 2 + e], c, s);
          const float x0 = bf16_lo(w[e]), x1 = bf16_hi(w[e]);
          w[e] = pack_bf16x2(x0 * c - x1 * s, x0 * s + x1 * c);
        }
      }
      qf[kk] = w;
    }
  }

  // ---- key range of the workgroup ----
  int j_lo = 0, j_hi = p.S - 1;
  if (p.causal) {
    j_hi = min(p.S - 1, p0 + p.bm - 1);
    if (p.W > 0) j_lo = max(0, p0 - p.W + 1);
  }
  const int t_lo = j_lo / kPfBN, t_hi = j_hi / kPfBN;

  const uint16_t* kbase = p.k + ((size_t)b * p.Hkv + kvh) * p.S * D;
  const uint16_t* vbase = p.v + ((size_t)b * p.Hkv + kvh) * p.S * D;

  u32x4 kreg[REP], vreg[REP];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int r = 0; r < REP; r++) {
      const int ci = tid + r * kPfThreads;
      const int krow = ci / (D / 8), col = (ci % (D / 8)) * 8;
      const int j = t * kPfBN + krow;
      if (j < p.S) {
        kreg[r] = *(const u32x4*)(kbase + (size_t)j * D + col);
        vreg[r] = *(const u32x4*)(vbase + (size_t)j * D + col);
      } else {
        kreg[r] = u32x4{0, 0, 0, 0};
        vreg[r] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < REP; r++) {
      const int ci = tid + r * kPfThreads;
      const int krow = ci / (D / 8), col = (ci % (D / 8)) * 8;
      *(u32x4*)(&ks[buf][krow * KS + col]) = kreg[r];
      *(u32x4*)(&vs[buf][krow * VS + col]) = vreg[r];
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; db++) oacc[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;

  load_tile(t_lo);
  store_tile(0);
  __syncthreads();

  for (int t = t_lo; t <= t_hi; t++) {
    const int buf = (t - t_lo) & 1;
    const bool more = t < t_hi;
    if (more) load_tile(t + 1);  // in flight while this tile computes

    const int j0 = t * kPfBN;
    const int cls = classify_tile(j0, pw, p.S, p.causal, p.W);
    if (cls != kSkip) {
      // S^T = K Q^T for keys j0 .. j0+63 (two 32-key blocks)
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; kb++) {
        sacc[kb] = f32x16{};
        const uint16_t* krow = &ks[buf][(kb * 32 + r32) * KS + 8 * g];
#pragma unroll
        for (int kk = 0; kk < KK; kk++)
          sacc[kb] = mfma32(*(const u32x4*)(krow + 16 * kk), qf[kk], sacc[kb]);
      }
      if (cls == kPartial) {
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int j = j0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            bool vis = j < p.S;
            if (p.causal) vis = vis && j <= row && (p.W == 0 || row - j < p.W);
            if (!vis) sacc[kb][r] = kNegInf;
          }
      }
      // row max over this lane's 32 keys and the partner lane's 32 keys
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++) mx = fmaxf(mx, sacc[kb][r]);
      mx = wave_max_xor(mx, 32);
      const float m_new = fmaxf(m_run, mx * p.sc);
      const float m_use = m_new == kNegInf ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float lsum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], p.sc, -m_use));
          sacc[kb][r] = e;
          lsum += e;
        }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < DB; db++) oacc[db] *= alpha;

      // P^T as bf16 B operands: block kb, half c covers keys kb*32 + 16c + (0..15)
      u32x4 pk[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int c = 0; c < 2; c++)
#pragma unroll
          for (int e = 0; e < 4; e++)
            pk[kb][c][e] = pack_bf16x2(sacc[kb][8 * c + 2 * e], sacc[kb][8 * c + 2 * e + 1]);

      // O^T += V^T P^T. Operand k-index 8g+e <-> key kb*32 + 16c + 4g + e (e < 4)
      // and kb*32 + 16c + 8 + 4g + (e - 4) (e >= 4), matching the S^T layout.
      const int j16 = lane & 15;
      const int dsub = 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);
#pragma unroll
      for (int db = 0; db < DB; db++) {
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
          for (int c = 0; c < 2; c++) {
            const int key = kb * 32 + 16 * c + 4 * g + (j16 >> 2);
            const uint16_t* vp = &vs[buf][key * VS + db * 32 + dsub];
            const u32x2 lo = lds_read_tr16(vp);
            const u32x2 hi = lds_read_tr16(vp + 8 * VS);
            oacc[db] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pk[kb][c], oacc[db]);
          }
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, rounded to bf16 ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (row < p.S) {
    const float inv = 1.0f / l_tot;
    uint16_t* orow = p.o + (((size_t)b * p.Hq + head) * p.S + row) * D;
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        const int d = db * 32 + 8 * q4 + 4 * g;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * q4 + 0] * inv, oacc[db][4 * q4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv);
        *(u32x2*)(orow + d) = w;
      }
  }
}

}  // namespace apex
