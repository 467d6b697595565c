// prefill_kernel.hpp -- flash-style attention prefill for gfx950 in bf16:
//   O = softmax(Q K^T / sqrt(d_h)) V with GQA, causal and window masks
// (APEX-1 Mathematical Reference, Part 2, §6.2 "Formula", §8.2 GQA head map,
// §10.2 window mask, §11.1 prefix-bidirectional regime), Q rotated by RoPE
// (Part 1, §4.2) as its tile loads.
//
// Work decomposition
//   One workgroup = 4 waves = 128 query rows that all read the same KV head:
//   g_pack query heads of one GQA group x (128 / g_pack) consecutive positions.
//   Each wave owns 32 rows (one head, 32 positions). K/V tiles of 64 keys are
//   staged once in LDS and reused by all 4 waves, i.e. by all g_pack heads.
//   Tiles are visited only inside the rows' visible key range; per wave a
//   tile is computed without a mask or masked element by element.
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
// Pipeline (one barrier per 64-key tile)
//   K and V tiles go from HBM/L2 straight into LDS (global_load_lds_dwordx4,
//   no registers in between). Tile t's iteration issues the loads of V(t+1)
//   and K(t+2), computes S(t+1) = K(t+1) Q^T on the matrix cores while the
//   vector ALUs run the softmax of S(t), then accumulates P(t) V(t).
//   LDS rows are unpadded; 16-byte chunks are XOR-swizzled per row so that
//   both the K reads (16 rows, same chunk) and the transposed V reads (4 rows
//   x 4 chunks per half wave) hit distinct banks.
//
// Online softmax (fp32, log2 units): Q is multiplied by log2(e)/sqrt(d_h) as
// it is rotated and rounded to bf16, so a score is already the exponent for
// exp2. Each S^T chain starts its accumulator at -m (the running max as it
// was when the chain was issued) instead of zero, so the matrix cores deliver
// s - m and a probability costs one exp2, with no per-score vector arithmetic.
// The running max only moves when a tile's max exceeds it by more than 8:
// probabilities stay <= 2^8, and O and the running sum l are rescaled by
// exp2(m_old - m_new) only then; a tile whose chain started from an older m
// has its exponentials recomputed with the difference (rare: the first tiles
// of a row). O / l is exact for any such choice of m.
#pragma once
#include "device_common.hpp"

namespace apex {

// Four waves (128 query rows) per workgroup and two workgroups per CU: while
// one workgroup waits in its prologue (Q and first tiles in flight) or at a
// barrier, the other one's waves keep the SIMDs busy.
constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kPfRows = kPfWaves * 32;  // query rows per workgroup
constexpr int kPfBN = 64;               // keys per K/V tile
constexpr float kLazyMax = 8.0f;        // log2 headroom before the max moves

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;  // already rotated
  const uint16_t* v;
  uint16_t* o;
  int S, Hq, Hkv, G;
  int causal, W;
  int P;              // prefix rows (bidirectional within [0, P)); <= S
  long long m0;
  RopeTurns turns;    // theta_i / (2 pi) of the rotated pairs (YaRN applied)
  int apply_rope;     // rotate q while it loads
  int g_pack;         // query heads per workgroup (divides G, <= kPfWaves)
  int bm;             // positions per workgroup = kPfRows / g_pack
  int n_pos_tiles;    // ceil(S / bm)
  int n_head_packs;   // G / g_pack
  int n_groups;       // B * Hkv * n_head_packs
  float sc;           // log2(e) / sqrt(d_h)
};

// Physical 16-byte slot of logical chunk c in LDS row r of CPR chunks (and,
// being an involution, the logical chunk held in slot c). For 8 and 16 chunks
// the chunk index is XORed with row bits; for 24 chunks (a 192-wide row) the
// low three bits are, inside each group of eight. Either way the 16 rows that
// one K read touches with the same chunk land in 16 distinct bank groups.
template <int CPR>
__device__ __forceinline__ int slot(int c, int r) {
  static_assert(CPR == 8 || CPR == 16 || CPR == 24, "row width");
  if (CPR == 16) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  if (CPR == 8) return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  return (c & ~7) | ((c & 7) ^ ((r >> 1) & 7));
}

// True when every key of [j0, j0 + kPfBN) is visible to every row of
// [r0, r0 + 32) (Part 2, §10.2, §11.1), so the tile needs no mask: it lies
// below the smallest last-visible key of the rows (P - 1 for prefix rows, the
// row itself otherwise) and at or above the largest first-visible key (0 for
// prefix rows, row - W + 1 in a window).
// Bitwise, not short-circuit, so that it adds no branch to the loop body.
__device__ __forceinline__ bool tile_is_full(int j0, int r0, int S, int causal, int W, int P) {
  const int j1 = j0 + kPfBN - 1;
  const int min_hi = r0 < P ? P - 1 : r0;
  const int max_lo = ((W > 0) & (r0 + 31 >= P)) ? r0 + 32 - W : 0;
  return (j1 < S) & ((causal == 0) | ((j1 <= min_hi) & (j0 >= max_lo)));
}

// DQK: width of the q and k rows; DV: width of the v and o rows; DR: the
// last DR dims of q and k carry RoPE (DQK = DV = DR = d_h for the standard
// layers; DQK = d_h + d_r, DV = d_h, DR = d_r for MLA with decoupled RoPE,
// Part 2, §9.3).
template <int DQK, int DV, int DR>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_bf16_kernel(PrefillParams p) {
  static_assert(DQK % 16 == 0 && DV % 32 == 0 && DR % 16 == 0 && DR <= DQK, "head size");
  constexpr int RBK = DQK * 2, RBV = DV * 2;       // bytes per LDS row of K, V
  constexpr int CPRK = RBK / 16, CPRV = RBV / 16;  // 16-byte chunks per row
  constexpr int TILEK = kPfBN * RBK;               // bytes per K tile
  constexpr int TILEV = kPfBN * RBV;               // bytes per V tile
  constexpr int LOADSK = TILEK / 1024 / kPfWaves;  // 1 KB direct loads per wave per tile
  constexpr int LOADSV = TILEV / 1024 / kPfWaves;
  constexpr int KK = DQK / 16;                     // MFMA steps over the q.k width
  constexpr int KR = (DQK - DR) / 16;              // first step of the RoPE part
  constexpr int DB = DV / 32;                      // 32-wide blocks of the v width
  static_assert(LOADSK * kPfWaves * 1024 == TILEK && LOADSV * kPfWaves * 1024 == TILEV,
                "tile split");

  constexpr int NP = DR / 2;  // rotated pairs per row
  constexpr int CH = NP / 2;  // 16-byte chunks (two (cos, sin) pairs) per table row
  static_assert(CH == 16 || CH == 32, "angle table swizzle");
  static_assert(32 * NP * 8 <= TILEV, "angle table fits one V slot");

  __shared__ __attribute__((aligned(1024))) unsigned char kbuf[2][TILEK];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf[2][TILEV];
  // The Q angle table is needed only while Q loads, before V slot 1 first
  // receives a tile (after the prologue's second barrier): it borrows it.
  float2* const cs_lds = (float2*)vbuf[1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar
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

  // ---- key range of the workgroup ----
  int j_lo = 0, j_hi = p.S - 1;
  if (p.causal) {
    j_hi = min(p.S - 1, p0 + p.bm - 1);
    if (p0 < p.P) j_hi = max(j_hi, p.P - 1);               // prefix rows see the whole prefix
    if (p.W > 0 && p0 >= p.P) j_lo = max(0, p0 - p.W + 1);
  }
  const int t_lo = j_lo / kPfBN, t_hi = j_hi / kPfBN;

  const uint16_t* kg = p.k + ((size_t)b * p.Hkv + kvh) * p.S * DQK;
  const uint16_t* vg = p.v + ((size_t)b * p.Hkv + kvh) * p.S * DV;

  // ---- direct HBM -> LDS tile loads: lane order = physical LDS order ----
  // Byte offset inside a tile of the 16 bytes each lane copies per load: the
  // lane fills physical slot pc of the tile, which holds logical chunk
  // slot(pc % CPR, row) of row pc / CPR.
  uint32_t ldk_off[LOADSK], ldv_off[LOADSV];
#pragma unroll
  for (int i = 0; i < LOADSK; i++) {
    const int pc = (wave + i * kPfWaves) * 64 + lane;
    const int r = pc / CPRK;
    ldk_off[i] = (uint32_t)(r * RBK + (slot<CPRK>(pc % CPRK, r) << 4));
  }
#pragma unroll
  for (int i = 0; i < LOADSV; i++) {
    const int pc = (wave + i * kPfWaves) * 64 + lane;
    const int r = pc / CPRV;
    ldv_off[i] = (uint32_t)(r * RBV + (slot<CPRV>(pc % CPRV, r) << 4));
  }
  // The buffer resource of tile t covers the rows t*kPfBN .. S-1, so rows
  // past the sequence end arrive as zeros (and are masked anyway).
  auto issue_k = [&](unsigned char* dst, int t) {
    const buffer_rsrc r =
        make_buffer_rsrc(kg + (size_t)t * kPfBN * DQK, (uint32_t)(p.S - t * kPfBN) * RBK);
#pragma unroll
    for (int i = 0; i < LOADSK; i++)
      buffer_to_lds16(r, ldk_off[i],
                      (APEX_LDS void*)(uintptr_t)(lds_addr(dst) + (wave + i * kPfWaves) * 1024));
  };
  auto issue_v = [&](unsigned char* dst, int t) {
    const buffer_rsrc r =
        make_buffer_rsrc(vg + (size_t)t * kPfBN * DV, (uint32_t)(p.S - t * kPfBN) * RBV);
#pragma unroll
    for (int i = 0; i < LOADSV; i++)
      buffer_to_lds16(r, ldv_off[i],
                      (APEX_LDS void*)(uintptr_t)(lds_addr(dst) + (wave + i * kPfWaves) * 1024));
  };

  // When all waves hold the same 32 positions (a pack of 4 heads), cos/sin of
  // (m0 + p0 + r) theta_i are formed once per workgroup into an LDS table
  // [32 rows][NP pairs] and shared by the heads; 16-byte chunks are XORed
  // with the row so the 16 rows one read cycle serves hit distinct banks.
  // Thread tid fills the entries of pair tid % NP (kPfThreads is a multiple
  // of NP), so it needs one frequency, fetched before the big loads.
  static_assert(kPfThreads % NP == 0, "one frequency per thread");
  const bool shared_cs = p.apply_rope && pos_blocks == 1;
  const double my_turns = shared_cs ? p.turns.v[tid % NP] : 0.0;

  // ---- Q^T operand: lane holds row `row`, dims 16kk + 8g .. +7 ----
  // Its loads go out first so their latency overlaps the first tiles'; the
  // buffer covers this head's S rows, so rows past S read as zeros.
  u32x4 qf[KK];
  {
    const buffer_rsrc qr =
        make_buffer_rsrc(p.q + ((size_t)b * p.Hq + head) * p.S * DQK, (uint32_t)p.S * RBK);
    const uint32_t qoff = (uint32_t)row * RBK + 16 * g;
#pragma unroll
    for (int kk = 0; kk < KK; kk++) qf[kk] = buffer_load16(qr, qoff + 32 * kk);
  }

  issue_k(kbuf[0], t_lo);
  issue_v(vbuf[0], t_lo);
  if (t_lo < t_hi) issue_k(kbuf[1], t_lo + 1);

  // The angles are formed while the loads are in flight and written to LDS
  // after them (the table shares LDS with the tiles' direct loads).
  constexpr int NE = 32 * NP / kPfThreads;  // table entries per thread
  const int pr = tid % NP;
  float tc[NE], ts[NE];
  if (shared_cs) {
#pragma unroll
    for (int i = 0; i < NE; i++) {  // entries carry the score scale
      rope_cs_fast(p.m0 + p0 + tid / NP + i * (kPfThreads / NP), my_turns, tc[i], ts[i]);
      tc[i] *= p.sc;
      ts[i] *= p.sc;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's tile loads have landed
  if (shared_cs) {
#pragma unroll
    for (int i = 0; i < NE; i++) {
      const int r = tid / NP + i * (kPfThreads / NP);
      cs_lds[(r * CH + ((pr >> 1) ^ (r & (CH - 1)))) * 2 + (pr & 1)] = float2{tc[i], ts[i]};
    }
  }
  __syncthreads();  // every wave's tile loads and table entries are in LDS

  // ---- RoPE and score scale of the Q operand ----
  // q' = RoPE(q) * log2(e)/sqrt(d_h), rounded to bf16 once; dims outside the
  // rotated part (and all of them when nothing is rotated) are only scaled.
  const int kr_end = p.apply_rope ? KR : KK;
#pragma unroll
  for (int kk = 0; kk < KK; kk++)
    if (kk < kr_end) {
#pragma unroll
      for (int e = 0; e < 4; e++)
        qf[kk][e] = pack_bf16x2(bf16_lo(qf[kk][e]) * p.sc, bf16_hi(qf[kk][e]) * p.sc);
    }
  if (p.apply_rope) {
#pragma unroll
    for (int kk = KR; kk < KK; kk++) {  // the RoPE part: pairs of a DR-wide head
      const int pr0 = (16 * kk + 8 * g - (DQK - DR)) / 2;  // first of this lane's 4 pairs
      float c[4], s[4];
      if (shared_cs) {
        const int sw = r32 & (CH - 1);
        const f32x4 a = *(const f32x4*)&cs_lds[(r32 * CH + ((pr0 >> 1) ^ sw)) * 2];
        const f32x4 z = *(const f32x4*)&cs_lds[(r32 * CH + (((pr0 >> 1) + 1) ^ sw)) * 2];
        c[0] = a[0]; s[0] = a[1]; c[1] = a[2]; s[1] = a[3];
        c[2] = z[0]; s[2] = z[1]; c[3] = z[2]; s[3] = z[3];
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++) {
          rope_cs_fast(p.m0 + row, p.turns.v[pr0 + e], c[e], s[e]);
          c[e] *= p.sc;
          s[e] *= p.sc;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float x0 = bf16_lo(qf[kk][e]), x1 = bf16_hi(qf[kk][e]);
        qf[kk][e] = pack_bf16x2(x0 * c[e] - x1 * s[e], x0 * s[e] + x1 * c[e]);
      }
    }
  }

  // ---- per-lane LDS offsets (loop invariant) ----
  // K operand: row kb*32 + r32, logical chunk 2kk + g. With 24-chunk rows
  // the offsets are formed in the loop instead of held: the swizzle only
  // flips bits 5-6 of the byte offset (kk mod 4 selects which), and kk / 4
  // adds 128 bytes, so offset(kk) = (offset(0) ^ 32 (kk mod 4)) + 128 (kk / 4).
  constexpr bool kXorK = CPRK == 24;
  int k_off[kXorK ? 1 : KK];
#pragma unroll
  for (int kk = 0; kk < (kXorK ? 1 : KK); kk++)
    k_off[kk] = r32 * RBK + (slot<CPRK>(2 * kk + g, r32) << 4);
  const uint32_t kq = lds_addr(kbuf[0]) + (uint32_t)k_off[0];
  auto k_operand = [&](const unsigned char* kb_lds, int kb, int kk) {
    if (kXorK) {
      const uint32_t a = (opaque(kq) ^ (uint32_t)(32 * (kk & 3))) +
                         (uint32_t)(kb_lds - &kbuf[0][0]) + kb * 32 * RBK + 128 * (kk >> 2);
      return lds_read16_at(a);
    }
    return *(const u32x4*)(kb_lds + kb * 32 * RBK + k_off[kk]);
  };
  // V^T operand via ds_read_b64_tr_b16: lane j16 of 16-lane group qg reads 8 bytes
  // at row key + j16/4, columns 32db + 16(qg&1) + 4(j16&3): logical chunk
  // 4db + 2(qg&1) + (j16&3)/2, half (j16&1). Rows +8 give the k-indices 4..7.
  const int j16 = lane & 15;
  const int vrow = 4 * g + (j16 >> 2);
  int v_off[2][DB];
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int r = vrow + 8 * h;
#pragma unroll
    for (int db = 0; db < DB; db++) {
      const int chunk = 4 * db + 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1);
      v_off[h][db] = r * RBV + (slot<CPRV>(chunk, r) << 4) + ((j16 & 1) << 3);
    }
  }

  // S^T - m for 64 keys: both 32-key chains start from -m (every element of
  // a lane holds its row's value).
  auto qk = [&](const unsigned char* kb_lds, f32x16 (&s)[2], float m) {
    f32x16 negm;
#pragma unroll
    for (int r = 0; r < 16; r++) negm[r] = -m;
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      s[kb] = negm;
#pragma unroll
      for (int kk = 0; kk < KK; kk++)
        s[kb] = mfma32(k_operand(kb_lds, kb, kk), qf[kk], s[kb]);
    }
  };

  // visible keys of this lane's row: [vis_lo, vis_hi]
  const int vis_hi = !p.causal ? p.S - 1 : (row < p.P ? p.P - 1 : min(row, p.S - 1));
  const int vis_lo = (p.causal && p.W > 0 && row >= p.P) ? row - p.W + 1 : 0;
  const unsigned vis_span = (unsigned)(vis_hi - vis_lo);

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; db++) oacc[db] = f32x16{};
  // m_run: running row max (log2 units, -inf until a key is seen); m_use:
  // its finite stand-in, which O and l are relative to and the next S^T chain
  // starts from; m_a: the value the chain of s_cur started from.
  float m_run = kNegInf, m_use = 0.0f, m_a = 0.0f, l_run = 0.0f;

  // Tile t's mask (unless the tile is full) and the row max of its scores,
  // absolute (both halves of the wave hold keys of the row).
  // The max is taken first over the unmasked scores, so that it needs no
  // branch and can run beside the P V matrix instructions; a partial tile
  // (rare: the diagonal and window edges) is then masked and its max retaken.
  auto row_max = [&](const f32x16 (&sc)[2]) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int r = 0; r < 16; r++) mx = fmaxf(mx, sc[kb][r]);
    return fmaxf(mx, lane_xor32(mx));
  };
  auto mask_max = [&](int t, f32x16 (&sc)[2], bool full, float m_from) {
    float mx = row_max(sc);
    if (!full) {
      const int base = t * kPfBN + 4 * g - vis_lo;
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const unsigned off = (unsigned)(base + kb * 32 + 8 * (r >> 2) + (r & 3));
          sc[kb][r] = off <= vis_span ? sc[kb][r] : kNegInf;
        }
      mx = row_max(sc);
    }
    return mx + m_from;
  };

  f32x16 sa[2], sb[2];
  qk(kbuf[0], sa, 0.0f);
  const bool full_lo = tile_is_full(t_lo * kPfBN, pw, p.S, p.causal, p.W, p.P);
  float mx_a = mask_max(t_lo, sa, full_lo, 0.0f), mx_b = kNegInf;
  __syncthreads();  // every wave is done with kbuf[0] before K(t_lo + 2) lands there

  // One 64-key tile. On entry s_cur = S(t) - m_a, masked, with row max mx_cur.
  // The max update comes first, so S(t+1) - m = K(t+1) Q^T - m is issued to
  // the matrix cores with the current m while the vector ALUs run the
  // exponentials of S(t); then O += P(t) V(t), beside which S(t+1) is masked
  // and its max taken. On the last tile (LAST) nothing further is loaded or
  // issued and no barrier follows: no wave reads the K buffers after the
  // previous tile's barrier.
  auto step = [&](int t, f32x16 (&s_cur)[2], f32x16 (&s_next)[2], float mx_cur, float& mx_next,
                  auto last_c) {
    constexpr bool LAST = decltype(last_c)::value != 0;
    const int it = t - t_lo;
    if (!LAST) {
      issue_v(vbuf[(it + 1) & 1], t + 1);
      if (t + 2 <= t_hi) issue_k(kbuf[it & 1], t + 2);
    }

    // the max moves (for every lane of the wave) only when some lane's tile
    // max exceeds its running max by more than kLazyMax
    if (__builtin_amdgcn_ballot_w64(mx_cur > m_run + kLazyMax) != 0) {  // wave-uniform, rare
      const float m_new = fmaxf(m_run, mx_cur);
      const float m_new_use = m_new == kNegInf ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new_use);
      m_run = m_new;
      m_use = m_new_use;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; db++) oacc[db] *= alpha;
    }
    // scores from a chain that started at an older m move to the current one
    if (__builtin_amdgcn_ballot_w64(m_use != m_a) != 0) {
      const float shift = m_use - m_a;
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++) s_cur[kb][r] -= shift;
    }
    m_a = m_use;

    if (!LAST) qk(kbuf[(it + 1) & 1], s_next, m_use);

    // P(t) = exp2(s - m), rounded to bf16 as the P V operand, and its row sum
    float lsum = 0.0f;
    u32x4 pk[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int c = 0; c < 2; c++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float e0 = __builtin_amdgcn_exp2f(s_cur[kb][8 * c + 2 * e]);
          const float e1 = __builtin_amdgcn_exp2f(s_cur[kb][8 * c + 2 * e + 1]);
          pk[kb][c][e] = pack_bf16x2(e0, e1);
          lsum = add_bf16x2(pk[kb][c][e], lsum);  // the row sum of the rounded P that P V uses
        }
    // the row sum is formed here, beside the S(t+1) matrix instructions, not
    // sunk to where l is next needed
    asm volatile("" ::"v"(lsum));
    l_run += lsum;

    // The two workgroups' waves share each SIMD; while this wave accumulates
    // P V it yields issue priority to a wave in its score/softmax phase, whose
    // vector work can then run beside these matrix-core instructions.
    __builtin_amdgcn_s_setprio(0);
    // O^T += V^T P^T. Operand k-index 8g+e <-> key kb*32 + 16c + 4g + e (e < 4)
    // and kb*32 + 16c + 8 + 4g + (e - 4) (e >= 4), matching the S^T layout.
    const unsigned char* vb = vbuf[it & 1];
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int c = 0; c < 2; c++) {
          const int koff = (kb * 32 + 16 * c) * RBV;
          const u32x2 lo = lds_read_tr16((const uint16_t*)(vb + koff + v_off[0][db]));
          const u32x2 hi = lds_read_tr16((const uint16_t*)(vb + koff + v_off[1][db]));
          oacc[db] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pk[kb][c], oacc[db]);
        }
    if (!LAST)
      mx_next = mask_max(t + 1, s_next,
                         tile_is_full((t + 1) * kPfBN, pw, p.S, p.causal, p.W, p.P), m_use);
    __builtin_amdgcn_s_setprio(1);  // back to the score/softmax phase
    if (!LAST) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // V(t+1), K(t+2) have landed
      __syncthreads();
    }
  };

  int t = t_lo;
  for (; t + 2 <= t_hi; t += 2) {
    step(t, sa, sb, mx_a, mx_b, Int<0>{});
    step(t + 1, sb, sa, mx_b, mx_a, Int<0>{});
  }
  if (t < t_hi) {
    step(t, sa, sb, mx_a, mx_b, Int<0>{});
    step(t + 1, sb, sa, mx_b, mx_a, Int<1>{});
  } else {
    step(t, sa, sb, mx_a, mx_b, Int<1>{});
  }

  // ---- epilogue: O = O^T / l, rounded to bf16 ----
  // A lane holds 4-dim pieces of one row, so direct stores would scatter over
  // 32 rows per instruction. The rows go through this wave's slice of the K
  // buffers (free after the last barrier) instead: written as held, read back
  // as whole 16-byte chunks, stored as four complete rows (1 KB contiguous)
  // per instruction. 16-byte chunks are XORed with the row against bank
  // conflicts.
  constexpr int CHV = DV / 8;  // 16-byte chunks per O row
  static_assert(kPfWaves * 32 * DV * 2 <= 2 * TILEK, "O staging fits the K buffers");
  const float l_tot = l_run + lane_xor32(l_run);
  const float inv = 1.0f / l_tot;
  unsigned char* const ost = &kbuf[0][0] + wave * 32 * DV * 2;
#pragma unroll
  for (int db = 0; db < DB; db++)
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      const int c = 4 * db + q4;  // chunk of dims 8c .. 8c+7; lane half g holds 4 of them
      u32x2 w;
      w[0] = pack_bf16x2(oacc[db][4 * q4 + 0] * inv, oacc[db][4 * q4 + 1] * inv);
      w[1] = pack_bf16x2(oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv);
      *(u32x2*)(ost + r32 * (DV * 2) + ((c ^ (r32 & (CHV - 1))) << 4) + 8 * g) = w;
    }
  uint16_t* const ohead = p.o + ((size_t)b * p.Hq + head) * p.S * DV;
#pragma unroll
  for (int i = 0; i < 32 * CHV / 64; i++) {
    const int rr = i * (64 / CHV) + lane / CHV, c = lane % CHV;
    const u32x4 v = *(const u32x4*)(ost + rr * (DV * 2) + ((c ^ (rr & (CHV - 1))) << 4));
    if (pw + rr < p.S) *(u32x4*)(ohead + (size_t)(pw + rr) * DV + 8 * c) = v;
  }
}

}  // namespace apex
