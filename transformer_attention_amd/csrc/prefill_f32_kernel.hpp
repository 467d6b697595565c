// prefill_f32_kernel.hpp -- attention prefill with fp32 storage and fp32 math
// (APEX-1 Mathematical Reference, Part 2, §6.2, §8.2, §10.2, §11.1; Q rotated by
// RoPE, Part 1, §4.2, as it loads).
//
// The fp32 workloads are small (correctness-sized), so this kernel is a plain
// vector-ALU flash loop tuned for latency rather than throughput: eight lanes
// share one query row and a workgroup covers 32 rows of one query head, so
// even a short sequence spreads over many workgroups. K/V tiles of 32 keys
// are staged in LDS; the next tile's loads are in flight in registers while
// the current one is computed. For a tile, each lane forms the partial dot products of
// its eighth of the head dimension with all 32 keys; a reduce-scatter across
// the row's eight lanes (three exchange rounds) leaves each lane with the full
// scores of four keys, so the mask, the exponentials and the row sums are
// spread over the lanes; the probabilities are then gathered back so each lane
// accumulates P V over its eighth of the output dimension. One online softmax
// update (running max and sum in fp32) per tile.
#pragma once
#include "device_common.hpp"

namespace apex {

constexpr int kF32Threads = 256;
constexpr int kF32Lanes = 8;                       // lanes sharing one query row
constexpr int kF32Rows = kF32Threads / kF32Lanes;  // query rows per workgroup
constexpr int kF32BN = 32;                         // keys per LDS tile
constexpr int kF32Own = kF32BN / kF32Lanes;        // keys whose full score a lane holds

struct PrefillF32Params {
  const float* q;
  const float* k;  // already rotated
  const float* v;
  float* o;
  int S, Hq, Hkv, G;
  int causal, W;
  int P;              // prefix rows (bidirectional within [0, P)); <= S
  long long m0;
  RopeTurns turns;    // theta_i / (2 pi) per pair (YaRN applied)
  int apply_rope;
  float scale;  // 1 / sqrt(d_h), times the YaRN temperature
};

// One exchange round of the reduce-scatter: of the N values v[0..N) (keys
// split into a lower and an upper half), the lane whose `up` bit is set keeps
// the upper half and the other lane of the pair (lane ^ mask) the lower one;
// each sends the half it gives up and adds what it receives to the half it
// keeps, which ends in v[0..N/2).
template <int N>
__device__ __forceinline__ void reduce_half(float (&v)[kF32BN], bool up, int mask) {
#pragma unroll
  for (int i = 0; i < N / 2; i++) {
    const float send = up ? v[i] : v[N / 2 + i];
    const float keep = up ? v[N / 2 + i] : v[i];
    v[i] = keep + __shfl_xor(send, mask, 64);
  }
}

template <int D>
__global__ __launch_bounds__(kF32Threads) void prefill_f32_kernel(PrefillF32Params p) {
  constexpr int H = D / kF32Lanes;  // dims per lane
  static_assert(H % 4 == 0 && kF32Lanes == 8 && kF32BN == 32, "lane split");
  __shared__ __attribute__((aligned(16))) float kt[kF32BN][D];
  __shared__ __attribute__((aligned(16))) float vt[kF32BN][D];
  __shared__ double turns_lds[D / 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int sub = tid & (kF32Lanes - 1);  // dims sub*H .. +H-1; after the reduction, keys 4 sub .. +3
  const int grp = lane & ~(kF32Lanes - 1);
  const int r0 = blockIdx.x * kF32Rows;
  const int row = r0 + tid / kF32Lanes;
  const int h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / p.G;

  // The frequency, the first K/V tile and the q row are all requested before
  // anything waits for one of them.
  const double my_turns = (p.apply_rope && tid < D / 2) ? p.turns.v[tid] : 0.0;

  int j_lo = 0, j_hi = p.S - 1;
  if (p.causal) {
    j_hi = min(p.S - 1, r0 + kF32Rows - 1);
    if (r0 < p.P) j_hi = max(j_hi, p.P - 1);             // prefix rows see the whole prefix
    if (p.W > 0 && r0 >= p.P) j_lo = max(0, r0 - p.W + 1);
  }
  const float* kbase = p.k + ((size_t)b * p.Hkv + kvh) * p.S * D;
  const float* vbase = p.v + ((size_t)b * p.Hkv + kvh) * p.S * D;
  float m_run = kNegInf, l_run = 0.0f;

  // a tile is kF32BN rows of D floats; thread tid moves the float4s tid + n * kF32Threads
  constexpr int NL = kF32BN * D / 4 / kF32Threads;
  static_assert(NL * kF32Threads * 4 == kF32BN * D, "tile split");
  float4 kn[NL], vn[NL];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int n = 0; n < NL; n++) {
      const int i = tid + n * kF32Threads, jr = i / (D / 4), c4 = i % (D / 4);
      const bool ok = j0 + jr < p.S;
      const size_t off = (size_t)(j0 + jr) * D + 4 * c4;
      kn[n] = ok ? *(const float4*)(kbase + off) : float4{0.f, 0.f, 0.f, 0.f};
      vn[n] = ok ? *(const float4*)(vbase + off) : float4{0.f, 0.f, 0.f, 0.f};
    }
  };
  const int j_first = (j_lo / kF32BN) * kF32BN;
  load_tile(j_first);

  float q[H], acc[H];
  const float* qrow = p.q + (((size_t)b * p.Hq + h) * p.S + row) * D + sub * H;
#pragma unroll
  for (int t = 0; t < H; t++) {
    q[t] = row < p.S ? qrow[t] : 0.0f;
    acc[t] = 0.0f;
  }
  if (p.apply_rope) {
    if (tid < D / 2) turns_lds[tid] = my_turns;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < H; t += 2) {  // pairs (2i, 2i+1) never straddle two lanes' slices
      float c, s;
      rope_cs_accurate(p.m0 + row, turns_lds[(sub * H + t) / 2], c, s);
      const float a = q[t], bb = q[t + 1];
      q[t] = a * c - bb * s;
      q[t + 1] = a * s + bb * c;
    }
  }

  for (int j0 = j_first; j0 <= j_hi; j0 += kF32BN) {
    __syncthreads();  // every lane is done reading the previous tile
#pragma unroll
    for (int n = 0; n < NL; n++) {
      const int i = tid + n * kF32Threads, jr = i / (D / 4), c4 = i % (D / 4);
      *(float4*)&kt[jr][4 * c4] = kn[n];
      *(float4*)&vt[jr][4 * c4] = vn[n];
    }
    __syncthreads();
    if (j0 + kF32BN <= j_hi) load_tile(j0 + kF32BN);

    // partial q.k over this lane's dims for every key of the tile
    float part[kF32BN];
#pragma unroll
    for (int jj = 0; jj < kF32BN; jj++) {
      float d = 0.0f;
#pragma unroll
      for (int t = 0; t < H; t++) d += q[t] * kt[jj][sub * H + t];
      part[jj] = d;
    }
    // reduce-scatter over the row's lanes: part[0..3] = full scores of keys 4 sub .. +3
    reduce_half<32>(part, (sub & 4) != 0, 4);
    reduce_half<16>(part, (sub & 2) != 0, 2);
    reduce_half<8>(part, (sub & 1) != 0, 1);

    float sc[kF32Own];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < kF32Own; i++) {
      const int j = j0 + kF32Own * sub + i;
      bool vis = j < p.S;
      if (p.causal)
        vis = vis && (row < p.P ? j < p.P : (j <= row && (p.W == 0 || row - j < p.W)));
      sc[i] = vis ? part[i] * p.scale : kNegInf;
      mx = fmaxf(mx, sc[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = expf(m_run - m_use);
    float e[kF32Own], lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < kF32Own; i++) {
      e[i] = expf(sc[i] - m_use);
      lsum += e[i];
    }
    lsum += __shfl_xor(lsum, 1, 64);
    lsum += __shfl_xor(lsum, 2, 64);
    lsum += __shfl_xor(lsum, 4, 64);
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int t = 0; t < H; t++) acc[t] *= alpha;
    // P V: the probability of key jj is held by lane grp + jj / 4 as e[jj % 4]
#pragma unroll
    for (int jj = 0; jj < kF32BN; jj++) {
      const float ej = __shfl(e[jj % kF32Own], grp + jj / kF32Own, 64);
#pragma unroll
      for (int t = 0; t < H; t++) acc[t] += ej * vt[jj][sub * H + t];
    }
    m_run = m_new;
  }

  if (row < p.S) {
    const float inv = 1.0f / l_run;
    float* orow = p.o + (((size_t)b * p.Hq + h) * p.S + row) * D + sub * H;
#pragma unroll
    for (int t = 0; t < H; t += 4)
      *(float4*)(orow + t) = float4{acc[t] * inv, acc[t + 1] * inv, acc[t + 2] * inv, acc[t + 3] * inv};
  }
}

}  // namespace apex
