// prefill_f32_kernel.hpp -- attention prefill with fp32 storage and fp32 math
// (APEX-1 Mathematical Reference, Part 2, §6.2, §8.2, §10.2, §11.1; Q rotated by
// RoPE, Part 1, §4.2, as it loads).
//
// The fp32 workloads are small (correctness-sized), so this kernel is a plain
// vector-ALU flash loop: two lanes share one query row, each holding half of
// the head dimension of q and of the output accumulator; the two half dot
// products are summed with one lane exchange. A workgroup covers 128
// consecutive rows of one query head; K/V tiles of 32 keys are staged in LDS
// and read by broadcast. Scores of a tile are formed first, then one online
// softmax update (running max and sum in fp32) per tile.
#pragma once
#include "device_common.hpp"

namespace apex {

constexpr int kF32Threads = 256;
constexpr int kF32Rows = kF32Threads / 2;
constexpr int kF32BN = 32;

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

template <int D>
__global__ __launch_bounds__(kF32Threads) void prefill_f32_kernel(PrefillF32Params p) {
  constexpr int H = D / 2;  // dims per lane
  __shared__ float kt[kF32BN][D];
  __shared__ float vt[kF32BN][D];
  __shared__ double turns_lds[D / 2];

  const int tid = threadIdx.x;
  const int half = tid & 1;
  const int r0 = blockIdx.x * kF32Rows;
  const int row = r0 + (tid >> 1);
  const int h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / p.G;

  if (p.apply_rope) {
    if (tid < D / 2) turns_lds[tid] = p.turns.v[tid];
    __syncthreads();
  }

  float q[H], acc[H];
  const float* qrow = p.q + (((size_t)b * p.Hq + h) * p.S + row) * D + half * H;
#pragma unroll
  for (int t = 0; t < H; t++) {
    q[t] = row < p.S ? qrow[t] : 0.0f;
    acc[t] = 0.0f;
  }
  if (p.apply_rope) {
#pragma unroll
    for (int t = 0; t < H; t += 2) {
      float c, s;
      rope_cs_accurate(p.m0 + row, turns_lds[(half * H + t) / 2], c, s);
      const float a = q[t], bb = q[t + 1];
      q[t] = a * c - bb * s;
      q[t + 1] = a * s + bb * c;
    }
  }

  int j_lo = 0, j_hi = p.S - 1;
  if (p.causal) {
    j_hi = min(p.S - 1, r0 + kF32Rows - 1);
    if (r0 < p.P) j_hi = max(j_hi, p.P - 1);             // prefix rows see the whole prefix
    if (p.W > 0 && r0 >= p.P) j_lo = max(0, r0 - p.W + 1);
  }
  const float* kbase = p.k + ((size_t)b * p.Hkv + kvh) * p.S * D;
  const float* vbase = p.v + ((size_t)b * p.Hkv + kvh) * p.S * D;
  float m_run = kNegInf, l_run = 0.0f;

  for (int j0 = (j_lo / kF32BN) * kF32BN; j0 <= j_hi; j0 += kF32BN) {
    __syncthreads();
    for (int i = tid; i < kF32BN * D; i += kF32Threads) {
      const int jr = i / D, col = i % D;
      const bool ok = j0 + jr < p.S;
      kt[jr][col] = ok ? kbase[(size_t)(j0 + jr) * D + col] : 0.0f;
      vt[jr][col] = ok ? vbase[(size_t)(j0 + jr) * D + col] : 0.0f;
    }
    __syncthreads();
    float sc[kF32BN];
    float mx = kNegInf;
#pragma unroll
    for (int jj = 0; jj < kF32BN; jj++) {
      float dot = 0.0f;
#pragma unroll
      for (int t = 0; t < H; t++) dot += q[t] * kt[jj][half * H + t];
      dot += __shfl_xor(dot, 1, 64);
      const int j = j0 + jj;
      bool vis = j < p.S;
      if (p.causal)
        vis = vis && (row < p.P ? j < p.P : (j <= row && (p.W == 0 || row - j < p.W)));
      sc[jj] = vis ? dot * p.scale : kNegInf;
      mx = fmaxf(mx, sc[jj]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = expf(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < H; t++) acc[t] *= alpha;
#pragma unroll
    for (int jj = 0; jj < kF32BN; jj++) {
      const float e = expf(sc[jj] - m_use);
      l_run += e;
#pragma unroll
      for (int t = 0; t < H; t++) acc[t] += e * vt[jj][half * H + t];
    }
    m_run = m_new;
  }

  if (row < p.S) {
    const float inv = 1.0f / l_run;
    float* orow = p.o + (((size_t)b * p.Hq + h) * p.S + row) * D + half * H;
#pragma unroll
    for (int t = 0; t < H; t++) orow[t] = acc[t] * inv;
  }
}

}  // namespace apex
