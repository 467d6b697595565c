// rope_kernel.hpp -- standalone rotary position embedding over [B, H, S, d_h]
// (APEX-1 Mathematical Reference, Part 1, §4.2 "Core Idea", §4.3 "Frequency
// Formula", §4.4 "Compact Form" with adjacent pairs (2i, 2i+1)).
//
// HBM-bound elementwise pass. A thread owns one 8-element chunk (4 pairs) of
// the head vector for kRopeRows consecutive positions of one (b, h): it issues
// all of their loads first, forms cos/sin of p*theta_i exactly (fp64 turns,
// accurate fp32 sincos) for the first position and steps to the next
// positions by one complex multiplication with (cos theta_i, sin theta_i),
// taken from a per-block table, then stores the rows. Consecutive threads
// cover consecutive chunks of a row, so a wave reads and writes whole rows
// (coalesced 16- or 32-byte accesses).
//
// A row may be wider than the rotated part: with MLA's decoupled RoPE (Part 2,
// §9.3) only the last d_r dims of each [content | rope] row turn, with the
// frequencies of a d_r-wide head. The other chunks are copied when the output
// is a separate buffer and left alone in place.
#pragma once
#include "device_common.hpp"

namespace apex {

constexpr int kRopeRows = 4;
constexpr int kRopeThreads = 256;

struct RopeParams {
  const void* src;
  void* dst;           // may equal src
  long long n_bh;      // B * H
  int S;
  int d_h;             // width of the rotated part (its frequencies follow d_h)
  int row_len;         // elements per row, >= d_h; the rotated part is the last d_h
  long long m0;
  RopeTurns turns;     // theta_i / (2 pi) of the d_h / 2 pairs (YaRN applied)
};

template <typename T>
struct RopeIO;

template <>
struct RopeIO<uint16_t> {  // bf16: 8 elements = 16 bytes
  static __device__ __forceinline__ void load(const void* p, size_t off, float* x) {
    u32x4 w = *(const u32x4*)((const uint16_t*)p + off);
#pragma unroll
    for (int e = 0; e < 4; e++) { x[2 * e] = bf16_lo(w[e]); x[2 * e + 1] = bf16_hi(w[e]); }
  }
  static __device__ __forceinline__ void store(void* p, size_t off, const float* x) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; e++) w[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    *(u32x4*)((uint16_t*)p + off) = w;
  }
};

template <>
struct RopeIO<float> {  // fp32: 8 elements = 32 bytes
  static __device__ __forceinline__ void load(const void* p, size_t off, float* x) {
    const f32x4* s = (const f32x4*)((const float*)p + off);
    f32x4 a = s[0], b = s[1];
#pragma unroll
    for (int e = 0; e < 4; e++) { x[e] = a[e]; x[4 + e] = b[e]; }
  }
  static __device__ __forceinline__ void store(void* p, size_t off, const float* x) {
    f32x4* d = (f32x4*)((float*)p + off);
    d[0] = f32x4{x[0], x[1], x[2], x[3]};
    d[1] = f32x4{x[4], x[5], x[6], x[7]};
  }
};

template <typename T>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(RopeParams p) {
  __shared__ double turns_lds[kMaxRopePairs];  // theta_i / (2 pi), i < d_h / 2
  __shared__ float step_c[kMaxRopePairs], step_s[kMaxRopePairs];  // cos, sin of theta_i
  if ((int)threadIdx.x < p.d_h / 2) {
    const double turns = p.turns.v[threadIdx.x];
    turns_lds[threadIdx.x] = turns;
    rope_cs_accurate(1, turns, step_c[threadIdx.x], step_s[threadIdx.x]);
  }
  __syncthreads();
  // Chunks of 8 visited per row: the whole row out of place, the rotated part
  // in place; chunk index rc0 is the first rotated one.
  const int rc0 = (p.row_len - p.d_h) >> 3;
  const int first = p.src == p.dst ? rc0 : 0;
  const int chunks = (p.row_len >> 3) - first;
  const int row_blocks = (p.S + kRopeRows - 1) / kRopeRows;
  const long long total = p.n_bh * row_blocks * chunks;
  for (long long t = blockIdx.x * (long long)kRopeThreads + threadIdx.x; t < total;
       t += (long long)gridDim.x * kRopeThreads) {
    const int ch = first + (int)(t % chunks);
    const long long rb_all = t / chunks;
    const int rb = (int)(rb_all % row_blocks);
    const long long bh = rb_all / row_blocks;
    const int s0 = rb * kRopeRows;
    const int rows = min(kRopeRows, p.S - s0);
    const size_t off0 = ((size_t)bh * p.S + s0) * p.row_len + ch * 8;
    float x[kRopeRows][8];
#pragma unroll
    for (int r = 0; r < kRopeRows; r++)
      if (r < rows) RopeIO<T>::load(p.src, off0 + (size_t)r * p.row_len, x[r]);
    if (ch >= rc0) {
      const int pi = (ch - rc0) * 4;  // first pair of this chunk in the rotated part
      float c[4], s[4];
#pragma unroll
      for (int e = 0; e < 4; e++) rope_cs_accurate(p.m0 + s0, turns_lds[pi + e], c[e], s[e]);
#pragma unroll
      for (int r = 0; r < kRopeRows; r++) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float a = x[r][2 * e], b = x[r][2 * e + 1];
          x[r][2 * e] = a * c[e] - b * s[e];
          x[r][2 * e + 1] = a * s[e] + b * c[e];
          const float cs = step_c[pi + e], ss = step_s[pi + e];
          const float cn = c[e] * cs - s[e] * ss;
          s[e] = c[e] * ss + s[e] * cs;
          c[e] = cn;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kRopeRows; r++)
      if (r < rows) RopeIO<T>::store(p.dst, off0 + (size_t)r * p.row_len, x[r]);
  }
}

}  // namespace apex
