// rmsnorm_kernel.hpp -- y = x / sqrt(mean(x^2) + eps) * gamma over rows of d
// features (APEX-1 Mathematical Reference, Part 1, §3.2 "Formula").
//
// HBM-bound: every byte of x is read once and every byte of y written once.
// One wave owns a row at a time; lane l holds the 16-byte chunks l, l + 64,
// l + 128, ... of it, so each wave-wide load or store covers 1 KB of
// contiguous memory. gamma is staged in LDS once per workgroup and reused
// for all the rows its waves visit (grid-stride over rows). The sum of
// squares is accumulated in fp32 and reduced across the wave with lane
// exchanges; the output is rounded once from fp32.
#pragma once
#include "device_common.hpp"

namespace apex {

constexpr int kRmsThreads = 256;  // 4 waves, one row each at a time

struct RmsNormParams {
  const void* x;
  const void* gamma;
  void* y;        // may equal x
  long long rows;
  int d;          // multiple of 8
  float eps;
};

// 8 consecutive features of one row: 16 bytes of bf16 or 32 bytes of fp32.
template <typename T>
struct RmsChunk;

template <>
struct RmsChunk<uint16_t> {
  static constexpr int kBytes = 16;
  u32x4 w;
  __device__ __forceinline__ void load(const void* p, size_t chunk) {
    w = *((const u32x4*)p + chunk);
  }
  __device__ __forceinline__ float get(int e) const {
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
  }
  __device__ __forceinline__ void keep_packed() { asm volatile("" : "+v"(w)); }
  __device__ __forceinline__ static void store(void* p, size_t chunk, const float* v) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; e++) o[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
    *((u32x4*)p + chunk) = o;
  }
};

template <>
struct RmsChunk<float> {
  static constexpr int kBytes = 32;
  f32x4 a, b;
  __device__ __forceinline__ void load(const void* p, size_t chunk) {
    const f32x4* s = (const f32x4*)p + 2 * chunk;
    a = s[0];
    b = s[1];
  }
  __device__ __forceinline__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
  __device__ __forceinline__ void keep_packed() {}
  __device__ __forceinline__ static void store(void* p, size_t chunk, const float* v) {
    f32x4* o = (f32x4*)p + 2 * chunk;
    o[0] = f32x4{v[0], v[1], v[2], v[3]};
    o[1] = f32x4{v[4], v[5], v[6], v[7]};
  }
};

// NC = chunks per lane (ceil(d / 512)): the row lives in registers between
// the sum of squares and the scaled store.
template <typename T, int NC>
__global__ __launch_bounds__(kRmsThreads) void rmsnorm_kernel(RmsNormParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char g_lds[NC * 64 * RmsChunk<T>::kBytes];
  const int lane = threadIdx.x & 63;
  const long long wave0 = (long long)blockIdx.x * (kRmsThreads / 64) + (threadIdx.x >> 6);
  const long long n_waves = (long long)gridDim.x * (kRmsThreads / 64);
  const int nch = p.d >> 3;
  const float inv_d = 1.0f / (float)p.d;

  const int gwords = nch * RmsChunk<T>::kBytes / 16;
  for (int i = threadIdx.x; i < gwords; i += kRmsThreads)
    ((u32x4*)g_lds)[i] = ((const u32x4*)p.gamma)[i];
  __syncthreads();

  for (long long row = wave0; row < p.rows; row += n_waves) {
    const size_t base = (size_t)row * nch;
    RmsChunk<T> xv[NC];
#pragma unroll
    for (int c = 0; c < NC; c++)
      if (lane + 64 * c < nch) xv[c].load(p.x, base + lane + 64 * c);
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; c++)
      if (lane + 64 * c < nch)
#pragma unroll
        for (int e = 0; e < 8; e++) ss = __builtin_fmaf(xv[c].get(e), xv[c].get(e), ss);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float inv_rms = 1.0f / __builtin_sqrtf(ss * inv_d + p.eps);
#pragma unroll
    for (int c = 0; c < NC; c++)
      if (lane + 64 * c < nch) {
        RmsChunk<T> g;
        g.load(g_lds, lane + 64 * c);
        xv[c].keep_packed();  // unpack again here rather than hold the fp32 values
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; e++) o[e] = xv[c].get(e) * inv_rms * g.get(e);
        RmsChunk<T>::store(p.y, base + lane + 64 * c, o);
      }
  }
}

}  // namespace apex
