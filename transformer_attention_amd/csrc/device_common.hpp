// device_common.hpp -- gfx950 building blocks shared by the RoPE, prefill and
// decode kernels: vector types, bf16 packing, MFMA wrappers, the transposing
// LDS read, and the RoPE angle evaluation.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace apex {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define APEX_LDS __attribute__((address_space(3)))

constexpr float kNegInf = -__builtin_inff();
constexpr double kInvTwoPi = 0.15915494309189533576888376337251436;  // 1 / (2 pi)

// ---- bf16 <-> fp32 -------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Round two fp32 values to bf16 (nearest even) and pack them, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float a) {
  return __builtin_bit_cast(uint16_t, (__bf16)a);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// ---- MFMA ------------------------------------------------------------------
// v_mfma_f32_32x32x16_bf16. Lane l supplies A[l%32][8(l/32)+e] and
// B[8(l/32)+e][l%32], e = 0..7; D[8(r/4)+4(l/32)+r%4][l%32] lands in reg r.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// v_mfma_f32_16x16x32_bf16. Lane l supplies A[l%16][8(l/16)+e] and
// B[8(l/16)+e][l%16]; D[4(l/16)+r][l%16] lands in reg r.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j names an 8-byte
// chunk (4 bf16); lane i receives element i%4 of the chunks named by lanes
// i/4, 4+i/4, 8+i/4, 12+i/4. When lane j points at row (r0 + j/4), columns
// c0 + 4(j%4) .. +3 of a row-major LDS matrix, lane i receives the column
// c0 + i over the rows r0 .. r0+3: a 4x16 transpose.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((APEX_LDS i16x4*)(APEX_LDS void*)p);
  return __builtin_bit_cast(u32x2, v);
}

// global_load_lds_dwordx4: each lane copies 16 bytes from its global address
// straight into LDS at lds_base + 16 * lane (lds_base wave-uniform), without
// passing through registers. The builtin exists only for the device target, so
// the host pass of this file (which only emits launch stubs) does not see it.
__device__ __forceinline__ void global_to_lds16(const void* src, APEX_LDS void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
#endif
}

// buffer_load_dwordx4 ... lds: the same copy as global_to_lds16, addressed
// through a buffer resource (wave-uniform base and byte size, built on the
// scalar unit) plus a per-lane byte offset. Lanes whose offset lies at or
// past the resource's size read zeros instead of memory.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t buffer_rsrc;
__device__ __forceinline__ buffer_rsrc make_buffer_rsrc(const void* base, uint32_t bytes) {
  // raw buffer: stride 0, range-checked against `bytes`, 32-bit data format
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void buffer_to_lds16(buffer_rsrc r, uint32_t voffset, APEX_LDS void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, voffset, 0, 0, 0);
}
// 16 bytes into registers through a buffer resource (zeros past its size).
__device__ __forceinline__ u32x4 buffer_load16(buffer_rsrc r, uint32_t voffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 0));
}
#else
struct buffer_rsrc {};
__device__ __forceinline__ buffer_rsrc make_buffer_rsrc(const void*, uint32_t) { return {}; }
__device__ __forceinline__ void buffer_to_lds16(buffer_rsrc, uint32_t, APEX_LDS void*) {}
__device__ __forceinline__ u32x4 buffer_load16(buffer_rsrc, uint32_t) { return u32x4{}; }
#endif

// ---- RoPE angles -------------------------------------------------------------
// YaRN (Part 1, §5.3-5.4) at scale factor s >= 1 with beta_fast = 32 and
// beta_slow = 1: by the wavelength 2 pi / theta, a frequency below 32 stays,
// one above s is divided by s, and one in between is divided by t s + 1 - t
// with t = (wavelength - 1) / (s - 1) held to [0, 1]. s = 1: unchanged.
__host__ __device__ inline double yarn_theta(double theta, double s) {
  if (s == 1.0) return theta;
  const double wavelength = 1.0 / (theta * kInvTwoPi);
  if (wavelength < 32.0) return theta;
  if (wavelength > s) return theta / s;
  const double t = fmin(fmax((wavelength - 1.0) / (s - 1.0), 0.0), 1.0);
  return theta / (t * s + (1.0 - t));
}
// turns_i = theta_i / (2 pi) with theta_i = b^(-2i/d_h) after YaRN (fp64).
__host__ __device__ inline double rope_turns(int i, int d_h, double base, double yarn_s) {
  return yarn_theta(pow(base, -2.0 * (double)i / (double)d_h), yarn_s) * kInvTwoPi;
}
// The turns of every pair of a rotated head of up to 128 dims, formed once on
// the host per call and passed by value with the kernel arguments.
constexpr int kMaxRopePairs = 64;
struct RopeTurns {
  double v[kMaxRopePairs];
};
inline RopeTurns make_rope_turns(int d_rot, double base, double yarn_s) {
  RopeTurns t{};
  for (int i = 0; i < d_rot / 2 && i < kMaxRopePairs; i++) t.v[i] = rope_turns(i, d_rot, base, yarn_s);
  return t;
}
// The angle pos * theta_i is formed in fp64 as turns and reduced to [-1/2, 1/2]
// before any fp32 step, so large positions lose no accuracy.
__device__ __forceinline__ float reduced_turns(int64_t pos, double turns) {
  double t = (double)pos * turns;
  return (float)(t - rint(t));
}
// Accurate fp32 cos / sin of the reduced angle (used where outputs stay fp32).
__device__ __forceinline__ void rope_cs_accurate(int64_t pos, double turns, float& c, float& s) {
  float x = 2.0f * reduced_turns(pos, turns);  // angle / pi in [-1, 1]
  sincospif(x, &s, &c);
}
// Hardware sine / cosine of the reduced angle (v_sin_f32 / v_cos_f32 take
// turns), used where the rotated value is rounded to bf16 right after.
__device__ __forceinline__ void rope_cs_fast(int64_t pos, double turns, float& c, float& s) {
  float x = reduced_turns(pos, turns);
  s = __builtin_amdgcn_sinf(x);
  c = __builtin_amdgcn_cosf(x);
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

// The value held by lane l ^ 32, through v_permlane32_swap (no LDS round
// trip): swapping the upper half of one copy with the lower half of another
// leaves lane l's partner in the first copy for l >= 32, the second for l < 32.
__device__ __forceinline__ float lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// acc + the two bf16 halves of w (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

// LDS byte address of a __shared__ object, and reads at an LDS byte address.
// Keeping per-lane base addresses in registers the compiler cannot see through
// (opaque) lets every buffer/row offset ride in the 16-bit immediate field of
// the ds_read instructions instead of costing one base register each.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(APEX_LDS const void*)p;
}
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ u32x4 lds_read16_at(uint32_t addr) {
  return *(APEX_LDS const u32x4*)(uintptr_t)addr;
}
__device__ __forceinline__ u32x2 lds_read_tr16_at(uint32_t addr) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((APEX_LDS i16x4*)(uintptr_t)addr);
  return __builtin_bit_cast(u32x2, v);
}

template <int N>
struct Int {
  static constexpr int value = N;
};

}  // namespace apex
