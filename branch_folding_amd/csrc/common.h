// Device-side building blocks shared by the folded verify-layer kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specfold {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
// Number of compute units the work-splitting policies plan for (MI355X).
constexpr int kPlanCUs = 256;

// ------------------------------------------------------------------------------------
// Conversions.  bf16 rounding is round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
// ------------------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 16 bytes of T unpacked to floats: 8 values for bf16, 4 for f32.
template <typename T> struct Pack16 {
  static constexpr int kElems = 16 / sizeof(T);
};

__device__ __forceinline__ void unpack16(const uint4& u, float (&f)[8], bf16) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __uint_as_float(w[e] << 16);
    f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(const uint4& u, float (&f)[4], float) {
  f[0] = __uint_as_float(u.x);
  f[1] = __uint_as_float(u.y);
  f[2] = __uint_as_float(u.z);
  f[3] = __uint_as_float(u.w);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// pairs convert with one v_cvt_pk_bf16_f32 each (round to nearest even)
__device__ __forceinline__ uint4 pack16(const float (&f)[8], bf16) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = __builtin_bit_cast(uint32_t,
                              __builtin_convertvector(f32x2{f[2 * e], f[2 * e + 1]}, bf16x2));
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ uint4 pack16(const float (&f)[4], float) {
  uint4 u;
  u.x = __float_as_uint(f[0]);
  u.y = __float_as_uint(f[1]);
  u.z = __float_as_uint(f[2]);
  u.w = __float_as_uint(f[3]);
  return u;
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
// Streaming load: data read exactly once (weights), marked non-temporal so it does not
// displace reused data (the shared activation tile) from the caches.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(void* p, const uint4& v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// ------------------------------------------------------------------------------------
// Wave reductions (64 lanes).
// ------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// Reduce across the four 16-lane groups (lanes l, l^16, l^32, l^48) in the VALU.
// v_permlane16_swap exchanges the odd 16-lane rows of its first operand with the even rows
// of its second (v_permlane32_swap: the upper 32 lanes of the first with the lower 32 of
// the second); with the same value in both operands every lane gets back {its own value,
// lane l^16's} (resp. l^32's), in some order.  No LDS round trip, unlike ds_bpermute.
__device__ __forceinline__ float group4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ------------------------------------------------------------------------------------
// MFMA 16x16 tiles.  A "k-step" covers 64 bytes of the contraction dimension: every lane
// holds 16 contiguous bytes (8 bf16 / 4 f32) of its row at byte offset (lane/16)*16.
// bf16 issues one v_mfma_f32_16x16x32_bf16; f32 issues four v_mfma_f32_16x16x4_f32, the
// e-th consuming element e of every lane.  Both operands use the same k permutation, so
// the product is the plain dot product over the 64-byte k-step.
// Output layout (both types): lane l holds C[(l/16)*4 + r][l%16], r = 0..3.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mma_kstep(const uint4& a, const uint4& b, f32x4 c, bf16) {
  bf16x8 av = __builtin_bit_cast(bf16x8, a);
  bf16x8 bv = __builtin_bit_cast(bf16x8, b);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_kstep(const uint4& a, const uint4& b, f32x4 c, float) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

// Direct-to-LDS 16-byte load (global_load_lds_dwordx4: lane i writes LDS bytes
// [lds_base + 16 i, lds_base + 16 i + 16); lds_base must be wave-uniform).  Issued from
// inline asm so that the compiler's wait-count pass does not see an LDS write: reads it
// cannot tell apart from the stage being filled (the attention's transposed V reads carry no
// alias information), or loads issued by only some of a workgroup's waves, would make it
// drain every load in flight before each LDS read.  A kernel using it orders these loads
// itself (s_waitcnt vmcnt + s_barrier before a stage is read); M0 is restored.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[b]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[g], off\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [g] "v"(g), [b] "s"(lds_base)
      : "memory");
}

// dma16 with the nontemporal hint: for data read once (streamed weights), so that its lines
// do not displace data that other CUs are still re-reading from L2.
__device__ __forceinline__ void dma16_nt(const void* g, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[b]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[g], off nt\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [g] "v"(g), [b] "s"(lds_base)
      : "memory");
}

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace specfold
