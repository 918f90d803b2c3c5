// Device-side helpers shared by the ConvRot kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace convrot {

// Raise the dynamic-LDS limit of `n` kernels to bytes[i], once per device (the
// attribute belongs to the device's copy of the kernel, so a process driving
// several GPUs sets it on each).  `done` holds one bit per device id below 64;
// two threads racing on a first call both set the same values, which is
// harmless.
inline hipError_t set_lds_limits_once(const void* const* kernels, const int* bytes, int n,
                                      std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  for (int i = 0; i < n; ++i) {
    e = hipFuncSetAttribute(kernels[i], hipFuncAttributeMaxDynamicSharedMemorySize, bytes[i]);
    if (e != hipSuccess) return e;
  }
  if (bit) done.fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

constexpr int kWave = 64;
constexpr int kBlock = 128;  // Hadamard block along the contraction axis

// 1/sqrt(128) in binary64: fl64(sqrt 2) * 2^-4 (exact scaling of a correctly
// rounded sqrt).  Writing 1.0 / sqrt(128.0) would round twice and land one ulp
// low, so the literal is spelled out.
constexpr double kInvSqrt128 = 0x1.6a09e667f3bcdp-4;

// bf16 bit patterns <-> fp32.
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// Two fp32 -> packed bf16 pair with the hardware conversion (round to nearest
// even, v_cvt_pk_bf16_f32).
typedef __bf16 convrot_bf16x2 __attribute__((ext_vector_type(2)));
typedef float convrot_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  convrot_f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, convrot_bf16x2));
}

// Correctly rounded fp32 quotient r / s for a per-row divisor s with a
// precomputed inv = RN(1/s) (Markstein's correction step: the residual
// e = r - q0*s is exact under FMA and q0 + e*inv rounds to RN(r/s)).  Valid
// whenever s, 1/s and the quotient are normal numbers; callers route rows with
// extreme scales through the IEEE division instead.  Where the quotient is
// subnormal its value only ever rounds to the integer 0, so that case is benign.
__device__ __forceinline__ float quot_rn(float r, float s, float inv) {
  float q0 = r * inv;
  float e = __builtin_fmaf(-q0, s, r);
  return __builtin_fmaf(e, inv, q0);
}

// Round-half-even of |t| < 2^22 to an integer, returned as the low byte of the
// bit pattern of t + 1.5*2^23 (the addition itself performs the RNE rounding;
// in the binade [2^23, 2^24) the low mantissa bits hold the integer in two's
// complement).
__device__ __forceinline__ uint32_t rne_low_byte_bits(float t) {
  return __float_as_uint(t + 12582912.0f);
}

// Pack the low bytes of four words into one word (byte i from word i).
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2,
                                                   uint32_t b3) {
  uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);  // [b0.0, b1.0, 0, 0]
  uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);  // [b2.0, b3.0, 0, 0]
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);          // [lo.0, lo.1, hi.0, hi.1]
}

// Exchange with the other half of the wave: vdst's upper 32 lanes swap with
// src0's lower 32 lanes (v_permlane32_swap).  Returns {vdst', src0'}.
__device__ __forceinline__ void swap_halves(uint32_t& vdst, uint32_t& src0) {
  auto r = __builtin_amdgcn_permlane32_swap(vdst, src0, false, false);
  vdst = r[0];
  src0 = r[1];
}
__device__ __forceinline__ void swap_halves(double& vdst, double& src0) {
  uint64_t a = __builtin_bit_cast(uint64_t, vdst), b = __builtin_bit_cast(uint64_t, src0);
  uint32_t alo = (uint32_t)a, ahi = (uint32_t)(a >> 32), blo = (uint32_t)b, bhi = (uint32_t)(b >> 32);
  swap_halves(alo, blo);
  swap_halves(ahi, bhi);
  vdst = __builtin_bit_cast(double, ((uint64_t)ahi << 32) | alo);
  src0 = __builtin_bit_cast(double, ((uint64_t)bhi << 32) | blo);
}
__device__ __forceinline__ void swap_halves(float& vdst, float& src0) {
  uint32_t a = __float_as_uint(vdst), b = __float_as_uint(src0);
  swap_halves(a, b);
  vdst = __uint_as_float(a);
  src0 = __uint_as_float(b);
}

// Row maxima of |r|.  Every quantizer takes them with the IEEE 754-2019
// maximum, which returns NaN when either operand is NaN (v_maximum3_f32 on
// gfx950, at the cost of the NaN-dropping v_max3_f32): a NaN or infinite
// rotated value then makes the row's maximum non-finite, and the quantizers
// give such a row a NaN scale and zero codes instead of silently dropping it.
__device__ __forceinline__ float max_nan(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
// The quantizers' NaN scale: the canonical quiet NaN, so that the scale of a
// non-finite row has one bit pattern on every path.
constexpr uint32_t kScaleNaNBits = 0x7fc00000u;

// A row scale s of the int8 input gradient's epilogue (the gradient's s_g),
// applied to an int32 sum |acc| < 2^31 before the fp32 inverse rotation.  Up to
// 2^96 the epilogue uses s as it is.  A larger scale is used as m * 2^e (frexp,
// exact, m in [0.5, 1)): the products and the rotation's sums are formed with m
// and 2^e joins the final constant 1/sqrt(128), so no intermediate leaves the
// fp32 range where the result does not.  While values stay normal, scaling by
// a power of two commutes with every rounding, so such rows get the plain
// chain's result scaled exactly.  A NaN scale (a non-finite row) is used as it
// is.  (The forward needs no split: it applies the weight's scale first.)
constexpr float kSplitRowScale = 0x1p96f;
struct RowScale {
  float m;  // s, or its frexp mantissa when s > 2^96
  int e;    // 0, or the frexp exponent
};
__device__ __forceinline__ RowScale row_scale(float s) {
  const bool big = s > kSplitRowScale;
  return {big ? __builtin_amdgcn_frexp_mantf(s) : s, big ? __builtin_amdgcn_frexp_expf(s) : 0};
}

// Cross-lane maxima of non-negative floats, NaN included (row maxima of |r|,
// from +0 under max_nan): on such values the order of the bit patterns as
// unsigned integers is the order of the floats, and a positive NaN's bits lie
// above +inf's, so the lanes combine with integer max and a NaN survives.
//
// DPP lane patterns within each 16-lane row (gfx9 dpp_ctrl encodings).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]: lane i <- i ^ 1
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]: lane i <- i ^ 2
constexpr int kDppRowMirror = 0x140;   // lane i <- 15 - i within the row
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within each 8 lanes

template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
  return v > o ? v : o;
}

// Max over aligned groups of n consecutive lanes (n = 1, 2, 4, 8 or 16) of each
// 16-lane row; every lane of a group receives its group's max.  After the two
// quad steps a lane holds its quad's max; the half-row mirror pairs each quad
// with the other quad of its 8 lanes, the row mirror each 8 with the other 8.
__device__ __forceinline__ float group_max(float v, int n) {
  uint32_t u = __float_as_uint(v);
  if (n > 1) u = max_dpp<kDppQuadXor1>(u);
  if (n > 2) u = max_dpp<kDppQuadXor2>(u);
  if (n > 4) u = max_dpp<kDppHalfMirror>(u);
  if (n > 8) u = max_dpp<kDppRowMirror>(u);
  return __uint_as_float(u);
}

// Max with the lane 16 apart (rows 0 and 1, rows 2 and 3).  permlane16_swap of
// a value with itself leaves rows (0,0,2,2) in one result and (1,1,3,3) in the
// other.
__device__ __forceinline__ float max_xor16(float v) {
  const uint32_t u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0] > r[1] ? r[0] : r[1]);
}

// Max with the lane 32 apart (the two wave halves).
__device__ __forceinline__ float max_xor32(float v) {
  const uint32_t u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0] > r[1] ? r[0] : r[1]);
}

// Wait for all outstanding vector-memory operations of this wave (including
// loads that write LDS directly).
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0f70);
  asm volatile("" ::: "memory");
}


// 32-bit LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left alone (gfx9 encoding: vmcnt
// bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | (((N >> 4) & 3) << 14));
  asm volatile("" ::: "memory");
}

// 16-byte direct global->LDS load (lane i's bytes land at lds_base + 16 i;
// lds_base must be wave-uniform).  Issued through inline asm so that the
// compiler does not fence every later LDS access on it: callers order the
// data with explicit vmcnt waits (and barriers when other waves read it).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}

// dma16 with the non-temporal cache policy, for data read exactly once (the
// rows of a weight or embedding being quantized).
__device__ __forceinline__ void dma16_nt(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}

// 16-byte store with the non-temporal cache policy, for outputs that this
// library does not read back (measured faster than plain stores on gfx950 for
// long write streams).
__device__ __forceinline__ void store16_nt(void* dst, uint4 v) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(dst));
}

// 4-byte direct global->LDS load (lane i's word lands at lds_base + 4 i); the
// same ordering rules as dma16.
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}


}  // namespace convrot
