// LoRA down projection of the ConvRot INT8 forward: xa = bf16(x . A^T).
//
// The quantized layers stay LoRA-trainable and the LoRA branch receives the
// unrotated input ("LoRA Training Guide for MOSS-Image", section 7.1, ConvRot
// INT8 scope bullet), so the branch reads x itself, not q_x.  The up
// projection (xa . B^T, scaled) is added inside the GEMM's epilogue.
//
// One workgroup (16 waves) owns 32 rows of x; wave w contracts the 64-wide
// k-blocks w, w + 16, ... two at a time (all loads of a pair issued before its
// MFMAs) with v_mfma_f32_32x32x16_bf16 (A's rows padded to 32 with zeros), and
// the sixteen partial 32 x 32 tiles are summed through LDS.
// Within a 64-wide k-block, lane half h holds elements 32 h .. 32 h + 31 of its
// row, and MFMA step s takes elements 32 h + 8 s .. + 7 of both operands: the
// same permutation of k on both sides, so every lane loads 64 contiguous bytes.
#include "common.h"
#include "kernels.h"

namespace convrot {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kLoraWaves = 16;

__global__ __launch_bounds__(64 * kLoraWaves) void lora_down_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const uint16_t* __restrict__ A, int R,
    uint16_t* __restrict__ xa) {
  __shared__ float part[kLoraWaves][16][64];  // each wave's 16 accumulators per lane
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * 32;
  int64_t m = m0 + (lane & 31);
  m = m < M ? m : M - 1;  // rows past the end reload the last row (discarded)
  const int r = lane & 31;
  const bool r_ok = r < R;
  const uint16_t* xrow = x + m * K + 32 * h;
  const uint16_t* arow = A + (int64_t)(r_ok ? r : 0) * K + 32 * h;
  v16f acc = {};
  const int64_t nkb = K / 64;
  for (int64_t kb = wave; kb < nkb; kb += 2 * kLoraWaves) {
    const bool two = kb + kLoraWaves < nkb;  // wave-uniform
    uint4 xv[2][4], av[2][4];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int64_t b = p == 0 ? kb : (two ? kb + kLoraWaves : kb);
#pragma unroll
      for (int s = 0; s < 4; ++s) xv[p][s] = *reinterpret_cast<const uint4*>(xrow + b * 64 + 8 * s);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        av[p][s] = r_ok ? *reinterpret_cast<const uint4*>(arow + b * 64 + 8 * s) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (p == 1 && !two) break;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, xv[p][s]),
                                                       __builtin_bit_cast(v8bf, av[p][s]), acc, 0, 0, 0);
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) part[wave][v][lane] = acc[v];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kLoraWaves; ++w) s += part[w][v][lane];
    // output element: row m0 + 8 (v / 4) + 4 h + v % 4, column r
    const int64_t mo = m0 + 8 * (v >> 2) + 4 * h + (v & 3);
    if (r_ok && mo < M) xa[mo * R + r] = (uint16_t)f32_to_bf16_rne(s);
  }
}

}  // namespace

hipError_t launch_lora_down(const uint16_t* x, int64_t M, int64_t K, const uint16_t* A, int R,
                            uint16_t* xa, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const int64_t grid = (M + 31) / 32;
  if (grid > 0x7fffffff || R > 32 || K % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lora_down_kernel, dim3((unsigned)grid), dim3(64 * kLoraWaves), 0, stream, x,
                     M, K, A, R, xa);
  return hipGetLastError();
}

}  // namespace convrot
