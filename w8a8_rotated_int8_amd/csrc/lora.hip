// LoRA down projection of the ConvRot INT8 forward: xa = bf16(x . A^T).
//
// The quantized layers stay LoRA-trainable and the LoRA branch receives the
// unrotated input ("LoRA Training Guide for MOSS-Image", section 7.1, ConvRot
// INT8 scope bullet), so the branch reads x itself, not q_x.  The up
// projection (xa . B^T, scaled) is added inside the GEMM's epilogue.
//
// One workgroup (8 waves) owns 16 rows of x; wave w contracts the 64-wide
// k-blocks w, w + 8, ... with v_mfma_f32_16x16x32_bf16, one 16-column tile per
// 16 rows of A, and the eight partial tiles are summed through LDS in a fixed
// order.  16-row tiles give 256 workgroups for 4096 tokens, one per CU.
// Within a 64-wide k-block, lane group g = lane / 16 holds elements
// 16 g .. 16 g + 15 of its row (32 contiguous bytes), and MFMA step s takes
// elements 16 g + 8 s .. + 7 of both operands: the same permutation of k on
// both sides.  A wave issues the loads of 8 k-blocks (all of its share of
// K = 4096) before the first multiply.
#include "common.h"
#include "kernels.h"

namespace convrot {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kDownWaves = 8;
constexpr int kDownGroup = 8;   // k-blocks per load group (all of K = 4096)

template <int NT>  // 16-row tiles of A (R = 16 NT)
struct DownGroup {
  uint4 x[kDownGroup][2];
  uint4 a[kDownGroup][NT][2];
};

template <int NT>
__global__ __launch_bounds__(64 * kDownWaves) void lora_down_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const uint16_t* __restrict__ A,
    uint16_t* __restrict__ xa) {
  __shared__ float part[kDownWaves][NT][4][64];  // each wave's accumulators per lane
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  int64_t m = m0 + row;
  m = m < M ? m : M - 1;  // rows past the end reload the last row (discarded)
  const uint16_t* xrow = x + m * K + 16 * g;
  const uint16_t* arow = A + (int64_t)row * K + 16 * g;  // tile t adds 16 t rows
  const int nkb = (int)(K / 64);
  const int nj = nkb > wave ? (nkb - wave + kDownWaves - 1) / kDownWaves : 0;  // this wave's blocks

  // Group j0 covers this wave's blocks j0 .. j0 + kDownGroup - 1; blocks past
  // the wave's last one reload it (valid addresses).
  auto load = [&](int j0, DownGroup<NT>& d) {
#pragma unroll
    for (int u = 0; u < kDownGroup; ++u) {
      const int j = j0 + u < nj ? j0 + u : nj - 1;
      const int64_t b = (int64_t)(wave + kDownWaves * j) * 64;
#pragma unroll
      for (int s = 0; s < 2; ++s) d.x[u][s] = *reinterpret_cast<const uint4*>(xrow + b + 8 * s);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          d.a[u][t][s] = *reinterpret_cast<const uint4*>(arow + 16 * t * K + b + 8 * s);
    }
  };
  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  // Blocks past the wave's last one multiply zeros.
  auto mul = [&](const DownGroup<NT>& d, int j0) {
#pragma unroll
    for (int u = 0; u < kDownGroup; ++u) {
      const bool ok = j0 + u < nj;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint4 xs = ok ? d.x[u][s] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, xs),
                                                           __builtin_bit_cast(v8bf, d.a[u][t][s]),
                                                           acc[t], 0, 0, 0);
      }
    }
  };
  DownGroup<NT> d;
  for (int j0 = 0; j0 < nj; j0 += kDownGroup) {
    load(j0, d);
    __builtin_amdgcn_sched_barrier(0);  // keep every load of the group ahead of the multiplies
    mul(d, j0);
  }
  // lane l holds rows 4 (l / 16) + v, column l % 16 of each tile
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) part[wave][t][v][lane] = acc[t][v];
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < 256 * NT) {
    const int l = tid & 63, v = (tid >> 6) & 3, t = tid >> 8;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kDownWaves; ++w) sum += part[w][t][v][l];
    const int64_t mo = m0 + 4 * (l >> 4) + v;
    if (mo < M) xa[mo * (16 * NT) + 16 * t + (l & 15)] = (uint16_t)f32_to_bf16_rne(sum);
  }
}

}  // namespace

hipError_t launch_lora_down(const uint16_t* x, int64_t M, int64_t K, const uint16_t* A, int R,
                            uint16_t* xa, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const int64_t grid = (M + 15) / 16;
  if (grid > 0x7fffffff || (R != 16 && R != 32) || K % 64 || K / 64 > 0x7fffffff)
    return hipErrorInvalidValue;
  if (R == 16)
    hipLaunchKernelGGL(lora_down_kernel<1>, dim3((unsigned)grid), dim3(64 * kDownWaves), 0, stream,
                       x, M, K, A, xa);
  else
    hipLaunchKernelGGL(lora_down_kernel<2>, dim3((unsigned)grid), dim3(64 * kDownWaves), 0, stream,
                       x, M, K, A, xa);
  return hipGetLastError();
}

}  // namespace convrot
