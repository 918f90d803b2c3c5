// Row dequantization + inverse rotation on gfx950: the quantized embedding
// lookup and the transient bf16 weight of the bf16 input gradient.
//
// Sources: sd-scripts pull request 2461, Summary, utils bullet (the quantized
// embedding keeps its rows in the rotated basis, so the lookup dequantizes the
// rows and applies the inverse rotation; the default backward dequantizes the
// weight transiently to bf16); "LoRA Training Guide for MOSS-Image" section 7.1
// (the bf16 backward dequantizes transiently).
//
// out = bf16( (s * q) * R ): R is symmetric and orthogonal, so the inverse
// rotation is R itself.  The Walsh-Hadamard transform runs on the int8 codes in
// fp32, where every partial sum is an integer of magnitude <= 127 * 128 and
// therefore exact; the row scale and 1/sqrt(128) are applied once at the end.
//
// Lane layout as in the row quantizer: a wave owns 32 consecutive 128-blocks;
// lane L < 32 holds the first 64 codes of block L, lane L + 32 the second 64;
// six butterfly stages run in the lane, the seventh across the wave halves.
#include "common.h"
#include "kernels.h"

namespace convrot {
namespace {

// Inverse-rotate the 64 codes of this lane's half block (raw: 4 x 16 bytes).
// On return w[e] (e < 32) is output 32h + e and w[e + 32] is output 64 + 32h + e
// of the block, before scaling.
__device__ __forceinline__ void fwht_codes(const uint4 raw[4], float w[64]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t d[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) w[16 * i + 4 * j + b] = (float)(int8_t)(d[j] >> (8 * b));
  }
#pragma unroll
  for (int bit = 1; bit < 64; bit <<= 1) {
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      if (e & bit) continue;
      float u = w[e], v = w[e | bit];
      w[e] = u + v;
      w[e | bit] = u - v;
    }
  }
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    swap_halves(w[e], w[e + 32]);
    float u = w[e], v = w[e + 32];
    w[e] = u + v;
    w[e + 32] = u - v;
  }
}

// LDS position (16-byte units) of chunk c (0..7) of int8 block b.
__device__ __forceinline__ int lds_chunk8(int b, int c) { return (b << 3) | (c ^ (b & 7)); }

__global__ __launch_bounds__(256) void embedding_lookup_kernel(
    const int32_t* __restrict__ ids, int64_t T, const int8_t* __restrict__ qe,
    const float* __restrict__ se, int64_t V, int D, uint16_t* __restrict__ out,
    int32_t* __restrict__ oob) {
  __shared__ __align__(16) uint8_t lds[4][4096];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  const int nb = D / kBlock;
  uint8_t* my = lds[wave];
  const int p = lane & 31, h = lane >> 5;

  int64_t id = -1;
  if (t < T) id = ids[t];
  const bool valid = t < T && id >= 0 && id < V;
  if (t < T && !valid && lane == 0 && oob) atomicAdd(oob, 1);
  const float rs = valid ? se[id] * (float)kInvSqrt128 : 0.f;

  for (int b0 = 0; b0 < nb; b0 += 32) {
    const int span = nb - b0 < 32 ? nb - b0 : 32;
    if (valid) {
      const int8_t* row = qe + id * (int64_t)D + (int64_t)b0 * kBlock;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int slot = i * 64 + lane;
        int b = slot >> 3;
        int c = (slot & 7) ^ (b & 7);
        if (b < span) load_lds_16(row + b * kBlock + 16 * c, my + i * 1024);
      }
    }
    wait_vmem();
    __builtin_amdgcn_wave_barrier();
    uint4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      raw[i] = valid ? *reinterpret_cast<const uint4*>(my + 16 * lds_chunk8(p, 4 * h + i))
                     : make_uint4(0, 0, 0, 0);
    __builtin_amdgcn_wave_barrier();  // LDS reads done before the next span overwrites
    float w[64];
    fwht_codes(raw, w);
    if (t < T && p < span) {
      uint16_t* dst = out + t * (int64_t)D + (int64_t)(b0 + p) * kBlock;
      uint4* d0 = reinterpret_cast<uint4*>(dst + 32 * h);
      uint4* d1 = reinterpret_cast<uint4*>(dst + 64 + 32 * h);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        d0[g] = make_uint4(pack_bf16x2(w[8 * g] * rs, w[8 * g + 1] * rs),
                           pack_bf16x2(w[8 * g + 2] * rs, w[8 * g + 3] * rs),
                           pack_bf16x2(w[8 * g + 4] * rs, w[8 * g + 5] * rs),
                           pack_bf16x2(w[8 * g + 6] * rs, w[8 * g + 7] * rs));
        d1[g] = make_uint4(pack_bf16x2(w[32 + 8 * g] * rs, w[32 + 8 * g + 1] * rs),
                           pack_bf16x2(w[32 + 8 * g + 2] * rs, w[32 + 8 * g + 3] * rs),
                           pack_bf16x2(w[32 + 8 * g + 4] * rs, w[32 + 8 * g + 5] * rs),
                           pack_bf16x2(w[32 + 8 * g + 6] * rs, w[32 + 8 * g + 7] * rs));
      }
    }
  }
}

// W_hat^T [K, N]: a workgroup covers 64 weight rows (n) x 2 blocks (256 k).
// Item (n_local, b_local) is handled by a lane pair; results are transposed
// through LDS so the global writes are 128-byte runs of one k-row.
__global__ __launch_bounds__(256) void dequant_weight_t_kernel(
    const int8_t* __restrict__ qw, const float* __restrict__ sw, int64_t N, int64_t K,
    uint16_t* __restrict__ what_t) {
  __shared__ __align__(16) uint16_t tile[256][64 + 8];  // [k_local][n_local], padded
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = lane & 31, h = lane >> 5;
  const int item = wave * 32 + p;
  const int n_local = item & 63, b_local = item >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int64_t n = n0 + n_local;
  const int64_t kblk = (int64_t)blockIdx.y * 2 + b_local;
  const bool valid = n < N && kblk * kBlock < K;

  uint4 raw[4];
  const uint4* src = reinterpret_cast<const uint4*>(qw + (valid ? n * K + kblk * kBlock + 64 * h : 0));
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = valid ? src[i] : make_uint4(0, 0, 0, 0);
  const float rs = valid ? sw[n] * (float)kInvSqrt128 : 0.f;
  float w[64];
  fwht_codes(raw, w);
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    tile[b_local * 128 + 32 * h + e][n_local] = (uint16_t)f32_to_bf16_rne(w[e] * rs);
    tile[b_local * 128 + 64 + 32 * h + e][n_local] = (uint16_t)f32_to_bf16_rne(w[e + 32] * rs);
  }
  __syncthreads();
  // 256 k-rows x 8 chunks of 8 n (16 bytes)
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    int idx = it * 256 + threadIdx.x;
    int kl = idx >> 3, c = idx & 7;
    int64_t k = (int64_t)blockIdx.y * 256 + kl;
    int64_t nn = n0 + 8 * c;
    if (k >= K || nn >= N) continue;
    const uint16_t* s = &tile[kl][8 * c];
    uint16_t* d = what_t + k * N + nn;
    if (nn + 8 <= N && (N & 7) == 0) {
      uint4 v = make_uint4(s[0] | ((uint32_t)s[1] << 16), s[2] | ((uint32_t)s[3] << 16),
                           s[4] | ((uint32_t)s[5] << 16), s[6] | ((uint32_t)s[7] << 16));
      *reinterpret_cast<uint4*>(d) = v;
    } else {
      for (int u = 0; u < 8 && nn + u < N; ++u) d[u] = s[u];
    }
  }
}

}  // namespace

hipError_t launch_embedding_lookup(const int32_t* ids, int64_t T, const int8_t* qe,
                                   const float* se, int64_t V, int64_t D, uint16_t* out,
                                   int32_t* oob, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  int64_t grid = (T + 3) / 4;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(embedding_lookup_kernel, dim3((unsigned)grid), dim3(256), 0, stream, ids, T,
                     qe, se, V, (int)D, out, oob);
  return hipGetLastError();
}

hipError_t launch_dequant_weight_t(const int8_t* qw, const float* sw, int64_t N, int64_t K,
                                   uint16_t* what_t, hipStream_t stream) {
  if (N <= 0 || K <= 0) return hipSuccess;
  int64_t gx = (N + 63) / 64, gy = (K + 255) / 256;
  if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dequant_weight_t_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0,
                     stream, qw, sw, N, K, what_t);
  return hipGetLastError();
}

}  // namespace convrot
