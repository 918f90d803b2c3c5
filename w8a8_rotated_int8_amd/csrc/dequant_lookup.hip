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

// Store the bf16 outputs of a span of `span` blocks (this lane holds 64 of
// them, see fwht_codes) scaled by rs: staged in LDS (8 KB per wave), then
// written as whole 1 KB runs (lane i of step j writes 16-byte chunk 64j + i)
// with non-temporal stores: 82 -> 63 us for 32768 tokens of 4096 (measured).
// Chunk c of block c/16 sits at c ^ (c/16 & 15) (conflict-free writes).
__device__ __forceinline__ void store_span(uint16_t* span_out, int span, const float w[64],
                                           float rs, uint8_t* stg) {
  const int lane = threadIdx.x & 63;
  const int p = lane & 31, h = lane >> 5;
  auto phys = [](int c) { return c ^ ((c >> 4) & 15); };
  if (p < span) {
#pragma unroll
    for (int run = 0; run < 2; ++run) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float* v = w + 32 * run + 8 * g;
        const int c = 16 * p + 8 * run + 4 * h + g;
        *reinterpret_cast<uint4*>(stg + 16 * phys(c)) =
            make_uint4(pack_bf16x2(v[0] * rs, v[1] * rs), pack_bf16x2(v[2] * rs, v[3] * rs),
                       pack_bf16x2(v[4] * rs, v[5] * rs), pack_bf16x2(v[6] * rs, v[7] * rs));
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): staging writes landed
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
  const int nchunks = span * 16;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = 64 * j + lane;
    if (c < nchunks)
      store16_nt(span_out + 8 * c, *reinterpret_cast<const uint4*>(stg + 16 * phys(c)));
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // staging reads retired before it is reused
}

// Issue the 4 direct-to-LDS loads of a row span of span (1..32) int8 blocks;
// slots past the span reload its last chunk so every lane issues 4 loads.
__device__ __forceinline__ void stage_row(const int8_t* row, int span, uint8_t* buf) {
  const int lane = threadIdx.x & 63;
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_u32(buf));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = i * 64 + lane;
    int b = slot >> 3;
    int c = (slot & 7) ^ (b & 7);
    if (b >= span) { b = span - 1; c = 7; }
    dma16(row + b * kBlock + 16 * c, base + i * 1024);
  }
}

// D <= 4096: persistent waves, one token at a time; the next token's row is
// loaded into the second LDS buffer while the current one is transformed.
// Token ids are fetched 64 at a time into one register and broadcast with
// readlane, so no scalar load sits between two row loads.
__global__ __launch_bounds__(256) void embedding_lookup_kernel(
    const int32_t* __restrict__ ids, int64_t T, const int8_t* __restrict__ qe,
    const float* __restrict__ se, int64_t V, int D, uint16_t* __restrict__ out,
    int32_t* __restrict__ oob) {
  __shared__ __align__(16) uint8_t lds[4][2][4096];
  __shared__ __align__(16) uint8_t stage_out[4][8192];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = lane & 31, h = lane >> 5;
  const int span = D / kBlock;
  const int64_t wstride = (int64_t)gridDim.x * 4;
  const int64_t t0 = (int64_t)blockIdx.x * 4 + wave;
  if (t0 >= T) return;
  const int64_t ntok = (T - 1 - t0) / wstride + 1;  // tokens of this wave
  auto valid_id = [&](int id) { return id >= 0 && (int64_t)id < V; };
  int id_reg = 0;
  float sc_reg = 0.f;
  auto load_ids = [&](int64_t k0) {  // ids and row scales of tokens k0 .. k0+63
    const int64_t t = t0 + (k0 + lane) * wstride;
    id_reg = (k0 + lane < ntok) ? ids[t] : 0;
    sc_reg = valid_id(id_reg) ? se[id_reg] * (float)kInvSqrt128 : 0.f;
  };
  load_ids(0);
  int id = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(id_reg, 0));
  float rs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc_reg), 0));
  if (valid_id(id)) stage_row(qe + (int64_t)id * D, span, lds[wave][0]);
  int cur = 0;
  for (int64_t k = 0; k < ntok; ++k) {
    const int64_t t = t0 + k * wstride;
    int nid = 0;
    float nrs = 0.f;
    const bool more = k + 1 < ntok;
    if (more) {
      if (((k + 1) & 63) == 0) {
        wait_vm_n<0>();  // the row load in flight must not pass the id load
        load_ids(k + 1);
      }
      nid = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(id_reg, (int)((k + 1) & 63)));
      nrs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc_reg),
                                                                (int)((k + 1) & 63)));
    }
    if (more && valid_id(nid)) {
      stage_row(qe + (int64_t)nid * D, span, lds[wave][cur ^ 1]);
      wait_vm_n<4>();
    } else {
      wait_vm_n<0>();
    }
    const bool valid = valid_id(id);
    if (!valid && lane == 0 && oob) atomicAdd(oob, 1);
    uint4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      raw[i] = valid ? *reinterpret_cast<const uint4*>(lds[wave][cur] + 16 * lds_chunk8(p, 4 * h + i))
                     : make_uint4(0, 0, 0, 0);
    float w[64];
    fwht_codes(raw, w);
    store_span(out + t * (int64_t)D, span, w, rs, stage_out[wave]);
    id = nid;
    rs = nrs;
    cur ^= 1;
  }
}

// D > 4096: one token per wave, the row processed in 4096-wide spans.
__global__ __launch_bounds__(256) void embedding_lookup_long_kernel(
    const int32_t* __restrict__ ids, int64_t T, const int8_t* __restrict__ qe,
    const float* __restrict__ se, int64_t V, int D, uint16_t* __restrict__ out,
    int32_t* __restrict__ oob) {
  __shared__ __align__(16) uint8_t lds[4][4096];
  __shared__ __align__(16) uint8_t stage_out[4][8192];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int nb = D / kBlock;
  const int p = lane & 31, h = lane >> 5;
  const int64_t id = ids[t];
  const bool valid = id >= 0 && id < V;
  if (!valid && lane == 0 && oob) atomicAdd(oob, 1);
  const float rs = valid ? se[id] * (float)kInvSqrt128 : 0.f;
  for (int b0 = 0; b0 < nb; b0 += 32) {
    const int span = nb - b0 < 32 ? nb - b0 : 32;
    if (valid) stage_row(qe + id * (int64_t)D + (int64_t)b0 * kBlock, span, lds[wave]);
    wait_vm_n<0>();
    uint4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      raw[i] = valid ? *reinterpret_cast<const uint4*>(lds[wave] + 16 * lds_chunk8(p, 4 * h + i))
                     : make_uint4(0, 0, 0, 0);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // LDS reads retired before the next span overwrites
    float w[64];
    fwht_codes(raw, w);
    store_span(out + t * (int64_t)D + (int64_t)b0 * kBlock, span, w, rs, stage_out[wave]);
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
  if (D <= 4096) {
    int dev = 0, n_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    int64_t grid = (T + 3) / 4;
    // at most four workgroups per CU: two are resident at a time (64 KB of LDS
    // each), the other two start as those finish
    const int64_t cap = 4 * (int64_t)n_cu;
    if (grid > cap) grid = cap;
    hipLaunchKernelGGL(embedding_lookup_kernel, dim3((unsigned)grid), dim3(256), 0, stream, ids,
                       T, qe, se, V, (int)D, out, oob);
  } else {
    int64_t grid = (T + 3) / 4;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(embedding_lookup_long_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       ids, T, qe, se, V, (int)D, out, oob);
  }
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
