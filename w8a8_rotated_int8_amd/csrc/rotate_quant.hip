// Row rotation + symmetric per-row int8 quantization on gfx950.
//
// Implements the weight quantizer, the online activation quantizer and the
// row-chunked embedding quantizer of the ConvRot INT8 layer ("LoRA Training
// Guide for MOSS-Image" section 7.1, "ConvRot INT8"; sd-scripts pull request
// 2461, Summary, kernels and utils bullets), and the dY quantizer of the int8
// input gradient (same guide section: the opt-in int8 backward routes grad_x
// through the int8 GEMM).
//
// Arithmetic (bit-exact by construction):
//   rotate:   per 128-block, S_j = sum_i H[i][j] x_i computed by a fast
//             Walsh-Hadamard transform in binary64.  bf16 inputs make every
//             partial sum exact (a block's magnitude spread would have to exceed
//             2^38 before binary64 rounds), so the butterfly order cannot change
//             the result; r_j = fl32(fl64(S_j * c)), c = 1/sqrt(128).
//   fold:     (dY quantizer) r_n = fl32(fl32(dY_n) * s_w[n]); no rotation.
//   quantize: a = max|r|, s = fl32(a/127), code = RNE(fl32(r/s)); all-zero row
//             -> s = 0, codes 0.
//
// Work layout.  A wave owns a span of up to 32 consecutive 128-blocks (4096
// elements): one row of K = 4096, several short rows packed together, or a
// 4096-wide slice of a long row (then the workgroup's waves share the row and
// combine their maxima through LDS).  The span is copied to LDS with direct
// 16-byte global->LDS loads (coalesced, XOR-swizzled so the transposed reads
// are bank-conflict free); lane L < 32 then holds the first half (64 values) of
// block L, lane L + 32 the second half.  Six butterfly stages run inside the
// lane; the seventh pairs lane L with L + 32 through v_permlane32_swap.
#pragma clang fp contract(off)

#include "common.h"
#include "kernels.h"

namespace convrot {
namespace {

constexpr int kSpanBlocks = 32;                  // blocks per wave span
constexpr int kSpanBytes = kSpanBlocks * 256;    // bf16 bytes per wave span
constexpr int kMaxWavesPerRow = CONVROT_MAX_ROW_LEN_BLOCKS / kSpanBlocks;

enum Mode { kRotate = 0, kFold = 1 };

// LDS position (in 16-byte units) of chunk c (0..15) of block b.
__device__ __forceinline__ int lds_chunk(int b, int c) { return (b << 4) | (c ^ (b & 7)); }

// Quantize one staged span: read the lane's 64 values from LDS, rotate (or
// fold the column scale), reduce the row maxima, quantize and store.
template <int MODE>
__device__ __forceinline__ void quantize_span(const uint8_t* my_lds, int span_blocks, int nb,
                                              int64_t span_elem0, int blk_in_row0, int64_t row0,
                                              int waves_per_row, int8_t* __restrict__ q,
                                              float* __restrict__ scale,
                                              const float* __restrict__ colscale,
                                              float* seg_max_wave, float* row_part_max) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int p = lane & 31;   // block within the span
  const int h = lane >> 5;   // which half of the block
  const bool active = p < span_blocks;

  // ---- read the lane's 64 values ------------------------------------------
  uint4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    raw[i] = *reinterpret_cast<const uint4*>(my_lds + 16 * lds_chunk(p, 8 * h + i));
  }

  float r[64];
  if (MODE == kRotate) {
    double v[64];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = (double)bf16lo_to_f32(w[j]);
        v[8 * i + 2 * j + 1] = (double)bf16hi_to_f32(w[j]);
      }
    }
    if (!active) {
#pragma unroll
      for (int e = 0; e < 64; ++e) v[e] = 0.0;
    }
    // in-lane butterflies over index bits 0..5 (element 64h + e of the block)
#pragma unroll
    for (int bit = 1; bit < 64; bit <<= 1) {
#pragma unroll
      for (int e = 0; e < 64; ++e) {
        if (e & bit) continue;
        double a = v[e], b = v[e | bit];
        v[e] = a + b;
        v[e | bit] = a - b;
      }
    }
    // bit 6 pairs lane L with lane L + 32.  After the swap the lower lane holds
    // (A[e], B[e]) and the upper lane (A[e+32], B[e+32]) in (v[e], v[e+32]).
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      swap_halves(v[e], v[e + 32]);
      double a = v[e], b = v[e + 32];
      v[e] = a + b;        // output index 32h + e
      v[e + 32] = a - b;   // output index 64 + 32h + e
    }
#pragma unroll
    for (int e = 0; e < 64; ++e) r[e] = (float)(v[e] * kInvSqrt128);
  } else {
    // fold the per-column scale: element 64h + e of block p
    const int64_t col0 = active ? (int64_t)(blk_in_row0 + (waves_per_row == 1 ? p % nb : p)) * kBlock +
                                      64 * h
                                : 0;
    const float4* cs = reinterpret_cast<const float4*>(colscale + col0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
      float4 s0 = active ? cs[2 * i] : make_float4(0.f, 0.f, 0.f, 0.f);
      float4 s1 = active ? cs[2 * i + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
      float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r[8 * i + 2 * j] = bf16lo_to_f32(w[j]) * sc[2 * j];
        r[8 * i + 2 * j + 1] = bf16hi_to_f32(w[j]) * sc[2 * j + 1];
      }
    }
    if (!active) {
#pragma unroll
      for (int e = 0; e < 64; ++e) r[e] = 0.f;
    }
  }

  // ---- row absmax ------------------------------------------------------------
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 64; ++e) m = fmaxf(m, fabsf(r[e]));
  m = fmaxf(m, __shfl_xor(m, 32, kWave));  // both halves of the block
  if (waves_per_row == 1) {
    if ((nb & (nb - 1)) == 0) {
      m = wave_max_xor(m, nb);             // aligned segments of nb lanes
    } else {
      if (lane < 32) seg_max_wave[lane] = m;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      int first = (p / nb) * nb;
      float mm = 0.f;
      for (int j = 0; j < nb; ++j) mm = fmaxf(mm, seg_max_wave[(first + j) & 31]);
      m = mm;
    }
  } else {
    m = wave_max_xor(m, 32);
    if (lane == 0) row_part_max[wave] = m;
    __syncthreads();
    float mm = 0.f;
    for (int w = 0; w < waves_per_row; ++w) mm = fmaxf(mm, row_part_max[w]);
    m = mm;
  }

  const float s = m / 127.0f;                          // IEEE binary32 division
  const bool fast = s > 0x1p-100f && s < 0x1p100f;
  const float inv = s > 0.f ? 1.0f / s : 0.f;          // RN(1/s)

  // ---- quantize + store --------------------------------------------------------
  // Quotients: the 3-operation correctly rounded form when every lane's row
  // scale is in range (wave-uniform branch), else the IEEE division per lane.
  float t[64];
  if (__builtin_amdgcn_ballot_w64(!fast) == 0) {
#pragma unroll
    for (int e = 0; e < 64; ++e) t[e] = quot_rn(r[e], s, inv);
  } else {
#pragma unroll
    for (int e = 0; e < 64; ++e) t[e] = fast ? quot_rn(r[e], s, inv) : (s > 0.f ? r[e] / s : 0.f);
  }
  uint32_t packed[16];
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    packed[g] = pack_low_bytes(rne_low_byte_bits(t[4 * g]), rne_low_byte_bits(t[4 * g + 1]),
                               rne_low_byte_bits(t[4 * g + 2]), rne_low_byte_bits(t[4 * g + 3]));
  }
  // Stage the codes of the span in LDS (its own input buffer, already read)
  // and store whole 1 KB runs: lane i of step j writes 16-byte chunk 64j + i.
  // Chunk c of block c/8 sits at c ^ (c/8 & 7) (conflict-free writes).
  uint8_t* stg = const_cast<uint8_t*>(my_lds);
  auto phys = [](int c) { return c ^ ((c >> 3) & 7); };
  if (active) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = MODE == kRotate ? 8 * p + (g < 2 ? 2 * h + g : 4 + 2 * h + (g - 2))
                                    : 8 * p + 4 * h + g;
      *reinterpret_cast<uint4*>(stg + 16 * phys(c)) =
          make_uint4(packed[4 * g], packed[4 * g + 1], packed[4 * g + 2], packed[4 * g + 3]);
    }
    bool writes_scale = waves_per_row == 1 ? (h == 0 && p % nb == 0) : (wave == 0 && lane == 0);
    if (writes_scale) scale[row0 + (waves_per_row == 1 ? p / nb : 0)] = s;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): staging writes landed
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
  const int nchunks = span_blocks * 8;
  int8_t* dst = q + span_elem0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = 64 * j + lane;
    if (c < nchunks)
      *reinterpret_cast<uint4*>(dst + 16 * c) = *reinterpret_cast<const uint4*>(stg + 16 * phys(c));
  }
}

// Issue the 8 direct-to-LDS loads of a span of span_blocks (>= 1) blocks.
// Slots past the span reload its last chunk so every lane always issues the
// same number of loads (the vmcnt bookkeeping relies on it).
__device__ __forceinline__ void stage_span(const uint16_t* __restrict__ x, int64_t span_elem0,
                                           int span_blocks, uint8_t* my_lds) {
  const int lane = threadIdx.x & 63;
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_u32(my_lds));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int slot = i * 64 + lane;
    int b = slot >> 4;
    int c = (slot & 15) ^ (b & 7);
    if (b >= span_blocks) { b = span_blocks - 1; c = 15; }
    dma16(x + span_elem0 + (int64_t)b * kBlock + c * 8, base + i * 1024);
  }
}

// Short rows (K <= 4096): persistent waves, each owning a task of
// rows_per_wave packed rows at a time; the next task's span is loaded into the
// second LDS buffer while the current one is quantized.
template <int MODE>
__global__ __launch_bounds__(256) void rotate_quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int K, int8_t* __restrict__ q,
    float* __restrict__ scale, const float* __restrict__ colscale, int rows_per_wave) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ float seg_max[4][kSpanBlocks];
  const int wave = threadIdx.x >> 6;
  const int nb = K / kBlock;
  const int64_t ntasks = (rows + rows_per_wave - 1) / rows_per_wave;
  const int64_t wstride = (int64_t)gridDim.x * (blockDim.x >> 6);
  uint8_t* bufs = lds + wave * 2 * kSpanBytes;
  auto span_of = [&](int64_t task, int64_t& row0, int& blocks) {
    row0 = task * rows_per_wave;
    const int64_t rh = rows - row0;
    blocks = (rh < rows_per_wave ? (int)rh : rows_per_wave) * nb;
  };
  int64_t task = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
  if (task < ntasks) {
    int64_t r0;
    int nbk;
    span_of(task, r0, nbk);
    stage_span(x, r0 * (int64_t)K, nbk, bufs);
  }
  int cur = 0;
  for (; task < ntasks; task += wstride) {
    const int64_t next = task + wstride;
    if (next < ntasks) {
      int64_t r1;
      int nb1;
      span_of(next, r1, nb1);
      stage_span(x, r1 * (int64_t)K, nb1, bufs + (cur ^ 1) * kSpanBytes);
      wait_vm_n<8>();
    } else {
      wait_vm_n<0>();
    }
    int64_t r0;
    int nbk;
    span_of(task, r0, nbk);
    quantize_span<MODE>(bufs + cur * kSpanBytes, nbk, nb, r0 * (int64_t)K, 0, r0, 1, q, scale,
                        colscale, seg_max[wave], nullptr);
    cur ^= 1;
  }
}

// Long rows (K > 4096): one row per workgroup, one 4096-wide slice per wave;
// the waves combine their maxima through LDS.
template <int MODE>
__global__ __launch_bounds__(512) void rotate_quant_long_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int K, int8_t* __restrict__ q,
    float* __restrict__ scale, const float* __restrict__ colscale, int waves_per_row) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ float row_part_max[kMaxWavesPerRow];
  const int wave = threadIdx.x >> 6;
  const int nb = K / kBlock;
  const int64_t row0 = blockIdx.x;
  const int blk_in_row0 = wave * kSpanBlocks;
  const int rem = nb - blk_in_row0;
  const int span_blocks = rem < kSpanBlocks ? rem : kSpanBlocks;
  const int64_t span_elem0 = row0 * (int64_t)K + (int64_t)blk_in_row0 * kBlock;
  uint8_t* my_lds = lds + wave * kSpanBytes;
  stage_span(x, span_elem0, span_blocks, my_lds);
  wait_vm_n<0>();
  quantize_span<MODE>(my_lds, span_blocks, nb, span_elem0, blk_in_row0, row0, waves_per_row, q,
                      scale, colscale, nullptr, row_part_max);
}

}  // namespace

RowPlan plan_rows(int K) {
  RowPlan pl;
  int nb = K / kBlock;
  if (nb <= kSpanBlocks) {
    pl.rows_per_wave = kSpanBlocks / nb;
    pl.waves_per_row = 1;
    pl.threads = 256;
  } else {
    pl.rows_per_wave = 1;
    pl.waves_per_row = (nb + kSpanBlocks - 1) / kSpanBlocks;
    pl.threads = 64 * pl.waves_per_row;
  }
  return pl;
}

hipError_t launch_rotate_quant(const uint16_t* x, int64_t rows, int K, int8_t* q, float* scale,
                               const float* colscale, bool fold, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  RowPlan pl = plan_rows(K);
  static int n_cu = 0;
  static bool configured = false;
  if (!configured) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int max_lds = kMaxWavesPerRow * kSpanBytes;
    const void* ks[2] = {(const void*)rotate_quant_long_kernel<kRotate>,
                         (const void*)rotate_quant_long_kernel<kFold>};
    for (const void* k : ks) {
      e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
      if (e != hipSuccess) return e;
    }
    configured = true;
  }
  if (pl.waves_per_row == 1) {
    const int64_t tasks = (rows + pl.rows_per_wave - 1) / pl.rows_per_wave;
    int64_t grid = (tasks + 3) / 4;
    const int64_t cap = 2 * (int64_t)(n_cu > 0 ? n_cu : 256);  // two resident workgroups per CU
    if (grid > cap) grid = cap;
    const size_t lds = 4 * 2 * kSpanBytes;
    if (fold)
      hipLaunchKernelGGL(rotate_quant_rows_kernel<kFold>, dim3((unsigned)grid), dim3(256), lds,
                         stream, x, rows, K, q, scale, colscale, pl.rows_per_wave);
    else
      hipLaunchKernelGGL(rotate_quant_rows_kernel<kRotate>, dim3((unsigned)grid), dim3(256), lds,
                         stream, x, rows, K, q, scale, colscale, pl.rows_per_wave);
  } else {
    if (rows > 0x7fffffff) return hipErrorInvalidValue;
    const size_t lds = (size_t)pl.waves_per_row * kSpanBytes;
    if (fold)
      hipLaunchKernelGGL(rotate_quant_long_kernel<kFold>, dim3((unsigned)rows), dim3(pl.threads),
                         lds, stream, x, rows, K, q, scale, colscale, pl.waves_per_row);
    else
      hipLaunchKernelGGL(rotate_quant_long_kernel<kRotate>, dim3((unsigned)rows), dim3(pl.threads),
                         lds, stream, x, rows, K, q, scale, colscale, pl.waves_per_row);
  }
  return hipGetLastError();
}

}  // namespace convrot
