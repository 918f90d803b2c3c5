// Row rotation + symmetric per-row int8 quantization on gfx950.
//
// Implements the weight quantizer, the online activation quantizer and the
// row-chunked embedding quantizer of the ConvRot INT8 layer ("LoRA Training
// Guide for MOSS-Image" section 7.1, "ConvRot INT8"; sd-scripts pull request
// 2461, Summary, kernels and utils bullets), and the dY quantizer of the int8
// input gradient (same guide section: the opt-in int8 backward routes grad_x
// through the int8 GEMM).
//
// The span arithmetic and lane layout are described in span_quant.h.
#pragma clang fp contract(off)

#include "common.h"
#include "kernels.h"
#include "span_quant.h"

namespace convrot {
namespace {

#ifndef CONVROT_SPAN
#define CONVROT_SPAN 16
#endif
// Blocks per wave span.  With 16 a wave holds 32 values per lane and fits in
// 128 VGPRs, so four waves share a SIMD (32: two passes, ~150 VGPRs, three).
constexpr int kSpan = CONVROT_SPAN;

// Short rows (K < 128 * kSpan): one task of rows_per_wave packed rows per wave,
// in its own LDS buffer; the resident waves of a SIMD cover each other's load
// latency.  STREAM (weights): loads and code stores bypass-cache (read once,
// not read back soon).
template <int MODE, int SB, bool STREAM>
__global__ __launch_bounds__(256) void rotate_quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int K, int8_t* __restrict__ q,
    float* __restrict__ scale, const float* __restrict__ colscale, int rows_per_wave) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ float seg_max[4][SB];
  const int wave = threadIdx.x >> 6;
  const int nb = K / kBlock;
  const int64_t ntasks = (rows + rows_per_wave - 1) / rows_per_wave;
  const int64_t task = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
  if (task >= ntasks) return;
  uint8_t* buf = lds + wave * span_bytes<SB>();
  const int64_t r0 = task * rows_per_wave;
  const int64_t rh = rows - r0;
  const int nbk = (rh < rows_per_wave ? (int)rh : rows_per_wave) * nb;
  stage_span<SB, STREAM>(x, r0 * (int64_t)K, nbk, buf);
  uint8_t* cs = lds + 4 * span_bytes<SB>() + wave * SB * 512;  // fold mode: column scales
  if constexpr (MODE == kFold) stage_colscale<SB>(colscale, nbk, nb, cs);
  wait_vm_n<0>();
  quantize_span<MODE, SB, STREAM>(buf, nbk, nb, r0 * (int64_t)K, r0, 1, q, scale, seg_max[wave],
                                  nullptr, cs);
}

// Long rows (K >= 128 * kSpan), rotate mode: one row per workgroup, one
// SB-block slice per wave; the waves combine their maxima through LDS.
template <int MODE, int SB, bool STREAM>
__global__ __launch_bounds__(SB == 16 ? 1024 : 512) void rotate_quant_long_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int K, int8_t* __restrict__ q,
    float* __restrict__ scale, const float* __restrict__ colscale, int waves_per_row) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ float row_part_max[CONVROT_MAX_ROW_LEN_BLOCKS / SB];
  const int wave = threadIdx.x >> 6;
  const int nb = K / kBlock;
  const int64_t row0 = blockIdx.x;
  const int blk_in_row0 = wave * SB;
  const int rem = nb - blk_in_row0;
  const int span_blocks = rem < SB ? rem : SB;
  const int64_t span_elem0 = row0 * (int64_t)K + (int64_t)blk_in_row0 * kBlock;
  uint8_t* my_lds = lds + wave * span_bytes<SB>();
  stage_span<SB, STREAM>(x, span_elem0, span_blocks, my_lds);
  wait_vm_n<0>();
  quantize_span<MODE, SB, STREAM>(my_lds, span_blocks, nb, span_elem0, row0,
                                  waves_per_row, q, scale, nullptr, row_part_max);
}

// Rows of exactly 4096 values (32 blocks; the attention and packed-stream
// activations, most weights and the token embedding): one wave per row at a
// time.  Lane L holds half h = L >> 5 of block b = L & 31: elements 64 h + e
// (e < 64), 64 values in binary64.  Six butterfly stages run inside the lane
// (element bits 0-5) and one across lanes L and L + 32 (bit 6,
// v_permlane32_swap): half the cross-lane work of the 32-value span layout,
// and the row maximum needs no exchange between waves.
//
// After the last stage lane (h, b) holds outputs 32 h + e in v[e] and
// 64 + 32 h + e in v[e + 32] (e < 32) of block b.
//
// The 64 values take ~196 VGPRs, so two waves share a SIMD; to keep the SIMD
// busy the waves are persistent and load the next row into a second LDS buffer
// while they compute the current one.  LDS per wave: two 8 KB row buffers,
// chunk c (16 bytes) of block b at 16 b + (c ^ (b & 7)); the current buffer
// then stages the row's 4 KB of codes, chunk k at k ^ ((k >> 3) & 7).
constexpr int kRow4kBlocks = 32;
constexpr int kRow4kBytes = kRow4kBlocks * 256;
// Below this many rows a wave gets too few rows to pipeline their loads and the
// two-wave-per-row span kernel (four waves per SIMD) is as fast or faster
// (same-box A/B, us: 4096 rows 13.9 vs 14.5; 20480 rows 50.2 vs 50.3; 248320
// rows 721-726 vs 678-679).
constexpr int64_t kRow4kMinRows = 8192;

template <bool STREAM>
__device__ __forceinline__ void stage_row4k(const uint16_t* __restrict__ x, int64_t row,
                                            uint8_t* buf) {
  // slot i * 64 + lane holds chunk c of block b: whole 1 KB runs of the row per
  // load instruction
  const int lane = threadIdx.x & 63;
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_u32(buf));
  const uint16_t* src = x + row * (kRow4kBlocks * kBlock);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int slot = i * 64 + lane;
    const int b = slot >> 4;
    const int c = (slot & 15) ^ (b & 7);
    if constexpr (STREAM) dma16_nt(src + b * kBlock + c * 8, base + i * 1024);
    else dma16(src + b * kBlock + c * 8, base + i * 1024);
  }
}

template <bool STREAM>
__device__ __forceinline__ void quantize_row4k(const uint8_t* buf_in, uint8_t* buf, int64_t row,
                                               int8_t* __restrict__ q, float* __restrict__ scale) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int b = lane & 31;
  const int h = lane >> 5;
  double v[64];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 raw =
        *reinterpret_cast<const uint4*>(buf_in + 16 * ((b << 4) | ((8 * h + i) ^ (b & 7))));
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = (double)bf16lo_to_f32(w[j]);
      v[8 * i + 2 * j + 1] = (double)bf16hi_to_f32(w[j]);
    }
  }
#pragma unroll
  for (int bit = 1; bit < 64; bit <<= 1) {
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      if (e & bit) continue;
      const double a = v[e], c = v[e | bit];
      v[e] = a + c;
      v[e | bit] = a - c;
    }
    __builtin_amdgcn_sched_barrier(0);  // one stage at a time (register pressure)
  }
  // element bit 6: lane L with L + 32
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    swap_halves(v[e], v[e + 32]);
    const double a = v[e], c = v[e + 32];
    v[e] = a + c;
    v[e + 32] = a - c;
  }
  float r[64];
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 64; ++e) {
    r[e] = (float)(v[e] * kInvSqrt128);
    m = max_nan(m, fabsf(r[e]));
  }
  m = max_xor32(max_xor16(group_max(m, 16)));  // the whole row: every lane

  // s = fl32(m / 127), t = fl32(r / s): the 3-operation correctly rounded form
  // for ordinary rows (m is wave-uniform, so is the branch), IEEE division with
  // the clamp to +-127 otherwise (a subnormal s can push |t| past 127.5), and
  // the NaN scale with codes 0 for a non-finite maximum
  float s, t[64];
  if (m >= 0x1p-64f && m <= 0x1p100f) {
    s = quot_rn(m, 127.0f, kInv127);
    const float inv = 1.0f / s;
#pragma unroll
    for (int e = 0; e < 64; ++e) t[e] = quot_rn(r[e], s, inv);
  } else {
    // a non-finite maximum gives the NaN scale, and s > 0 fails: codes 0
    s = m <= 0x1.fffffep127f ? m / 127.0f : __uint_as_float(kScaleNaNBits);
#pragma unroll
    for (int e = 0; e < 64; ++e) t[e] = s > 0.f ? fminf(fmaxf(r[e] / s, -127.0f), 127.0f) : 0.f;
  }
  // codes of outputs 32 h + e (e < 32): row bytes 128 b + 32 h + e, chunks
  // 8 b + 2 h and + 1; outputs 64 + 32 h + e: chunks 8 b + 4 + 2 h and + 1
  auto phys = [](int k) { return k ^ ((k >> 3) & 7); };
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    uint32_t pk[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int e = 16 * grp + 4 * d;
      pk[d] = pack_low_bytes(rne_low_byte_bits(t[e]), rne_low_byte_bits(t[e + 1]),
                             rne_low_byte_bits(t[e + 2]), rne_low_byte_bits(t[e + 3]));
    }
    const int chunk = 8 * b + (grp < 2 ? 2 * h + grp : 4 + 2 * h + (grp - 2));
    *reinterpret_cast<uint4*>(buf + 16 * phys(chunk)) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): staging writes landed
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
  int8_t* dst = q + row * (kRow4kBlocks * kBlock);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = 64 * j + lane;
    const uint4 val = *reinterpret_cast<const uint4*>(buf + 16 * phys(c));
    if constexpr (STREAM) store16_nt(dst + 16 * c, val);
    else *reinterpret_cast<uint4*>(dst + 16 * c) = val;
  }
  if (lane == 0) scale[row] = s;
}

template <bool STREAM>
__global__ __launch_bounds__(256) void rotate_quant_row4k_kernel(const uint16_t* __restrict__ x,
                                                                 int64_t rows,
                                                                 int8_t* __restrict__ q,
                                                                 float* __restrict__ scale) {
  __shared__ __align__(16) uint8_t lds[4][2][kRow4kBytes];
  const int wave = threadIdx.x >> 6;
  const int64_t stride = (int64_t)gridDim.x * 4;
  int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= rows) return;
  stage_row4k<STREAM>(x, row, lds[wave][0]);
  wait_vm_n<0>();
  for (int cur = 0;; cur ^= 1) {
    const int64_t next = row + stride;
    if (next < rows) stage_row4k<STREAM>(x, next, lds[wave][cur ^ 1]);
    quantize_row4k<STREAM>(lds[wave][cur], lds[wave][cur], row, q, scale);
    row = next;
    if (row >= rows) break;
    // Outstanding vector-memory operations, in issue order: this row's 8 loads
    // (issued before the previous row's arithmetic), then the previous row's 4
    // code stores and its scale store.  They retire in order, so once at most 5
    // are left the row has landed in LDS.
    wait_vm_n<5>();
  }
}

// Fold mode, rows of at least one span (N >= 128 * kSpan): one row per
// workgroup and no LDS staging.  Folding has no data flow between elements, so
// lane t of the workgroup takes the 4-element units t + j * blockDim.x
// (j < kFoldUnits): the row's bf16 loads, the column-scale loads and the code
// stores are each contiguous across a wave's lanes.  The waves combine their
// maxima through LDS.  The arithmetic per element and per row is that of the
// span quantizer's fold mode: r = fl32(dY) * s_w, a = max |r|, s = fl32(a/127),
// code = RNE(fl32(r/s)).
constexpr int kFoldUnits = 8;

__global__ __launch_bounds__(1024) void fold_quant_rows_kernel(
    const uint16_t* __restrict__ dy, int N, int8_t* __restrict__ q, float* __restrict__ scale,
    const float* __restrict__ colscale) {
  __shared__ float part[16];
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;
  const int units = N >> 2;
  const int64_t row = blockIdx.x;
  const uint2* src = reinterpret_cast<const uint2*>(dy + row * (int64_t)N);
  const float4* cs = reinterpret_cast<const float4*>(colscale);
  uint2 raw[kFoldUnits];
  float4 sc[kFoldUnits];
#pragma unroll
  for (int j = 0; j < kFoldUnits; ++j) {
    const int u = j * nthr + tid;
    raw[j] = u < units ? src[u] : make_uint2(0u, 0u);
    sc[j] = u < units ? cs[u] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float r[kFoldUnits][4];
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < kFoldUnits; ++j) {
    r[j][0] = bf16lo_to_f32(raw[j].x) * sc[j].x;
    r[j][1] = bf16hi_to_f32(raw[j].x) * sc[j].y;
    r[j][2] = bf16lo_to_f32(raw[j].y) * sc[j].z;
    r[j][3] = bf16hi_to_f32(raw[j].y) * sc[j].w;
#pragma unroll
    for (int e = 0; e < 4; ++e) m = max_nan(m, fabsf(r[j][e]));
  }
  m = max_xor32(max_xor16(group_max(m, 16)));
  if (lane == 0) part[wave] = m;
  __syncthreads();
  m = 0.f;
  for (int w = 0; w < nwaves; ++w) m = max_nan(m, part[w]);

  // m is the same in every lane, so both branches are workgroup-uniform.
  float s, t[kFoldUnits][4];
  if (m >= 0x1p-64f && m <= 0x1p100f) {
    s = quot_rn(m, 127.0f, kInv127);
    const float inv = 1.0f / s;
#pragma unroll
    for (int j = 0; j < kFoldUnits; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) t[j][e] = quot_rn(r[j][e], s, inv);
  } else {
    // Extreme rows: IEEE division.  When s is subnormal its rounding error can
    // push |t| past 127.5 (a folded maximum of 2^-140 gives s = 2^-147 and
    // t = 128), so the codes are clamped to [-127, 127]; a zero s (a/127
    // underflowed) gives codes 0, and so does the NaN scale of a non-finite
    // maximum.
    s = m <= 0x1.fffffep127f ? m / 127.0f : __uint_as_float(kScaleNaNBits);
#pragma unroll
    for (int j = 0; j < kFoldUnits; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        t[j][e] = s > 0.f ? fminf(fmaxf(r[j][e] / s, -127.0f), 127.0f) : 0.f;
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(q + row * (int64_t)N);
#pragma unroll
  for (int j = 0; j < kFoldUnits; ++j) {
    const int u = j * nthr + tid;
    if (u < units)
      dst[u] = pack_low_bytes(rne_low_byte_bits(t[j][0]), rne_low_byte_bits(t[j][1]),
                              rne_low_byte_bits(t[j][2]), rne_low_byte_bits(t[j][3]));
  }
  if (tid == 0) scale[row] = s;
}

}  // namespace

// Rows shorter than a span are packed into one; longer rows are split into
// span-wide slices, one per wave.
RowPlan plan_rows(int K) {
  RowPlan pl;
  int nb = K / kBlock;
  if (nb < kSpan) {
    pl.rows_per_wave = kSpan / nb;
    pl.waves_per_row = 1;
    pl.threads = 256;
  } else {
    pl.rows_per_wave = 1;
    pl.waves_per_row = (nb + kSpan - 1) / kSpan;
    pl.threads = 64 * pl.waves_per_row;
  }
  return pl;
}

hipError_t launch_rotate_quant(const uint16_t* x, int64_t rows, int K, int8_t* q, float* scale,
                               const float* colscale, bool fold, bool weights, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (fold && weights) return hipErrorInvalidValue;
  RowPlan pl = plan_rows(K);
  {
    static std::atomic<uint64_t> configured{0};
    const int max_lds = CONVROT_MAX_ROW_LEN_BLOCKS * 256;
    const void* ks[2] = {(const void*)rotate_quant_long_kernel<kRotate, kSpan, false>,
                         (const void*)rotate_quant_long_kernel<kRotate, kSpan, true>};
    const int lim[2] = {max_lds, max_lds};
    hipError_t e = set_lds_limits_once(ks, lim, 2, configured);
    if (e != hipSuccess) return e;
  }
  if (K / kBlock < kSpan) {
    const int64_t tasks = (rows + pl.rows_per_wave - 1) / pl.rows_per_wave;
    const int64_t grid = (tasks + 3) / 4;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (fold)
      hipLaunchKernelGGL((rotate_quant_rows_kernel<kFold, kSpan, false>), dim3((unsigned)grid),
                         dim3(256), 4 * (span_bytes<kSpan>() + kSpan * 512), stream, x, rows, K, q,
                         scale, colscale, pl.rows_per_wave);
    else if (weights)
      hipLaunchKernelGGL((rotate_quant_rows_kernel<kRotate, kSpan, true>), dim3((unsigned)grid),
                         dim3(256), 4 * span_bytes<kSpan>(), stream, x, rows, K, q, scale, colscale,
                         pl.rows_per_wave);
    else
      hipLaunchKernelGGL((rotate_quant_rows_kernel<kRotate, kSpan, false>), dim3((unsigned)grid),
                         dim3(256), 4 * span_bytes<kSpan>(), stream, x, rows, K, q, scale, colscale,
                         pl.rows_per_wave);
  } else if (K == kRow4kBlocks * kBlock && !fold && rows >= kRow4kMinRows) {
    // persistent: two workgroups of four waves per CU (two waves per SIMD)
    int dev = 0, n_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    int64_t grid = (rows + 3) / 4;
    if (grid > 2 * (int64_t)n_cu) grid = 2 * (int64_t)n_cu;
    if (weights)
      hipLaunchKernelGGL(rotate_quant_row4k_kernel<true>, dim3((unsigned)grid), dim3(256), 0,
                         stream, x, rows, q, scale);
    else
      hipLaunchKernelGGL(rotate_quant_row4k_kernel<false>, dim3((unsigned)grid), dim3(256), 0,
                         stream, x, rows, q, scale);
  } else if (fold) {
    if (rows > 0x7fffffff) return hipErrorInvalidValue;
    const int units = K / 4;
    const int waves = (units + 64 * kFoldUnits - 1) / (64 * kFoldUnits);  // <= 16 for K <= 32768
    hipLaunchKernelGGL(fold_quant_rows_kernel, dim3((unsigned)rows), dim3(64 * waves), 0, stream,
                       x, K, q, scale, colscale);
  } else {
    if (rows > 0x7fffffff) return hipErrorInvalidValue;
    const size_t lds = (size_t)pl.waves_per_row * span_bytes<kSpan>();
    if (weights)
      hipLaunchKernelGGL((rotate_quant_long_kernel<kRotate, kSpan, true>), dim3((unsigned)rows),
                         dim3(pl.threads), lds, stream, x, rows, K, q, scale, colscale,
                         pl.waves_per_row);
    else
      hipLaunchKernelGGL((rotate_quant_long_kernel<kRotate, kSpan, false>),
                         dim3((unsigned)rows), dim3(pl.threads), lds, stream, x, rows, K, q, scale,
                         colscale, pl.waves_per_row);
  }
  return hipGetLastError();
}

}  // namespace convrot
