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
  if constexpr (MODE == kFold) stage_colscale<SB>(colscale, nbk, nb, 0, 1, cs);
  wait_vm_n<0>();
  quantize_span<MODE, SB, MODE == kFold, STREAM>(buf, nbk, nb, r0 * (int64_t)K, 0, r0, 1, q,
                                                 scale, colscale, seg_max[wave], nullptr, cs);
}

// Long rows (K >= 128 * kSpan): one row per workgroup, one SB-block slice per
// wave; the waves combine their maxima through LDS.  CSL (fold mode): the
// column scales of each slice are staged in LDS past the rows' slices.
template <int MODE, int SB, bool CSL, bool STREAM>
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
  uint8_t* cs = lds + waves_per_row * span_bytes<SB>() + wave * SB * 512;
  if constexpr (CSL)
    stage_colscale<SB>(colscale, span_blocks, nb, blk_in_row0, waves_per_row, cs);
  wait_vm_n<0>();
  quantize_span<MODE, SB, CSL, STREAM>(my_lds, span_blocks, nb, span_elem0, blk_in_row0, row0,
                                       waves_per_row, q, scale, colscale, nullptr, row_part_max,
                                       cs);
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
  // Fold-mode column scales staged in LDS cost 8 KB per wave beside its 4 KB
  // span.  They are staged when a CU still holds at least 12 waves of the
  // kernel that way (3 per SIMD; measured: 8 slices per row, one workgroup of 8
  // waves per CU, ran 5% slower than reading the scales from global memory).
  constexpr int kMaxCslWaves = 12;
  constexpr int kLdsPerCu = 160 * 1024;
  {
    static std::atomic<uint64_t> configured{0};
    const int max_lds = CONVROT_MAX_ROW_LEN_BLOCKS * 256;
    const void* ks[4] = {(const void*)rotate_quant_long_kernel<kRotate, kSpan, false, false>,
                         (const void*)rotate_quant_long_kernel<kRotate, kSpan, false, true>,
                         (const void*)rotate_quant_long_kernel<kFold, kSpan, false, false>,
                         (const void*)rotate_quant_long_kernel<kFold, kSpan, true, false>};
    const int lim[4] = {max_lds, max_lds, max_lds,
                        kMaxCslWaves * (span_bytes<kSpan>() + kSpan * 512)};
    hipError_t e = set_lds_limits_once(ks, lim, 4, configured);
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
  } else {
    if (rows > 0x7fffffff) return hipErrorInvalidValue;
    const size_t lds = (size_t)pl.waves_per_row * span_bytes<kSpan>();
    const int csl_wg = pl.waves_per_row * (span_bytes<kSpan>() + kSpan * 512);
    const bool csl = pl.waves_per_row <= kMaxCslWaves &&
                     (kLdsPerCu / csl_wg) * pl.waves_per_row >= 12;
    if (fold && csl)
      hipLaunchKernelGGL((rotate_quant_long_kernel<kFold, kSpan, true, false>), dim3((unsigned)rows),
                         dim3(pl.threads), lds + (size_t)pl.waves_per_row * kSpan * 512, stream, x,
                         rows, K, q, scale, colscale, pl.waves_per_row);
    else if (fold)
      hipLaunchKernelGGL((rotate_quant_long_kernel<kFold, kSpan, false, false>), dim3((unsigned)rows),
                         dim3(pl.threads), lds, stream, x, rows, K, q, scale, colscale,
                         pl.waves_per_row);
    else if (weights)
      hipLaunchKernelGGL((rotate_quant_long_kernel<kRotate, kSpan, false, true>), dim3((unsigned)rows),
                         dim3(pl.threads), lds, stream, x, rows, K, q, scale, colscale,
                         pl.waves_per_row);
    else
      hipLaunchKernelGGL((rotate_quant_long_kernel<kRotate, kSpan, false, false>),
                         dim3((unsigned)rows), dim3(pl.threads), lds, stream, x, rows, K, q, scale,
                         colscale, pl.waves_per_row);
  }
  return hipGetLastError();
}

}  // namespace convrot
