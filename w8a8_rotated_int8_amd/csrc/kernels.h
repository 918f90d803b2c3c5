// Internal launchers of the ConvRot kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define CONVROT_MAX_ROW_LEN_BLOCKS 256  // 32768 / 128

namespace convrot {

struct RowPlan {
  int rows_per_wave;  // rows packed in one wave (short rows), else 1
  int waves_per_row;  // waves sharing one row (long rows), else 1
  int threads;        // workgroup size
};

RowPlan plan_rows(int K);

// Rotate (fold == false) or scale-fold (fold == true, colscale[K]) each row of
// x [rows, K] and quantize it per row to int8 codes q and fp32 scales.
// weights: x is read once and q is not read back soon (load-time quantization),
// so both move with the non-temporal cache policy; activations and gradients
// are read again (LoRA branch) or their codes are (the GEMM that follows).
hipError_t launch_rotate_quant(const uint16_t* x, int64_t rows, int K, int8_t* q, float* scale,
                               const float* colscale, bool fold, bool weights,
                               hipStream_t stream);

// Epilogues of the tiled GEMM out[j][i] = sum_k P[i][k] * Q[j][k].
enum GemmEpilogue {
  kEpiI32 = 0,         // int32 out
  kEpiDequantBf16 = 1, // bf16( fl32(acc) * sj[j] * si[i] (+ bias[i]) )
  kEpiInvRotBf16 = 2,  // bf16( inverse-rotate along i of fl32(acc) * sj[j] )
  kEpiBf16 = 3,        // bf16(acc) of an fp32 accumulation
  kEpiDequantLoraBf16 = 4,  // kEpiDequantBf16 + lora_scale * (lora_b[i] . lora_xa[j])
};

struct GemmArgs {
  const void* P;      // [I, Kc] row-major, or [Kc, I] when transposed
  const void* Q;      // [J, Kc] row-major
  int64_t I, J, Kc;   // Kc in elements
  int64_t ldp, ldq;   // row strides in elements
  void* out;          // [J, I] row-major
  int64_t ldo;
  const float* si;    // per-i scale (dequant epilogue)
  const float* sj;    // per-j scale
  const uint16_t* bias;  // per-i bf16 bias or nullptr
  // LoRA epilogue only: lora_b [I, lora_r] and lora_xa [J, lora_r], bf16
  const uint16_t* lora_b;
  const uint16_t* lora_xa;
  int lora_r;           // 16 or 32
  float lora_scale;
};

// int8 operands (MFMA i32 32x32x32).  p_transposed: P is given as [Kc, I].
hipError_t launch_gemm_i8(const GemmArgs& a, int epilogue, bool p_transposed, hipStream_t stream);
// Output tile (i x j) of the one-pass dequantizing int8 GEMM out[J, I] over
// K: 256 x 256 once the launch fills the chip, else 128 x 128 or 128 x 64
// where the cost model puts them ahead, with a four-stage operand ring up to
// 256 tiles (one workgroup per CU); 128 x 128 keeps two stages beyond that
// (two per CU).  The tile changes no result.
enum GemmTile { kTile256x256 = 0, kTile128x128 = 1, kTile128x128Deep = 2, kTile128x64 = 3 };
int dequant_tile(int64_t I, int64_t J, int64_t K);
// Split-K int8 GEMM with the dequantizing epilogue (kEpiDequantBf16
// semantics, bit-identical results): S K-slices into int32 partials
// [S, J, I] (caller-provided), then one reduce + dequantize launch.  Needs
// Kc % (S * 128) == 0 and I % 4 == 0.
hipError_t launch_gemm_i8_splitk_dequant(const GemmArgs& a, int S, int32_t* partial,
                                         hipStream_t stream);
// Split count for a forward of M tokens, N outputs, K inputs (1 = no split).
int splitk_factor(int64_t M, int64_t N, int64_t K);

// Forward contraction + dequantization for at most kSmallM activation rows, or
// at most kSmallM output columns over many rows (gemm_small_m.hip);
// small_m_mode says when the forward takes it (0: it does not).
constexpr int64_t kSmallM = 128;
int small_m_mode(int64_t M, int64_t N, int64_t K);
// K-slices of the few-row forward's split form (1: one pass); when above 1 the
// forward passes int32 partials [S, M, N] (caller-provided workspace).
int small_m_split(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_small_m(const int8_t* qx, const float* sx, const int8_t* qw,
                               const float* sw, const uint16_t* bias, int64_t M, int64_t N,
                               int64_t K, uint16_t* y, int32_t* partial, hipStream_t stream);
// The whole forward of very few rows (at most 8 / ceil(K / 2048)) in one
// launch: each workgroup rotates and quantizes x's rows itself, in LDS, with
// the activation quantizer's code, then runs the few-row contraction.
bool small_m_fused(int64_t M, int64_t N, int64_t K);
hipError_t launch_linear_fwd_small_m_fused(const uint16_t* x, const int8_t* qw, const float* sw,
                                           const uint16_t* bias, int64_t M, int64_t N, int64_t K,
                                           uint16_t* y, hipStream_t stream);
// Sum S int32 partials [S, J, I] and dequantize to out[j][i] with the forward
// epilogue (s_j[j], then s_i[i], then bias[i]).  Needs I % 4 == 0.
hipError_t launch_splitk_dequant(const int32_t* partial, int S, int64_t J, int64_t I,
                                 const float* si, const float* sj, const uint16_t* bias,
                                 uint16_t* out, hipStream_t stream);

// bf16 operands (MFMA f32 32x32x16), both row-major, kEpiBf16.
hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t stream);

// LoRA down projection xa [M, R] = bf16(x [M, K] . A [R, K]^T), R <= 32, K % 64 == 0.
hipError_t launch_lora_down(const uint16_t* x, int64_t M, int64_t K, const uint16_t* A, int R,
                            uint16_t* xa, hipStream_t stream);

// W_hat^T [K, N] bf16 from q_w [N, K], s_w [N].
hipError_t launch_dequant_weight_t(const int8_t* qw, const float* sw, int64_t N, int64_t K,
                                   uint16_t* what_t, hipStream_t stream);

// Embedding lookup with row dequantization and inverse rotation.
hipError_t launch_embedding_lookup(const int32_t* ids, int64_t T, const int8_t* qe,
                                   const float* se, int64_t V, int64_t D, uint16_t* out,
                                   int32_t* oob, hipStream_t stream);

}  // namespace convrot
