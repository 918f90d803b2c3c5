// Host-side argument checks of the C ABI, one function per entry point.
//
// Plain C++ with no HIP call, so the same checks can be built for the host
// alone (with the address and undefined-behaviour sanitizers) and driven with
// bad arguments without a GPU.  Each function returns
//   CONVROT_OK   the call may go ahead (the workspace size and the device are
//                checked by the caller afterwards),
//   kNoOp        an empty batch (0 rows, tokens or ids) whose other sizes are
//                valid: enqueue nothing and return CONVROT_OK,
//   or the error status of include/convrot.h, in this order of precedence:
//   CONVROT_EINVAL (null pointer, size <= 0, misaligned pointer), then
//   CONVROT_ESHAPE (block, multiples of 128, limits).
//
// Limits: every row, column and id count fits in int32, and every tensor has at
// most 2^40 elements, so no byte count or offset computed from them overflows.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/convrot.h"

namespace convrot {
namespace check {

constexpr int kNoOp = 1;
constexpr int64_t kBlockLen = 128;
constexpr int64_t kMaxDim = 0x7fffffff;
constexpr int64_t kMaxElems = (int64_t)1 << 40;

inline bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline bool a16_or_null(const void* p) { return p == nullptr || a16(p); }
inline bool a256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255) == 0; }
inline bool row_len_ok(int64_t K) {
  return K > 0 && K % kBlockLen == 0 && K <= CONVROT_MAX_ROW_LEN;
}
// a x b elements, both positive.
inline bool dims_ok(int64_t a, int64_t b) {
  return a <= kMaxDim && b <= kMaxDim && a <= kMaxElems / b;
}
inline bool rank_ok(int32_t R) { return R == 16 || R == 32; }

// convrot_quantize_weight / _quantize_act / _bwd_quant_dy.  fold: the dY
// quantizer, whose column scales colscale[K] are required.
inline int quantize_rows(const void* x, int64_t rows, int64_t K, const void* q, const void* s,
                         int64_t chunk_rows, const void* colscale, bool fold) {
  if (rows == 0 && K > 0 && chunk_rows >= 0) return row_len_ok(K) ? kNoOp : CONVROT_ESHAPE;
  if (!x || !q || !s || rows <= 0 || K <= 0 || chunk_rows < 0) return CONVROT_EINVAL;
  if (fold && !colscale) return CONVROT_EINVAL;
  if (!a16(x) || !a16(q) || !a16(s) || !a16_or_null(colscale)) return CONVROT_EINVAL;
  if (!row_len_ok(K) || !dims_ok(rows, K)) return CONVROT_ESHAPE;
  return CONVROT_OK;
}

inline int quantize_weight(const void* w, int64_t rows, int64_t cols, int32_t block,
                           int64_t chunk_rows, const void* q, const void* scale) {
  if (block != kBlockLen) return (rows == 0 || (w && q && scale)) ? CONVROT_ESHAPE : CONVROT_EINVAL;
  return quantize_rows(w, rows, cols, q, scale, chunk_rows, nullptr, false);
}

inline int gemm_i8_bf16(const void* qx, const void* sx, const void* qw, const void* sw,
                        int64_t M, int64_t N, int64_t K, const void* bias, const void* y) {
  if (M == 0 && N > 0 && K > 0) return K % kBlockLen == 0 ? kNoOp : CONVROT_ESHAPE;
  if (!qx || !sx || !qw || !sw || !y || M <= 0 || N <= 0 || K <= 0) return CONVROT_EINVAL;
  if (!a16(qx) || !a16(sx) || !a16(qw) || !a16(sw) || !a16(y) || !a16_or_null(bias))
    return CONVROT_EINVAL;
  if (K % kBlockLen || !dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, N)) return CONVROT_ESHAPE;
  return CONVROT_OK;
}

// The forward's tensors (convrot_linear_fwd_noalloc takes no workspace).
inline int linear_fwd_noalloc(const void* x, int64_t M, int64_t K, const void* qw, const void* sw,
                              int64_t N, const void* bias, const void* y) {
  if (M == 0 && N > 0 && K > 0) return row_len_ok(K) ? kNoOp : CONVROT_ESHAPE;
  if (!x || !qw || !sw || !y || M <= 0 || N <= 0 || K <= 0) return CONVROT_EINVAL;
  if (!a16(x) || !a16(qw) || !a16(sw) || !a16(y) || !a16_or_null(bias)) return CONVROT_EINVAL;
  if (!row_len_ok(K) || !dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, N)) return CONVROT_ESHAPE;
  return CONVROT_OK;
}

// ... and with the caller's workspace (non-null, 256-byte aligned).
inline int linear_fwd(const void* x, int64_t M, int64_t K, const void* qw, const void* sw,
                      int64_t N, const void* bias, const void* y, const void* workspace) {
  const bool empty = M == 0 && N > 0 && K > 0;
  if (!empty && (!workspace || !a256(workspace))) return CONVROT_EINVAL;
  return linear_fwd_noalloc(x, M, K, qw, sw, N, bias, y);
}

inline int linear_fwd_lora(const void* x, int64_t M, int64_t K, const void* qw, const void* sw,
                           int64_t N, const void* bias, const void* lora_a, const void* lora_b,
                           int32_t R, const void* y, const void* workspace) {
  if (M == 0 && N > 0 && K > 0) return (row_len_ok(K) && rank_ok(R)) ? kNoOp : CONVROT_ESHAPE;
  if (!x || !qw || !sw || !y || !lora_a || !lora_b || !workspace || M <= 0 || N <= 0 || K <= 0)
    return CONVROT_EINVAL;
  if (!a16(x) || !a16(qw) || !a16(sw) || !a16(y) || !a16(lora_a) || !a16(lora_b) ||
      !a16_or_null(bias) || !a256(workspace))
    return CONVROT_EINVAL;
  if (!row_len_ok(K) || !rank_ok(R) || !dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, N))
    return CONVROT_ESHAPE;
  return CONVROT_OK;
}

inline int lora_down(const void* x, int64_t M, int64_t K, const void* lora_a, int32_t R,
                     const void* xa) {
  if (M == 0 && K > 0) return (row_len_ok(K) && rank_ok(R)) ? kNoOp : CONVROT_ESHAPE;
  if (!x || !lora_a || !xa || M <= 0 || K <= 0) return CONVROT_EINVAL;
  if (!a16(x) || !a16(lora_a) || !a16(xa)) return CONVROT_EINVAL;
  if (!row_len_ok(K) || !rank_ok(R) || !dims_ok(M, K)) return CONVROT_ESHAPE;
  return CONVROT_OK;
}

// b_layout 0: b [N, K]; 1: b [K, N] (contraction along the rows of b).
inline int gemm_i8_i32(const void* a, const void* b, int64_t M, int64_t N, int64_t K,
                       int32_t b_layout, const void* acc) {
  const bool layout_ok = b_layout == 0 || b_layout == 1;
  if (M == 0 && N > 0 && K > 0 && layout_ok)
    return (K % kBlockLen == 0 && (b_layout == 0 || N % kBlockLen == 0)) ? kNoOp : CONVROT_ESHAPE;
  if (!a || !b || !acc || M <= 0 || N <= 0 || K <= 0) return CONVROT_EINVAL;
  if (!a16(a) || !a16(b) || !a16(acc)) return CONVROT_EINVAL;
  if (!layout_ok) return CONVROT_EINVAL;
  if (K % kBlockLen || (b_layout == 1 && N % kBlockLen)) return CONVROT_ESHAPE;
  if (!dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, N)) return CONVROT_ESHAPE;
  return CONVROT_OK;
}

inline int dequant_weight_t(const void* qw, const void* sw, int64_t N, int64_t K,
                            const void* what_t) {
  if (!qw || !sw || !what_t || N <= 0 || K <= 0) return CONVROT_EINVAL;
  if (!a16(qw) || !a16(sw) || !a16(what_t)) return CONVROT_EINVAL;
  if (K % kBlockLen || !dims_ok(N, K)) return CONVROT_ESHAPE;
  return CONVROT_OK;
}

inline int linear_bwd_dx(const void* dy, int64_t M, int64_t N, const void* qw, const void* sw,
                         int64_t K, int32_t mode, const void* dx, const void* workspace) {
  const bool mode_ok = mode == CONVROT_BWD_BF16 || mode == CONVROT_BWD_INT8;
  if (M == 0 && N > 0 && K > 0 && mode_ok)
    return (K % kBlockLen == 0 && N % kBlockLen == 0 &&
            (mode != CONVROT_BWD_INT8 || N <= CONVROT_MAX_ROW_LEN))
               ? kNoOp
               : CONVROT_ESHAPE;
  if (!dy || !qw || !sw || !dx || !workspace || M <= 0 || N <= 0 || K <= 0) return CONVROT_EINVAL;
  if (!mode_ok) return CONVROT_EINVAL;
  if (!a16(dy) || !a16(qw) || !a16(sw) || !a16(dx) || !a256(workspace)) return CONVROT_EINVAL;
  if (K % kBlockLen || N % kBlockLen) return CONVROT_ESHAPE;
  if (mode == CONVROT_BWD_INT8 && N > CONVROT_MAX_ROW_LEN) return CONVROT_ESHAPE;
  if (!dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, N)) return CONVROT_ESHAPE;
  return CONVROT_OK;
}

// oob_count: one device int32, 4-byte aligned, may be null.
inline int embedding_lookup(const void* ids, int64_t T, const void* qe, const void* se, int64_t V,
                            int64_t D, const void* out, const void* oob_count) {
  if (T == 0 && V > 0 && D > 0) return D % kBlockLen == 0 ? kNoOp : CONVROT_ESHAPE;
  if (!ids || !qe || !se || !out || T <= 0 || V <= 0 || D <= 0) return CONVROT_EINVAL;
  if (!a16(ids) || !a16(qe) || !a16(se) || !a16(out) ||
      (reinterpret_cast<uintptr_t>(oob_count) & 3))
    return CONVROT_EINVAL;
  if (D % kBlockLen || !dims_ok(T, D) || !dims_ok(V, D)) return CONVROT_ESHAPE;
  return CONVROT_OK;
}

}  // namespace check
}  // namespace convrot
