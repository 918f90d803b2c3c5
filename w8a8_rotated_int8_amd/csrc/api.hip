// C ABI of libconvrot.so: argument validation, workspace layout and launches.
// Declarations and the contract of every entry point are in include/convrot.h.
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/convrot.h"
#include "common.h"
#include "kernels.h"
#include "validate.h"

namespace convrot {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CONVROT_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return CONVROT_EDEVICE;
  int st = g_device_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return CONVROT_EHIP;
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_device_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? CONVROT_OK : CONVROT_EDEVICE;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline int hip_status(hipError_t e) { return e == hipSuccess ? CONVROT_OK : CONVROT_EHIP; }

// Status of the host-side checks (validate.h) as the entry point returns it:
// an empty batch enqueues nothing and succeeds.
inline int checked(int st) { return st == check::kNoOp ? CONVROT_OK : st; }

// Rows already validated (check::quantize_rows).
int quantize_rows_launch(const uint16_t* x, int64_t rows, int64_t K, int8_t* q, float* s,
                         int64_t chunk_rows, const float* colscale, bool fold, bool weights,
                         hipStream_t stream) {
  int st = check_device();
  if (st) return st;
  if (chunk_rows == 0 || chunk_rows > rows) chunk_rows = rows;
  for (int64_t r0 = 0; r0 < rows; r0 += chunk_rows) {
    int64_t n = rows - r0 < chunk_rows ? rows - r0 : chunk_rows;
    hipError_t e = launch_rotate_quant(x + r0 * K, n, (int)K, q + r0 * K, s + r0, colscale, fold,
                                       weights, stream);
    if (e != hipSuccess) return CONVROT_EHIP;
  }
  return CONVROT_OK;
}

size_t fwd_workspace(int64_t M, int64_t K) { return align256((size_t)M * K) + align256(4 * (size_t)M); }
// The forward also holds the int32 partials of a split-K GEMM when the shape
// has too few output tiles to fill the chip (small M, or skinny N).
size_t fwd_splitk_workspace(int64_t M, int64_t N, int64_t K) {
  const int S = small_m_mode(M, N, K) ? small_m_split(M, N, K) : splitk_factor(M, N, K);
  return S > 1 ? align256((size_t)S * M * N * 4) : 0;
}
// The allocation-free forward's scratch: q_x, s_x and any split-K partials
// live in this array instead of a caller workspace.  Each GPU the library runs
// on holds its own copy until the process ends.  Host code never uses the
// array's name as an address: the device address is looked up once per device
// (hipGetSymbolAddress) and kept in g_scratch.
constexpr size_t kScratchBytes = CONVROT_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device (null until looked up)

int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CONVROT_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return CONVROT_EDEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CONVROT_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CONVROT_OK;
}

size_t bwd_int8_workspace(int64_t M, int64_t N) {
  return align256((size_t)M * N) + align256(4 * (size_t)M);
}
size_t bwd_bf16_workspace(int64_t N, int64_t K) { return align256(2 * (size_t)N * K); }

}  // namespace
}  // namespace convrot

using namespace convrot;

extern "C" {

const char* convrot_status_string(int status) {
  switch (status) {
    case CONVROT_OK: return "ok";
    case CONVROT_EINVAL: return "invalid argument (null pointer, non-positive size or misaligned pointer)";
    case CONVROT_ESHAPE: return "unsupported shape (block must be 128; contraction length a multiple of 128 within limits)";
    case CONVROT_EWORKSPACE: return "workspace too small";
    case CONVROT_EHIP: return "HIP runtime or launch error";
    case CONVROT_EDEVICE: return "current device is not gfx950";
    case CONVROT_ESCRATCH: return "the call needs more scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

size_t convrot_workspace_bytes(int32_t op, int64_t M, int64_t N, int64_t K, int32_t mode) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  if (!check::dims_ok(M, K) || !check::dims_ok(N, K) || !check::dims_ok(M, N)) return 0;
  if (op == CONVROT_OP_LINEAR_FWD) return fwd_workspace(M, K) + fwd_splitk_workspace(M, N, K);
  if (op == CONVROT_OP_LINEAR_FWD_LORA)
    return (mode == 16 || mode == 32) ? fwd_workspace(M, K) + align256(2 * (size_t)M * mode) : 0;
  if (op == CONVROT_OP_LINEAR_BWD_DX) {
    if (mode == CONVROT_BWD_INT8) return bwd_int8_workspace(M, N);
    if (mode == CONVROT_BWD_BF16) return bwd_bf16_workspace(N, K);
  }
  return 0;
}

int convrot_quantize_weight(const uint16_t* w, int64_t rows, int64_t cols, int32_t block,
                            int64_t chunk_rows, int8_t* q, float* scale, hipStream_t stream) {
  int st = check::quantize_weight(w, rows, cols, block, chunk_rows, q, scale);
  if (st) return checked(st);
  return quantize_rows_launch(w, rows, cols, q, scale, chunk_rows, nullptr, false, true, stream);
}

int convrot_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* qx, float* sx,
                         hipStream_t stream) {
  int st = check::quantize_rows(x, M, K, qx, sx, 0, nullptr, false);
  if (st) return checked(st);
  return quantize_rows_launch(x, M, K, qx, sx, 0, nullptr, false, false, stream);
}

int convrot_bwd_quant_dy(const uint16_t* dy, int64_t M, int64_t N, const float* sw, int8_t* qg,
                         float* sg, hipStream_t stream) {
  int st = check::quantize_rows(dy, M, N, qg, sg, 0, sw, true);
  if (st) return checked(st);
  return quantize_rows_launch(dy, M, N, qg, sg, 0, sw, true, false, stream);
}

int convrot_gemm_i8_bf16(const int8_t* qx, const float* sx, const int8_t* qw, const float* sw,
                         int64_t M, int64_t N, int64_t K, const uint16_t* bias, uint16_t* y,
                         hipStream_t stream) {
  int st = check::gemm_i8_bf16(qx, sx, qw, sw, M, N, K, bias, y);
  if (st) return checked(st);
  st = check_device();
  if (st) return st;
  GemmArgs a{};
  a.P = qw; a.Q = qx; a.I = N; a.J = M; a.Kc = K; a.ldp = K; a.ldq = K;
  a.out = y; a.ldo = N; a.si = sw; a.sj = sx; a.bias = bias;
  return hip_status(launch_gemm_i8(a, kEpiDequantBf16, false, stream));
}

}  // extern "C"

namespace {

// The forward's launches on an already validated call.
int linear_fwd_launch(const uint16_t* x, int64_t M, int64_t K, const int8_t* qw, const float* sw,
                      int64_t N, const uint16_t* bias, uint16_t* y, void* workspace,
                      hipStream_t stream) {
  if (small_m_fused(M, N, K))  // one launch: q_x and s_x never leave LDS
    return hip_status(launch_linear_fwd_small_m_fused(x, qw, sw, bias, M, N, K, y, stream));
  int8_t* qx = static_cast<int8_t*>(workspace);
  float* sx = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + align256((size_t)M * K));
  hipError_t e = launch_rotate_quant(x, M, (int)K, qx, sx, nullptr, false, false, stream);
  if (e != hipSuccess) return CONVROT_EHIP;
  int32_t* partial = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + fwd_workspace(M, K));
  if (small_m_mode(M, N, K))
    return hip_status(launch_gemm_small_m(qx, sx, qw, sw, bias, M, N, K, y, partial, stream));
  GemmArgs a{};
  a.P = qw; a.Q = qx; a.I = N; a.J = M; a.Kc = K; a.ldp = K; a.ldq = K;
  a.out = y; a.ldo = N; a.si = sw; a.sj = sx; a.bias = bias;
  const int S = splitk_factor(M, N, K);
  if (S > 1) return hip_status(launch_gemm_i8_splitk_dequant(a, S, partial, stream));
  return hip_status(launch_gemm_i8(a, kEpiDequantBf16, false, stream));
}

}  // namespace

extern "C" {

int convrot_linear_fwd(const uint16_t* x, int64_t M, int64_t K, const int8_t* qw,
                       const float* sw, int64_t N, const uint16_t* bias, uint16_t* y,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check::linear_fwd(x, M, K, qw, sw, N, bias, y, workspace);
  if (st) return checked(st);
  if (workspace_bytes < fwd_workspace(M, K) + fwd_splitk_workspace(M, N, K))
    return CONVROT_EWORKSPACE;
  st = check_device();
  if (st) return st;
  return linear_fwd_launch(x, M, K, qw, sw, N, bias, y, workspace, stream);
}

int convrot_linear_fwd_noalloc(const uint16_t* x, int64_t M, int64_t K, const int8_t* qw,
                               const float* sw, int64_t N, const uint16_t* bias, uint16_t* y,
                               hipStream_t stream) {
  int st = check::linear_fwd_noalloc(x, M, K, qw, sw, N, bias, y);
  if (st) return checked(st);
  if (fwd_workspace(M, K) + fwd_splitk_workspace(M, N, K) > kScratchBytes) return CONVROT_ESCRATCH;
  st = check_device();
  if (st) return st;
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st) return st;
  return linear_fwd_launch(x, M, K, qw, sw, N, bias, y, ws, stream);
}

int convrot_linear_fwd_lora(const uint16_t* x, int64_t M, int64_t K, const int8_t* qw,
                            const float* sw, int64_t N, const uint16_t* bias,
                            const uint16_t* lora_a, const uint16_t* lora_b, int32_t R,
                            float lora_scale, uint16_t* y, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  int st = check::linear_fwd_lora(x, M, K, qw, sw, N, bias, lora_a, lora_b, R, y, workspace);
  if (st) return checked(st);
  const size_t xa_off = fwd_workspace(M, K);
  if (workspace_bytes < xa_off + align256(2 * (size_t)M * R)) return CONVROT_EWORKSPACE;
  st = check_device();
  if (st) return st;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int8_t* qx = reinterpret_cast<int8_t*>(ws);
  float* sx = reinterpret_cast<float*>(ws + align256((size_t)M * K));
  uint16_t* xa = reinterpret_cast<uint16_t*>(ws + xa_off);
  hipError_t e = launch_rotate_quant(x, M, (int)K, qx, sx, nullptr, false, false, stream);
  if (e == hipSuccess) e = launch_lora_down(x, M, K, lora_a, R, xa, stream);
  if (e != hipSuccess) return CONVROT_EHIP;
  GemmArgs a{};
  a.P = qw; a.Q = qx; a.I = N; a.J = M; a.Kc = K; a.ldp = K; a.ldq = K;
  a.out = y; a.ldo = N; a.si = sw; a.sj = sx; a.bias = bias;
  a.lora_b = lora_b; a.lora_xa = xa; a.lora_r = R; a.lora_scale = lora_scale;
  return hip_status(launch_gemm_i8(a, kEpiDequantLoraBf16, false, stream));
}

int convrot_lora_down(const uint16_t* x, int64_t M, int64_t K, const uint16_t* lora_a,
                      int32_t R, uint16_t* xa, hipStream_t stream) {
  int st = check::lora_down(x, M, K, lora_a, R, xa);
  if (st) return checked(st);
  st = check_device();
  if (st) return st;
  return hip_status(launch_lora_down(x, M, K, lora_a, R, xa, stream));
}

int convrot_gemm_i8_i32(const int8_t* a_, const int8_t* b, int64_t M, int64_t N, int64_t K,
                        int32_t b_layout, int32_t* acc, hipStream_t stream) {
  int st = check::gemm_i8_i32(a_, b, M, N, K, b_layout, acc);
  if (st) return checked(st);
  st = check_device();
  if (st) return st;
  GemmArgs a{};
  a.P = b; a.Q = a_; a.I = N; a.J = M; a.Kc = K; a.ldp = b_layout == 0 ? K : N; a.ldq = K;
  a.out = acc; a.ldo = N;
  return hip_status(launch_gemm_i8(a, kEpiI32, b_layout == 1, stream));
}

int convrot_dequant_weight_t(const int8_t* qw, const float* sw, int64_t N, int64_t K,
                             uint16_t* what_t, hipStream_t stream) {
  int st = check::dequant_weight_t(qw, sw, N, K, what_t);
  if (st) return checked(st);
  st = check_device();
  if (st) return st;
  return hip_status(launch_dequant_weight_t(qw, sw, N, K, what_t, stream));
}

int convrot_linear_bwd_dx(const uint16_t* dy, int64_t M, int64_t N, const int8_t* qw,
                          const float* sw, int64_t K, int32_t mode, uint16_t* dx,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check::linear_bwd_dx(dy, M, N, qw, sw, K, mode, dx, workspace);
  if (st) return checked(st);
  if (workspace_bytes < convrot_workspace_bytes(CONVROT_OP_LINEAR_BWD_DX, M, N, K, mode))
    return CONVROT_EWORKSPACE;
  st = check_device();
  if (st) return st;
  if (mode == CONVROT_BWD_INT8) {
    int8_t* qg = static_cast<int8_t*>(workspace);
    float* sg = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + align256((size_t)M * N));
    hipError_t e = launch_rotate_quant(dy, M, (int)N, qg, sg, sw, true, false, stream);
    if (e != hipSuccess) return CONVROT_EHIP;
    GemmArgs a{};
    a.P = qw; a.Q = qg; a.I = K; a.J = M; a.Kc = N; a.ldp = K; a.ldq = N;
    a.out = dx; a.ldo = K; a.sj = sg;
    return hip_status(launch_gemm_i8(a, kEpiInvRotBf16, true, stream));
  }
  uint16_t* what_t = static_cast<uint16_t*>(workspace);
  hipError_t e = launch_dequant_weight_t(qw, sw, N, K, what_t, stream);
  if (e != hipSuccess) return CONVROT_EHIP;
  GemmArgs a{};
  a.P = what_t; a.Q = dy; a.I = K; a.J = M; a.Kc = N; a.ldp = N; a.ldq = N;
  a.out = dx; a.ldo = K;
  return hip_status(launch_gemm_bf16(a, stream));
}

int convrot_embedding_lookup(const int32_t* ids, int64_t T, const int8_t* qe, const float* se,
                             int64_t V, int64_t D, uint16_t* out, int32_t* oob_count,
                             hipStream_t stream) {
  int st = check::embedding_lookup(ids, T, qe, se, V, D, out, oob_count);
  if (st) return checked(st);
  st = check_device();
  if (st) return st;
  return hip_status(launch_embedding_lookup(ids, T, qe, se, V, D, out, oob_count, stream));
}

}  // extern "C"
