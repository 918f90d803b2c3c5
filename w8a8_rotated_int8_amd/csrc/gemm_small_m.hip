// Forward int8 contraction for few activation rows (M <= 128): one caption of
// the text encoder at a time, the training guide's text-encoder quantization
// ("LoRA Training Guide for MOSS-Image", section 7.1, text encoder bullet).
//
// y[m][n] = bf16( fl32( fl32( float(acc[m][n]) * s_w[n] ) * s_x[m] ) (+ bias[n]) ),
// acc[m][n] = sum_k q_x[m][k] q_w[n][k]: the same int32 sums and the same fp32
// epilogue operations as the tiled GEMM, so the output is identical to it.
//
// With 256 x 256 output tiles a caption fills a handful of CUs; here a
// workgroup owns 16 output columns (16 rows of q_w, read exactly once) and all
// M rows of q_x, which stay in L2 and are re-read by every workgroup.  The 8
// waves split K in 64-wide steps (v_mfma_i32_16x16x64_i8: q_x's rows are the A
// operand, 16 per tile, q_w's the B operand); lane group g = lane / 16 loads
// bytes 16 g .. 16 g + 15 of a step for both operands, the same permutation of
// k on both sides.  A wave issues all loads of a group of steps before
// multiplying, and the 8 waves add their int32 tiles into LDS with integer
// atomics (exact, so the order does not matter).
#pragma clang fp contract(off)

#include "common.h"
#include "kernels.h"
#include "span_quant.h"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kSmWaves = 8;

// Output element (m, nn) of the contraction of the few rows (m < M) with the
// many (nn < N).  Plain: the few rows are q_x's (tokens), the many q_w's, and
// y[m][nn] = bf16(fl32(fl32(float(acc) * s_w[nn]) * s_x[m]) (+ bias[nn])).
// Swapped (SW, few output columns): the few rows are q_w's and the many q_x's,
// with sx / sw / M / N passed in those roles; the same operations in the same
// order give y[nn][m] = bf16(fl32(fl32(float(acc) * s_w[m]) * s_x[nn]) (+ bias[m])).
template <bool SW>
__device__ __forceinline__ void store_out(int32_t acc, int64_t m, int64_t nn, int64_t M,
                                          int64_t N, const float* __restrict__ sx,
                                          const float* __restrict__ sw,
                                          const uint16_t* __restrict__ bias,
                                          uint16_t* __restrict__ y) {
  // the weight's scale first, then the activation's (the tiled GEMM's order)
  float f = (float)acc;
  if constexpr (SW) {
    f = f * sx[m];
    f = f * sw[nn];
    if (bias) f = f + __uint_as_float((uint32_t)bias[m] << 16);
    y[nn * M + m] = (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu);
  } else {
    f = f * sw[nn];
    f = f * sx[m];
    if (bias) f = f + __uint_as_float((uint32_t)bias[nn] << 16);
    y[m * N + nn] = (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu);
  }
}

// T: 16-row tiles of q_x (M <= 16 T); G: 64-wide k-steps per load group.
template <int T, int G, bool SW>
__global__ __launch_bounds__(64 * kSmWaves) void gemm_small_m_kernel(
    const int8_t* __restrict__ qx, const float* __restrict__ sx, const int8_t* __restrict__ qw,
    const float* __restrict__ sw, const uint16_t* __restrict__ bias, int64_t M, int64_t N,
    int64_t K, uint16_t* __restrict__ y) {
  __shared__ int32_t part[T][4][64];  // the waves' int32 sums (LDS integer adds)
  for (int i = threadIdx.x; i < T * 256; i += 64 * kSmWaves) (&part[0][0][0])[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t n = n0 + r < N ? n0 + r : N - 1;  // columns past the end reload the last one
  const int8_t* wrow = qw + n * K + 16 * g;
  const int8_t* xrow[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int64_t m = 16 * t + r < M ? 16 * t + r : M - 1;
    xrow[t] = qx + m * K + 16 * g;
  }
  const int nks = (int)(K / 64);
  const int nj = nks > wave ? (nks - wave + kSmWaves - 1) / kSmWaves : 0;  // this wave's steps
  v4i acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = v4i{0, 0, 0, 0};
  for (int j0 = 0; j0 < nj; j0 += G) {
    uint4 wv[G], xv[G][T];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int j = j0 + u < nj ? j0 + u : nj - 1;  // past the wave's last step: reload it
      const int64_t kb = (int64_t)(wave + kSmWaves * j) * 64;
      wv[u] = *reinterpret_cast<const uint4*>(wrow + kb);
#pragma unroll
      for (int t = 0; t < T; ++t) xv[u][t] = *reinterpret_cast<const uint4*>(xrow[t] + kb);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the group ahead of the multiplies
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const uint4 w = j0 + u < nj ? wv[u] : make_uint4(0, 0, 0, 0);  // reloaded steps add 0
#pragma unroll
      for (int t = 0; t < T; ++t)
        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, xv[u][t]),
                                                       __builtin_bit_cast(v4i, w), acc[t], 0, 0, 0);
    }
  }
  // lane l holds rows 4 (l / 16) + v of tile t, column l % 16
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) atomicAdd(&part[t][v][lane], acc[t][v]);
  __syncthreads();
  for (int idx = threadIdx.x; idx < T * 256; idx += 64 * kSmWaves) {
    const int l = idx & 63, v = (idx >> 6) & 3, t = idx >> 8;
    const int64_t m = 16 * t + 4 * (l >> 4) + v;
    const int64_t nn = n0 + (l & 15);
    if (m < M && nn < N) store_out<SW>(part[t][v][l], m, nn, M, N, sx, sw, bias, y);
  }
}

// The forward of at most eight rows in one launch, the activation's rotation
// and quantization fused into the contraction ("Add ConvRot INT8
// quantization", sd-scripts pull request 2461, Summary, kernels bullet: online
// rotation and dynamic quantization inside the matmul).  Every workgroup
// rotates and quantizes the rows of x itself, with the activation quantizer's
// own device code (quantize_span, 16-block spans, the same split of a row over
// waves as rotate_quant_long_kernel), so its codes and scales equal the
// two-launch forward's bit for bit; they stay in LDS (codes row-major).  A row
// of K values takes ceil(K / 2048) waves, so the 8 waves hold 8 / that many
// rows.  The rows' spans arrive by direct loads issued ahead of the wave's
// first G q_w steps, and the wait for the spans leaves those G loads in
// flight: the quantization runs while the weight stream is on its way.  The
// contraction and epilogue are gemm_small_m_kernel's for one row tile.
constexpr int kFusedCodes = 16384;  // bytes of codes in LDS (rows x K)

template <int G>
__global__ __launch_bounds__(64 * kSmWaves) void gemm_small_m_fused_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ qw, const float* __restrict__ sw,
    const uint16_t* __restrict__ bias, int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y) {
  __shared__ __align__(16) uint8_t spans[kSmWaves][span_bytes<16>()];
  __shared__ __align__(16) int8_t qx[kFusedCodes];
  __shared__ float sx[kSmWaves];
  __shared__ float row_part_max[kSmWaves];
  __shared__ float seg_max[kSmWaves][16];
  __shared__ int32_t part[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int i = threadIdx.x; i < 256; i += 64 * kSmWaves) (&part[0][0])[i] = 0;

  // This wave's span: blocks 16 jw .. 16 jw + 15 of row m (rows m >= M: none).
  const int nb = (int)(K / kBlock);
  const int wpr = (nb + 15) >> 4;
  const int m = wave / wpr, jw = wave - m * wpr;
  const bool has_span = m < M;
  const int blk0 = 16 * jw;
  const int span_blocks = nb - blk0 < 16 ? nb - blk0 : 16;
  const int64_t span_elem0 = (int64_t)m * K + (int64_t)blk0 * kBlock;
  if (has_span) stage_span<16, false>(x, span_elem0, span_blocks, spans[wave]);
  __builtin_amdgcn_sched_barrier(0);

  // The wave's 64-byte k-steps of its 16 q_w rows; steps past the wave's last
  // reload the row's last step, and their products are dropped.
  const int r = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t n = n0 + r < N ? n0 + r : N - 1;  // columns past the end reload the last one
  const int8_t* wrow = qw + n * K + 16 * g;
  const int nks = (int)(K / 64);
  const int nj = nks > wave ? (nks - wave + kSmWaves - 1) / kSmWaves : 0;
  auto step_of = [&](int j) { return (int64_t)(j < nj ? wave + kSmWaves * j : nks - 1) * 64; };
  uint4 wv[G];
#pragma unroll
  for (int u = 0; u < G; ++u) wv[u] = *reinterpret_cast<const uint4*>(wrow + step_of(u));
  __builtin_amdgcn_sched_barrier(0);

  // The span's loads are older than the G weight loads: vmcnt(G) means they
  // landed.  This needs at least G loads issued after them: each step is one
  // 16-byte load, and the compiler cannot merge the repeated past-the-end
  // steps (their addresses depend on nj and K, known only at run time).
  wait_vm_n<G>();
  if (has_span)
    quantize_span<kRotate, 16, false>(spans[wave], span_blocks, nb, span_elem0, m, wpr, qx, sx,
                                      seg_max[wave], row_part_max + m * wpr, nullptr, m * wpr);
  else if (wpr > 1)
    __syncthreads();  // a wave without a row joins the one row-maximum barrier of quantize_span
  __syncthreads();    // every row's codes and scale are in LDS

  const int8_t* xrow = qx + (int64_t)(r < M ? r : M - 1) * K + 16 * g;
  v4i acc = v4i{0, 0, 0, 0};
  for (int j0 = 0; j0 < nj; j0 += G) {
    if (j0 > 0) {
#pragma unroll
      for (int u = 0; u < G; ++u) wv[u] = *reinterpret_cast<const uint4*>(wrow + step_of(j0 + u));
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const uint4 xv = *reinterpret_cast<const uint4*>(xrow + step_of(j0 + u));
      const uint4 w = j0 + u < nj ? wv[u] : make_uint4(0, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, xv),
                                                  __builtin_bit_cast(v4i, w), acc, 0, 0, 0);
    }
  }
  // lane l holds rows 4 (l / 16) + v, column l % 16
#pragma unroll
  for (int v = 0; v < 4; ++v) atomicAdd(&part[v][lane], acc[v]);
  __syncthreads();
  for (int idx = threadIdx.x; idx < 256; idx += 64 * kSmWaves) {
    const int l = idx & 63, v = idx >> 6;
    const int64_t mm = 4 * (l >> 4) + v;
    const int64_t nn = n0 + (l & 15);
    if (mm < M && nn < N) store_out<false>(part[v][l], mm, nn, M, N, sx, sw, bias, y);
  }
}

// The same contraction with q_x staged through LDS.  K runs in chunks of 512
// bytes; a chunk of all 16 T rows of q_x arrives by whole-line direct loads
// (8 T instructions of 1 KB, T per wave) into a ring of NB LDS buffers, NB - 1
// chunks ahead of the one being multiplied, and wave w multiplies the chunk's
// 64-byte step w.  Row r's 16-byte piece c sits at r * 512 + 16 (c ^ (r & 15)), so the 16
// rows of one fragment read fall in different banks.  The waves' q_w steps of
// every chunk (K <= 4096: at most 8 per wave) are loaded at the start, before
// the first chunk's direct loads, and the explicit wait for that chunk covers
// them.  They are ordinary loads: the compiler must know when their registers
// are written.  (Loads issued through inline asm were tried: the compiler then
// took the registers as written at once and was free to copy them before the
// data arrived, which it did in some instances.)
constexpr int kSmChunk = 512;
constexpr int kSmMaxChunks = 8;

template <int T, int NB, bool SW>
__global__ __launch_bounds__(64 * kSmWaves) void gemm_small_m_lds_kernel(
    const int8_t* __restrict__ qx, const float* __restrict__ sx, const int8_t* __restrict__ qw,
    const float* __restrict__ sw, const uint16_t* __restrict__ bias, int64_t M, int64_t N,
    int64_t K, uint16_t* __restrict__ y) {
  static_assert(NB == 2 || NB == 3, "two or three chunk buffers");
  extern __shared__ __align__(16) uint8_t xs[];  // NB buffers of 16 T rows x 512 bytes
  __shared__ int32_t part[T][4][64];
  for (int i = threadIdx.x; i < T * 256; i += 64 * kSmWaves) (&part[0][0][0])[i] = 0;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t n = n0 + r < N ? n0 + r : N - 1;  // columns past the end reload the last one
  const int nch = (int)(K / kSmChunk);
  uint4 wv[kSmMaxChunks];
  {
    const int8_t* wrow = qw + n * K + 64 * wave + 16 * g;
#pragma unroll
    for (int c = 0; c < kSmMaxChunks; ++c)  // past the last chunk: reload it (unused)
      wv[c] = *reinterpret_cast<const uint4*>(wrow + (c < nch ? c : nch - 1) * kSmChunk);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the q_w loads ahead of the chunk loop
  constexpr int kBuf = 16 * T * kSmChunk;
  const uint32_t xs_base = __builtin_amdgcn_readfirstlane(lds_u32(xs));
  auto stage = [&](int c, int b) {
#pragma unroll
    for (int it = 0; it < T; ++it) {
      const int inst = it * kSmWaves + wave;  // 1 KB piece of the chunk
      const int slot = inst * 64 + lane;
      const int row = slot >> 5;
      const int pc = (slot & 31) ^ (row & 15);  // the 16-byte piece this lane fetches
      const int64_t m = row < M ? row : M - 1;  // rows past the end reload the last one
      dma16(qx + m * K + (int64_t)c * kSmChunk + 16 * pc, xs_base + b * kBuf + inst * 1024);
    }
  };
  v4i acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int c = 0; c < NB - 1; ++c)
    if (c < nch) stage(c, c);
#pragma unroll
  for (int c = 0; c < kSmMaxChunks; ++c) {
    if (c >= nch) break;
    // this wave's part of chunk c landed (and, older, its q_w loads); with
    // three buffers chunk c + 1 may still be in flight.  The first wait is a
    // full one: after it the compiler knows that every q_w load has landed and
    // inserts no waits of its own later (those would count the direct loads
    // issued since, which it does not see, and wait for them too).
    if (c > 0 && NB == 3 && c + 1 < nch) wait_vm_n<T>();
    else wait_vm_n<0>();
    __syncthreads();  // every wave's part landed; every wave is done with chunk c - 1
    if (c + NB - 1 < nch) stage(c + NB - 1, (c + NB - 1) % NB);
    const uint8_t* buf = xs + (c % NB) * kBuf;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int row = 16 * t + r;
      const uint4 xf =
          *reinterpret_cast<const uint4*>(buf + row * kSmChunk + 16 * ((4 * wave + g) ^ r));
      acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, xf),
                                                     __builtin_bit_cast(v4i, wv[c]), acc[t], 0,
                                                     0, 0);
    }
  }
  // lane l holds rows 4 (l / 16) + v of tile t, column l % 16
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) atomicAdd(&part[t][v][lane], acc[t][v]);
  __syncthreads();
  for (int idx = threadIdx.x; idx < T * 256; idx += 64 * kSmWaves) {
    const int l = idx & 63, v = (idx >> 6) & 3, t = idx >> 8;
    const int64_t m = 16 * t + 4 * (l >> 4) + v;
    const int64_t nn = n0 + (l & 15);
    if (m < M && nn < N) store_out<SW>(part[t][v][l], m, nn, M, N, sx, sw, bias, y);
  }
}

// Split-K form, for three or more row tiles.  The one-pass kernels above read
// all of q_x in every workgroup (16 output columns each), and those re-reads
// from L2 bound them.  Here workgroup (x, y) owns the kSmCols 16-column tiles
// from 16 kSmCols x and the K-slice [kSmSlice y, kSmSlice (y + 1)): four times
// the columns per q_x byte read, with the K split restoring the workgroup
// count.  The q_w steps of both 512-byte chunks of the slice are loaded first,
// then both chunks of q_x are staged at once in the swizzled layout of
// gemm_small_m_lds_kernel; wave w multiplies step w of each chunk against its
// column tiles, the waves add their tiles in LDS with integer atomics, and the
// int32 sums go to partial[y][m][n].  The dequantizing launch after it adds
// the slices (exact) and applies the fp32 epilogue in store_out's order, so
// the output is bit-identical to the one-pass kernels'.
constexpr int kSmCols = 4;
constexpr int kSmSlice = 2 * kSmChunk;

template <int T>
__global__ __launch_bounds__(64 * kSmWaves) void gemm_small_m_splitk_kernel(
    const int8_t* __restrict__ qx, const int8_t* __restrict__ qw, int64_t M, int64_t N,
    int64_t K, int32_t* __restrict__ partial) {
  extern __shared__ __align__(16) uint8_t xs[];  // 2 chunks of 16 T rows x 512 bytes
  __shared__ int32_t part[T][kSmCols][4][64];
  for (int i = threadIdx.x; i < T * kSmCols * 256; i += 64 * kSmWaves) (&part[0][0][0][0])[i] = 0;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16 * kSmCols;
  const int64_t k0 = (int64_t)blockIdx.y * kSmSlice;
  uint4 wv[2][kSmCols];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int j = 0; j < kSmCols; ++j) {
      const int64_t n = n0 + 16 * j + r < N ? n0 + 16 * j + r : N - 1;  // past the end: reload
      wv[c][j] = *reinterpret_cast<const uint4*>(qw + n * K + k0 + c * kSmChunk + 64 * wave + 16 * g);
    }
  __builtin_amdgcn_sched_barrier(0);  // the q_w loads ahead of the direct loads
  constexpr int kBuf = 16 * T * kSmChunk;
  const uint32_t xs_base = __builtin_amdgcn_readfirstlane(lds_u32(xs));
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int it = 0; it < T; ++it) {
      const int inst = it * kSmWaves + wave;  // 1 KB piece of the chunk
      const int slot = inst * 64 + lane;
      const int row = slot >> 5;
      const int pc = (slot & 31) ^ (row & 15);  // the 16-byte piece this lane fetches
      const int64_t m = row < M ? row : M - 1;  // rows past the end reload the last one
      dma16(qx + m * K + k0 + c * kSmChunk + 16 * pc, xs_base + c * kBuf + inst * 1024);
    }
  wait_vm_n<0>();
  __syncthreads();  // every wave's pieces landed; part is zeroed
  v4i acc[T][kSmCols];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int j = 0; j < kSmCols; ++j) acc[t][j] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int row = 16 * t + r;
      const uint4 xf = *reinterpret_cast<const uint4*>(xs + c * kBuf + row * kSmChunk +
                                                       16 * ((4 * wave + g) ^ r));
#pragma unroll
      for (int j = 0; j < kSmCols; ++j)
        acc[t][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, xf),
                                                          __builtin_bit_cast(v4i, wv[c][j]),
                                                          acc[t][j], 0, 0, 0);
    }
  // lane l holds rows 4 (l / 16) + v of row tile t, column l % 16 of column tile j
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int j = 0; j < kSmCols; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) atomicAdd(&part[t][j][v][lane], acc[t][j][v]);
  __syncthreads();
  int32_t* out = partial + (int64_t)blockIdx.y * M * N;
  for (int idx = threadIdx.x; idx < T * kSmCols * 256; idx += 64 * kSmWaves) {
    const int l = idx & 63, v = (idx >> 6) & 3, j = (idx >> 8) & (kSmCols - 1), t = idx >> 10;
    const int64_t m = 16 * t + 4 * (l >> 4) + v;
    const int64_t nn = n0 + 16 * j + (l & 15);
    if (m < M && nn < N) out[m * N + nn] = part[t][j][v][l];
  }
}

template <int T>
hipError_t launch_split_t(const int8_t* qx, const float* sx, const int8_t* qw, const float* sw,
                          const uint16_t* bias, int64_t M, int64_t N, int64_t K, uint16_t* y,
                          int32_t* partial, hipStream_t stream) {
  static_assert(kSmCols == 4, "the partial store decodes the column tile with a 2-bit mask");
  constexpr int kLds = 2 * 16 * T * kSmChunk;  // + T KB x kSmCols of static int32 sums
  static_assert(kLds + T * kSmCols * 1024 <= 160 * 1024, "fits the 160 KB of LDS");
  static std::atomic<uint64_t> configured{0};
  const void* k = (const void*)gemm_small_m_splitk_kernel<T>;
  hipError_t e = set_lds_limits_once(&k, &kLds, 1, configured);
  if (e != hipSuccess) return e;
  const int64_t gx = (N + 16 * kSmCols - 1) / (16 * kSmCols);
  const int64_t S = K / kSmSlice;
  hipLaunchKernelGGL((gemm_small_m_splitk_kernel<T>), dim3((unsigned)gx, (unsigned)S),
                     dim3(64 * kSmWaves), kLds, stream, qx, qw, M, N, K, partial);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_dequant(partial, (int)S, M, N, sw, sx, bias, y, stream);
}

// In kernel terms: M few rows (qx, sx), N many (qw, sw); SW when the few are
// the weight's rows (see store_out).
template <int T, bool SW>
hipError_t launch_t(const int8_t* qx, const float* sx, const int8_t* qw, const float* sw,
                    const uint16_t* bias, int64_t M, int64_t N, int64_t K, uint16_t* y,
                    hipStream_t stream) {
  const int64_t grid = (N + 15) / 16;
  // Staging q_x pays from 3 row tiles on (measured, graph replays at K = 4096:
  // M = 77 17.2 -> 14.2 us, M = 128 23.6 -> 17.6 us); at M <= 16 its chunk
  // barriers cost more than the re-reads they save (7.9 -> 9.4 us at M = 1).
  if (T >= 3 && K % kSmChunk == 0 && K / kSmChunk <= kSmMaxChunks) {
    // three buffers (two chunks in flight) where they fit beside the 1 KB per
    // tile of int32 sums in the 160 KB of LDS
    constexpr int NB = 3 * 16 * T * kSmChunk + T * 1024 <= 160 * 1024 ? 3 : 2;
    constexpr int kLds = NB * 16 * T * kSmChunk;
    static std::atomic<uint64_t> configured{0};
    const void* k = (const void*)gemm_small_m_lds_kernel<T, NB, SW>;
    hipError_t e = set_lds_limits_once(&k, &kLds, 1, configured);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_small_m_lds_kernel<T, NB, SW>), dim3((unsigned)grid),
                       dim3(64 * kSmWaves), kLds, stream, qx, sx, qw, sw, bias, M, N, K, y);
    return hipGetLastError();
  }
  constexpr int G = T <= 4 ? 8 : 4;
  hipLaunchKernelGGL((gemm_small_m_kernel<T, G, SW>), dim3((unsigned)grid), dim3(64 * kSmWaves),
                     0, stream, qx, sx, qw, sw, bias, M, N, K, y);
  return hipGetLastError();
}

template <bool SW>
hipError_t launch_few(const int8_t* qx, const float* sx, const int8_t* qw, const float* sw,
                      const uint16_t* bias, int64_t M, int64_t N, int64_t K, uint16_t* y,
                      hipStream_t stream) {
  switch ((M + 15) / 16) {
    case 1: return launch_t<1, SW>(qx, sx, qw, sw, bias, M, N, K, y, stream);
    case 2: return launch_t<2, SW>(qx, sx, qw, sw, bias, M, N, K, y, stream);
    case 3: return launch_t<3, SW>(qx, sx, qw, sw, bias, M, N, K, y, stream);
    case 4: return launch_t<4, SW>(qx, sx, qw, sw, bias, M, N, K, y, stream);
    case 5: return launch_t<5, SW>(qx, sx, qw, sw, bias, M, N, K, y, stream);
    case 6: return launch_t<6, SW>(qx, sx, qw, sw, bias, M, N, K, y, stream);
    case 7: return launch_t<7, SW>(qx, sx, qw, sw, bias, M, N, K, y, stream);
    default: return launch_t<8, SW>(qx, sx, qw, sw, bias, M, N, K, y, stream);
  }
}

}  // namespace

// The split form for few rows: three or more row tiles, K beyond what the
// staged one-pass kernel holds (K > 4096, whole 1 KB slices) and N % 4 == 0 for
// the dequantizing launch.  Measured (forward, graph replays, same box):
// 128 x 8192 x 8192 73.6 -> 51.6 us, 100 x 8192 x 1000 33.7 -> 18.2 us,
// 77 x 8192 x 4096 28.2 -> 25.8 us; at K = 4096 the pipelined one-pass kernel
// stays faster (77 x 4096 x 4096 13.0 against 16.0 us split), and taking
// K >= 12288 into this form lost to the tiled split-K (77 x 16384 x 4096 33.4
// against 44.5 us).
static bool small_m_split_fits(int64_t M, int64_t N, int64_t K) {
  return M > 32 && M <= kSmallM && N >= 1 && N % 4 == 0 && K % kSmSlice == 0 &&
         K > (int64_t)kSmChunk * kSmMaxChunks && K <= (int64_t)CONVROT_MAX_ROW_LEN_BLOCKS * kBlock;
}

int small_m_mode(int64_t M, int64_t N, int64_t K) {
  if (K % 64 || K > 8192) return 0;
  // Measured against split-K (forward, M = 1..128, K = 4096): faster for every
  // N up to 8192 (77 x 4096 x 32: 17.5 -> 11.2 us; 77 x 4096 x 512: 21.8 ->
  // 11.7 us); with N >= 12288 the per-workgroup re-reads of q_x (768
  // workgroups) and with K = 12288 the 8-way K split per workgroup lose.
  if (M >= 1 && M <= kSmallM && N >= 1 && N <= 8192) return 1;
  // Few output columns (a skinny weight) over many tokens: the same kernel
  // with the roles swapped, each workgroup reading 16 token rows once.
  if (N >= 1 && N <= kSmallM && M >= 2048 && M <= 0x7ffffff0) return 2;
  return 0;
}

// Rows the fused few-row forward holds: ceil(K / 2048) waves per row of the 8.
static int fused_rows(int64_t K) { return kSmWaves / (int)((K / kBlock + 15) / 16); }

bool small_m_fused(int64_t M, int64_t N, int64_t K) {
  if (small_m_mode(M, N, K) != 1 || small_m_split(M, N, K) > 1 || K % kBlock) return false;
  return M <= fused_rows(K) && M * K <= kFusedCodes;
}

hipError_t launch_linear_fwd_small_m_fused(const uint16_t* x, const int8_t* qw, const float* sw,
                                           const uint16_t* bias, int64_t M, int64_t N, int64_t K,
                                           uint16_t* y, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (!small_m_fused(M, N, K)) return hipErrorInvalidValue;
  const int64_t grid = (N + 15) / 16;
  hipLaunchKernelGGL(gemm_small_m_fused_kernel<8>, dim3((unsigned)grid), dim3(64 * kSmWaves), 0,
                     stream, x, qw, sw, bias, M, N, K, y);
  return hipGetLastError();
}

int small_m_split(int64_t M, int64_t N, int64_t K) {
  if (small_m_mode(M, N, K) != 1 || !small_m_split_fits(M, N, K)) return 1;
  return (int)(K / kSmSlice);
}

hipError_t launch_gemm_small_m(const int8_t* qx, const float* sx, const int8_t* qw,
                               const float* sw, const uint16_t* bias, int64_t M, int64_t N,
                               int64_t K, uint16_t* y, int32_t* partial, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int mode = small_m_mode(M, N, K);
  if (mode == 1 && small_m_split(M, N, K) > 1) {
    if (!partial) return hipErrorInvalidValue;
    switch ((M + 15) / 16) {
      case 3: return launch_split_t<3>(qx, sx, qw, sw, bias, M, N, K, y, partial, stream);
      case 4: return launch_split_t<4>(qx, sx, qw, sw, bias, M, N, K, y, partial, stream);
      case 5: return launch_split_t<5>(qx, sx, qw, sw, bias, M, N, K, y, partial, stream);
      case 6: return launch_split_t<6>(qx, sx, qw, sw, bias, M, N, K, y, partial, stream);
      case 7: return launch_split_t<7>(qx, sx, qw, sw, bias, M, N, K, y, partial, stream);
      default: return launch_split_t<8>(qx, sx, qw, sw, bias, M, N, K, y, partial, stream);
    }
  }
  if (mode == 1) return launch_few<false>(qx, sx, qw, sw, bias, M, N, K, y, stream);
  if (mode == 2) return launch_few<true>(qw, sw, qx, sx, bias, N, M, K, y, stream);
  return hipErrorInvalidValue;
}

}  // namespace convrot
