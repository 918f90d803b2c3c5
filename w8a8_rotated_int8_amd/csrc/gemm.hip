// Tiled MFMA GEMM for gfx950: out[j][i] = sum_k P[i][k] * Q[j][k].
//
// This is the int8 x int8 -> int32 contraction of the ConvRot INT8 layer
// (sd-scripts pull request 2461, Summary, kernels bullet: fused int8 GEMM with
// a dequantization epilogue; "LoRA Training Guide for MOSS-Image" section 7.1:
// the input gradient through the int8 GEMM or through a transient bf16
// dequantization), in four epilogue flavours:
//   forward:         P = q_w [N, K], Q = q_x [M, K]; y[m][n] =
//                    bf16(fl32(acc) * s_x[m] * s_w[n] (+ bias[n]))
//   int8 grad_x:     P = q_w read as [N, K] but contracted along its rows
//                    (transposed in registers), Q = q_g [M, N]; the epilogue
//                    scales by s_g[m] and applies the inverse rotation along k
//                    inside each 128-block (one wave owns whole blocks)
//   raw int32:       test and timing hook
//   bf16 grad_x:     bf16 operands, fp32 accumulation
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves (2 x 2, each wave
// 128 x 128 = 4 x 4 MFMA 32x32 tiles), 128 contraction bytes per stage, two
// LDS stages (128 KB).  Row-major operands are staged with direct 16-byte
// global->LDS loads; each 128-byte LDS row is XOR-swizzled by
// (row ^ row >> 3) & 7 so that both the MFMA fragment reads (32 consecutive
// rows) and the transposed writes (rows 8 apart) are bank-conflict free.  The
// MFMA "A" operand is P, so each lane ends with 4 consecutive i for one j:
// the epilogue writes 8-byte (bf16) or 16-byte (int32) pieces of an output row.
#include "common.h"
#include "kernels.h"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kTile = 256;
constexpr int kBK = 128;                       // contraction bytes per stage
constexpr int kStage = kTile * kBK;            // bytes per operand per stage
constexpr int kLdsBytes = 4 * kStage;          // 2 stages x (P, Q)

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kBK + 16 * (chunk ^ swz(row));
}

template <bool BF16>
struct AccT;
template <>
struct AccT<false> {
  typedef v16i type;
};
template <>
struct AccT<true> {
  typedef v16f type;
};

__device__ __forceinline__ v16i mfma(uint4 a, uint4 b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(v4i, a),
                                              __builtin_bit_cast(v4i, b), c, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma(uint4 a, uint4 b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// Stage rows [row0, row0 + 256) x bytes [kb0, kb0 + 128) of a row-major operand.
// Rows past the end are clamped to the last row (their results are discarded).
__device__ __forceinline__ void stage_rows(const uint8_t* base, int64_t ld_bytes, int64_t row0,
                                           int64_t nrows, int64_t kb0, uint8_t* lds_stage,
                                           int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int blk = i * 4 + wave;            // 1 KB block of the stage = 8 rows
    int slot = blk * 64 + lane;
    int row = slot >> 3;
    int chunk = (slot & 7) ^ swz(row);
    int64_t gr = row0 + row;
    gr = gr < nrows ? gr : nrows - 1;
    load_lds_16(base + gr * ld_bytes + kb0 + 16 * chunk, lds_stage + blk * 1024);
  }
}

// 4 x 4 byte transpose: out[c] byte r = in[r] byte c.
__device__ __forceinline__ void transpose4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                             uint32_t& o0, uint32_t& o1, uint32_t& o2,
                                             uint32_t& o3) {
  uint32_t t0 = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  uint32_t t1 = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
  uint32_t u0 = __builtin_amdgcn_perm(d, c, 0x05010400u);  // c0 d0 c1 d1
  uint32_t u1 = __builtin_amdgcn_perm(d, c, 0x07030602u);  // c2 d2 c3 d3
  o0 = __builtin_amdgcn_perm(u0, t0, 0x05040100u);         // a0 b0 c0 d0
  o1 = __builtin_amdgcn_perm(u0, t0, 0x07060302u);         // a1 b1 c1 d1
  o2 = __builtin_amdgcn_perm(u1, t1, 0x05040100u);         // a2 b2 c2 d2
  o3 = __builtin_amdgcn_perm(u1, t1, 0x07060302u);         // a3 b3 c3 d3
}

// Transposed int8 operand: source [Kc, I] (I contiguous).  Each lane loads a
// 16 (k) x 8 (i) byte block with 8-byte loads (32 lanes cover the 256 i of the
// tile in one row), transposes it in registers and writes 8 LDS rows (one per
// i) of 16 k-bytes each.
struct TransposedRegs {
  uint2 r[16];
};

__device__ __forceinline__ void load_transposed(const int8_t* src, int64_t ld, int64_t I,
                                                int64_t i0, int64_t k0, int wave, int lane,
                                                TransposedRegs& t) {
  int ic = lane & 31;
  int kg = (lane >> 5) + 2 * wave;
  int64_t i = i0 + 8 * ic;
  i = i + 8 <= I ? i : I - 8;
  const int8_t* p = src + (k0 + 16 * kg) * ld + i;
#pragma unroll
  for (int r = 0; r < 16; ++r) t.r[r] = *reinterpret_cast<const uint2*>(p + r * ld);
}

__device__ __forceinline__ void store_transposed(const TransposedRegs& t, uint8_t* lds_stage,
                                                 int wave, int lane) {
  int ic = lane & 31;
  int kg = (lane >> 5) + 2 * wave;
  uint32_t o[8][4];  // o[j][d]: bytes (k = 4d .. 4d+3) of column i = 8 ic + j
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    transpose4x4(t.r[4 * d].x, t.r[4 * d + 1].x, t.r[4 * d + 2].x, t.r[4 * d + 3].x, o[0][d],
                 o[1][d], o[2][d], o[3][d]);
    transpose4x4(t.r[4 * d].y, t.r[4 * d + 1].y, t.r[4 * d + 2].y, t.r[4 * d + 3].y, o[4][d],
                 o[5][d], o[6][d], o[7][d]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    *reinterpret_cast<uint4*>(lds_stage + lds_off(8 * ic + j, kg)) =
        make_uint4(o[j][0], o[j][1], o[j][2], o[j][3]);
  }
}

template <int EPI, bool PT, bool BF16>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  typedef typename AccT<BF16>::type acc_t;
  constexpr int esz = BF16 ? 2 : 1;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wi = wave & 1, wj = wave >> 1;
  const int64_t i0 = (int64_t)blockIdx.x * kTile;
  const int64_t j0 = (int64_t)blockIdx.y * kTile;
  const int64_t kbytes = a.Kc * esz;
  const int nk = (int)(kbytes / kBK);

  const uint8_t* P = static_cast<const uint8_t*>(a.P);
  const uint8_t* Q = static_cast<const uint8_t*>(a.Q);

  auto Ps = [&](int buf) { return lds + buf * 2 * kStage; };
  auto Qs = [&](int buf) { return lds + buf * 2 * kStage + kStage; };

  acc_t acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = acc_t{};

  TransposedRegs tr;
  // prologue: stage 0
  stage_rows(Q, a.ldq * esz, j0, a.J, 0, Qs(0), wave, lane);
  if (PT) {
    load_transposed(static_cast<const int8_t*>(a.P), a.ldp, a.I, i0, 0, wave, lane, tr);
    store_transposed(tr, Ps(0), wave, lane);
  } else {
    stage_rows(P, a.ldp * esz, i0, a.I, 0, Ps(0), wave, lane);
  }

  int buf = 0;
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmem();
    __syncthreads();
    const bool more = kt + 1 < nk;
    if (more) {
      int64_t kb = (int64_t)(kt + 1) * kBK;
      stage_rows(Q, a.ldq * esz, j0, a.J, kb, Qs(buf ^ 1), wave, lane);
      if (PT) {
        load_transposed(static_cast<const int8_t*>(a.P), a.ldp, a.I, i0, kb, wave, lane, tr);
      } else {
        stage_rows(P, a.ldp * esz, i0, a.I, kb, Ps(buf ^ 1), wave, lane);
      }
    }
    const uint8_t* ps = Ps(buf);
    const uint8_t* qs = Qs(buf);
#pragma unroll
    for (int s = 0; s < kBK / 32; ++s) {
      uint4 pf[4], qf[4];
      const int chunk = 2 * s + (lane >> 5);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        pf[t] = *reinterpret_cast<const uint4*>(ps + lds_off(wi * 128 + t * 32 + (lane & 31), chunk));
        qf[t] = *reinterpret_cast<const uint4*>(qs + lds_off(wj * 128 + t * 32 + (lane & 31), chunk));
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = mfma(pf[x], qf[y], acc[x][y]);
    }
    if (PT && more) store_transposed(tr, Ps(buf ^ 1), wave, lane);
    buf ^= 1;
  }

  // ---- epilogue -------------------------------------------------------------
  const int h = lane >> 5;
  if (EPI == kEpiInvRotBf16) {
    const int64_t iblk = i0 + wi * 128;
    if (iblk >= a.I) return;
    uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int64_t j = j0 + wj * 128 + y * 32 + (lane & 31);
      const float sjv = j < a.J ? a.sj[j] : 0.f;
      float w[64];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int r = 0; r < 16; ++r) w[x * 16 + r] = (float)acc[x][y][r] * sjv;
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
      if (j < a.J) {
        const float cf = (float)kInvSqrt128;
        uint16_t* orow = out + j * a.ldo + iblk;
#pragma unroll
        for (int q4 = 0; q4 < 8; ++q4) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int e = 4 * q4 + 32 * half;
            const int il = ((q4 & 3) << 3) | ((q4 >> 2) << 5) | (h << 6) | (half << 2);
            uint2 pk = make_uint2(pack_bf16x2(w[e] * cf, w[e + 1] * cf),
                                  pack_bf16x2(w[e + 2] * cf, w[e + 3] * cf));
            *reinterpret_cast<uint2*>(orow + il) = pk;
          }
        }
      }
    }
    return;
  }

#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const int64_t j = j0 + wj * 128 + y * 32 + (lane & 31);
    if (j >= a.J) continue;
    float sjv = 1.f;
    if (EPI == kEpiDequantBf16) sjv = a.sj[j];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t i = i0 + wi * 128 + x * 32 + 8 * g + 4 * h;
        if (i >= a.I) continue;
        const bool full = i + 4 <= a.I;
        if (EPI == kEpiI32) {
          int32_t* orow = static_cast<int32_t*>(a.out) + j * a.ldo;
          int v0 = (int)acc[x][y][4 * g], v1 = (int)acc[x][y][4 * g + 1],
              v2 = (int)acc[x][y][4 * g + 2], v3 = (int)acc[x][y][4 * g + 3];
          if (full) {
            *reinterpret_cast<int4*>(orow + i) = make_int4(v0, v1, v2, v3);
          } else {
            int vv[4] = {v0, v1, v2, v3};
            for (int u = 0; u < 4 && i + u < a.I; ++u) orow[i + u] = vv[u];
          }
        } else {
          float v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = (float)acc[x][y][4 * g + u];
          if (EPI == kEpiDequantBf16) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              int64_t iu = i + u < a.I ? i + u : a.I - 1;
              float sv = a.si[iu];
              float t = v[u] * sjv * sv;
              if (a.bias) t = t + bf16lo_to_f32(a.bias[iu]);
              v[u] = t;
            }
          }
          uint16_t* orow = static_cast<uint16_t*>(a.out) + j * a.ldo;
          if (full) {
            *reinterpret_cast<uint2*>(orow + i) =
                make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          } else {
            for (int u = 0; u < 4 && i + u < a.I; ++u) orow[i + u] = (uint16_t)f32_to_bf16_rne(v[u]);
          }
        }
      }
    }
  }
}

template <int EPI, bool PT, bool BF16>
hipError_t launch(const GemmArgs& a, hipStream_t stream) {
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_kernel<EPI, PT, BF16>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    configured = true;
  }
  int64_t gi = (a.I + kTile - 1) / kTile, gj = (a.J + kTile - 1) / kTile;
  if (gi <= 0 || gj <= 0) return hipSuccess;
  if (gi > 0x7fffffff || gj > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_kernel<EPI, PT, BF16>), dim3((unsigned)gi, (unsigned)gj), dim3(256),
                     kLdsBytes, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_i8(const GemmArgs& a, int epilogue, bool p_transposed, hipStream_t stream) {
  if (p_transposed) {
    if (epilogue == kEpiI32) return launch<kEpiI32, true, false>(a, stream);
    if (epilogue == kEpiInvRotBf16) return launch<kEpiInvRotBf16, true, false>(a, stream);
    return hipErrorInvalidValue;
  }
  if (epilogue == kEpiI32) return launch<kEpiI32, false, false>(a, stream);
  if (epilogue == kEpiDequantBf16) return launch<kEpiDequantBf16, false, false>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t stream) {
  return launch<kEpiBf16, false, true>(a, stream);
}

}  // namespace convrot
