// Tiled MFMA GEMM for gfx950: out[j][i] = sum_k P[i][k] * Q[j][k].
//
// This is the int8 x int8 -> int32 contraction of the ConvRot INT8 layer
// (sd-scripts pull request 2461, Summary, kernels bullet: fused int8 GEMM with
// a dequantization epilogue; "LoRA Training Guide for MOSS-Image" section 7.1:
// the input gradient through the int8 GEMM or through a transient bf16
// dequantization), in four epilogue flavours:
//   forward:         P = q_w [N, K], Q = q_x [M, K]; y[m][n] =
//                    bf16(fl32(fl32(fl32(acc) * s_w[n]) * s_x[m]) (+ bias[n]))
//   int8 grad_x:     P = q_w read as [N, K] but contracted along its rows
//                    (staged as is, transposed by the LDS reads), Q = q_g
//                    [M, N]; the epilogue
//                    scales by s_g[m] and applies the inverse rotation along k
//                    inside each 128-block (one wave owns whole blocks)
//   raw int32:       test and timing hook
//   bf16 grad_x:     bf16 operands, fp32 accumulation
//
// Tiling: a UI x UJ output tile per workgroup (256 x 256; the dequantizing
// forward also has 128 x 128 and 128 x 64 forms for launches that would leave
// CUs idle).  WI x WJ waves split it into wave tiles of (UI/WI) x (UJ/WJ),
// each a grid of 32x32 MFMA tiles.  The contraction advances BK bytes per
// stage through a ring of STAGES LDS buffers; loads run STAGES-1 stages ahead
// of the MFMAs.  Row-major operands
// are staged with direct 16-byte global->LDS loads.  LDS rows (BK bytes) are
// XOR-swizzled at 16-byte granularity so that the MFMA fragment reads (32
// consecutive rows, one 16-byte chunk each) hit distinct banks.  P is the MFMA
// "A" operand, so each lane ends with 4 consecutive i for one j: the epilogue
// writes 8-byte (bf16) or 16-byte (int32) pieces of an output row.
//
// Workgroups are mapped to tiles XCD-aware: the hardware deals workgroups to
// the 8 XCDs round-robin, so consecutive dispatch ids are first regrouped per
// XCD, and each XCD then walks a compact block of tiles (GROUP_J j-tiles wide)
// whose P and Q rows are shared through that XCD's L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

#ifndef CONVROT_GEMM_WI
#define CONVROT_GEMM_WI 2
#endif
#ifndef CONVROT_GEMM_WJ
#define CONVROT_GEMM_WJ 4
#endif
#ifndef CONVROT_GEMM_BK
#define CONVROT_GEMM_BK 128
#endif
#ifndef CONVROT_GEMM_STAGES
#define CONVROT_GEMM_STAGES 2
#endif
#ifndef CONVROT_GEMM_GROUP_J
#define CONVROT_GEMM_GROUP_J 4
#endif


namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kTile = 256;
constexpr int kNumXcd = 8;

// 16-byte chunk swizzle of an LDS row of BK bytes.
template <int BK>
__device__ __forceinline__ int swz(int row) {
  if constexpr (BK == 128) return (row ^ (row >> 3)) & 7;
  else return (row >> 1) & 3;
}
template <int BK>
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * BK + 16 * (chunk ^ swz<BK>(row));
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

template <int N>
__device__ __forceinline__ void wait_vm() { wait_vm_n<N>(); }
// Wait until at most `later` stages of LOADS direct-to-LDS loads each are in flight.
template <int LOADS, int MAXLATER>
__device__ __forceinline__ void wait_stages(int later) {
  if constexpr (MAXLATER >= 4) { if (later >= 4) { wait_vm<LOADS * 4>(); return; } }
  if constexpr (MAXLATER >= 3) { if (later >= 3) { wait_vm<LOADS * 3>(); return; } }
  if constexpr (MAXLATER >= 2) { if (later >= 2) { wait_vm<LOADS * 2>(); return; } }
  if constexpr (MAXLATER >= 1) { if (later >= 1) { wait_vm<LOADS>(); return; } }
  wait_vm<0>();
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would wait for every outstanding load, including the prefetched stages.
// Callers wait explicitly for the data they need before it.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("s_barrier" ::: "memory");
}

// Dispatch id -> (i tile, j tile), XCD-aware (see the file comment).
// `tile` is the launch-order index of the tile (the dispatch id of a
// one-tile-per-workgroup launch).
__device__ __forceinline__ void tile_of(int64_t gi, int64_t gj, int64_t tile, int& ti, int& tj) {
  const int64_t nb = gi * gj;
  int64_t b = tile;
  if (nb % kNumXcd == 0) b = (b % kNumXcd) * (nb / kNumXcd) + b / kNumXcd;
  const int64_t G = CONVROT_GEMM_GROUP_J;
  const int64_t per_group = G * gi;
  const int64_t group = b / per_group;
  const int64_t first_j = group * G;
  const int64_t gsize = gj - first_j < G ? gj - first_j : G;
  const int64_t r = b % per_group;
  tj = (int)(first_j + r % gsize);
  ti = (int)(r / gsize);
}

// Dequantizing epilogue of four consecutive outputs i .. i+3 of row j:
// v = fl32(fl32(fl32(acc) * s_i) * s_j) (+ bias_i), each operation rounded to
// fp32 in this order (no contraction), so every path that uses it rounds
// identically.  In the forward s_i is the weight's row scale and s_j the
// activation's: the static weight scale comes first, so the first product stays
// below 2^31 * s_i and no activation scale, however large, can make an
// intermediate overflow where the result does not (only a weight scale beyond
// ~2^96, |W| ~ 1e31, could).
__device__ __forceinline__ void dequant4(float v[4], float sjv, const float* si,
                                         const uint16_t* bias, int64_t i, int64_t I) {
#pragma clang fp contract(off)
  if (i + 4 <= I) {
    const float4 s4 = *reinterpret_cast<const float4*>(si + i);
    v[0] = v[0] * s4.x * sjv;
    v[1] = v[1] * s4.y * sjv;
    v[2] = v[2] * s4.z * sjv;
    v[3] = v[3] * s4.w * sjv;
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t iu = i + u < I ? i + u : I - 1;
      v[u] = v[u] * si[iu] * sjv;
    }
  }
  if (bias) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t iu = i + u < I ? i + u : I - 1;
      v[u] = v[u] + __uint_as_float((uint32_t)bias[iu] << 16);
    }
  }
}

// dequant4 with the tile's 256 s_i values staged in LDS (si_tile[i - i0]):
// the same operations in the same order.
__device__ __forceinline__ void dequant4_tile(float v[4], float sjv, const float* si_tile,
                                              const uint16_t* bias, int64_t i, int64_t i0,
                                              int64_t I) {
#pragma clang fp contract(off)
  if (i + 4 <= I) {
    const float4 s4 = *reinterpret_cast<const float4*>(si_tile + (i - i0));
    v[0] = v[0] * s4.x * sjv;
    v[1] = v[1] * s4.y * sjv;
    v[2] = v[2] * s4.z * sjv;
    v[3] = v[3] * s4.w * sjv;
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t iu = i + u < I ? i + u : I - 1;
      v[u] = v[u] * si_tile[iu - i0] * sjv;
    }
  }
  if (bias) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t iu = i + u < I ? i + u : I - 1;
      v[u] = v[u] + __uint_as_float((uint32_t)bias[iu] << 16);
    }
  }
}

// dequant4_tile with the four s_i values of i .. i+3 already in registers (s4,
// read from the staged tile scales once per tile rather than once per 32-row
// slice): the same operations in the same order.  Past the end of a ragged
// tile (i + 4 > I) the values come from the staged copy element by element.
__device__ __forceinline__ void dequant4_pre(float v[4], float sjv, float4 s4,
                                             const float* si_tile, const uint16_t* bias,
                                             int64_t i, int64_t i0, int64_t I) {
#pragma clang fp contract(off)
  if (i + 4 <= I) {
    v[0] = v[0] * s4.x * sjv;
    v[1] = v[1] * s4.y * sjv;
    v[2] = v[2] * s4.z * sjv;
    v[3] = v[3] * s4.w * sjv;
    if (bias) {
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = v[u] + __uint_as_float((uint32_t)bias[i + u] << 16);
    }
  } else {
    dequant4_tile(v, sjv, si_tile, bias, i, i0, I);
  }
}

// One UI x UJ output tile (i x j; 256 x 256 unless a smaller tile gives a
// launch more workgroups); every thread of the workgroup takes part.  LDS at
// `lds`: the operand ring (STAGES * (UI + UJ) * BK bytes), plus 32 KB for the
// LoRA epilogue or 4 * UI bytes for the tile's s_i values of the dequantizing
// one.
template <int EPI, bool PT, bool BF16, int WI, int WJ, int BK, int STAGES, int UI = kTile,
          int UJ = kTile>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int64_t tile, uint8_t* lds) {
  typedef typename AccT<BF16>::type acc_t;
  constexpr int esz = BF16 ? 2 : 1;
  constexpr int NT = 64 * WI * WJ;
  constexpr int TI = UI / WI, TJ = UJ / WJ;  // wave tile
  constexpr int NI = TI / 32, NJ = TJ / 32;  // MFMA tiles per wave
  constexpr int kStageP = UI * BK, kStageQ = UJ * BK;  // bytes per operand per stage
  constexpr int kBuf = kStageP + kStageQ;              // one stage of both operands
  constexpr int kRing = STAGES * kBuf;
  constexpr int kLoadsPerStage = (UI + UJ) * (BK / 16) / NT;  // DMA per thread per stage
  static_assert(UI * (BK / 16) % NT == 0 && UJ * (BK / 16) % NT == 0,
                "every thread issues the same number of stage loads");
  static_assert(NI >= 1 && NJ >= 1 && TI % 32 == 0 && TJ % 32 == 0, "whole 32x32 MFMA tiles");
  static_assert(!PT || (UI == kTile && UJ == kTile && BK == 128 && (NT == 256 || NT == 512) &&
                        STAGES == 2),
                "transposed P: 256 x 256 tiles, BK 128, 4 or 8 waves, 2 stages");
  static_assert(EPI != kEpiDequantLoraBf16 || (UI == kTile && UJ == kTile),
                "LoRA epilogue: 256 x 256 tiles");
  static_assert(EPI != kEpiDequantBf16 || UI <= NT, "UI / 64 waves load the tile's s_i values");
  static_assert(EPI != kEpiInvRotBf16 || TI == 128, "inverse rotation needs 128-wide wave tiles");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wi = wave % WI, wj = wave / WI;
  const int64_t gi = (a.I + UI - 1) / UI, gj = (a.J + UJ - 1) / UJ;
  int ti, tj;
  tile_of(gi, gj, tile, ti, tj);
  const int64_t i0 = (int64_t)ti * UI;
  const int64_t j0 = (int64_t)tj * UJ;
  const int nk = (int)(a.Kc * esz / BK);
  // Dequantizing epilogues read s_j and s_i.  Loaded there, after the main
  // loop, their latency sat in front of every store (~3 us per 4096^3
  // launch); s_j is loaded into registers now and the dequantizing kernel's
  // UI s_i values are copied to LDS together with the first stage.
  constexpr bool kScales =
      EPI == kEpiDequantBf16 || EPI == kEpiDequantLoraBf16 || EPI == kEpiInvRotBf16;
  // The LoRA epilogue of rank 16 leaves 16 KB of its 32 KB LDS region free,
  // enough for the s_i values too; rank 32 reads them from global memory.
  constexpr bool kTileScales = EPI == kEpiDequantBf16 && !PT;
  const bool tile_scales = kTileScales || (EPI == kEpiDequantLoraBf16 && a.lora_r == 16);
  const float* const si_tile = reinterpret_cast<const float*>(
      lds + kRing + (EPI == kEpiDequantLoraBf16 ? 2 * kTile * 32 : 0));
  float sj_pre[NJ];
#pragma unroll
  for (int y = 0; y < NJ; ++y) {
    const int64_t j = j0 + wj * TJ + y * 32 + (lane & 31);
    sj_pre[y] = kScales && j < a.J ? a.sj[j] : 0.f;
  }
  // LoRA epilogue: the tile's 256 rows of lora_b (i) and lora_xa (j), R bf16
  // each, are copied to LDS past the operand ring now, long before the
  // epilogue reads them as MFMA fragments.
  uint8_t* const lora_lds = lds + kRing;
  if constexpr (EPI == kEpiDequantLoraBf16) {
    const int per_row = a.lora_r / 8;  // 16-byte pieces per row
    for (int c = threadIdx.x; c < 2 * kTile * per_row; c += NT) {
      const int op = c >= kTile * per_row;
      const int cc = c - op * kTile * per_row;
      const int row = cc / per_row, piece = cc % per_row;
      int64_t g = (op ? j0 : i0) + row;
      const int64_t lim = op ? a.J : a.I;
      g = g < lim ? g : lim - 1;
      const uint16_t* src = (op ? a.lora_xa : a.lora_b) + g * a.lora_r + 8 * piece;
      *reinterpret_cast<uint4*>(lora_lds + (op * kTile + row) * a.lora_r * 2 + 16 * piece) =
          *reinterpret_cast<const uint4*>(src);
    }
  }

  const uint8_t* P = static_cast<const uint8_t*>(a.P);
  const uint8_t* Q = static_cast<const uint8_t*>(a.Q);
  auto Ps = [&](int buf) { return lds + buf * kBuf; };
  auto Qs = [&](int buf) { return lds + buf * kBuf + kStageP; };

  acc_t acc[NI][NJ];
#pragma unroll
  for (int x = 0; x < NI; ++x)
#pragma unroll
    for (int y = 0; y < NJ; ++y) acc[x][y] = acc_t{};

  // The transposed P of the int8 input gradient (q_w read as [k][i]) is
  // staged in its natural layout and transposed by the LDS reads.
  constexpr bool TR = PT;
  {
    // Per-thread source pointers and LDS destinations of the stage loads,
    // computed once: a stage load is then one 64-bit add per instruction.
    constexpr int kDmaP = UI * (BK / 16) / NT, kDmaQ = UJ * (BK / 16) / NT;  // per stage
    const uint8_t* src[kDmaP + kDmaQ];
    uint32_t dst_off[kDmaP + kDmaQ];
#pragma unroll
    for (int op = 0; op < 2; ++op) {
#pragma unroll
      for (int it = 0; it < (op ? kDmaQ : kDmaP); ++it) {
        const int blk = it * (NT / 64) + wave;
        const int slot = blk * 64 + lane;
        if (TR && op == 0) {
          // P in its natural layout [k][i]: the stage holds BK k-rows of the
          // tile's 256 i-bytes; 16-byte position q of row n holds piece
          // q ^ 2 (n & 7).  A 32-lane half of a transpose read touches 8 rows
          // and two adjacent pieces (an even one and the next), which then
          // land in 16 different positions: no bank conflicts.
          const int n = slot >> 4, q = slot & 15;
          int64_t col = i0 + 16 * (q ^ (2 * (n & 7)));
          col = col + 16 <= a.I ? col : a.I - 16;  // columns past the end: valid, unused
          src[it] = P + (int64_t)n * a.ldp + col;
          dst_off[it] = blk * 1024;
          continue;
        }
        const int row = slot / (BK / 16);
        const int chunk = (slot % (BK / 16)) ^ swz<BK>(row);
        const int64_t row0 = op ? j0 : i0, nrows = op ? a.J : a.I;
        int64_t gr = row0 + row;
        gr = gr < nrows ? gr : nrows - 1;
        src[op * kDmaP + it] = (op ? Q : P) + gr * ((op ? a.ldq : a.ldp) * esz) + 16 * chunk;
        dst_off[op * kDmaP + it] = (op ? kStageP : 0) + blk * 1024;  // uniform
      }
    }
    const uint32_t lds_base = lds_u32(lds);
    // The P and Q loads of stage kt into buffer buf.
    auto issue_p = [&](int kt, int buf) {
      const int64_t kb = (int64_t)kt * BK;
      const int64_t kbp = TR ? kb * a.ldp : kb;  // P advances by rows when it is [k][i]
      const uint32_t b0 = lds_base + buf * kBuf;
#pragma unroll
      for (int d = 0; d < kDmaP; ++d) dma16(src[d] + kbp, b0 + dst_off[d]);
    };
    auto issue_q = [&](int kt, int buf) {
      const int64_t kb = (int64_t)kt * BK;
      const uint32_t b0 = lds_base + buf * kBuf;
#pragma unroll
      for (int d = kDmaP; d < kDmaP + kDmaQ; ++d) dma16(src[d] + kb, b0 + dst_off[d]);
    };
    auto issue = [&](int kt, int buf) {
      issue_p(kt, buf);
      issue_q(kt, buf);
    };
    constexpr int SL = BK / 32;
    static_assert(SL % 2 == 0, "fragment double buffer alternates per slice");
    uint4 F[2][NI + NJ];
    auto read_frags = [&](int buf, int s, uint4* f) {
      const uint8_t* ps = Ps(buf);
      const uint8_t* qs = Qs(buf);
      const int chunk = 2 * s + (lane >> 5);
      if constexpr (TR) {
        // ds_read_b64_tr_b8: in each 16-lane group, lane j < 8 receives byte j
        // of the 8-byte rows addressed by the group's even lanes, lane j >= 8
        // byte j - 8 of those of its odd lanes.  Even lane 2m and odd lane
        // 2m + 1 address k-row n0 + m at i-offsets +0 and +8, so lane j gets
        // k-rows n0 .. n0 + 7 of output row i = base + j: two reads (n0 and
        // n0 + 8) give the 16 k-contiguous bytes of the MFMA's A operand,
        // the same layout as the row-major path.
        const lds_u8* ps3 = (const lds_u8*)ps;
        const int a16 = lane & 15;
        const int n0 = 32 * s + 16 * (lane >> 5) + (a16 >> 1);
#pragma unroll
        for (int t = 0; t < NI; ++t) {
          const int ib = wi * TI + t * 32 + 16 * ((lane >> 4) & 1) + 8 * (a16 & 1);
          const int pc = ib >> 4, hb = 8 * (a16 & 1);
          const int pos = 16 * (pc ^ (2 * (n0 & 7))) + hb;  // rows n0 and n0 + 8 alike
          const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(ps3 + n0 * 256 + pos));
          const v2i hi =
              __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(ps3 + (n0 + 8) * 256 + pos));
          f[t] = make_uint4((uint32_t)lo.x, (uint32_t)lo.y, (uint32_t)hi.x, (uint32_t)hi.y);
        }
      } else {
#pragma unroll
        for (int t = 0; t < NI; ++t)
          f[t] = *reinterpret_cast<const uint4*>(ps + lds_off<BK>(wi * TI + t * 32 + (lane & 31), chunk));
      }
#pragma unroll
      for (int t = 0; t < NJ; ++t)
        f[NI + t] = *reinterpret_cast<const uint4*>(qs + lds_off<BK>(wj * TJ + t * 32 + (lane & 31), chunk));
    };
    if (tile_scales) {
      // older than the stage loads, so complete once stage 0 is, and published
      // by the same barrier
      if (wave < UI / 64) {
        const int64_t i = i0 + wave * 64 + lane;
        dma4(static_cast<const float*>(a.si) + (i < a.I ? i : a.I - 1),
             lds_u32(si_tile) + wave * 256);
      }
    }
    // all STAGES buffers start filled; the buffer of stage kt is refilled with
    // stage kt + STAGES at the end of stage kt
#pragma unroll
    for (int st = 0; st < STAGES; ++st)
      if (st < nk) issue(st, st);
    {
      const int later = nk - 1 < STAGES - 1 ? nk - 1 : STAGES - 1;
      wait_stages<kLoadsPerStage, STAGES - 1>(later);
      raw_barrier();
    }
    read_frags(0, 0, F[0]);
    // One stage.  HAS_NEXT is a compile-time flag (the final stage is peeled
    // off the loop) so that no control-flow join sits between the fragment
    // reads of stage kt+1 and the MFMAs of stage kt's last slice: at such a
    // join the waitcnt insertion becomes conservative and would make those
    // MFMAs wait for the reads just issued.
    // MFMAs of slice s with the fragment reads of the next slice interleaved
    // one read per MFMA, so neither wave of a SIMD issues a burst of reads
    // while the matrix pipe waits.
    auto mfma_slice = [&](int s) {
#pragma unroll
      for (int x = 0; x < NI; ++x)
#pragma unroll
        for (int y = 0; y < NJ; ++y) acc[x][y] = mfma(F[s & 1][x], F[s & 1][NI + y], acc[x][y]);
      // a transposed P fragment takes two 8-byte transpose reads
      constexpr int NR = (TR ? 2 : 1) * NI + NJ, NM = NI * NJ;
      constexpr int NP = NR < NM ? NR : NM;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      }
      if constexpr (NM > NP) __builtin_amdgcn_sched_group_barrier(0x008, NM - NP, 0);
      if constexpr (NR > NP) __builtin_amdgcn_sched_group_barrier(0x100, NR - NP, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    // One stage.  HAS_NEXT is a compile-time flag (the final stage is peeled
    // off the loop) so that no control-flow join sits between the fragment
    // reads of stage kt+1 and the MFMAs of stage kt's last slice: at such a
    // join the waitcnt insertion becomes conservative and would make those
    // MFMAs wait for the reads just issued.
    auto stage = [&](int kt, auto has_next) {
      constexpr bool HAS_NEXT = decltype(has_next)::value;
      const int buf = kt % STAGES;
#pragma unroll
      for (int s = 0; s < SL; ++s) {
        const bool last = s + 1 == SL;
        if (!last) {
          read_frags(buf, s + 1, F[(s + 1) & 1]);
          mfma_slice(s);
          // the Q half of the refill started at the end of stage kt-1
          if (s == 0 && kt >= 1 && kt - 1 + STAGES < nk) issue_q(kt - 1 + STAGES, (kt - 1) % STAGES);
        } else if constexpr (HAS_NEXT) {
          // Retire this wave's reads of stage kt, wait for stage kt+1 (at most
          // min(STAGES-2, nk-2-kt) later stages in flight) and publish; the
          // MFMAs of earlier slices keep the matrix pipe busy meanwhile.
          __builtin_amdgcn_s_waitcnt(0xc07f);
          const int later = nk - 2 - kt < STAGES - 2 ? nk - 2 - kt : STAGES - 2;
          wait_stages<kLoadsPerStage, STAGES - 2>(later);
          raw_barrier();
          __builtin_amdgcn_sched_barrier(0);
          read_frags((kt + 1) % STAGES, 0, F[(s + 1) & 1]);
          mfma_slice(s);
          // refill the buffer of stage kt (every wave is past its reads of
          // it: the barrier above): the P half now, the Q half after the
          // first slice of stage kt+1.  All eight waves issuing a whole
          // stage's loads at once right after the barrier queued 64 KB of
          // requests together and held the waves behind them; split, the
          // 4096^3 forward GEMM measured ~3% faster (same-box A/B, 61.8-62.5
          // vs 60.0-60.7 us).  The wait at the end of stage kt+1 still covers
          // both halves: it leaves in flight only the STAGES - 2 stages issued
          // after stage kt+2 (with two stages it waits for every load).
          static_assert(STAGES >= 2, "the split refill needs a second buffer");
          if (kt + STAGES < nk) issue_p(kt + STAGES, buf);
        } else {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int x = 0; x < NI; ++x)
#pragma unroll
            for (int y = 0; y < NJ; ++y) acc[x][y] = mfma(F[s & 1][x], F[s & 1][NI + y], acc[x][y]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    for (int kt = 0; kt + 1 < nk; ++kt) stage(kt, std::true_type{});
    if (nk > 0) stage(nk - 1, std::false_type{});
  }

  // ---- epilogue -------------------------------------------------------------
  const int h = lane >> 5;
  if constexpr (EPI == kEpiI32) {
#pragma unroll
    for (int y = 0; y < NJ; ++y) {
      const int64_t j = j0 + wj * TJ + y * 32 + (lane & 31);
      if (j >= a.J) continue;
      int32_t* orow = static_cast<int32_t*>(a.out) + j * a.ldo;
#pragma unroll
      for (int x = 0; x < NI; ++x) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t i = i0 + wi * TI + x * 32 + 8 * g + 4 * h;
          if (i >= a.I) continue;
          int vv[4] = {(int)acc[x][y][4 * g], (int)acc[x][y][4 * g + 1],
                       (int)acc[x][y][4 * g + 2], (int)acc[x][y][4 * g + 3]};
          if (i + 4 <= a.I) {
            *reinterpret_cast<int4*>(orow + i) = make_int4(vv[0], vv[1], vv[2], vv[3]);
          } else {
            for (int u = 0; u < 4 && i + u < a.I; ++u) orow[i + u] = vv[u];
          }
        }
      }
    }
  } else {
    // bf16 results: each wave stages its TJ x TI sub-tile in LDS (rows of TI
    // bf16, 16-byte chunks XOR-swizzled by the row), then writes 16-byte
    // pieces of contiguous output rows, so every store instruction covers whole
    // cache lines instead of 16 bytes of 32 different rows.
    constexpr int kRowBytes = TI * 2;
    constexpr int kChunkMask = TI / 8 - 1;
    static_assert(WI * WJ * TJ * kRowBytes <= kRing, "staging fits the LDS ring");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes (LoRA rows) landed
    raw_barrier();  // all waves are done with the operand ring
    uint8_t* stg = lds + wave * TJ * kRowBytes;
    auto put8 = [&](int jl, int il, uint32_t lo, uint32_t hi) {
      const int pos = (il >> 3) ^ (jl & kChunkMask);
      *reinterpret_cast<uint2*>(stg + jl * kRowBytes + pos * 16 + (il & 7) * 2) = make_uint2(lo, hi);
    };
    // Write the staged rows 32 y0 .. 32 (y0 + ny) - 1 of this wave's sub-tile:
    // 16-byte chunks of contiguous output rows, 64 lanes per step.  The
    // dequantizing epilogues (with or without LoRA) call it after each y, so the
    // stores of one slice are in flight while the next is converted.  The stores
    // are non-temporal: nothing here reads the output back, and the 4096^3
    // forward measured ~1.3 us faster than with plain stores.
    uint16_t* out = static_cast<uint16_t*>(a.out);
    auto flush = [&](int y0, int ny) {
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes landed
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
      const int kChunks = 32 * ny * (TI / 8);
#pragma unroll 4
      for (int c0 = 0; c0 < kChunks; c0 += 64) {
        const int idx = c0 + lane;
        const int jl = 32 * y0 + idx / (TI / 8), c = idx % (TI / 8);
        const uint4 v = *reinterpret_cast<const uint4*>(stg + jl * kRowBytes + ((c ^ (jl & kChunkMask)) * 16));
        const int64_t j = j0 + wj * TJ + jl;
        const int64_t i = i0 + wi * TI + 8 * c;
        if (j >= a.J || i >= a.I) continue;
        uint16_t* dst = out + j * a.ldo + i;
        if (i + 8 <= a.I) {
          store16_nt(dst, v);
        } else {
          const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
          for (int u = 0; u < 8 && i + u < a.I; ++u) dst[u] = (uint16_t)(wds[u >> 1] >> (16 * (u & 1)));
        }
      }
    };
    if constexpr (EPI == kEpiInvRotBf16) {
      static_assert(TI == 128, "one wave owns whole 128-blocks along i");
#pragma unroll
      for (int y = 0; y < NJ; ++y) {
        const int jl = y * 32 + (lane & 31);
        const int64_t j = j0 + wj * TJ + jl;
        // a row scale beyond 2^96 enters as its mantissa, and its 2^e joins the
        // final constant 1/sqrt(128) (exact; see row_scale)
        const RowScale sj = row_scale(sj_pre[y]);
        float w[64];
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int r = 0; r < 16; ++r) w[x * 16 + r] = (float)acc[x][y][r] * sj.m;
        // w index bits 0-1 -> i bits 0-1, bits 2-3 -> i bits 3-4, bits 4-5 ->
        // i bits 5-6; the lane half h is i bit 2.
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
        const float cf = __builtin_ldexpf((float)kInvSqrt128, sj.e);
#pragma unroll
        for (int q4 = 0; q4 < 8; ++q4) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int e = 4 * q4 + 32 * half;
            const int il = ((q4 & 3) << 3) | ((q4 >> 2) << 5) | (h << 6) | (half << 2);
            put8(jl, il, pack_bf16x2(w[e] * cf, w[e + 1] * cf),
                 pack_bf16x2(w[e + 2] * cf, w[e + 3] * cf));
          }
        }
      }
      flush(0, NJ);
    } else {
      constexpr bool kDequant = EPI == kEpiDequantBf16 || EPI == kEpiDequantLoraBf16;
      constexpr bool kLora = EPI == kEpiDequantLoraBf16;
      // LoRA up projection: per 32 x 32 tile, lora_b rows (i) . lora_xa rows
      // (j) over the rank with v_mfma_f32_32x32x16_bf16 (one or two k-steps),
      // whose accumulator layout matches acc[x][y]; fragments come from the
      // rows staged in LDS at the start of the tile.
      auto lora_frag = [&](int op, int row, int kk) {
        return *reinterpret_cast<const uint4*>(lora_lds + (op * kTile + row) * a.lora_r * 2 +
                                               16 * h + 32 * kk);
      };
      // the lane's s_i values (four per (x, g), the same for every y), read from
      // the staged tile scales once: 0.5 us less per 4096^3 launch than
      // re-reading them for each 32-row slice (same-box A/B, 60.2 -> 59.6 us)
      float4 si4[NI][4];
      if constexpr (kTileScales) {
#pragma unroll
        for (int x = 0; x < NI; ++x)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            si4[x][g] = *reinterpret_cast<const float4*>(si_tile + (wi * TI + x * 32 + 8 * g + 4 * h));
      }
#pragma unroll
      for (int y = 0; y < NJ; ++y) {
        const int jl = y * 32 + (lane & 31);
        float sjv = 1.f;
        if constexpr (kDequant) sjv = sj_pre[y];
#pragma unroll
        for (int x = 0; x < NI; ++x) {
          v16f lo = {};
          if constexpr (kLora) {
            const int ri = wi * TI + x * 32 + (lane & 31), rj = wj * TJ + y * 32 + (lane & 31);
            lo = mfma(lora_frag(0, ri, 0), lora_frag(1, rj, 0), lo);
            if (a.lora_r > 16) lo = mfma(lora_frag(0, ri, 1), lora_frag(1, rj, 1), lo);
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int il = x * 32 + 8 * g + 4 * h;
            const int64_t i = i0 + wi * TI + il;
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = (float)acc[x][y][4 * g + u];
            if constexpr (kTileScales) {
              dequant4_pre(v, sjv, si4[x][g], si_tile, a.bias, i, i0, a.I);
            } else if constexpr (kLora) {
              if (tile_scales) dequant4_tile(v, sjv, si_tile, a.bias, i, i0, a.I);
              else dequant4(v, sjv, a.si, a.bias, i, a.I);
            } else if constexpr (kDequant) {
              dequant4(v, sjv, a.si, a.bias, i, a.I);
            }
            if constexpr (kLora) {
#pragma unroll
              for (int u = 0; u < 4; ++u) v[u] = v[u] + a.lora_scale * lo[4 * g + u];
            }
            put8(jl, il, pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          }
        }
        flush(y, 1);
      }
    }
  }
}

// A smaller tile keeps its registers within two workgroups per CU.
template <int EPI, bool PT, bool BF16, int WI, int WJ, int BK, int STAGES, int UI = kTile,
          int UJ = kTile>
__global__ __launch_bounds__(64 * WI * WJ, UI * UJ < kTile * kTile ? 2 : 1) void gemm_kernel(
    GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  gemm_tile<EPI, PT, BF16, WI, WJ, BK, STAGES, UI, UJ>(a, blockIdx.x, lds);
}

// Split-K: workgroup (slice s, tile t) with blockIdx = s * tiles + t contracts
// K-slice s of both row-major int8 operands into the int32 partial tile
// partial[s] ([J, I], row stride I).
template <int WI, int WJ, int BK, int STAGES>
__global__ __launch_bounds__(64 * WI * WJ, 1) void gemm_splitk_kernel(GemmArgs a, int64_t tiles,
                                                                      int64_t k_slice,
                                                                      int32_t* partial) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int64_t s = blockIdx.x / tiles;
  GemmArgs b = a;
  b.P = static_cast<const int8_t*>(a.P) + s * k_slice;
  b.Q = static_cast<const int8_t*>(a.Q) + s * k_slice;
  b.Kc = k_slice;
  b.out = partial + s * a.J * a.I;
  b.ldo = a.I;
  gemm_tile<kEpiI32, false, false, WI, WJ, BK, STAGES>(b, blockIdx.x % tiles, lds);
}

// y[j][i..i+3] = dequant4( sum_s partial[s][j][i..i+3] ) as bf16; one thread
// per 4 outputs (I % 4 == 0).
__global__ __launch_bounds__(256) void splitk_dequant_kernel(const int32_t* __restrict__ partial,
                                                             int S, int64_t J, int64_t I,
                                                             const float* __restrict__ si,
                                                             const float* __restrict__ sj,
                                                             const uint16_t* __restrict__ bias,
                                                             uint16_t* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // quad index
  const int64_t per_row = I / 4;
  if (q >= J * per_row) return;
  const int64_t j = q / per_row, i = 4 * (q % per_row);
  int4 acc = *reinterpret_cast<const int4*>(partial + j * I + i);
  for (int s = 1; s < S; ++s) {
    const int4 p = *reinterpret_cast<const int4*>(partial + (s * J + j) * I + i);
    acc.x += p.x;
    acc.y += p.y;
    acc.z += p.z;
    acc.w += p.w;
  }
  float v[4] = {(float)acc.x, (float)acc.y, (float)acc.z, (float)acc.w};
  dequant4(v, sj[j], si, bias, i, I);
  *reinterpret_cast<uint2*>(out + j * I + i) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

template <int EPI, bool PT, bool BF16, int WI, int WJ, int BK, int STAGES, int UI = kTile,
          int UJ = kTile>
hipError_t launch(const GemmArgs& a, hipStream_t stream) {
  // operand ring, plus the LoRA rows of one tile (2 x 256 rows x up to 32 bf16)
  // or the tile's s_i values
  constexpr int kLds = STAGES * (UI + UJ) * BK + (EPI == kEpiDequantLoraBf16 ? 2 * kTile * 64 : 0) +
                       (EPI == kEpiDequantBf16 && !PT ? UI * 4 : 0);
  auto kern = gemm_kernel<EPI, PT, BF16, WI, WJ, BK, STAGES, UI, UJ>;
  {
    static std::atomic<uint64_t> configured{0};
    const void* k = (const void*)kern;
    hipError_t e = set_lds_limits_once(&k, &kLds, 1, configured);
    if (e != hipSuccess) return e;
  }
  const int64_t gi = (a.I + UI - 1) / UI, gj = (a.J + UJ - 1) / UJ;
  if (gi <= 0 || gj <= 0) return hipSuccess;
  if (gi * gj > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)(gi * gj)), dim3(64 * WI * WJ), kLds, stream, a);
  return hipGetLastError();
}

constexpr int kWI = CONVROT_GEMM_WI, kWJ = CONVROT_GEMM_WJ;
constexpr int kBK = CONVROT_GEMM_BK, kStages = CONVROT_GEMM_STAGES;

}  // namespace

// Cost model of the dequantizing GEMM's launch forms inside the forward (the
// quantizer has just written q_x, so little of it is in L2), in microseconds
// per 4096 of K, fitted to graph-replayed forwards of out[J, I] at K = 4096
// and 16384, J = 129 .. 4096, I = 4096 .. 16384 on one MI355X, and taken as
// linear in K:
//  * 256 x 256 tiles (8 waves, one workgroup per CU): ~44 us up to 128 tiles,
//    ~51 us towards 192;
//  * 128 x 64 tiles (i x j) with a four-stage ring (4 waves of 64 x 32, 96 KB
//    of LDS, one workgroup per CU) up to 256 tiles: ~12.9 us up to 96 tiles
//    plus ~0.0194 us per further tile (five stages measured slower);
//  * 128 x 128 tiles with a four-stage ring (4 waves, 128 KB of LDS, one
//    workgroup per CU) up to 256 tiles: ~17 us up to 64 tiles plus ~0.0375 us
//    per further tile.  Two stages left the loads exposed when q_x and the
//    weights come from beyond L2 (M = 300: 24.6 against 18.8 us);
//  * 128 x 128 tiles with two stages (64 KB, two workgroups per CU) beyond 256
//    tiles: ~28 us at 256 and ~0.0445 us per further tile up to 512; beyond
//    that a third round of workgroups made it slower than 256 x 256 tiles
//    (M = 2500: ~58 against ~47 us), so it is not used there;
//  * split-K over 256 x 256 tiles: ~13.8 us per workgroup besides its K-slice
//    (prologue and int32 partial stores), 8.1 ns per contraction byte with up
//    to 128 workgroups and 12.5 ns with the whole chip busy, plus the reduce
//    launch reading the partials at ~3.8 TB/s.
// A 256 x 256 tile moves ~1.5x fewer LDS bytes per multiply-add than a
// 128 x 128 one, and that one ~1.5x fewer than 128 x 64 (direct loads plus
// fragment reads), so the larger tile wins once its launch fills the chip;
// before that, smaller tiles put more CUs to work.
namespace {

double est_tiles256(int64_t t, int64_t K) { return (double)K / 4096.0 * (t <= 128 ? 44.0 : 51.0); }
double est_tiles128(int64_t t, int64_t K) {
  if (t > 512) return 1e30;
  const double g = t <= 256 ? 17.0 + (double)(t > 64 ? t - 64 : 0) * 0.0375
                            : 28.0 + (double)(t - 256) * 0.0445;
  return (double)K / 4096.0 * g;
}
double est_tiles64(int64_t t, int64_t K) {
  if (t > 256) return 1e30;
  return (double)K / 4096.0 * (12.9 + (double)(t > 96 ? t - 96 : 0) * 0.0194);
}
double est_splitk(int64_t t256, int S, int64_t M, int64_t N, int64_t K) {
  const int64_t W = t256 * S;
  const double per_byte = W <= 128   ? 0.0081
                          : W >= 256 ? 0.0125
                                     : 0.0081 + (double)(W - 128) * (0.0125 - 0.0081) / 128.0;
  const double waves = (double)((W + 255) / 256);
  return waves * (13.8 + (double)(K / S) * per_byte) + (double)S * M * N * 4.0 / 3.8e6;
}
int64_t tiles_of(int64_t I, int64_t J, int64_t ui, int64_t uj) {
  return ((I + ui - 1) / ui) * ((J + uj - 1) / uj);
}
// The one-pass form the model puts first, and its estimate.
int one_pass_tile(int64_t I, int64_t J, int64_t K, double* est) {
  const int64_t t256 = tiles_of(I, J, 256, 256), t128 = tiles_of(I, J, 128, 128);
  int best = kTile256x256;
  double e = est_tiles256(t256, K);
  if (t256 < 192) {
    const double e128 = est_tiles128(t128, K), e64 = est_tiles64(tiles_of(I, J, 128, 64), K);
    if (e128 < e) {
      best = t128 <= 256 ? kTile128x128Deep : kTile128x128;
      e = e128;
    }
    if (e64 < e) {
      best = kTile128x64;
      e = e64;
    }
  }
  if (est) *est = e;
  return best;
}

}  // namespace

int dequant_tile(int64_t I, int64_t J, int64_t K) { return one_pass_tile(I, J, K, nullptr); }

hipError_t launch_gemm_i8(const GemmArgs& a, int epilogue, bool p_transposed, hipStream_t stream) {
  if (p_transposed) {
    if (epilogue == kEpiI32) return launch<kEpiI32, true, false, 2, 4, 128, 2>(a, stream);
    if (epilogue == kEpiInvRotBf16) return launch<kEpiInvRotBf16, true, false, 2, 4, 128, 2>(a, stream);
    return hipErrorInvalidValue;
  }
  if (epilogue == kEpiI32) return launch<kEpiI32, false, false, kWI, kWJ, kBK, kStages>(a, stream);
  if (epilogue == kEpiDequantBf16) {
    switch (dequant_tile(a.I, a.J, a.Kc)) {
      case kTile128x64: return launch<kEpiDequantBf16, false, false, 2, 2, 128, 4, 128, 64>(a, stream);
      case kTile128x128Deep: return launch<kEpiDequantBf16, false, false, 2, 2, 128, 4, 128, 128>(a, stream);
      case kTile128x128: return launch<kEpiDequantBf16, false, false, 2, 2, 128, 2, 128, 128>(a, stream);
      default: return launch<kEpiDequantBf16, false, false, kWI, kWJ, kBK, kStages>(a, stream);
    }
  }
  if (epilogue == kEpiDequantLoraBf16) {
    if (a.lora_r != 16 && a.lora_r != 32) return hipErrorInvalidValue;
    return launch<kEpiDequantLoraBf16, false, false, kWI, kWJ, kBK, kStages>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_i8_splitk_dequant(const GemmArgs& a, int S, int32_t* partial,
                                         hipStream_t stream) {
  if (S < 1 || a.Kc % (S * kBK) || a.I % 4) return hipErrorInvalidValue;
  constexpr int kLds = kStages * 2 * kTile * kBK;
  auto kern = gemm_splitk_kernel<kWI, kWJ, kBK, kStages>;
  {
    static std::atomic<uint64_t> configured{0};
    const void* k = (const void*)kern;
    hipError_t e = set_lds_limits_once(&k, &kLds, 1, configured);
    if (e != hipSuccess) return e;
  }
  const int64_t gi = (a.I + kTile - 1) / kTile, gj = (a.J + kTile - 1) / kTile;
  const int64_t tiles = gi * gj;
  if (tiles <= 0) return hipSuccess;
  if (tiles * S > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)(tiles * S)), dim3(64 * kWI * kWJ), kLds, stream, a, tiles,
                     a.Kc / S, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_dequant(partial, S, a.J, a.I, a.si, a.sj, a.bias,
                               static_cast<uint16_t*>(a.out), stream);
}

hipError_t launch_splitk_dequant(const int32_t* partial, int S, int64_t J, int64_t I,
                                 const float* si, const float* sj, const uint16_t* bias,
                                 uint16_t* out, hipStream_t stream) {
  if (S < 1 || I % 4) return hipErrorInvalidValue;
  const int64_t quads = J * (I / 4);
  const int64_t blocks = (quads + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(splitk_dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, partial, S,
                     J, I, si, sj, bias, out);
  return hipGetLastError();
}

int splitk_factor(int64_t M, int64_t N, int64_t K) {
  // S (a divisor of K/128, at most 32) where the cost model above puts the
  // split launch below the best one-pass tile; S = 1 keeps the one pass.
  const int64_t t256 = tiles_of(N, M, 256, 256);
  if (t256 >= 128 || N % 4 || small_m_mode(M, N, K)) return 1;
  const int64_t kb = K / kBlock;
  int best = 1;
  double best_t = 0.0;
  one_pass_tile(N, M, K, &best_t);
  for (int S = 2; S <= 32 && S <= kb; ++S) {
    if (kb % S) continue;
    const double t = est_splitk(t256, S, M, N, K);
    if (t < best_t) {
      best = S;
      best_t = t;
    }
  }
  return best;
}

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t stream) {
  return launch<kEpiBf16, false, true, kWI, kWJ, kBK, kStages>(a, stream);
}

}  // namespace convrot
