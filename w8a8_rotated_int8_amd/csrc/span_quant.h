// Span quantizer: the device-side rotate (or scale-fold) + per-row int8
// quantization of a span of up to SB (16 or 32) consecutive 128-blocks held in
// LDS, used by the row quantizer kernels.
//
// Arithmetic:
//   rotate:   per 128-block, S_j = sum_i H[i][j] x_i computed by a fast
//             Walsh-Hadamard transform in binary64; r_j = fl32(fl64(S_j * c)),
//             c = 1/sqrt(128).  Every partial sum of bf16 inputs is exact, and
//             the butterfly order cannot change the result, as long as a block's
//             magnitude spread (largest over smallest nonzero |x_i|) stays under
//             about 2^38.  Past that, binary64 rounds some partial sums and the
//             result may depend on the order of the additions (GELU outputs near
//             -inf reach such spreads; a host emulation of this butterfly order
//             checks those rows against the index-order sum).
//   fold:     (dY quantizer) r_n = fl32(fl32(dY_n) * s_w[n]); no rotation.
//   quantize: a = max|r|, s = fl32(a/127), code = clamp(RNE(fl32(r/s)), +-127);
//             s = 0 (all-zero row, or a/127 underflowed) -> codes 0; a row with
//             a NaN or infinite r (non-finite input, or fl32 overflow of the
//             rotation) -> s = NaN (canonical quiet NaN) and codes 0.
//
// Work layout.  A wave owns a span of SB blocks: several short rows packed
// together, or an SB-block slice of a longer row (then the workgroup's waves
// share the row and combine their maxima through LDS).  The span is copied to
// LDS with direct 16-byte global->LDS loads (coalesced, XOR-swizzled so the
// transposed reads are bank-conflict free) and processed in passes of 16
// blocks: in pass k lane 16 g + p holds elements 32 g .. 32 g + 31 of block
// 16 k + p.  Five butterfly stages run inside the lane, the sixth pairs lane L
// with L + 16 (v_permlane16_swap) and the seventh with L + 32
// (v_permlane32_swap).  A 16-block span keeps 32 values per lane and fits in
// ~100 VGPRs (four waves per SIMD); a 32-block span keeps 64 (~150 VGPRs).
// Fold mode comes here only for packed short rows, with the column scales
// staged in LDS beside the span; rows of a span or longer are folded by a
// kernel of their own that needs no transposed layout.
#pragma once

#include "common.h"
#include "kernels.h"

namespace convrot {
namespace {

constexpr int kSpanBlocks = 32;                  // largest span (blocks per wave)
constexpr int kSpanBytes = kSpanBlocks * 256;    // bf16 bytes of the largest span

// bf16 bytes of a span of SB blocks.
template <int SB>
constexpr int span_bytes() { return SB * 256; }

enum Mode { kRotate = 0, kFold = 1 };

constexpr float kInv127 = 0x1.020408p-7f;  // RN(1/127)

// LDS position (in 16-byte units) of chunk c (0..15) of block b.
__device__ __forceinline__ int lds_chunk(int b, int c) { return (b << 4) | (c ^ (b & 7)); }

// Exchange with the neighbouring 16-lane row: rows 1 and 3 of vdst swap with
// rows 0 and 2 of src0 (v_permlane16_swap).
__device__ __forceinline__ void swap_rows16(double& vdst, double& src0) {
  uint64_t a = __builtin_bit_cast(uint64_t, vdst), b = __builtin_bit_cast(uint64_t, src0);
  auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)a, (uint32_t)b, false, false);
  auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(a >> 32), (uint32_t)(b >> 32), false, false);
  vdst = __builtin_bit_cast(double, ((uint64_t)hi[0] << 32) | lo[0]);
  src0 = __builtin_bit_cast(double, ((uint64_t)hi[1] << 32) | lo[1]);
}

// Quantize one staged span: per pass read the lane's 32 values from LDS and
// rotate them (or fold the column scale); then reduce the row maxima,
// quantize, stage the codes in LDS and store them.
//
// Rotation data flow: the in-lane stages cover element bits 0-4 (register
// index e).  Each cross-lane swap pairs v[e] with v[e + 16] and exchanges
// register bit 4 with a lane bit, so that the butterfly partners meet in one
// lane.  After both, lane quarter q = L >> 4 holds outputs 16 q + e in v[e]
// and 64 + 16 q + e in v[e + 16] (e < 16).
//
// A row shared by several waves (waves_per_row > 1) is held by waves
// row_wave0 .. row_wave0 + waves_per_row - 1 of the workgroup; they exchange
// their maxima through row_part_max[0 .. waves_per_row - 1] (the row's own
// slots) at one workgroup barrier, which every wave of the workgroup must
// reach, and wave row_wave0 writes the row's scale.
template <int MODE, int SB = kSpanBlocks, bool STREAM = false>
__device__ __forceinline__ void quantize_span(const uint8_t* my_lds, int span_blocks, int nb,
                                              int64_t span_elem0, int64_t row0,
                                              int waves_per_row, int8_t* __restrict__ q,
                                              float* __restrict__ scale,
                                              float* seg_max_wave, float* row_part_max,
                                              const uint8_t* cs_lds = nullptr,
                                              int row_wave0 = 0) {
#pragma clang fp contract(off)
  static_assert(SB == 16 || SB == 32, "a span is one or two passes of 16 blocks");
  constexpr int NP = SB / 16;  // passes
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int p = lane & 15;   // block within the pass
  const int g = lane >> 4;   // which quarter of the block

  float r[NP][32];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    // keep the two passes apart: interleaving them would hold both passes'
    // binary64 working sets at once
    __builtin_amdgcn_sched_barrier(0);
    const int b = 16 * k + p;
    const bool active = b < span_blocks;
    if constexpr (NP > 1) {
      if (k == 1 && span_blocks <= 16) {  // wave-uniform: the span fits in one pass
#pragma unroll
        for (int e = 0; e < 32; ++e) r[NP - 1][e] = 0.f;
        continue;
      }
    }
    uint4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      raw[i] = *reinterpret_cast<const uint4*>(my_lds + 16 * lds_chunk(b, 4 * g + i));
    if (MODE == kRotate) {
      double v[32];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = (double)bf16lo_to_f32(w[j]);
          v[8 * i + 2 * j + 1] = (double)bf16hi_to_f32(w[j]);
        }
      }
      if (!active) {
#pragma unroll
        for (int e = 0; e < 32; ++e) v[e] = 0.0;
      }
#pragma unroll
      for (int bit = 1; bit < 32; bit <<= 1) {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          if (e & bit) continue;
          double a = v[e], c = v[e | bit];
          v[e] = a + c;
          v[e | bit] = a - c;
        }
        __builtin_amdgcn_sched_barrier(0);  // one stage at a time (register pressure)
      }
      // element bit 5: lane L with L + 16
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        swap_rows16(v[e], v[e + 16]);
        double a = v[e], c = v[e + 16];
        v[e] = a + c;
        v[e + 16] = a - c;
      }
      // element bit 6: lane L with L + 32
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        swap_halves(v[e], v[e + 16]);
        double a = v[e], c = v[e + 16];
        v[e] = a + c;
        v[e + 16] = a - c;
      }
#pragma unroll
      for (int e = 0; e < 32; ++e) r[k][e] = (float)(v[e] * kInvSqrt128);
    } else {
      // fold the per-column scale: element 32 g + e of block b.  The span's
      // scales were staged at cs_lds by stage_colscale (chunk c of block b at
      // b * 32 + (c ^ (b & 15))).
      auto scale4 = [&](int i2) {  // floats 32 g + 4 i2 .. + 3 of block b
        return *reinterpret_cast<const float4*>(cs_lds + b * 512 + 16 * ((8 * g + i2) ^ (b & 15)));
      };
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
        float4 s0 = scale4(2 * i);
        float4 s1 = scale4(2 * i + 1);
        float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          r[k][8 * i + 2 * j] = bf16lo_to_f32(w[j]) * sc[2 * j];
          r[k][8 * i + 2 * j + 1] = bf16hi_to_f32(w[j]) * sc[2 * j + 1];
        }
      }
      if (!active) {
#pragma unroll
        for (int e = 0; e < 32; ++e) r[k][e] = 0.f;
      }
    }
  }

  // ---- row absmax ------------------------------------------------------------
  float m[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    m[k] = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) m[k] = max_nan(m[k], fabsf(r[k][e]));
    m[k] = max_xor32(max_xor16(m[k]));  // the four quarters of the block
  }
  float mall = m[0];
#pragma unroll
  for (int k = 1; k < NP; ++k) mall = max_nan(mall, m[k]);
  if (waves_per_row == 1) {
    if (nb == SB) {
      const float mm = group_max(mall, 16);
#pragma unroll
      for (int k = 0; k < NP; ++k) m[k] = mm;
    } else if ((nb & (nb - 1)) == 0) {
#pragma unroll
      for (int k = 0; k < NP; ++k) m[k] = group_max(m[k], nb);  // aligned segments of nb blocks
    } else {
      if (g == 0) {
#pragma unroll
        for (int k = 0; k < NP; ++k) seg_max_wave[16 * k + p] = m[k];
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        const int first = ((16 * k + p) / nb) * nb;
        float mm = 0.f;
        for (int j = 0; j < nb; ++j) {
          const int idx = first + j;
          if (idx < SB) mm = max_nan(mm, seg_max_wave[idx]);
        }
        m[k] = mm;
      }
    }
  } else {
    const float mw = group_max(mall, 16);
    if (lane == 0) row_part_max[wave - row_wave0] = mw;
    __syncthreads();
    float mm = 0.f;
    for (int w = 0; w < waves_per_row; ++w) mm = max_nan(mm, row_part_max[w]);
#pragma unroll
    for (int k = 0; k < NP; ++k) m[k] = mm;
  }

  // ---- quantize + stage + store -------------------------------------------------
  // Codes are staged in LDS (the span's own input buffer, already read) and
  // stored as whole 1 KB runs: lane i of step j writes 16-byte chunk 64 j + i.
  // Chunk c of block c/8 sits at c ^ (c/8 & 7) (conflict-free writes).
  uint8_t* stg = const_cast<uint8_t*>(my_lds);
  auto phys = [](int c) { return c ^ ((c >> 3) & 7); };
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int b = 16 * k + p;
    // s = fl32(m / 127) and the quotients fl32(r / s), both correctly rounded.
    // When every lane's row max is in [2^-64, 2^100] (wave-uniform branch) both
    // use the 3-operation form with the correctly rounded reciprocal (for the
    // divisor 127 checked exhaustively over all significands); otherwise the
    // IEEE division per lane.
    const bool fast = m[k] >= 0x1p-64f && m[k] <= 0x1p100f;
    float s, t[32];
    if (__builtin_amdgcn_ballot_w64(!fast) == 0) {
      s = quot_rn(m[k], 127.0f, kInv127);
      const float inv = 1.0f / s;                      // RN(1/s)
#pragma unroll
      for (int e = 0; e < 32; ++e) t[e] = quot_rn(r[k][e], s, inv);
    } else {
      // IEEE binary32 division; a non-finite maximum (a NaN or infinite
      // rotated value in the row) gives the NaN scale, whose codes are 0
      s = m[k] <= 0x1.fffffep127f ? m[k] / 127.0f : __uint_as_float(kScaleNaNBits);
      const float inv = s > 0.f ? 1.0f / s : 0.f;
      // A subnormal s carries a relative rounding error that can push |t| past
      // 127.5 (e.g. a = 2^-140: s = 2^-147, t = 128), so the codes are clamped
      // to [-127, 127] here; a zero s (a/127 underflowed) gives codes 0.
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float te = fast ? quot_rn(r[k][e], s, inv) : (s > 0.f ? r[k][e] / s : 0.f);
        t[e] = fminf(fmaxf(te, -127.0f), 127.0f);
      }
    }
    uint32_t packed[8];
#pragma unroll
    for (int gg = 0; gg < 8; ++gg) {
      packed[gg] = pack_low_bytes(rne_low_byte_bits(t[4 * gg]), rne_low_byte_bits(t[4 * gg + 1]),
                                  rne_low_byte_bits(t[4 * gg + 2]), rne_low_byte_bits(t[4 * gg + 3]));
    }
    if (b < span_blocks) {
      const int c_lo = 8 * b + (MODE == kRotate ? g : 2 * g);
      const int c_hi = 8 * b + (MODE == kRotate ? 4 + g : 2 * g + 1);
      *reinterpret_cast<uint4*>(stg + 16 * phys(c_lo)) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      *reinterpret_cast<uint4*>(stg + 16 * phys(c_hi)) = make_uint4(packed[4], packed[5], packed[6], packed[7]);
      if (waves_per_row == 1 && g == 0 && b % nb == 0) scale[row0 + b / nb] = s;
    }
    if (k == 0 && waves_per_row > 1 && wave == row_wave0 && lane == 0) scale[row0] = s;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): staging writes landed
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
  const int nchunks = span_blocks * 8;
  int8_t* dst = q + span_elem0;
#pragma unroll
  for (int j = 0; j < SB / 8; ++j) {
    const int c = 64 * j + lane;
    if (c < nchunks) {
      const uint4 v = *reinterpret_cast<const uint4*>(stg + 16 * phys(c));
      // codes of a weight are not read again soon; activation and gradient
      // codes are, by the GEMM that follows
      if constexpr (STREAM) store16_nt(dst + 16 * c, v);
      else *reinterpret_cast<uint4*>(dst + 16 * c) = v;
    }
  }
}

// Issue the SB/4 direct-to-LDS loads of a span of span_blocks (1..SB) blocks.
// Slots past the span reload its last chunk so every lane always issues the
// same number of loads (the vmcnt bookkeeping relies on it).
// STREAM: the rows are read once (load-time weight quantization): loads with
// the non-temporal cache policy.
template <int SB = kSpanBlocks, bool STREAM = false>
__device__ __forceinline__ void stage_span(const uint16_t* __restrict__ x, int64_t span_elem0,
                                           int span_blocks, uint8_t* my_lds) {
  const int lane = threadIdx.x & 63;
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_u32(my_lds));
#pragma unroll
  for (int i = 0; i < SB / 4; ++i) {
    const int slot = i * 64 + lane;
    int b = slot >> 4;
    int c = (slot & 15) ^ (b & 7);
    if (b >= span_blocks) { b = span_blocks - 1; c = 15; }
    if constexpr (STREAM) dma16_nt(x + span_elem0 + (int64_t)b * kBlock + c * 8, base + i * 1024);
    else dma16(x + span_elem0 + (int64_t)b * kBlock + c * 8, base + i * 1024);
  }
}

// Fold mode, short rows packed into a span (block b of the span is block
// b % nb of its row): copy the per-column scales of the span's blocks (128
// floats, 32 chunks of 16 bytes per block) to LDS with coalesced direct loads, SB / 2 per
// lane.  Chunk c of span block b lands at b * 32 + (c ^ (b & 15)): the fold
// pass reads chunk 8 g + i of block p in lanes 16 g + p, and the XOR spreads
// those 16 lanes over 16 different bank groups.  Blocks past the span reload
// a chunk of its last block (never read).
template <int SB>
__device__ __forceinline__ void stage_colscale(const float* __restrict__ colscale, int span_blocks,
                                               int nb, uint8_t* cs_lds) {
  const int lane = threadIdx.x & 63;
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_u32(cs_lds));
#pragma unroll
  for (int i = 0; i < SB / 2; ++i) {
    const int slot = i * 64 + lane;
    int b = slot >> 5;
    int c = (slot & 31) ^ (b & 15);
    if (b >= span_blocks) { b = span_blocks - 1; c = 0; }
    dma16(colscale + (int64_t)(b % nb) * kBlock + 4 * c, base + i * 1024);
  }
}

}  // namespace
}  // namespace convrot

