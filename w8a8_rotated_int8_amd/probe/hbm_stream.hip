// Streaming reference for the HBM-bound kernels' rooflines (not part of the
// layer): the rate a plain grid-stride kernel reaches on this GPU for a given
// mix of reads and writes, with the same 16-byte non-temporal loads and stores
// the layer's quantizer and lookup use.  bench.py reports it beside the 8 TB/s
// datasheet peak: writes stream markedly slower than reads on this chip, so the
// practical ceiling of a kernel depends on its read/write mix.
//
// A second probe measures the LDS read rate of one CU, in bytes per shader
// clock, for a given number of waves each streaming 16-byte reads (the GEMM's
// fragment reads), timed with the shader cycle counter inside the kernel.
//
// A third measures the matrix cores' sustained rate: back-to-back independent
// MFMAs (the GEMMs' int8 32x32x32 and bf16 32x32x16 forms) on register
// operands, no memory traffic, with the shader clock they ran at.  Under a long
// dense load the chip lowers its clock to stay within its power limit, so this
// is the practical matrix peak the GEMMs can be held against, beside the
// datasheet figure at 2.4 GHz.
//
// Built into libhbm_probe.so by build.py; three C entry points.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int hbm_v4u __attribute__((ext_vector_type(4)));

namespace {

// mix 0: read in[0, n) only (n = in_chunks);  1: write out[0, n) and read
// in[i / 2] for even i (1 read : 2 writes, the lookup's mix);  2: copy (1 : 1);
// 3: write out[i] from in[i] and in[n + i] (2 reads : 1 write, the quantizer's
// mix).  n = out_chunks for mixes 1-3.  Chunks are 16 bytes.
__global__ __launch_bounds__(256) void hbm_stream_kernel(const hbm_v4u* __restrict__ in,
                                                         hbm_v4u* __restrict__ out, int64_t n,
                                                         int mix) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (mix == 0) {
    hbm_v4u acc = {0u, 0u, 0u, 0u};
    for (int64_t i = i0; i < n; i += stride) acc ^= __builtin_nontemporal_load(in + i);
    // never true for the probe's data (all bytes equal): keeps the loads alive
    if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) out[0] = acc;
    return;
  }
  for (int64_t i = i0; i < n; i += stride) {
    hbm_v4u v = {(unsigned)i, 1u, 2u, 3u};
    if (mix == 1) {
      if ((i & 1) == 0) v ^= __builtin_nontemporal_load(in + (i >> 1));
    } else if (mix == 2) {
      v ^= __builtin_nontemporal_load(in + i);
    } else {
      v ^= __builtin_nontemporal_load(in + i);
      v ^= __builtin_nontemporal_load(in + n + i);
    }
    __builtin_nontemporal_store(v, out + i);
  }
}

// Each of blockDim.x / 64 waves reads 16-byte pieces of a 64 KB LDS buffer,
// eight independent reads per step over distinct 8 KB quarters, conflict-free
// (lane l at +16 l).  Thread 0 records the cycles between two barriers that
// bracket the reads.  The sink store never happens for the probe's data (the
// xor of the reads cannot reach the constant) and keeps the reads alive.
__global__ __launch_bounds__(1024) void lds_read_kernel(int steps, hbm_v4u* __restrict__ sink,
                                                        unsigned long long* __restrict__ cycles) {
  __shared__ __align__(16) hbm_v4u buf[4096];
  for (int i = threadIdx.x; i < 4096; i += blockDim.x) buf[i] = hbm_v4u{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  hbm_v4u acc = {0u, 0u, 0u, 0u};
  unsigned idx = (unsigned)(wave * 64 + lane) & 4095u;
  __syncthreads();
  const unsigned long long t0 = __builtin_readcyclecounter();
  for (int it = 0; it < steps; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= buf[(idx + 512u * u) & 4095u];
    idx = (idx + 192u) & 4095u;
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_readcyclecounter();
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
  if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
}

typedef int mfma_v4i __attribute__((ext_vector_type(4)));
typedef int mfma_v16i __attribute__((ext_vector_type(16)));
typedef float mfma_v16f __attribute__((ext_vector_type(16)));
typedef __bf16 mfma_v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t xorshift32(uint32_t x) {
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  return x;
}

// Each wave issues 8 * steps MFMAs into two independent accumulators, taking
// its operands from four A and four B register sets in turn, so that the
// multiplier inputs change from one instruction to the next as in a GEMM.  The
// operands decide the power the matrix cores draw, and with it the clock the
// chip holds:
//   kind 0  int8, uniformly random bytes (every bit toggles at random);
//   kind 1  int8, code-like bytes: the sum of four uniform 6-bit values less
//           126 (range +-126, sigma ~37, about the spread of per-row int8 codes
//           of rotated Gaussian rows);
//   kind 2  int8, zero operands (no switching: the clock stays at its maximum);
//   kind 3  bf16 32x32x16, random signs and mantissas in +-[1, 2).
// Thread 0 records the shader-clock cycles and the 100 MHz real-time ticks
// between two barriers around the loop.  The sink store needs the xor of all
// accumulators to hit a constant (it keeps the MFMAs alive; the sink is sized
// for it).
__device__ __forceinline__ int probe_operand(int kind, uint32_t& x) {
  x = xorshift32(x);
  if (kind == 0) return (int)x;
  if (kind == 2) return 0;
  if (kind == 3) return (int)((x & 0x807f807fu) | 0x3f803f80u);
  uint32_t w = 0;
#pragma unroll
  for (int byte = 0; byte < 4; ++byte) {
    x = xorshift32(x);
    const int v = (int)(x & 63) + (int)((x >> 8) & 63) + (int)((x >> 16) & 63) + (int)((x >> 24) & 63) - 126;
    w |= (uint32_t)(v & 0xff) << (8 * byte);
  }
  return (int)w;
}

template <int KIND>
__global__ __launch_bounds__(512) void mfma_probe_kernel(int steps, mfma_v16i* __restrict__ sink,
                                                         unsigned long long* __restrict__ stamps) {
  constexpr bool kBf16 = KIND == 3;
  uint32_t x = 0x9e3779b9u ^ ((uint32_t)(blockIdx.x * blockDim.x + threadIdx.x) * 0x85ebca6bu);
  mfma_v4i a[4], b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      a[k][c] = probe_operand(KIND, x);
      b[k][c] = probe_operand(KIND, x);
    }
  mfma_v16i acc_i[2];
  mfma_v16f acc_f[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    acc_i[k] = mfma_v16i{};
    acc_f[k] = mfma_v16f{};
  }
  __syncthreads();
  const unsigned long long c0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < steps; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = u & 1, ka = u & 3, kb = (u + (u >> 2)) & 3;
      if constexpr (kBf16)
        acc_f[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(mfma_v8bf, a[ka]),
                                                           __builtin_bit_cast(mfma_v8bf, b[kb]),
                                                           acc_f[k], 0, 0, 0);
      else
        acc_i[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ka], b[kb], acc_i[k], 0, 0, 0);
    }
  }
  __syncthreads();
  const unsigned long long c1 = __builtin_readcyclecounter();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  int h = 0;
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) h ^= kBf16 ? __float_as_int(acc_f[k][e]) : acc_i[k][e];
  if (h == 0x2545f491) sink[blockIdx.x * blockDim.x + threadIdx.x] = acc_i[0];
  if (threadIdx.x == 0) {
    stamps[2 * blockIdx.x] = c1 - c0;
    stamps[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// Matrix-core probe: `blocks` workgroups of `threads` threads (a multiple of
// 64, at most 512), each wave issuing 8 * steps MFMAs of the given kind (0-2:
// int8 32x32x32, 65536 ops each, with random, code-like or zero operands; 3:
// bf16 32x32x16, 32768 flops each).  `sink` holds blocks * threads * 64 bytes
// (written only if an accumulator hash hits a constant), `stamps` 2 * blocks
// 64-bit values: per workgroup the shader cycles and the 100 MHz real-time
// ticks of its loop.  Returns 0, or -1 on bad arguments / a failed launch.
int mfma_probe_run(int kind, int threads, int steps, int blocks, void* sink, void* stamps,
                   hipStream_t stream) {
  if (kind < 0 || kind > 3 || threads <= 0 || threads > 512 || threads % 64 || steps <= 0 ||
      blocks <= 0 || !sink || !stamps)
    return -1;
  if (((uintptr_t)sink & 15) || ((uintptr_t)stamps & 7)) return -1;
  mfma_v16i* sk = static_cast<mfma_v16i*>(sink);
  unsigned long long* st = static_cast<unsigned long long*>(stamps);
  const dim3 grid((unsigned)blocks), block((unsigned)threads);
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_probe_kernel<0>, grid, block, 0, stream, steps, sk, st); break;
    case 1: hipLaunchKernelGGL(mfma_probe_kernel<1>, grid, block, 0, stream, steps, sk, st); break;
    case 2: hipLaunchKernelGGL(mfma_probe_kernel<2>, grid, block, 0, stream, steps, sk, st); break;
    default: hipLaunchKernelGGL(mfma_probe_kernel<3>, grid, block, 0, stream, steps, sk, st); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// LDS read probe: `blocks` workgroups of `threads` threads (a multiple of 64,
// at most 1024), each wave issuing 8 * steps 16-byte reads per lane.  `sink`
// holds blocks * threads * 16 bytes (never written in practice), `cycles`
// blocks 64-bit counts.  Returns 0, or -1 on bad arguments / a failed launch.
int lds_probe_read(int threads, int steps, int blocks, void* sink, void* cycles,
                   hipStream_t stream) {
  if (threads <= 0 || threads > 1024 || threads % 64 || steps <= 0 || blocks <= 0 || !sink || !cycles)
    return -1;
  if (((uintptr_t)sink & 15) || ((uintptr_t)cycles & 7)) return -1;
  hipLaunchKernelGGL(lds_read_kernel, dim3((unsigned)blocks), dim3((unsigned)threads), 0, stream, steps,
                     static_cast<hbm_v4u*>(sink), static_cast<unsigned long long*>(cycles));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}


// Stream `bytes` of output (mix 0: of input) in the given mix.  `in` must hold
// at least: mix 0 bytes; mix 1 bytes / 2; mix 2 bytes; mix 3 2 * bytes.  `out`
// holds `bytes` (mix 0: 16).  bytes % 16 == 0, 16-byte aligned buffers.
// Returns 0, or -1 on bad arguments / a failed launch.
int hbm_probe_stream(const void* in, void* out, int64_t bytes, int mix, int grid,
                     hipStream_t stream) {
  if (!in || !out || bytes <= 0 || bytes % 16 || mix < 0 || mix > 3 || grid <= 0) return -1;
  if (((uintptr_t)in & 15) || ((uintptr_t)out & 15)) return -1;
  hipLaunchKernelGGL(hbm_stream_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     static_cast<const hbm_v4u*>(in), static_cast<hbm_v4u*>(out), bytes / 16, mix);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
