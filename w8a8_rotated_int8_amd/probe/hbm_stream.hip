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
// Built into libhbm_probe.so by build.py; two C entry points.
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

}  // namespace

extern "C" {

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
