// Streaming reference for the HBM-bound kernels' rooflines (not part of the
// layer): the rate a plain grid-stride kernel reaches on this GPU for a given
// mix of reads and writes, with the same 16-byte non-temporal loads and stores
// the layer's quantizer and lookup use.  bench.py reports it beside the 8 TB/s
// datasheet peak: writes stream markedly slower than reads on this chip, so the
// practical ceiling of a kernel depends on its read/write mix.
//
// Built into libhbm_probe.so by build.py; one C entry point.
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

}  // namespace

extern "C" {

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
