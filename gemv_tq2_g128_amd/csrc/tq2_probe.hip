// Reference kernels for the benchmark (libtq2_probe.so, not part of libtq2):
// a plain streaming read of a buffer and an empty kernel, launched with a
// caller-chosen grid of 256-thread blocks.  With the decode GEMV's grid and
// byte count they give the time one launch of that shape costs, and how fast
// such a launch can stream the same bytes, beside the GEMV's own time.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kProbeThreads = 256;

// Grid-stride read of n16 16-byte words, four independent (guarded) loads in
// flight per thread per step, with the non-temporal hint (the fastest plain
// read of a stream touched once, as the decode GEMV's weight loads are).  The words are folded into one value per
// thread, stored only if it equals a constant the data never has to match,
// so the loads cannot be dropped and almost nothing is written.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4* __restrict__ p,
                                                                    size_t n16,
                                                                    uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const size_t stride = size_t(gridDim.x) * kProbeThreads;
  for (size_t i = size_t(blockIdx.x) * kProbeThreads + threadIdx.x; i < n16; i += 4 * stride) {
    typedef unsigned int ntv4 __attribute__((ext_vector_type(4)));
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t idx = i + size_t(j) * stride;
      if (idx < n16) {
        const ntv4 t = __builtin_nontemporal_load(reinterpret_cast<const ntv4*>(p) + idx);
        v[j] = make_uint4(t[0], t[1], t[2], t[3]);
      } else {
        v[j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (acc == 0x9E3779B9u) out[blockIdx.x] = acc;
}

__global__ __launch_bounds__(kProbeThreads) void probe_empty_kernel() {}

}  // namespace

extern "C" {

// Streams `bytes` (a multiple of 16) from the device buffer `buf` with `blocks`
// blocks of 256 threads; `out` is a device buffer of `blocks` uint32 that is
// written only for one improbable folded value.  Returns 0, or -1 on a bad
// argument, -6 on a launch error.
int tq2_probe_read(const void* buf, size_t bytes, void* out, int blocks, void* stream) {
  if (!buf || !out || blocks <= 0 || bytes % 16) return -1;
  hipLaunchKernelGGL(probe_read_kernel, dim3(blocks), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), bytes / 16,
                     static_cast<uint32_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// An empty kernel of `blocks` blocks of 256 threads.
int tq2_probe_empty(int blocks, void* stream) {
  if (blocks <= 0) return -1;
  hipLaunchKernelGGL(probe_empty_kernel, dim3(blocks), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
