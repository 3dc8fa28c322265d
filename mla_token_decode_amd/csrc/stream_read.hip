// Cold read-stream probe for gfx950: the HBM read rate a plain streaming
// kernel reaches on this device, the practical ceiling against which the
// decode kernels' KV stream is judged (their roofline is the published 8 TB/s).
// Built as a library of its own (libmla_stream.so); only the benchmark loads
// it.
//
// Every lane reads 16-byte words with non-temporal loads, eight in flight
// per lane; consecutive lanes read consecutive words, so each wave load covers
// 1 KB.  Layout 0 strides over the whole buffer (grid stride); layout 1 gives
// each workgroup one contiguous share.  The words are folded with XOR and
// written only when the fold equals a fixed value, so the loads cannot be
// dropped and the kernel writes (almost surely) nothing.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kInFlight = 8;

template <int LAYOUT>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p, size_t n,
                                                                unsigned* sink) {
  // layout 0: lane i reads words i, i + stride, ...; layout 1: the workgroup's
  // share [lo, hi), lane j reads lo + j, lo + j + 256, ...
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  const size_t lo = LAYOUT == 0 ? 0 : (size_t)blockIdx.x * per;
  const size_t hi = LAYOUT == 0 ? n : (lo + per < n ? lo + per : n);
  const size_t stride = LAYOUT == 0 ? (size_t)gridDim.x * kThreads : (size_t)kThreads;
  size_t i = LAYOUT == 0 ? (size_t)blockIdx.x * kThreads + threadIdx.x : lo + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kInFlight - 1) * stride < hi; i += kInFlight * stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= v[k];
  }
  for (; i < hi; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  const unsigned f = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (f == 0x9e3779b9u) sink[0] = f;
}

}  // namespace

// Read `bytes` (a multiple of 16, > 0) at the 16-byte aligned device address
// `buf` with `blocks` workgroups of 256 threads (1 .. 65536) in `layout` 0
// (grid stride) or 1 (a contiguous share per workgroup) on `stream`; `sink`:
// one writable device word.  Returns 0, or a hipError_t value (the launch's),
// or -1 for arguments outside these rules (nothing launched).
extern "C" int mla_stream_read(const void* buf, size_t bytes, unsigned* sink, int blocks, int layout,
                               void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0 ||
      blocks < 1 || blocks > 65536 || (layout != 0 && layout != 1))
    return -1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* p = static_cast<const u32x4*>(buf);
  if (layout == 0)
    hipLaunchKernelGGL(stream_read_kernel<0>, dim3(blocks), dim3(kThreads), 0, s, p, bytes / 16, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<1>, dim3(blocks), dim3(kThreads), 0, s, p, bytes / 16, sink);
  return static_cast<int>(hipGetLastError());
}
