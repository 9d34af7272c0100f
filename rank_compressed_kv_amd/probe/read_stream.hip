// HBM read-stream probe, a measurement aid kept apart from libpalu: it gives
// the read bandwidth a streaming kernel reaches on this GPU, the practical
// ceiling beside the published 8 TB/s for kernels that only read their data
// once (the decode kernels' latents).
//
// Each workgroup reads one contiguous chunk of the buffer with 16-byte
// non-temporal loads, kInflight of them in flight per thread, and folds the
// words into one xor per workgroup (written out, so no load can be dropped).
// Every index is below n16; the last chunk may be short.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int kInflight>
__global__ void read_stream_kernel(const u32x4* __restrict__ src, size_t n16, size_t per_wg,
                                   uint32_t* out) {
  const size_t base = static_cast<size_t>(blockIdx.x) * per_wg;
  if (base >= n16) {
    if (threadIdx.x == 0) out[blockIdx.x] = 0;
    return;
  }
  const size_t end = base + per_wg < n16 ? base + per_wg : n16;
  uint32_t acc = 0;
  for (size_t i = base + threadIdx.x; i < end; i += static_cast<size_t>(blockDim.x) * kInflight) {
    u32x4 v[kInflight];
#pragma unroll
    for (int u = 0; u < kInflight; ++u) {
      size_t j = i + static_cast<size_t>(u) * blockDim.x;
      if (j >= end) j = end - 1;
      v[u] = __builtin_nontemporal_load(src + j);
    }
#pragma unroll
    for (int u = 0; u < kInflight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  acc ^= __shfl_xor(acc, 1);
  if (threadIdx.x == 0) out[blockIdx.x] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16, src 16-byte aligned) once; out needs one
// uint32 per workgroup. grid 1..65536, threads 64..1024 (a multiple of 64),
// inflight 4, 8 or 16. Returns 0, or -1 for arguments out of range (nothing
// is launched), or the HIP launch error.
extern "C" __attribute__((visibility("default"))) int palu_probe_read_stream(
    const void* src, size_t bytes, uint32_t* out, int grid, int threads, int inflight,
    void* stream) {
  if (!src || !out || bytes == 0 || bytes % 16 || grid < 1 || grid > 65536 || threads < 64 ||
      threads > 1024 || threads % 64 || (inflight != 4 && inflight != 8 && inflight != 16))
    return -1;
  const size_t n16 = bytes / 16;
  const size_t per = (n16 + grid - 1) / grid;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4* s = static_cast<const u32x4*>(src);
  if (inflight == 4) read_stream_kernel<4><<<grid, threads, 0, st>>>(s, n16, per, out);
  else if (inflight == 8) read_stream_kernel<8><<<grid, threads, 0, st>>>(s, n16, per, out);
  else read_stream_kernel<16><<<grid, threads, 0, st>>>(s, n16, per, out);
  return static_cast<int>(hipGetLastError());
}
