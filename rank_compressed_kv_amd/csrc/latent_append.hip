// Cache write of one new token per sequence: h = x A (Palu author response,
// answer to Q2 on ESPACE: the down-projection output is what is cached).
// Each thread owns one latent column of one of the two caches; x is staged in
// LDS in chunks and A is read row by row, coalesced across the threads.
#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 1024;

template <typename T>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendParams p) {
  const int b = blockIdx.y;
  const bool is_v = blockIdx.z == 1;
  const int col = blockIdx.x * kThreads + threadIdx.x;   // in [0, G*r)
  const int pos = p.pos[b];
  if (pos < 0 || pos >= p.L) return;                    // whole block agrees
  const int width = p.G * p.r;
  const T* x = static_cast<const T*>(p.x) + static_cast<size_t>(b) * p.dm;
  const T* A = static_cast<const T*>(is_v ? p.a_v : p.a_k);
  __shared__ float xs[kChunk];
  float acc = 0.f;
  for (int i0 = 0; i0 < p.dm; i0 += kChunk) {
    const int len = min(kChunk, p.dm - i0);
    __syncthreads();
    for (int i = threadIdx.x; i < len; i += kThreads) xs[i] = load_f32(x, i0 + i);
    __syncthreads();
    if (col < width) {
      for (int i = 0; i < len; ++i)
        acc = fmaf(xs[i], load_f32(A, static_cast<size_t>(i0 + i) * width + col), acc);
    }
  }
  if (col >= width) return;
  const int g = col / p.r, k = col % p.r;
  T* h = static_cast<T*>(is_v ? p.h_v : p.h_k);
  store_elem(h, ((static_cast<size_t>(b) * p.G + g) * p.L + pos) * p.r + k, acc);
}

}  // namespace

hipError_t launch_append(const AppendParams& p, int dtype, hipStream_t st) {
  const dim3 grid((p.G * p.r + kThreads - 1) / kThreads, p.B, 2);
  if (dtype == 0) append_kernel<float><<<grid, kThreads, 0, st>>>(p);
  else append_kernel<uint16_t><<<grid, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace palu
