// Cache write of one new token per sequence: h = x A (Palu author response,
// answer to Q2 on ESPACE: the down-projection output is what is cached).
//
// x [B, d_model] times A [d_model, G*r] is a skinny product whose cost is
// reading A once (4 MiB per matrix at d_model 4096, G*r 512 in bf16). To read A
// once with enough workgroups to fill the chip, the d_model sum is split:
//   pass 1: workgroup (column block, row slice) reads a [64 x 256] block of
//           A_k or A_v (coalesced rows) and the matching x columns for every
//           sequence, and writes fp32 partial sums to the workspace;
//   pass 2: one thread per (sequence, column) adds the row-slice partials in a
//           fixed order, rounds (bf16: nearest, ties to even) and writes row
//           pos[b] of the cache.
// Both passes sum in fp32.
#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;       // d_model rows per slice
constexpr int kRowBatch = 32;   // A loads a thread keeps in flight
constexpr int kBatchChunk = 8;  // sequences accumulated per pass over a slice
constexpr int kMaxBatchLDS = 32;

template <typename T>
__global__ __launch_bounds__(kThreads) void append_partial_kernel(AppendParams p) {
  const int width = p.G * p.r;
  const int col = blockIdx.x * kThreads + threadIdx.x;     // in [0, 2*width)
  const int i0 = blockIdx.y * kRows;
  const int rows = min(kRows, p.dm - i0);
  __shared__ float xs[kMaxBatchLDS][kRows];
  const bool is_v = col >= width;
  const int c = is_v ? col - width : col;
  const T* A = static_cast<const T*>(is_v ? p.a_v : p.a_k);
  const T* x = static_cast<const T*>(p.x);
  for (int b0 = 0; b0 < p.B; b0 += kMaxBatchLDS) {
    const int nb = min(kMaxBatchLDS, p.B - b0);
    __syncthreads();
    for (int e = threadIdx.x; e < nb * kRows; e += kThreads) {
      const int bb = e / kRows, i = e % kRows;
      xs[bb][i] = i < rows ? load_f32(x, static_cast<size_t>(b0 + bb) * p.dm + i0 + i) : 0.f;
    }
    __syncthreads();
    if (col >= 2 * width) continue;
    for (int bc = 0; bc < nb; bc += kBatchChunk) {
      float acc[kBatchChunk];
#pragma unroll
      for (int j = 0; j < kBatchChunk; ++j) acc[j] = 0.f;
      for (int ib = 0; ib < rows; ib += kRowBatch) {
        float a[kRowBatch];
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u)   // all loads first: they overlap in flight
          a[u] = ib + u < rows ? load_f32(A, static_cast<size_t>(i0 + ib + u) * width + c) : 0.f;
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u)
#pragma unroll
          for (int j = 0; j < kBatchChunk; ++j) acc[j] = fmaf(xs[bc + j][ib + u], a[u], acc[j]);
      }
      for (int j = 0; j < kBatchChunk && bc + j < nb; ++j)
        p.part[(static_cast<size_t>(blockIdx.y) * p.B + b0 + bc + j) * 2 * width + col] = acc[j];
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void append_finish_kernel(AppendParams p) {
  const int width = p.G * p.r;
  const int col = blockIdx.x * kThreads + threadIdx.x;
  const int b = blockIdx.y;
  if (col >= 2 * width) return;
  const int pos = p.pos[b];
  if (pos < 0 || pos >= p.L) return;
  const int nks = (p.dm + kRows - 1) / kRows;
  const size_t stride = static_cast<size_t>(p.B) * 2 * width;
  const float* src = p.part + static_cast<size_t>(b) * 2 * width + col;
  float acc = 0.f;
  for (int k0 = 0; k0 < nks; k0 += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = k0 + u < nks ? src[(k0 + u) * stride] : 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) acc += v[u];   // slices added in order
  }
  const bool is_v = col >= width;
  const int c = is_v ? col - width : col;
  const int g = c / p.r, k = c % p.r;
  T* h = static_cast<T*>(is_v ? p.h_v : p.h_k);
  store_elem(h, ((static_cast<size_t>(b) * p.G + g) * p.L + pos) * p.r + k, acc);
}

}  // namespace

size_t append_workspace_bytes(int B, int dm, int G, int r) {
  const size_t nks = (dm + kRows - 1) / kRows;
  return nks * B * 2 * size_t(G) * r * sizeof(float);
}

hipError_t launch_append(const AppendParams& p, int dtype, hipStream_t st) {
  const int cols = 2 * p.G * p.r;
  const dim3 g1((cols + kThreads - 1) / kThreads, (p.dm + kRows - 1) / kRows);
  const dim3 g2((cols + kThreads - 1) / kThreads, p.B);
  if (dtype == 0) {
    append_partial_kernel<float><<<g1, kThreads, 0, st>>>(p);
    append_finish_kernel<float><<<g2, kThreads, 0, st>>>(p);
  } else {
    append_partial_kernel<uint16_t><<<g1, kThreads, 0, st>>>(p);
    append_finish_kernel<uint16_t><<<g2, kThreads, 0, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace palu
