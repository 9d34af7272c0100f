// Cache write of one new token per sequence: h = x A (Palu author response,
// answer to Q2 on ESPACE: the down-projection output is what is cached).
//
// x [B, d_model] times A [d_model, G*r] is a skinny product whose cost is
// reading A once (4 MiB per matrix at d_model 4096, G*r 512 in bf16). To read A
// once with the whole chip and every load of a thread in flight together, the
// d_model sum is split:
//   pass 1: workgroup (128-column block of [A_k | A_v], 128-row slice): thread
//           (8-column chunk, row group) issues its eight 16-byte loads at once,
//           accumulates x[b, row] * A[row, col] for every sequence, and the
//           row groups are added (lane shuffles, then LDS) into one fp32
//           partial per (slice, sequence, column) in the workspace;
//   pass 2: one thread per (sequence, column) adds the slice partials in a
//           fixed order, rounds (bf16: nearest, ties to even) and writes row
//           pos[b] of the cache.
// Both passes sum in fp32.
#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 128;          // d_model rows per slice
constexpr int kCols = 128;          // columns per block (16 chunks of 8)
constexpr int kRowGroups = 16;      // threads per column chunk; 8 rows each
constexpr int kBatchChunk = 8;      // sequences accumulated per pass

template <typename T>
__global__ __launch_bounds__(kThreads) void append_partial_kernel(AppendParams p) {
  const int width = p.G * p.r;                 // columns of one matrix
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cc = tid % 16, rg = tid / 16;      // 8-column chunk, row group
  const int col0 = blockIdx.x * kCols + 8 * cc;  // in [0, 2*width)
  const int i0 = blockIdx.y * kRows;
  const int rows = min(kRows, p.dm - i0);
  const bool active = col0 < 2 * width;
  const bool is_v = col0 >= width;
  const int c = is_v ? col0 - width : col0;
  const T* A = static_cast<const T*>(is_v ? p.a_v : p.a_k);
  const T* x = static_cast<const T*>(p.x);

  // all of this thread's A rows (rg + 16 i) first, 16 bytes each
  float a[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = rg + kRowGroups * i;
    if (active && row < rows) load8_f32(A + static_cast<size_t>(i0 + row) * width + c, a[i]);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) a[i][e] = 0.f;
  }
  __shared__ float xs[kBatchChunk][kRows];
  __shared__ float red[kThreads / 64][kBatchChunk][kCols];
  for (int b0 = 0; b0 < p.B; b0 += kBatchChunk) {
    const int nb = min(kBatchChunk, p.B - b0);
    __syncthreads();
    for (int e = tid; e < kBatchChunk * kRows; e += kThreads) {
      const int bb = e / kRows, i = e % kRows;
      xs[bb][i] = bb < nb && i < rows ? load_f32(x, static_cast<size_t>(b0 + bb) * p.dm + i0 + i) : 0.f;
    }
    __syncthreads();
    float acc[kBatchChunk][8];
#pragma unroll
    for (int bb = 0; bb < kBatchChunk; ++bb) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[bb][e] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xv = xs[bb][rg + kRowGroups * i];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[bb][e] = fmaf(xv, a[i][e], acc[bb][e]);
      }
    }
    // add the four row groups of this wave (lanes cc, cc+16, cc+32, cc+48),
    // then the four waves through LDS
#pragma unroll
    for (int bb = 0; bb < kBatchChunk; ++bb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[bb][e];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc[bb][e] = v;
      }
    if (lane < 16) {
#pragma unroll
      for (int bb = 0; bb < kBatchChunk; ++bb)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wave][bb][8 * cc + e] = acc[bb][e];
    }
    __syncthreads();
    for (int e = tid; e < nb * kCols; e += kThreads) {
      const int bb = e / kCols, cl = e % kCols;
      const int col = blockIdx.x * kCols + cl;
      if (col < 2 * width) {
        const float v = (red[0][bb][cl] + red[1][bb][cl]) + (red[2][bb][cl] + red[3][bb][cl]);
        p.part[(static_cast<size_t>(blockIdx.y) * p.B + b0 + bb) * 2 * width + col] = v;
      }
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
  for (int k0 = 0; k0 < nks; k0 += 32) {
    float v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) v[u] = k0 + u < nks ? src[(k0 + u) * stride] : 0.f;
#pragma unroll
    for (int u = 0; u < 32; ++u) acc += v[u];   // slices added in order
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

bool append_shape_supported(int G, int r) { return (G * r) % 8 == 0; }

hipError_t launch_append(const AppendParams& p, int dtype, hipStream_t st) {
  const int cols = 2 * p.G * p.r;
  const dim3 g1((cols + kCols - 1) / kCols, (p.dm + kRows - 1) / kRows);
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
