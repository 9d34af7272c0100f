// Cache write of one new token per sequence, h = x A (Palu author response,
// answer to Q2 on ESPACE: the down-projection output is what is cached), from
// a projection stored transposed: A^T [G*r, d_model], each latent's d_model
// weights contiguous (the layout of a torch.nn.Linear weight).
//
// In that layout a latent column is one contiguous run, so a workgroup can
// own whole columns and finish them itself: one pass, with no partial sums in
// the workspace and no hand-off between workgroups (the [d_model, G*r] form
// has to split d_model over workgroups to read its rows coalesced).
//   workgroup: 4 consecutive columns of [A_k | A_v] (never straddling the two:
//              G*r is a multiple of 8), all of d_model, 8 sequences a pass;
//   thread t:  the 8-element chunks t, t + 256, ... of d_model; each chunk
//              is one 16-byte load per column and per sequence (x), issued
//              two chunks at a time with no branch around them, and 4 x 8
//              fp32 running sums (fmaf, chunk order);
//   reduction: the 256 threads' sums go through LDS; thread (output o, part
//              p) adds threads 32 p .. 32 p + 31 in order, then the eight
//              parts are added by lane exchanges (xor 1, 2, 4): a fixed
//              order, so the result does not depend on timing.
// The cache row pos[b] gets the sum rounded to the cache dtype (bf16: nearest,
// ties to even); rows with pos outside [0, L) are skipped.
//
// The launch can carry the next decode call's query absorption as extra
// workgroups past the append's, as the [d_model, G*r] form's launch does.
#include "absorb_device.h"
#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

constexpr int kThreads = 256;
constexpr int kCols = 4;       // output columns per workgroup
constexpr int kSeq = 8;        // sequences per pass
constexpr int kSlab = 2;       // chunks per thread loaded together
constexpr int kOut = kCols * kSeq;

template <typename T, bool kFuse>
__global__ __launch_bounds__(kThreads) void append_t_kernel(AppendParams p) {
  __shared__ float red[kThreads][kOut + 1];
  const int width = p.G * p.r;
  const int nblk = 2 * width / kCols;
  if constexpr (kFuse) {
    static_assert(sizeof(red) >= kAbsHeadChunk * 2 * kMaxHalfDim * sizeof(float),
                  "the reduction buffer holds the absorption's query rows");
    if (static_cast<int>(blockIdx.x) >= nblk) {
      const int u = blockIdx.x - nblk;
      if (u >= p.ab.units) return;
      absorb_rows<T, kThreads>(p.ab, u % p.ab.Hkv, (u / p.ab.Hkv) % p.ab.B,
                               u / (p.ab.Hkv * p.ab.B),
                               reinterpret_cast<float (*)[2 * kMaxHalfDim]>(&red[0][0]));
      return;
    }
  }
  const int tid = threadIdx.x;
  const int col0 = blockIdx.x * kCols;
  const bool is_v = col0 >= width;
  const int c0 = is_v ? col0 - width : col0;
  const T* A = static_cast<const T*>(is_v ? p.a_v : p.a_k) + static_cast<size_t>(c0) * p.dm;
  const T* x = static_cast<const T*>(p.x);
  T* h = static_cast<T*>(is_v ? p.h_v : p.h_k);
  const int nk = p.dm / 8;                     // 8-element chunks of d_model
  const int o = tid >> 3, part = tid & 7;      // reduction: output o = (column, sequence)

  for (int b0 = 0; b0 < p.B; b0 += kSeq) {
    float acc[kCols][kSeq];
#pragma unroll
    for (int c = 0; c < kCols; ++c)
#pragma unroll
      for (int s = 0; s < kSeq; ++s) acc[c][s] = 0.f;
    for (int k0 = tid; k0 < nk; k0 += kThreads * kSlab) {
      // every load of the slab first (chunks past d_model read the last chunk
      // and are not added; sequences past B read the last sequence, whose sums
      // are never stored)
      Raw8<T> a[kSlab][kCols], xv[kSlab][kSeq];
#pragma unroll
      for (int i = 0; i < kSlab; ++i) {
        const int kc = min(k0 + i * kThreads, nk - 1);
#pragma unroll
        for (int c = 0; c < kCols; ++c) a[i][c].load(A + static_cast<size_t>(c) * p.dm + 8 * kc);
#pragma unroll
        for (int s = 0; s < kSeq; ++s)
          xv[i][s].load(x + static_cast<size_t>(min(b0 + s, p.B - 1)) * p.dm + 8 * kc);
      }
#pragma unroll
      for (int i = 0; i < kSlab; ++i) {
        if (k0 + i * kThreads < nk) {
#pragma unroll
          for (int c = 0; c < kCols; ++c)
#pragma unroll
            for (int s = 0; s < kSeq; ++s)
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[c][s] = fmaf(xv[i][s][e], a[i][c][e], acc[c][s]);
        }
      }
    }
    __syncthreads();                           // the previous pass's reads of red are done
#pragma unroll
    for (int c = 0; c < kCols; ++c)
#pragma unroll
      for (int s = 0; s < kSeq; ++s) red[tid][c * kSeq + s] = acc[c][s];
    __syncthreads();
    float sum = red[32 * part][o];
#pragma unroll
    for (int i = 1; i < 32; ++i) sum += red[32 * part + i][o];
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    sum += __shfl_xor(sum, 4);
    if (part == 0) {
      const int c = o / kSeq, b = b0 + o % kSeq;
      if (b < p.B) {
        const int pos = p.pos[b];
        if (pos >= 0 && pos < p.L) {
          const int cl = c0 + c, g = cl / p.r, k = cl % p.r;
          store_elem(h, ((static_cast<size_t>(b) * p.G + g) * p.L + pos) * p.r + k, sum);
        }
      }
    }
  }
}

}  // namespace

long append_t_blocks(const AppendParams& p) { return 2L * p.G * p.r / kCols; }

int append_t_threads() { return kThreads; }

hipError_t launch_append_t(const AppendParams& p, int dtype, hipStream_t st) {
  const long n = append_t_blocks(p) + (p.ab.units > 0 ? p.ab.units : 0);
  if (n > 0x7fffffffL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(n));
  const bool fuse = p.ab.units > 0;
  if (dtype == 0) {
    if (fuse) append_t_kernel<float, true><<<grid, kThreads, 0, st>>>(p);
    else append_t_kernel<float, false><<<grid, kThreads, 0, st>>>(p);
  } else {
    if (fuse) append_t_kernel<uint16_t, true><<<grid, kThreads, 0, st>>>(p);
    else append_t_kernel<uint16_t, false><<<grid, kThreads, 0, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace palu
