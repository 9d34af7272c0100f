// Plain VALU context-split attention kernel for any dtype and shape in range.
// It handles one query head per workgroup (the latents are re-read per head);
// the MFMA kernels are the fast path for bf16, this one is the path for fp32
// caches and for shapes the fast kernels do not take.
//
// Method (Palu author responses on OpenReview):
//   K_j = H_k B_k[:, cols(j)]  ("Why Palu Requires Fewer Global Memory Access")
//   keys are rotated after reconstruction (clarification of W1)
//   value latents are summed with the attention weights and B_v is applied
//   once afterwards (clarification of W1)
// Split-context softmax: each workgroup keeps a running max m (log2 units),
// sum l and unnormalised latent sum u; the merge rescales and adds them.
#include <math.h>

#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

constexpr int kThreads = 256;
constexpr int kTileTokens = 8;          // tokens per inner tile
constexpr int kLanesPerToken = kThreads / kTileTokens;   // 32
constexpr int kMaxRankPerThread = 2;    // rank <= 512

template <typename T, bool kAbsorbed>
__global__ __launch_bounds__(kThreads) void split_generic_kernel(DecodeParams p) {
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int n = clamp_len(p.lens, b, p.L);
  const int t0 = split * p.split_tokens;
  if (t0 >= n) return;
  const int t1 = min(n, t0 + p.split_tokens);
  const int j = h / p.gqa, g = j / p.s, jl = j % p.s;
  const int r = p.r, d = p.d, half = d / 2;
  const int dq = kAbsorbed ? r : d;

  extern __shared__ float smem[];
  float* qs = smem;                        // [dq]
  float* hk = qs + dq;                     // [kTileTokens][r]
  float* hv = hk + kTileTokens * r;        // [kTileTokens][r]
  float* kt = hv + kTileTokens * r;        // [kTileTokens][d] rebuilt keys
  float* sc = kt + kTileTokens * d;        // [kTileTokens]

  if (kAbsorbed) {
    const float* qt = p.qt + (static_cast<size_t>(b) * p.Hq + h) * r;
    for (int k = tid; k < r; k += kThreads) qs[k] = qt[k];
  } else {
    const T* q = static_cast<const T*>(p.q) + (static_cast<size_t>(b) * p.Hq + h) * d;
    for (int c = tid; c < d; c += kThreads) qs[c] = load_f32(q, c) * p.scale_log2;
  }
  const size_t row0 = (static_cast<size_t>(b) * p.G + g) * p.L;
  const T* Hk = static_cast<const T*>(p.h_k) + row0 * r;
  const T* Hv = static_cast<const T*>(p.h_v) + row0 * r;
  const T* Bk = kAbsorbed ? nullptr
                          : static_cast<const T*>(p.b_k) + static_cast<size_t>(g) * r * p.Dg + jl * d;

  float m = -INFINITY, l = 0.f;
  float u[kMaxRankPerThread];
#pragma unroll
  for (int i = 0; i < kMaxRankPerThread; ++i) u[i] = 0.f;

  for (int tt = t0; tt < t1; tt += kTileTokens) {
    const int nt = min(kTileTokens, t1 - tt);
    __syncthreads();
    for (int e = tid; e < nt * r; e += kThreads) {
      hk[e] = load_f32(Hk, static_cast<size_t>(tt) * r + e);
      hv[e] = load_f32(Hv, static_cast<size_t>(tt) * r + e);
    }
    __syncthreads();
    if (!kAbsorbed) {
      for (int e = tid; e < nt * d; e += kThreads) {
        const int t = e / d, c = e % d;
        float acc = 0.f;
        for (int k = 0; k < r; ++k) acc = fmaf(hk[t * r + k], load_f32(Bk, static_cast<size_t>(k) * p.Dg + c), acc);
        kt[e] = acc;
      }
      __syncthreads();
      if (p.rope) {
        for (int e = tid; e < nt * half; e += kThreads) {
          const int t = e / half, i = e % half;
          float cs, sn;
          rope_cos_sin(p.omega_rev[i], tt + t, cs, sn);
          const float x = kt[t * d + i], y = kt[t * d + i + half];
          kt[t * d + i] = x * cs - y * sn;
          kt[t * d + i + half] = x * sn + y * cs;
        }
        __syncthreads();
      }
    }
    {  // scores in log2 units: kLanesPerToken lanes per token, then a lane reduction
      const int t = tid / kLanesPerToken, lt = tid % kLanesPerToken;
      float acc = 0.f;
      if (t < nt) {
        const float* row = kAbsorbed ? hk + t * r : kt + t * d;
        for (int c = lt; c < dq; c += kLanesPerToken) acc = fmaf(qs[c], row[c], acc);
      }
#pragma unroll
      for (int off = kLanesPerToken / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kLanesPerToken);
      if (lt == 0 && t < nt) sc[t] = acc;
    }
    __syncthreads();
    float mt = -INFINITY;
    for (int t = 0; t < nt; ++t) mt = fmaxf(mt, sc[t]);
    const float mn = fmaxf(m, mt);
    const float alpha = exp2f(m - mn);
    float pt[kTileTokens];
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < kTileTokens; ++t) {
      pt[t] = t < nt ? exp2f(sc[t] - mn) : 0.f;
      lsum += pt[t];
    }
    l = l * alpha + lsum;
    m = mn;
#pragma unroll
    for (int i = 0; i < kMaxRankPerThread; ++i) {
      const int k = tid + i * kThreads;
      if (k < r) {
        float acc = u[i] * alpha;
#pragma unroll
        for (int t = 0; t < kTileTokens; ++t)
          if (t < nt) acc = fmaf(pt[t], hv[t * r + k], acc);
        u[i] = acc;
      }
    }
  }
  const size_t slot = (static_cast<size_t>(b) * p.Hq + h) * p.n_split + split;
  if (tid == 0) {
    p.part_ml[slot * 2] = m;
    p.part_ml[slot * 2 + 1] = l;
  }
#pragma unroll
  for (int i = 0; i < kMaxRankPerThread; ++i) {
    const int k = tid + i * kThreads;
    if (k < r) p.part_u[slot * r + k] = u[i];
  }
}

}  // namespace

size_t generic_split_smem(const DecodeParams& p, int absorbed) {
  const int dq = absorbed ? p.r : p.d;
  return sizeof(float) * (dq + 2 * kTileTokens * p.r + kTileTokens * p.d + kTileTokens);
}

hipError_t launch_split_generic(const DecodeParams& p, int dtype, int absorbed, hipStream_t st) {
  const dim3 grid(p.n_split, p.Hq, p.B);
  const size_t sm = generic_split_smem(p, absorbed);
  if (dtype == 0) {
    if (absorbed) split_generic_kernel<float, true><<<grid, kThreads, sm, st>>>(p);
    else split_generic_kernel<float, false><<<grid, kThreads, sm, st>>>(p);
  } else {
    if (absorbed) split_generic_kernel<uint16_t, true><<<grid, kThreads, sm, st>>>(p);
    else split_generic_kernel<uint16_t, false><<<grid, kThreads, sm, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace palu
