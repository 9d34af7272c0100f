// The two small passes around the context-split kernel.
//
// absorb_q: for the absorbed-key mode, q~ = q B_k[g][:, cols(j)]^T for every
//   query head (Palu author response on OpenReview, clarification of W1: only
//   a rotary embedding forces the keys to be rebuilt; without it B_k can be
//   applied to the query). One workgroup per (KV head, sequence) serves the
//   KV head's query heads together, so each B_k row segment is read once per
//   workgroup; q~ is stored in fp32, pre-multiplied by scale * log2(e).
//
// merge: combine the per-split softmax states (m, l, u) of one query head,
//   u* = sum_s 2^(m_s - M) u_s / sum_s 2^(m_s - M) l_s, then apply the value
//   reconstruction once, out = u* B_v[g][:, cols(j)] (clarification of W1:
//   values are never rebuilt, B_v acts after the weighted sum). Work is spread
//   over thread phases (splits for u*, rows of B_v for out) so that many
//   independent loads are in flight instead of one long dependent loop.
#include <math.h>

#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

constexpr int kThreads = 256;
constexpr int kHeadChunk = 8;       // query heads absorbed per pass
constexpr int kWeightChunk = 1024;  // split weights staged in LDS per pass

template <typename T, bool kVec8>
__global__ __launch_bounds__(kThreads) void absorb_q_kernel(DecodeParams p) {
  const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int g = j / p.s, jl = j % p.s;
  __shared__ float qs[kHeadChunk][2 * kMaxHalfDim];
  const T* Bk = static_cast<const T*>(p.b_k) + static_cast<size_t>(g) * p.r * p.Dg + jl * p.d;
  for (int h0 = 0; h0 < p.gqa; h0 += kHeadChunk) {
    const int nh = min(kHeadChunk, p.gqa - h0);
    const int head0 = j * p.gqa + h0;
    __syncthreads();
    for (int e = tid; e < kHeadChunk * p.d; e += kThreads) {
      const int hh = e / p.d, c = e % p.d;
      qs[hh][c] = hh < nh ? load_f32(static_cast<const T*>(p.q),
                                     (static_cast<size_t>(b) * p.Hq + head0 + hh) * p.d + c)
                          : 0.f;
    }
    __syncthreads();
    for (int k = tid; k < p.r; k += kThreads) {
      float acc[kHeadChunk];
#pragma unroll
      for (int hh = 0; hh < kHeadChunk; ++hh) acc[hh] = 0.f;
      const T* row = Bk + static_cast<size_t>(k) * p.Dg;
      if (kVec8) {
        for (int c0 = 0; c0 < p.d; c0 += 64) {      // eight 16-byte loads in flight
          float v[64];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            if (c0 + 8 * u < p.d) load8_f32(row + c0 + 8 * u, v + 8 * u);
            else
#pragma unroll
              for (int e = 0; e < 8; ++e) v[8 * u + e] = 0.f;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            if (c0 + 8 * u >= p.d) break;
#pragma unroll
            for (int hh = 0; hh < kHeadChunk; ++hh)
#pragma unroll
              for (int e = 0; e < 8; ++e)
                acc[hh] = fmaf(qs[hh][c0 + 8 * u + e], v[8 * u + e], acc[hh]);
          }
        }
      } else {
        for (int c = 0; c < p.d; ++c) {
          const float v = load_f32(row, c);
#pragma unroll
          for (int hh = 0; hh < kHeadChunk; ++hh) acc[hh] = fmaf(qs[hh][c], v, acc[hh]);
        }
      }
      for (int hh = 0; hh < nh; ++hh)
        p.qt[(static_cast<size_t>(b) * p.Hq + head0 + hh) * p.r + k] = acc[hh] * p.scale_log2;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void merge_kernel(DecodeParams p) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int n = clamp_len(p.lens, b, p.L);
  const int ns = (n + p.split_tokens - 1) / p.split_tokens;
  float* out = p.out + (static_cast<size_t>(b) * p.Hq + h) * p.d;
  if (ns == 0) {
    for (int c = tid; c < p.d; c += kThreads) out[c] = 0.f;
    return;
  }
  const int j = h / p.gqa, g = j / p.s, jl = j % p.s;
  const size_t base = (static_cast<size_t>(b) * p.Hq + h) * p.n_split;
  const float* ml = p.part_ml + base * 2;
  const float* pu = p.part_u + base * p.r;

  __shared__ float red[kThreads];
  __shared__ float wts[kWeightChunk];
  __shared__ float us[2 * kThreads];   // r <= 512

  // M = max_s m_s
  float mloc = -INFINITY;
  for (int sp = tid; sp < ns; sp += kThreads) mloc = fmaxf(mloc, ml[sp * 2]);
  red[tid] = mloc;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();

  // thread phases over splits for u*: phases = 256 / r (at least 1)
  const int phases = p.r >= kThreads ? 1 : kThreads / p.r;
  const int kq = p.r >= kThreads ? tid : tid % p.r;
  const int ph = p.r >= kThreads ? 0 : tid / p.r;
  const bool active = ph < phases;
  float u0 = 0.f, u1 = 0.f, lsum = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kWeightChunk) {
    const int cnt = min(kWeightChunk, ns - s0);
    __syncthreads();
    for (int e = tid; e < cnt; e += kThreads) {
      const float w = exp2f(ml[(s0 + e) * 2] - M);
      wts[e] = w;
      lsum = fmaf(w, ml[(s0 + e) * 2 + 1], lsum);
    }
    __syncthreads();
    if (active) {
      const bool two = kq + kThreads < p.r;
      for (int e0 = ph; e0 < cnt; e0 += 8 * phases) {   // eight splits' loads in flight
        float w[8], a[8], b2[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = e0 + u * phases;
          const bool ok = e < cnt;
          const float* row = pu + static_cast<size_t>(s0 + (ok ? e : 0)) * p.r;
          w[u] = ok ? wts[e] : 0.f;
          a[u] = ok ? row[kq] : 0.f;
          b2[u] = ok && two ? row[kq + kThreads] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          u0 = fmaf(w[u], a[u], u0);
          u1 = fmaf(w[u], b2[u], u1);
        }
      }
    }
  }
  // total weight: block sum of lsum
  red[tid] = lsum;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float inv = 1.f / red[0];
  __syncthreads();
  // reduce u over phases (phases > 1 only when r < 256)
  if (phases == 1) {
    us[kq] = u0 * inv;
    if (kq + kThreads < p.r) us[kq + kThreads] = u1 * inv;
    __syncthreads();
  } else {
    red[tid] = active ? u0 : 0.f;
    __syncthreads();
    if (tid < p.r) {
      float a = 0.f;
      for (int q = 0; q < phases; ++q) a += red[q * p.r + tid];
      us[tid] = a * inv;
    }
    __syncthreads();
  }

  // out = u* B_v[:, cols(j)]
  const T* Bv = static_cast<const T*>(p.b_v) + static_cast<size_t>(g) * p.r * p.Dg + jl * p.d;
  if (p.d % 8 == 0) {
    // thread = (row group, 8-column chunk); all of its rows' 16-byte loads go out
    // together, then the row groups are added through LDS (groups * d == 2048)
    __shared__ float red2[2048];
    const int ncc = p.d / 8, ngroups = kThreads / ncc;
    const int cc = tid % ncc, rg = tid / ncc;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k0 = rg; k0 < p.r; k0 += 8 * ngroups) {
      float v[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u * ngroups;
        if (k < p.r) load8_f32(Bv + static_cast<size_t>(k) * p.Dg + 8 * cc, v[u]);
        else
#pragma unroll
          for (int e = 0; e < 8; ++e) v[u][e] = 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u * ngroups;
        const float w = k < p.r ? us[k] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, v[u][e], acc[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red2[rg * p.d + 8 * cc + e] = acc[e];
    __syncthreads();
    if (tid < p.d) {
      float a = 0.f;
      for (int q = 0; q < ngroups; ++q) a += red2[q * p.d + tid];
      out[tid] = a;
    }
    return;
  }
  // any even d: thread (column c, row phase kp), then reduce phases
  const int kph = kThreads / p.d;           // d <= 256, so at least 1
  const int c = tid % p.d, kp = tid / p.d;
  float acc = 0.f;
  if (kp < kph) {
    const int per = (p.r + kph - 1) / kph;
    const int k0 = kp * per, k1 = min(p.r, k0 + per);
#pragma unroll 8
    for (int k = k0; k < k1; ++k) acc = fmaf(us[k], load_f32(Bv, static_cast<size_t>(k) * p.Dg + c), acc);
  }
  red[tid] = acc;
  __syncthreads();
  if (tid < p.d) {
    float a = 0.f;
    for (int q = 0; q < kph; ++q) a += red[q * p.d + tid];
    out[tid] = a;
  }
}

}  // namespace

hipError_t launch_absorb_q(const DecodeParams& p, int dtype, hipStream_t st) {
  const dim3 grid(p.Hkv, p.B);
  const bool v8 = p.d % 8 == 0;
  if (dtype == 0) {
    if (v8) absorb_q_kernel<float, true><<<grid, kThreads, 0, st>>>(p);
    else absorb_q_kernel<float, false><<<grid, kThreads, 0, st>>>(p);
  } else {
    if (v8) absorb_q_kernel<uint16_t, true><<<grid, kThreads, 0, st>>>(p);
    else absorb_q_kernel<uint16_t, false><<<grid, kThreads, 0, st>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const DecodeParams& p, int dtype, hipStream_t st) {
  const dim3 grid(p.Hq, p.B);
  if (dtype == 0) merge_kernel<float><<<grid, kThreads, 0, st>>>(p);
  else merge_kernel<uint16_t><<<grid, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace palu
