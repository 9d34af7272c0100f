// The two small passes around the context-split kernel. Both are latency
// bound (a few MB of L2-resident data), so each thread issues all of its loads
// at the start and the work costs about one memory round trip.
//
// absorb_q: for the absorbed-key mode, q~ = q B_k[g][:, cols(j)]^T for every
//   query head (Palu author response on OpenReview, clarification of W1: only
//   a rotary embedding forces the keys to be rebuilt; without it B_k can be
//   applied to the query). Workgroups over (KV head, sequence, slice of r);
//   each thread loads its piece of a B_k row at once and the pieces of a row
//   are added with lane shuffles; q~ is stored in fp32 pre-multiplied by
//   scale * log2(e).
//
// merge: combine the per-split softmax states (m, l, u) of one query head,
//   u* = sum_s 2^(m_s - M) u_s / sum_s 2^(m_s - M) l_s, then apply the value
//   reconstruction once, out = u* B_v[g][:, cols(j)] (clarification of W1:
//   values are never rebuilt, B_v acts after the weighted sum).
#include <math.h>

#include "absorb_device.h"
#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

constexpr int kThreads = 256;
constexpr int kWarps = kThreads / 64;
constexpr int kAbsRows = 64;        // rows of r per absorb workgroup (general form)

// General form (any even d <= 256): thread = (row, quarter of d).
template <typename T, bool kVec8>
__global__ __launch_bounds__(kThreads) void absorb_q_kernel(DecodeParams p) {
  const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int g = j / p.s, jl = j % p.s;
  const int kq = tid / 4, qtr = tid % 4;               // row in the slice, quarter of d
  const int k = blockIdx.z * kAbsRows + kq;
  const int dq = (p.d + 3) / 4;                        // columns per quarter
  const int c0 = qtr * dq, c1 = min(p.d, c0 + dq);
  __shared__ float qs[kAbsHeadChunk][2 * kMaxHalfDim];
  const T* row = static_cast<const T*>(p.b_k) + static_cast<size_t>(g) * p.r * p.Dg +
                 static_cast<size_t>(min(k, p.r - 1)) * p.Dg + jl * p.d;
  // the quarter-row of B_k: at most 64 columns, loaded at once
  float v[64];
  if (kVec8 && dq % 8 == 0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (8 * u < dq) load8_f32(row + c0 + 8 * u, v + 8 * u);
      else
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * u + e] = 0.f;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 64; ++e) v[e] = c0 + e < c1 ? load_f32(row, c0 + e) : 0.f;
  }
  for (int h0 = 0; h0 < p.gqa; h0 += kAbsHeadChunk) {
    const int nh = min(kAbsHeadChunk, p.gqa - h0);
    const int head0 = j * p.gqa + h0;
    __syncthreads();
    for (int e = tid; e < kAbsHeadChunk * p.d; e += kThreads) {
      const int hh = e / p.d, c = e % p.d;
      qs[hh][c] = hh < nh ? load_f32(static_cast<const T*>(p.q),
                                     (static_cast<size_t>(b) * p.Hq + head0 + hh) * p.d + c)
                          : 0.f;
    }
    __syncthreads();
    float acc[kAbsHeadChunk];
#pragma unroll
    for (int hh = 0; hh < kAbsHeadChunk; ++hh) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 64; ++e)
        if (c0 + e < c1) a = fmaf(qs[hh][c0 + e], v[e], a);
      a += __shfl_xor(a, 1);       // the four quarters of a row are adjacent lanes
      a += __shfl_xor(a, 2);
      acc[hh] = a;
    }
    if (qtr == 0 && k < p.r)
      for (int hh = 0; hh < nh; ++hh)
        p.qt[(static_cast<size_t>(b) * p.Hq + head0 + hh) * p.r + k] = acc[hh] * p.scale_log2;
  }
}

// Fast form when d/8 is a power of two <= 32 (absorb_rows): workgroup (KV
// head, sequence, kAbsRowsPer*256*8/d rows of r).
template <typename T>
__global__ __launch_bounds__(kThreads) void absorb_q_vec_kernel(DecodeParams p) {
  __shared__ float qs[kAbsHeadChunk][2 * kMaxHalfDim];
  absorb_rows<T, kThreads>(absorb_args(p), blockIdx.x, blockIdx.y, blockIdx.z, qs);
}

// q~ = q (the uncompressed baseline: keys are the cached rows themselves),
// pre-multiplied by scale * log2(e) like the absorbed queries
template <typename T>
__global__ __launch_bounds__(kThreads) void prescale_q_kernel(DecodeParams p) {
  const size_t n = static_cast<size_t>(p.B) * p.Hq * p.d;
  const size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n) p.qt[i] = load_f32(static_cast<const T*>(p.q), i) * p.scale_log2;
}

constexpr int kBvRows = 16;        // B_v rows per thread kept in flight
constexpr int kSplitBatch = 16;    // split partials per thread kept in flight
constexpr int kSplitLDS = 1024;    // split weights staged in LDS per chunk

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void merge_kernel(DecodeParams p) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, warp = tid >> 6;
  const int n = clamp_len(p.lens, b, p.L);
  const int ns = (n + p.split_tokens - 1) / p.split_tokens;
  const bool full = p.full_rank != 0 || p.latent_out != 0;   // no B_v: out = u*
  const int ow = full ? p.r : p.d;                            // output width
  float* out = p.out + (static_cast<size_t>(b) * p.Hq + h) * ow;
  if (ns == 0) {
    for (int c = tid; c < ow; c += kThreads) out[c] = 0.f;
    return;
  }
  const int j = h / p.gqa, g = j / p.s, jl = j % p.s;
  const size_t base = (static_cast<size_t>(b) * p.Hq + h) * p.n_split;
  const float* ml = p.part_ml + base * 2;
  const float* pu = p.part_u + base * p.r;
  const T* Bv = full ? nullptr
                     : static_cast<const T*>(p.b_v) + static_cast<size_t>(g) * p.r * p.Dg + jl * p.d;

  __shared__ float wred[kWarps];
  __shared__ float wts[kSplitLDS];
  __shared__ float us[2 * kThreads];   // r <= 512
  __shared__ float red2[2048];

  // ---- 1. issue every independent load at once: the first B_v rows, this
  //         thread's split state, the first split partials of its u* entries
  const bool vec = p.d % 8 == 0;
  const int ncc = vec ? p.d / 8 : 1, ngroups = kThreads / ncc;
  const int cc = tid % ncc, rg = tid / ncc;
  // B_v rows as raw bits, rows past r (or threads past the row groups) read a
  // valid row whose weight is 0
  Raw8<T> bv[kBvRows];
  if (vec && !full) {
#pragma unroll
    for (int i = 0; i < kBvRows; ++i) {
      const int k = min(min(rg, ngroups - 1) + i * ngroups, p.r - 1);
      bv[i].load(Bv + static_cast<size_t>(k) * p.Dg + 8 * cc);
    }
  }
  const int phases = p.r >= kThreads ? 1 : kThreads / p.r;
  const int kq = p.r >= kThreads ? tid : tid % p.r;
  const int ph = p.r >= kThreads ? 0 : tid / p.r;
  const bool active = ph < phases;
  const bool two = kq + kThreads < p.r;
  float ua[kSplitBatch], ub[kSplitBatch];
  auto load_u = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kSplitBatch; ++u) {
      const int sp = s0 + ph + u * phases;
      const bool ok = active && sp < ns;
      const float* rowp = pu + static_cast<size_t>(ok ? sp : 0) * p.r;
      ua[u] = ok ? rowp[kq] : 0.f;
      ub[u] = ok && two ? rowp[kq + kThreads] : 0.f;
    }
  };
  load_u(0);
  const bool one_pass = ns <= kThreads;      // each thread holds one split's state
  float my_m = -INFINITY, my_l = 0.f;
  if (tid < ns) {
    my_m = ml[tid * 2];
    my_l = ml[tid * 2 + 1];
  }

  // ---- 2. M = max_s m_s (wave shuffles, one LDS step)
  float mloc = my_m;
  for (int sp = tid + kThreads; sp < ns; sp += kThreads) mloc = fmaxf(mloc, ml[sp * 2]);
  mloc = wave_max(mloc);
  if (lane == 0) wred[warp] = mloc;
  __syncthreads();
  float M = wred[0];
#pragma unroll
  for (int w = 1; w < kWarps; ++w) M = fmaxf(M, wred[w]);
  __syncthreads();

  // ---- 3. u* = sum_s w_s u_s / L, w_s = 2^(m_s - M), in chunks of kSplitLDS
  float u0 = 0.f, u1 = 0.f, lsum = 0.f;
  for (int c0 = 0; c0 < ns; c0 += kSplitLDS) {
    const int cnt = min(kSplitLDS, ns - c0);
    if (c0 > 0) __syncthreads();
    for (int e = tid; e < cnt; e += kThreads) {
      const float m = one_pass ? my_m : ml[(c0 + e) * 2];
      const float l = one_pass ? my_l : ml[(c0 + e) * 2 + 1];
      const float w = exp2f(m - M);
      wts[e] = w;
      lsum = fmaf(w, l, lsum);
    }
    __syncthreads();
    for (int s0 = c0; s0 < c0 + cnt; s0 += kSplitBatch * phases) {
      if (s0 > 0) load_u(s0);
#pragma unroll
      for (int u = 0; u < kSplitBatch; ++u) {
        const int sp = s0 + ph + u * phases;
        const float w = active && sp < c0 + cnt ? wts[sp - c0] : 0.f;
        u0 = fmaf(w, ua[u], u0);
        u1 = fmaf(w, ub[u], u1);
      }
    }
  }
  lsum = wave_sum(lsum);
  if (lane == 0) wred[warp] = lsum;
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kWarps; ++w) L += wred[w];
  const float inv = 1.f / L;
  // reduce u over the split phases (phases > 1 only when r < 256)
  if (phases == 1) {
    us[kq] = u0 * inv;
    if (two) us[kq + kThreads] = u1 * inv;
  } else {
    red2[tid] = active ? u0 : 0.f;
    __syncthreads();
    if (tid < p.r) {
      float a = 0.f;
      for (int q = 0; q < phases; ++q) a += red2[q * p.r + tid];
      us[tid] = a * inv;
    }
  }
  __syncthreads();
  if (full) {
    for (int c = tid; c < p.r; c += kThreads) out[c] = us[c];
    return;
  }

  // ---- 4. out = u* B_v[:, cols(j)]
  if (vec) {
    // thread = (row group, 8-column chunk); row groups added through LDS
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kBvRows; ++i) {
      const int k = rg + i * ngroups;
      const float w = rg < ngroups && k < p.r ? us[k] : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, bv[i][e], acc[e]);
    }
    for (int k0 = rg + kBvRows * ngroups; k0 < p.r; k0 += kBvRows * ngroups) {
#pragma unroll
      for (int i = 0; i < kBvRows; ++i) {
        const int k = min(k0 + i * ngroups, p.r - 1);
        bv[i].load(Bv + static_cast<size_t>(k) * p.Dg + 8 * cc);
      }
#pragma unroll
      for (int i = 0; i < kBvRows; ++i) {
        const int k = k0 + i * ngroups;
        const float w = rg < ngroups && k < p.r ? us[k] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, bv[i][e], acc[e]);
      }
    }
    if (rg < ngroups) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red2[rg * p.d + 8 * cc + e] = acc[e];
    }
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
  red2[tid] = acc;
  __syncthreads();
  if (tid < p.d) {
    float a = 0.f;
    for (int q = 0; q < kph; ++q) a += red2[q * p.d + tid];
    out[tid] = a;
  }
}

// Merge for up to kFastSplits splits, d/8 a power of two <= 32, r <= 512:
// every wave reduces the split states itself (lane s holds split s), so the
// only workgroup barriers are the two around the B_v product, and every load
// (split states, partials of the first 16 splits, the first 16 B_v rows of the
// thread) is issued before any arithmetic.
constexpr int kFastSplits = 64;

template <typename T>
__global__ __launch_bounds__(kThreads) void merge_fast_kernel(DecodeParams p) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int j = h / p.gqa, g = j / p.s, jl = j % p.s;
  const size_t base = (static_cast<size_t>(b) * p.Hq + h) * p.n_split;
  const float* ml = p.part_ml + base * 2;
  const float* pu = p.part_u + base * p.r;
  const bool full = p.full_rank != 0 || p.latent_out != 0;   // no B_v: out = u*
  const T* Bv = full ? nullptr
                     : static_cast<const T*>(p.b_v) + static_cast<size_t>(g) * p.r * p.Dg + jl * p.d;
  const int ncc = p.d / 8, ngroups = kThreads / ncc;
  const int cc = tid % ncc, rg = tid / ncc;
  const int nrow = (p.r + ngroups - 1) / ngroups;      // B_v rows of this thread

  // Loads do not wait for the sequence length: the first 16 splits' states
  // and partials (all inside the workspace) are requested together with the
  // length and B_v, and entries of splits >= ns are discarded afterwards.
  Raw8<T> bv[16];
  auto load_bv = [&](int i0) {   // rows past r read row r-1 (finite, weight 0)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = min(rg + ngroups * (i0 + i), p.r - 1);
      bv[i].load(Bv + static_cast<size_t>(k) * p.Dg + 8 * cc);
    }
  };
  // thread t holds u entries t and t + 256 of 16 splits at a time
  float ua[16], ub[16];
  auto load_u = [&](int s0) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int sp = min(s0 + u, p.n_split - 1);
      const float* row = pu + static_cast<size_t>(sp) * p.r;
      ua[u] = tid < p.r ? row[tid] : 0.f;
      ub[u] = tid + kThreads < p.r ? row[tid + kThreads] : 0.f;
    }
  };
  const int n = clamp_len(p.lens, b, p.L);
  const float ms_raw = lane < p.n_split ? ml[2 * lane] : 0.f;
  const float ls_raw = lane < p.n_split ? ml[2 * lane + 1] : 0.f;
  load_u(0);
  if (!full) load_bv(0);
  const int ns = (n + p.split_tokens - 1) / p.split_tokens;
  const int ow = full ? p.r : p.d;                            // output width
  float* out = p.out + (static_cast<size_t>(b) * p.Hq + h) * ow;
  if (ns == 0) {
    for (int c = tid; c < ow; c += kThreads) out[c] = 0.f;
    return;
  }
  const float ms = lane < ns ? ms_raw : -INFINITY;
  const float ls = lane < ns ? ls_raw : 0.f;

  // split weights 2^(m_s - M) and L = sum_s w_s l_s, in every wave
  const float M = wave_max(ms);
  const float w = lane < ns ? exp2f(ms - M) : 0.f;
  const float L = wave_sum(w * ls);
  float u0 = 0.f, u1 = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 16) {
    if (s0 > 0) load_u(s0);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (s0 + u < ns) {              // uniform; later splits hold stale data
        const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s0 + u));
        u0 = fmaf(ws, ua[u], u0);
        u1 = fmaf(ws, ub[u], u1);
      }
    }
  }
  __shared__ float us[2 * kThreads];
  __shared__ float red[2048];
  const float inv = 1.f / L;
  if (full) {
    if (tid < p.r) out[tid] = u0 * inv;
    if (tid + kThreads < p.r) out[tid + kThreads] = u1 * inv;
    return;
  }
  if (tid < p.r) us[tid] = u0 * inv;
  if (tid + kThreads < p.r) us[tid + kThreads] = u1 * inv;
  __syncthreads();

  // out = u* B_v[:, cols(j)]: thread (row group, 8-column chunk), groups added in LDS
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < nrow; i0 += 16) {
    if (i0 > 0) load_bv(i0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = rg + ngroups * (i0 + i);
      const float wv = k < p.r ? us[k] : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(wv, bv[i][e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg * p.d + 8 * cc + e] = acc[e];
  __syncthreads();
  if (tid < p.d) {
    float a = 0.f;
    for (int q = 0; q < ngroups; ++q) a += red[q * p.d + tid];
    out[tid] = a;
  }
}

}  // namespace

hipError_t launch_absorb_q(const DecodeParams& p, int dtype, hipStream_t st) {
  if (absorb_carriable(absorb_args(p))) {
    const dim3 grid(p.Hkv, p.B, absorb_slices(absorb_args(p), kThreads));
    if (dtype == 0) absorb_q_vec_kernel<float><<<grid, kThreads, 0, st>>>(p);
    else absorb_q_vec_kernel<uint16_t><<<grid, kThreads, 0, st>>>(p);
    return hipGetLastError();
  }
  const dim3 grid(p.Hkv, p.B, (p.r + kAbsRows - 1) / kAbsRows);
  const bool v8 = p.d % 32 == 0;     // quarters of d in whole 16-byte chunks
  if (dtype == 0) {
    if (v8) absorb_q_kernel<float, true><<<grid, kThreads, 0, st>>>(p);
    else absorb_q_kernel<float, false><<<grid, kThreads, 0, st>>>(p);
  } else {
    if (v8) absorb_q_kernel<uint16_t, true><<<grid, kThreads, 0, st>>>(p);
    else absorb_q_kernel<uint16_t, false><<<grid, kThreads, 0, st>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_prescale_q(const DecodeParams& p, int dtype, hipStream_t st) {
  const size_t n = static_cast<size_t>(p.B) * p.Hq * p.d;
  const dim3 grid(static_cast<unsigned>((n + kThreads - 1) / kThreads));
  if (dtype == 0) prescale_q_kernel<float><<<grid, kThreads, 0, st>>>(p);
  else prescale_q_kernel<uint16_t><<<grid, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_merge(const DecodeParams& p, int dtype, hipStream_t st) {
  const dim3 grid(p.Hq, p.B);
  const int ncc = p.d / 8;
  if (p.d % 8 == 0 && ncc <= 32 && (ncc & (ncc - 1)) == 0 && p.r <= 2 * kThreads &&
      p.n_split <= kFastSplits) {
    if (dtype == 0) merge_fast_kernel<float><<<grid, kThreads, 0, st>>>(p);
    else merge_fast_kernel<uint16_t><<<grid, kThreads, 0, st>>>(p);
    return hipGetLastError();
  }
  if (dtype == 0) merge_kernel<float><<<grid, kThreads, 0, st>>>(p);
  else merge_kernel<uint16_t><<<grid, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace palu
