// The query absorption of one workgroup, shared by its own launch and by the
// append launch that carries it as extra workgroups (Palu author response on
// OpenReview, clarification of W1: without a rotary embedding B_k can be
// applied to the query, q~ = q B_k[g][:, cols(j)]^T).
//
// Workgroup (KV head j, sequence b, slice z of kAbsRowsPer * kThreads / (d / 8)
// rows of r); thread (row group kr, 8-column chunk): kAbsRowsPer 16-byte loads
// of B_k, rows kr, kr + kThreads / (d / 8), ... of the slice, all issued
// together; the query heads of KV head j staged in LDS (qs, supplied by the
// caller: at least kAbsHeadChunk rows of 2 * kMaxHalfDim floats), and the
// chunks of a row added with lane shuffles; q~ is stored in fp32
// pre-multiplied by scale * log2(e). Needs d / 8 a power of two <= 32.
#pragma once

#include "device_util.h"
#include "palu_internal.h"

namespace palu {

constexpr int kAbsHeadChunk = 8;   // query heads absorbed per pass

template <typename T, int kThreads>
__device__ __forceinline__ void absorb_rows(const AbsorbArgs& a, int j, int b, int z,
                                            float (*qs)[2 * kMaxHalfDim]) {
  const int tid = threadIdx.x;
  const int g = j / a.s, jl = j % a.s;
  const int ncc = a.d / 8, rows = kThreads / ncc;
  const int cc = tid % ncc, kr = tid / ncc;
  const int k0 = z * rows * kAbsRowsPer + kr;
  const T* col = static_cast<const T*>(a.b_k) + static_cast<size_t>(g) * a.r * a.Dg + jl * a.d +
                 8 * cc;
  float v[kAbsRowsPer][8];
#pragma unroll
  for (int i = 0; i < kAbsRowsPer; ++i)
    load8_f32(col + static_cast<size_t>(min(k0 + i * rows, a.r - 1)) * a.Dg, v[i]);
  for (int h0 = 0; h0 < a.gqa; h0 += kAbsHeadChunk) {
    const int nh = min(kAbsHeadChunk, a.gqa - h0);
    const int head0 = j * a.gqa + h0;
    __syncthreads();
    for (int e = tid; e < nh * a.d; e += kThreads) {
      const int hh = e / a.d, c = e % a.d;
      qs[hh][c] = load_f32(static_cast<const T*>(a.q),
                           (static_cast<size_t>(b) * a.Hq + head0 + hh) * a.d + c);
    }
    __syncthreads();
    for (int hh = 0; hh < nh; ++hh) {
      const float4 q0 = *reinterpret_cast<const float4*>(&qs[hh][8 * cc]);
      const float4 q1 = *reinterpret_cast<const float4*>(&qs[hh][8 * cc + 4]);
      float s[kAbsRowsPer];
#pragma unroll
      for (int i = 0; i < kAbsRowsPer; ++i) {
        float t = q0.x * v[i][0];
        t = fmaf(q0.y, v[i][1], t); t = fmaf(q0.z, v[i][2], t); t = fmaf(q0.w, v[i][3], t);
        t = fmaf(q1.x, v[i][4], t); t = fmaf(q1.y, v[i][5], t); t = fmaf(q1.z, v[i][6], t);
        s[i] = fmaf(q1.w, v[i][7], t);
      }
      for (int off = 1; off < ncc; off <<= 1)
#pragma unroll
        for (int i = 0; i < kAbsRowsPer; ++i) s[i] += __shfl_xor(s[i], off);
      if (cc == 0) {
        float* dst = a.qt + (static_cast<size_t>(b) * a.Hq + head0 + hh) * a.r;
#pragma unroll
        for (int i = 0; i < kAbsRowsPer; ++i)
          if (k0 + i * rows < a.r) dst[k0 + i * rows] = s[i] * a.scale_log2;
      }
    }
  }
}

}  // namespace palu
