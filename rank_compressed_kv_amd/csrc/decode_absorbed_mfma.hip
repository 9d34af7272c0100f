// Context-split decode kernel for the absorbed-key mode, bf16 latents, on the
// gfx950 matrix cores.
//
// Method (Palu author response on OpenReview, "Why Palu Requires Fewer Global
// Memory Access" and the clarification of W1): without a rotary embedding the
// reconstruction matrix of the keys moves onto the query, q~ = q B_k^T, so the
// score of token t is <q~, h_k[t]> and no key is rebuilt; the value path sums
// value latents with the attention weights and applies B_v later (merge pass).
//
// One wave owns one (batch, group, context split) and all of the group's query
// heads (up to 16), so every latent byte is read from HBM exactly once. Per
// 16-token tile:
//   scores  S^T[16 tok x 16 heads] = H_k[16 x r] * Q~^T        bf16 MFMA 16x16x32,
//           q~ split as hi + lo bf16 (two MFMAs) so the query keeps ~16 bits;
//   softmax online, base 2, per head, with a lazy running max (the stored max
//           moves only when a tile exceeds it by kLazy, so most tiles skip the
//           rescale; the result is exact either way);
//   values  U^T[r x 16 heads] += H_v^T[r x 16 tok] * P^T       fp32 MFMA 16x16x4:
//           each lane feeds one bf16->fp32 latent per MFMA, so the value latents
//           are used straight from their natural [token][r] rows, no transpose,
//           and P stays in fp32.
// Lane layouts (wave64): for 16x16x32 bf16, lane l holds A[l%16][k-slot(l/16)]
// and B[k-slot(l/16)][l%16] (8 values each); for 16x16x4 fp32 one value each
// with k = l/16; the result holds D[4*(l/16)+i][l%16], i < 4.
// Loads: 16-byte global loads in the natural cache layout, two tiles in flight
// (ping-pong register buffers). Rows past the split's end are clamped to its
// last valid row and masked, so nothing outside [t0, len) is ever read.
#include <math.h>

#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLazy = 8.0f;   // log2 units: p <= 2^8 between rescales

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

template <int R>
struct Tile {
  uint4 k[R / 32];        // H_k row (lane%16): 8 latents at 32c + 8*(lane/16)
  uint4 v[4][R / 128];    // H_v rows 4*(lane/16)+i: 8 latents at 128h + 8*(lane%16)
};

template <int R>
__device__ __forceinline__ void load_tile(Tile<R>& tl, const uint16_t* Hk, const uint16_t* Hv,
                                          int tok0, int last, int ln, int kb) {
  const int rk = min(tok0 + ln, last);
#pragma unroll
  for (int c = 0; c < R / 32; ++c)
    tl.k[c] = *reinterpret_cast<const uint4*>(Hk + static_cast<size_t>(rk) * R + 32 * c + 8 * kb);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rv = min(tok0 + 4 * kb + i, last);
#pragma unroll
    for (int h = 0; h < R / 128; ++h)
      tl.v[i][h] = *reinterpret_cast<const uint4*>(Hv + static_cast<size_t>(rv) * R + 128 * h + 8 * ln);
  }
}

template <int R>
struct State {
  floatx4 acc[R / 128][8];   // U^T: r = 128h + 8*(4*(lane/16)+i) + j, head lane%16
  float m;                   // stored running max (log2 units) of head lane%16
  float l;                   // this lane's share of the running sum
};

template <int R>
__device__ __forceinline__ void compute_tile(State<R>& st, const Tile<R>& tl, const bf16x8* qhi,
                                             const bf16x8* qlo, int tok0, int t1, int kb) {
  floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < R / 32; ++c) {
    const bf16x8 a = as_bf16x8(tl.k[c]);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qhi[c], s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qlo[c], s, 0, 0, 0);
  }
  // s[i]: score of token tok0 + 4*kb + i for head lane%16
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (tok0 + 4 * kb + i >= t1) s[i] = -INFINITY;
  float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (__any(mx > st.m + kLazy)) {
    const float mn = fmaxf(st.m, mx);
    const float alpha = exp2f(st.m - mn);
    st.m = mn;
    st.l *= alpha;
#pragma unroll
    for (int h = 0; h < R / 128; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) st.acc[h][j] *= alpha;
  }
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = exp2f(s[i] - st.m);
    st.l += p[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < R / 128; ++h) {
      const uint32_t w[4] = {tl.v[i][h].x, tl.v[i][h].y, tl.v[i][h].z, tl.v[i][h].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a = (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
        st.acc[h][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, p[i], st.acc[h][j], 0, 0, 0);
      }
    }
  }
}

template <int R>
__global__ __launch_bounds__(64) void split_absorbed_mfma_kernel(DecodeParams p) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, ln = lane & 15, kb = lane >> 4;
  const int n = clamp_len(p.lens, b, p.L);
  const int t0 = split * p.split_tokens;
  if (t0 >= n) return;
  const int t1 = min(n, t0 + p.split_tokens);
  const int last = t1 - 1;

  // absorbed queries of the group's heads (B operand), hi/lo bf16 split
  bf16x8 qhi[R / 32], qlo[R / 32];
  {
    const bool valid = ln < p.nq;
    const float* qt = p.qt + (static_cast<size_t>(b) * p.Hq + g * p.nq + (valid ? ln : 0)) * R;
#pragma unroll
    for (int c = 0; c < R / 32; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = valid ? qt[32 * c + 8 * kb + e] : 0.f;
        const float hi = __uint_as_float(__float_as_uint(x) & 0xffff0000u);
        const uint16_t lo = f32_to_bf16_rne(x - hi);
        qhi[c][e] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(__float_as_uint(hi) >> 16));
        qlo[c][e] = __builtin_bit_cast(__bf16, lo);
      }
    }
  }

  const size_t row0 = (static_cast<size_t>(b) * p.G + g) * p.L;
  const uint16_t* Hk = static_cast<const uint16_t*>(p.h_k) + row0 * R;
  const uint16_t* Hv = static_cast<const uint16_t*>(p.h_v) + row0 * R;

  State<R> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int h = 0; h < R / 128; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[h][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = (t1 - t0 + 15) / 16;
  Tile<R> ta, tb;
  load_tile<R>(ta, Hk, Hv, t0, last, ln, kb);
  for (int it = 0; it < ntiles; it += 2) {
    load_tile<R>(tb, Hk, Hv, t0 + 16 * (it + 1), last, ln, kb);
    compute_tile<R>(st, ta, qhi, qlo, t0 + 16 * it, t1, kb);
    if (it + 1 >= ntiles) break;
    load_tile<R>(ta, Hk, Hv, t0 + 16 * (it + 2), last, ln, kb);
    compute_tile<R>(st, tb, qhi, qlo, t0 + 16 * (it + 1), t1, kb);
  }

  // head totals: sum the four lane groups' shares
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (ln >= p.nq) return;
  const int head = g * p.nq + ln;
  const size_t slot = (static_cast<size_t>(b) * p.Hq + head) * p.n_split + split;
  if (kb == 0) {
    p.part_ml[slot * 2] = st.m;
    p.part_ml[slot * 2 + 1] = l;
  }
  float* u = p.part_u + slot * R;
#pragma unroll
  for (int h = 0; h < R / 128; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r0 = 128 * h + 8 * (4 * kb + i);
      float4 lo4 = {st.acc[h][0][i], st.acc[h][1][i], st.acc[h][2][i], st.acc[h][3][i]};
      float4 hi4 = {st.acc[h][4][i], st.acc[h][5][i], st.acc[h][6][i], st.acc[h][7][i]};
      *reinterpret_cast<float4*>(u + r0) = lo4;
      *reinterpret_cast<float4*>(u + r0 + 4) = hi4;
    }
}

}  // namespace

bool absorbed_mfma_supported(const DecodeParams& p, int dtype) {
  return dtype == 1 && (p.r == 128 || p.r == 256) && p.nq <= 16;
}

hipError_t launch_split_absorbed_mfma(const DecodeParams& p, hipStream_t st) {
  const dim3 grid(p.n_split, p.G, p.B);
  if (p.r == 128) split_absorbed_mfma_kernel<128><<<grid, 64, 0, st>>>(p);
  else if (p.r == 256) split_absorbed_mfma_kernel<256><<<grid, 64, 0, st>>>(p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace palu
