// Context-split decode kernel for the absorbed-key mode, bf16 latents, on the
// gfx950 matrix cores.
//
// Method (Palu author response on OpenReview, "Why Palu Requires Fewer Global
// Memory Access" and the clarification of W1): without a rotary embedding the
// reconstruction matrix of the keys moves onto the query, q~ = q B_k^T, so the
// score of token t is <q~, h_k[t]> and no key is rebuilt; the value path sums
// value latents with the attention weights and applies B_v later (merge pass).
//
// One workgroup owns one (batch, group, context split) and all of the group's
// query heads (up to 16), so every latent byte is read from HBM exactly once;
// its four waves take the split's 16-token tiles round-robin (adjacent tiles
// stream together, which measured ~13% faster than giving each wave a
// contiguous quarter) and combine their softmax states in LDS at the end.
// Per tile:
//   scores  S^T[16 tok x 16 heads] = H_k[16 x r] * Q~^T        bf16 MFMA 16x16x32,
//           q~ split as hi + lo bf16 (two MFMAs) so the query keeps ~16 bits,
//           read from LDS;
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
// per wave while a third is consumed (three register buffers). Rows past the split's end are clamped to its
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

// Absorbed queries in LDS as the MFMA B operand: [hi|lo][head][k] bf16, rows
// padded by 8 elements so the 16 heads' 16-byte reads spread over the banks.
template <int R>
struct QTile {
  static constexpr int kStride = R + 8;
  uint16_t v[2][16][kStride];
};

template <int R>
__device__ __forceinline__ void compute_tile(State<R>& st, const Tile<R>& tl, const QTile<R>& qs,
                                             int tok0, int t1, int ln, int kb) {
  floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < R / 32; ++c) {
    const bf16x8 a = as_bf16x8(tl.k[c]);
    const bf16x8 qh = as_bf16x8(*reinterpret_cast<const uint4*>(&qs.v[0][ln][32 * c + 8 * kb]));
    const bf16x8 ql = as_bf16x8(*reinterpret_cast<const uint4*>(&qs.v[1][ln][32 * c + 8 * kb]));
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh, s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql, s, 0, 0, 0);
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

constexpr int kWaves = 4;   // waves per workgroup; tiles are dealt round-robin

template <int R>
__global__ __launch_bounds__(64 * kWaves) void split_absorbed_mfma_kernel(DecodeParams p) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, kb = lane >> 4;
  const int n = clamp_len(p.lens, b, p.L);
  const int s0 = split * p.split_tokens;
  if (s0 >= n) return;                                   // whole workgroup
  const int t1 = min(n, s0 + p.split_tokens);
  const int last = t1 - 1;

  // absorbed queries of the group's heads, split hi/lo bf16 (padding heads are 0)
  __shared__ QTile<R> qs;
  for (int e = threadIdx.x; e < 16 * R; e += 64 * kWaves) {
    const int hd = e / R, k = e % R;
    const float x = hd < p.nq ? p.qt[(static_cast<size_t>(b) * p.Hq + g * p.nq + hd) * R + k] : 0.f;
    const float hi = __uint_as_float(__float_as_uint(x) & 0xffff0000u);
    qs.v[0][hd][k] = static_cast<uint16_t>(__float_as_uint(hi) >> 16);
    qs.v[1][hd][k] = f32_to_bf16_rne(x - hi);
  }
  __syncthreads();

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

  // tiles of 16 tokens dealt round-robin: wave w takes tiles w, w+4, ..., so the
  // four waves stream adjacent 8 KiB blocks together. Three register buffers:
  // two tiles in flight while one is consumed; loads past the end read the last
  // valid row again (cached, never out of range).
  const int ntiles = (t1 - s0 + 15) / 16;
  const int mine = (ntiles - wave + kWaves - 1) / kWaves;  // may be 0
  if (mine > 0) {
    const int step = 16 * kWaves;
    const int first = s0 + 16 * wave;
    Tile<R> ta, tb, tc;
    load_tile<R>(ta, Hk, Hv, first, last, ln, kb);
    load_tile<R>(tb, Hk, Hv, first + step, last, ln, kb);
    for (int it = 0; it < mine; it += 3) {
      load_tile<R>(tc, Hk, Hv, first + step * (it + 2), last, ln, kb);
      compute_tile<R>(st, ta, qs, first + step * it, t1, ln, kb);
      if (it + 1 >= mine) break;
      load_tile<R>(ta, Hk, Hv, first + step * (it + 3), last, ln, kb);
      compute_tile<R>(st, tb, qs, first + step * (it + 1), t1, ln, kb);
      if (it + 2 >= mine) break;
      load_tile<R>(tb, Hk, Hv, first + step * (it + 4), last, ln, kb);
      compute_tile<R>(st, tc, qs, first + step * (it + 2), t1, ln, kb);
    }
  }

  // merge the waves' states in LDS: waves 1..3 publish, wave 0 combines.
  // Layout [wave][value][lane] keeps consecutive lanes on consecutive banks.
  constexpr int kVals = 4 * 8 * (R / 128);
  __shared__ float xacc[kWaves - 1][kVals][64];
  __shared__ float xm[kWaves - 1][64], xl[kWaves - 1][64];
  if (wave > 0) {
    int v = 0;
#pragma unroll
    for (int h = 0; h < R / 128; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) xacc[wave - 1][v++][lane] = st.acc[h][j][i];
    xm[wave - 1][lane] = st.m;
    xl[wave - 1][lane] = st.l;
  }
  __syncthreads();
  if (wave > 0) return;
  float mw[kWaves - 1];
  float M = st.m;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) {
    mw[w] = xm[w][lane];
    M = fmaxf(M, mw[w]);
  }
  const float a0 = exp2f(st.m - M);   // wave 0 always has a tile: M is finite
  float wgt[kWaves - 1];
  float l = st.l * a0;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) {
    wgt[w] = exp2f(mw[w] - M);         // 0 for a wave that saw no token
    l += wgt[w] * xl[w][lane];
  }
  {
    int v = 0;
#pragma unroll
    for (int h = 0; h < R / 128; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i, ++v) {
          float a = st.acc[h][j][i] * a0;
#pragma unroll
          for (int w = 0; w < kWaves - 1; ++w) a = fmaf(wgt[w], xacc[w][v][lane], a);
          st.acc[h][j][i] = a;
        }
  }

  // head totals: sum the four lane groups' shares
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (ln >= p.nq) return;
  const int head = g * p.nq + ln;
  const size_t slot = (static_cast<size_t>(b) * p.Hq + head) * p.n_split + split;
  if (kb == 0) {
    p.part_ml[slot * 2] = M;
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
  if (p.r == 128) split_absorbed_mfma_kernel<128><<<grid, 64 * kWaves, 0, st>>>(p);
  else if (p.r == 256) split_absorbed_mfma_kernel<256><<<grid, 64 * kWaves, 0, st>>>(p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace palu
