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
// query heads (up to 16), so every latent byte is read from HBM exactly once.
// Its four waves take the split's 16-token tiles round-robin (adjacent tiles
// stream together, which measured ~13% faster than contiguous quarters per
// wave) and combine their softmax states in LDS at the end. Per tile:
//   scores  S^T[16 tok x 16 heads] = H_k[16 x r] * Q~^T, bf16 MFMA 16x16x32,
//           q~ split as hi + lo bf16 (two MFMAs, ~16 bits kept), read from LDS;
//   softmax online, base 2, per head, with a lazy running max (the stored max
//           moves only when a tile exceeds it by kLazy, so most tiles skip the
//           rescale; the result is exact either way);
//   values  U^T[r x 16 heads] += H_v^T[r x 16 tok] * P^T, bf16 MFMA 16x16x16
//           with P split as hi + lo bf16. The tile's value latents go through
//           a wave-private LDS tile so each lane can gather one latent column
//           over four tokens (the MFMA contracts over tokens); groups of
//           four rows are offset by 32 bytes so those gathers hit distinct
//           banks.
// Lane layouts (wave64): 16x16x32 lane l holds A[l%16][k-slot l/16] and
// B[k-slot l/16][l%16], eight bf16 each; 16x16x16 the same with four; the
// result holds D[4*(l/16)+i][l%16]. A score tile leaves lane l with tokens
// 4*(l/16)+i of head l%16, which is exactly the 16x16x16 k-slot of P^T, so the
// weights never leave their lane.
// Loads: 16-byte global loads; H_k in the MFMA operand pattern (row l%16),
// H_v as contiguous 1 KiB per instruction; a ring of register buffers per wave
// keeps the next tiles in flight while one is consumed. Rows past the split's end are
// clamped to its last valid row and masked, so nothing outside [t0, len) is
// ever read.
#include <math.h>

#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLazy = 8.0f;   // log2 units: p <= 2^8 between rescales
constexpr int kTile = 16;       // tokens per tile
#ifndef ABS_WAVES
#define ABS_WAVES 4     // waves per workgroup (one per SIMD; measured better than 8)
#endif

constexpr int kWaves = ABS_WAVES;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

// q~ in LDS as the score MFMA's B operand: [hi|lo][head][k] bf16; rows padded
// by 16 elements (32 bytes: a row stride of 32 mod 64 bytes keeps the 16
// heads' 16-byte reads free of bank conflicts on gfx950).
template <int R>
struct QTile {
  static constexpr int kStride = R + 16;
  uint16_t v[2][16][kStride];
};

// byte offset of (row, column byte) in a wave's value tile [16][R] bf16: each
// group of four rows is shifted by 32 bytes, so the four lane groups of a
// gather (rows 4*kb..4*kb+3, same columns) hit different banks while every
// address stays one per-lane base plus an immediate
template <int R>
__device__ __forceinline__ int vtile_off(int row, int cb) {
  return row * (2 * R) + (row >> 2) * 32 + cb;
}
template <int R>
constexpr int kVTileBytes = kTile * R * 2 + 3 * 32;
// key tile rows padded by 32 bytes (a row stride of 32 mod 64 bytes keeps the
// 16 rows of an operand read free of bank conflicts on gfx950)
template <int R>
constexpr int kKStride = 2 * R + 32;
template <int R>
constexpr int kKTileBytes = kTile * kKStride<R>;

template <int R>
struct State {
  floatx4 acc[R / 16];   // U^T: r = 16*rb + 4*(lane/16) + i, head lane%16
  float m;               // stored running max (log2 units) of head lane%16
  float l;               // this lane's share of the running sum
};

// scores of a tile (log2 units), masked past t1
template <int R>
__device__ __forceinline__ floatx4 scores(const char* kt, const QTile<R>& qs, int tok0, int t1,
                                          int lane) {
  const int ln = lane & 15, kb = lane >> 4;
  // four independent accumulators (hi/lo x even/odd chunk) keep the MFMA
  // dependency chains short; they are added at the end
  floatx4 acc4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc4[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < R / 32; ++c) {
    const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(kt + ln * kKStride<R> + 2 * (32 * c + 8 * kb)));
    const bf16x8 qh = as_bf16x8(*reinterpret_cast<const uint4*>(&qs.v[0][ln][32 * c + 8 * kb]));
    const bf16x8 ql = as_bf16x8(*reinterpret_cast<const uint4*>(&qs.v[1][ln][32 * c + 8 * kb]));
    acc4[2 * (c & 1)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh, acc4[2 * (c & 1)], 0, 0, 0);
    acc4[2 * (c & 1) + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql, acc4[2 * (c & 1) + 1], 0, 0, 0);
  }
  floatx4 s = (acc4[0] + acc4[2]) + (acc4[1] + acc4[3]);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (tok0 + 4 * kb + i >= t1) s[i] = -INFINITY;
  return s;
}

// online softmax update and the value product from the staged LDS tile
template <int R>
__device__ __forceinline__ void softmax_values(State<R>& st, floatx4 s, const char* vt, int lane) {
  const int ln = lane & 15, kb = lane >> 4;
  float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (__any(mx > st.m + kLazy)) {
    const float mn = fmaxf(st.m, mx);
    const float alpha = exp2f(st.m - mn);
    st.m = mn;
    st.l *= alpha;
#pragma unroll
    for (int rb = 0; rb < R / 16; ++rb) st.acc[rb] *= alpha;
  }
  // P^T operand: k-slot e of lane group kb is token 4*kb + e; hi + lo bf16
  short4v ph, pl;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float p = exp2f(s[e] - st.m);
    st.l += p;
    const float hi = __uint_as_float(__float_as_uint(p) & 0xffff0000u);
    ph[e] = static_cast<short>(__float_as_uint(hi) >> 16);
    pl[e] = static_cast<short>(f32_to_bf16_rne(p - hi));
  }
  // values: gather H_v^T[16*rb + ln][tokens 4*kb .. 4*kb+3] from the LDS tile
  // (four row blocks at a time, hi parts first: an MFMA never waits on the one
  // just before it)
  constexpr int kU = R / 16 < 4 ? R / 16 : 4;            // R / 16 is a multiple
  const char* vb = vt + vtile_off<R>(4 * kb, 2 * ln);
#pragma unroll
  for (int rb0 = 0; rb0 < R / 16; rb0 += kU) {
    short4v a[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        a[u][e] = *reinterpret_cast<const short*>(vb + e * (2 * R) + 32 * (rb0 + u));
#pragma unroll
    for (int u = 0; u < kU; ++u)
      st.acc[rb0 + u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[u], ph, st.acc[rb0 + u], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < kU; ++u)
      st.acc[rb0 + u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[u], pl, st.acc[rb0 + u], 0, 0, 0);
  }
}

// Two blocks of 16 query heads from the same tile (groups of 17..32 heads):
// each K chunk read from LDS feeds both blocks' score MFMAs, and each value
// gather both blocks' value MFMAs, so a latent byte is read once per
// workgroup for all its heads.
template <int R>
__device__ __forceinline__ void scores2(const char* kt, const QTile<R>* qs, int tok0, int t1,
                                        int lane, floatx4 (&s)[2]) {
  const int ln = lane & 15, kb = lane >> 4;
  floatx4 acc4[2][4];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc4[hb][q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < R / 32; ++c) {
    const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(kt + ln * kKStride<R> + 2 * (32 * c + 8 * kb)));
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const bf16x8 qh = as_bf16x8(*reinterpret_cast<const uint4*>(&qs[hb].v[0][ln][32 * c + 8 * kb]));
      const bf16x8 ql = as_bf16x8(*reinterpret_cast<const uint4*>(&qs[hb].v[1][ln][32 * c + 8 * kb]));
      acc4[hb][2 * (c & 1)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh, acc4[hb][2 * (c & 1)], 0, 0, 0);
      acc4[hb][2 * (c & 1) + 1] =
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql, acc4[hb][2 * (c & 1) + 1], 0, 0, 0);
    }
  }
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    s[hb] = (acc4[hb][0] + acc4[hb][2]) + (acc4[hb][1] + acc4[hb][3]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (tok0 + 4 * kb + i >= t1) s[hb][i] = -INFINITY;
  }
}

template <int R>
__device__ __forceinline__ void softmax_values2(State<R> (&st)[2], const floatx4 (&s)[2],
                                                const char* vt, int lane) {
  const int ln = lane & 15, kb = lane >> 4;
  short4v ph[2], pl[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    float mx = fmaxf(fmaxf(s[hb][0], s[hb][1]), fmaxf(s[hb][2], s[hb][3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__any(mx > st[hb].m + kLazy)) {
      const float mn = fmaxf(st[hb].m, mx);
      const float alpha = exp2f(st[hb].m - mn);
      st[hb].m = mn;
      st[hb].l *= alpha;
#pragma unroll
      for (int rb = 0; rb < R / 16; ++rb) st[hb].acc[rb] *= alpha;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = exp2f(s[hb][e] - st[hb].m);
      st[hb].l += p;
      const float hi = __uint_as_float(__float_as_uint(p) & 0xffff0000u);
      ph[hb][e] = static_cast<short>(__float_as_uint(hi) >> 16);
      pl[hb][e] = static_cast<short>(f32_to_bf16_rne(p - hi));
    }
  }
  constexpr int kU = R / 16 < 4 ? R / 16 : 4;
  const char* vb = vt + vtile_off<R>(4 * kb, 2 * ln);
#pragma unroll
  for (int rb0 = 0; rb0 < R / 16; rb0 += kU) {
    short4v a[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        a[u][e] = *reinterpret_cast<const short*>(vb + e * (2 * R) + 32 * (rb0 + u));
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int u = 0; u < kU; ++u)
        st[hb].acc[rb0 + u] =
            __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[u], ph[hb], st[hb].acc[rb0 + u], 0, 0, 0);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int u = 0; u < kU; ++u)
        st[hb].acc[rb0 + u] =
            __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[u], pl[hb], st[hb].acc[rb0 + u], 0, 0, 0);
  }
}

// NHB: blocks of 16 query heads a workgroup serves (one, or two for groups of
// more than 16 heads)
template <int R, int NHB>
struct Smem {
  QTile<R> q[NHB];
  union {
    struct {                                         // per-wave tiles (streaming)
      char kt[kWaves][kKTileBytes<R>];
      char vt[kWaves][kVTileBytes<R>];
    } t;
    struct {                                         // every wave's softmax state
      float acc[kWaves][4 * (R / 16)][64];
      float m[kWaves][64], l[kWaves][64];
    } x;
  } u;
};

template <int R, int NHB, bool kShared>
__global__ __launch_bounds__(64 * kWaves, 1) void split_absorbed_mfma_kernel(DecodeParams p) {
  // a workgroup serves NHB blocks of 16 query heads; heads of a group beyond
  // them go to further head slices (workgroups that read the same latents,
  // shared through one XCD's L2)
  constexpr int kHS = 16 * NHB;
  const int nslice = (p.nq + kHS - 1) / kHS;
  const SplitUnit un = split_unit(p.n_split, p.G, p.B, nslice);
  if (!un.live) return;
  const int split = un.split, g = un.g, b = un.b;
  const int hq0 = un.hs * kHS;                           // first query head of the slice
  int nqs[NHB];                                          // query heads of each block (<= 0: none)
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) nqs[hb] = min(16, p.nq - hq0 - 16 * hb);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, kb = lane >> 4;
  const int n = clamp_len(p.lens, b, p.L);
  const int s0 = split * p.split_tokens;
  if (s0 >= n) return;                                   // whole workgroup
  const int t1 = min(n, s0 + p.split_tokens);
  const int last = t1 - 1;

  __shared__ Smem<R, NHB> sm;
  const size_t row0 = (static_cast<size_t>(b) * p.G + g) * p.L;
  const uint16_t* Hk = static_cast<const uint16_t*>(p.h_k) + row0 * R;
  const uint16_t* Hv = static_cast<const uint16_t*>(p.h_v) + row0 * R;

  // 16-token tiles dealt round-robin: wave w takes tiles w, w+4, ...; the
  // registers of a tile are refilled with the next one as soon as the tile
  // is copied into the wave's LDS tiles; loads past the end read the last
  // valid row again (cached, never out of range)
  const int ntiles = (t1 - s0 + kTile - 1) / kTile;
  const int mine = (ntiles - wave + kWaves - 1) / kWaves;   // may be 0
  const int step = kTile * kWaves;
  const int first = s0 + kTile * wave;
  // one tile in registers (vector types: arrays of uint4 here ended up in
  // scratch memory)
  typedef uint32_t u32v __attribute__((ext_vector_type(R / 8)));
  auto fetch = [&](u32v& nkv, u32v& nvv, int tok0) {
    const int rk = min(tok0 + ln, last);
#pragma unroll
    for (int c = 0; c < R / 32; ++c) {
      const uint4 t = load_tile16<kShared>(Hk + static_cast<size_t>(rk) * R + 32 * c + 8 * kb);
      nkv[4 * c] = t.x; nkv[4 * c + 1] = t.y; nkv[4 * c + 2] = t.z; nkv[4 * c + 3] = t.w;
    }
#pragma unroll
    for (int q = 0; q < R / 32; ++q) {
      const int flat = q * 1024 + lane * 16;          // byte within the tile's 16 rows
      const int rv = min(tok0 + flat / (2 * R), last);
      const uint4 t = load_tile16<kShared>(Hv + static_cast<size_t>(rv) * R + (flat % (2 * R)) / 2);
      nvv[4 * q] = t.x; nvv[4 * q + 1] = t.y; nvv[4 * q + 2] = t.z; nvv[4 * q + 3] = t.w;
    }
  };
  // the first tile's loads go out before anything waits
  u32v ka, va;
  if (mine > 0) fetch(ka, va, first);

  // absorbed queries of the group's heads, split hi/lo bf16 (padding heads
  // are 0): all of a thread's loads are issued before the first is used
  {
    constexpr int kQ = 16 * R / (64 * kWaves);
    const float* qrow = p.qt + (static_cast<size_t>(b) * p.Hq + g * p.nq + hq0) * R;
    float qx[NHB][kQ];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int nh = nqs[hb];                            // a block without heads reads nothing
#pragma unroll
      for (int u = 0; u < kQ; ++u) {
        const int e = threadIdx.x + u * 64 * kWaves, hd = e / R, k = e % R;
        if constexpr (NHB == 1) qx[hb][u] = qrow[min(hd, nh - 1) * R + k];   // nh >= 1
        else qx[hb][u] = nh > 0 ? qrow[(16 * hb + min(hd, nh - 1)) * R + k] : 0.f;
      }
    }
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int u = 0; u < kQ; ++u) {
        const int e = threadIdx.x + u * 64 * kWaves, hd = e / R, k = e % R;
        const float x = hd < nqs[hb] ? qx[hb][u] : 0.f;
        const float hi = __uint_as_float(__float_as_uint(x) & 0xffff0000u);
        sm.q[hb].v[0][hd][k] = static_cast<uint16_t>(__float_as_uint(hi) >> 16);
        sm.q[hb].v[1][hd][k] = f32_to_bf16_rne(x - hi);
      }
  }
  barrier_lds();            // the first tiles stay in flight

  State<R> st[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    st[hb].m = -INFINITY;
    st[hb].l = 0.f;
#pragma unroll
    for (int rb = 0; rb < R / 16; ++rb) st[hb].acc[rb] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  if (mine > 0) {
    char* kt = sm.u.t.kt[wave];
    char* vt = sm.u.t.vt[wave];
    auto stage = [&](const u32v& nkv, const u32v& nvv) {
#pragma unroll
      for (int c = 0; c < R / 32; ++c)
        *reinterpret_cast<uint4*>(kt + ln * kKStride<R> + 2 * (32 * c + 8 * kb)) =
            uint4{nkv[4 * c], nkv[4 * c + 1], nkv[4 * c + 2], nkv[4 * c + 3]};
#pragma unroll
      for (int q = 0; q < R / 32; ++q) {
        const int flat = q * 1024 + lane * 16;
        *reinterpret_cast<uint4*>(vt + vtile_off<R>(flat / (2 * R), flat % (2 * R))) =
            uint4{nvv[4 * q], nvv[4 * q + 1], nvv[4 * q + 2], nvv[4 * q + 3]};
      }
    };
    for (int j = 0; j < mine; ++j) {
      stage(ka, va);
      fetch(ka, va, first + step * (j + 1));
      if constexpr (NHB == 1) {
        const floatx4 s = scores<R>(kt, sm.q[0], first + step * j, t1, lane);
        softmax_values<R>(st[0], s, vt, lane);
      } else {
        floatx4 s[2];
        scores2<R>(kt, sm.q, first + step * j, t1, lane, s);
        softmax_values2<R>(st, s, vt, lane);
      }
    }
  }

  // merge: after a barrier (the tiles' space is reused) every wave publishes
  // its state, then after one more every thread combines one (head, lane
  // group, row block) slice of all of them (a side that saw no token has m =
  // -inf and weight 0) and writes it. [slot][value][lane] keeps consecutive
  // lanes on consecutive banks. Head blocks go one after the other through
  // the same space.
  const int th = threadIdx.x;
  const int cln = th % 16, ckb = (th / 16) % 4, crq = th / 64;   // head, lane group, first row block
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < R / 16; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.u.x.acc[wave][4 * rb + i][lane] = st[hb].acc[rb][i];
    sm.u.x.m[wave][lane] = st[hb].m;
    sm.u.x.l[wave][lane] = st[hb].l;
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.u.x.m[w][cln]);
    float aw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm.u.x.m[w][cln];
      aw[w] = mw == -INFINITY ? 0.f : exp2f(mw - M);
    }
    if constexpr (NHB == 1) {
      if (cln >= nqs[0]) return;
    } else {
      if (cln >= nqs[hb]) continue;                      // the next block's barriers follow
    }
    {
      const int head = g * p.nq + hq0 + 16 * hb + cln;
      const size_t slot = (static_cast<size_t>(b) * p.Hq + head) * p.n_split + split;
      if (th < 16) {
        float l = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          l += aw[w] * ((sm.u.x.l[w][cln] + sm.u.x.l[w][16 + cln]) +
                        (sm.u.x.l[w][32 + cln] + sm.u.x.l[w][48 + cln]));
        p.part_ml[slot * 2] = M;
        p.part_ml[slot * 2 + 1] = l;
      }
      // latents 16 rb + 4 ckb + i of head cln
      float* u = p.part_u + slot * R;
      for (int rb = crq; rb < R / 16; rb += kWaves) {
        float4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          v.x = fmaf(aw[w], sm.u.x.acc[w][4 * rb + 0][16 * ckb + cln], v.x);
          v.y = fmaf(aw[w], sm.u.x.acc[w][4 * rb + 1][16 * ckb + cln], v.y);
          v.z = fmaf(aw[w], sm.u.x.acc[w][4 * rb + 2][16 * ckb + cln], v.z);
          v.w = fmaf(aw[w], sm.u.x.acc[w][4 * rb + 3][16 * ckb + cln], v.w);
        }
        *reinterpret_cast<float4*>(u + 16 * rb + 4 * ckb) = v;
      }
    }
  }
}

}  // namespace

bool absorbed_mfma_supported(const DecodeParams& p, int dtype) {
  return dtype == 1 && (p.r == 32 || p.r == 64 || p.r == 128 || p.r == 256);
}

int absorbed_head_slices(int nq) { return (nq + 15) / 16; }

int absorbed_mfma_slices(int nq) { return nq > 16 ? (nq + 31) / 32 : 1; }

template <int R, int NHB>
hipError_t launch_blocks(const DecodeParams& p, hipStream_t st) {
  const int nslice = (p.nq + 16 * NHB - 1) / (16 * NHB);
  if (nslice == 1) {
    split_absorbed_mfma_kernel<R, NHB, false><<<dim3(p.n_split, p.G, p.B), 64 * kWaves, 0, st>>>(p);
  } else {
    const long ids = split_unit_ids(p.n_split, p.G, p.B, nslice);
    if (ids == 0) return hipErrorInvalidValue;
    split_absorbed_mfma_kernel<R, NHB, true>
        <<<dim3(static_cast<unsigned>(ids)), 64 * kWaves, 0, st>>>(p);
  }
  return hipGetLastError();
}

// groups of more than 16 query heads: two head blocks a workgroup
template <int R>
hipError_t launch_rank(const DecodeParams& p, hipStream_t st) {
  return p.nq > 16 ? launch_blocks<R, 2>(p, st) : launch_blocks<R, 1>(p, st);
}

hipError_t launch_split_absorbed_mfma(const DecodeParams& p, hipStream_t st) {
  switch (p.r) {
    case 32: return launch_rank<32>(p, st);
    case 64: return launch_rank<64>(p, st);
    case 128: return launch_rank<128>(p, st);
    case 256: return launch_rank<256>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace palu
