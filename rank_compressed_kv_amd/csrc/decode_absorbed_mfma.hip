// Context-split decode kernel for the absorbed-key mode on the gfx950 matrix
// cores: bf16 latents, or int8 latents with one scale per cached row.
//
// Method (Palu author response on OpenReview, "Why Palu Requires Fewer Global
// Memory Access" and the clarification of W1): without a rotary embedding the
// reconstruction matrix of the keys moves onto the query, q~ = q B_k^T, so the
// score of token t is <q~, h_k[t]> and no key is rebuilt; the value path sums
// value latents with the attention weights and applies B_v later (merge pass).
// The same kernel serves the uncompressed baseline (q~ = q, full K and V).
//
// One workgroup owns one (batch, group, context split) and 16 query heads of
// the group (groups with more heads get further head slices, whose workgroups
// read the same latents through one XCD's L2), so every latent byte is read
// from HBM once. Its four waves take the split's 16-token tiles round-robin
// (adjacent tiles stream together) and combine their softmax states in LDS at
// the end. Per tile:
//   scores  S^T[16 tok x 16 heads] = H_k[16 x r] * Q~^T, MFMA 16x16x32, q~
//           split as hi + lo (two MFMAs, ~16 bits kept), read from LDS;
//   softmax online, base 2, per head, with a lazy running max (the stored max
//           moves only when a tile exceeds it by kLazy, so most tiles skip the
//           rescale; the result is exact either way);
//   values  U^T[r x 16 heads] += H_v^T[r x 16 tok] * P^T, MFMA 16x16x16 with P
//           split as hi + lo. The value latents are gathered from a
//           wave-private LDS tile so each lane can take one latent column over
//           four tokens (the MFMA contracts over tokens); groups of four rows
//           are offset by 32 bytes so those gathers hit distinct banks.
// bf16 latents use bf16 MFMAs. int8 latents (code times the row's scale) are
// widened to fp16 (exact for |code| <= 127) as they are copied into the LDS
// tiles and use fp16 MFMAs: a tile's key scales multiply its scores, its value
// scales fold into the weights (p_t s_t), and the running sum l keeps p_t.
// To keep fp16 operands in range whatever the magnitudes, each head's q~ is
// divided by a power of two near its largest entry (undone on the scores)
// and the value scales by the split's largest one (undone on the partials).
// Lane layouts (wave64): 16x16x32 lane l holds A[l%16][k-slot l/16] and
// B[k-slot l/16][l%16], eight 16-bit values each; 16x16x16 the same with four;
// the result holds D[4*(l/16)+i][l%16]. A score tile leaves lane l with tokens
// 4*(l/16)+i of head l%16, which is exactly the 16x16x16 k-slot of P^T, so the
// weights never leave their lane.
// Loads: 16-byte non-temporal loads (the latents are read once) of the next
// tile into registers while the current one, already in LDS, is consumed.
// Rows past the split's end are clamped to its last valid row and masked, so
// nothing outside [t0, len) is ever read.
#include <math.h>

#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLazy = 8.0f;   // log2 units: p <= 2^8 between rescales
constexpr int kTile = 16;       // tokens per tile
#ifndef ABS_WAVES
#define ABS_WAVES 4     // waves per workgroup (one per SIMD; measured better than 8)
#endif
constexpr int kWaves = ABS_WAVES;

// x ~ hi + lo in two 16-bit floats (fp16 or bf16, nearest even each): the
// MFMA operand bits of both terms
template <bool kF16>
__device__ __forceinline__ void split16(float x, uint16_t& hi, uint16_t& lo) {
  if constexpr (kF16) {
    const _Float16 h = static_cast<_Float16>(x);
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, static_cast<_Float16>(x - static_cast<float>(h)));
  } else {
    const __bf16 h = static_cast<__bf16>(x);
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x - static_cast<float>(h)));
  }
}

// four int8 codes -> four fp16 values, exactly: with u = code + 128 (the byte
// XOR 0x80), the fp16 with bits 0x64uu is 1024 + u; one byte permute per pair
// of codes and one packed fp16 subtraction of 1152 give the codes
__device__ __forceinline__ uint2 i8x4_to_f16x4(uint32_t w) {
  const uint32_t x = w ^ 0x80808080u;
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);
  const half2v bias = {static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
  const half2v a = __builtin_bit_cast(half2v, lo) - bias;
  const half2v c = __builtin_bit_cast(half2v, hi) - bias;
  return uint2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, c)};
}

template <bool kF16>
__device__ __forceinline__ floatx4 mfma32(uint4 a, uint4 b, floatx4 c) {
  if constexpr (kF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                  __builtin_bit_cast(half8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <bool kF16>
__device__ __forceinline__ floatx4 mfma16(short4v a, short4v b, floatx4 c) {
  if constexpr (kF16)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4, a),
                                                 __builtin_bit_cast(half4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// q~ in LDS as the score MFMA's B operand: [hi|lo][head][k] 16-bit; rows padded
// by 8 elements so the 16 heads' 16-byte reads spread over the banks.
template <int R>
struct QTile {
  static constexpr int kStride = R + 8;
  uint16_t v[2][16][kStride];
};

// byte offset of (row, column byte) in a wave's value tile [16][R] (16-bit):
// each group of four rows is shifted by 32 bytes, so the four lane groups of a
// gather (rows 4*kb..4*kb+3, same columns) hit different banks while every
// address stays one per-lane base plus an immediate
template <int R>
__device__ __forceinline__ int vtile_off(int row, int cb) {
  return row * (2 * R) + (row >> 2) * 32 + cb;
}
template <int R>
constexpr int kVTileBytes = kTile * R * 2 + 3 * 32;
// key tile rows padded by 16 bytes: the 16 rows of an operand read start on
// different banks
template <int R>
constexpr int kKStride = 2 * R + 16;
template <int R>
constexpr int kKTileBytes = kTile * kKStride<R>;

template <int R>
struct State {
  floatx4 acc[R / 16];   // U^T: r = 16*rb + 4*(lane/16) + i, head lane%16
  float m;               // stored running max (log2 units) of head lane%16
  float l;               // this lane's share of the running sum
};

// scores of a tile (log2 units; int8: times the key scales), masked past t1
template <int R, bool kF16>
__device__ __forceinline__ floatx4 scores(const char* kt, const QTile<R>& qs, int tok0, int t1,
                                          int lane, floatx4 sk) {
  const int ln = lane & 15, kb = lane >> 4;
  // four independent accumulators (hi/lo x even/odd chunk) keep the MFMA
  // dependency chains short; they are added at the end
  floatx4 acc4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc4[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < R / 32; ++c) {
    const uint4 a = *reinterpret_cast<const uint4*>(kt + ln * kKStride<R> + 2 * (32 * c + 8 * kb));
    const uint4 qh = *reinterpret_cast<const uint4*>(&qs.v[0][ln][32 * c + 8 * kb]);
    const uint4 ql = *reinterpret_cast<const uint4*>(&qs.v[1][ln][32 * c + 8 * kb]);
    acc4[2 * (c & 1)] = mfma32<kF16>(a, qh, acc4[2 * (c & 1)]);
    acc4[2 * (c & 1) + 1] = mfma32<kF16>(a, ql, acc4[2 * (c & 1) + 1]);
  }
  floatx4 s = (acc4[0] + acc4[2]) + (acc4[1] + acc4[3]);
  if constexpr (kF16) s *= sk;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (tok0 + 4 * kb + i >= t1) s[i] = -INFINITY;
  return s;
}

// online softmax update and the value product from the staged LDS tile; sv
// (int8 latents) holds the value scales of the lane's four tokens
template <int R, bool kF16>
__device__ __forceinline__ void softmax_values(State<R>& st, floatx4 s, const char* vt, int lane,
                                               floatx4 sv) {
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
  // P^T operand: k-slot e of lane group kb is token 4*kb + e; hi + lo
  short4v ph, pl;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float pe = exp2f(s[e] - st.m);
    st.l += pe;
    uint16_t h, lo;
    split16<kF16>(kF16 ? pe * sv[e] : pe, h, lo);
    ph[e] = static_cast<short>(h);
    pl[e] = static_cast<short>(lo);
  }
  // values: gather H_v^T[16*rb + ln][tokens 4*kb .. 4*kb+3] from the LDS tile
  const char* vb = vt + vtile_off<R>(4 * kb, 2 * ln);
#pragma unroll
  for (int rb = 0; rb < R / 16; ++rb) {
    short4v a;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      a[e] = *reinterpret_cast<const short*>(vb + e * (2 * R) + 32 * rb);
    st.acc[rb] = mfma16<kF16>(a, ph, st.acc[rb]);
    st.acc[rb] = mfma16<kF16>(a, pl, st.acc[rb]);
  }
}

template <int R>
struct Smem {
  QTile<R> q;
  float qc[16];              // int8: power of two each head's q~ was divided by
  float svmax[kWaves];       // int8: each wave's largest value scale
  union {
    struct {                                         // per-wave tiles (streaming)
      char kt[kWaves][kKTileBytes<R>];
      char vt[kWaves][kVTileBytes<R>];
    } t;
    struct {                                         // softmax states (final merge)
      float acc[kWaves / 2][4 * (R / 16)][64];
      float m[kWaves / 2][64], l[kWaves / 2][64];
    } x;
  } u;
};

// st <- st (+) the state another wave published in slot w; a side that saw no
// token has m = -inf and weight 0
template <int R>
__device__ __forceinline__ void combine(State<R>& st, const Smem<R>& sm, int w, int lane) {
  const float mo = sm.u.x.m[w][lane];
  const float M = fmaxf(st.m, mo);
  const float a = st.m == -INFINITY ? 0.f : exp2f(st.m - M);
  const float c = mo == -INFINITY ? 0.f : exp2f(mo - M);
  st.m = M;
  st.l = st.l * a + sm.u.x.l[w][lane] * c;
#pragma unroll
  for (int rb = 0; rb < R / 16; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      st.acc[rb][i] = st.acc[rb][i] * a + sm.u.x.acc[w][4 * rb + i][lane] * c;
}

template <int R>
__device__ __forceinline__ void publish(const State<R>& st, Smem<R>& sm, int w, int lane) {
#pragma unroll
  for (int rb = 0; rb < R / 16; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.u.x.acc[w][4 * rb + i][lane] = st.acc[rb][i];
  sm.u.x.m[w][lane] = st.m;
  sm.u.x.l[w][lane] = st.l;
}

// The next tile of a wave in registers (vector types: arrays of uint4 here
// ended up in scratch memory). bf16: the key rows in the score operand
// pattern (row lane%16) and the value rows contiguous, 1 KiB per instruction.
// int8: both contiguous, 16 codes per lane and instruction, plus the key and
// value scales of the lane's four tokens 4*(lane/16) .. +3.
template <int R, bool kI8>
struct Pending {
  typedef uint32_t u32v __attribute__((ext_vector_type(R / 8)));
  u32v k, v;
};
template <int R>
struct Pending<R, true> {
  typedef uint32_t u32v __attribute__((ext_vector_type(R / 16)));
  u32v k, v;
  floatx4 sk, sv;
};

template <int R, bool kShared, bool kI8>
__global__ __launch_bounds__(64 * kWaves, 1) void split_absorbed_mfma_kernel(DecodeParams p) {
  // query heads of a group beyond 16 go to further head slices (workgroups
  // that read the same latents, shared through one XCD's L2)
  const int nslice = (p.nq + 15) / 16;
  const SplitUnit un = split_unit(p.n_split, p.G, p.B, nslice);
  if (!un.live) return;
  const int split = un.split, g = un.g, b = un.b;
  const int hq0 = un.hs * 16;                            // first query head of the slice
  const int nqs = min(16, p.nq - hq0);                   // its query heads
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, kb = lane >> 4;
  const int n = clamp_len(p.lens, b, p.L);
  const int s0 = split * p.split_tokens;
  if (s0 >= n) return;                                   // whole workgroup
  const int t1 = min(n, s0 + p.split_tokens);
  const int last = t1 - 1;

  __shared__ Smem<R> sm;
  const size_t row0 = (static_cast<size_t>(b) * p.G + g) * p.L;
  const float* qrow = p.qt + (static_cast<size_t>(b) * p.Hq + g * p.nq + hq0) * R;
  // absorbed queries of the slice's heads, split hi/lo (padding heads are 0)
  if constexpr (kI8) {
    // the split's largest value scale (scales are >= 0)
    float smax = 0.f;
    for (int t = s0 + static_cast<int>(threadIdx.x); t < t1; t += 64 * kWaves)
      smax = fmaxf(smax, p.s_v[row0 + t]);
    // one wave per head: scale by a power of two 2^e <= max |q~_h| < 2^(e+1)
    for (int hd = wave; hd < 16; hd += kWaves) {
      float x[R / 64];
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < R / 64; ++j) {
        x[j] = hd < nqs ? qrow[hd * R + lane + 64 * j] : 0.f;
        amax = fmaxf(amax, fabsf(x[j]));
      }
#pragma unroll
      for (int o = 32; o >= 1; o /= 2) amax = fmaxf(amax, __shfl_xor(amax, o));
      const uint32_t eb = __float_as_uint(amax) & 0x7F800000u;
      const float c = (eb == 0u || eb == 0x7F800000u) ? 1.f : __uint_as_float(eb);
      const float inv = 1.f / c;                     // exact: c is a power of two
#pragma unroll
      for (int j = 0; j < R / 64; ++j)
        split16<true>(x[j] * inv, sm.q.v[0][hd][lane + 64 * j], sm.q.v[1][hd][lane + 64 * j]);
      if (lane == 0) sm.qc[hd] = c;
    }
#pragma unroll
    for (int o = 32; o >= 1; o /= 2) smax = fmaxf(smax, __shfl_xor(smax, o));
    if (lane == 0) sm.svmax[wave] = smax;
  } else {
    for (int e = threadIdx.x; e < 16 * R; e += 64 * kWaves) {
      const int hd = e / R, k = e % R;
      const float x = hd < nqs ? qrow[hd * R + k] : 0.f;
      split16<false>(x, sm.q.v[0][hd][k], sm.q.v[1][hd][k]);
    }
  }
  __syncthreads();
  // int8: scores are multiplied by qc * s_k, value weights by s_v / vref, and
  // the partial sums by vref
  float qc = 1.f, vref = 1.f;
  if constexpr (kI8) {
    qc = sm.qc[ln];
    float m = sm.svmax[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, sm.svmax[w]);
    if (m > 0.f && m < INFINITY) vref = m;
  }
  const float vinv = 1.f / vref;

  State<R> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int rb = 0; rb < R / 16; ++rb) st.acc[rb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // 16-token tiles dealt round-robin: wave w takes tiles w, w+4, ...; loads
  // past the end read the last valid row again (never out of range)
  const int ntiles = (t1 - s0 + kTile - 1) / kTile;
  const int mine = (ntiles - wave + kWaves - 1) / kWaves;   // may be 0
  if (mine > 0) {
    char* kt = sm.u.t.kt[wave];
    char* vt = sm.u.t.vt[wave];
    const int step = kTile * kWaves;
    const int first = s0 + kTile * wave;
    Pending<R, kI8> nx;
    auto fetch = [&](int tok0) {
      if constexpr (kI8) {
        const int8_t* Hk = static_cast<const int8_t*>(p.h_k) + row0 * R;
        const int8_t* Hv = static_cast<const int8_t*>(p.h_v) + row0 * R;
#pragma unroll
        for (int q = 0; q < R / 64; ++q) {
          const int flat = q * 1024 + lane * 16;          // byte within the tile's 16 rows
          const size_t off = static_cast<size_t>(min(tok0 + flat / R, last)) * R + flat % R;
          const uint4 a = load_tile16<kShared>(Hk + off);
          const uint4 c = load_tile16<kShared>(Hv + off);
          nx.k[4 * q] = a.x; nx.k[4 * q + 1] = a.y; nx.k[4 * q + 2] = a.z; nx.k[4 * q + 3] = a.w;
          nx.v[4 * q] = c.x; nx.v[4 * q + 1] = c.y; nx.v[4 * q + 2] = c.z; nx.v[4 * q + 3] = c.w;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const size_t t = row0 + min(tok0 + 4 * kb + i, last);
          nx.sk[i] = p.s_k[t];
          nx.sv[i] = p.s_v[t];
        }
      } else {
        const uint16_t* Hk = static_cast<const uint16_t*>(p.h_k) + row0 * R;
        const uint16_t* Hv = static_cast<const uint16_t*>(p.h_v) + row0 * R;
        const int rk = min(tok0 + ln, last);
#pragma unroll
        for (int c = 0; c < R / 32; ++c) {
          const uint4 t = load_tile16<kShared>(Hk + static_cast<size_t>(rk) * R + 32 * c + 8 * kb);
          nx.k[4 * c] = t.x; nx.k[4 * c + 1] = t.y; nx.k[4 * c + 2] = t.z; nx.k[4 * c + 3] = t.w;
        }
#pragma unroll
        for (int q = 0; q < R / 32; ++q) {
          const int flat = q * 1024 + lane * 16;          // byte within the tile's 16 rows
          const int rv = min(tok0 + flat / (2 * R), last);
          const uint4 t = load_tile16<kShared>(Hv + static_cast<size_t>(rv) * R + (flat % (2 * R)) / 2);
          nx.v[4 * q] = t.x; nx.v[4 * q + 1] = t.y; nx.v[4 * q + 2] = t.z; nx.v[4 * q + 3] = t.w;
        }
      }
    };
    // copy the pending tile into the wave's LDS tiles (int8: widened to fp16)
    // and keep its scales for the consumer
    floatx4 sk = {1.f, 1.f, 1.f, 1.f}, sv = {1.f, 1.f, 1.f, 1.f};
    auto stage = [&]() {
      if constexpr (kI8) {
#pragma unroll
        for (int q = 0; q < R / 64; ++q) {
          const int flat = q * 1024 + lane * 16;
          const int row = flat / R, col = flat % R;       // 16 codes -> 32 bytes
          const uint2 k0 = i8x4_to_f16x4(nx.k[4 * q]), k1 = i8x4_to_f16x4(nx.k[4 * q + 1]);
          const uint2 k2 = i8x4_to_f16x4(nx.k[4 * q + 2]), k3 = i8x4_to_f16x4(nx.k[4 * q + 3]);
          char* kd = kt + row * kKStride<R> + 2 * col;
          *reinterpret_cast<uint4*>(kd) = uint4{k0.x, k0.y, k1.x, k1.y};
          *reinterpret_cast<uint4*>(kd + 16) = uint4{k2.x, k2.y, k3.x, k3.y};
          const uint2 v0 = i8x4_to_f16x4(nx.v[4 * q]), v1 = i8x4_to_f16x4(nx.v[4 * q + 1]);
          const uint2 v2 = i8x4_to_f16x4(nx.v[4 * q + 2]), v3 = i8x4_to_f16x4(nx.v[4 * q + 3]);
          char* vd = vt + vtile_off<R>(row, 2 * col);
          *reinterpret_cast<uint4*>(vd) = uint4{v0.x, v0.y, v1.x, v1.y};
          *reinterpret_cast<uint4*>(vd + 16) = uint4{v2.x, v2.y, v3.x, v3.y};
        }
        sk = nx.sk * qc;
        sv = nx.sv * vinv;
      } else {
#pragma unroll
        for (int c = 0; c < R / 32; ++c)
          *reinterpret_cast<uint4*>(kt + ln * kKStride<R> + 2 * (32 * c + 8 * kb)) =
              uint4{nx.k[4 * c], nx.k[4 * c + 1], nx.k[4 * c + 2], nx.k[4 * c + 3]};
#pragma unroll
        for (int q = 0; q < R / 32; ++q) {
          const int flat = q * 1024 + lane * 16;
          *reinterpret_cast<uint4*>(vt + vtile_off<R>(flat / (2 * R), flat % (2 * R))) =
              uint4{nx.v[4 * q], nx.v[4 * q + 1], nx.v[4 * q + 2], nx.v[4 * q + 3]};
        }
      }
    };
    fetch(first);
    for (int j = 0; j < mine; ++j) {
      stage();
      fetch(first + step * (j + 1));
      const floatx4 s = scores<R, kI8>(kt, sm.q, first + step * j, t1, lane, sk);
      softmax_values<R, kI8>(st, s, vt, lane, sv);
    }
  }

  // merge the waves' states in LDS (the value tiles' space, after a barrier),
  // halving the number of live states each round: waves [h, 2h) publish,
  // waves [0, h) fold in the state of wave + h. [slot][value][lane] keeps
  // consecutive lanes on consecutive banks.
#pragma unroll
  for (int h = kWaves / 2; h >= 1; h /= 2) {
    __syncthreads();
    if (wave >= h && wave < 2 * h) publish<R>(st, sm, wave - h, lane);
    __syncthreads();
    if (wave < h) combine<R>(st, sm, wave, lane);
  }
  if (wave > 0) return;
  const float M = st.m;
  float l = st.l;

  // head totals: sum the four lane groups' shares
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (ln >= nqs) return;
  const int head = g * p.nq + hq0 + ln;
  const size_t slot = (static_cast<size_t>(b) * p.Hq + head) * p.n_split + split;
  if (kb == 0) {
    p.part_ml[slot * 2] = M;
    p.part_ml[slot * 2 + 1] = l;
  }
  float* u = p.part_u + slot * R;
#pragma unroll
  for (int rb = 0; rb < R / 16; ++rb) {
    if constexpr (kI8) st.acc[rb] *= vref;
    *reinterpret_cast<float4*>(u + 16 * rb + 4 * kb) =
        float4{st.acc[rb][0], st.acc[rb][1], st.acc[rb][2], st.acc[rb][3]};
  }
}

template <int R, bool kI8>
hipError_t launch_rank(const DecodeParams& p, hipStream_t st) {
  const int nslice = absorbed_head_slices(p.nq);
  if (nslice == 1) {
    split_absorbed_mfma_kernel<R, false, kI8><<<dim3(p.n_split, p.G, p.B), 64 * kWaves, 0, st>>>(p);
  } else {
    const long ids = split_unit_ids(p.n_split, p.G, p.B, nslice);
    if (ids == 0) return hipErrorInvalidValue;
    split_absorbed_mfma_kernel<R, true, kI8>
        <<<dim3(static_cast<unsigned>(ids)), 64 * kWaves, 0, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

bool absorbed_mfma_supported(const DecodeParams& p, int dtype) {
  return dtype == 1 && (p.r == 32 || p.r == 64 || p.r == 128 || p.r == 256);
}

bool absorbed_i8_supported(const DecodeParams& p, int dtype) {
  return dtype == 1 && (p.r == 64 || p.r == 128 || p.r == 256);
}

int absorbed_head_slices(int nq) { return (nq + 15) / 16; }

hipError_t launch_split_absorbed_mfma(const DecodeParams& p, hipStream_t st) {
  if (p.latent_i8) {
    switch (p.r) {
      case 64: return launch_rank<64, true>(p, st);
      case 128: return launch_rank<128, true>(p, st);
      case 256: return launch_rank<256, true>(p, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (p.r) {
    case 32: return launch_rank<32, false>(p, st);
    case 64: return launch_rank<64, false>(p, st);
    case 128: return launch_rank<128, false>(p, st);
    case 256: return launch_rank<256, false>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace palu
