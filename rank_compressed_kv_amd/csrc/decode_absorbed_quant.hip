// Context-split decode kernel for the absorbed-key mode over an int8 or int4
// latent cache (per-token quantisation of the latents, Palu author response
// to reviewer Fsn9 on W1/W2: codes with one fp32 scale per cached row, h =
// code * scale), on the gfx950 matrix cores.
//
// The scores and the value sum are those of the bf16 kernel (absorbed keys:
// q~ = q B_k^T scored against the key latents, value latents summed with the
// weights, B_v applied in the merge); what differs is the cache and the data
// path:
//   - the quantised cache is stored in 32-token blocks whose byte order is that of
//     the MFMA operands (the append kernel writes it), so every 16-byte load of
//     a lane holds exactly the operand bytes that lane needs: no LDS staging,
//     no gathers, fully coalesced 1 KiB per load instruction;
//   - codes become fp16 operands in registers as exact subnormals (a byte
//     permute or a nibble mask per pair of codes; value operands also lose
//     their bias in one packed subtraction) and are multiplied on fp16 MFMAs,
//     16x16x32 for the scores (16 tokens x 16 heads over 32 latents) and for
//     the values (r x 16 heads over 32 tokens);
//   - a block's key scales multiply its scores, its value scales fold into the
//     weights (p_t s_t; the running sum l keeps p_t). q~ is divided per head
//     by a power of two near its largest entry and the value scales by the
//     split's largest one, so fp16 operands stay in range whatever the
//     magnitudes; both are undone in fp32. q~ and the weights are each
//     rounded once to fp16 (11 significant bits; relative error 2^-12 per
//     entry, averaging out over the 256 latents of a score and the tokens of
//     a sum): the codes carry at most 8 bits, and the bf16 kernel's two-term
//     operands would double the MFMAs of a kernel that is not HBM-bound.
// One workgroup owns one (batch, group, context split) and 16 query heads;
// its waves (four for int8, eight for int4) take the split's 32-token
// blocks round-robin and combine
// their softmax states in LDS at the end. A wave holds two blocks in
// registers: the next one is requested before the current one is multiplied
// (non-temporal loads: the cache is read once). Blocks are read whole: rows
// past the length inside the last block are masked (their codes are finite
// whatever they hold; their scales are replaced by 0 before use), and no byte
// outside the cache is touched.
// A rotated cache (Hadamard rows, see the append) is read the same way: q~ is
// rotated in the prologue and each split's value sum rotated back before it
// is written, so the merge and B_k, B_v are those of the plain cache.
#include <math.h>

#include <type_traits>

#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// waves per workgroup: an int4 wave fits in half a SIMD's registers, so two
// waves per SIMD keep twice the blocks in flight (measured 39 -> 35 us at
// Llama-3-8B, 32K context); an int8 wave needs a whole SIMD's registers
template <int kBits>
constexpr int kWavesFor = kBits == 4 ? 8 : 4;
constexpr float kV = 8.f;         // value weights' extra power of two (fp16 range: 2^8 kV kF)
constexpr int kBlock = 32;       // tokens per cache block and per wave step
constexpr float kLazy = 8.0f;    // log2 units: p <= 2^8 between rescales


// Codes enter the matrix cores as fp16 subnormals: the fp16 with bits 0x00uu
// is u * 2^-24 exactly, so a byte or a nibble moved into the low bits of a
// 16-bit lane is already an operand. They are biased codes (u = code + 128
// after flipping an int8 code's sign bit; u = code + 8 as an int4 cache
// stores it). Key operands keep the bias, which leaves once per head and
// token: the score accumulators start at -bias * sum_k q_k (a product of
// bounded size per token). Value operands take it off exactly, in fp16,
// before the product: a bias inside the weighted sum over thousands of tokens
// would cancel against a sum thousands of times larger than the result, which
// the matrix cores' accumulation does not carry accurately enough. The factor
// 2^-24 goes into the head's exponent factor and the output scale.

// four int8 codes -> two fp16 pairs u * 2^-24 (u = code + 128)
__device__ __forceinline__ uint2 i8x4_operand(uint32_t w) {
  const uint32_t x = w ^ 0x80808080u;
  return uint2{__builtin_amdgcn_perm(0u, x, 0x0C010C00u), __builtin_amdgcn_perm(0u, x, 0x0C030C02u)};
}
// eight int4 codes (biased nibbles, operand element 2m in nibble m and 2m+1
// in nibble m+4) -> fp16 pairs: pairs 0 and 2 (nibbles 0/4 of w and of w >>
// 8) are u * 2^-24, pairs 1 and 3 (nibbles 1/5) 16u * 2^-24; the other
// operand carries 1/16 at those positions (elements k % 8 in {2, 3, 6, 7})
__device__ __forceinline__ uint4 i4x8_operand(uint32_t w) {
  const uint32_t w8 = w >> 8;
  return uint4{w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u};
}
__device__ __forceinline__ uint32_t sub_f16x2(uint32_t a, _Float16 b) {
  const half2v bb = {b, b};
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, a) - bb);
}
// key operands (biased): eight int8 codes from two words, or eight int4 codes
__device__ __forceinline__ uint4 key_operand8(uint32_t w0, uint32_t w1) {
  const uint2 a = i8x4_operand(w0), b = i8x4_operand(w1);
  return uint4{a.x, a.y, b.x, b.y};
}
__device__ __forceinline__ uint4 key_operand4(uint32_t w) { return i4x8_operand(w); }
// value operands: the codes themselves (code * 2^-24, or 16 code * 2^-24 at
// the scaled int4 positions), exact subnormal differences
__device__ __forceinline__ uint4 value_operand8(uint32_t w0, uint32_t w1) {
  const _Float16 b = static_cast<_Float16>(0x1p-17f);            // 128 * 2^-24
  const uint4 a = key_operand8(w0, w1);
  return uint4{sub_f16x2(a.x, b), sub_f16x2(a.y, b), sub_f16x2(a.z, b), sub_f16x2(a.w, b)};
}
__device__ __forceinline__ uint4 value_operand4(uint32_t w) {
  const _Float16 b8 = static_cast<_Float16>(0x1p-21f);           // 8 * 2^-24
  const _Float16 b128 = static_cast<_Float16>(0x1p-17f);         // 16 * 8 * 2^-24
  const uint4 a = i4x8_operand(w);
  return uint4{sub_f16x2(a.x, b8), sub_f16x2(a.y, b128), sub_f16x2(a.z, b8), sub_f16x2(a.w, b128)};
}

__device__ __forceinline__ floatx4 mfma(uint4 a, uint4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

// Walsh-Hadamard butterflies for a rotated cache (Sylvester's H_r, H_r H_r =
// r I): the pair (x_i, x_i+m) becomes (x_i + x_i+m, x_i - x_i+m), over every
// bit m of the index. The index bits sit in lanes (shuffles) or in registers.
__device__ __forceinline__ float bfly_lane(float x, int lane, int m) {
  const float o = __shfl_xor(x, m);
  return (lane & m) ? o - x : x + o;
}

// q~ in LDS as the score MFMA's B operand: [hi|lo][head][k] fp16 bits; rows
// padded by 8 elements so the 16 heads' 16-byte reads spread over the banks
template <int R, int kWaves>
struct Smem {
  union {
    uint16_t q[16][R + 8];
    float urot[16][R + 4];   // merged value sums of a rotated cache (after the loop)
  };
  float qc[16];              // power of two each head's q~ was divided by
  float qbias[16];           // -bias * sum_k q_k * 2^-24: the score accumulators' start
  float svmax[kWaves];       // each wave's largest value scale
  floatx4 acc[kWaves][R / 16][64];   // every wave's value sums (final merge), 16 B a lane
  float m[kWaves][64], l[kWaves][64];
};

template <int R>
struct State {
  floatx4 acc[R / 16];   // U^T: r = 16*rb + 4*(lane/16) + i, head lane%16
  float m;               // stored running max (log2 units) of head lane%16
  float l;               // this lane's share of the running sum
};

// One cache block in registers: R*kBits/256 16-byte words of each matrix
// (word i of lane l is bytes [1024 i + 16 l, +16) of the block) and the key
// and value scales of the lane's eight tokens 4*(l/16) + i and 16 + 4*(l/16)
// + i.
template <int R, int kBits>
struct Block {
  typedef uint32_t u32v __attribute__((ext_vector_type(R * kBits / 64)));
  u32v k, v;
  floatx4 sk0, sk1, sv0, sv1;
};

template <int R, bool kShared, int kBits>
__global__ __launch_bounds__(64 * kWavesFor<kBits>, 1) void split_absorbed_int_kernel(DecodeParams p) {
  constexpr int kWaves = kWavesFor<kBits>;
  // every key and value product carries kF * 2^-24 (int4: 16 u against q~ / 16
  // or 16 q~ against u; the subnormal codes' 2^-24)
  constexpr float kF = kBits == 4 ? 16.f : 1.f;
  constexpr int kRowBytes = R * kBits / 8;               // bytes of a cached row
  const int nslice = (p.nq + 15) / 16;
  const SplitUnit un = split_unit(p.n_split, p.G, p.B, nslice);
  if (!un.live) return;
  const int split = un.split, g = un.g, b = un.b;
  const int hq0 = un.hs * 16;                            // first query head of the slice
  const int nqs = min(16, p.nq - hq0);                   // its query heads
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, kb = lane >> 4;
  const int n = clamp_len(p.lens, b, p.L);
  const int s0 = split * p.split_tokens;                 // a multiple of 64
  if (s0 >= n) return;                                   // whole workgroup
  const int t1 = min(n, s0 + p.split_tokens);

  __shared__ Smem<R, kWaves> sm;
  const size_t row0 = (static_cast<size_t>(b) * p.G + g) * p.L;
  const int8_t* Hk = static_cast<const int8_t*>(p.h_k) + row0 * kRowBytes;
  const int8_t* Hv = static_cast<const int8_t*>(p.h_v) + row0 * kRowBytes;
  const int nblk = (t1 - s0 + kBlock - 1) / kBlock;
  const int mine = (nblk - wave + kWaves - 1) / kWaves;   // blocks of this wave, may be 0
  auto tok_of = [&](int j) { return s0 + kBlock * (wave + kWaves * j); };

  // one matrix's words of the block at t0 (t0 % 32 == 0) and the scales of
  // the lane's eight tokens (16-byte aligned: L % 32 == 0)
  auto fetch_half = [&](typename Block<R, kBits>::u32v& w, floatx4& s0v, floatx4& s1v,
                        const int8_t* H, const float* S, int t0) {
    const size_t base = static_cast<size_t>(t0) * kRowBytes + lane * 16;
#pragma unroll
    for (int i = 0; i < R * kBits / 256; ++i) {
      const uint4 a = load_tile16<kShared>(H + base + i * 1024);
      w[4 * i] = a.x; w[4 * i + 1] = a.y; w[4 * i + 2] = a.z; w[4 * i + 3] = a.w;
    }
    const size_t srow = row0 + t0 + 4 * kb;
    const float4 a0 = *reinterpret_cast<const float4*>(S + srow);
    const float4 a1 = *reinterpret_cast<const float4*>(S + srow + 16);
    s0v = floatx4{a0.x, a0.y, a0.z, a0.w};
    s1v = floatx4{a1.x, a1.y, a1.z, a1.w};
  };
  auto fetch = [&](Block<R, kBits>& x, int t0) {
    fetch_half(x.k, x.sk0, x.sk1, Hk, p.s_k, t0);
    fetch_half(x.v, x.sv0, x.sv1, Hv, p.s_v, t0);
  };
  Block<R, kBits> xa, xb;

  {
    // every load of this prologue is issued before the first is used: the
    // split's value scales (4096 tokens per round, indexes clamped to the
    // split) and the q~ entries of this wave's heads
    constexpr int kS = 4096 / (64 * kWaves);
    float svx[kS];
    auto load_scales = [&](int base) {
#pragma unroll
      for (int u = 0; u < kS; ++u)
        svx[u] = p.s_v[row0 + min(base + static_cast<int>(threadIdx.x) + u * 64 * kWaves, t1 - 1)];
    };
    load_scales(s0);
    constexpr int kH = 16 / kWaves;
    const float* qrow = p.qt + (static_cast<size_t>(b) * p.Hq + g * p.nq + hq0) * R;
    float qx[kH][R / 64];
#pragma unroll
    for (int i = 0; i < kH; ++i)
#pragma unroll
      for (int j = 0; j < R / 64; ++j)
        qx[i][j] = qrow[min(wave + kWaves * i, nqs - 1) * R + lane + 64 * j];
    // splits longer than 4096 tokens (not planned by the library; a caller
    // may ask for them) take further rounds of scale loads here, before any
    // block is requested
    float smax = 0.f;
    if (t1 - s0 > 4096) {
      for (int base = s0;;) {
#pragma unroll
        for (int u = 0; u < kS; ++u) smax = fmaxf(smax, svx[u]);
        base += 4096;
        if (base >= t1) break;
        load_scales(base);
      }
    }
    // then the first blocks' loads: issued after the prologue's own loads (a
    // compiler-only barrier keeps that order), so that waiting for those
    // (memory counters drain in issue order) leaves the blocks in flight
    // through the prologue. The requests are unconditional (a wave without
    // blocks reads the split's first block, unused): after a conditional
    // request the compiler could no longer count them and drained them all.
    asm volatile("" ::: "memory");
    fetch(xa, mine > 0 ? tok_of(0) : s0);
    // the split's largest value scale (scales are >= 0; clamped duplicates
    // do not change a maximum)
    if (t1 - s0 <= 4096) {
#pragma unroll
      for (int u = 0; u < kS; ++u) smax = fmaxf(smax, svx[u]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o /= 2) smax = fmaxf(smax, __shfl_xor(smax, o));
    if (lane == 0) sm.svmax[wave] = smax;
    // one wave per head: q~ scaled by a power of two (below), fp16
#pragma unroll
    for (int i = 0; i < kH; ++i) {
      const int hd = wave + kWaves * i;
      if (hd >= nqs) {
#pragma unroll
        for (int j = 0; j < R / 64; ++j) qx[i][j] = 0.f;   // padding heads are 0
      }
      if (p.hadamard) {
        // rotated cache: score <q~, h> = <q~ H_r / r, h''>; latent lane + 64 j
#pragma unroll
        for (int m = 1; m < 64; m *= 2)
#pragma unroll
          for (int j = 0; j < R / 64; ++j) qx[i][j] = bfly_lane(qx[i][j], lane, m);
#pragma unroll
        for (int m = 1; m < R / 64; m *= 2)
#pragma unroll
          for (int j = 0; j < R / 64; ++j)
            if (!(j & m)) {
              const float a = qx[i][j], c = qx[i][j + m];
              qx[i][j] = a + c;
              qx[i][j + m] = a - c;
            }
#pragma unroll
        for (int j = 0; j < R / 64; ++j) qx[i][j] *= 1.f / R;   // exact: R = 2^k
      }
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < R / 64; ++j) amax = fmaxf(amax, fabsf(qx[i][j]));
#pragma unroll
      for (int o = 32; o >= 1; o /= 2) amax = fmaxf(amax, __shfl_xor(amax, o));
      // q~ / c with c = 2^(e-10), 2^e <= max |q~_h| < 2^(e+1): entries up to
      // 2^11, so all but the smallest entries stay normal fp16
      const uint32_t eb = __float_as_uint(amax) & 0x7F800000u;
      const float c0 = (eb == 0u || eb == 0x7F800000u) ? 1.f : __uint_as_float(eb);
      const float boost = c0 >= 0x1p-100f ? 1024.f : 1.f;
      const float c = c0 / boost;                    // exact: powers of two
      const float inv = boost / c0;
      // int4: latents k % 8 in {2, 3, 6, 7} (k = lane + 64 j) meet operands
      // scaled by 16, so the other latents' q~ is multiplied by 16 (exact):
      // every product then carries kF = 16
      const bool plain = kBits == 4 && !((lane >> 1) & 1);
      const float ks = plain ? 16.f : 1.f;
      float qsum = 0.f;                              // sum_k of q~_k / c
#pragma unroll
      for (int j = 0; j < R / 64; ++j) {
        const _Float16 h = static_cast<_Float16>(qx[i][j] * inv * ks);   // nearest even
        sm.q[hd][lane + 64 * j] = __builtin_bit_cast(uint16_t, h);
        qsum += static_cast<float>(h) * (plain ? 0.0625f : 1.f);
      }
#pragma unroll
      for (int o = 32; o >= 1; o /= 2) qsum += __shfl_xor(qsum, o);
      if (lane == 0) {
        sm.qc[hd] = c;
        sm.qbias[hd] = -(kBits == 8 ? 128.f : 8.f) * qsum * (kF * 0x1p-24f);
      }
    }
  }
  barrier_lds();            // the first tiles stay in flight
  // scores are multiplied by qc * s_k, value weights by s_v / vref and the
  // partial sums by vref
  const float qc = sm.qc[ln] * (0x1p24f / kF);          // the products' kF * 2^-24 too
  const float qb = sm.qbias[ln];
  float vref = sm.svmax[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) vref = fmaxf(vref, sm.svmax[w]);
  if (!(vref > 0.f && vref < INFINITY)) vref = 1.f;
  const float vinv = 1.f / vref;
  // value weights times kV (small weights stay normal fp16 longer: weights
  // reach 2^8 kV kF <= 2^15), and for int4 those of the tokens whose operand
  // elements carry u, not 16 u (k-slot elements 0, 1, 4, 5: the lane's tokens
  // i = 0, 1 of each half) times 16, so every product carries kV kF
  const float vw = vinv * kV;
  const floatx4 vinvv = kBits == 4 ? floatx4{vw * 16.f, vw * 16.f, vw, vw}
                                   : floatx4{vw, vw, vw, vw};

  State<R> st;
  st.m = -INFINITY;
  st.l = 0.f;

#pragma unroll
  for (int rb = 0; rb < R / 16; ++rb) st.acc[rb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // masked: the block may reach past the split's end (only a wave's last
  // block can: every other block of a wave lies whole inside the split)
  auto compute = [&](const Block<R, kBits>& x, int t0, auto masked) {
    // q~ is read from LDS again for every block: held in registers across the
    // loop it would take 128 of them at r = 256 (a compiler-only barrier keeps
    // the reads inside)
    asm volatile("" ::: "memory");
    // scores of the two 16-token halves: S^T[16 tok x 16 heads] of half h
    // (even and odd chunks in separate accumulators: four independent chains)
    floatx4 se[2] = {{qb, qb, qb, qb}, {qb, qb, qb, qb}};
    floatx4 so[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < R / 32; ++c) {
      const uint4 qh = *reinterpret_cast<const uint4*>(&sm.q[ln][32 * c + 8 * kb]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // key chunk c of half h: int8 word h*R/64 + c/2, bytes 8*(c%2) .. +8;
        // int4 the lane's 32-bit unit h*R/32 + c
        uint4 a;
        if constexpr (kBits == 8) {
          const int w = 4 * (h * (R / 64) + c / 2) + 2 * (c % 2);
          a = key_operand8(x.k[w], x.k[w + 1]);
        } else {
          a = key_operand4(x.k[h * (R / 32) + c]);
        }
        if (c % 2 == 0) se[h] = mfma(a, qh, se[h]);
        else so[h] = mfma(a, qh, so[h]);
      }
    }
    // scores in units of qc * 2^-24 (qc the head's power-of-two divisor),
    // bias already out: that factor is applied in the exponent
    floatx4 sc[2] = {(se[0] + so[0]) * x.sk0, (se[1] + so[1]) * x.sk1};
    floatx4 sv[2] = {x.sv0 * vinvv, x.sv1 * vinvv};
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 16 * h + 4 * kb + i >= t1) {
            sc[h][i] = -INFINITY;
            sv[h][i] = 0.f;
          }
    }
    // online softmax over the block's 32 tokens of head ln
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mx *= qc;                                            // qc > 0: the true maximum
    if (__any(mx > st.m + kLazy)) {
      const float mn = fmaxf(st.m, mx);
      const float alpha = exp2f(st.m - mn);
      st.m = mn;
      st.l *= alpha;
#pragma unroll
      for (int rb = 0; rb < R / 16; ++rb) st.acc[rb] *= alpha;
    }
    // P^T operand: k-slot 8*kb + j is token 4*kb + j (j < 4) or 16 + 4*kb + j - 4
    // weights (v_exp_f32: arguments <= kLazy, results below 2^-126 flush to
    // 0, far under the fp16 operands' resolution), rounded once to fp16
    uint32_t ph[4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float pe0 = __builtin_amdgcn_exp2f(fmaf(qc, sc[h][i], -st.m));
        const float pe1 = __builtin_amdgcn_exp2f(fmaf(qc, sc[h][i + 1], -st.m));
        st.l += pe0 + pe1;
        const half2v w = {static_cast<_Float16>(pe0 * sv[h][i]),
                          static_cast<_Float16>(pe1 * sv[h][i + 1])};
        ph[2 * h + i / 2] = __builtin_bit_cast(uint32_t, w);
      }
    const uint4 bh = {ph[0], ph[1], ph[2], ph[3]};
    // values: U^T[16 rb .. +16, heads] += H_v^T[., 32 tokens] P^T; latent rows
    // 16*rb + ln of the lane's eight tokens in word rb/2, bytes 8*(rb%2) .. +8
    // (four row blocks at a time)
    static_assert(R % 64 == 0, "row blocks come in fours");
#pragma unroll
    for (int rb0 = 0; rb0 < R / 16; rb0 += 4) {
      uint4 a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int rb = rb0 + u;
        if constexpr (kBits == 8) {
          const int w = 4 * (rb / 2) + 2 * (rb % 2);
          a[u] = value_operand8(x.v[w], x.v[w + 1]);
        } else {
          a[u] = value_operand4(x.v[rb]);                // the lane's unit rb
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) st.acc[rb0 + u] = mfma(a[u], bh, st.acc[rb0 + u]);
    }
  };
  // the hot loops fetch unconditionally (a fetch under a branch made the
  // compiler wait for the current block before issuing the next one); the
  // last blocks are peeled off
  if (mine > 0) {
    // two register sets: the next block is requested before the current one
    // is multiplied
    int j = 0;
    for (; j + 2 < mine; j += 2) {
      fetch(xb, tok_of(j + 1));
      compute(xa, tok_of(j), std::false_type{});
      fetch(xa, tok_of(j + 2));
      compute(xb, tok_of(j + 1), std::false_type{});
    }
    if (j + 1 < mine) {
      fetch(xb, tok_of(j + 1));
      compute(xa, tok_of(j), std::false_type{});
      compute(xb, tok_of(j + 1), std::true_type{});
    } else {
      compute(xa, tok_of(j), std::true_type{});
    }
  }

  // merge: every wave publishes its state, then after one barrier every
  // thread combines one (head, lane group, row block) slice of all of them
  // (a side that saw no token has m = -inf and weight 0) and writes it
#pragma unroll
  for (int rb = 0; rb < R / 16; ++rb) sm.acc[wave][rb][lane] = st.acc[rb];
  sm.m[wave][lane] = st.m;
  sm.l[wave][lane] = st.l;
  __syncthreads();
  const int th = threadIdx.x;
  const int cln = th % 16, ckb = (th / 16) % 4, crq = th / 64;   // head, lane group, first row block
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.m[w][cln]);
  float aw[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float mw = sm.m[w][cln];
    aw[w] = mw == -INFINITY ? 0.f : exp2f(mw - M);
  }
  float uscale = vref * (0x1p24f / (kF * kV));         // the products' factors
  const int head = g * p.nq + hq0 + cln;
  const size_t slot = (static_cast<size_t>(b) * p.Hq + head) * p.n_split + split;
  if (th < 16 && cln < nqs) {
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      l += aw[w] * ((sm.l[w][cln] + sm.l[w][16 + cln]) + (sm.l[w][32 + cln] + sm.l[w][48 + cln]));
    p.part_ml[slot * 2] = M;
    p.part_ml[slot * 2 + 1] = l;
  }
  // latents 16 rb + 4 ckb + i of head cln
  for (int rb = crq; rb < R / 16; rb += kWaves) {
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const floatx4 a = sm.acc[w][rb][16 * ckb + cln];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = fmaf(aw[w], a[i], v[i]);
    }
    if (p.hadamard) {
      *reinterpret_cast<float4*>(&sm.urot[cln][16 * rb + 4 * ckb]) = float4{v[0], v[1], v[2], v[3]};
    } else if (cln < nqs) {
      v *= uscale;
      *reinterpret_cast<float4*>(p.part_u + slot * R + 16 * rb + 4 * ckb) =
          float4{v[0], v[1], v[2], v[3]};
    }
  }
  if (!p.hadamard) return;
  // rotated cache: u = u'' H_r / r, one wave per head, latents 4 lane .. +3:
  // butterflies over the two index bits inside the lane, then over lane bits
  __syncthreads();
  uscale *= 1.f / R;                                     // exact: R = 2^k
  constexpr int nq4 = R / 4;                             // lanes holding latents
  for (int hd = wave; hd < nqs; hd += kWaves) {
    float4 v = lane < nq4 ? *reinterpret_cast<const float4*>(&sm.urot[hd][4 * lane])
                          : float4{0.f, 0.f, 0.f, 0.f};
    const float a0 = v.x + v.y, a1 = v.x - v.y, a2 = v.z + v.w, a3 = v.z - v.w;
    v = float4{a0 + a2, a1 + a3, a0 - a2, a1 - a3};
#pragma unroll
    for (int m = 1; m < nq4; m *= 2)
      v = float4{bfly_lane(v.x, lane, m), bfly_lane(v.y, lane, m), bfly_lane(v.z, lane, m),
                 bfly_lane(v.w, lane, m)};
    if (lane < nq4) {
      const size_t sl = (static_cast<size_t>(b) * p.Hq + g * p.nq + hq0 + hd) * p.n_split + split;
      *reinterpret_cast<float4*>(p.part_u + sl * R + 4 * lane) =
          float4{v.x * uscale, v.y * uscale, v.z * uscale, v.w * uscale};
    }
  }
}

template <int R, int kBits>
hipError_t launch_rank(const DecodeParams& p, hipStream_t st) {
  const int nslice = absorbed_head_slices(p.nq);
  if (nslice == 1) {
    split_absorbed_int_kernel<R, false, kBits>
        <<<dim3(p.n_split, p.G, p.B), 64 * kWavesFor<kBits>, 0, st>>>(p);
  } else {
    const long ids = split_unit_ids(p.n_split, p.G, p.B, nslice);
    if (ids == 0) return hipErrorInvalidValue;
    split_absorbed_int_kernel<R, true, kBits>
        <<<dim3(static_cast<unsigned>(ids)), 64 * kWavesFor<kBits>, 0, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

bool absorbed_quant_supported(const DecodeParams& p, int dtype) {
  return dtype == 1 && (p.r == 64 || p.r == 128 || p.r == 256) && p.L % kBlock == 0;
}

hipError_t launch_split_absorbed_quant(const DecodeParams& p, hipStream_t st) {
  switch (p.r * 16 + p.qbits) {
    case 64 * 16 + 8: return launch_rank<64, 8>(p, st);
    case 128 * 16 + 8: return launch_rank<128, 8>(p, st);
    case 256 * 16 + 8: return launch_rank<256, 8>(p, st);
    case 64 * 16 + 4: return launch_rank<64, 4>(p, st);
    case 128 * 16 + 4: return launch_rank<128, 4>(p, st);
    case 256 * 16 + 4: return launch_rank<256, 4>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace palu
