// Device pieces shared by the rebuilt-key decode kernels that give each wave
// one KV head's B_k^T (or a latent half of it) for the whole split: operand
// types and conversions, lane-group reductions, the rotation table and the
// query operand.
//
// The rotary embedding turns the pair (f, f + 64) of a key by the 2x2
// rotation of the CommVQ author response (proof of Property 1), angle
// t * omega_f at position t; the table holds 2^-8 (cos, sin) for the 16
// tokens of a tile (the rebuilt keys enter fp16 scaled by 2^-8).
#pragma once

#include <math.h>

#include <utility>

#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace wave {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;          // tokens per tile
constexpr int kD = 128;            // head dim
constexpr int kAnchor = 32;        // tiles between exact cos/sin evaluations
constexpr float kLazy = 8.0f;      // log2 units: p <= 2^8 between rescales
constexpr float kKeyScale = 1.0f / 256.0f;   // rebuilt keys enter fp16 times 2^-8

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

// a ~ hi + lo with hi = bf16(a) and lo = bf16(a - hi), both nearest-even, for a
// pair of values: about 16 significant bits in two bf16 terms
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a, b}, bf16x2));
  const float ah = __uint_as_float(hi << 16), bh = __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a - ah, b - bh}, bf16x2));
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a, b}, halfx2));
}

// max and sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups
// of a 16x16 MFMA result) with the gfx950 lane-swap moves: a swap of a
// register with itself leaves each lane's own value in one result and its
// partner's in the other, which is all a symmetric reduction needs
__device__ __forceinline__ float max_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// x + its value in lane l ^ 16 (lane groups 0 + 1 and 2 + 3)
__device__ __forceinline__ float add_pair_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1, fully
// expanded whatever the body's size (the slot schedules rely on it).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Keeps a register value in an AGPR: an empty asm statement whose operand
// must live there. Matrix-core instructions read their A and B operands from
// AGPRs directly, so B_k^T stays in the AGPRs and the VGPRs are left to
// everything else; no instruction is emitted.
__device__ __forceinline__ void hold_in_agpr(u32x4& v) { asm volatile("" : "+a"(v)); }

// The gfx950 transposing LDS read (ds_read_b64_tr_b16): a 16-lane group reads
// four 32-byte rows and each lane gets one 16-bit column of the four rows.
__device__ __forceinline__ short4v read_tr16(const char* p) {
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
  return __builtin_bit_cast(short4v, v);
}

// K tile rows padded by 32 B: a row stride of 32 mod 64 bytes is what keeps
// the operand read (16 rows, one 16-byte piece each per 16-lane group) free
// of LDS bank conflicts on gfx950 (measured: a 16 mod 64 stride runs the same
// read at about 60% of the conflict-free rate); V tile rows padded by 32 B
// (the four rows of a 16-lane transposing read cover all banks). R: latents
// in a row.
template <int R>
constexpr int kKStride = 2 * R + 32;
template <int R>
constexpr int kVStride = 2 * R + 32;

// B_k^T of one KV head as the key MFMA's A operand, held in AGPRs: lane (ln,
// kb) of column block blk, chunk c holds column 16 blk + ln, latents lat0 +
// 32 c + 8 kb .. +8. Bt points at the head's first column; rstride is the
// transposed copy's row length (the full rank).
template <int kC>
__device__ __forceinline__ void load_bkt(u32x4 (&bt)[8][kC], const uint16_t* Bt, int rstride,
                                         int lat0, int ln, int kb) {
#pragma unroll
  for (int blk = 0; blk < 8; ++blk)
#pragma unroll
    for (int c = 0; c < kC; ++c)
      bt[blk][c] = *reinterpret_cast<const u32x4*>(
          Bt + static_cast<size_t>(16 * blk + ln) * rstride + lat0 + 32 * c + 8 * kb);
#pragma unroll
  for (int blk = 0; blk < 8; ++blk)
#pragma unroll
    for (int c = 0; c < kC; ++c) hold_in_agpr(bt[blk][c]);
}

// q of query head ln of a KV head (heads head0 .. head0 + gqa - 1) as the
// score MFMA's B operand, fp16: lane (ln, kb), MFMA m (block pair m, m + 4)
// holds columns 16 m + 4 kb + j and 16 (m + 4) + 4 kb + j, j < 4, scaled by a
// power of two that puts the head's largest |q| in [256, 512) (exact: bf16 q
// has 8 significant bits); the factor goes back into the returned log2-unit
// score factor of head ln. Lanes ln >= gqa get a zero query.
__device__ __forceinline__ float q_operand(const DecodeParams& p, int b, int head0, int gqa,
                                           int ln, int kb, int lane, uint4 (*qop)[64]) {
  const bool qvalid = ln < gqa;
  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                         (static_cast<size_t>(b) * p.Hq + head0 + (qvalid ? ln : 0)) * kD;
  uint2 qw[8];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    qw[2 * m] = *reinterpret_cast<const uint2*>(qrow + 16 * m + 4 * kb);
    qw[2 * m + 1] = *reinterpret_cast<const uint2*>(qrow + 16 * (m + 4) + 4 * kb);
  }
  float qf[4][8];
  float qmax = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint2 w = qw[2 * m + h];
      const float v[4] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qf[m][4 * h + j] = qvalid ? v[j] : 0.f;
        qmax = fmaxf(qmax, fabsf(qf[m][4 * h + j]));
      }
    }
  qmax = max_groups(qmax);
  int ex = 0;
  (void)frexpf(qmax, &ex);                             // qmax = mant * 2^ex, mant in [0.5, 1)
  const float qs = qmax > 0.f ? ldexpf(1.f, 9 - ex) : 1.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    uint32_t u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = pack_f16x2(qf[m][2 * j] * qs, qf[m][2 * j + 1] * qs);
    qop[m][lane] = uint4{u[0], u[1], u[2], u[3]};
  }
  return p.scale_log2 * (qmax > 0.f ? ldexpf(1.f, ex - 1) : 256.f);
}

// The rotation table in LDS: rtab[buf][f / 2][t - tok0][f % 2] for the 16
// tokens t of a tile and f < 64, two tiles (a lane's frequencies f, f + 1 are
// one 16-byte row and the 16 tokens' rows are contiguous), the rotation of
// each frequency over one tile (rstep) and omega_f / (2 pi) for the exact
// evaluations (orev).
struct RotTable {
  float2 rtab[2][32][kTile][2];
  float2 rstep[64];
  double orev[64];
};

// Thread entry e of the table is (token tid % 16, frequency tid / 16 + e *
// kThreads / 16): one per-thread slot plus e times a constant stride. Every
// kAnchor tiles the entries are evaluated from the angle; in between a
// tile's entry is the previous tile's times the 16-position step of its
// frequency (one exact complex product). Without rotary embedding the table
// holds (2^-8, 0).
template <int kThreads>
struct Rot {
  static constexpr int kRE = 1024 / kThreads;          // entries per thread
  static constexpr int kFStep = kThreads / 16;         // frequency step between entries
  static constexpr int kSlotStep = (kFStep / 2) * kTile * 2;   // float2 elements between entries
  RotTable& t;
  int f0, gt;
  bool rope;
  __device__ __forceinline__ Rot(RotTable& tab, int tid, bool r)
      : t(tab), f0(tid >> 4), gt(tid & 15), rope(r) {}
  // the per-frequency constants; a barrier must follow before any use
  __device__ __forceinline__ void init(const DecodeParams& p, int tid) {
    if (tid < 64) {
      float c = 1.f, sn = 0.f;
      if (rope) rope_cos_sin(p.omega_rev[tid], kTile, c, sn);
      t.rstep[tid] = float2{c, sn};
      t.orev[tid] = p.omega_rev[tid];
    }
  }
  __device__ __forceinline__ float2* slot(int buf) { return &t.rtab[buf][f0 >> 1][gt][f0 & 1]; }
  // the table of the tile starting at tok0 into buffer buf, from the angles
  __device__ __forceinline__ void exact(int tok0, int buf) {
    float2* dst = slot(buf);
#pragma unroll
    for (int e = 0; e < kRE; ++e) {
      float c = 1.f, sn = 0.f;
      if (rope) rope_cos_sin(t.orev[f0 + e * kFStep], tok0 + gt, c, sn);
      dst[e * kSlotStep] = float2{c * kKeyScale, sn * kKeyScale};
    }
  }
  // the table of tile nt into buffer nt & 1 from tile nt - 1's (buffer
  // (nt - 1) & 1, which nothing rewrites before the next barrier): every
  // read first (step_read), then the products and writes (step_write); the
  // two halves may sit apart in a schedule
  struct StepRegs {
    float2 o[kRE], st[kRE];
  };
  __device__ __forceinline__ void step_read(int nt, StepRegs& r) {
    const float2* src = slot((nt - 1) & 1);
#pragma unroll
    for (int e = 0; e < kRE; ++e) {
      r.o[e] = src[e * kSlotStep];
      r.st[e] = t.rstep[f0 + e * kFStep];
    }
  }
  __device__ __forceinline__ void step_write(int nt, const StepRegs& r) {
    float2* dst = slot(nt & 1);
#pragma unroll
    for (int e = 0; e < kRE; ++e)
      dst[e * kSlotStep] = float2{r.o[e].x * r.st[e].x - r.o[e].y * r.st[e].y,
                                  r.o[e].y * r.st[e].x + r.o[e].x * r.st[e].y};
  }
  __device__ __forceinline__ void step(int nt) {
    StepRegs r;
    step_read(nt, r);
    step_write(nt, r);
  }
};

}  // namespace wave
}  // namespace palu
