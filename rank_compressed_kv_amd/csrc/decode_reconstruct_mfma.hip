// Context-split decode kernel for the reconstruct mode (keys rebuilt per tile
// and rotated), bf16 latents, on the gfx950 matrix cores.
//
// Method (Palu author response on OpenReview): K_i = H_i B_i is rebuilt from the
// cached latents and kept on chip ("Why Palu Requires Fewer Global Memory
// Access": tiling and fusion keep the reconstructed K in shared memory and
// registers); the rotary embedding is the reason keys must be rebuilt at all
// (clarification of W1), and it turns each pair by the 2x2 rotation of the
// CommVQ response (proof of Property 1). Values stay in latent space: the
// weighted sum runs over h_v rows and B_v is applied in the merge pass.
//
// Shapes served: head_dim 128, at most four query heads per KV head, rank 32,
// 64, 128, 256 or 512, any number of KV heads per group (the head slice is the
// largest of 4, 2, 1 heads that divides it and leaves every wave a 16-row block
// of value latents).
// A workgroup owns one (batch, group, context split, slice of HW KV heads) and
// walks its 16-token tiles. A KV head's 128 columns are 8 blocks of 16; the
// rotary pair (f, f + 64) joins block c with block c + 4. Each wave owns kP
// such block pairs of one head (2 kP blocks), so rotation never leaves a wave,
// and its slice of B_k^T (32 kP columns x r, read once from a transposed copy
// in the workspace) stays in registers for the whole split:
//   rank <= 256: kP = 2, two waves per head, up to four heads (eight waves),
//                two heads at rank 64 and one at rank 32;
//   rank 512:    kP = 1, four waves per head, up to two heads (eight waves).
// When the slice is smaller than the group, the workgroups of one context
// split that differ only in their head slice get launch ids 8 apart, which
// places them on the same XCD at about the same time, so the latent tiles they
// all read are shared through that XCD's L2 (those loads use ordinary caching;
// a split read by one workgroup streams with non-temporal loads).
// Per tile:
//   keys     K^T[16 cols x 16 tok] = B_k^T[cols x r] * H_k^T[r x tok] per block,
//            bf16 MFMA 16x16x32, H_k from the tile in LDS. Lane l ends up with
//            columns 16*cb + 4*(l/16) + i of token l%16.
//   rotate   in place with cos/sin of t*omega_f from a table in LDS that all
//            waves share; the table advances by one exact complex product per
//            tile (t grows by 16) and is recomputed from the angle every
//            kAnchor tiles.
//   scores   that layout is the A operand of a 16x16x16 MFMA (k = the block's
//            16 columns): S^T[tok x q heads] = K_rot * Q^T with keys split hi +
//            lo bf16 (two MFMAs, ~16 bits kept) and exact bf16 q; each wave
//            stores its partial scores in LDS.
//   softmax  online, base 2, run by every wave for all query heads of the
//            slice (lane ln adds the partial scores of query head ln's KV
//            head), so the weights and rescale factors stay in registers.
//   values   wave w adds H_v^T[r slice w] * P^T for all query heads of the
//            slice (bf16 MFMA 16x16x16, P split hi + lo), gathering value
//            columns from the tile in LDS (four-row groups offset by 32 B:
//            conflict-free).
// Loads: 16-byte pieces of each tile go through two register stages (two tiles
// in flight) into a ring of three LDS tile buffers; rows past the split's end
// are clamped to its last valid row and masked. One workgroup barrier per
// tile, after the partial scores (the partial scores and the rotation table
// are double-buffered); it orders LDS only, so the loads stay in flight.
#include <math.h>

#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 16;        // tokens per tile
constexpr int kD = 128;          // head dim
constexpr int kNBuf = 3;         // LDS tile buffers
constexpr int kAnchor = 32;      // tiles between exact cos/sin evaluations

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

// a ~ hi + lo with hi = bf16(a) and lo = bf16(a - hi) (round to nearest even,
// one packed conversion per pair): about 16 significant bits in two bf16 terms.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a, b}, bf16x2));
  const float ah = __uint_as_float(hi << 16), bh = __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{a - ah, b - bh}, bf16x2));
}
__device__ __forceinline__ void split_bf16x4(floatx4 v, short4v& hi, short4v& lo) {
  uint32_t h0, h1, l0, l1;
  split_bf16x2(v[0], v[1], h0, l0);
  split_bf16x2(v[2], v[3], h1, l1);
  hi = __builtin_bit_cast(short4v, uint2{h0, h1});
  lo = __builtin_bit_cast(short4v, uint2{l0, l1});
}
__device__ __forceinline__ float lane_xor(float x, int addr) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(x)));
}

// K tile: rows padded by 32 B (a row stride of 32 mod 64 bytes keeps the 16
// rows of an operand read free of bank conflicts on gfx950)
template <int R>
constexpr int kKStride = 2 * R + 32;
// V tile: groups of four rows offset by 32 B (conflict-free column gathers)
template <int R>
__device__ __forceinline__ int vtile_off(int row, int cb) {
  return row * (2 * R) + (row >> 2) * 32 + cb;
}
template <int R>
constexpr int kVBytes = kTile * 2 * R + 3 * 32;

template <int R, int kP, int HW>
struct Shape {
  static constexpr int kNB = 2 * kP;             // column blocks per wave
  static constexpr int kWPH = 4 / kP;            // waves per KV head
  static constexpr int kWaves = HW * kWPH;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRB = R / (16 * kWaves);  // 16-row value blocks per wave
  static constexpr int kPieces = (2 * R + kThreads - 1) / kThreads;  // 16-B pieces per matrix
  static constexpr int kRE = 1024 / kThreads;    // rotation-table entries per thread
  static_assert(kRB >= 1 && kRB * 16 * kWaves == R, "rank must split evenly over the waves");
};

template <int R, int kWaves>
struct Smem {
  char k[kNBuf][kTile * kKStride<R>];
  char v[kNBuf][kVBytes<R>];
  // partial scores of each wave (its lanes' float4), two tiles; a wave's block
  // is padded by 32 B so that the blocks of two KV heads' waves, read by one
  // 8-lane group, fall on different LDS banks
  float4 spart[2][kWaves][66];
  // cos, sin of t * omega_f for the 16 tokens t of a tile, f < 64, two tiles:
  // rtab[buf][f / 2][t - tok0][f % 2]: a lane's frequencies f, f + 1 are one
  // 16-byte row, and the 16 tokens' rows are contiguous (conflict-free reads)
  float2 rtab[2][32][kTile][2];
};

template <int R, int kP, int HW, bool kShared>
__global__ __launch_bounds__((Shape<R, kP, HW>::kThreads)) void split_reconstruct_mfma_kernel(
    DecodeParams p) {
  using S = Shape<R, kP, HW>;
  constexpr int kNB = S::kNB, kWPH = S::kWPH, kWaves = S::kWaves, kThreads = S::kThreads;
  constexpr int kRB = S::kRB, kPieces = S::kPieces, kRE = S::kRE;
  const int nslice = p.s / HW;
  const SplitUnit un = split_unit(p.n_split, p.G, p.B, nslice);
  if (!un.live) return;
  const int split = un.split, g = un.g, b = un.b, hs = un.hs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, kb = lane >> 4;
  const int jl = wave / kWPH, part = wave % kWPH;        // KV head in the slice, column part
  const int n = clamp_len(p.lens, b, p.L);
  const int s0 = split * p.split_tokens;
  if (s0 >= n) return;                                   // whole workgroup
  const int t1 = min(n, s0 + p.split_tokens);
  const int last = t1 - 1;
  const int gqa = p.gqa;                                 // query heads per KV head (<= 4)
  const int nqs = HW * gqa;                              // query heads of the slice (<= 16)
  const int head0 = g * p.nq + hs * nqs;                 // first query head of the slice
  const int kvh = hs * HW + jl;                          // KV head within the group

  __shared__ Smem<R, kWaves> sm;

  // owned 16-column blocks: pair i (< kP) joins block part*kP + i and its +4 partner
  auto cbs = [part](int j) { return part * kP + (j % kP) + 4 * (j / kP); };

  // ---- operands held for the whole split -----------------------------------
  // B_k^T as the A operand: lane (ln, kb) of block j, chunk c holds column
  // 16*cbs(j) + ln, latents 32c + 8kb .. +8
  const uint16_t* Bt = static_cast<const uint16_t*>(p.bkt) +
                       (static_cast<size_t>(g) * p.Dg + kvh * kD) * R;
  uint4 bk[kNB][R / 32];
#pragma unroll
  for (int j = 0; j < kNB; ++j)
#pragma unroll
    for (int c = 0; c < R / 32; ++c)
      bk[j][c] = *reinterpret_cast<const uint4*>(Bt + static_cast<size_t>(16 * cbs(j) + ln) * R + 32 * c + 8 * kb);
  // q of this KV head's query heads as the score B operand: lane (ln = head
  // slot, kb) of block j holds columns 16*cbs(j) + 4kb .. +4 (exact bf16)
  short4v qb[kNB];
  {
    const bool valid = ln < gqa;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                           (static_cast<size_t>(b) * p.Hq + head0 + jl * gqa + (valid ? ln : 0)) * kD;
#pragma unroll
    for (int j = 0; j < kNB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) qb[j][e] = valid ? static_cast<short>(qrow[16 * cbs(j) + 4 * kb + e]) : 0;
  }

  // rotation table: thread entry e is (token gt = idx % 16, frequency
  // f = idx / 16) with idx = tid + e * kThreads; it keeps cos/sin of
  // (tok0 + gt) * omega_f and writes them for each tile; every kAnchor tiles
  // they are evaluated from the angle, in between they advance by one exact
  // complex product with the 16-position step.
  const bool rope = p.rope != 0;
  float rc[kRE], rs[kRE], stc[kRE], sts[kRE];
#pragma unroll
  for (int e = 0; e < kRE; ++e) {
    rc[e] = 1.f; rs[e] = 0.f; stc[e] = 1.f; sts[e] = 0.f;
    if (rope) rope_cos_sin(p.omega_rev[(tid + e * kThreads) >> 4], kTile, stc[e], sts[e]);
  }
  auto rope_exact = [&](int tok0) {
    if (rope) {
#pragma unroll
      for (int e = 0; e < kRE; ++e) {
        const int idx = tid + e * kThreads;
        rope_cos_sin(p.omega_rev[idx >> 4], tok0 + (idx & 15), rc[e], rs[e]);
      }
    }
  };
  auto rope_advance = [&]() {
#pragma unroll
    for (int e = 0; e < kRE; ++e) {
      const float c1 = rc[e] * stc[e] - rs[e] * sts[e], s1 = rs[e] * stc[e] + rc[e] * sts[e];
      rc[e] = c1; rs[e] = s1;
    }
  };
  auto rope_write = [&](int buf) {
#pragma unroll
    for (int e = 0; e < kRE; ++e) {
      const int idx = tid + e * kThreads, f = idx >> 4;
      sm.rtab[buf][f >> 1][idx & 15][f & 1] = float2{rc[e], rs[e]};
    }
  };
  // the tables of tiles 0 and 1; the thread state then stands at tile 1
  rope_exact(s0);
  rope_write(0);
  if (rope) rope_advance();
  rope_write(1);
  const int x16 = (lane ^ 16) << 2, x32 = (lane ^ 32) << 2;   // bpermute addresses

  // ---- softmax state: every wave keeps it for all query heads of the slice
  // (lane ln = query head ln of the slice), so the weights never go through LDS
  float m = -INFINITY, l = 0.f;
  // value-latent sums for all query heads of the slice over this wave's r
  // slice: acc[rb] holds r = wave*R/kWaves + 16*rb + 4*kb + i for head slot ln
  floatx4 acc[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) acc[rb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const size_t row0 = (static_cast<size_t>(b) * p.G + g) * p.L;
  const uint16_t* Hk = static_cast<const uint16_t*>(p.h_k) + row0 * R;
  const uint16_t* Hv = static_cast<const uint16_t*>(p.h_v) + row0 * R;
  const int ntiles = (t1 - s0 + kTile - 1) / kTile;

  // Keys and scores of tile it (needs the K tile and the rotation table of
  // tile it): rebuild the owned key blocks, rotate them and store this wave's
  // partial scores.
  auto keys_scores = [&](int it) {
    const char* kt = sm.k[it % kNBuf];
    // keys of the owned blocks: K^T[16*cbs(j) + 4kb + i][token ln]
    floatx4 kk[kNB];
#pragma unroll
    for (int j = 0; j < kNB; ++j) kk[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < R / 32; ++c) {
      const bf16x8 h = as_bf16x8(*reinterpret_cast<const uint4*>(kt + ln * kKStride<R> + 2 * (32 * c + 8 * kb)));
#pragma unroll
      for (int j = 0; j < kNB; ++j)
        kk[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(bk[j][c]), h, kk[j], 0, 0, 0);
    }
    // rotate the pairs (f, f + 64): f = 16*cbs(i) + 4kb + e, token ln
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      // frequencies 16 cbs(i) + 4 kb + (0, 1) and (2, 3)
      const int f2 = 2 * (4 * cbs(i) + kb);
      const float4 r01 = *reinterpret_cast<const float4*>(&sm.rtab[it & 1][f2][ln][0]);
      const float4 r23 = *reinterpret_cast<const float4*>(&sm.rtab[it & 1][f2 + 1][ln][0]);
      const float c4[4] = {r01.x, r01.z, r23.x, r23.z}, s4[4] = {r01.y, r01.w, r23.y, r23.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = kk[i][e], y = kk[i + kP][e];
        kk[i][e] = x * c4[e] - y * s4[e];
        kk[i + kP][e] = x * s4[e] + y * c4[e];
      }
    }
    // partial scores S^T[token 4kb+i][head slot ln] over the owned blocks
    floatx4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      short4v ah, al;
      split_bf16x4(kk[j], ah, al);
      s1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, qb[j], s1, 0, 0, 0);
      s2 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, qb[j], s2, 0, 0, 0);
    }
    const floatx4 sc = s1 + s2;
    sm.spart[it & 1][wave][lane] = float4{sc[0], sc[1], sc[2], sc[3]};
  };
  // Softmax and values of tile it (after every wave's partial scores are in
  // LDS). Every wave runs the online softmax of all query heads of the slice,
  // lane ln for query head ln (KV head ln / gqa, whose waves' partial scores
  // it adds), and multiplies its own r slice of the value sums; the weights
  // stay in the lane that computed them.
  auto softmax_values = [&](int it) {
    const int tok0 = s0 + it * kTile;
    const bool hv = ln < nqs;
    floatx4 sc = {0.f, 0.f, 0.f, 0.f};
    if (hv) {
      const int jh = ln / gqa, slot = ln - jh * gqa;
#pragma unroll
      for (int w = 0; w < kWPH; ++w) {
        const float4 o = sm.spart[it & 1][jh * kWPH + w][slot + 16 * kb];
        sc[0] += o.x; sc[1] += o.y; sc[2] += o.z; sc[3] += o.w;
      }
    }
    sc *= p.scale_log2;
    if (tok0 + kTile > t1) {                             // last tile of the split
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tok0 + 4 * kb + i >= t1) sc[i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, lane_xor(mx, x16));
    mx = fmaxf(mx, lane_xor(mx, x32));
    const float mn = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    floatx4 pv;
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(sc[i] - mn);
    l = l * alpha + ((pv[0] + pv[1]) + (pv[2] + pv[3]));
    short4v ph, pl;
    split_bf16x4(pv, ph, pl);
    const char* vt = sm.v[it % kNBuf];
    const char* vb = vt + vtile_off<R>(4 * kb, 2 * (wave * (R / kWaves) + ln));
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      short4v a;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = *reinterpret_cast<const short*>(vb + e * (2 * R) + 32 * rb);
      acc[rb] *= alpha;
      acc[rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, ph, acc[rb], 0, 0, 0);
      acc[rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pl, acc[rb], 0, 0, 0);
    }
  };
  // the rotation table of tile nt into buffer nt & 1 (the thread state moves
  // from tile nt - 1 to nt)
  auto rope_next = [&](int nt) {
    if (nt % kAnchor == 0) rope_exact(s0 + nt * kTile);
    else if (rope) rope_advance();
    rope_write(nt & 1);
  };

  // Loads: thread piece i (< kPieces) is the 16-byte piece tid + i*kThreads of
  // the tile (byte 16*that in a row-major tile of 16 rows), if below 2R. Two
  // tiles wait in registers (stages a and b, vector types so they stay in
  // registers) and two ahead of the one being consumed are in LDS.
  typedef uint32_t u32v __attribute__((ext_vector_type(4 * kPieces)));
  auto fetch = [&](int tok0, u32v& k, u32v& v) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int pc = tid + i * kThreads;
      if (pc < 2 * R) {
        const int prow = (pc * 16) / (2 * R), pcol = (pc * 16) % (2 * R);
        const size_t row = static_cast<size_t>(min(tok0 + prow, last)) * (2 * R) + pcol;
        const uint4 a = load_tile16<kShared>(reinterpret_cast<const char*>(Hk) + row);
        const uint4 c = load_tile16<kShared>(reinterpret_cast<const char*>(Hv) + row);
        k[4 * i] = a.x; k[4 * i + 1] = a.y; k[4 * i + 2] = a.z; k[4 * i + 3] = a.w;
        v[4 * i] = c.x; v[4 * i + 1] = c.y; v[4 * i + 2] = c.z; v[4 * i + 3] = c.w;
      }
    }
  };
  auto put = [&](int buf, const u32v& k, const u32v& v) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int pc = tid + i * kThreads;
      if (pc < 2 * R) {
        const int prow = (pc * 16) / (2 * R), pcol = (pc * 16) % (2 * R);
        *reinterpret_cast<uint4*>(sm.k[buf] + prow * kKStride<R> + pcol) =
            uint4{k[4 * i], k[4 * i + 1], k[4 * i + 2], k[4 * i + 3]};
        *reinterpret_cast<uint4*>(sm.v[buf] + vtile_off<R>(prow, pcol)) =
            uint4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
      }
    }
  };

  // One barrier per tile. Iteration it (after the barrier that follows the
  // partial scores of tile it): the softmax and values of tile it; the copy
  // of tile it+2 into LDS (its buffer last held tile it-1, finished before
  // that barrier) and the request of tile it+4 into the same register stage;
  // the rotation table of tile it+2 (its buffer last served tile it); the
  // keys and partial scores of tile it+1 (their buffer last served tile
  // it-1); the barrier. Two register stages alternate, so each request has
  // two iterations to arrive; the barrier orders LDS only, so requests stay
  // in flight across it; the requests are unconditional (rows past the split
  // clamp to its last one).
  u32v ka, va, kb2, vb2;
  fetch(s0, ka, va);
  put(0, ka, va);
  fetch(s0 + kTile, ka, va);
  put(1, ka, va);
  fetch(s0 + 2 * kTile, ka, va);
  fetch(s0 + 3 * kTile, kb2, vb2);
  barrier_lds();
  keys_scores(0);
  barrier_lds();
  // With eight waves, each SIMD runs waves w and w + 4: the upper four take
  // the keys of tile it+1 before the softmax of tile it (the two touch
  // different buffers), so one wave's key MFMAs overlap the other's softmax.
  const bool keys_first = kWaves >= 8 && wave >= kWaves / 2;
  auto iteration = [&](int it, u32v& k, u32v& v) {
    if (keys_first && it + 1 < ntiles) keys_scores(it + 1);
    softmax_values(it);
    put((it + 2) % kNBuf, k, v);
    fetch(s0 + (it + 4) * kTile, k, v);
    if (it + 2 < ntiles) rope_next(it + 2);
    if (!keys_first && it + 1 < ntiles) keys_scores(it + 1);
    barrier_lds();
  };
  for (int it = 0; it < ntiles; it += 2) {
    iteration(it, ka, va);
    if (it + 1 >= ntiles) break;
    iteration(it + 1, kb2, vb2);
  }

  // ---- partials: this wave's r slice for every query head; (m, l) by wave 0
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (wave == 0 && ln < nqs && kb == 0) {
    const int head = head0 + ln;
    const size_t slot = (static_cast<size_t>(b) * p.Hq + head) * p.n_split + split;
    p.part_ml[slot * 2] = m;
    p.part_ml[slot * 2 + 1] = l;
  }
  if (ln < nqs) {
    const int head = head0 + ln;
    const size_t slot = (static_cast<size_t>(b) * p.Hq + head) * p.n_split + split;
    float* u = p.part_u + slot * R + wave * (R / kWaves);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      *reinterpret_cast<float4*>(u + 16 * rb + 4 * kb) = float4{acc[rb][0], acc[rb][1], acc[rb][2], acc[rb][3]};
  }
}

// B_k [G][r][D_g] -> B_k^T [G][D_g][r] through 32x32 LDS tiles
template <typename T>
__global__ __launch_bounds__(256) void transpose_bk_kernel(DecodeParams p) {
  __shared__ T tile[32][33];
  const int g = blockIdx.z;
  const int c0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;   // 8 rows per pass
  const T* src = static_cast<const T*>(p.b_k) + static_cast<size_t>(g) * p.r * p.Dg;
  T* dst = static_cast<T*>(p.bkt) + static_cast<size_t>(g) * p.Dg * p.r;
  for (int y = ty; y < 32; y += 8) {
    const int k = k0 + y, c = c0 + tx;
    if (k < p.r && c < p.Dg) tile[y][tx] = src[static_cast<size_t>(k) * p.Dg + c];
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    const int c = c0 + y, k = k0 + tx;
    if (k < p.r && c < p.Dg) dst[static_cast<size_t>(c) * p.r + k] = tile[tx][y];
  }
}

template <int R, int kP, int HW>
hipError_t launch_shape(const DecodeParams& p, hipStream_t st) {
  using S = Shape<R, kP, HW>;
  const int nslice = p.s / HW;
  if (nslice == 1) {
    const dim3 grid(p.n_split, p.G, p.B);
    split_reconstruct_mfma_kernel<R, kP, HW, false><<<grid, S::kThreads, 0, st>>>(p);
  } else {
    const long ids = split_unit_ids(p.n_split, p.G, p.B, nslice);
    if (ids == 0) return hipErrorInvalidValue;
    split_reconstruct_mfma_kernel<R, kP, HW, true>
        <<<dim3(static_cast<unsigned>(ids)), S::kThreads, 0, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

int reconstruct_heads_per_wg(int r, int s) {
  // every wave needs at least one 16-row block of value latents: r >= 16 * waves
  if (r == 512 || r == 64) return s % 2 == 0 ? 2 : 1;
  if (r == 128 || r == 256) return s % 4 == 0 ? 4 : (s % 2 == 0 ? 2 : 1);
  if (r == 32) return 1;
  return 0;
}

int reconstruct_waves_per_wg(int r, int s) {
  const int hw = reconstruct_heads_per_wg(r, s);
  return (r == 512 ? 4 : 2) * hw;
}

bool reconstruct_mfma_supported(const DecodeParams& p, int dtype) {
  return dtype == 1 && p.d == kD && p.gqa <= 4 && reconstruct_heads_per_wg(p.r, p.s) > 0;
}

hipError_t launch_transpose_bk(const DecodeParams& p, int dtype, hipStream_t st) {
  const dim3 grid((p.Dg + 31) / 32, (p.r + 31) / 32, p.G);
  if (dtype == 0) transpose_bk_kernel<float><<<grid, 256, 0, st>>>(p);
  else transpose_bk_kernel<uint16_t><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_split_reconstruct_mfma(const DecodeParams& p, hipStream_t st) {
  switch (p.r * 8 + reconstruct_heads_per_wg(p.r, p.s)) {
    case 128 * 8 + 4: return launch_shape<128, 2, 4>(p, st);
    case 128 * 8 + 2: return launch_shape<128, 2, 2>(p, st);
    case 128 * 8 + 1: return launch_shape<128, 2, 1>(p, st);
    case 256 * 8 + 4: return launch_shape<256, 2, 4>(p, st);
    case 256 * 8 + 2: return launch_shape<256, 2, 2>(p, st);
    case 256 * 8 + 1: return launch_shape<256, 2, 1>(p, st);
    case 512 * 8 + 2: return launch_shape<512, 1, 2>(p, st);
    case 512 * 8 + 1: return launch_shape<512, 1, 1>(p, st);
    case 64 * 8 + 2: return launch_shape<64, 2, 2>(p, st);
    case 64 * 8 + 1: return launch_shape<64, 2, 1>(p, st);
    case 32 * 8 + 1: return launch_shape<32, 2, 1>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace palu
