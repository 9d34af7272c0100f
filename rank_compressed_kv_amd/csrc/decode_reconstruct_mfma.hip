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
// Shape served: head_dim 128, four KV heads per group, at most four query heads
// per KV head, rank 128 or 256. One workgroup owns one (batch, group, context
// split) and walks its 16-token tiles; its eight waves are (KV head, half):
// a wave owns the 16-column blocks {2h, 2h+1, 2h+4, 2h+5} of its head, so the
// rotary pair (f, f + 64) never leaves a wave, and its slice of B_k^T (r x 64
// columns, read once from a transposed copy in the workspace) stays in
// registers for the whole split. Per tile:
//   keys     K^T[16 cols x 16 tok] = B_k^T[cols x r] * H_k^T[r x tok] per block,
//            bf16 MFMA 16x16x32, H_k from the tile in LDS. Lane l ends up with
//            columns 16*cb + 4*(l/16) + i of token l%16.
//   rotate   in place; cos/sin of t*omega_f advance by one exact complex
//            product per tile (t grows by 16) and are recomputed from the angle
//            every kAnchor tiles.
//   scores   that layout is the A operand of a 16x16x16 MFMA (k = the block's
//            16 columns): S^T[tok x q heads] = K_rot * Q^T with keys split hi +
//            lo bf16 (two MFMAs, ~16 bits kept) and exact bf16 q; the two
//            halves of a head add their partial scores through LDS.
//   softmax  online, base 2, by the first wave of each head.
//   values   P and the rescale factors go through LDS; wave w adds
//            H_v^T[r slice w] * P^T for all query heads of the group (bf16 MFMA
//            16x16x16, P split hi + lo), gathering value columns from the tile
//            in LDS (four-row groups offset by 32 B: conflict-free).
// Loads: 16-byte pieces of each tile are moved into kStages register stages
// (kStages tiles in flight) and then into a ring of three LDS tile buffers;
// rows past the split's end are clamped to its last valid row and masked.
#include <math.h>

#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kHeads = 4;        // KV heads per group
constexpr int kWaves = 2 * kHeads;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16;        // tokens per tile
constexpr int kD = 128;          // head dim
constexpr int kNB = 3;           // LDS tile buffers
constexpr int kAnchor = 32;      // tiles between exact cos/sin evaluations

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

// K tile: rows padded by 16 B so the 16 rows of an operand read hit distinct banks
template <int R>
constexpr int kKStride = 2 * R + 16;
// V tile: groups of four rows offset by 32 B (conflict-free column gathers)
template <int R>
__device__ __forceinline__ int vtile_off(int row, int cb) {
  return row * (2 * R) + (row >> 2) * 32 + cb;
}
template <int R>
constexpr int kVBytes = kTile * 2 * R + 3 * 32;

template <int R>
struct Smem {
  char k[kNB][kTile * kKStride<R>];
  char v[kNB][kVBytes<R>];
  float4 spart[kWaves][64];   // partial scores of each wave (its lanes' float4)
  float pt[16][kTile];        // P of the group's query heads for the current tile
  float alpha[16];            // rescale factor of each query head for this tile
  // cos, sin of t * omega_f for the 16 tokens t of the current tile, f < 64:
  // rtab[f / 4][t - tok0][f % 4] (a lane's four frequencies are 32 contiguous B)
  float2 rtab[16][kTile][4];
};

// A tile is 16 rows x R bf16 per matrix = 2R pieces of 16 B; threads below 2R
// move one piece of H_k and one of H_v. Byte offset of a thread's piece within
// a row-major tile of 16 rows:
template <int R>
__device__ __forceinline__ int piece_row(int tid) { return (tid * 16) / (2 * R); }
template <int R>
__device__ __forceinline__ int piece_col(int tid) { return (tid * 16) % (2 * R); }

template <int R>
__global__ __launch_bounds__(kThreads) void split_reconstruct_mfma_kernel(DecodeParams p) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, kb = lane >> 4;
  const int jl = wave >> 1, half = wave & 1;             // KV head in the group, column half
  const int n = clamp_len(p.lens, b, p.L);
  const int s0 = split * p.split_tokens;
  if (s0 >= n) return;                                   // whole workgroup
  const int t1 = min(n, s0 + p.split_tokens);
  const int last = t1 - 1;
  const int gqa = p.gqa;                                 // query heads per KV head (<= 4)
  const int nq = p.nq;                                   // query heads of the group (<= 16)

  __shared__ Smem<R> sm;

  // owned 16-column blocks: cbs(j) = 2*half + j (j < 2) and their +64 partners
  auto cbs = [half](int j) { return 2 * half + (j & 1) + 4 * (j >> 1); };

  // ---- operands held for the whole split -----------------------------------
  // B_k^T as the A operand: lane (ln, kb) of block j, chunk c holds column
  // 16*cbs(j) + ln, latents 32c + 8kb .. +8
  const uint16_t* Bt = static_cast<const uint16_t*>(p.bkt) +
                       (static_cast<size_t>(g) * p.Dg + jl * kD) * R;
  uint4 bk[4][R / 32];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int c = 0; c < R / 32; ++c)
      bk[j][c] = *reinterpret_cast<const uint4*>(Bt + static_cast<size_t>(16 * cbs(j) + ln) * R + 32 * c + 8 * kb);
  // q of this KV head's query heads as the score B operand: lane (ln = head
  // slot, kb) of block j holds columns 16*cbs(j) + 4kb .. +4 (exact bf16)
  short4v qb[4];
  {
    const bool valid = ln < gqa;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                           (static_cast<size_t>(b) * p.Hq + g * nq + jl * gqa + (valid ? ln : 0)) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) qb[j][e] = valid ? static_cast<short>(qrow[16 * cbs(j) + 4 * kb + e]) : 0;
  }
  // rotation table: thread (gt = tid % 16, fa = tid / 16) keeps cos/sin of
  // (tok0 + gt) * omega for f = fa and fa + 32 and writes them for each tile;
  // every kAnchor tiles they are evaluated from the angle, in between they
  // advance by one exact complex product with the 16-position step.
  const bool rope = p.rope != 0;
  const int gt = tid & 15, fa = tid >> 4, fb = fa + 32;
  float ca = 1.f, sa = 0.f, cb = 1.f, sb = 0.f;
  float stca = 1.f, stsa = 0.f, stcb = 1.f, stsb = 0.f;
  if (rope) {
    rope_cos_sin(p.omega_rev[fa], kTile, stca, stsa);
    rope_cos_sin(p.omega_rev[fb], kTile, stcb, stsb);
  }
  auto rope_exact = [&](int tok0) {
    if (rope) {
      rope_cos_sin(p.omega_rev[fa], tok0 + gt, ca, sa);
      rope_cos_sin(p.omega_rev[fb], tok0 + gt, cb, sb);
    }
  };
  auto rope_advance = [&]() {
    const float c1 = ca * stca - sa * stsa, s1 = sa * stca + ca * stsa;
    const float c2 = cb * stcb - sb * stsb, s2 = sb * stcb + cb * stsb;
    ca = c1; sa = s1; cb = c2; sb = s2;
  };
  auto rope_write = [&]() {
    sm.rtab[fa >> 2][gt][fa & 3] = float2{ca, sa};
    sm.rtab[fb >> 2][gt][fb & 3] = float2{cb, sb};
  };
  rope_exact(s0);
  rope_write();
  const int x16 = (lane ^ 16) << 2, x32 = (lane ^ 32) << 2;   // bpermute addresses

  // ---- softmax state of the owned query heads (lane ln = head slot) ---------
  float m = -INFINITY, l = 0.f;
  // value-latent sums for all query heads over this wave's r slice:
  // acc[rb] holds r = wave*R/8 + 16*rb + 4*kb + i for query head ln
  constexpr int kRB = R / (16 * kWaves);
  floatx4 acc[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) acc[rb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const size_t row0 = (static_cast<size_t>(b) * p.G + g) * p.L;
  const uint16_t* Hk = static_cast<const uint16_t*>(p.h_k) + row0 * R;
  const uint16_t* Hv = static_cast<const uint16_t*>(p.h_v) + row0 * R;
  const int ntiles = (t1 - s0 + kTile - 1) / kTile;

  auto process = [&](int it) {
    const int tok0 = s0 + it * kTile;
    const char* kt = sm.k[it % kNB];
    const char* vt = sm.v[it % kNB];
    // keys of the owned blocks: K^T[16*cbs(j) + 4kb + i][token ln]
    floatx4 kk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kk[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < R / 32; ++c) {
      const bf16x8 h = as_bf16x8(*reinterpret_cast<const uint4*>(kt + ln * kKStride<R> + 2 * (32 * c + 8 * kb)));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        kk[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(bk[j][c]), h, kk[j], 0, 0, 0);
    }
    // rotate the pairs (f, f + 64): f = 16*cbs(j) + 4kb + i, token ln
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float4* rt = reinterpret_cast<const float4*>(&sm.rtab[4 * cbs(j) + kb][ln][0]);
      const float4 r01 = rt[0];
      const float4 r23 = rt[1];
      const float c4[4] = {r01.x, r01.z, r23.x, r23.z}, s4[4] = {r01.y, r01.w, r23.y, r23.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = kk[j][i], y = kk[j + 2][i];
        kk[j][i] = x * c4[i] - y * s4[i];
        kk[j + 2][i] = x * s4[i] + y * c4[i];
      }
    }
    // partial scores S^T[token 4kb+i][head slot ln] over the owned blocks
    floatx4 sc = {0.f, 0.f, 0.f, 0.f}, sc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      short4v ah, al;
      split_bf16x4(kk[j], ah, al);
      sc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, qb[j], sc, 0, 0, 0);
      sc2 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, qb[j], sc2, 0, 0, 0);
    }
    sc += sc2;
    sm.spart[wave][lane] = float4{sc[0], sc[1], sc[2], sc[3]};
    __syncthreads();
    // every wave has rotated this tile: the table can take the next one
    if (it + 1 < ntiles) {
      if ((it + 1) % kAnchor == 0) rope_exact(tok0 + kTile);
      else if (rope) rope_advance();
      rope_write();
    }
    // softmax of the owned heads by the first wave of each KV head
    if (half == 0) {
      const float4 o = sm.spart[wave + 1][lane];
      sc[0] += o.x; sc[1] += o.y; sc[2] += o.z; sc[3] += o.w;
      sc *= p.scale_log2;
      if (tok0 + kTile > t1) {                           // last tile of the split
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
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(sc[i] - mn);
      l = l * alpha + ((pv[0] + pv[1]) + (pv[2] + pv[3]));
      if (ln < gqa) {
        const int hg = jl * gqa + ln;                    // query head within the group
        *reinterpret_cast<float4*>(&sm.pt[hg][4 * kb]) = float4{pv[0], pv[1], pv[2], pv[3]};
        if (kb == 0) sm.alpha[hg] = alpha;
      }
    }
    __syncthreads();
    // values: this wave's r slice for all query heads of the group
    {
      const bool hv = ln < nq;
      const float4 pp = hv ? *reinterpret_cast<const float4*>(&sm.pt[ln][4 * kb]) : float4{0.f, 0.f, 0.f, 0.f};
      const float al = hv ? sm.alpha[ln] : 1.f;
      short4v ph, pl;
      split_bf16x4(floatx4{pp.x, pp.y, pp.z, pp.w}, ph, pl);
      const char* vb = vt + vtile_off<R>(4 * kb, 2 * (wave * (R / kWaves) + ln));
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        short4v a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = *reinterpret_cast<const short*>(vb + e * (2 * R) + 32 * rb);
        acc[rb] *= al;
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, ph, acc[rb], 0, 0, 0);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pl, acc[rb], 0, 0, 0);
      }
    }
  };

  // Loads: each thread below 2R moves one 16-byte piece of H_k and of H_v per
  // tile; two tiles wait in registers (stages a and b) while one is in LDS.
  const bool mover = tid < 2 * R;
  const int prow = piece_row<R>(tid), pcol = piece_col<R>(tid);
  const char* gk = reinterpret_cast<const char*>(Hk) + pcol;
  const char* gv = reinterpret_cast<const char*>(Hv) + pcol;
  const int ko = prow * kKStride<R> + pcol, vo = vtile_off<R>(prow, pcol);
  auto fetch = [&](int tok0, uint4& k, uint4& v) {
    if (mover) {
      const size_t row = static_cast<size_t>(min(tok0 + prow, last)) * (2 * R);
      k = load_stream16(gk + row);
      v = load_stream16(gv + row);
    }
  };
  auto put = [&](int buf, const uint4& k, const uint4& v) {
    if (mover) {
      *reinterpret_cast<uint4*>(sm.k[buf] + ko) = k;
      *reinterpret_cast<uint4*>(sm.v[buf] + vo) = v;
    }
  };
  uint4 ka, va, kb2, vb2;
  fetch(s0, ka, va);
  put(0, ka, va);
  fetch(s0 + kTile, ka, va);
  fetch(s0 + 2 * kTile, kb2, vb2);
  for (int it = 0; it < ntiles; it += 2) {
    // stage a holds tile it+1: to LDS (its buffer held tile it-2, finished by
    // everyone), then fetch tile it+3 into it
    put((it + 1) % kNB, ka, va);
    fetch(s0 + (it + 3) * kTile, ka, va);
    __syncthreads();
    process(it);
    if (it + 1 < ntiles) {
      put((it + 2) % kNB, kb2, vb2);
      fetch(s0 + (it + 4) * kTile, kb2, vb2);
      __syncthreads();
      process(it + 1);
    }
  }

  // ---- partials: this wave's r slice for every query head; (m, l) by owners
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (half == 0 && ln < gqa && kb == 0) {
    const int head = g * nq + jl * gqa + ln;
    const size_t slot = (static_cast<size_t>(b) * p.Hq + head) * p.n_split + split;
    p.part_ml[slot * 2] = m;
    p.part_ml[slot * 2 + 1] = l;
  }
  if (ln < nq) {
    const int head = g * nq + ln;
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

}  // namespace

bool reconstruct_mfma_supported(const DecodeParams& p, int dtype) {
  return dtype == 1 && p.d == kD && p.s == kHeads && p.gqa <= 4 && (p.r == 128 || p.r == 256);
}

hipError_t launch_transpose_bk(const DecodeParams& p, int dtype, hipStream_t st) {
  const dim3 grid((p.Dg + 31) / 32, (p.r + 31) / 32, p.G);
  if (dtype == 0) transpose_bk_kernel<float><<<grid, 256, 0, st>>>(p);
  else transpose_bk_kernel<uint16_t><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_split_reconstruct_mfma(const DecodeParams& p, hipStream_t st) {
  const dim3 grid(p.n_split, p.G, p.B);
  if (p.r == 128) split_reconstruct_mfma_kernel<128><<<grid, kThreads, 0, st>>>(p);
  else if (p.r == 256) split_reconstruct_mfma_kernel<256><<<grid, kThreads, 0, st>>>(p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace palu
