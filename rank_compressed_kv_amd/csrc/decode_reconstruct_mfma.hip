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
// split); its four waves are the group's four KV heads and walk the split's
// 16-token tiles together:
//   keys     K^T[128 cols x 16 tok] = B_k^T[cols x r] * H_k^T[r x tok] per 16-col
//            block, bf16 MFMA 16x16x32. Each wave holds its head's B_k^T (read
//            once, from a transposed copy in the workspace) in registers for
//            the whole split; H_k comes from the tile in LDS.
//   rotate   the result leaves lane l with columns 16*cb + 4*(l/16) + i of
//            token l%16, so the pair (f, f+64) sits in one lane (blocks cb and
//            cb+4). cos/sin of t*omega_f advance by one exact complex product per
//            tile (t grows by 16) and are recomputed from the angle every
//            kAnchor tiles.
//   scores   that layout is the A operand of a 16x16x16 MFMA (k = the 16
//            columns of a block), so S^T[tok x q heads] = K_rot * Q^T chains on
//            the matrix cores; keys are split into hi + lo bf16 (two MFMAs,
//            ~16 bits kept), q is exact bf16, the scale is applied to the fp32
//            result.
//   softmax  online, base 2, per query head in the wave that owns its KV head.
//   values   P and the rescale factors go through LDS; wave w then adds
//            H_v^T[r slice w] * P^T for all query heads of the group (bf16 MFMA
//            16x16x16, P split hi + lo), gathering value columns from the tile
//            in LDS (four-row groups offset by 32 B: conflict-free).
// Loads: each thread moves 64 B of a tile (16 B loads) into registers two
// tiles ahead and writes them to a ring of three LDS tile buffers; rows past
// the split's end are clamped to its last valid row and masked.
#include <math.h>

#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;        // = KV heads per group
constexpr int kTile = 16;        // tokens per tile
constexpr int kD = 128;          // head dim
constexpr int kBlocks = kD / 16; // 16-column blocks per head
constexpr int kNB = 3;           // LDS tile buffers
constexpr int kAnchor = 32;      // tiles between exact cos/sin evaluations

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}

// K tile: rows padded by 16 B so 16 lanes reading 16 B of 16 rows hit distinct banks
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
  float pt[16][kTile];        // P of the group's query heads for the current tile
  float alpha[16];            // rescale factor of each query head for this tile
};

// one tile of H_k and H_v: 16 rows x R bf16 each = 32*R bytes; every thread of
// the workgroup moves 32*R / 256 bytes, i.e. R/128 16-byte pieces of each
template <int R>
struct Stage {
  uint4 k[R / 128];
  uint4 v[R / 128];
};

template <int R>
__device__ __forceinline__ void load_stage(Stage<R>& sg, const uint16_t* Hk, const uint16_t* Hv,
                                           int tok0, int last, int tid) {
#pragma unroll
  for (int q = 0; q < R / 128; ++q) {
    const int flat = (q * 256 + tid) * 16;               // byte in the tile's 16 rows
    const int row = min(tok0 + flat / (2 * R), last);
    const int cb = flat % (2 * R);
    sg.k[q] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(Hk + static_cast<size_t>(row) * R) + cb);
    sg.v[q] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(Hv + static_cast<size_t>(row) * R) + cb);
  }
}

template <int R>
__device__ __forceinline__ void store_stage(const Stage<R>& sg, char* kt, char* vt, int tid) {
#pragma unroll
  for (int q = 0; q < R / 128; ++q) {
    const int flat = (q * 256 + tid) * 16;
    const int row = flat / (2 * R), cb = flat % (2 * R);
    *reinterpret_cast<uint4*>(kt + row * kKStride<R> + cb) = sg.k[q];
    *reinterpret_cast<uint4*>(vt + vtile_off<R>(row, cb)) = sg.v[q];
  }
}

__device__ __forceinline__ short bf16_bits_rne(float x) {
  return static_cast<short>(f32_to_bf16_rne(x));
}

template <int R>
__global__ __launch_bounds__(64 * kWaves) void split_reconstruct_mfma_kernel(DecodeParams p) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, kb = lane >> 4;
  const int jl = wave;                                   // this wave's KV head in the group
  const int n = clamp_len(p.lens, b, p.L);
  const int s0 = split * p.split_tokens;
  if (s0 >= n) return;                                   // whole workgroup
  const int t1 = min(n, s0 + p.split_tokens);
  const int last = t1 - 1;
  const int gqa = p.gqa;                                 // query heads per KV head (<= 4)
  const int nq = p.nq;                                   // query heads of the group (<= 16)

  __shared__ Smem<R> sm;

  // ---- operands held for the whole split -----------------------------------
  // B_k^T rows (this head's 128 columns) as the A operand: lane (ln, kb) of
  // block cb, chunk c holds column 16cb + ln, latents 32c + 8kb .. +8
  const uint16_t* Bt = static_cast<const uint16_t*>(p.bkt) +
                       (static_cast<size_t>(g) * p.Dg + jl * kD) * R;
  uint4 bk[kBlocks][R / 32];
#pragma unroll
  for (int cb = 0; cb < kBlocks; ++cb)
#pragma unroll
    for (int c = 0; c < R / 32; ++c)
      bk[cb][c] = *reinterpret_cast<const uint4*>(Bt + static_cast<size_t>(16 * cb + ln) * R + 32 * c + 8 * kb);
  // q of this KV head's query heads as the score B operand: lane (ln = head
  // slot, kb) of block cb holds columns 16cb + 4kb .. +4 (exact bf16)
  short4v qb[kBlocks];
  {
    const bool valid = ln < gqa;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                           (static_cast<size_t>(b) * p.Hq + g * nq + jl * gqa + (valid ? ln : 0)) * kD;
#pragma unroll
    for (int cb = 0; cb < kBlocks; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) qb[cb][e] = valid ? static_cast<short>(qrow[16 * cb + 4 * kb + e]) : 0;
  }
  // rotation state: this lane's token is tok0 + ln; its frequencies are
  // f = 16*cb + 4*kb + i for cb < 4, i < 4
  float cs[4][4], sn[4][4], cstep[4][4], sstep[4][4];
  const bool rope = p.rope != 0;
  auto anchor = [&](int tok) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (rope) rope_cos_sin(p.omega_rev[16 * cb + 4 * kb + i], tok + ln, cs[cb][i], sn[cb][i]);
        else { cs[cb][i] = 1.f; sn[cb][i] = 0.f; }
      }
  };
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (rope) rope_cos_sin(p.omega_rev[16 * cb + 4 * kb + i], kTile, cstep[cb][i], sstep[cb][i]);
      else { cstep[cb][i] = 1.f; sstep[cb][i] = 0.f; }
    }

  // ---- softmax state of the owned query heads (lane ln = head slot) ---------
  float m = -INFINITY, l = 0.f;
  // value-latent sums for all query heads over this wave's r slice:
  // acc[rb] holds r = wave*R/4 + 16*rb + 4*kb + i for query head ln
  floatx4 acc[R / 64];
#pragma unroll
  for (int rb = 0; rb < R / 64; ++rb) acc[rb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const size_t row0 = (static_cast<size_t>(b) * p.G + g) * p.L;
  const uint16_t* Hk = static_cast<const uint16_t*>(p.h_k) + row0 * R;
  const uint16_t* Hv = static_cast<const uint16_t*>(p.h_v) + row0 * R;
  const int ntiles = (t1 - s0 + kTile - 1) / kTile;

  // prologue: tile 0 into LDS, tile 1 staged in registers
  Stage<R> sg;
  load_stage<R>(sg, Hk, Hv, s0, last, tid);
  store_stage<R>(sg, sm.k[0], sm.v[0], tid);
  load_stage<R>(sg, Hk, Hv, s0 + kTile, last, tid);

  for (int it = 0; it < ntiles; ++it) {
    const int tok0 = s0 + it * kTile;
    // tile it+1 to LDS (its buffer held tile it-2, finished by everyone), then
    // fetch tile it+2 into the staging registers
    store_stage<R>(sg, sm.k[(it + 1) % kNB], sm.v[(it + 1) % kNB], tid);
    load_stage<R>(sg, Hk, Hv, tok0 + 2 * kTile, last, tid);
    __syncthreads();
    const char* kt = sm.k[it % kNB];
    const char* vt = sm.v[it % kNB];

    // keys of this head: K^T[16cb + 4kb + i][token ln]
    floatx4 kk[kBlocks];
#pragma unroll
    for (int cb = 0; cb < kBlocks; ++cb) kk[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < R / 32; ++c) {
      const bf16x8 h = as_bf16x8(*reinterpret_cast<const uint4*>(kt + ln * kKStride<R> + 2 * (32 * c + 8 * kb)));
#pragma unroll
      for (int cb = 0; cb < kBlocks; ++cb)
        kk[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(bk[cb][c]), h, kk[cb], 0, 0, 0);
    }
    // rotate the pairs (f, f + 64) and advance cos/sin by 16 positions
    if (it % kAnchor == 0) anchor(tok0);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = kk[cb][i], y = kk[cb + 4][i];
        const float c = cs[cb][i], s = sn[cb][i];
        kk[cb][i] = x * c - y * s;
        kk[cb + 4][i] = x * s + y * c;
        cs[cb][i] = c * cstep[cb][i] - s * sstep[cb][i];
        sn[cb][i] = s * cstep[cb][i] + c * sstep[cb][i];
      }
    // scores S^T[token 4kb+i][head slot ln] = K_rot . q over the 8 blocks
    floatx4 sc = {0.f, 0.f, 0.f, 0.f}, sc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < kBlocks; ++cb) {
      short4v ah, al;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const short hb = bf16_bits_rne(kk[cb][i]);
        ah[i] = hb;
        al[i] = bf16_bits_rne(kk[cb][i] - __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(hb)) << 16));
      }
      sc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, qb[cb], sc, 0, 0, 0);
      sc2 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, qb[cb], sc2, 0, 0, 0);
    }
    sc += sc2;
    // online softmax for the owned heads (lanes ln < gqa carry real heads)
    float pv[4];
    {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[i] *= p.scale_log2;
        if (tok0 + 4 * kb + i >= t1) sc[i] = -INFINITY;
        mx = fmaxf(mx, sc[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m, mx);
      const float alpha = exp2f(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = exp2f(sc[i] - mn);
        l += pv[i];
      }
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
      const float pa[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float hi = __uint_as_float(__float_as_uint(pa[e]) & 0xffff0000u);
        ph[e] = static_cast<short>(__float_as_uint(hi) >> 16);
        pl[e] = bf16_bits_rne(pa[e] - hi);
      }
      const char* vb = vt + vtile_off<R>(4 * kb, 2 * (wave * (R / 4) + ln));
#pragma unroll
      for (int rb = 0; rb < R / 64; ++rb) {
        short4v a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = *reinterpret_cast<const short*>(vb + e * (2 * R) + 32 * rb);
        acc[rb] *= al;
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, ph, acc[rb], 0, 0, 0);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pl, acc[rb], 0, 0, 0);
      }
    }
  }

  // ---- partials: this wave's r slice for every query head; (m, l) by owners
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (ln < gqa && kb == 0) {
    const int head = g * nq + jl * gqa + ln;
    const size_t slot = (static_cast<size_t>(b) * p.Hq + head) * p.n_split + split;
    p.part_ml[slot * 2] = m;
    p.part_ml[slot * 2 + 1] = l;
  }
  if (ln < nq) {
    const int head = g * nq + ln;
    const size_t slot = (static_cast<size_t>(b) * p.Hq + head) * p.n_split + split;
    float* u = p.part_u + slot * R + wave * (R / 4);
#pragma unroll
    for (int rb = 0; rb < R / 64; ++rb)
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
  return dtype == 1 && p.d == kD && p.s == kWaves && p.gqa <= 4 && (p.r == 128 || p.r == 256);
}

hipError_t launch_transpose_bk(const DecodeParams& p, int dtype, hipStream_t st) {
  const dim3 grid((p.Dg + 31) / 32, (p.r + 31) / 32, p.G);
  if (dtype == 0) transpose_bk_kernel<float><<<grid, 256, 0, st>>>(p);
  else transpose_bk_kernel<uint16_t><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_split_reconstruct_mfma(const DecodeParams& p, hipStream_t st) {
  const dim3 grid(p.n_split, p.G, p.B);
  if (p.r == 128) split_reconstruct_mfma_kernel<128><<<grid, 64 * kWaves, 0, st>>>(p);
  else if (p.r == 256) split_reconstruct_mfma_kernel<256><<<grid, 64 * kWaves, 0, st>>>(p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace palu
