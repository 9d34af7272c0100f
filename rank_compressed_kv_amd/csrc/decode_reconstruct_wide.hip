// Context-split decode kernel for the reconstruct mode (keys rebuilt per tile
// and rotated) at rank 256, bf16 latents, on the gfx950 matrix cores: each
// wave holds one KV head's whole B_k^T (128 columns x 256 latents, all 256
// AGPRs of a lane) for the split.
//
// Method (Palu author response on OpenReview): K_i = H_i B_i is rebuilt from
// the cached latents and kept on chip ("Why Palu Requires Fewer Global Memory
// Access"); the rotary embedding is why keys must be rebuilt at all
// (clarification of W1). Values stay in latent space: the weighted sum runs
// over h_v rows and B_v is applied in the merge pass.
//
// Shapes served: head_dim 128, at most four query heads per KV head, rank 256,
// a multiple of four KV heads per group. A workgroup has four waves, one per
// KV head of its slice, and owns one (batch, group, context split, slice);
// the waves share the latent tiles (read from HBM once per workgroup into
// LDS) and the rotation table. Per 16-token tile, wave of KV head j:
//   keys     K^T[16 cols x 16 tok] = B_k^T[cols x r] * H_k^T[r x tok] for the 8
//            column blocks, bf16 MFMA 16x16x32;
//   rotate   the pair (f, f + 64) is block blk and blk + 4 at the same
//            register, so a lane rotates its own values;
//   scores   S[tok x q heads] by fp16 MFMA 16x16x32 from the rotated keys
//            rounded once to fp16 and q in fp16 after a per-head power-of-two
//            scale;
//   softmax  online, base 2, lazy rescale;
//   values   U[rows x r] += P[rows x 16 tok] * H_v[16 tok x r], bf16 MFMA
//            16x16x16: rows 0..3 the bf16 parts of the weights, rows 4..7 the
//            remainders; the H_v operand comes from the LDS tile with the
//            transposing read.
// The next tile's key MFMAs are interleaved slot by slot with this tile's
// rotations, packs and score MFMAs (one wave per SIMD: the matrix core and
// the VALU only work at once when one wave's code interleaves them); the
// softmax and values follow in their own block (at this rank the registers
// do not allow them to be interleaved too).
// Loads: 16-byte pieces of each tile go through one of two register stages
// (a tile is requested two iterations before its LDS copy) into a ring of
// four LDS buffers; rows past the split's end are clamped to its last valid
// row and masked.
#include "reconstruct_wave_util.h"

namespace palu {
namespace {

using namespace wave;

constexpr int R = 256;             // rank
constexpr int kC = R / 32;         // 32-latent key chunks
constexpr int kRB = R / 16;        // 16-latent value blocks
constexpr int kWaves = 4;          // waves (KV heads) per workgroup
constexpr int kNBuf = 4;           // LDS tile buffers

struct Smem {
  char k[kNBuf][kTile * kKStride<R>];
  char v[kNBuf][kTile * kVStride<R>];
  RotTable rot;
  uint4 qop[kWaves][4][64];        // each wave's q operand: qop[wave][m][lane]
};

template <bool kShared>
__global__ __launch_bounds__(64 * kWaves, 1) void split_reconstruct_wide_kernel(DecodeParams p) {
  constexpr int kThreads = 64 * kWaves;
  constexpr int kPieces = 2 * R / kThreads;                     // 16-B pieces per matrix
  static_assert(2 * R % kThreads == 0, "whole pieces per thread");
  const int nslice = p.s / kWaves;
  const SplitUnit un = split_unit(p.n_split, p.G, p.B, nslice);
  if (!un.live) return;
  const int split = un.split, g = un.g, b = un.b, hs = un.hs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, kb = lane >> 4;
  const int n = clamp_len(p.lens, b, p.L);
  const int s0 = split * p.split_tokens;
  if (s0 >= n) return;                                   // whole workgroup
  const int t1 = min(n, s0 + p.split_tokens);
  const int last = t1 - 1;
  const int gqa = p.gqa;                                 // query heads per KV head (<= 4)
  const int kvh = hs * kWaves + wave;                    // this wave's KV head in the group
  const int head0 = g * p.nq + kvh * gqa;                // its first query head

  __shared__ Smem sm;

  const size_t row0 = (static_cast<size_t>(b) * p.G + g) * p.L;
  const char* Hk = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.h_k) + row0 * R);
  const char* Hv = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.h_v) + row0 * R);
  const int ntiles = (t1 - s0 + kTile - 1) / kTile;

  // Loads: thread piece i (< kPieces) is the 16-byte piece tid + i*kThreads of
  // the tile (byte 16*that in a row-major tile of 16 rows of 2R bytes). Two
  // tiles wait in registers (vector types, so they stay in registers; stage
  // it & 1 holds tile it+2 at iteration it) and the two ahead of the one
  // being consumed are in LDS. The first two tiles are requested before
  // anything else, so their latency overlaps the B_k^T loads and the set-up.
  typedef uint32_t u32v __attribute__((ext_vector_type(4 * kPieces)));
  // a piece's byte offset inside its tile's rows (the same for every tile, so
  // a tile only moves the scalar base; the split's last tile clamps its rows)
  uint32_t poff[kPieces];
#pragma unroll
  for (int i = 0; i < kPieces; ++i) poff[i] = 16u * static_cast<uint32_t>(tid + i * kThreads);
  auto fetch = [&](int tok0, u32v& k, u32v& v) {
    const bool tail = tok0 + kTile > t1;
    const size_t base = static_cast<size_t>(min(tok0, last)) * (2 * R);
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      uint32_t o = poff[i];
      if (tail) {
        asm volatile("" : "+v"(o));                      // keeps the clamp inside this rare branch
        const int row = min(static_cast<int>(o / (2 * R)), last - min(tok0, last));
        o = static_cast<uint32_t>(row * (2 * R)) + o % (2 * R);
      }
      const uint4 a = load_tile16<kShared>(Hk + base + o);
      const uint4 c = load_tile16<kShared>(Hv + base + o);
      k[4 * i] = a.x; k[4 * i + 1] = a.y; k[4 * i + 2] = a.z; k[4 * i + 3] = a.w;
      v[4 * i] = c.x; v[4 * i + 1] = c.y; v[4 * i + 2] = c.z; v[4 * i + 3] = c.w;
    }
  };
  auto put = [&](int buf, const u32v& k, const u32v& v) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int pc = tid + i * kThreads;
      const int prow = (pc * 16) / (2 * R), pcol = (pc * 16) % (2 * R);
      *reinterpret_cast<uint4*>(sm.k[buf] + prow * kKStride<R> + pcol) =
          uint4{k[4 * i], k[4 * i + 1], k[4 * i + 2], k[4 * i + 3]};
      *reinterpret_cast<uint4*>(sm.v[buf] + prow * kVStride<R> + pcol) =
          uint4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    }
  };

  u32v stk0, stv0, stk1, stv1;
  fetch(s0, stk0, stv0);
  fetch(s0 + kTile, stk1, stv1);

  u32x4 bt[8][kC];
  load_bkt<kC>(bt, static_cast<const uint16_t*>(p.bkt) + (static_cast<size_t>(g) * p.Dg + kvh * kD) * R,
               R, 0, ln, kb);
  const float hscale = q_operand(p, b, head0, gqa, ln, kb, lane, sm.qop[wave]);
  Rot<kThreads> rot(sm.rot, tid, p.rope != 0);
  rot.init(p, tid);
  barrier_lds();                                         // rstep and orev before any use

  // softmax state of query head ln (lanes ln >= gqa carry a zero query and
  // are never written out); acc[rb] holds rows 4 kb .. 4 kb + 3 of latent
  // 16 rb + ln (kb = 0: the bf16 parts of query heads 0..3, kb = 1: the
  // remainders)
  float m_run = -INFINITY, l_run = 0.f;
  floatx4 acc[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) acc[rb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // the ring's next buffer (the buffer of tile it is carried through the
  // loop rather than computed as it % kNBuf, which keeps the LDS addresses
  // one register plus an immediate offset)
  auto next_buf = [](int bf) { return bf + 1 == kNBuf ? 0 : bf + 1; };

  // keys of the tile in buffer bf (K tile in LDS): kk[blk] = K^T of column
  // block blk
  auto keys = [&](int bf, floatx4 (&kk)[8]) {
    const char* kt = sm.k[bf] + ln * kKStride<R> + 16 * kb;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) kk[blk] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const bf16x8 h = as_bf16x8(*reinterpret_cast<const uint4*>(kt + 64 * c));
#pragma unroll
      for (int blk = 0; blk < 8; ++blk)
        kk[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bt[blk][c]), h,
                                                          kk[blk], 0, 0, 0);
    }
  };

  // tile it's softmax and values, after the running max of its scores (sc:
  // the raw scores, mx: their scaled maximum in log2 units). Tiles go in
  // pairs: the first's weights wait in registers (pv_pair) and one bf16 MFMA
  // 16x16x32 per value block takes both tiles' 32 tokens (k slot 8 kb + j is
  // token 4 kb + j of the first tile for j < 4, token 4 kb + j - 4 of the
  // second for j >= 4: a lane's own weights and its transposing reads of the
  // two V tiles); a tile without a partner (an odd count's last) takes the
  // 16x16x16 form.
  const bool rhi = ln < gqa;                             // P row ln: bf16 part of head ln
  const bool rlo = ln >= 4 && ln - 4 < gqa;              // P row ln: remainder of head ln - 4
  const int vrow = 4 * kb + (ln >> 2), vcol = 4 * (ln & 3);   // transposing-read source
  floatx4 pv_pair = {0.f, 0.f, 0.f, 0.f};                // the pair's first tile's weights
  // the P operand of four weights: rows 0..3 bf16(p) of head ln, rows 4..7 the
  // remainders of head ln - 4 (moved four lanes up inside each 16-lane row)
  auto p_operand = [&](floatx4 pv) {
    uint32_t h0, h1, lo0, lo1;
    split_bf16x2(pv[0], pv[1], h0, lo0);
    split_bf16x2(pv[2], pv[3], h1, lo1);
    const uint32_t lo0s = __builtin_amdgcn_update_dpp(0u, lo0, 0x114, 0xf, 0xf, true);
    const uint32_t lo1s = __builtin_amdgcn_update_dpp(0u, lo1, 0x114, 0xf, 0xf, true);
    const uint32_t a0 = rhi ? h0 : (rlo ? lo0s : 0u), a1 = rhi ? h1 : (rlo ? lo1s : 0u);
    return __builtin_bit_cast(short4v, uint2{a0, a1});
  };
  // kMode: 0 a tile alone, 1 the first of a pair (weights kept), 2 the second
  // (values of both; bfp: the first's buffer)
  auto softmax_values = [&](int bf, int bfp, floatx4 sc, float mx, auto kMode) {
    constexpr int mode = kMode;
    if (__any(mx > m_run + kLazy)) {                     // wave-uniform, rare
      const float mn = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - mn);
      m_run = mn;
      l_run *= alpha;
      if constexpr (mode == 2) pv_pair *= alpha;         // this lane's head's factor
      // acc rows belong to heads 0..3: take each head's factor from its lane
      float ah[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ah[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), i));
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rb][i] *= ah[i];
    }
    // weights 2^(s hscale - m) <= 2^kLazy by the hardware exp2 (results below
    // 2^-126 flush to zero, which a weight of that size is anyway); masked
    // tokens (s = -inf) give 0
    floatx4 pv;
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], hscale, -m_run));
    l_run += (pv[0] + pv[1]) + (pv[2] + pv[3]);
    if constexpr (mode == 1) {
      pv_pair = pv;
    } else if constexpr (mode == 0) {
      // U[row][16 rb + ln] += sum_t P[row][t] H_v[t][16 rb + ln]
      const short4v pa = p_operand(pv);
      const char* vb = sm.v[bf] + vrow * kVStride<R> + 2 * vcol;
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, read_tr16(vb + 32 * rb), acc[rb], 0, 0, 0);
    } else {
      const short8v pa = __builtin_shufflevector(p_operand(pv_pair), p_operand(pv), 0, 1, 2, 3, 4, 5, 6, 7);
      const char* va = sm.v[bfp] + vrow * kVStride<R> + 2 * vcol;
      const char* vb = sm.v[bf] + vrow * kVStride<R> + 2 * vcol;
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const short8v hv = __builtin_shufflevector(read_tr16(va + 32 * rb), read_tr16(vb + 32 * rb),
                                                   0, 1, 2, 3, 4, 5, 6, 7);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pa),
                                                          __builtin_bit_cast(bf16x8, hv), acc[rb], 0, 0, 0);
      }
    }
  };

  // Prologue: tiles 0 and 1 into LDS, tiles 2 and 3 in the register stages,
  // the rotation table of tile 0, the keys of tile 0.
  put(0, stk0, stv0);
  put(1, stk1, stv1);
  fetch(s0 + 2 * kTile, stk0, stv0);
  __builtin_amdgcn_sched_barrier(0);                     // stage 0's loads are the older ones
  fetch(s0 + 3 * kTile, stk1, stv1);
  rot.exact(s0, 0);
  barrier_lds();
  floatx4 kx[8], ky[8];
  keys(0, kx);
  int cb = 0;                                            // buffer of tile it

  // Iteration it (after the barrier that made tiles it and it+1 and tile
  // it's rotation table visible). Region 1 is one straight run of code
  // written as 8 kC slots in a fixed order (the compiler may not move code
  // across slots): slot (c, blk) issues the key MFMA of tile it+1's column
  // block blk and chunk c, then its share of the work items of tile it: the
  // LDS copy of tile it+2 from its register stage (its buffer last held tile
  // it-2) and the request of tile it+4 into the stage, the rotation-table
  // reads, the 16 pair rotations, the four fp16 packs and score MFMAs, the
  // last tile's mask and the running max. H_k chunks are read two chunks
  // ahead. Region 2: the rare rescale, tile it's softmax and values, the
  // rotation table of tile it+1 (its buffer last served tile it-1); the
  // barrier.
  constexpr int kSlots = 8 * kC;
  constexpr int kItems = 32;
  auto region1 = [&](int it, int bf, floatx4 (&cur)[8], floatx4 (&nxt)[8], u32v& stk, u32v& stv,
                     floatx4& sc, float& mx) {
    const int tok0 = s0 + it * kTile;
    const int bf1 = next_buf(bf), bf2 = next_buf(bf1);   // tiles it+1, it+2
    const char* kt = sm.k[bf1] + ln * kKStride<R> + 16 * kb;
    const uint4* qo = &sm.qop[wave][0][lane];
    // H_k chunks in a ring of three, each read two chunks (16 MFMAs) ahead
    u32x4 h[3];
    h[0] = *reinterpret_cast<const u32x4*>(kt);
    h[1] = *reinterpret_cast<const u32x4*>(kt + 64);
    float4 rt[4][2];
    uint4 a16[4], q16[4];
    sc = floatx4{0.f, 0.f, 0.f, 0.f};
    // items in order: 0 the LDS copy, 1 the request, then the table rows of
    // block b read one block ahead of its four pair rotations (2: rows 0,
    // 3: rows 1, 4-7: rotations 0, 8: rows 2, 9-12: rotations 1, 13: rows 3,
    // 14-17: rotations 2, 18-21: rotations 3 and the q operands of the score
    // MFMAs), 22-25 the packs, 26-29 the score MFMAs, 30 the mask of the
    // split's last tile, 31 the running max
    auto rows = [&](int blk) {
      rt[blk][0] = *reinterpret_cast<const float4*>(&sm.rot.rtab[it & 1][8 * blk + 2 * kb][ln][0]);
      rt[blk][1] = *reinterpret_cast<const float4*>(&sm.rot.rtab[it & 1][8 * blk + 2 * kb + 1][ln][0]);
    };
    auto rotate = [&](int blk, int i) {                 // pair (f, f + 64), f = 16 blk + 4 kb + i
      const float4 r = rt[blk][i / 2];
      const float c = i % 2 ? r.z : r.x, sn = i % 2 ? r.w : r.y;
      const float x = cur[blk][i], y = cur[blk + 4][i];
      cur[blk][i] = x * c - y * sn;
      cur[blk + 4][i] = x * sn + y * c;
    };
    auto item = [&](auto W) {
      constexpr int w = W;
      if constexpr (w == 0) {
        put(bf2, stk, stv);
      } else if constexpr (w == 1) {
        fetch(s0 + (it + 4) * kTile, stk, stv);
      } else if constexpr (w == 2 || w == 3) {
        rows(w - 2);
      } else if constexpr (w < 8) {
        rotate(0, w - 4);
      } else if constexpr (w == 8) {
        rows(2);
      } else if constexpr (w < 13) {
        rotate(1, w - 9);
      } else if constexpr (w == 13) {
        rows(3);
      } else if constexpr (w < 22) {
        rotate(2 + (w - 14) / 4, (w - 14) % 4);
        if constexpr (w >= 18) q16[w - 18] = qo[64 * (w - 18)];   // score MFMA w-18's q, early
      } else if constexpr (w < 26) {                     // fp16 A operand of score MFMA m
        constexpr int m = w - 22;
        a16[m] = uint4{pack_f16x2(cur[m][0], cur[m][1]), pack_f16x2(cur[m][2], cur[m][3]),
                       pack_f16x2(cur[m + 4][0], cur[m + 4][1]),
                       pack_f16x2(cur[m + 4][2], cur[m + 4][3])};
      } else if constexpr (w < 30) {                     // S[token 4 kb + i][head ln]
        constexpr int m = w - 26;
        sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a16[m]),
                                                    __builtin_bit_cast(f16x8, q16[m]), sc,
                                                    0, 0, 0);
      } else if constexpr (w == 30) {                    // the split's last tile: its tail masked
        if (tok0 + kTile > t1) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[i] = tok0 + 4 * kb + i < t1 ? sc[i] : -INFINITY;
        }
      } else {                                           // in log2 units (hscale > 0)
        mx = hscale * max_groups(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
      }
    };
    static_for<kSlots>([&](auto S) {
      constexpr int slot = S, c = slot / 8, blk = slot % 8;
      if constexpr (blk == 0 && c + 2 < kC) h[(c + 2) % 3] = *reinterpret_cast<const u32x4*>(kt + 64 * (c + 2));
      const floatx4 acc_in = c == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : nxt[blk];
      hold_in_agpr(bt[blk][c]);
      nxt[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bt[blk][c]),
                                                         __builtin_bit_cast(bf16x8, h[c % 3]),
                                                         acc_in, 0, 0, 0);
      constexpr int w0 = slot * kItems / kSlots, w1 = (slot + 1) * kItems / kSlots;
      static_for<w1 - w0>([&](auto J) { item(std::integral_constant<int, w0 + J>{}); });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto iteration = [&](int it, floatx4 (&cur)[8], floatx4 (&nxt)[8], u32v& stk, u32v& stv,
                       auto kMode) {
    floatx4 sc;
    float mx;
    region1(it, cb, cur, nxt, stk, stv, sc, mx);
    softmax_values(cb, cb == 0 ? kNBuf - 1 : cb - 1, sc, mx, kMode);
    cb = next_buf(cb);
    if (it + 1 < ntiles) {
      if ((it + 1) % kAnchor == 0) rot.exact(s0 + (it + 1) * kTile, (it + 1) & 1);
      else rot.step(it + 1);
    }
    barrier_lds();
  };
  // whole pairs in the loop (both halves every trip, so the compiler's wait
  // counts see stage 0's loads as the older ones at the loop's head), an odd
  // last tile after it
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    iteration(it, kx, ky, stk0, stv0, std::integral_constant<int, 1>{});
    iteration(it + 1, ky, kx, stk1, stv1, std::integral_constant<int, 2>{});
  }
  if (it < ntiles) iteration(it, kx, ky, stk0, stv0, std::integral_constant<int, 0>{});

  // ---- partials of this wave's query heads: the remainder rows (kb = 1) are
  // added to the bf16 rows (kb = 0); the sum l over the four lane groups
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[rb][i] = add_pair_groups(acc[rb][i]);
  l_run = sum_groups(l_run);
  if (kb == 0 && ln < gqa) {
    const size_t slot = (static_cast<size_t>(b) * p.Hq + head0 + ln) * p.n_split + split;
    p.part_ml[slot * 2] = m_run;
    p.part_ml[slot * 2 + 1] = l_run;
  }
  if (kb == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < gqa) {
        const size_t slot = (static_cast<size_t>(b) * p.Hq + head0 + i) * p.n_split + split;
        float* u = p.part_u + slot * R;
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) u[16 * rb + ln] = acc[rb][i];
      }
    }
  }
}

hipError_t launch_wide(const DecodeParams& p, hipStream_t st) {
  const int nslice = p.s / kWaves;
  if (nslice == 1) {
    const dim3 grid(p.n_split, p.G, p.B);
    split_reconstruct_wide_kernel<false><<<grid, 64 * kWaves, 0, st>>>(p);
  } else {
    const long ids = split_unit_ids(p.n_split, p.G, p.B, nslice);
    if (ids == 0) return hipErrorInvalidValue;
    split_reconstruct_wide_kernel<true><<<dim3(static_cast<unsigned>(ids)), 64 * kWaves, 0, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

bool reconstruct_wide_supported(const DecodeParams& p, int dtype) {
  return dtype == 1 && p.d == kD && p.gqa <= 4 && p.r == R && p.s % kWaves == 0;
}

hipError_t launch_split_reconstruct_wide(const DecodeParams& p, hipStream_t st) {
  return p.r == R ? launch_wide(p, st) : hipErrorInvalidValue;
}

}  // namespace palu
