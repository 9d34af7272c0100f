// Context-split decode kernel for the reconstruct mode (keys rebuilt per tile
// and rotated) at rank 512, bf16 latents, on the gfx950 matrix cores: each
// wave holds a quarter of one KV head's B_k^T (the 32 columns of one rotary
// block pair x 512 latents, 128 AGPRs of a lane) for the split, which leaves
// room for two waves on every SIMD.
//
// Method (Palu author response on OpenReview): K_i = H_i B_i is rebuilt from
// the cached latents and kept on chip ("Why Palu Requires Fewer Global Memory
// Access"); the rotary embedding is why keys must be rebuilt at all
// (clarification of W1). Values stay in latent space: the weighted sum runs
// over h_v rows and B_v is applied in the merge pass.
//
// Shapes served: head_dim 128, at most four query heads per KV head, rank 512,
// an even number of KV heads per group. A workgroup owns one (batch, group,
// context split, slice of two KV heads) and has eight waves: wave w takes KV
// head w % 2 of the slice and quarter c = w / 2, i.e. column blocks c and
// c + 4 of the head's eight (the rotary pairs (f, f + 64) of f = 16 c .. 16 c
// + 15). Per 16-token tile, wave (head, c):
//   keys     K^T[16 cols x 16 tok] of its two column blocks, bf16 MFMA
//            16x16x32 over the sixteen 32-latent chunks, H_k from the LDS
//            tile;
//   rotate   its block pair, cos/sin from the table in LDS shared by all
//            waves (advanced by one exact complex product per tile,
//            re-anchored from the angle every kAnchor tiles);
//   scores   the partial S[tok x q heads] over its 32 columns by one fp16
//            MFMA 16x16x32 from the rotated keys rounded once to fp16 and q
//            in fp16 after a per-head power-of-two scale (q held in
//            registers); the four quarters' partial scores meet in LDS on
//            the tile's barrier and every quarter adds them in the same
//            order, so the four waves of a head hold the same scores and
//            softmax state;
//   softmax  online, base 2, lazy rescale, one iteration after the scores
//            (they are whole only after the barrier);
//   values   its latent quarter: U[rows x 128] += P[rows x tok] H_v[tok x
//            128] with P hi in rows 0..3 and lo in rows 4..7, the H_v operand
//            read from the LDS tile with the transposing read; two consecutive
//            tiles share one bf16 MFMA 16x16x32 per 16-latent block (k slot
//            8 kb + j is token 4 kb + j of the first tile for j < 4 and of
//            the second for j >= 4), the first tile's weights waiting in
//            registers and rescaled with the state if the second raises the
//            max; an odd count's last tile takes the 16x16x16 form.
// The next tile's key MFMAs are interleaved slot by slot with this tile's
// rotations, pack and score MFMA; the two waves on a SIMD fill each other's
// gaps (the softmax's dependent chain, LDS and exp latencies).
// Loads: 16-byte pieces of each tile go through a register stage into LDS
// rings of two K and five V buffers (a tile's values run an iteration after
// its scores, and a pair's first V tile stays until the pair's second is
// summed); rows past the split's end are clamped to its last valid row and
// masked. One barrier per tile.
#include "reconstruct_wave_util.h"

namespace palu {
namespace {

using namespace wave;

constexpr int R = 512;             // rank
constexpr int kC = R / 32;         // 32-latent key chunks
constexpr int kHeads = 2;          // KV heads per workgroup
constexpr int kParts = 4;          // waves (column quarters) per KV head
constexpr int kWaves = kParts * kHeads;
constexpr int kThreads = 64 * kWaves;
constexpr int kVB = R / kParts / 16;   // 16-latent value blocks per wave
constexpr int kNBuf = 2;           // LDS K tile buffers
constexpr int kVBuf = 5;           // LDS V tile buffers (a tile's values run an iteration late)

struct Smem {
  char k[kNBuf][kTile * kKStride<R>];
  char v[kVBuf][kTile * kVStride<R>];
  uint4 qop[kWaves][64];           // each wave's score q operand (block pair qc)
  RotTable rot;
  floatx4 sp[2][kWaves][64];       // partial scores, by tile parity
};
// the q operands of all four block pairs are built in V buffers 2 and 3
// (first written by the loop, after the prologue's barriers)
static_assert(2 * kTile * kVStride<R> >= kWaves * 4 * 64 * 16, "q operand staging fits");
static_assert(sizeof(Smem) <= 160 * 1024, "fits the LDS of a CU");

template <bool kShared>
__global__ __launch_bounds__(kThreads, 1) void split_reconstruct_quarter_kernel(DecodeParams p) {
  constexpr int kPieces = 2 * R / kThreads;              // 16-B pieces per matrix
  static_assert(2 * R % kThreads == 0, "whole pieces per thread");
  const int nslice = p.s / kHeads;
  const SplitUnit un = split_unit(p.n_split, p.G, p.B, nslice);
  if (!un.live) return;
  const int split = un.split, g = un.g, b = un.b, hs = un.hs;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jh = wave % kHeads, qc = wave / kHeads;      // KV head of the slice, column quarter
  const int ln = lane & 15, kb = lane >> 4;
  const int n = clamp_len(p.lens, b, p.L);
  const int s0 = split * p.split_tokens;
  if (s0 >= n) return;                                   // whole workgroup
  const int t1 = min(n, s0 + p.split_tokens);
  const int last = t1 - 1;
  const int gqa = p.gqa;                                 // query heads per KV head (<= 4)
  const int kvh = hs * kHeads + jh;                      // this wave's KV head in the group
  const int head0 = g * p.nq + kvh * gqa;                // its first query head

  __shared__ Smem sm;

  const size_t row0 = (static_cast<size_t>(b) * p.G + g) * p.L;
  const char* Hk = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.h_k) + row0 * R);
  const char* Hv = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.h_v) + row0 * R);
  const int ntiles = (t1 - s0 + kTile - 1) / kTile;

  // Loads: thread piece i (< kPieces) is the 16-byte piece tid + i*kThreads of
  // the tile (byte 16*that in a row-major tile of 16 rows of 2R bytes). One
  // tile waits in registers (vector types, so they stay in registers) and
  // the two ahead of the one being consumed are in LDS. The first two tiles
  // are requested before anything else, so their latency overlaps the
  // B_k^T loads and the set-up.
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
  auto put = [&](int kbuf, int vbuf, const u32v& k, const u32v& v) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int pc = tid + i * kThreads;
      const int prow = (pc * 16) / (2 * R), pcol = (pc * 16) % (2 * R);
      *reinterpret_cast<uint4*>(sm.k[kbuf] + prow * kKStride<R> + pcol) =
          uint4{k[4 * i], k[4 * i + 1], k[4 * i + 2], k[4 * i + 3]};
      *reinterpret_cast<uint4*>(sm.v[vbuf] + prow * kVStride<R> + pcol) =
          uint4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    }
  };

  u32v stk, stv, st1k, st1v;
  fetch(s0, stk, stv);
  fetch(s0 + kTile, st1k, st1v);

  // this wave's B_k^T quarter: bt[lb][c], columns 16 (qc + 4 lb) + ln,
  // latents 32 c + 8 kb .. +8 (from the transposed copy)
  u32x4 bt[2][kC];
  {
    const uint16_t* Bt = static_cast<const uint16_t*>(p.bkt) + (static_cast<size_t>(g) * p.Dg + kvh * kD) * R;
#pragma unroll
    for (int lb = 0; lb < 2; ++lb)
#pragma unroll
      for (int c = 0; c < kC; ++c)
        bt[lb][c] = *reinterpret_cast<const u32x4*>(
            Bt + static_cast<size_t>(16 * (qc + 4 * lb) + ln) * R + 32 * c + 8 * kb);
#pragma unroll
    for (int lb = 0; lb < 2; ++lb)
#pragma unroll
      for (int c = 0; c < kC; ++c) hold_in_agpr(bt[lb][c]);
  }
  float hscale;
  {
    uint4 (*qall)[64] = reinterpret_cast<uint4 (*)[64]>(sm.v[2]) + 4 * wave;
    hscale = q_operand(p, b, head0, gqa, ln, kb, lane, qall);
    sm.qop[wave][lane] = qall[qc][lane];                 // this wave's own rows: no barrier needed
  }
  Rot<kThreads> rot(sm.rot, tid, p.rope != 0);
  rot.init(p, tid);
  barrier_lds();                                         // rstep and orev before any use

  // softmax state of query head ln (lanes ln >= gqa carry a zero query and
  // are never written out); acc[rb] holds rows 4 kb .. 4 kb + 3 of latent
  // 128 qc + 16 rb + ln (kb = 0: the bf16 parts of query heads 0..3, kb = 1:
  // the remainders)
  float m_run = -INFINITY, l_run = 0.f;
  floatx4 acc[kVB];
#pragma unroll
  for (int rb = 0; rb < kVB; ++rb) acc[rb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // the rings' next buffers (the buffers of tile it are carried through the
  // loop, which keeps the LDS addresses one register plus an immediate offset)
  auto next_buf = [](int bf) { return bf + 1 == kNBuf ? 0 : bf + 1; };
  auto next_vbuf = [](int bf) { return bf + 1 == kVBuf ? 0 : bf + 1; };

  // keys of the tile in buffer bf: kk[lb] = K^T of column block qc + 4 lb
  auto keys = [&](int bf, floatx4 (&kk)[2]) {
    const char* kt = sm.k[bf] + ln * kKStride<R> + 16 * kb;
#pragma unroll
    for (int lb = 0; lb < 2; ++lb) kk[lb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const bf16x8 h = as_bf16x8(*reinterpret_cast<const uint4*>(kt + 64 * c));
#pragma unroll
      for (int lb = 0; lb < 2; ++lb)
        kk[lb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bt[lb][c]), h,
                                                         kk[lb], 0, 0, 0);
    }
  };

  // tile it's softmax and values from its full scores (sc: raw scores, mx:
  // their scaled maximum in log2 units)
  const bool rhi = ln < gqa;                             // P row ln: bf16 part of head ln
  const bool rlo = ln >= 4 && ln - 4 < gqa;              // P row ln: remainder of head ln - 4
  const int vrow = 4 * kb + (ln >> 2), vcol = 4 * (ln & 3);   // transposing-read source
  // kMode: 0 a tile alone, 1 the first of a pair (weights kept in pv_pair),
  // 2 the second (values of both; bfp: the first's V buffer)
  floatx4 pv_pair;
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
      for (int rb = 0; rb < kVB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rb][i] *= ah[i];
    }
    // weights 2^(s hscale - m) <= 2^kLazy by the hardware exp2 (results below
    // 2^-126 flush to zero, which a weight of that size is anyway); masked
    // tokens (s = -inf) give 0. The P operand: rows 0..3 bf16(p) of head ln,
    // rows 4..7 the remainders of head ln - 4 (moved four lanes up inside
    // each 16-lane row)
    floatx4 pv;
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], hscale, -m_run));
    l_run += (pv[0] + pv[1]) + (pv[2] + pv[3]);
    auto p_operand = [&](floatx4 w) {
      uint32_t h0, h1, lo0, lo1;
      split_bf16x2(w[0], w[1], h0, lo0);
      split_bf16x2(w[2], w[3], h1, lo1);
      const uint32_t lo0s = __builtin_amdgcn_update_dpp(0u, lo0, 0x114, 0xf, 0xf, true);
      const uint32_t lo1s = __builtin_amdgcn_update_dpp(0u, lo1, 0x114, 0xf, 0xf, true);
      const uint32_t a0 = rhi ? h0 : (rlo ? lo0s : 0u), a1 = rhi ? h1 : (rlo ? lo1s : 0u);
      return __builtin_bit_cast(short4v, uint2{a0, a1});
    };
    // U[row][128 qc + 16 rb + ln] += sum_t P[row][t] H_v[t][128 qc + 16 rb + ln]
    const char* vb = sm.v[bf] + vrow * kVStride<R> + 2 * vcol + (R / 2) * qc;
    if constexpr (mode == 1) {
      pv_pair = pv;
    } else if constexpr (mode == 0) {
      const short4v pa = p_operand(pv);
#pragma unroll
      for (int rb = 0; rb < kVB; ++rb)
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, read_tr16(vb + 32 * rb), acc[rb], 0, 0, 0);
    } else {
      const short8v pa = __builtin_shufflevector(p_operand(pv_pair), p_operand(pv), 0, 1, 2, 3, 4, 5, 6, 7);
      const char* va = sm.v[bfp] + vrow * kVStride<R> + 2 * vcol + (R / 2) * qc;
#pragma unroll
      for (int rb = 0; rb < kVB; ++rb) {
        const short8v hv = __builtin_shufflevector(read_tr16(va + 32 * rb), read_tr16(vb + 32 * rb),
                                                   0, 1, 2, 3, 4, 5, 6, 7);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pa),
                                                          __builtin_bit_cast(bf16x8, hv), acc[rb], 0, 0, 0);
      }
    }
  };

  // Prologue: tiles 0 and 1 into LDS, tile 2 in the register stage, the
  // rotation table of tile 0, the keys of tile 0.
  put(0, 0, stk, stv);
  put(1, 1, st1k, st1v);
  fetch(s0 + 2 * kTile, stk, stv);
  rot.exact(s0, 0);
  barrier_lds();
  floatx4 kx[2], ky[2];
  keys(0, kx);
  barrier_lds();                                         // tile 0's K buffer takes tile 2 next
  int cb = 0, cvb = 0;                                   // K and V buffers of tile it
  int pvb = 0;                                           // V buffer of tile it-1

  // Iteration it (after the barrier that made tiles it and it+1 and tile
  // it's rotation table visible). Region 1 is one straight run of code
  // written as 2 kC slots in a fixed order (the compiler may not move code
  // across slots): slot (c, lb) issues the key MFMA of tile it+1's block
  // qc + 4 lb and chunk c (H_k chunks read two chunks ahead), then its share
  // of the work items of tile it: the LDS copy of tile it+2 from the register
  // stage (its K buffer last held tile it, whose keys were formed before the
  // last barrier; its V buffer tile it-3) and the request of tile it+3 into
  // the stage, the rotation-table rows of the wave's block pair, its four
  // pair rotations, the fp16 pack and the partial score MFMA (its q operand
  // read a few items earlier). Then tile it-1's softmax and values (its
  // partial scores in LDS since the last barrier), tile it's partial scores
  // into LDS, the rotation table of tile it+1 (its buffer last served tile
  // it-1); the barrier.
  constexpr int kSlots = 2 * kC;
  enum : int { kPut = 0, kFetch, kRows, kRot0, kQ = kRot0 + 2, kRot2, kPack = kRot2 + 2, kScore, kN };
  auto region1 = [&](int it, int bf, int vbf, floatx4 (&cur)[2], floatx4 (&nxt)[2], floatx4& sc) {
    const int bf1 = next_buf(bf), bf2 = next_buf(bf1);   // tiles it+1, it+2
    const int vbf2 = next_vbuf(next_vbuf(vbf));          // V of tile it+2
    const char* kt = sm.k[bf1] + ln * kKStride<R> + 16 * kb;
    // H_k chunks in a ring of three, each read two chunks (4 MFMAs) ahead
    u32x4 h[3];
    h[0] = *reinterpret_cast<const u32x4*>(kt);
    h[1] = *reinterpret_cast<const u32x4*>(kt + 64);
    float4 rt[2];
    uint4 a16, q16;
    sc = floatx4{0.f, 0.f, 0.f, 0.f};
    auto item = [&](auto W) {
      constexpr int w = W;
      if constexpr (w == kPut) {
        put(bf2, vbf2, stk, stv);
      } else if constexpr (w == kFetch) {
        fetch(s0 + (it + 3) * kTile, stk, stv);
      } else if constexpr (w == kRows) {                 // frequencies 16 qc + 4 kb + 0..3
        rt[0] = *reinterpret_cast<const float4*>(&sm.rot.rtab[it & 1][8 * qc + 2 * kb][ln][0]);
        rt[1] = *reinterpret_cast<const float4*>(&sm.rot.rtab[it & 1][8 * qc + 2 * kb + 1][ln][0]);
      } else if constexpr (w == kQ) {                    // q of the score MFMA of block pair qc
        q16 = sm.qop[wave][lane];
      } else if constexpr ((w >= kRot0 && w < kRot0 + 2) || (w >= kRot2 && w < kRot2 + 2)) {
        constexpr int i = w < kQ ? w - kRot0 : w - kRot2 + 2;   // pair (f, f + 64), f = 16 qc + 4 kb + i
        const float4 r = rt[i / 2];
        const float c = i % 2 ? r.z : r.x, sn = i % 2 ? r.w : r.y;
        const float x = cur[0][i], y = cur[1][i];
        cur[0][i] = x * c - y * sn;
        cur[1][i] = x * sn + y * c;
      } else if constexpr (w == kPack) {                 // fp16 A operand of the score MFMA
        a16 = uint4{pack_f16x2(cur[0][0], cur[0][1]), pack_f16x2(cur[0][2], cur[0][3]),
                    pack_f16x2(cur[1][0], cur[1][1]), pack_f16x2(cur[1][2], cur[1][3])};
      } else {
        static_assert(w == kScore, "unknown item");      // S[token 4 kb + i][head ln], partial
        sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a16),
                                                    __builtin_bit_cast(f16x8, q16), sc, 0, 0, 0);
      }
    };
    static_for<kSlots>([&](auto S) {
      constexpr int slot = S, c = slot / 2, lb = slot % 2;
      if constexpr (lb == 0 && c + 2 < kC) h[(c + 2) % 3] = *reinterpret_cast<const u32x4*>(kt + 64 * (c + 2));
      const floatx4 acc_in = c == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : nxt[lb];
      hold_in_agpr(bt[lb][c]);
      nxt[lb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bt[lb][c]),
                                                        __builtin_bit_cast(bf16x8, h[c % 3]),
                                                        acc_in, 0, 0, 0);
      constexpr int w0 = slot * kN / kSlots, w1 = (slot + 1) * kN / kSlots;
      static_for<w1 - w0>([&](auto J) { item(std::integral_constant<int, w0 + J>{}); });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // tile pt's softmax and values, one iteration after its scores: the four
  // quarters' partial scores (in LDS since the barrier that ended tile pt's
  // iteration) added in quarter order by every wave of the head, the mask of
  // the split's last tile, the running max
  auto softmax_of = [&](int pt, int vbuf, auto kMode) {
    floatx4 sc = sm.sp[pt & 1][jh][lane];
#pragma unroll
    for (int c = 1; c < kParts; ++c) {
      const floatx4 o = sm.sp[pt & 1][jh + kHeads * c][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] += o[i];
    }
    const int tok0 = s0 + pt * kTile;
    if (tok0 + kTile > t1) {                             // the split's last tile: its tail masked
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = tok0 + 4 * kb + i < t1 ? sc[i] : -INFINITY;
    }
    const float mx = hscale * max_groups(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    softmax_values(vbuf, vbuf == 0 ? kVBuf - 1 : vbuf - 1, sc, mx, kMode);
  };
  // Iteration it: region 1, then tile it-1's softmax and values (kPrev: its
  // mode; none in the first iteration), tile it's partial scores into LDS,
  // the rotation table of tile it+1, the barrier.
  auto iteration = [&](int it, floatx4 (&cur)[2], floatx4 (&nxt)[2], auto kPrev) {
    constexpr int prev = kPrev;                          // -1: no tile it-1
    floatx4 sc;
    region1(it, cb, cvb, cur, nxt, sc);
    if constexpr (prev >= 0) softmax_of(it - 1, pvb, std::integral_constant<int, prev>{});
    sm.sp[it & 1][wave][lane] = sc;
    pvb = cvb;
    cb = next_buf(cb);
    cvb = next_vbuf(cvb);
    if (it + 1 < ntiles) {
      if ((it + 1) % kAnchor == 0) rot.exact(s0 + (it + 1) * kTile, (it + 1) & 1);
      else rot.step(it + 1);
    }
    barrier_lds();
  };
  // tiles go in pairs (even, odd): an even tile's softmax keeps its weights
  // (mode 1), the odd one's takes both tiles' values (mode 2); an even last
  // tile stands alone (mode 0)
  iteration(0, kx, ky, std::integral_constant<int, -1>{});
  int it = 1;
  for (; it + 1 < ntiles; it += 2) {
    iteration(it, ky, kx, std::integral_constant<int, 1>{});
    iteration(it + 1, kx, ky, std::integral_constant<int, 2>{});
  }
  if (it < ntiles) iteration(it, ky, kx, std::integral_constant<int, 1>{});
  if ((ntiles - 1) % 2) softmax_of(ntiles - 1, pvb, std::integral_constant<int, 2>{});
  else softmax_of(ntiles - 1, pvb, std::integral_constant<int, 0>{});

  // ---- partials of this wave's query heads (latent quarter qc): the
  // remainder rows (kb = 1) are added to the bf16 rows (kb = 0); the sum l over
  // the four lane groups (all quarters hold the same m and l: quarter 0
  // writes them)
#pragma unroll
  for (int rb = 0; rb < kVB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[rb][i] = add_pair_groups(acc[rb][i]);
  l_run = sum_groups(l_run);
  if (qc == 0 && kb == 0 && ln < gqa) {
    const size_t slot = (static_cast<size_t>(b) * p.Hq + head0 + ln) * p.n_split + split;
    p.part_ml[slot * 2] = m_run;
    p.part_ml[slot * 2 + 1] = l_run;
  }
  if (kb == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < gqa) {
        const size_t slot = (static_cast<size_t>(b) * p.Hq + head0 + i) * p.n_split + split;
        float* u = p.part_u + slot * R + (R / kParts) * qc;
#pragma unroll
        for (int rb = 0; rb < kVB; ++rb) u[16 * rb + ln] = acc[rb][i];
      }
    }
  }
}

hipError_t launch_quarter(const DecodeParams& p, hipStream_t st) {
  const int nslice = p.s / kHeads;
  if (nslice == 1) {
    const dim3 grid(p.n_split, p.G, p.B);
    split_reconstruct_quarter_kernel<false><<<grid, kThreads, 0, st>>>(p);
  } else {
    const long ids = split_unit_ids(p.n_split, p.G, p.B, nslice);
    if (ids == 0) return hipErrorInvalidValue;
    split_reconstruct_quarter_kernel<true><<<dim3(static_cast<unsigned>(ids)), kThreads, 0, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

bool reconstruct_quarter_supported(const DecodeParams& p, int dtype) {
  return dtype == 1 && p.d == kD && p.gqa <= 4 && p.r == R && p.s % kHeads == 0;
}

hipError_t launch_split_reconstruct_quarter(const DecodeParams& p, hipStream_t st) {
  return p.r == R ? launch_quarter(p, st) : hipErrorInvalidValue;
}

}  // namespace palu
