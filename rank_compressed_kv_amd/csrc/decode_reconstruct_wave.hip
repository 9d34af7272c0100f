// Context-split decode kernel for the reconstruct mode (keys rebuilt per tile
// and rotated), bf16 latents, on the gfx950 matrix cores: one wave per KV head.
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
// 64 or 128, and either a multiple of four KV heads per group or groups of
// one or two KV heads (rank 256 has a kernel of its own). A workgroup has
// four waves, one per KV head, and owns one context split of one batch row
// for four consecutive KV heads: a slice of one group, or four (two) whole
// groups of one (two) KV heads, each group with its own latent tile. Each
// wave keeps its KV head's whole B_k^T (128 columns x r latents, from a
// transposed copy in the workspace) in registers for the split, so a wave
// rebuilds, rotates and scores its head's keys on its own: no partial scores
// cross waves, and each wave runs the online softmax of its own query heads
// only. The waves of a group share its latent tiles (read from HBM once per
// workgroup into LDS, loaded by those waves); all four share the rotation
// table (same tokens); their softmax states never meet (each wave writes its
// heads' split partials itself).
// Per 16-token tile, wave of KV head j:
//   keys     K^T[16 cols x 16 tok] = B_k^T[cols x r] * H_k^T[r x tok] for the 8
//            column blocks, bf16 MFMA 16x16x32, H_k from the tile in LDS. Lane
//            l holds columns 16 blk + 4 (l/16) + i of token l%16.
//   rotate   the pair (f, f + 64) is block blk and blk + 4 at the same register,
//            so a lane rotates its own values; cos and sin of t * omega_f come
//            from a table in LDS that all waves share (computed once per tile
//            by the workgroup: each entry is the previous tile's entry times
//            the frequency's 16-position step, one exact complex product,
//            and every kAnchor tiles it is evaluated from the fp64-reduced
//            angle), stored times 2^-8 so the rotated keys come out scaled into
//            fp16's range.
//   scores   S[tok x q heads] by fp16 MFMA 16x16x32: the rotated keys rounded
//            once to fp16 (the A operand needs no reshuffle: block pairs
//            (m, m+4) fill a lane's eight k-slots) against q, held in LDS in
//            fp16 after a per-head power-of-two scale (exact: bf16 q has 8
//            significant bits); fp32 accumulation. Once the keys are packed,
//            the key registers take the next tile's key MFMAs, which run
//            under this tile's softmax and values (one wave per SIMD: the
//            overlap has to come from inside the wave).
//   softmax  online, base 2, lazy rescale (the stored max moves only when a
//            tile exceeds it by kLazy); lane l%16 = query head.
//   values   U[rows x r] += P[rows x 16 tok] * H_v[16 tok x r], bf16 MFMA
//            16x16x16: rows 0..3 hold the weights of the (up to four) query
//            heads rounded to bf16, rows 4..7 the remainders (p - bf16(p)), so
//            the weights keep ~16 bits; the H_v operand comes straight from
//            the LDS tile with the gfx950 transposing read (ds_read_b64_tr_b16:
//            a 16-lane group reads four 32-byte token rows and each lane gets
//            one latent column of the four tokens).
// Loads: 16-byte pieces of each tile go through two register stages into a
// ring of four LDS buffers; rows past the split's end are
// clamped to its last valid row and masked. One workgroup barrier per tile
// (LDS only, so the loads stay in flight across it).
#include "reconstruct_wave_util.h"

namespace palu {
namespace {

using namespace wave;

constexpr int kNBuf = 4;           // LDS tile buffers

// K tile row stride: 32 mod 64 bytes keeps the operand reads free of bank
// conflicts; the four-group rank-32 form takes 16 mod 64 (one key chunk a
// tile, so its few reads may conflict) to stay within half the LDS, which
// lets two of its workgroups share a CU
template <int R, int NG>
constexpr int kKS = NG == 4 && R == 32 ? 2 * R + 16 : kKStride<R>;

// NG: latent tiles a workgroup streams at once (one per head group it covers)
template <int R, int NG>
struct Smem {
  char k[kNBuf][NG][kTile * kKS<R, NG>];
  char v[kNBuf][NG][kTile * kVStride<R>];
  RotTable rot;
  // q of each wave's query heads as the score MFMA's B operand (fp16), lane
  // order: qop[wave][m][lane]
  uint4 qop[4][4][64];
};

// Work items of an iteration (see the kernel's main loop) and the two orders
// they are issued in.
enum Item : int {
  kPut = 0, kFetch = 1, kP = 2, kRows0 = 3, kVRead0 = 7, kVMfma0 = 11, kRot0 = 15,
  kPack0 = 31, kRope = 35, kScore0 = 36, kMask = 40, kMax = 41
};
#define ROT(b) kRot0 + 4 * (b), kRot0 + 4 * (b) + 1, kRot0 + 4 * (b) + 2, kRot0 + 4 * (b) + 3
// the order of the items; they are spread evenly over the key MFMAs
constexpr int kOrder[] = {
    kPut, kFetch, kP, kRows0, kRows0 + 1, kVRead0, ROT(0), kVRead0 + 1, kVMfma0, kRows0 + 2,
    ROT(1), kVRead0 + 2, kVMfma0 + 1, kRows0 + 3, ROT(2), kVRead0 + 3, kVMfma0 + 2, ROT(3),
    kVMfma0 + 3, kPack0, kPack0 + 1, kPack0 + 2, kPack0 + 3, kRope, kScore0, kScore0 + 1,
    kScore0 + 2, kScore0 + 3, kMask, kMax};
#undef ROT
template <int N>
constexpr int count_of(const int (&)[N]) { return N; }

template <int R, int HW, int NG, bool kShared>
__global__ __launch_bounds__(64 * HW, NG > 1 ? 2 : 1) void split_reconstruct_wave_kernel(DecodeParams p) {
  constexpr int kThreads = 64 * HW;
  constexpr int kWS = HW / NG;                                  // waves (KV heads) sharing a tile
  constexpr int kST = 64 * kWS;                                 // threads that load a tile
  constexpr int kPieces = (2 * R + kST - 1) / kST;              // 16-B pieces per matrix
  constexpr int kC = R / 32;                                    // 32-latent key chunks
  constexpr int kRB = R / 16;                                   // 16-latent value blocks
  static_assert(HW % NG == 0, "whole groups per workgroup");
  // NG = 1: the HW KV heads are a slice of one group; NG > 1: groups of
  // HW / NG KV heads, NG consecutive groups a workgroup (units over (split,
  // group block, batch))
  const int nslice = NG > 1 ? 1 : p.s / HW;
  const SplitUnit un = split_unit(p.n_split, p.G / NG, p.B, nslice);
  if (!un.live) return;
  const int split = un.split, b = un.b, hs = un.hs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gs = NG > 1 ? wave / kWS : 0;               // this wave's tile slot
  const int g = un.g * NG + gs;                          // its group
  const int stid = tid - gs * kST;                       // its thread's index among the slot's loaders
  const int ln = lane & 15, kb = lane >> 4;
  const int n = clamp_len(p.lens, b, p.L);
  const int s0 = split * p.split_tokens;
  if (s0 >= n) return;                                   // whole workgroup
  const int t1 = min(n, s0 + p.split_tokens);
  const int last = t1 - 1;
  const int gqa = p.gqa;                                 // query heads per KV head (<= 4)
  const int kvh = NG > 1 ? wave % kWS : hs * HW + wave;  // this wave's KV head in its group
  const int head0 = g * p.nq + kvh * gqa;                // its first query head

  __shared__ Smem<R, NG> sm;

  // ---- operands held for the whole split -----------------------------------
  // B_k^T as the key MFMA's A operand (column 16 blk + ln, latents 32 c + 8 kb
  // .. +8 in lane (ln, kb) of block blk, chunk c), from the transposed copy
  u32x4 bt[8][kC];
  load_bkt<kC>(bt, static_cast<const uint16_t*>(p.bkt) + (static_cast<size_t>(g) * p.Dg + kvh * kD) * R,
               R, 0, ln, kb);
  const float hscale = q_operand(p, b, head0, gqa, ln, kb, lane, sm.qop[wave]);

  // the rotation table (shared by the waves; filled by all threads)
  Rot<kThreads> rot(sm.rot, tid, p.rope != 0);
  rot.init(p, tid);
  barrier_lds();                                         // rstep and orev before any use

  // ---- softmax state of query head ln (lanes ln >= gqa carry a zero query
  // and are never written out)
  float m_run = -INFINITY, l_run = 0.f;
  // value-latent sums: acc[rb] holds rows 4 kb .. 4 kb + 3 of latent 16 rb + ln
  // (kb = 0: the bf16 parts of query heads 0..3, kb = 1: the remainders)
  floatx4 acc[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) acc[rb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const size_t row0 = (static_cast<size_t>(b) * p.G + g) * p.L;
  const uint16_t* Hk = static_cast<const uint16_t*>(p.h_k) + row0 * R;
  const uint16_t* Hv = static_cast<const uint16_t*>(p.h_v) + row0 * R;
  const int ntiles = (t1 - s0 + kTile - 1) / kTile;

  // keys of tile it (K tile in LDS): kk[blk] = K^T of column block blk
  auto keys = [&](int it, floatx4 (&kk)[8]) {
    const char* kt = sm.k[it % kNBuf][gs];
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) kk[blk] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const bf16x8 h = as_bf16x8(*reinterpret_cast<const uint4*>(kt + ln * kKS<R, NG> + 2 * (32 * c + 8 * kb)));
#pragma unroll
      for (int blk = 0; blk < 8; ++blk)
        kk[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bt[blk][c]), h,
                                                          kk[blk], 0, 0, 0);
    }
  };

  // The softmax and values of a tile run one iteration after its scores
  // (inside the next tile's schedule). First the rare rescale, in its own
  // small block: when a tile's max exceeds the stored max by more than
  // kLazy, the stored max moves and the sums are scaled down.
  const bool rhi = ln < gqa;                             // P row ln: bf16 part of head ln
  const bool rlo = ln >= 4 && ln - 4 < gqa;              // P row ln: remainder of head ln - 4
  const int vrow = 4 * kb + (ln >> 2), vcol = 4 * (ln & 3);   // transposing-read source
  auto rescale = [&](float mx) {
    if (__any(mx > m_run + kLazy)) {                     // wave-uniform, rare
      const float mn = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - mn);
      m_run = mn;
      l_run *= alpha;
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
  };
  // the P operand of a tile's raw scores: weights 2^(s hscale - m) <= 2^kLazy by the
  // hardware exp2 (results below 2^-126 flush to zero, which a weight of
  // that size is anyway; masked tokens, s = -inf, give 0); rows 0..3 bf16(p)
  // of head ln, rows 4..7 the remainders of head ln - 4 (moved four lanes up
  // inside each 16-lane row)
  auto p_operand = [&](floatx4 sc) {
    floatx4 pv;
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], hscale, -m_run));
    l_run += (pv[0] + pv[1]) + (pv[2] + pv[3]);
    uint32_t h0, h1, lo0, lo1;
    split_bf16x2(pv[0], pv[1], h0, lo0);
    split_bf16x2(pv[2], pv[3], h1, lo1);
    const uint32_t lo0s = __builtin_amdgcn_update_dpp(0u, lo0, 0x114, 0xf, 0xf, true);
    const uint32_t lo1s = __builtin_amdgcn_update_dpp(0u, lo1, 0x114, 0xf, 0xf, true);
    const uint32_t a0 = rhi ? h0 : (rlo ? lo0s : 0u), a1 = rhi ? h1 : (rlo ? lo1s : 0u);
    return __builtin_bit_cast(short4v, uint2{a0, a1});
  };
  // values: U[row][16 rb + ln] += sum_t P[row][t] H_v[t][16 rb + ln], value
  // blocks in four groups
  auto vgroup = [](int g, int& b0, int& b1) { b0 = g * kRB / 4; b1 = (g + 1) * kRB / 4; };

  // Loads: thread piece i (< kPieces) is the 16-byte piece stid + i*kST of
  // the tile (byte 16*that in a row-major tile of 16 rows), if below 2R. Two
  // tiles wait in registers (stages a and b, vector types so they stay in
  // registers) and two ahead of the one being consumed are in LDS.
  typedef uint32_t u32v __attribute__((ext_vector_type(4 * kPieces)));
  // (the piece guard is a compile-time true when the threads divide the tile,
  // so the loads and copies add no branch to the iteration's straight run)
  constexpr bool kWhole = (2 * R) % kST == 0;
  auto fetch = [&](int tok0, u32v& k, u32v& v) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int pc = stid + i * kST;
      if (kWhole || pc < 2 * R) {
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
      const int pc = stid + i * kST;
      if (kWhole || pc < 2 * R) {
        const int prow = (pc * 16) / (2 * R), pcol = (pc * 16) % (2 * R);
        *reinterpret_cast<uint4*>(sm.k[buf][gs] + prow * kKS<R, NG> + pcol) =
            uint4{k[4 * i], k[4 * i + 1], k[4 * i + 2], k[4 * i + 3]};
        *reinterpret_cast<uint4*>(sm.v[buf][gs] + prow * kVStride<R> + pcol) =
            uint4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
      }
    }
  };

  // An iteration is one straight run of code written as 8 kC slots in a
  // fixed order (the compiler may not move code across slots): slot
  // (c, blk) issues the key MFMA of tile it+1's column block blk and chunk
  // c, then its share of the VALU and LDS work items of the iteration: the
  // LDS copy of tile it+2 from its register stage (its buffer last held tile
  // it-2, finished before the last barrier) and the request of tile
  // it+2+kStages into the same stage (kStages whole iterations to arrive),
  // tile it-1's P operand, value reads and value MFMAs, tile it's
  // rotation-table reads, 16 pair rotations, fp16 packs, score MFMAs, mask
  // and running max, and the rotation table of tile it+1 (recurrence step;
  // every kAnchor tiles it is then overwritten by the exact values, outside
  // the run). The wave is alone on its SIMD, so only this interleaving lets
  // the matrix core and the VALU work at once. The next H_k chunk is read
  // half a chunk ahead.
  static_assert(R <= 128, "B_k^T of one KV head must fit the AGPRs");
  constexpr int kStages = 2;
  constexpr int kSlots = 8 * kC;
  u32v stg[kStages][2];
  fetch(s0, stg[0][0], stg[0][1]);
  put(0, stg[0][0], stg[0][1]);
  fetch(s0 + kTile, stg[0][0], stg[0][1]);
  put(1, stg[0][0], stg[0][1]);
#pragma unroll
  for (int i = 0; i < kStages; ++i) fetch(s0 + (2 + i) * kTile, stg[i][0], stg[i][1]);
  rot.exact(s0, 0);
  barrier_lds();
  floatx4 kx[8], ky[8];
  keys(0, kx);
  floatx4 sc_prev = {0.f, 0.f, 0.f, 0.f};                // scores of tile it-1
  float mx_prev = -INFINITY;

  auto iteration = [&](int it, floatx4 (&cur)[8], floatx4 (&nxt)[8], u32v& k, u32v& v,
                       auto kVals) {
    constexpr bool vals = kVals;                          // tile it-1 exists
    if constexpr (vals) rescale(mx_prev);
    const int tok0 = s0 + it * kTile;
    const char* kt = sm.k[(it + 1) % kNBuf][gs] + ln * kKS<R, NG> + 16 * kb;
    const char* vb = sm.v[(it + kNBuf - 1) % kNBuf][gs] + vrow * kVStride<R> + 2 * vcol;
    const uint4* qo = &sm.qop[wave][0][lane];
    u32x4 h[2];
    h[0] = *reinterpret_cast<const u32x4*>(kt);
    float4 rt[4][2];
    uint4 a16[4];
    short4v pa;
    short4v vr[kRB];
    floatx4 sc = {0.f, 0.f, 0.f, 0.f};
    float mx = 0.f;
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
    auto vread = [&](int g) {
      int b0, b1;
      vgroup(g, b0, b1);
#pragma unroll
      for (int rb = b0; rb < b1; ++rb) vr[rb] = read_tr16(vb + 32 * rb);
    };
    auto vmfma = [&](int g) {
      int b0, b1;
      vgroup(g, b0, b1);
#pragma unroll
      for (int rb = b0; rb < b1; ++rb)
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vr[rb], acc[rb], 0, 0, 0);
    };
    // items: 0 copy, 1 request, 2 P(it-1), 3-4 table rows of blocks 0-1, 5
    // value reads 0, 6-9 rotations of block 0, 10 value reads 1, 11 value
    // MFMAs 0, 12 rows 2, 13-16 rotations 1, 17 reads 2, 18 MFMAs 1, 19 rows
    // 3, 20-23 rotations 2, 24 reads 3, 25 MFMAs 2, 26-29 rotations 3, 30
    // MFMAs 3, 31-34 packs, 35 table of tile it+1, 36-39 score MFMAs, 40
    // the mask of the split's last tile, 41 running max
    auto item = [&](auto W) {
      constexpr int w = W;
      if constexpr (w == kPut) {
        put((it + 2) % kNBuf, k, v);
      } else if constexpr (w == kFetch) {
        fetch(s0 + (it + 2 + kStages) * kTile, k, v);
      } else if constexpr (w == kP) {
        if constexpr (vals) pa = p_operand(sc_prev);
      } else if constexpr (w >= kRows0 && w < kRows0 + 4) {
        rows(w - kRows0);
      } else if constexpr (w >= kVRead0 && w < kVRead0 + 4) {
        if constexpr (vals) vread(w - kVRead0);
      } else if constexpr (w >= kVMfma0 && w < kVMfma0 + 4) {
        if constexpr (vals) vmfma(w - kVMfma0);
      } else if constexpr (w >= kRot0 && w < kRot0 + 16) {
        rotate((w - kRot0) / 4, (w - kRot0) % 4);
      } else if constexpr (w >= kPack0 && w < kPack0 + 4) {   // fp16 A operand of score MFMA m
        constexpr int m = w - kPack0;
        a16[m] = uint4{pack_f16x2(cur[m][0], cur[m][1]), pack_f16x2(cur[m][2], cur[m][3]),
                       pack_f16x2(cur[m + 4][0], cur[m + 4][1]),
                       pack_f16x2(cur[m + 4][2], cur[m + 4][3])};
      } else if constexpr (w == kRope) {
        rot.step(it + 1);
      } else if constexpr (w >= kScore0 && w < kScore0 + 4) {   // S[token 4 kb + i][head ln]
        constexpr int m = w - kScore0;
        sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a16[m]),
                                                    __builtin_bit_cast(f16x8, qo[64 * m]), sc,
                                                    0, 0, 0);
      } else if constexpr (w == kMask) {                 // the split's last tile: its tail masked
        if (tok0 + kTile > t1) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[i] = tok0 + 4 * kb + i < t1 ? sc[i] : -INFINITY;
        }
      } else {                                           // in log2 units (hscale > 0)
        static_assert(w == kMax, "unknown item");
        mx = hscale * max_groups(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
      }
    };
    // one key MFMA: column block blk, chunk c of tile it+1 (the next H_k
    // chunk read half a chunk ahead)
    auto key_slot = [&](auto S) {
      constexpr int slot = S, c = slot / 8, blk = slot % 8;
      if constexpr (blk == 4 && c + 1 < kC) h[(c + 1) & 1] = *reinterpret_cast<const u32x4*>(kt + 64 * (c + 1));
      const floatx4 acc_in = c == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : nxt[blk];
      hold_in_agpr(bt[blk][c]);
      nxt[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bt[blk][c]),
                                                         __builtin_bit_cast(bf16x8, h[c & 1]),
                                                         acc_in, 0, 0, 0);
    };
    constexpr int kN = count_of(kOrder);
    static_for<kSlots>([&](auto S) {
      constexpr int slot = S;
      key_slot(S);
      constexpr int w0 = slot * kN / kSlots, w1 = (slot + 1) * kN / kSlots;
      static_for<w1 - w0>([&](auto J) { item(std::integral_constant<int, kOrder[w0 + J]>{}); });
      __builtin_amdgcn_sched_barrier(0);
    });
    if ((it + 1) % kAnchor == 0) rot.exact(s0 + (it + 1) * kTile, (it + 1) & 1);
    sc_prev = sc;
    mx_prev = mx;
    barrier_lds();
  };
  iteration(0, kx, ky, stg[0][0], stg[0][1], std::false_type{});
  for (int it = 1; it < ntiles; it += 2) {
    iteration(it, ky, kx, stg[1][0], stg[1][1], std::true_type{});
    if (it + 1 >= ntiles) break;
    iteration(it + 1, kx, ky, stg[0][0], stg[0][1], std::true_type{});
  }
  // the last tile's softmax and values
  {
    rescale(mx_prev);
    const short4v pa = p_operand(sc_prev);
    const char* vb = sm.v[(ntiles - 1) % kNBuf][gs] + vrow * kVStride<R> + 2 * vcol;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      acc[rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, read_tr16(vb + 32 * rb), acc[rb], 0, 0, 0);
  }

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

template <int R, int HW>
hipError_t launch_shape(const DecodeParams& p, hipStream_t st) {
  const int nslice = p.s / HW;
  if (nslice == 1) {
    const dim3 grid(p.n_split, p.G, p.B);
    split_reconstruct_wave_kernel<R, HW, 1, false><<<grid, 64 * HW, 0, st>>>(p);
  } else {
    const long ids = split_unit_ids(p.n_split, p.G, p.B, nslice);
    if (ids == 0) return hipErrorInvalidValue;
    split_reconstruct_wave_kernel<R, HW, 1, true>
        <<<dim3(static_cast<unsigned>(ids)), 64 * HW, 0, st>>>(p);
  }
  return hipGetLastError();
}

// groups of one or two KV heads: NG = 4 / s groups a four-wave workgroup
template <int R, int NG>
hipError_t launch_groups(const DecodeParams& p, hipStream_t st) {
  if (p.G % NG != 0) return hipErrorInvalidValue;
  const dim3 grid(p.n_split, p.G / NG, p.B);
  split_reconstruct_wave_kernel<R, 4, NG, false><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

// Four waves (KV heads) a workgroup always: with fewer, the workgroup's few
// waves fill the LDS ring and the rotation table alone, and the
// block-per-split kernel is faster (rank 32 with one KV head a workgroup: 481
// against 191 us at the Llama-3-8B shape). Groups of fewer than four KV
// heads therefore share a workgroup: four consecutive KV heads of four (or
// two) groups, each group's tile loaded by its own waves into its own ring.
bool reconstruct_wave_supported(const DecodeParams& p, int dtype) {
  if (dtype != 1 || p.d != kD || p.gqa > 4) return false;
  if (p.s % 4 == 0) return p.r == 32 || p.r == 64 || p.r == 128;
  // one or two KV heads a group: four consecutive KV heads (of four or two
  // groups) a workgroup, one latent tile per group (the four tiles of rank
  // 128 would not fit the LDS)
  if ((p.s == 1 || p.s == 2) && p.Hkv % 4 == 0)
    return p.r == 32 || p.r == 64 || (p.r == 128 && p.s == 2);
  return false;
}

hipError_t launch_split_reconstruct_wave(const DecodeParams& p, hipStream_t st) {
  if (p.s == 1) {
    switch (p.r) {
      case 32: return launch_groups<32, 4>(p, st);
      case 64: return launch_groups<64, 4>(p, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (p.s == 2) {
    switch (p.r) {
      case 32: return launch_groups<32, 2>(p, st);
      case 64: return launch_groups<64, 2>(p, st);
      case 128: return launch_groups<128, 2>(p, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (p.r) {
    case 32: return launch_shape<32, 4>(p, st);
    case 64: return launch_shape<64, 4>(p, st);
    case 128: return launch_shape<128, 4>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace palu
