// Cache write of one new token per sequence: h = x A (Palu author response,
// answer to Q2 on ESPACE: the down-projection output is what is cached).
//
// x [B, d_model] times A [d_model, G*r] is a skinny product whose cost is
// reading A once (4 MiB per matrix at d_model 4096, G*r 512 in bf16) and whose
// time is one memory latency if every load of the chip is in flight together.
// One launch does all of it, split over d_model:
//   every workgroup owns a block of columns of [A_k | A_v] (128 columns and
//   four waves for a dtype cache, 256 and eight for a quantised one) and a
//   128-row slice; thread (8-column chunk, row group of 8 rows) issues its
//   eight 16-byte loads at once and accumulates x[b, row] * A[row, col] for
//   every sequence. The 16 row groups are added in LDS in a fixed order and
//   the workgroup stores one fp32 partial per (slice, sequence, column) in
//   the workspace, then counts itself in the column block's arrival counter;
//   the last workgroup of a column block adds the slice partials in slice
//   order, rounds (bf16: nearest, ties to even), writes row pos[b] of the
//   cache and puts the counter back to zero for the next call.
// The result does not depend on which workgroup arrives last.
//
// Quantised caches (per-token quantisation of the latents, Palu author
// response to reviewer Fsn9 on W1/W2): each cached row of r latents is stored
// as int8 codes with one fp32 scale, amax / 127, codes round(h * 127 / amax)
// (nearest, ties to even; all in fp32), or as int4 codes with amax / 7. A
// row (r in {64, 128, 256} columns, aligned to r) never crosses a 256-column
// block, so the block's last arriver holds whole rows: it stages them in LDS
// and quantises them there, one wave per (sequence, row).
// With the Hadamard option (a quantisation-friendly enhancement the author
// responses name, answer to Q2) each fp32 row is first rotated by Sylvester's
// H_r, h'' = h H_r, which spreads an outlier latent over all r codes.
//
// The launch can also carry the next decode call's query absorption
// (q~ = q B_k^T, which reads neither the cache nor A): its workgroups come
// after the append's in the grid, each running one absorb_rows unit, so the
// two run side by side in one launch instead of one after the other.
#include "absorb_device.h"
#include "device_util.h"
#include "palu_internal.h"

namespace palu {
namespace {

constexpr int kRows = 128;          // d_model rows per slice
constexpr int kMinCols = 128;       // the narrower column block (counter area size)
constexpr size_t kCounterAlign = 256;

// Tiling of the two forms. dtype caches: 128-column blocks of four waves
// (measured 10.8 us against 11.6 us for the wider form at Llama-3-8B);
// quantised caches: 256-column blocks of eight waves, so that a block holds
// whole quantised rows (12.7 us against 14.4 us with a second hand-off).
template <bool kQuant>
struct Tiling {
  static constexpr int kThreads = kQuant ? 512 : 256;
  static constexpr int kCols = kQuant ? 256 : kMinCols;
  static constexpr int kChunks = kCols / 8;                   // 8-column chunks
  static constexpr int kRowGroups = kThreads / kChunks;       // threads per chunk
  static constexpr int kRowsPerThread = kRows / kRowGroups;
  static constexpr int kBatchChunk = kQuant ? 4 : 8;          // sequences per LDS round
  static constexpr int kXPer = kBatchChunk * kRows / kThreads;   // x entries per thread
  static constexpr int kReaders = kThreads / (2 * kChunks);   // sequences per final round
  // LDS slot of the 4-column quarter (chunk cc, half hf) of a block: the two
  // halves of a chunk are kChunks slots apart so a wave's 16-byte writes
  // spread over all banks; slot q holds columns col_of_slot(q) .. +4.
  static __device__ __forceinline__ int col_of_slot(int q) {
    return q < kChunks ? 8 * q : 8 * (q - kChunks) + 4;
  }
};

// Hand-off of the partials between workgroups on different XCDs, whose L2
// caches are not coherent with each other, in release/acquire terms:
//   writer: device-scope (agent) stores of the partials, then the workgroup
//           barrier (every wave's stores happen before it), then one thread's
//           counter increment with release semantics at agent scope, which
//           makes everything that happened before it visible at agent scope
//           before the increment is;
//   reader: the last arriver's increment reads the final count; after the
//           workgroup barrier every thread takes an agent-scope acquire fence
//           (which drops its stale cached lines), so ordinary 16-byte loads
//           see every partial.
// The stores themselves are agent-scope atomics so that the release has no
// dirty L2 lines of this data to write back.
__device__ __forceinline__ void store_coherent2(float* p, float a, float b) {
  const uint64_t bits = static_cast<uint64_t>(__float_as_uint(a)) |
                        (static_cast<uint64_t>(__float_as_uint(b)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), bits, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Byte offset of latent k of token t inside one (b, g) slab of the int8 cache.
// The slab is a run of 32-token blocks of 32 r bytes each, ordered as the
// decode kernel's MFMA operands so that 16-byte word i of lane l of a block is
// bytes [1024 i + 16 l, +16) (lane l = 16 kb + ln):
//   keys:   half h = (t%32)/16 of the block holds 16 tokens, ln = t%16; the
//           16 bytes of (word, kb, ln) are latents 32c + 8kb + j, c = 2 word' +
//           byte/8 (word' the word within the half), j = byte%8;
//   values: the 16 bytes of (word, kb, ln) are latent 16 rb + ln, rb = 2 word +
//           byte/8, of the tokens 4kb + j (j = byte%8 < 4) and 16 + 4kb + j - 4.
__device__ __forceinline__ size_t i8_key_offset(int t, int k, int r) {
  return static_cast<size_t>(t / 32) * 32 * r + ((t % 32) / 16) * 16 * r + (k / 64) * 1024 +
         ((k % 32) / 8) * 256 + (t % 16) * 16 + ((k / 32) % 2) * 8 + k % 8;
}
__device__ __forceinline__ size_t i8_value_offset(int t, int k, int r) {
  return static_cast<size_t>(t / 32) * 32 * r + (k / 32) * 1024 + ((t % 16) / 4) * 256 +
         (k % 16) * 16 + ((k / 16) % 2) * 8 + ((t % 32) / 16) * 4 + t % 4;
}

// int4 cache: byte of latent k of token t inside one (b, g) slab (32-token
// blocks of 16 r bytes, word w of lane l at 1024 w + 16 l as for int8) and the
// nibble it occupies (hi = 1: the high nibble). A lane's 32-bit unit holds its
// eight operand elements, element 2m in nibble m and 2m+1 in nibble m+4; keys:
// unit h*r/32 + c of half h and chunk c (elements: latents 32c + 8kb + j);
// values: unit rb (elements: tokens 4kb + j and 16 + 4kb + j - 4 of latent
// 16 rb + ln).
__device__ __forceinline__ size_t i4_byte(int t, int unit, int j, int lane, int r, int& hi) {
  const int pos = (j & 1) ? 4 + (j >> 1) : (j >> 1);   // nibble within the unit
  const int bl = unit * 4 + pos / 2;                     // byte within the lane's r/4
  hi = pos & 1;
  return static_cast<size_t>(t / 32) * 16 * r + (bl / 16) * 1024 + lane * 16 + bl % 16;
}
__device__ __forceinline__ size_t i4_key_byte(int t, int k, int r, int& hi) {
  const int unit = ((t % 32) / 16) * (r / 32) + k / 32;
  return i4_byte(t, unit, k % 8, 16 * ((k % 32) / 8) + t % 16, r, hi);
}
__device__ __forceinline__ size_t i4_value_byte(int t, int k, int r, int& hi) {
  const int tt = t % 32;
  return i4_byte(t, k / 16, (tt / 16) * 4 + tt % 4, 16 * ((tt % 16) / 4) + k % 16, r, hi);
}

// h H_r for the row a wave holds, four consecutive latents 4 lane + e per lane
// (lanes >= nq hold zeros): butterflies (x_i, x_i+m) -> (x_i + x_i+m,
// x_i - x_i+m) over the two index bits inside the lane, then over lane bits
__device__ __forceinline__ float4 hadamard_row(float4 v, int lane, int nq) {
  const float a = v.x + v.y, b = v.x - v.y, c = v.z + v.w, d = v.z - v.w;
  v = float4{a + c, b + d, a - c, b - d};
  for (int m = 1; m < nq; m *= 2) {                    // wave-uniform bound
    const float4 o = {__shfl_xor(v.x, m), __shfl_xor(v.y, m), __shfl_xor(v.z, m),
                      __shfl_xor(v.w, m)};
    const bool up = (lane & m) != 0;
    v = up ? float4{o.x - v.x, o.y - v.y, o.z - v.z, o.w - v.w}
           : float4{v.x + o.x, v.y + o.y, v.z + o.z, v.w + o.w};
  }
  return v;
}

// quantise one finished fp32 row (segment j = matrix j / G, group j % G of
// sequence b, four consecutive latents per lane: r in {64, 128, 256}, so nq
// <= 64) into the cache at pos: one wave
__device__ void quantize_row(const AppendParams& p, float4 v0, int j, int b, int pos, int lane) {
  const bool is_v = j >= p.G;
  const int g = is_v ? j - p.G : j;
  int8_t* h = static_cast<int8_t*>(is_v ? p.h_v : p.h_k);
  float* sc = is_v ? p.s_v : p.s_k;
  const int nq = p.r / 4;                              // float4 per row, <= 64
  if (lane >= nq) v0 = float4{0.f, 0.f, 0.f, 0.f};
  if (p.hadamard) v0 = hadamard_row(v0, lane, nq);
  float amax = fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w)));
#pragma unroll
  for (int o = 32; o >= 1; o /= 2) amax = fmaxf(amax, __shfl_xor(amax, o));
  // correctly rounded fp32 divisions (the HIP default); int4: 15 levels
  const float qmax = p.quant == 4 ? 7.f : 127.f;
  const float scale = amax > 0.f ? amax / qmax : 0.f;
  const float inv = amax > 0.f ? qmax / amax : 0.f;
  auto code = [&](float x) {
    const float c = fminf(fmaxf(rintf(x * inv), -qmax), qmax);
    return static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(c)));
  };
  auto code4 = [&](float x) {                          // biased nibble code + 8
    return static_cast<uint32_t>(static_cast<int>(fminf(fmaxf(rintf(x * inv), -7.f), 7.f)) + 8);
  };
  auto pack = [&](float4 v) {
    return code(v.x) | (code(v.y) << 8) | (code(v.z) << 16) | (code(v.w) << 24);
  };
  const size_t row = (static_cast<size_t>(b) * p.G + g) * p.L + pos;
  if (p.quant == 4) {
    // keys: the four latents 4 lane .. +3 fill two whole bytes; values: each
    // byte also holds another token's code (not written by this call), so
    // its other nibble is kept
    uint8_t* slab4 = reinterpret_cast<uint8_t*>(h) + (row - pos) * (p.r / 2);
    if (lane < nq) {
      const int k0 = 4 * lane;
      int hi;
      if (!is_v) {
        slab4[i4_key_byte(pos, k0, p.r, hi)] =
            static_cast<uint8_t>(code4(v0.x) | (code4(v0.z) << 4));
        slab4[i4_key_byte(pos, k0 + 1, p.r, hi)] =
            static_cast<uint8_t>(code4(v0.y) | (code4(v0.w) << 4));
      } else {
        const float e[4] = {v0.x, v0.y, v0.z, v0.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint8_t* byte = slab4 + i4_value_byte(pos, k0 + i, p.r, hi);
          const uint32_t u = code4(e[i]);
          *byte = static_cast<uint8_t>(hi ? ((*byte & 0x0Fu) | (u << 4)) : ((*byte & 0xF0u) | u));
        }
      }
    }
  } else {
    int8_t* slab = h + (row - pos) * p.r;
    // keys: four consecutive latents are four consecutive bytes; values: 16
    // bytes apart
    if (lane < nq) {
      const int k = 4 * lane;
      if (!is_v) {
        *reinterpret_cast<uint32_t*>(slab + i8_key_offset(pos, k, p.r)) = pack(v0);
      } else {
        const float e[4] = {v0.x, v0.y, v0.z, v0.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          slab[i8_value_offset(pos, k + i, p.r)] = static_cast<int8_t>(static_cast<uint8_t>(code(e[i])));
      }
    }
  }
  if (lane == 0) sc[row] = scale;
}

// kFuse: the launch also carries the query absorption of the decode call that
// follows, as workgroups past the last row slice (one absorb_rows unit each,
// staged in this kernel's reduction buffer, which they do not otherwise use);
// they share no data with the append's workgroups.
template <typename T, bool kQuant, bool kFuse>
__global__ __launch_bounds__(Tiling<kQuant>::kThreads) void append_kernel(AppendParams p) {
  using Tl = Tiling<kQuant>;
  constexpr int kThreads = Tl::kThreads, kCols = Tl::kCols, kChunks = Tl::kChunks;
  constexpr int kRowGroups = Tl::kRowGroups, kRowsPerThread = Tl::kRowsPerThread;
  constexpr int kBatchChunk = Tl::kBatchChunk, kXPer = Tl::kXPer, kReaders = Tl::kReaders;
  __shared__ float4 red[kRowGroups][kBatchChunk][2 * kChunks];
  if constexpr (kFuse) {
    static_assert(sizeof(red) >= kAbsHeadChunk * 2 * kMaxHalfDim * sizeof(float),
                  "the reduction buffer holds the absorption's query rows");
    if (static_cast<int>(blockIdx.y) >= p.nslices) {
      const int u = (blockIdx.y - p.nslices) * gridDim.x + blockIdx.x;
      if (u >= p.ab.units) return;
      absorb_rows<T, kThreads>(p.ab, u % p.ab.Hkv, (u / p.ab.Hkv) % p.ab.B,
                               u / (p.ab.Hkv * p.ab.B),
                               reinterpret_cast<float (*)[2 * kMaxHalfDim]>(&red[0][0][0]));
      return;
    }
  }
  const int width = p.G * p.r;                 // columns of one matrix
  const int tid = threadIdx.x;
  const int cc = tid % kChunks, rg = tid / kChunks;    // 8-column chunk, row group
  const int cb0 = blockIdx.x * kCols;
  const int col0 = cb0 + 8 * cc;               // in [0, 2*width)
  const int slice = blockIdx.y, nslices = p.nslices;
  const int i0 = slice * kRows;
  const int rows = min(kRows, p.dm - i0);
  const bool active = col0 < 2 * width;
  const bool is_v = col0 >= width;
  const int c = is_v ? col0 - width : col0;
  const T* A = static_cast<const T*>(is_v ? p.a_v : p.a_k);
  const T* x = static_cast<const T*>(p.x);
  const size_t prow = 2 * static_cast<size_t>(width);   // floats per (slice, sequence)

  // all of this thread's A rows (rg + kRowGroups i) first, 16 bytes each,
  // with no branch around the loads: rows past the slice read its last row
  // and columns past the block read column 0 (finite values; the matching x
  // entries are 0 and the results for such columns are never stored)
  Raw8<T> a[kRowsPerThread];
  const int ca = active ? c : 0;
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int row = min(rg + kRowGroups * i, rows - 1);
    a[i].load(A + static_cast<size_t>(i0 + row) * width + ca);
  }
  // x entries of a sequence chunk (kXPer per thread), issued right after the
  // A loads so both are in flight together
  static_assert(kXPer * kThreads == kBatchChunk * kRows, "whole x entries per thread");
  float xv[kXPer];
  auto load_x = [&](int b0) {
#pragma unroll
    for (int u = 0; u < kXPer; ++u) {
      const int e = tid + u * kThreads, bb = e / kRows, i = e % kRows;
      const int bc = min(b0 + bb, p.B - 1), ic = min(i, rows - 1);
      xv[u] = load_f32(x, static_cast<size_t>(bc) * p.dm + i0 + ic);
    }
  };
  load_x(0);
  __shared__ float xs[kBatchChunk][kRows];
  __shared__ int is_last;
  const int fb = tid / (2 * kChunks), fq = tid % (2 * kChunks);   // reader: sequence, slot
  const int fcol = cb0 + Tl::col_of_slot(fq);
  for (int b0 = 0; b0 < p.B; b0 += kBatchChunk) {
    const int nb = min(kBatchChunk, p.B - b0);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kXPer; ++u) {
      const int e = tid + u * kThreads, bb = e / kRows, i = e % kRows;
      xs[bb][i] = bb < nb && i < rows ? xv[u] : 0.f;
    }
    __syncthreads();
    if (b0 + kBatchChunk < p.B) load_x(b0 + kBatchChunk);
#pragma unroll
    for (int bb = 0; bb < kBatchChunk; ++bb) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
      for (int i = 0; i < kRowsPerThread; ++i) {
        const float xr = xs[bb][rg + kRowGroups * i];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(xr, a[i][e], acc[e]);
      }
      red[rg][bb][cc] = float4{acc[0], acc[1], acc[2], acc[3]};
      red[rg][bb][cc + kChunks] = float4{acc[4], acc[5], acc[6], acc[7]};
    }
    __syncthreads();
    // row groups added in order; one 16-byte partial per reading thread
    if (fb < nb) {
      float4 s = red[0][fb][fq];
#pragma unroll
      for (int k = 1; k < kRowGroups; ++k) {
        const float4 v = red[k][fb][fq];
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
      }
      if (fcol < 2 * width) {
        float* dst = p.part + (static_cast<size_t>(slice) * p.B + b0 + fb) * prow + fcol;
        store_coherent2(dst, s.x, s.y);
        store_coherent2(dst + 2, s.z, s.w);
      }
    }
  }

  // arrival: the barrier orders every wave's partial stores before the
  // counter increment, which releases them at agent scope; the last arriver
  // acquires them.
  __syncthreads();
  if (tid == 0)
    is_last = __hip_atomic_fetch_add(&p.counters[blockIdx.x], 1, __ATOMIC_ACQ_REL,
                                     __HIP_MEMORY_SCOPE_AGENT) == nslices - 1;
  __syncthreads();
  if (!is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // the finished rows of kReaders sequences at a time (quantised caches:
  // staged in LDS, then quantised one wave per (sequence, row segment))
  __shared__ float4 rowbuf[kQuant ? kReaders : 1][2 * kChunks];
  const int j0 = cb0 / p.r;                                   // first row segment
  const int nseg = kQuant ? (min(cb0 + kCols, 2 * width) - cb0) / p.r : 0;   // r divides 256
  const size_t sstride = static_cast<size_t>(p.B) * prow;
  for (int bq = 0; bq < p.B; bq += kReaders) {
    const int b = bq + fb;
    const int pos = b < p.B ? p.pos[b] : -1;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    if (b < p.B && fcol < 2 * width && pos >= 0 && pos < p.L) {
      const float* src = p.part + static_cast<size_t>(b) * prow + fcol;
      // up to 32 slices (d_model 4096) in flight at once, then added in order
      for (int s0 = 0; s0 < nslices; s0 += 32) {
        float4 v[32];
#pragma unroll
        for (int u = 0; u < 32; ++u)
          v[u] = *reinterpret_cast<const float4*>(src + min(s0 + u, nslices - 1) * sstride);
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          if (s0 + u < nslices) {
            acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w;
          }
        }
      }
      if constexpr (!kQuant) {
        const float r4[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = fcol + e;
          const bool v = col >= width;
          const int cl = v ? col - width : col;
          const int g = cl / p.r, k = cl % p.r;
          T* h = static_cast<T*>(v ? p.h_v : p.h_k);
          store_elem(h, ((static_cast<size_t>(b) * p.G + g) * p.L + pos) * p.r + k, r4[e]);
        }
      }
    }
    if constexpr (kQuant) {
      rowbuf[fb][(fcol - cb0) / 4] = acc;
      __syncthreads();
      const int wave = tid / 64, lane = tid % 64;
      for (int task = wave; task < kReaders * nseg; task += kThreads / 64) {
        const int bb = task / nseg, sg = task % nseg, bs = bq + bb;
        if (bs >= p.B) continue;
        const int ps = p.pos[bs];
        if (ps < 0 || ps >= p.L) continue;
        const float4 v0 = lane < p.r / 4 ? rowbuf[bb][(sg * p.r) / 4 + lane] : float4{0.f, 0.f, 0.f, 0.f};
        quantize_row(p, v0, j0 + sg, bs, ps, lane);
      }
      __syncthreads();
    }
  }
  if (tid == 0) __hip_atomic_store(&p.counters[blockIdx.x], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

size_t align_counters(size_t n) {
  return (n * sizeof(int32_t) + kCounterAlign - 1) / kCounterAlign * kCounterAlign;
}
// counter area: one per column block (of the narrower form)
size_t counter_bytes(int G, int r) {
  return align_counters((2 * static_cast<size_t>(G) * r + kMinCols - 1) / kMinCols);
}

}  // namespace

size_t append_workspace_bytes(int B, int dm, int G, int r) {
  const size_t nks = (dm + kRows - 1) / kRows;
  const size_t row = 2 * size_t(G) * r * sizeof(float);
  return counter_bytes(G, r) + nks * B * row;
}

void append_bind_workspace(AppendParams& p, void* workspace) {
  p.nslices = (p.dm + kRows - 1) / kRows;
  char* w = static_cast<char*>(workspace);
  p.counters = reinterpret_cast<int32_t*>(w);
  p.part = reinterpret_cast<float*>(w + counter_bytes(p.G, p.r));
}

hipError_t launch_append(const AppendParams& p, int dtype, hipStream_t st) {
  const int cols = 2 * p.G * p.r;
  const bool fuse = p.ab.units > 0;
  if (p.quant) {
    using Tl = Tiling<true>;
    const int bx = (cols + Tl::kCols - 1) / Tl::kCols;
    const dim3 grid(bx, p.nslices + (fuse ? (p.ab.units + bx - 1) / bx : 0));
    if (dtype == 0) {
      if (fuse) append_kernel<float, true, true><<<grid, Tl::kThreads, 0, st>>>(p);
      else append_kernel<float, true, false><<<grid, Tl::kThreads, 0, st>>>(p);
    } else {
      if (fuse) append_kernel<uint16_t, true, true><<<grid, Tl::kThreads, 0, st>>>(p);
      else append_kernel<uint16_t, true, false><<<grid, Tl::kThreads, 0, st>>>(p);
    }
  } else {
    using Tl = Tiling<false>;
    const int bx = (cols + Tl::kCols - 1) / Tl::kCols;
    const dim3 grid(bx, p.nslices + (fuse ? (p.ab.units + bx - 1) / bx : 0));
    if (dtype == 0) {
      if (fuse) append_kernel<float, false, true><<<grid, Tl::kThreads, 0, st>>>(p);
      else append_kernel<float, false, false><<<grid, Tl::kThreads, 0, st>>>(p);
    } else {
      if (fuse) append_kernel<uint16_t, false, true><<<grid, Tl::kThreads, 0, st>>>(p);
      else append_kernel<uint16_t, false, false><<<grid, Tl::kThreads, 0, st>>>(p);
    }
  }
  return hipGetLastError();
}

int append_threads(int quant) { return quant ? Tiling<true>::kThreads : Tiling<false>::kThreads; }

bool append_can_carry(const AppendParams& p, long units, long max_grid_y) {
  const int kc = p.quant ? Tiling<true>::kCols : Tiling<false>::kCols;
  const long bx = (2L * p.G * p.r + kc - 1) / kc;
  return units > 0 && units <= 0x7fffffffL && p.nslices + (units + bx - 1) / bx <= max_grid_y;
}

}  // namespace palu
