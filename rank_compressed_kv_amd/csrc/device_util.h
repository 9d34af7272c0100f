// Small device helpers shared by the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace palu {

// Storage element -> fp32. bf16 is held as raw 16-bit patterns: the value is
// the fp32 number whose upper half is those bits, so widening is exact.
__device__ __forceinline__ float load_f32(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_f32(const uint16_t* p, size_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16 bytes of a stream that is read once (latent tiles): a non-temporal load,
// which does not keep the lines in the caches. On MI355X this raised the rate
// of the latent stream from about 5.5 to 6.2 TB/s.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return uint4{v[0], v[1], v[2], v[3]};
}

// Eight consecutive elements kept as raw bits: loaded with no branch around
// them (callers clamp the address instead of skipping the load), so that many
// loads stay in flight together, and widened to fp32 only where they are used.
// (A load whose widening sits in the same conditional block as the load makes
// the compiler wait for it before the next one.)
template <typename T>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float operator[](int e) const {
    const uint32_t x = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
    return (e & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
  }
};
template <>
struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ float operator[](int e) const {
    const float4& h = e < 4 ? a : b;
    const int k = e & 3;
    return k == 0 ? h.x : k == 1 ? h.y : k == 2 ? h.z : h.w;
  }
};

// Eight consecutive elements widened to fp32 (16-byte aligned addresses).
__device__ __forceinline__ void load8_f32(const uint16_t* p, float* v) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void load8_f32(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// fp32 -> bf16, nearest with ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ void store_elem(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16_rne(v); }

// cos and sin of the rotary angle at integer position t for a pair whose
// frequency is omega_rev revolutions per position. The product and the
// removal of whole turns are done in fp64 (exact enough for t up to 2^31), so
// the fp32 sincos only sees an angle in [-pi, pi].
__device__ __forceinline__ void rope_cos_sin(double omega_rev, int t, float& c, float& s) {
  double rev = static_cast<double>(t) * omega_rev;
  rev -= rint(rev);
  const float ang = static_cast<float>(rev * 6.283185307179586476925);
  sincosf(ang, &s, &c);
}

__device__ __forceinline__ int clamp_len(const int32_t* lens, int b, int L) {
  if (!lens) return L;
  const int n = lens[b];
  return n < 0 ? 0 : (n > L ? L : n);
}

// Which (context split, batch, group, head slice) a workgroup of a
// context-split kernel owns. Units u = split + n_split*(g + G*b) are dealt to
// the 8 XCDs (workgroups go to the XCDs round-robin in linear id order) with
// a rotation: XCD c's workgroup in block a of eight units takes unit 8a + ((c
// - a) mod 8). Without it XCD c would always get the splits u = c (mod 8),
// i.e. the same split indices of every sequence whenever n_split is a
// multiple of 8 (or divides 8); with ragged lengths the late splits are empty
// for short sequences and whole XCDs would sit idle. With one head slice,
// blockIdx is (x, y, z) over (n_split, G, B) and the rotation covers the whole
// blocks only (a partial last block keeps its order). With several, the
// launch is one-dimensional: the units are padded to a multiple of 8 and the
// nslice workgroups of a unit get linear ids 8 apart, which puts them on the
// same XCD at about the same time, so the latent tiles they all read are
// shared through that XCD's L2.
struct SplitUnit {
  int split, g, b, hs;
  bool live;
};
__device__ __forceinline__ SplitUnit split_unit(int n_split, int G, int B, int nslice) {
  SplitUnit u{};
  const int units = n_split * G * B;
  int unit;
  if (nslice == 1) {
    const int k = blockIdx.x + n_split * (blockIdx.y + G * blockIdx.z);
    const int a = k >> 3;
    unit = 8 * a + 8 <= units ? 8 * a + ((k - a) & 7) : k;
    u.hs = 0;
  } else {
    const int id = blockIdx.x;
    const int lo = id & 7, hi = id >> 3;
    u.hs = hi % nslice;
    const int a = hi / nslice;
    unit = 8 * a + ((lo - a) & 7);
  }
  u.live = unit < units;
  u.split = unit % n_split;
  const int rest = unit / n_split;
  u.g = rest % G;
  u.b = rest / G;
  return u;
}
// number of one-dimensional workgroup ids for nslice > 1 (0 if too many)
inline long split_unit_ids(int n_split, int G, int B, int nslice) {
  const long units = static_cast<long>(n_split) * G * B;
  const long ids = (units + 7) / 8 * 8 * nslice;
  return ids > 0x7fffffffL ? 0 : ids;
}

// a 16-byte piece of a latent tile: ordinary (L2-cached) when several
// workgroups read the same tile, non-temporal otherwise
template <bool kShared>
__device__ __forceinline__ uint4 load_tile16(const void* ptr) {
  if constexpr (kShared) return *static_cast<const uint4*>(ptr);
  else return load_stream16(ptr);
}

// Workgroup barrier that orders LDS accesses only: global loads issued before
// it stay in flight (__syncthreads also orders global memory, which makes
// every wave wait for all of its outstanding loads first).
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace palu
