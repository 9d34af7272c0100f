// Internal interface between the host API (api.cpp) and the HIP kernels.
// Not installed; callers use include/palu.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace palu {

constexpr int kMaxHalfDim = 128;   // head_dim <= 256

// Everything a decode launch needs, passed by value as the kernel argument.
struct DecodeParams {
  const void* q;        // [B, Hq, d]
  const void* h_k;      // [B, G, L, r]
  const void* h_v;      // [B, G, L, r]
  const void* b_k;      // [G, r, Dg]
  const void* b_v;      // [G, r, Dg]
  const int32_t* lens;  // [B] or nullptr (all L)
  float* out;           // [B, Hq, d]
  float* qt;            // [B, Hq, r]     absorbed queries, pre-scaled to log2 units
  float* part_ml;       // [B, Hq, n_split, 2]   running max (log2 units) and sum
  float* part_u;        // [B, Hq, n_split, r]   unnormalised value-latent sums
  void* bkt;            // [G, Dg, r]  B_k transposed (reconstruct MFMA kernel)
  int32_t B, Hq, Hkv, d, G, r, L;
  int32_t s, gqa, nq, Dg;      // heads per group, q heads per kv head, q heads per group
  int32_t n_split, split_tokens;
  int32_t rope;                // 1 if rotary embedding is applied
  int32_t full_rank;           // 1: h_k, h_v are full K, V; no B_k, B_v
  int32_t latent_out;          // 1: out [B, Hq, r] holds u* (B_v left to the caller)
  int32_t qbits;               // 8 or 4: h_k, h_v hold int8 / int4 codes with row
                               // scales s_k, s_v (tiled order); 0: dtype latents
  int32_t hadamard;            // 1: the quantised rows are Hadamard-rotated
  const float* s_k;            // [B, G, L] (int8 latents)
  const float* s_v;
  float scale_log2;            // softmax scale * log2(e)
  // omega_i / (2 pi) in fp64 for i < d/2: the pair turns by t * omega_rev[i]
  // revolutions at position t
  double omega_rev[kMaxHalfDim];
};

// The query absorption's operands (absorbed-key mode): q~[b, j*gqa + h, k] =
// scale_log2 * q[b, j*gqa + h] . B_k[g][k, jl*d .. jl*d + d) for KV head
// j = g*s + jl. Shared by its own launch and the append launch that can
// carry it as extra workgroups.
struct AbsorbArgs {
  const void* q;      // [B, Hq, d]
  const void* b_k;    // [G, r, Dg]
  float* qt;          // [B, Hq, r] fp32
  int32_t B, Hq, Hkv, s, gqa, d, Dg, r;
  float scale_log2;
  int32_t units;      // workgroups of the carried form: Hkv * B * slices of r (0: none)
};

struct AppendParams {
  const void* x;      // [B, dm]
  const void* a_k;    // [dm, G*r]
  const void* a_v;
  void* h_k;          // [B, G, L, r]
  void* h_v;
  const int32_t* pos; // [B]
  int32_t* counters;  // one arrival counter per column block; zero between calls
  float* part;        // [ceil(dm/128), B, 2*G*r] fp32 row-slice partial sums
  int32_t B, dm, G, r, L;
  // quantised caches (h_k, h_v codes): per-row scales
  int32_t quant;      // 0: dtype cache; 8 or 4: quantised cache of that width
  int32_t hadamard;   // 1: rows rotated by the Hadamard matrix before quantising
  float* s_k;         // [B, G, L]
  float* s_v;
  int32_t nslices;    // row slices of d_model (workgroup rows of the append proper)
  int32_t a_layout;   // 0: a [dm, G*r]; 1: a^T [G*r, dm] (one-pass kernel, no workspace)
  AbsorbArgs ab;      // absorption carried by the launch (ab.units > 0)
};

// Kernel variants of the context-split decode step.
enum class SplitKernel {
  kGeneric = 0,        // VALU, any dtype/shape in range
  kAbsorbedMfma = 1,   // bf16, absorbed keys, r in {32, 64, 128, 256}
  kReconstructMfma = 2,  // bf16, rebuilt + rotated keys, d 128, <= 4 q heads per KV
                         // head, r in {32, ..., 512}: a KV head's columns split over waves
  kReconstructWave = 3,  // bf16, rebuilt + rotated keys, d 128, <= 4 q heads per KV
                         // head, r in {32, 64, 128}, KV heads per group a multiple
                         // of 4: one wave per KV head
  kReconstructWide = 4,  // the same at r 256 (B_k^T in all of a wave's AGPRs), KV
                         // heads per group a multiple of 4
  kReconstructQuarter = 5,  // the same at r 512: four waves per KV head, each with a
                            // quarter of its columns' B_k^T; KV heads per group even
};

const char* split_kernel_name(SplitKernel k);

// Launchers return hipSuccess or the launch error. dtype: 0 = f32, 1 = bf16.
hipError_t launch_absorb_q(const DecodeParams& p, int dtype, hipStream_t st);
// the absorption's operands of a call; units = 0 (set by the carrying launch)
__host__ __device__ inline AbsorbArgs absorb_args(const DecodeParams& p) {
  AbsorbArgs a{};
  a.q = p.q; a.b_k = p.b_k; a.qt = p.qt;
  a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.s = p.s; a.gqa = p.gqa; a.d = p.d; a.Dg = p.Dg;
  a.r = p.r;
  a.scale_log2 = p.scale_log2;
  a.units = 0;
  return a;
}
// whether the absorption has the one-load-per-thread form (d / 8 a power of
// two <= 32) that an append launch can carry
inline bool absorb_carriable(const AbsorbArgs& a) {
  const int ncc = a.d / 8;
  return a.d % 8 == 0 && ncc <= 32 && (ncc & (ncc - 1)) == 0;
}
// rows of r each thread of that form absorbs, and its workgroups (slices of
// r) per (KV head, sequence) at `threads` threads a workgroup
constexpr int kAbsRowsPer = 4;
inline int absorb_slices(const AbsorbArgs& a, int threads) {
  const int rows = threads / (a.d / 8) * kAbsRowsPer;
  return (a.r + rows - 1) / rows;
}
hipError_t launch_prescale_q(const DecodeParams& p, int dtype, hipStream_t st);   // q~ = q
hipError_t launch_split_generic(const DecodeParams& p, int dtype, int absorbed, hipStream_t st);
bool absorbed_mfma_supported(const DecodeParams& p, int dtype);
// int8 / int4 latents (tiled cache): bf16 q and B, r in {64, 128, 256}, L % 32 == 0
bool absorbed_quant_supported(const DecodeParams& p, int dtype);
hipError_t launch_split_absorbed_quant(const DecodeParams& p, hipStream_t st);
int absorbed_head_slices(int nq);   // workgroups per (split, b, g): 16 query heads each
// the bf16 absorbed kernel's workgroups per (split, b, g): 16 query heads, or
// 32 (two head blocks) each when a group has more than 16
int absorbed_mfma_slices(int nq);
hipError_t launch_split_absorbed_mfma(const DecodeParams& p, hipStream_t st);
bool reconstruct_mfma_supported(const DecodeParams& p, int dtype);
int reconstruct_heads_per_wg(int r, int s);   // KV heads per workgroup (0: not served)
int reconstruct_waves_per_wg(int r, int s);
hipError_t launch_transpose_bk(const DecodeParams& p, int dtype, hipStream_t st);
bool reconstruct_wave_supported(const DecodeParams& p, int dtype);
hipError_t launch_split_reconstruct_wave(const DecodeParams& p, hipStream_t st);
bool reconstruct_wide_supported(const DecodeParams& p, int dtype);   // four KV heads a workgroup
hipError_t launch_split_reconstruct_wide(const DecodeParams& p, hipStream_t st);
bool reconstruct_quarter_supported(const DecodeParams& p, int dtype);   // two KV heads a workgroup
hipError_t launch_split_reconstruct_quarter(const DecodeParams& p, hipStream_t st);
hipError_t launch_split_reconstruct_mfma(const DecodeParams& p, hipStream_t st);
hipError_t launch_merge(const DecodeParams& p, int dtype, hipStream_t st);
size_t append_workspace_bytes(int B, int dm, int G, int r);
// sets counters, part and nslices
void append_bind_workspace(AppendParams& p, void* workspace);
int append_threads(int quant);   // threads per append workgroup
// whether an append launch can take `units` absorb workgroups (grid rows
// within the device's bound max_grid_y)
bool append_can_carry(const AppendParams& p, long units, long max_grid_y);
hipError_t launch_append(const AppendParams& p, int dtype, hipStream_t st);
// the one-pass form for a^T [G*r, dm] (dtype caches): its append workgroups
// (the carried absorption's come after them) and threads per workgroup
long append_t_blocks(const AppendParams& p);
int append_t_threads();
hipError_t launch_append_t(const AppendParams& p, int dtype, hipStream_t st);

// The library's static device scratch (palu_decode_attn_noalloc): its size,
// and the device address of `device`'s copy (looked up once per device; the
// device must be current).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
hipError_t static_scratch(int device, void** ptr);

}  // namespace palu
