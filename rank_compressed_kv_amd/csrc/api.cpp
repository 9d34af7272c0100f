// Host side of libpalu: descriptor validation (before any HIP call), launch
// planning and dispatch onto the caller's stream. See include/palu.h.
// the library is built with hidden visibility; only the C ABI is exported
#pragma GCC visibility push(default)
#include "palu.h"
#pragma GCC visibility pop

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "palu_internal.h"

namespace palu {

size_t generic_split_smem(const DecodeParams& p, int absorbed);

namespace {

thread_local std::string g_error;

palu_status fail(palu_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
palu_status fail(palu_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

palu_status ok() {
  g_error.clear();
  return PALU_OK;
}

constexpr int kSplitQuantum = 64;    // split sizes are multiples of this many tokens
constexpr int kTargetWorkgroups = 1024;
constexpr int kAbsorbedWorkgroups = 256;   // one per CU on a 256-CU MI355X
constexpr int kTargetWaves = 2048;         // reconstruct kernel: eight per CU
constexpr int kWaveKernelWaves = 1024;     // one-wave-per-head kernel: four per CU

palu_status validate_attn(const palu_attn_desc* d) {
  if (!d) return fail(PALU_ERR_NULL, "descriptor is NULL");
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 ||
      d->n_groups < 1 || d->rank < 1 || d->max_ctx < 1)
    return fail(PALU_ERR_SHAPE, "all sizes must be positive");
  if (d->n_q_heads % d->n_kv_heads)
    return fail(PALU_ERR_SHAPE, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                d->n_q_heads, d->n_kv_heads);
  if (d->n_kv_heads % d->n_groups)
    return fail(PALU_ERR_SHAPE, "n_kv_heads (%d) is not a multiple of n_groups (%d)",
                d->n_kv_heads, d->n_groups);
  if (d->head_dim % 2 || d->head_dim > 2 * kMaxHalfDim)
    return fail(PALU_ERR_SHAPE, "head_dim (%d) must be even and at most %d", d->head_dim,
                2 * kMaxHalfDim);
  if (d->rank > 512) return fail(PALU_ERR_SHAPE, "rank (%d) must be at most 512", d->rank);
  if (d->split_tokens < 0 || d->split_tokens % kSplitQuantum)
    return fail(PALU_ERR_SHAPE, "split_tokens (%d) must be 0 or a positive multiple of %d",
                d->split_tokens, kSplitQuantum);
  if (d->dtype != PALU_F32 && d->dtype != PALU_BF16)
    return fail(PALU_ERR_UNSUPPORTED, "unknown dtype %d", d->dtype);
  if (d->mode != PALU_MODE_RECONSTRUCT && d->mode != PALU_MODE_ABSORBED &&
      d->mode != PALU_MODE_FULL_RANK)
    return fail(PALU_ERR_UNSUPPORTED, "unknown mode %d", d->mode);
  if (!(d->rope_theta >= 0.0) || std::isinf(d->rope_theta))
    return fail(PALU_ERR_UNSUPPORTED, "rope_theta must be finite and >= 0");
  if (d->prepared != 0 && d->prepared != 1)
    return fail(PALU_ERR_UNSUPPORTED, "prepared must be 0 or 1 (got %d)", d->prepared);
  if (d->mode == PALU_MODE_ABSORBED && d->rope_theta != 0.0)
    return fail(PALU_ERR_UNSUPPORTED,
                "ABSORBED mode needs rope_theta == 0: a rotated key cannot absorb B_k into q");
  if (d->mode == PALU_MODE_FULL_RANK) {
    if (d->rope_theta != 0.0)
      return fail(PALU_ERR_UNSUPPORTED, "FULL_RANK mode needs rope_theta == 0 (keys cached rotated)");
    if (d->n_groups != d->n_kv_heads || d->rank != d->head_dim)
      return fail(PALU_ERR_SHAPE, "FULL_RANK mode needs n_groups == n_kv_heads and rank == head_dim");
  }
  const double rows = double(d->batch) * d->n_groups * d->max_ctx;
  if (rows * d->rank > 9.0e15) return fail(PALU_ERR_SHAPE, "cache too large");
  return PALU_OK;
}

struct Plan {
  int n_split;
  int split_tokens;
  SplitKernel kernel;
};

// Shape fields of DecodeParams that kernel selection looks at.
DecodeParams shape_params(const palu_attn_desc* d) {
  DecodeParams p{};
  p.B = d->batch; p.Hq = d->n_q_heads; p.Hkv = d->n_kv_heads; p.d = d->head_dim;
  p.G = d->n_groups; p.r = d->rank; p.L = d->max_ctx;
  p.s = p.Hkv / p.G; p.gqa = p.Hq / p.Hkv; p.nq = p.Hq / p.G; p.Dg = p.s * p.d;
  return p;
}

// qbits: the int8 / int4 cache calls, whose kernel takes 16 query heads a
// workgroup whatever the group size (the bf16 kernel takes 32 in groups of
// more than 16): their plan has as many workgroups per split as that kernel
// launches, and never more splits than the bf16 plan the workspace is sized for
Plan make_plan(const palu_attn_desc* d, int qbits = 0) {
  Plan pl{};
  const DecodeParams sp = shape_params(d);
  pl.kernel = SplitKernel::kGeneric;
  if (d->mode != PALU_MODE_RECONSTRUCT && absorbed_mfma_supported(sp, d->dtype))
    pl.kernel = SplitKernel::kAbsorbedMfma;
  if (d->mode == PALU_MODE_RECONSTRUCT && reconstruct_mfma_supported(sp, d->dtype))
    pl.kernel = SplitKernel::kReconstructMfma;
  if (d->mode == PALU_MODE_RECONSTRUCT && reconstruct_wave_supported(sp, d->dtype))
    pl.kernel = SplitKernel::kReconstructWave;
  if (d->mode == PALU_MODE_RECONSTRUCT && reconstruct_wide_supported(sp, d->dtype))
    pl.kernel = SplitKernel::kReconstructWide;
  if (d->mode == PALU_MODE_RECONSTRUCT && reconstruct_quarter_supported(sp, d->dtype))
    pl.kernel = SplitKernel::kReconstructQuarter;
  int st = d->split_tokens;
  if (st == 0) {
    // Aim at a fixed number of (split, b, g) units: 256 for the generic
    // kernel, which launches one workgroup per query head of each unit, and
    // one workgroup per CU (256 CUs, all resident at once) for the absorbed
    // MFMA kernel, whose register use allows one wave per SIMD.
    double wg_target = pl.kernel == SplitKernel::kGeneric ? double(kTargetWorkgroups) / 4.0
                                                          : double(kAbsorbedWorkgroups);
    // the reconstruct MFMA kernel launches one workgroup per slice of KV heads,
    // and aims at about 2048 waves on the chip whatever its workgroup size
    double slices = 1;
    if (pl.kernel == SplitKernel::kAbsorbedMfma)
      slices = qbits ? absorbed_head_slices(sp.nq) : absorbed_mfma_slices(sp.nq);
    if (pl.kernel == SplitKernel::kReconstructMfma) {
      slices = sp.s / reconstruct_heads_per_wg(sp.r, sp.s);
      wg_target = double(kTargetWaves) / reconstruct_waves_per_wg(sp.r, sp.s);
    }
    // one wave per KV head: aim at one wave per SIMD (1024 waves), i.e. one
    // four-wave workgroup per CU
    // (groups of one or two KV heads share a workgroup: s / 4 of one a group)
    if (pl.kernel == SplitKernel::kReconstructWave || pl.kernel == SplitKernel::kReconstructWide) {
      slices = sp.s / 4.0;
      wg_target = double(kWaveKernelWaves) / 4;
      // groups of one or two KV heads at rank 32 (and two at rank 64): two
      // workgroups fit a CU (registers and LDS), so aim at two rounds of
      // CUs (measured at the Llama-3-8B shape: one KV head a group, rank 32,
      // 101 -> 79 us; two, rank 64, 121 -> 87 us; four rounds were slower)
      if (sp.s < 4 && (sp.r == 32 || (sp.r == 64 && sp.s == 2))) wg_target *= 2;
    }
    // four waves per KV head (column quarters), eight-wave workgroups, one
    // per CU: aim at eight rounds of workgroups. A workgroup's split runs
    // for about 100 us at 1024 tokens, so with ragged lengths (short
    // sequences leave their late splits empty) a single round would end on a
    // long tail; eight rounds keep it to a few percent and cost about 7% when
    // every sequence is full length (more workgroup set-ups)
    if (pl.kernel == SplitKernel::kReconstructQuarter) {
      slices = sp.s / 2;
      wg_target = double(kWaveKernelWaves) * 2;
    }
    const double want = double(d->max_ctx) * d->batch * d->n_groups * slices / wg_target;
    st = int(std::ceil(want / kSplitQuantum)) * kSplitQuantum;
    if (st < kSplitQuantum) st = kSplitQuantum;
    if (st > 4096) st = 4096;
  }
  pl.split_tokens = st;
  pl.n_split = (d->max_ctx + st - 1) / st;
  return pl;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WorkspaceLayout {
  size_t qt, ml, u, bkt, total;
};

WorkspaceLayout layout(const palu_attn_desc* d, const Plan& pl) {
  WorkspaceLayout w{};
  const size_t heads = size_t(d->batch) * d->n_q_heads;
  const size_t elem = d->dtype == PALU_BF16 ? 2 : 4;
  w.qt = 0;
  const size_t qt_bytes = d->mode != PALU_MODE_RECONSTRUCT ? align256(heads * d->rank * 4) : 0;
  w.ml = w.qt + qt_bytes;
  w.u = w.ml + align256(heads * pl.n_split * 2 * 4);
  w.bkt = w.u + align256(heads * pl.n_split * size_t(d->rank) * 4);
  const bool bkt = pl.kernel == SplitKernel::kReconstructMfma ||
                   pl.kernel == SplitKernel::kReconstructWave ||
                   pl.kernel == SplitKernel::kReconstructWide ||
                   pl.kernel == SplitKernel::kReconstructQuarter;
  const size_t bkt_bytes =
      bkt ? align256(size_t(d->n_kv_heads) * d->head_dim * d->rank * elem) : 0;
  w.total = w.bkt + bkt_bytes;
  return w;
}

// Profiling records: a call claims the next start/stop pair with one atomic
// increment, so calls from several host threads never share a pair.
struct Profiler {
  std::vector<hipEvent_t> start, stop;
  std::atomic<int> used{0};
  bool armed = false;
} g_prof;

// The device's largest grid extent in y (launches that carry extra
// workgroup rows must stay within it); read once per device.
long max_grid_y() {
  static std::atomic<long> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 65535;
  if (dev < 64) {
    const long c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxGridDimY, dev) != hipSuccess || v <= 0)
    v = 65535;
  if (dev < 64) cached[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace

const char* split_kernel_name(SplitKernel k) {
  switch (k) {
    case SplitKernel::kGeneric: return "split_generic_kernel";
    case SplitKernel::kAbsorbedMfma: return "split_absorbed_mfma_kernel";
    case SplitKernel::kReconstructMfma: return "split_reconstruct_mfma_kernel";
    case SplitKernel::kReconstructWave: return "split_reconstruct_wave_kernel";
    case SplitKernel::kReconstructWide: return "split_reconstruct_wide_kernel";
    case SplitKernel::kReconstructQuarter: return "split_reconstruct_quarter_kernel";
  }
  return "?";
}

}  // namespace palu

using namespace palu;

extern "C" {

const char* palu_status_string(int32_t s) {
  switch (s) {
    case PALU_OK: return "ok";
    case PALU_ERR_NULL: return "null pointer";
    case PALU_ERR_SHAPE: return "bad shape";
    case PALU_ERR_UNSUPPORTED: return "unsupported";
    case PALU_ERR_WORKSPACE: return "workspace too small";
    case PALU_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* palu_last_error(void) { return g_error.c_str(); }

palu_status palu_decode_attn_workspace(const palu_attn_desc* desc, size_t* bytes) {
  palu_status st = validate_attn(desc);
  if (st != PALU_OK) return st;
  if (!bytes) return fail(PALU_ERR_NULL, "bytes is NULL");
  *bytes = layout(desc, make_plan(desc)).total;
  return ok();
}

palu_status palu_decode_attn_plan(const palu_attn_desc* desc, int32_t* n_split,
                                  int32_t* split_tokens, const char** kernel) {
  palu_status st = validate_attn(desc);
  if (st != PALU_OK) return st;
  const Plan pl = make_plan(desc);
  if (n_split) *n_split = pl.n_split;
  if (split_tokens) *split_tokens = pl.split_tokens;
  if (kernel) *kernel = split_kernel_name(pl.kernel);
  return ok();
}

}  // extern "C"

namespace {

// the launch parameters every decode call (and its prepare step) shares:
// shapes, plan, workspace areas, scale, rotary frequencies
DecodeParams call_params(const palu_attn_desc* desc, const Plan& pl, const WorkspaceLayout& wl,
                         void* workspace) {
  const bool full = desc->mode == PALU_MODE_FULL_RANK;
  DecodeParams p = shape_params(desc);
  char* ws = static_cast<char*>(workspace);
  p.qt = reinterpret_cast<float*>(ws + wl.qt);
  p.part_ml = reinterpret_cast<float*>(ws + wl.ml);
  p.part_u = reinterpret_cast<float*>(ws + wl.u);
  p.bkt = ws + wl.bkt;
  p.n_split = pl.n_split; p.split_tokens = pl.split_tokens;
  const double scale = desc->scale > 0.f ? double(desc->scale) : 1.0 / std::sqrt(double(p.d));
  p.scale_log2 = float(scale * 1.4426950408889634);
  p.rope = desc->rope_theta > 0.0 ? 1 : 0;
  p.full_rank = full ? 1 : 0;
  p.latent_out = !full && desc->latent_out != 0 ? 1 : 0;
  p.hadamard = desc->hadamard;
  for (int i = 0; i < p.d / 2; ++i)
    p.omega_rev[i] = p.rope ? std::pow(desc->rope_theta, -2.0 * i / p.d) / (2.0 * M_PI) : 0.0;
  return p;
}

// the query-side operands of a call: q~ = q B_k^T (ABSORBED), q * scale
// (FULL_RANK), B_k^T (RECONSTRUCT on the MFMA kernel)
palu_status prepare_launch(const palu_attn_desc* desc, const DecodeParams& p, const Plan& pl,
                           hipStream_t s) {
  hipError_t e = hipSuccess;
  if (desc->mode == PALU_MODE_FULL_RANK) e = launch_prescale_q(p, desc->dtype, s);
  else if (desc->mode == PALU_MODE_ABSORBED) e = launch_absorb_q(p, desc->dtype, s);
  if (e != hipSuccess) return fail(PALU_ERR_DEVICE, "absorb_q launch: %s", hipGetErrorString(e));
  if (pl.kernel == SplitKernel::kReconstructMfma || pl.kernel == SplitKernel::kReconstructWave ||
      pl.kernel == SplitKernel::kReconstructWide || pl.kernel == SplitKernel::kReconstructQuarter)
    e = launch_transpose_bk(p, desc->dtype, s);
  if (e != hipSuccess) return fail(PALU_ERR_DEVICE, "transpose launch: %s", hipGetErrorString(e));
  return PALU_OK;
}

// the operand pointers a decode call needs for its mode
palu_status decode_pointers(const palu_attn_desc* desc, const void* q, const void* h_k,
                            const void* h_v, const void* b_k, const void* b_v, const float* out) {
  const bool full = desc->mode == PALU_MODE_FULL_RANK;
  const bool latent = !full && desc->latent_out != 0;
  if (!q || !h_k || !h_v || (!full && !b_k) || (!full && !latent && !b_v) || !out)
    return fail(PALU_ERR_NULL, "q, h_k, h_v, out, workspace and (as the mode needs) b_k, b_v "
                               "must be non-NULL");
  return PALU_OK;
}

// both decode entry points; s_k, s_v non-NULL selects int8 latents
palu_status decode(const palu_attn_desc* desc, const void* q, const void* h_k, const void* h_v,
                   const float* s_k, const float* s_v, int qbits, const void* b_k,
                   const void* b_v, const int32_t* seq_lens, float* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (decode_pointers(desc, q, h_k, h_v, b_k, b_v, out) != PALU_OK || !workspace)
    return fail(PALU_ERR_NULL, "q, h_k, h_v, out, workspace and (as the mode needs) b_k, b_v "
                               "must be non-NULL");
  const Plan pl = make_plan(desc, qbits);
  if (qbits && pl.kernel != SplitKernel::kAbsorbedMfma)
    return fail(PALU_ERR_UNSUPPORTED, "quantised latents need the absorbed MFMA kernel");
  const WorkspaceLayout wl = layout(desc, pl);
  if (workspace_bytes < wl.total)
    return fail(PALU_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, wl.total);

  DecodeParams p = call_params(desc, pl, wl, workspace);
  p.q = q; p.h_k = h_k; p.h_v = h_v; p.b_k = b_k; p.b_v = b_v;
  p.lens = seq_lens; p.out = out;
  p.qbits = qbits;
  p.s_k = s_k; p.s_v = s_v;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int absorbed = desc->mode != PALU_MODE_RECONSTRUCT;   // scores against q~
  hipError_t e = hipSuccess;
  if (!desc->prepared) {
    const palu_status ps = prepare_launch(desc, p, pl, s);
    if (ps != PALU_OK) return ps;
  }

  int rec = -1;
  if (g_prof.armed) {
    rec = g_prof.used.fetch_add(1, std::memory_order_relaxed);
    if (rec >= int(g_prof.start.size())) rec = -1;
  }
  if (rec >= 0) (void)hipEventRecord(g_prof.start[rec], s);
  switch (pl.kernel) {
    case SplitKernel::kAbsorbedMfma:
      e = p.qbits ? launch_split_absorbed_quant(p, s) : launch_split_absorbed_mfma(p, s);
      break;
    case SplitKernel::kReconstructMfma: e = launch_split_reconstruct_mfma(p, s); break;
    case SplitKernel::kReconstructWave: e = launch_split_reconstruct_wave(p, s); break;
    case SplitKernel::kReconstructWide: e = launch_split_reconstruct_wide(p, s); break;
    case SplitKernel::kReconstructQuarter: e = launch_split_reconstruct_quarter(p, s); break;
    default: e = launch_split_generic(p, desc->dtype, absorbed, s); break;
  }
  if (rec >= 0) (void)hipEventRecord(g_prof.stop[rec], s);
  if (e != hipSuccess) return fail(PALU_ERR_DEVICE, "split launch: %s", hipGetErrorString(e));

  e = launch_merge(p, desc->dtype, s);
  if (e != hipSuccess) return fail(PALU_ERR_DEVICE, "merge launch: %s", hipGetErrorString(e));
  return ok();
}

// both quantised decode entry points: bits 8 (int8) or 4 (int4)
palu_status decode_quant(const palu_attn_desc* desc, int bits, const void* q, const void* h_k,
                         const void* h_v, const float* s_k, const float* s_v, const void* b_k,
                         const void* b_v, const int32_t* seq_lens, float* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  palu_status st = validate_attn(desc);
  if (st != PALU_OK) return st;
  if (desc->mode != PALU_MODE_ABSORBED || desc->dtype != PALU_BF16 ||
      (desc->rank != 64 && desc->rank != 128 && desc->rank != 256))
    return fail(PALU_ERR_UNSUPPORTED,
                "int%d latents need mode ABSORBED, dtype BF16 and rank 64, 128 or 256 "
                "(got mode %d, dtype %d, rank %d)", bits, desc->mode, desc->dtype, desc->rank);
  if (desc->max_ctx % 32)
    return fail(PALU_ERR_SHAPE, "int%d cache needs max_ctx %% 32 == 0 (got %d)", bits,
                desc->max_ctx);
  if (desc->hadamard != 0 && desc->hadamard != 1)
    return fail(PALU_ERR_UNSUPPORTED, "hadamard must be 0 or 1 (got %d)", desc->hadamard);
  if (!absorbed_quant_supported(shape_params(desc), desc->dtype))
    return fail(PALU_ERR_UNSUPPORTED, "int%d latents: combination not provided", bits);
  if (!s_k || !s_v) return fail(PALU_ERR_NULL, "s_k and s_v must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(h_k) | reinterpret_cast<uintptr_t>(h_v) |
       reinterpret_cast<uintptr_t>(s_k) | reinterpret_cast<uintptr_t>(s_v)) % 16)
    return fail(PALU_ERR_SHAPE, "int%d caches and scales must be 16-byte aligned", bits);
  return decode(desc, q, h_k, h_v, s_k, s_v, bits, b_k, b_v, seq_lens, out, workspace,
                workspace_bytes, stream);
}

}  // namespace

extern "C" {

palu_status palu_decode_attn(const palu_attn_desc* desc, const void* q, const void* h_k,
                             const void* h_v, const void* b_k, const void* b_v,
                             const int32_t* seq_lens, float* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  palu_status st = validate_attn(desc);
  if (st != PALU_OK) return st;
  if (desc->hadamard)
    return fail(PALU_ERR_UNSUPPORTED, "hadamard applies to the int8 and int4 caches only");
  return decode(desc, q, h_k, h_v, nullptr, nullptr, 0, b_k, b_v, seq_lens, out, workspace,
                workspace_bytes, stream);
}

palu_status palu_decode_attn_noalloc(const palu_attn_desc* desc, const void* q, const void* h_k,
                                     const void* h_v, const void* b_k, const void* b_v,
                                     const int32_t* seq_lens, float* out, void* stream) {
  // every check on the host first, then the scratch's address (one lookup per
  // device), then the ordinary call on it
  palu_status st = validate_attn(desc);
  if (st != PALU_OK) return st;
  if (desc->hadamard)
    return fail(PALU_ERR_UNSUPPORTED, "hadamard applies to the int8 and int4 caches only");
  if (desc->prepared)
    return fail(PALU_ERR_UNSUPPORTED,
                "prepared = 1 needs a caller-owned workspace (use palu_decode_attn)");
  st = decode_pointers(desc, q, h_k, h_v, b_k, b_v, out);
  if (st != PALU_OK) return st;
  const size_t need = layout(desc, make_plan(desc)).total;
  if (need > kStaticScratchBytes)
    return fail(PALU_ERR_WORKSPACE,
                "this call needs %zu bytes of scratch; the library's static scratch holds %zu "
                "(use palu_decode_attn with a workspace)", need, kStaticScratchBytes);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess)
    return fail(PALU_ERR_DEVICE, "hipGetDevice failed");
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
      return fail(PALU_ERR_DEVICE, "hipStreamGetDevice failed");
    if (sdev != dev)
      return fail(PALU_ERR_UNSUPPORTED, "the stream belongs to device %d, the current device is "
                                        "%d", sdev, dev);
  }
  void* ws = nullptr;
  const hipError_t e = static_scratch(dev, &ws);
  if (e != hipSuccess)
    return fail(PALU_ERR_DEVICE, "static scratch lookup: %s", hipGetErrorString(e));
  return decode(desc, q, h_k, h_v, nullptr, nullptr, 0, b_k, b_v, seq_lens, out, ws,
                kStaticScratchBytes, stream);
}

palu_status palu_decode_attn_prepare(const palu_attn_desc* desc, const void* q, const void* b_k,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  palu_status st = validate_attn(desc);
  if (st != PALU_OK) return st;
  const bool full = desc->mode == PALU_MODE_FULL_RANK;
  if (!q || (!full && !b_k) || !workspace)
    return fail(PALU_ERR_NULL, "q, workspace and (except in FULL_RANK mode) b_k must be non-NULL");
  const Plan pl = make_plan(desc);
  const WorkspaceLayout wl = layout(desc, pl);
  if (workspace_bytes < wl.total)
    return fail(PALU_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, wl.total);
  DecodeParams p = call_params(desc, pl, wl, workspace);
  p.q = q; p.b_k = b_k;
  st = prepare_launch(desc, p, pl, static_cast<hipStream_t>(stream));
  return st == PALU_OK ? ok() : st;
}

palu_status palu_decode_attn_i8(const palu_attn_desc* desc, const void* q, const int8_t* h_k,
                                const int8_t* h_v, const float* s_k, const float* s_v,
                                const void* b_k, const void* b_v, const int32_t* seq_lens,
                                float* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return decode_quant(desc, 8, q, h_k, h_v, s_k, s_v, b_k, b_v, seq_lens, out, workspace,
                      workspace_bytes, stream);
}

palu_status palu_decode_attn_i4(const palu_attn_desc* desc, const void* q, const uint8_t* h_k,
                                const uint8_t* h_v, const float* s_k, const float* s_v,
                                const void* b_k, const void* b_v, const int32_t* seq_lens,
                                float* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return decode_quant(desc, 4, q, h_k, h_v, s_k, s_v, b_k, b_v, seq_lens, out, workspace,
                      workspace_bytes, stream);
}

}  // extern "C"

namespace {
hipError_t launch_append_any(const AppendParams& p, int dtype, hipStream_t st) {
  return p.a_layout == PALU_A_OUT_IN ? launch_append_t(p, dtype, st) : launch_append(p, dtype, st);
}

palu_status validate_append(const palu_append_desc* d) {
  if (!d) return fail(PALU_ERR_NULL, "descriptor is NULL");
  if (d->batch < 1 || d->d_model < 1 || d->n_groups < 1 || d->rank < 1 || d->max_ctx < 1)
    return fail(PALU_ERR_SHAPE, "all sizes must be positive");
  if (d->d_model > 65536 || d->rank > 512)
    return fail(PALU_ERR_SHAPE, "d_model must be <= 65536 and rank <= 512");
  if (double(d->n_groups) * d->rank > 65536.0 || (d->n_groups * d->rank) % 8)
    return fail(PALU_ERR_SHAPE, "n_groups * rank must be a multiple of 8 and <= 65536");
  if (d->dtype != PALU_F32 && d->dtype != PALU_BF16)
    return fail(PALU_ERR_UNSUPPORTED, "unknown dtype %d", d->dtype);
  if (d->a_layout != PALU_A_IN_OUT && d->a_layout != PALU_A_OUT_IN)
    return fail(PALU_ERR_UNSUPPORTED, "unknown a_layout %d", d->a_layout);
  if (d->a_layout == PALU_A_OUT_IN && d->d_model % 8)
    return fail(PALU_ERR_SHAPE, "a_layout PALU_A_OUT_IN needs d_model %% 8 == 0 (got %d)",
                d->d_model);
  return PALU_OK;
}

// workspace bytes of a validated descriptor's append
size_t append_need(const palu_append_desc* d) {
  if (d->a_layout == PALU_A_OUT_IN) return 0;
  return append_workspace_bytes(d->batch, d->d_model, d->n_groups, d->rank);
}

palu_status validate_append_quant(const palu_append_desc* d, int bits) {
  palu_status st = validate_append(d);
  if (st != PALU_OK) return st;
  if (d->a_layout != PALU_A_IN_OUT)
    return fail(PALU_ERR_UNSUPPORTED, "the int%d cache write takes a_layout PALU_A_IN_OUT only",
                bits);
  if (d->rank != 64 && d->rank != 128 && d->rank != 256)
    return fail(PALU_ERR_UNSUPPORTED, "int%d cache needs rank 64, 128 or 256 (got %d)", bits,
                d->rank);
  if (d->max_ctx % 32)
    return fail(PALU_ERR_SHAPE, "int%d cache needs max_ctx %% 32 == 0 (got %d)", bits,
                d->max_ctx);
  if (d->hadamard != 0 && d->hadamard != 1)
    return fail(PALU_ERR_UNSUPPORTED, "hadamard must be 0 or 1 (got %d)", d->hadamard);
  return PALU_OK;
}

// the checks of the append entry point qbits selects (0: dtype cache, 8 / 4:
// int8 / int4 cache with scales)
palu_status validate_append_call(const palu_append_desc* d, int qbits, const float* s_k,
                                 const float* s_v) {
  if (qbits != 0 && qbits != 8 && qbits != 4)
    return fail(PALU_ERR_UNSUPPORTED, "qbits must be 0, 8 or 4 (got %d)", qbits);
  palu_status st = qbits ? validate_append_quant(d, qbits) : validate_append(d);
  if (st != PALU_OK) return st;
  if (!qbits && d->hadamard)
    return fail(PALU_ERR_UNSUPPORTED, "hadamard applies to the int8 and int4 caches only");
  if (qbits && (!s_k || !s_v)) return fail(PALU_ERR_NULL, "s_k and s_v must be non-NULL");
  return PALU_OK;
}

// the launch parameters of an append (pointers and workspace checked)
palu_status append_params(const palu_append_desc* d, int qbits, const void* x, const void* a_k,
                          const void* a_v, void* h_k, void* h_v, float* s_k, float* s_v,
                          const int32_t* pos, void* workspace, size_t workspace_bytes,
                          AppendParams& p) {
  const bool quant = qbits != 0;
  const size_t need = append_need(d);
  if (!x || !a_k || !a_v || !h_k || !h_v || !pos || (need && !workspace))
    return fail(PALU_ERR_NULL, "x, a_k, a_v, h_k, h_v, pos and workspace must be non-NULL");
  if (quant && (reinterpret_cast<uintptr_t>(h_k) % 4 || reinterpret_cast<uintptr_t>(h_v) % 4))
    return fail(PALU_ERR_SHAPE, "int%d caches must be 4-byte aligned", qbits);
  if (workspace_bytes < need)
    return fail(PALU_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  if (need && reinterpret_cast<uintptr_t>(workspace) % 16)
    return fail(PALU_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  p = AppendParams{};
  p.x = x; p.a_k = a_k; p.a_v = a_v; p.h_k = h_k; p.h_v = h_v; p.pos = pos;
  p.B = d->batch; p.dm = d->d_model; p.G = d->n_groups; p.r = d->rank; p.L = d->max_ctx;
  p.quant = qbits;
  p.hadamard = d->hadamard;
  p.s_k = s_k; p.s_v = s_v;
  p.a_layout = d->a_layout;
  if (need) append_bind_workspace(p, workspace);
  return PALU_OK;
}

// every append entry point (descriptor already validated)
palu_status append(const palu_append_desc* d, int qbits, const void* x, const void* a_k,
                   const void* a_v, void* h_k, void* h_v, float* s_k, float* s_v,
                   const int32_t* pos, void* workspace, size_t workspace_bytes, void* stream) {
  AppendParams p;
  const palu_status st = append_params(d, qbits, x, a_k, a_v, h_k, h_v, s_k, s_v, pos,
                                       workspace, workspace_bytes, p);
  if (st != PALU_OK) return st;
  hipError_t e = launch_append_any(p, d->dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PALU_ERR_DEVICE, "append launch: %s", hipGetErrorString(e));
  return ok();
}
}  // namespace

extern "C" {

palu_status palu_latent_append_workspace(const palu_append_desc* d, size_t* bytes) {
  palu_status st = validate_append(d);
  if (st != PALU_OK) return st;
  if (!bytes) return fail(PALU_ERR_NULL, "bytes is NULL");
  *bytes = append_need(d);
  return ok();
}

palu_status palu_latent_append(const palu_append_desc* d, const void* x, const void* a_k,
                               const void* a_v, void* h_k, void* h_v, const int32_t* pos,
                               void* workspace, size_t workspace_bytes, void* stream) {
  palu_status st = validate_append_call(d, 0, nullptr, nullptr);
  if (st != PALU_OK) return st;
  return append(d, 0, x, a_k, a_v, h_k, h_v, nullptr, nullptr, pos, workspace, workspace_bytes,
                stream);
}

palu_status palu_latent_append_i8_workspace(const palu_append_desc* d, size_t* bytes) {
  palu_status st = validate_append_quant(d, 8);
  if (st != PALU_OK) return st;
  if (!bytes) return fail(PALU_ERR_NULL, "bytes is NULL");
  *bytes = append_workspace_bytes(d->batch, d->d_model, d->n_groups, d->rank);
  return ok();
}

palu_status palu_latent_append_i8(const palu_append_desc* d, const void* x, const void* a_k,
                                  const void* a_v, int8_t* h_k, int8_t* h_v, float* s_k,
                                  float* s_v, const int32_t* pos, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  palu_status st = validate_append_call(d, 8, s_k, s_v);
  if (st != PALU_OK) return st;
  return append(d, 8, x, a_k, a_v, h_k, h_v, s_k, s_v, pos, workspace, workspace_bytes, stream);
}

palu_status palu_latent_append_i4_workspace(const palu_append_desc* d, size_t* bytes) {
  palu_status st = validate_append_quant(d, 4);
  if (st != PALU_OK) return st;
  if (!bytes) return fail(PALU_ERR_NULL, "bytes is NULL");
  *bytes = append_workspace_bytes(d->batch, d->d_model, d->n_groups, d->rank);
  return ok();
}

palu_status palu_latent_append_i4(const palu_append_desc* d, const void* x, const void* a_k,
                                  const void* a_v, uint8_t* h_k, uint8_t* h_v, float* s_k,
                                  float* s_v, const int32_t* pos, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  palu_status st = validate_append_call(d, 4, s_k, s_v);
  if (st != PALU_OK) return st;
  return append(d, 4, x, a_k, a_v, h_k, h_v, s_k, s_v, pos, workspace, workspace_bytes, stream);
}

palu_status palu_latent_append_prepare(const palu_append_desc* ad, int32_t qbits, const void* x,
                                       const void* a_k, const void* a_v, void* h_k, void* h_v,
                                       float* s_k, float* s_v, const int32_t* pos,
                                       void* append_ws, size_t append_ws_bytes,
                                       const palu_attn_desc* attn, const void* q,
                                       const void* b_k, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  // every check of both calls before anything is launched
  palu_status st = validate_append_call(ad, qbits, s_k, s_v);
  if (st != PALU_OK) return st;
  AppendParams ap;
  st = append_params(ad, qbits, x, a_k, a_v, h_k, h_v, s_k, s_v, pos, append_ws,
                     append_ws_bytes, ap);
  if (st != PALU_OK) return st;
  st = validate_attn(attn);
  if (st != PALU_OK) return st;
  const bool full = attn->mode == PALU_MODE_FULL_RANK;
  if (!q || (!full && !b_k) || !workspace)
    return fail(PALU_ERR_NULL, "q, workspace and (except in FULL_RANK mode) b_k must be non-NULL");
  const Plan pl = make_plan(attn);
  const WorkspaceLayout wl = layout(attn, pl);
  if (workspace_bytes < wl.total)
    return fail(PALU_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, wl.total);
  DecodeParams dp = call_params(attn, pl, wl, workspace);
  dp.q = q; dp.b_k = b_k;

  // the two workspaces must not share a byte: in the carried launch the
  // absorb workgroups write q~ while the append's write partials and arrival
  // counters, and a counter left nonzero would make later appends skip rows
  {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(append_ws), a1 = a0 + append_ws_bytes;
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(workspace), w1 = w0 + workspace_bytes;
    if (a0 < w1 && w0 < a1)
      return fail(PALU_ERR_WORKSPACE, "the append workspace and the decode workspace overlap");
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  // the absorption rides in the append's launch when it can: one extra
  // workgroup per (KV head, sequence, slice of r rows)
  AbsorbArgs ab = absorb_args(dp);
  const bool cols = ap.a_layout == PALU_A_OUT_IN;
  long units = 0;
  if (absorb_carriable(ab))
    units = long(ab.Hkv) * ab.B *
            absorb_slices(ab, cols ? append_t_threads() : append_threads(qbits));
  const bool fits = cols ? units > 0 && append_t_blocks(ap) + units <= 0x7fffffffL
                         : append_can_carry(ap, units, max_grid_y());
  const bool carry = attn->mode == PALU_MODE_ABSORBED && attn->dtype == ad->dtype &&
                     absorb_carriable(ab) && fits;
  if (carry) {
    ab.units = int32_t(units);
    ap.ab = ab;
  }
  const hipError_t e = launch_append_any(ap, ad->dtype, s);
  if (e != hipSuccess) return fail(PALU_ERR_DEVICE, "append launch: %s", hipGetErrorString(e));
  if (!carry) {
    st = prepare_launch(attn, dp, pl, s);
    if (st != PALU_OK) return st;
  }
  return ok();
}

palu_status palu_profile_begin(int32_t max_records) {
  if (max_records < 1 || max_records > 100000)
    return fail(PALU_ERR_SHAPE, "max_records must be in 1..100000");
  if (g_prof.armed) return fail(PALU_ERR_UNSUPPORTED, "profiling already armed");
  g_prof.start.assign(max_records, nullptr);
  g_prof.stop.assign(max_records, nullptr);
  for (int i = 0; i < max_records; ++i) {
    // timing-only events: no system-scope fence (no cache write-back and
    // invalidation around the timed kernel)
    if (hipEventCreateWithFlags(&g_prof.start[i], hipEventDisableSystemFence) != hipSuccess ||
        hipEventCreateWithFlags(&g_prof.stop[i], hipEventDisableSystemFence) != hipSuccess)
      return fail(PALU_ERR_DEVICE, "hipEventCreate failed");
  }
  g_prof.used.store(0);
  g_prof.armed = true;
  return ok();
}

palu_status palu_profile_end(double* total_ms, int32_t* count) {
  if (!g_prof.armed) return fail(PALU_ERR_UNSUPPORTED, "profiling not armed");
  double sum = 0.0;
  palu_status st = PALU_OK;
  const int used = std::min(g_prof.used.load(), int(g_prof.start.size()));
  for (int i = 0; i < used; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_prof.stop[i]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_prof.start[i], g_prof.stop[i]) != hipSuccess) {
      st = fail(PALU_ERR_DEVICE, "event timing failed");
      break;
    }
    sum += ms;
  }
  if (total_ms) *total_ms = sum;
  if (count) *count = used;
  for (size_t i = 0; i < g_prof.start.size(); ++i) {
    if (g_prof.start[i]) (void)hipEventDestroy(g_prof.start[i]);
    if (g_prof.stop[i]) (void)hipEventDestroy(g_prof.stop[i]);
  }
  g_prof.start.clear();
  g_prof.stop.clear();
  g_prof.used.store(0);
  g_prof.armed = false;
  return st == PALU_OK ? ok() : st;
}

}  // extern "C"
