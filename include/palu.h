/*
 * palu.h - C ABI of libpalu: single-token decode attention over a low-rank
 * (Palu-style) latent KV cache on AMD Instinct MI355X (gfx950).
 *
 * The method, as the Palu author responses on OpenReview (paperhub page
 * "LWMS4pk2vK") state it:
 *   - answer to Q2 (ESPACE): at inference a down-projection h = x A is cached
 *     and a reconstruction y = h B rebuilds the full vector;
 *   - "Why Palu Requires Fewer Global Memory Access": per head group i the cache
 *     holds H_i (L x r) in place of the key K_i (L x d_h); K_i = H_i B_i with
 *     B_i (r x d_h); only q_i, H_i and B are read from global memory, and the
 *     rebuilt keys stay on chip;
 *   - "Quantitive Analysis": heads are decomposed per group (G-LRD); one group
 *     over all heads is the joint form (J-LRD);
 *   - clarification of W1: values are never rebuilt; B_v is applied after the
 *     attention-weighted sum of value latents, and key reconstruction is needed
 *     only because of the rotary embedding.
 * Attention itself is softmax(q K^T / sqrt(d)) V (CurDKV author response,
 * paperhub page "klmc4fwPLd", motivation of value-guided compression). The
 * rotary embedding turns each pair of a key by the 2x2 rotation
 * [[cos, -sin], [sin, cos]] (CommVQ author response, paperhub page
 * "sbbyCB39HN", proof of Property 1); frequencies theta^(-2i/d) and the pairing
 * (i, i + d/2) are this library's reading, the pages being silent on both.
 *
 * Conventions shared by every call
 *   - All tensor pointers are device pointers, owned by the caller, row-major
 *     with the last index contiguous. The library never allocates, frees or
 *     synchronises in these calls; it enqueues kernels on `stream`
 *     (a hipStream_t; NULL is the null stream) and returns.
 *   - Validation is done on the host before any HIP call; on an error nothing
 *     is launched and palu_last_error() gives a one-line reason (thread-local).
 *   - The library keeps no state between calls except that text and the
 *     optional profiling records below; calls are re-entrant (calls made
 *     while profiling is armed claim distinct records), except
 *     palu_profile_begin and palu_profile_end, which must not run while
 *     other calls are in progress.
 *   - Conditions only the device can see (a length above max_ctx, an append
 *     position outside [0, max_ctx)) are not errors: lengths are clamped to
 *     [0, max_ctx] and out-of-range append rows are skipped.
 */
#ifndef PALU_H
#define PALU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum palu_status {
  PALU_OK = 0,
  PALU_ERR_NULL = 1,        /* a required pointer is NULL                           */
  PALU_ERR_SHAPE = 2,       /* sizes inconsistent or out of the supported range    */
  PALU_ERR_UNSUPPORTED = 3, /* dtype/mode/theta combination not provided           */
  PALU_ERR_WORKSPACE = 4,   /* workspace smaller than palu_decode_attn_workspace   */
  PALU_ERR_DEVICE = 5       /* a HIP call or kernel launch failed                   */
} palu_status;

typedef enum palu_dtype { PALU_F32 = 0, PALU_BF16 = 1 } palu_dtype;

typedef enum palu_mode {
  /* rebuild K = H_k B_k per tile on chip, rotate, score against q */
  PALU_MODE_RECONSTRUCT = 0,
  /* no rotary embedding: score q~ = q B_k^T against H_k directly */
  PALU_MODE_ABSORBED = 1,
  /* the uncompressed baseline every speedup of the method is measured
   * against ("Why Palu Requires Fewer Global Memory Access": the full K_i is
   * read): h_k, h_v hold the full keys and values, one "group" per KV head,
   * rank = head_dim, no B matrices (b_k, b_v are ignored and may be NULL);
   * keys are cached already rotated, so rope_theta must be 0 */
  PALU_MODE_FULL_RANK = 2
} palu_mode;

/* Shapes: B = batch, Hq = query heads, Hkv = KV heads, d = head dim,
 * G = head groups, s = Hkv / G heads per group, D_g = s * d, r = rank per
 * group, L_cap = max_ctx. KV head j belongs to group j / s and uses columns
 * (j % s) * d .. (j % s + 1) * d of its group's B; query head h reads KV head
 * h / (Hq / Hkv). */
typedef struct palu_attn_desc {
  int32_t batch;        /* B   >= 1                                             */
  int32_t n_q_heads;    /* Hq, a multiple of n_kv_heads                          */
  int32_t n_kv_heads;   /* Hkv, a multiple of n_groups                           */
  int32_t head_dim;     /* d, even, 2..256                                       */
  int32_t n_groups;     /* G >= 1                                                */
  int32_t rank;         /* r, 1..512                                             */
  int32_t max_ctx;      /* L_cap >= 1: rows per (b, g) and the cache's row stride */
  int32_t dtype;        /* palu_dtype of q, h_k, h_v, b_k, b_v; out is fp32       */
  int32_t mode;         /* palu_mode                                             */
  int32_t split_tokens; /* tokens per context split; 0 picks one; else a multiple of 64 */
  float scale;          /* softmax scale; <= 0 means 1/sqrt(d)                   */
  double rope_theta;    /* RoPE base; 0 means none; must be 0 in ABSORBED mode   */
  int32_t latent_out;   /* 0: out [B, Hq, d] = u* B_v[g][:, cols(j)];
                           1: out [B, Hq, r] = u*, the attention-weighted sum of
                           value latents, and b_v is not read (may be NULL): the
                           caller applies B_v, e.g. fused with its output
                           projection (Palu author response, clarification of W1:
                           B_v acts after the weighted sum). FULL_RANK ignores it. */
  int32_t hadamard;     /* palu_decode_attn_i8 / _i4 only (0 elsewhere): 1 if the
                           quantised cache holds Hadamard-rotated rows (see
                           palu_latent_append_i8) */
  int32_t prepared;     /* 0: the decode call forms its query-side operands itself;
                           1: palu_decode_attn_prepare has formed them in this
                           workspace (same descriptor otherwise, same q and b_k)
                           and the call only reads them */
} palu_attn_desc;

/* Bytes of device workspace palu_decode_attn needs for this descriptor
 * (split partials and, in ABSORBED mode, the absorbed queries). */
palu_status palu_decode_attn_workspace(const palu_attn_desc* desc, size_t* bytes);

/* Launch plan for this descriptor: number of context splits, tokens per split
 * and the name of the main kernel (a static string). Any output may be NULL.
 * The int8 / int4 decode calls take 16 query heads a workgroup; for groups of
 * more than 16 query heads they use fewer splits than reported here (never
 * more, so palu_decode_attn_workspace covers them). */
palu_status palu_decode_attn_plan(const palu_attn_desc* desc, int32_t* n_split,
                                  int32_t* split_tokens, const char** kernel);

/* out[b, h, :] = sum_t softmax_t(scale * <q[b,h], RoPE_t(K_j[t])>) * V_j[t]
 * with K_j = h_k[b, g] B_k[g][:, cols(j)], V_j = h_v[b, g] B_v[g][:, cols(j)],
 * t in [0, len[b]); V_j is never formed: the weighted sum runs over h_v rows and
 * B_v is applied once per head afterwards.
 *   q        [B, Hq, d]          dtype
 *   h_k, h_v [B, G, L_cap, r]    dtype; rows >= len[b] are never read
 *   b_k, b_v [G, r, D_g]         dtype
 *   seq_lens [B] int32 on the device, or NULL for len[b] = L_cap
 *   out      [B, Hq, d] fp32 ([B, Hq, r] with latent_out); a sequence of length
 *            0 gives zeros
 *   workspace, workspace_bytes: device scratch of at least the size reported by
 *            palu_decode_attn_workspace; its contents are overwritten.
 * FULL_RANK mode: out[b, h, :] = sum_t softmax_t(scale * <q[b,h], h_k[b,j,t]>)
 * h_v[b,j,t] with j = h / (Hq / Hkv); needs n_groups == n_kv_heads and
 * rank == head_dim; b_k and b_v are not read.
 * Errors: NULL for a missing pointer (only seq_lens may be NULL, and b_k, b_v
 * in FULL_RANK mode or with latent_out), SHAPE (also FULL_RANK with n_groups != n_kv_heads or
 * rank != head_dim), UNSUPPORTED (ABSORBED or FULL_RANK with rope_theta != 0,
 * unknown dtype/mode, rope_theta < 0), WORKSPACE, DEVICE (launch failure). */
palu_status palu_decode_attn(const palu_attn_desc* desc, const void* q, const void* h_k,
                             const void* h_v, const void* b_k, const void* b_v,
                             const int32_t* seq_lens, float* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* palu_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. The call works in a scratch array the
 * library owns on each GPU (32 MiB, a static device array: each GPU the library
 * runs on holds its copy until the process ends) and allocates nothing.
 *   desc, q, h_k, h_v, b_k, b_v, seq_lens, out, stream: as for palu_decode_attn,
 *   on the current device (the stream, if not NULL, must belong to it).
 * Every call on a GPU shares that GPU's scratch, which keeps the last call's
 * contents: calls that overlap in time on one GPU (several streams, several
 * host threads) race and must be ordered by the caller.
 * Errors: those of palu_decode_attn; WORKSPACE when the call needs more
 * scratch than 32 MiB (palu_decode_attn_workspace gives the figure);
 * UNSUPPORTED for desc->prepared = 1 (prepared operands live in a caller's
 * workspace), hadamard, or a stream of another device; DEVICE when the
 * scratch's address cannot be looked up. Nothing is launched on an error. */
palu_status palu_decode_attn_noalloc(const palu_attn_desc* desc, const void* q, const void* h_k,
                                     const void* h_v, const void* b_k, const void* b_v,
                                     const int32_t* seq_lens, float* out, void* stream);

/* The query-side operands of a decode call, formed ahead of it: the absorbed
 * queries q~ = q B_k[g][:, cols(j)]^T (ABSORBED; the clarification of W1: with
 * no rotary embedding B_k moves onto the query), the scaled queries
 * (FULL_RANK), or B_k transposed for the matrix-core reconstruct kernel
 * (RECONSTRUCT), written into the call's workspace. They depend on q and b_k
 * only, not on the cache, so a caller can run this on another stream while
 * palu_latent_append writes the step's token, then make the decode call with
 * desc->prepared = 1 on the same workspace (after that stream's work). In
 * RECONSTRUCT mode the prepared operand is B_k transposed alone: it depends on
 * b_k only and decode calls read it without writing it, so one prepare serves
 * every later prepared call with the same descriptor, b_k and workspace (B_k
 * is a weight: the transpose can be formed once, not per decode step).
 *   q [B, Hq, d], b_k [G, r, D_g] dtype (b_k may be NULL in FULL_RANK mode);
 *   workspace as for palu_decode_attn (this call writes its query area).
 * Errors: as palu_decode_attn's descriptor checks, NULL, WORKSPACE, DEVICE. */
palu_status palu_decode_attn_prepare(const palu_attn_desc* desc, const void* q, const void* b_k,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* The int8 latent cache (per-token quantisation of the latents combined with
 * the low-rank cache, Palu author response to reviewer Fsn9 on W1/W2; "Avg.
 * Bits" with a scale shared by a group of elements, answer to Q4):
 *   codes h_k, h_v: B*G slabs of L_cap*r bytes; s_k, s_v [B, G, L_cap] fp32.
 *   Latent k of token t of slab (b, g) is codes * scale, the code byte of
 *   (t, k) sitting at this offset inside its slab (L_cap % 32 == 0, r in
 *   {64, 128, 256}; the order of the decode kernel's matrix-core operands):
 *     keys:   32r*(t/32) + 16r*((t%32)/16) + 1024*(k/64) + 256*((k%32)/8)
 *             + 16*(t%16) + 8*((k/32)%2) + k%8
 *     values: 32r*(t/32) + 1024*(k/32) + 256*((t%16)/4) + 16*(k%16)
 *             + 8*((k/16)%2) + 4*((t%32)/16) + t%4
 *   Each 32-token block is a permutation of its own 32 r bytes.
 *   With hadamard = 1 a row holds the codes of h'' = h H_r (H_r Sylvester's
 *   Hadamard matrix of order r, entries +-1; the author responses list fusing
 *   a Hadamard transform among the quantisation-friendly enhancements, answer
 *   to Q2) and the latent row is h = (codes * scale) H_r / r.
 *
 * palu_decode_attn over such a cache: same result as palu_decode_attn on the
 * dequantised latents, up to rounding.
 *   h_k, h_v, s_k, s_v  as above, 16-byte aligned; rows >= len[b] may be read
 *            when they share a 32-token block with row len[b]-1, but never
 *            change the result (whatever their bytes hold)
 *   q, b_k, b_v, seq_lens, out, workspace as in palu_decode_attn (the
 *            workspace size is palu_decode_attn_workspace's for desc)
 *   desc->hadamard: 1 for a rotated cache (the kernel rotates q~ and the
 *            value sums back; B_k and B_v are the unrotated ones)
 * Provided for mode ABSORBED, dtype BF16 and rank 64, 128 or 256
 * (latent_out allowed); anything else is UNSUPPORTED. Errors as in
 * palu_decode_attn, NULL for a missing s_k or s_v, SHAPE for L_cap % 32 != 0
 * or a misaligned cache or scale pointer. */
palu_status palu_decode_attn_i8(const palu_attn_desc* desc, const void* q, const int8_t* h_k,
                                const int8_t* h_v, const float* s_k, const float* s_v,
                                const void* b_k, const void* b_v, const int32_t* seq_lens,
                                float* out, void* workspace, size_t workspace_bytes,
                                void* stream);

/* The int4 latent cache: the same per-token scheme at 4 bits (the author
 * responses fix no code width for quantised latents; 4 bits halves the int8
 * cache again), codes in [-7, 7] stored as the nibble code + 8.
 *   codes h_k, h_v: B*G slabs of L_cap*r/2 bytes; s_k, s_v [B, G, L_cap] fp32.
 *   Latent k of token t of slab (b, g) is code * scale; with
 *     keys:   u = (r/32)*((t%32)/16) + k/32, l = 16*((k%32)/8) + t%16,
 *             e = (k%8)/4 + 2*(k%2), n = (k/2)%2
 *     values: u = k/16, l = 16*((t%16)/4) + k%16,
 *             e = (t%32)/16 + 2*(t%2), n = (t%4)/2
 *   its nibble is the high (n = 1) or low (n = 0) half of the byte at
 *     16r*(t/32) + 1024*(u/4) + 16*l + 4*(u%4) + e
 *   inside its slab (L_cap % 32 == 0, r in {64, 128, 256}): 32-bit unit u of
 *   lane l of the decode kernel's matrix-core operand, whose element 2m sits
 *   in nibble m and 2m+1 in nibble m+4. Each 32-token block is a permutation
 *   of its own 16 r bytes' nibbles. hadamard as for the int8 cache.
 *
 * palu_decode_attn over such a cache, as palu_decode_attn_i8 (same rules,
 * restrictions and errors, the int4 slabs in place of the int8 ones). */
palu_status palu_decode_attn_i4(const palu_attn_desc* desc, const void* q, const uint8_t* h_k,
                                const uint8_t* h_v, const float* s_k, const float* s_v,
                                const void* b_k, const void* b_v, const int32_t* seq_lens,
                                float* out, void* workspace, size_t workspace_bytes,
                                void* stream);

/* How the append's projections a_k, a_v are laid out in memory. Either way
 * the call computes h = x a with a of shape [d_model, G*r]. */
typedef enum palu_a_layout {
  /* a[d_model, G*r]: entry (i, c) at i * G*r + c, the product as written */
  PALU_A_IN_OUT = 0,
  /* a^T[G*r, d_model]: entry (i, c) at c * d_model + i, each latent's weights
   * contiguous (a torch.nn.Linear weight, out_features x in_features). The
   * dtype cache write then finishes each latent in one workgroup: one pass,
   * no workspace (size 0; the workspace pointer may be NULL). Needs d_model
   * % 8 == 0 (SHAPE); not offered for the int8 / int4 caches (UNSUPPORTED). */
  PALU_A_OUT_IN = 1
} palu_a_layout;

typedef struct palu_append_desc {
  int32_t batch;     /* B >= 1                                                    */
  int32_t d_model;   /* width of x, 1..65536                                      */
  int32_t n_groups;  /* G >= 1                                                    */
  int32_t rank;      /* r, 1..512                                                 */
  int32_t max_ctx;   /* L_cap: row stride of the cache                             */
  int32_t dtype;     /* palu_dtype of x, a_k, a_v and (except the int8 / int4 calls)
                        the cache */
  int32_t hadamard;  /* palu_latent_append_i8 / _i4 only (0 elsewhere): 1 rotates each
                        row by the Hadamard matrix before quantising */
  int32_t a_layout;  /* palu_a_layout of a_k and a_v; PALU_A_IN_OUT (0) in a
                        zero-initialised descriptor */
} palu_append_desc;

/* Bytes of device workspace palu_latent_append needs for this descriptor:
 * arrival counters (one int32 per 128 columns of [a_k | a_v], padded to 256
 * bytes) followed by fp32 partial sums over slices of 128 rows of d_model;
 * 0 with a_layout PALU_A_OUT_IN. */
palu_status palu_latent_append_workspace(const palu_append_desc* desc, size_t* bytes);

/* Cache write of one token per sequence (answer to Q2: h = x A):
 *   h_k[b, g, pos[b], :] = x[b] . a_k[:, g*r:(g+1)*r], likewise h_v with a_v.
 *   x [B, d_model]; a_k, a_v [d_model, G*r] (or transposed, see
 *   palu_a_layout); h_k, h_v [B, G, L_cap, r]; x, a_k, a_v 16-byte aligned;
 *   pos [B] int32 on the device; workspace: 16-byte aligned device memory of
 *   at least the size reported by palu_latent_append_workspace whose counter
 *   area (its first bytes, see above) is zero before the first call, e.g.
 *   allocated zeroed; every call that completes leaves it zero again and
 *   overwrites the rest. Calls that share a workspace must not overlap in
 *   time (same stream, or ordered by events). Products are summed in fp32 in
 *   a fixed order (PALU_A_IN_OUT: per 128-row slice, then the slices in
 *   order; PALU_A_OUT_IN: per thread over d_model chunks 2048 apart, then the
 *   256 threads' sums in order), so results do not depend on timing; a bf16
 *   cache stores the sum rounded to the nearest bf16 (ties to even). Rows with
 *   pos outside [0, L_cap) are left untouched. Errors: NULL, SHAPE (also
 *   G*r > 65536 or G*r not a multiple of 8), UNSUPPORTED (also an unknown
 *   a_layout), WORKSPACE (too small or misaligned), DEVICE. */
palu_status palu_latent_append(const palu_append_desc* desc, const void* x, const void* a_k,
                               const void* a_v, void* h_k, void* h_v, const int32_t* pos,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace palu_latent_append_i8 needs: the same areas as
 * palu_latent_append's (counters, then partial sums), under the same rule:
 * the counter area is zero before the first call. */
palu_status palu_latent_append_i8_workspace(const palu_append_desc* desc, size_t* bytes);

/* Quantised cache write of one token per sequence into the int8 cache that
 * palu_decode_attn_i8 reads (layout above): the fp32 row h = x[b] .
 * a[:, g*r:(g+1)*r], formed as in palu_latent_append (with desc->hadamard = 1
 * then rotated in fp32, h'' = h H_r), is stored as
 *   s[b, g, pos[b]] = amax / 127, code of latent k = round(h[k] * 127 / amax)
 * with amax = max_k |h[k]|, correctly rounded fp32 divisions, round to nearest
 * (ties to even) of the fp32 product, codes clamped to [-127, 127]; a row of
 * zeros stores scale 0 and codes 0.
 *   x, a_k, a_v, pos as in palu_latent_append (desc->dtype is theirs);
 *   h_k, h_v int8 slabs, 4-byte aligned; s_k, s_v [B, G, L_cap] fp32.
 * Needs r in {64, 128, 256} (UNSUPPORTED otherwise) and L_cap % 32 == 0
 * (SHAPE). Workspace rules, overlap rules and errors as in
 * palu_latent_append. */
palu_status palu_latent_append_i8(const palu_append_desc* desc, const void* x, const void* a_k,
                                  const void* a_v, int8_t* h_k, int8_t* h_v, float* s_k,
                                  float* s_v, const int32_t* pos, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Bytes of device workspace palu_latent_append_i4 needs (the same areas as
 * for palu_latent_append_i8, under the same zero-counter rule). */
palu_status palu_latent_append_i4_workspace(const palu_append_desc* desc, size_t* bytes);

/* Quantised cache write of one token per sequence into the int4 cache that
 * palu_decode_attn_i4 reads (layout above), as palu_latent_append_i8 with 7
 * in place of 127: s = amax / 7, code = round(h[k] * 7 / amax) clamped to
 * [-7, 7]. A value byte also holds the code of another token of the same
 * block (t xor 2), which is kept: the call reads and rewrites that byte, so
 * calls that write either token must not overlap. h_k, h_v 4-byte aligned.
 * Restrictions, workspace rules and errors as in palu_latent_append_i8. */
palu_status palu_latent_append_i4(const palu_append_desc* desc, const void* x, const void* a_k,
                                  const void* a_v, uint8_t* h_k, uint8_t* h_v, float* s_k,
                                  float* s_v, const int32_t* pos, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* One decode step's work ahead of its decode call, in as few launches as it
 * allows: the cache write that qbits selects (0: palu_latent_append, 8:
 * palu_latent_append_i8, 4: palu_latent_append_i4) and
 * palu_decode_attn_prepare for `attn`; the decode call then follows on the
 * same stream with attn->prepared = 1 and the same workspace. The two parts
 * are independent (the query-side operands read q and b_k, never the cache).
 * When attn is ABSORBED with the append's dtype and head_dim / 8 is a power
 * of two <= 32, the query absorption (the clarification of W1: B_k moves onto
 * the query) runs as extra workgroups of the append's launch, beside the
 * cache write, in one launch (unless those would exceed a launch grid's
 * 65535 rows, at very large batch); otherwise the two are launched one after
 * the other on `stream`. Either way the results are those of the two calls.
 *   ad, x, a_k, a_v, h_k, h_v, s_k, s_v, pos, append_ws, append_ws_bytes: as
 *     for the append call qbits selects (s_k, s_v unused and may be NULL for
 *     qbits 0; h_k, h_v are int8_t* / uint8_t* codes for qbits 8 / 4);
 *   attn, q, b_k, workspace, workspace_bytes: as for palu_decode_attn_prepare
 *     (attn->prepared is not read).
 * Errors: those of the two calls, checked before anything is launched;
 * UNSUPPORTED for qbits other than 0, 8 and 4; WORKSPACE also when the byte
 * ranges [append_ws, +append_ws_bytes) and [workspace, +workspace_bytes)
 * overlap. */
palu_status palu_latent_append_prepare(const palu_append_desc* ad, int32_t qbits, const void* x,
                                       const void* a_k, const void* a_v, void* h_k, void* h_v,
                                       float* s_k, float* s_v, const int32_t* pos,
                                       void* append_ws, size_t append_ws_bytes,
                                       const palu_attn_desc* attn, const void* q,
                                       const void* b_k, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Optional timing of the main decode kernel (the context-split kernel) with HIP
 * events on the stream it is launched on. palu_profile_begin(n) arms n records
 * (events are created here, once); each later palu_decode_attn call claims the
 * next start/stop pair (one atomic increment, so concurrent calls never share
 * a pair) and records it around that kernel, until n are used.
 * palu_profile_end waits for the recorded events, returns the summed
 * milliseconds and the count, releases the events and disarms. begin and end
 * themselves must not overlap any other call; for benchmarks. */
palu_status palu_profile_begin(int32_t max_records);
palu_status palu_profile_end(double* total_ms, int32_t* count);

/* A short text for a status code; any value is accepted (codes that are not
 * a palu_status give "unknown status"). */
const char* palu_status_string(int32_t status);
const char* palu_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PALU_H */
