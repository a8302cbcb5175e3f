/*
 * lla.h - C ABI of the MI355X (gfx950) latent-store decode library for Looped Latent
 * Attention (LLA).
 *
 * Method: "Looped Latent Attention: Cross-Loop KV Compression for Looped Transformers"
 * (arXiv 2607.15456v2).
 *   - Section 3, Eq. 1: the T per-loop keys (or values) of one token, layer and head are
 *     stacked as x = [x_1; ...; x_T] (pre-RoPE).
 *   - Section 3, Eq. 2: the cache stores c = (x - mu) W_down, with r_k (keys) or r_v
 *     (values) entries.
 *   - Section 3, Eq. 3: loop t is rebuilt on read as x_t = c W_up,t^T + mu_t.
 *   - Section 3, "RoPE and reconstruction": the model's RoPE is applied to the rebuilt
 *     keys; attention itself is unchanged (Figure 1).
 *   - Section 3, "The LLA-2D variant": one latent per token and layer rebuilds all heads.
 *   - Section 7 and Appendix A ("Decoding and caching"): the latent-store decoder caches
 *     only latents and rebuilds on read.
 *   - Appendix J ("Absorbed attention"): the value side may be applied to the
 *     softmax-weighted latent, sum_i a_i W c_i = W sum_i a_i c_i; with sum_i a_i = 1 the
 *     mean term passes through unchanged.
 *
 * Conventions shared by every entry point
 *   - All pointers named as device pointers must point to HIP device memory (or memory
 *     the device can address) and be 16-byte aligned. The caller owns every buffer; the
 *     library allocates nothing and keeps no state beyond cached device properties and
 *     the fixed scratch array of lla_decode_attn_noalloc.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and is
 *     asynchronous: no host synchronisation happens inside the library.
 *   - Arguments are validated on the host before anything is enqueued. A rejected call
 *     returns a negative lla_status and enqueues nothing. A launch failure is reported
 *     as LLA_ERR_HIP.
 *   - Floating-point outputs are float32. Accumulation is float32 throughout.
 *
 * Tensor layouts (row-major, no padding). Hc = H and d_in = d_head for the per-head
 * codec; Hc = 1 and d_in = H * d_head for LLA-2D. Element type of every codec and
 * cache tensor is `dims.dtype` (float32 or bfloat16).
 *   cache.c_k          [D][batch][Hc][n_max][r_k]   latents of keys
 *   cache.c_v          [D][batch][Hc][n_max][r_v]   latents of values
 *   codec.w_down_k_t   [D][Hc][r_k][T*d_in]          W_down of Eq. 2, stored transposed
 *   codec.mu_k         [D][Hc][T*d_in]               mu of Eq. 2 (mu_t is loop t's slice;
 *                                                    LLA-2D stacks (t, h, d), t outermost)
 *   codec.w_up_k       [D][T][H][d_head][r_k]        W_up,t of Eq. 3 for every loop/head
 *   (same for _v with r_v)
 *   codec.rope_table   built by lla_rope_table_build for (d_head, n_max, rope_base)
 */
#ifndef LLA_H_
#define LLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LLA_OK = 0,
  LLA_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned pointer, out of range */
  LLA_ERR_UNSUPPORTED = -2, /* valid but not built: a (d_head, r_k, r_v) or dtype combo */
  LLA_ERR_WORKSPACE = -3,   /* workspace smaller than lla_decode_workspace_bytes */
  LLA_ERR_HIP = -4          /* a HIP call or kernel launch failed */
} lla_status;

typedef enum { LLA_F32 = 0, LLA_BF16 = 1 } lla_dtype;
typedef enum { LLA_PER_HEAD = 0, LLA_2D = 1 } lla_variant;

/* Decode kernel family.
 *   LLA_PATH_RECONSTRUCT : rebuild each key tile with MFMA (K^T = W_up,k,t C_k^T + mu_k,t),
 *                          rotate it in registers, dot with q, online softmax. float32
 *                          caches rotate and dot in float32; bfloat16 caches round the
 *                          rebuilt key to float16 and contract the products of each pair
 *                          with cos and sin (float16) against [q0, q1, q1, -q0] on the
 *                          matrix cores, so their scores carry float16 rounding like the
 *                          fold's, and keys beyond 65504 in magnitude overflow.
 *   LLA_PATH_ROTARY_FOLD : the same scores via an exact rewrite: for every rotary pair i
 *                          q.R(j theta_i)k = cos(j theta_i) P_i + sin(j theta_i) Q_i with
 *                          P_i, Q_i linear in the latent, so the score is
 *                          c_j . (CS_j M) + CS_j m, where CS_j holds cos/sin of position j
 *                          (shared by all heads) and M (d_head x r_k) folds q into W_up.
 *                          bfloat16 only; CS and M enter the MFMA as float16, so each
 *                          folded score carries float16 rounding (relative 2^-11 of the
 *                          score's terms): outputs stay within 2e-2 of exact attention for
 *                          score spreads up to about 55 (scale * q.k in natural-log
 *                          units); M overflows float16 only past 65504, far beyond that.
 *   LLA_PATH_AUTO        : ROTARY_FOLD for the bfloat16 shapes a fold kernel is built for,
 *                          per head and LLA-2D (the narrow, wide or LLA-2D fold kernel);
 *                          RECONSTRUCT for everything else (float32, other shapes). */
typedef enum { LLA_PATH_AUTO = 0, LLA_PATH_RECONSTRUCT = 1, LLA_PATH_ROTARY_FOLD = 2 } lla_path;

typedef struct {
  int32_t T;        /* loops (recurrence steps) */
  int32_t D;        /* layers */
  int32_t H;        /* attention heads */
  int32_t d_head;   /* head width; 64 or 128 */
  int32_t r_k;      /* key latent size; multiple of 16 */
  int32_t r_v;      /* value latent size; multiple of 8 */
  int32_t batch;    /* sequences */
  int32_t n_max;    /* cache capacity in tokens per sequence */
  int32_t variant;  /* lla_variant */
  int32_t dtype;    /* lla_dtype of latents and codec weights */
  float rope_base;  /* RoPE base, e.g. 10000 */
  float scale;      /* score scale; 0 selects 1/sqrt(d_head) */
} lla_dims;

typedef struct {
  const void* w_down_k_t; /* encode only */
  const void* mu_k;
  const void* w_up_k;
  const void* w_down_v_t; /* encode only */
  const void* mu_v;
  const void* w_up_v;
  const void* rope_table; /* decode only */
} lla_codec;

typedef struct {
  void* c_k;
  void* c_v;
} lla_cache;

typedef struct {
  int32_t num_splits; /* context splits per (sequence, head, loop); 0 = choose */
  int32_t path;       /* lla_path */
} lla_decode_opts;

/* A paged latent cache (Appendix D, Table 9 and Appendix J, "Eviction and long-context
 * prefill": token eviction composes with the latent codec). Latents live in pages of 16
 * tokens; each layer's pool is cache.c_k [D][num_pages][Hc][16][r_k] (c_v likewise), and
 * logical token j of sequence b is row j % 16 of page block_table[b * max_blocks + j / 16].
 * Positions for RoPE are the logical slots j, so evicting pages and listing the kept ones
 * in order (sinks, then the most recent pages) gives StreamingLLM's cache-relative
 * positions without touching the stored latents, which are kept before RoPE. */
typedef struct {
  const int32_t* block_table; /* device int32 [batch][max_blocks], 4-byte aligned */
  int32_t max_blocks;         /* max_blocks * 16 >= dims.n_max (the logical capacity) */
  int32_t num_pages;          /* pages in each layer's pool */
} lla_pages;

/* Human-readable name of a status code. Never NULL. */
const char* lla_status_string(int32_t status);

/* Compression ratio rho of Eq. 4 for these dims: 2 T H d_head / ((r_k + r_v) Hc).
 * Returns a negative value when dims is NULL or has non-positive sizes. */
double lla_compression_ratio(const lla_dims* dims);

/* Bytes one token occupies in the latent cache over all D layers:
 * D * Hc * (r_k + r_v) * sizeof(dtype) (Section 7, Table 5 "KV / token").
 * Returns a negative value on invalid dims. */
double lla_cache_bytes_per_token(const lla_dims* dims);

/* Size in bytes of the RoPE table for dims (d_head, n_max). */
size_t lla_rope_table_bytes(const lla_dims* dims);

/* Fill `table` (device, lla_rope_table_bytes(dims) bytes) with cos/sin of p*theta_i,
 * theta_i = rope_base^(-2i/d_head), for every position p < n_max, evaluated in float64
 * and rounded once (float32 and float16 copies). Pairs are interleaved (2i, 2i+1), as
 * in RoFormer, which the LLA paper cites for RoPE. Build once per (d_head, n_max,
 * rope_base) and pass it in lla_codec.rope_table. */
int32_t lla_rope_table_build(const lla_dims* dims, void* table, void* stream);

/* Encode (Section 3, Eq. 2): for every sequence b, new token j < n_new and latent head
 * hc, c = (x - mu) W_down for keys and values of `layer`, stored with round-to-nearest-
 * even into cache row pos_start + j.
 *   x_k, x_v : device, [batch][n_new][Hc][T][d_in] of dtype, pre-RoPE, loop t of the
 *              stacked vector at [t][*] (Eq. 1). Must be the finished T-loop values.
 *   requires 0 <= layer < D, n_new >= 0, 0 <= pos_start, pos_start + n_new <= n_max.
 * n_new == 0 enqueues nothing and returns LLA_OK. */
int32_t lla_encode(const lla_dims* dims, const lla_codec* codec, const lla_cache* cache,
                   int32_t layer, const void* x_k, const void* x_v, int32_t pos_start,
                   int32_t n_new, void* stream);

/* Workspace bytes lla_decode_attn needs for this call shape (0 is never returned for
 * valid dims; returns 0 on invalid arguments). */
size_t lla_decode_workspace_bytes(const lla_dims* dims, int32_t n_ctx, int32_t loop_count,
                                  const lla_decode_opts* opts);

/* Latent-store decode attention for one layer and loops loop_begin .. loop_begin +
 * loop_count - 1 (Section 7; Eqs. 3 and RoPE after reconstruction; Appendix J value
 * identity). For every sequence b, head h and loop t:
 *   K_t[j] = RoPE_j(c_k[j] W_up,k,t^T + mu_k,t),  V_t[j] = c_v[j] W_up,v,t^T + mu_v,t,
 *   out[b][h][t] = softmax_j(scale * q . K_t[j]) V_t   over j < len_b,
 * with RoPE at position j = the cache slot. The value side is computed as
 * (sum_j a_j c_v[j]) W_up,v,t^T + mu_v,t.
 *   q        : device float32 [batch][H][loop_count][d_head], queries already rotated.
 *   out      : device float32 [batch][H][loop_count][d_head]; len_b == 0 gives zeros.
 *   ctx_lens : device int32 [batch] or NULL. NULL: len_b = n_ctx for all b. Otherwise
 *              len_b = ctx_lens[b], clamped by the kernels to [0, n_ctx].
 *   requires 0 <= n_ctx <= n_max, 0 <= layer < D, 0 <= loop_begin,
 *            1 <= loop_count, loop_begin + loop_count <= T.
 *   workspace: device, >= lla_decode_workspace_bytes(dims, n_ctx, loop_count, opts).
 *   opts     : NULL for defaults. */
int32_t lla_decode_attn(const lla_dims* dims, const lla_codec* codec, const lla_cache* cache,
                        int32_t layer, int32_t n_ctx, const int32_t* ctx_lens, const float* q,
                        int32_t loop_begin, int32_t loop_count, float* out, void* workspace,
                        size_t workspace_bytes, const lla_decode_opts* opts, void* stream);

/* Number of context splits lla_decode_attn would use (after `opts`), for reporting. */
int32_t lla_decode_num_splits(const lla_dims* dims, int32_t n_ctx, int32_t loop_count,
                              const lla_decode_opts* opts);

/* Decoupled-RoPE absorbed decode (Appendix J, "Absorbed attention": an MLA-style content
 * path without RoPE plus a small explicit rotary branch that all loops of a token share).
 * Dimensions 0 .. d_rope-1 of every head are the rotary branch, d_rope .. d_head-1 the
 * content path. For every sequence b, head h and loop t:
 *   key_t[j] = [ k_rope[j] ; (c_k[j] W_up,k,t^T + mu_k,t)[d_rope ..] ]   (no RoPE here)
 *   out[b][h][t] = softmax_j(scale * q . key_t[j]) V_t   over j < len_b,
 * computed without rebuilding keys: q~ = W_up,k,t[d_rope ..]^T q[d_rope ..] scores the
 * latent directly, and the value side is (sum_j a_j c_v[j]) W_up,v,t^T + mu_v,t.
 *   k_rope : device [D][batch][H][n_max][d_rope] in the cache dtype: the rotary keys,
 *            already rotated to their positions (RoPE of the slot index), one per token
 *            for every loop. Written by the caller.
 *   d_rope : 16 <= d_rope < d_head, a multiple of 16; built shapes are listed by
 *            lla_decode_absorbed_supported.
 *   q      : device float32 [batch][H][loop_count][d_head]; entries 0 .. d_rope-1 are the
 *            rotated rotary query, the rest the content query.
 *   scale  : dims->scale, 0 = 1/sqrt(d_head).
 *   other arguments and errors as lla_decode_attn (the path field of opts is ignored);
 *   workspace >= lla_decode_absorbed_workspace_bytes(dims, d_rope, n_ctx, loop_count, opts)
 *   (the split partials). */
size_t lla_decode_absorbed_workspace_bytes(const lla_dims* dims, int32_t d_rope, int32_t n_ctx,
                                           int32_t loop_count, const lla_decode_opts* opts);
int32_t lla_decode_attn_absorbed(const lla_dims* dims, const lla_codec* codec,
                                 const lla_cache* cache, const void* k_rope, int32_t d_rope,
                                 int32_t layer, int32_t n_ctx, const int32_t* ctx_lens,
                                 const float* q, int32_t loop_begin, int32_t loop_count,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 const lla_decode_opts* opts, void* stream);
/* 1 when a kernel is built for (dims' dtype, d_head, r_k, r_v, d_rope), else 0. */
int32_t lla_decode_absorbed_supported(const lla_dims* dims, int32_t d_rope);

/* lla_decode_attn_absorbed over a paged cache (see lla_pages): cache.c_k and cache.c_v are
 * the latent pools and k_rope is the rotary-key pool, device
 * [D][num_pages][H][16][d_rope] in the cache dtype: the rotary key of logical token j of
 * sequence b and head h is row j % 16 of head h's rows in page
 * block_table[b * max_blocks + j / 16], written by the caller (rotated at the logical
 * slot j, like the latents' RoPE positions). Same result as the dense call on the
 * gathered rows. Unlike the latents, whose RoPE is applied at decode time at the current
 * logical slot, the stored rotary keys keep the positions they were rotated at: after an
 * eviction moves kept tokens to new logical slots, the caller re-rotates their rotary
 * keys if it wants cache-relative positions for them too. A context split spans at most 4096 tokens, so num_splits of opts may be
 * raised to that. workspace >= lla_decode_absorbed_paged_workspace_bytes(...). Other
 * arguments and errors as lla_decode_attn_absorbed, plus `pages` (validated as described
 * at lla_pages; table entries outside the pool are clamped into it). */
size_t lla_decode_absorbed_paged_workspace_bytes(const lla_dims* dims, int32_t d_rope,
                                                 int32_t n_ctx, int32_t loop_count,
                                                 const lla_decode_opts* opts);
int32_t lla_decode_attn_absorbed_paged(const lla_dims* dims, const lla_codec* codec,
                                       const lla_cache* cache, const lla_pages* pages,
                                       const void* k_rope, int32_t d_rope, int32_t layer,
                                       int32_t n_ctx, const int32_t* ctx_lens, const float* q,
                                       int32_t loop_begin, int32_t loop_count, float* out,
                                       void* workspace, size_t workspace_bytes,
                                       const lla_decode_opts* opts, void* stream);

/* Materialised reconstruction of a slot range of one layer (Section 3, Eq. 3 and "RoPE
 * and reconstruction"): the second pass of the latent-store decoder's two-pass prefill,
 * streamed one layer at a time (Appendix A, "Decoding and caching"; Appendix J,
 * "Eviction and long-context prefill"). For loops t = loop_begin .. loop_begin +
 * loop_count - 1, every sequence b, head h and slot j in [pos_start, pos_start + n_tok):
 *   k_out[t - loop_begin][b][h][j] = RoPE_j(c_k[j] W_up,k,t^T + mu_k,t)
 *   v_out[t - loop_begin][b][h][j] = c_v[j] W_up,v,t^T + mu_v,t
 *   k_out, v_out : device [loop_count][batch][H][n_max][d_head] in dims->dtype (the
 *                  layout of one layer of the uncompressed cache that
 *                  lla_decode_attn_teacher reads); only the rows of the slot range are
 *                  written. Either may be NULL (that axis is skipped), not both.
 *                  bfloat16 outputs are rounded once, to nearest even.
 *   codec  : w_up_*, mu_* of the axes asked for; rope_table when k_out is given.
 *   requires 0 <= layer < D, 0 <= loop_begin, 1 <= loop_count, loop_begin + loop_count
 *            <= T, 0 <= pos_start, 0 <= n_tok, pos_start + n_tok <= n_max.
 * n_tok == 0 enqueues nothing. Errors as lla_decode_attn; shapes not built (r not in
 * 16, 24, 32, 64, 96, 128, 160, 256) give LLA_ERR_UNSUPPORTED. */
int32_t lla_reconstruct(const lla_dims* dims, const lla_codec* codec, const lla_cache* cache,
                        int32_t layer, int32_t loop_begin, int32_t loop_count, int32_t pos_start,
                        int32_t n_tok, void* k_out, void* v_out, void* stream);

/* lla_encode into a paged cache: the latents of logical tokens pos_start .. pos_start +
 * n_new - 1 of every sequence are written to the rows their pages name. Arguments and
 * errors as lla_encode, plus `pages` (validated as described at lla_pages). The block
 * table's entries for the written logical pages must be pages of the pool; an entry
 * outside [0, num_pages) is clamped into it (no access outside the pool, wrong rows). */
int32_t lla_encode_paged(const lla_dims* dims, const lla_codec* codec, const lla_cache* cache,
                         const lla_pages* pages, int32_t layer, const void* x_k, const void* x_v,
                         int32_t pos_start, int32_t n_new, void* stream);

/* Projection-fused encode (Section 3, Eqs. 1-2; Appendix J, "Eviction and long-context
 * prefill": the per-loop keys and values of a prompt need never be stored). A looped
 * layer applies the same key and value projections at every loop, x_t = h_t W_proj, to
 * that loop's input h_t. Eq. 2 is linear in the stacked vector, so
 *   c = sum_t (x_t - mu_t) W_down[rows of loop t],
 * and each loop's term can be added as soon as h_t exists. One call handles loop `loop`
 * of `layer` for keys and values: it forms x_t for the n_new new tokens of every
 * sequence, subtracts mu_t and adds the term to `acc`; the call for loop T - 1 rounds the
 * sum once (to nearest even) and writes cache rows pos_start .. pos_start + n_new - 1.
 *   proj->w_k, proj->w_v : device bfloat16 [D][H * d_head][d_model], the key and value
 *            projections of every layer stored as a linear layer stores its weight
 *            (output features x input features): x_t[h d_head + j] = h_t . row
 *            (h d_head + j); proj->d_model a positive multiple of 32.
 *   h      : device bfloat16 [batch][n_new][d_model], the hidden states that enter the
 *            projections at this loop.
 *   acc    : device float32, acc_bytes >= lla_encode_fused_acc_bytes(dims, n_new) (the
 *            float32 running sums of every new token, latent head and entry, tokens
 *            rounded up to whole blocks of 256; the order inside is the library's own):
 *            owned by the caller and kept between the calls of one layer. Loop 0
 *            overwrites it (no clearing needed); loops 1 .. T-1 read and update it.
 *   codec  : w_down_k_t, mu_k, w_down_v_t, mu_v as for lla_encode.
 * The T calls of a layer must run in loop order 0 .. T-1 with the same acc, n_new and
 * pos_start, on one stream (or ordered by the caller); the cache rows hold the result
 * only after loop T - 1. Built for bfloat16, d_head 128 and r_k, r_v in {16, 32, 64, 96,
 * 128, 160}, per head and LLA-2D; other shapes give LLA_ERR_UNSUPPORTED. Otherwise
 * arguments and errors as lla_encode, plus LLA_ERR_INVALID_ARG for 0 > loop or loop >= T
 * and LLA_ERR_WORKSPACE for a short acc. n_new == 0 enqueues nothing. */
typedef struct {
  const void* w_k;
  const void* w_v;
  int32_t d_model;
} lla_proj;
size_t lla_encode_fused_acc_bytes(const lla_dims* dims, int32_t n_new);
int32_t lla_encode_fused(const lla_dims* dims, const lla_codec* codec, const lla_proj* proj,
                         const lla_cache* cache, int32_t layer, int32_t loop, const void* h,
                         int32_t pos_start, int32_t n_new, float* acc, size_t acc_bytes,
                         void* stream);

/* lla_decode_attn over a paged cache (logical tokens 0 .. len_b - 1 through the block
 * table; RoPE at the logical slot). Paths as lla_decode_attn: the rotary fold kernels
 * (bfloat16 shapes they are built for, per head and LLA-2D), else the reconstruct path;
 * asking for the rotary fold elsewhere gives LLA_ERR_UNSUPPORTED. On the fold kernels a
 * context split spans at most 4096 tokens (256 pages, whose indices a workgroup keeps
 * in LDS), so num_splits of opts may be raised to that. workspace >=
 * lla_decode_paged_workspace_bytes(dims, n_ctx, loop_count, opts). Other arguments and
 * errors as lla_decode_attn; block table entries as for lla_encode_paged. */
size_t lla_decode_paged_workspace_bytes(const lla_dims* dims, int32_t n_ctx, int32_t loop_count,
                                        const lla_decode_opts* opts);
int32_t lla_decode_attn_paged(const lla_dims* dims, const lla_codec* codec, const lla_cache* cache,
                              const lla_pages* pages, int32_t layer, int32_t n_ctx,
                              const int32_t* ctx_lens, const float* q, int32_t loop_begin,
                              int32_t loop_count, float* out, void* workspace,
                              size_t workspace_bytes, const lla_decode_opts* opts, void* stream);
/* Number of context splits lla_decode_attn_paged would use (after `opts`), for reporting;
 * 0 on invalid arguments. */
int32_t lla_decode_paged_num_splits(const lla_dims* dims, int32_t n_ctx, int32_t loop_count,
                                    const lla_decode_opts* opts);

/* Uncompressed decode over the loop-indexed cache that the latent store replaces (Section
 * 3, "Teacher cache": every loop of every layer keeps its own key and value; Section 7,
 * Table 5: the teacher's serving path). For every sequence b, head h and loop t:
 *   out[b][h][t] = softmax_j(scale * q . k_cache[t][b][h][j]) v_cache[t][b][h]  over j < len_b.
 *   k_cache : device [D][T][batch][H][n_max][d_head] in dims->dtype: keys of every loop,
 *             already rotated to their positions. Written by the caller.
 *   v_cache : device [D][T][batch][H][n_max][d_head] in dims->dtype: values of every loop.
 *   q, out, ctx_lens, layer, n_ctx, loop_begin, loop_count: as lla_decode_attn.
 *   scale   : dims->scale, 0 = 1/sqrt(d_head).
 * Only T, D, H, batch, n_max, d_head, dtype and scale of dims are read (the codec fields
 * r_k, r_v, variant and rope_base are ignored). Built shapes are listed by
 * lla_decode_teacher_supported (d_head 64 or 128). num_splits of opts applies; its path
 * field is ignored.
 *   workspace >= lla_decode_teacher_workspace_bytes(dims, n_ctx, loop_count, opts)
 *   (the split partials; may be 0 bytes, then workspace may be NULL).
 * Errors as lla_decode_attn. */
size_t lla_decode_teacher_workspace_bytes(const lla_dims* dims, int32_t n_ctx, int32_t loop_count,
                                          const lla_decode_opts* opts);
int32_t lla_decode_attn_teacher(const lla_dims* dims, const void* k_cache, const void* v_cache,
                                int32_t layer, int32_t n_ctx, const int32_t* ctx_lens,
                                const float* q, int32_t loop_begin, int32_t loop_count,
                                float* out, void* workspace, size_t workspace_bytes,
                                const lla_decode_opts* opts, void* stream);
/* 1 when a kernel is built for (dims' dtype, d_head), else 0. */
int32_t lla_decode_teacher_supported(const lla_dims* dims);
/* Number of context splits lla_decode_attn_teacher would use (after `opts`), for
 * reporting; 0 on invalid arguments. */
int32_t lla_decode_teacher_num_splits(const lla_dims* dims, int32_t n_ctx, int32_t loop_count,
                                      const lla_decode_opts* opts);

/* lla_decode_attn without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The split partials go to a device array of LLA_NOALLOC_SCRATCH_BYTES that
 * the library holds on each GPU it runs on, from the first such call on that GPU until
 * the process ends; the call itself allocates nothing. Arguments, results and errors are
 * those of lla_decode_attn with `workspace` taken from that array, except:
 *   - LLA_ERR_WORKSPACE when lla_decode_workspace_bytes(dims, n_ctx, loop_count, opts)
 *     exceeds LLA_NOALLOC_SCRATCH_BYTES (fewer splits in opts, or a smaller batch, fit);
 *   - LLA_ERR_HIP when the array's device address cannot be found on the current device.
 * The array is shared by every call on one GPU: two calls whose kernels may overlap on
 * that GPU (different streams, or different host threads) race and can give wrong
 * results. Serialise them on one stream. */
#define LLA_NOALLOC_SCRATCH_BYTES (8u << 20)
int32_t lla_decode_attn_noalloc(const lla_dims* dims, const lla_codec* codec,
                                const lla_cache* cache, int32_t layer, int32_t n_ctx,
                                const int32_t* ctx_lens, const float* q, int32_t loop_begin,
                                int32_t loop_count, float* out, const lla_decode_opts* opts,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LLA_H_ */
