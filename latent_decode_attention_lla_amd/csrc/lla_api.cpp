// C ABI of the LLA latent-store decode library: host-side validation and dispatch to the
// gfx950 kernels (launch planning in lla_plan.h). See include/lla.h for the contract of
// every entry point. Nothing here allocates device memory or synchronises the stream.
#include "lla.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "lla_kernels.h"
#include "lla_plan.h"

namespace {

constexpr double kLog2e = 1.4426950408889634;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(const lla_dims& d) { return d.dtype == LLA_F32 ? 4 : 2; }
int latent_heads(const lla_dims& d) { return d.variant == LLA_PER_HEAD ? d.H : 1; }
int d_in(const lla_dims& d) { return d.variant == LLA_PER_HEAD ? d.d_head : d.H * d.d_head; }

// Shape checks shared by every entry point.
int32_t check_dims(const lla_dims* d) {
  if (d == nullptr) return LLA_ERR_INVALID_ARG;
  if (d->T < 1 || d->D < 1 || d->H < 1 || d->batch < 1 || d->n_max < 1) return LLA_ERR_INVALID_ARG;
  if (d->d_head < 2 || d->d_head % 2 != 0) return LLA_ERR_INVALID_ARG;
  if (d->r_k < 1 || d->r_v < 1) return LLA_ERR_INVALID_ARG;
  if (d->variant != LLA_PER_HEAD && d->variant != LLA_2D) return LLA_ERR_INVALID_ARG;
  if (d->dtype != LLA_F32 && d->dtype != LLA_BF16) return LLA_ERR_INVALID_ARG;
  if (!(d->rope_base > 0.f) || !std::isfinite(d->rope_base)) return LLA_ERR_INVALID_ARG;
  if (!(d->scale >= 0.f) || !std::isfinite(d->scale)) return LLA_ERR_INVALID_ARG;
  // Built shapes: d_head 64 or 128, r_k a multiple of 16, r_v a multiple of 8.
  if (d->d_head != 64 && d->d_head != 128) return LLA_ERR_UNSUPPORTED;
  if (d->r_k % 16 != 0 || d->r_v % 8 != 0) return LLA_ERR_UNSUPPORTED;
  // Index arithmetic inside the kernels is 32-bit per (sequence, head) plane offset
  // products and 64-bit for whole-tensor offsets; keep the per-plane sizes in range.
  if (static_cast<long long>(d->n_max) * (d->r_k > d->r_v ? d->r_k : d->r_v) >= (1LL << 31))
    return LLA_ERR_UNSUPPORTED;
  return LLA_OK;
}

int32_t hip_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? LLA_OK : LLA_ERR_HIP;
}

// Uncompressed decode: only the attention shape matters (no codec fields).
int32_t check_teacher_dims(const lla_dims* d) {
  if (d == nullptr) return LLA_ERR_INVALID_ARG;
  if (d->T < 1 || d->D < 1 || d->H < 1 || d->batch < 1 || d->n_max < 1) return LLA_ERR_INVALID_ARG;
  if (d->d_head < 2 || d->d_head % 2 != 0) return LLA_ERR_INVALID_ARG;
  if (d->dtype != LLA_F32 && d->dtype != LLA_BF16) return LLA_ERR_INVALID_ARG;
  if (!(d->scale >= 0.f) || !std::isfinite(d->scale)) return LLA_ERR_INVALID_ARG;
  if (!lla::decode_teacher_supported(d->dtype, d->d_head)) return LLA_ERR_UNSUPPORTED;
  if (static_cast<long long>(d->n_max) * d->d_head >= (1LL << 31)) return LLA_ERR_UNSUPPORTED;
  return LLA_OK;
}

// Paged cache checks: the block table covers the logical capacity n_max, the pool is
// non-empty, and the table is readable as int32.
int32_t check_pages(const lla_dims& d, const lla_pages* pg) {
  if (pg == nullptr || pg->block_table == nullptr) return LLA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(pg->block_table) & 3u) != 0) return LLA_ERR_INVALID_ARG;
  if (pg->num_pages < 1 || pg->max_blocks < 1) return LLA_ERR_INVALID_ARG;
  if (static_cast<long long>(pg->max_blocks) * lla::kPage < d.n_max) return LLA_ERR_INVALID_ARG;
  if (static_cast<long long>(d.batch) * pg->max_blocks >= (1LL << 31)) return LLA_ERR_UNSUPPORTED;
  return LLA_OK;
}

// The paged decode runs the same kernel as the dense one: a fold kernel where one is built
// for the shape, else the reconstruct kernel.
int paged_path(const lla_dims& d, const lla_decode_opts* opts) {
  const int want = opts ? opts->path : LLA_PATH_AUTO;
  const bool fold = fold_kind(d) != kFoldNone;
  if (want == LLA_PATH_AUTO) return fold ? LLA_PATH_ROTARY_FOLD : LLA_PATH_RECONSTRUCT;
  if (want == LLA_PATH_ROTARY_FOLD && !fold) return -1;
  return want;
}

Plan plan_paged(const lla_dims& d, int n_ctx, int loop_count, const lla_decode_opts* opts) {
  const bool fold = paged_path(d, opts) == LLA_PATH_ROTARY_FOLD;
  lla_decode_opts o{0, fold ? LLA_PATH_ROTARY_FOLD : LLA_PATH_RECONSTRUCT};
  if (opts != nullptr) o.num_splits = opts->num_splits;
  Plan p = plan_splits(d, n_ctx, loop_count, &o);
  // the fold kernels keep a split's page indices in LDS: at most kMaxSplitPages pages
  constexpr int kMaxLen = lla::kMaxSplitPages * lla::kPage;
  if (fold && fold_kind(d) != kFoldNone && p.split_len > kMaxLen) {
    p.split_len = kMaxLen;
    p.S = (n_ctx + kMaxLen - 1) / kMaxLen;
  }
  return p;
}

// Absorbed decode over a paged cache: the absorbed plan, with a split's page indices
// (at most kMaxSplitPages) kept in LDS.
Plan plan_absorbed_paged(const lla_dims& d, int n_ctx, int loop_count, const lla_decode_opts* opts) {
  Plan p = plan_absorbed(d, n_ctx, loop_count, opts);
  constexpr int kMaxLen = lla::kMaxSplitPages * lla::kPage;
  if (p.split_len > kMaxLen) {
    p.split_len = kMaxLen;
    p.S = (n_ctx + kMaxLen - 1) / kMaxLen;
  }
  return p;
}

}  // namespace

extern "C" {

const char* lla_status_string(int32_t status) {
  switch (status) {
    case LLA_OK: return "ok";
    case LLA_ERR_INVALID_ARG: return "invalid argument";
    case LLA_ERR_UNSUPPORTED: return "unsupported shape, dtype or path";
    case LLA_ERR_WORKSPACE: return "workspace too small";
    case LLA_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

double lla_compression_ratio(const lla_dims* d) {
  if (d == nullptr || d->T < 1 || d->H < 1 || d->d_head < 1 || d->r_k < 1 || d->r_v < 1) return -1.0;
  const double teacher = 2.0 * d->T * d->H * d->d_head;
  const double latent = static_cast<double>(d->r_k + d->r_v) * (d->variant == LLA_2D ? 1 : d->H);
  return teacher / latent;
}

double lla_cache_bytes_per_token(const lla_dims* d) {
  if (d == nullptr || d->D < 1 || d->H < 1 || d->r_k < 1 || d->r_v < 1) return -1.0;
  if (d->dtype != LLA_F32 && d->dtype != LLA_BF16) return -1.0;
  const double hc = d->variant == LLA_2D ? 1.0 : d->H;
  return static_cast<double>(d->D) * hc * (d->r_k + d->r_v) * static_cast<double>(elem_bytes(*d));
}

size_t lla_rope_table_bytes(const lla_dims* d) {
  if (d == nullptr || d->n_max < 1 || d->d_head < 2) return 0;
  const size_t n_pad = (static_cast<size_t>(d->n_max) + 15) / 16 * 16;
  return static_cast<size_t>(d->n_max) * d->d_head * 4 + n_pad * d->d_head * 2;
}

int32_t lla_rope_table_build(const lla_dims* d, void* table, void* stream) {
  const int32_t st = check_dims(d);
  if (st != LLA_OK) return st;
  if (table == nullptr || !aligned16(table)) return LLA_ERR_INVALID_ARG;
  float* t32 = static_cast<float*>(table);
  uint16_t* t16 = reinterpret_cast<uint16_t*>(static_cast<char*>(table) +
                                               static_cast<size_t>(d->n_max) * d->d_head * 4);
  lla::launch_rope_table(d->d_head, d->n_max, static_cast<double>(d->rope_base), t32, t16,
                         static_cast<hipStream_t>(stream));
  return hip_status();
}

int32_t lla_encode(const lla_dims* d, const lla_codec* codec, const lla_cache* cache,
                   int32_t layer, const void* x_k, const void* x_v, int32_t pos_start,
                   int32_t n_new, void* stream) {
  int32_t st = check_dims(d);
  if (st != LLA_OK) return st;
  if (codec == nullptr || cache == nullptr) return LLA_ERR_INVALID_ARG;
  if (layer < 0 || layer >= d->D) return LLA_ERR_INVALID_ARG;
  if (n_new < 0 || pos_start < 0 || static_cast<long long>(pos_start) + n_new > d->n_max)
    return LLA_ERR_INVALID_ARG;
  const void* ptrs[] = {x_k, x_v, codec->w_down_k_t, codec->w_down_v_t, codec->mu_k, codec->mu_v,
                        cache->c_k, cache->c_v};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return LLA_ERR_INVALID_ARG;
  const int Hc = latent_heads(*d);
  const int K = d->T * d_in(*d);
  if (!lla::encode_supported(d->dtype, d->r_k, K) || !lla::encode_supported(d->dtype, d->r_v, K))
    return LLA_ERR_UNSUPPORTED;
  if (n_new == 0) return LLA_OK;
  // tokens are tiled over (sequence, new token) with a 32-bit flattened index
  if (static_cast<long long>(d->batch) * n_new >= (1LL << 31) - 64) return LLA_ERR_UNSUPPORTED;
  const size_t es = elem_bytes(*d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int rs[2] = {d->r_k, d->r_v};
  const void* xs[2] = {x_k, x_v};
  const void* wds[2] = {codec->w_down_k_t, codec->w_down_v_t};
  const void* mus[2] = {codec->mu_k, codec->mu_v};
  void* cs[2] = {cache->c_k, cache->c_v};
  for (int ax = 0; ax < 2; ++ax) {
    const int r = rs[ax];
    lla::EncodeArgs a;
    a.x = xs[ax];
    a.w_down_t = static_cast<const char*>(wds[ax]) + static_cast<size_t>(layer) * Hc * r * K * es;
    a.mu = static_cast<const char*>(mus[ax]) + static_cast<size_t>(layer) * Hc * K * es;
    a.c = static_cast<char*>(cs[ax]) +
          static_cast<size_t>(layer) * d->batch * Hc * static_cast<size_t>(d->n_max) * r * es;
    a.B = d->batch;
    a.Hc = Hc;
    a.Kdim = K;
    a.n_new = n_new;
    a.pos_start = pos_start;
    a.n_max = d->n_max;
    if (!lla::launch_encode(d->dtype, r, a, s)) return LLA_ERR_UNSUPPORTED;
  }
  return hip_status();
}

size_t lla_encode_fused_acc_bytes(const lla_dims* d, int32_t n_new) {
  if (check_dims(d) != LLA_OK || n_new < 0) return 0;
  // float32 running sums of every (token, latent head, entry), tokens padded to whole
  // 256-token blocks (the kernels keep them in their own tile order)
  const size_t tok = (static_cast<size_t>(d->batch) * n_new + 255) / 256 * 256;
  return tok * latent_heads(*d) * static_cast<size_t>(d->r_k + d->r_v) * 4;
}

int32_t lla_encode_fused(const lla_dims* d, const lla_codec* codec, const lla_proj* proj,
                         const lla_cache* cache, int32_t layer, int32_t loop, const void* h,
                         int32_t pos_start, int32_t n_new, float* acc, size_t acc_bytes,
                         void* stream) {
  int32_t st = check_dims(d);
  if (st != LLA_OK) return st;
  if (codec == nullptr || proj == nullptr || cache == nullptr) return LLA_ERR_INVALID_ARG;
  if (layer < 0 || layer >= d->D || loop < 0 || loop >= d->T) return LLA_ERR_INVALID_ARG;
  if (n_new < 0 || pos_start < 0 || static_cast<long long>(pos_start) + n_new > d->n_max)
    return LLA_ERR_INVALID_ARG;
  if (proj->d_model < 32 || proj->d_model % 32 != 0) return LLA_ERR_INVALID_ARG;
  const void* ptrs[] = {h, acc, proj->w_k, proj->w_v, codec->w_down_k_t, codec->w_down_v_t,
                        codec->mu_k, codec->mu_v, cache->c_k, cache->c_v};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return LLA_ERR_INVALID_ARG;
  if (!lla::encode_fused_supported(d->dtype, d->d_head, d->r_k) ||
      !lla::encode_fused_supported(d->dtype, d->d_head, d->r_v))
    return LLA_ERR_UNSUPPORTED;
  // token and weight offsets inside the kernel are 32-bit per row block
  if (static_cast<long long>(d->batch) * n_new >= (1LL << 31) - 256) return LLA_ERR_UNSUPPORTED;
  if (static_cast<long long>(proj->d_model) * d->H * d->d_head >= (1LL << 31))
    return LLA_ERR_UNSUPPORTED;
  if (n_new == 0) return LLA_OK;
  if (acc_bytes < lla_encode_fused_acc_bytes(d, n_new)) return LLA_ERR_WORKSPACE;
  const int Hc = latent_heads(*d);
  const int din = d_in(*d);
  const size_t K = static_cast<size_t>(d->T) * din;
  const size_t es = elem_bytes(*d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int rs[2] = {d->r_k, d->r_v};
  const void* wps[2] = {proj->w_k, proj->w_v};
  const void* wds[2] = {codec->w_down_k_t, codec->w_down_v_t};
  const void* mus[2] = {codec->mu_k, codec->mu_v};
  void* cs[2] = {cache->c_k, cache->c_v};
  lla::FusedArgs fa[2];
  for (int ax = 0; ax < 2; ++ax) {
    const int r = rs[ax];
    lla::FusedArgs& a = fa[ax];
    a.h = h;
    a.w_proj = static_cast<const char*>(wps[ax]) +
               static_cast<size_t>(layer) * proj->d_model * d->H * d->d_head * es;
    a.w_down_t = static_cast<const char*>(wds[ax]) + static_cast<size_t>(layer) * Hc * r * K * es;
    a.mu = static_cast<const char*>(mus[ax]) + static_cast<size_t>(layer) * Hc * K * es;
    a.c = static_cast<char*>(cs[ax]) +
          static_cast<size_t>(layer) * d->batch * Hc * static_cast<size_t>(d->n_max) * r * es;
    a.acc = acc;
    a.Ntok = d->batch * n_new;
    a.n_new = n_new;
    a.pos_start = pos_start;
    a.n_max = d->n_max;
    a.H = d->H;
    a.Hc = Hc;
    a.T = d->T;
    a.d_in = din;
    a.d_model = proj->d_model;
    a.loop = loop;
    a.RT = d->r_k + d->r_v;
    a.ao = ax == 0 ? 0 : d->r_k;
  }
  const bool per_head = d->variant == LLA_PER_HEAD;
  if (per_head && lla::encode_fused_kv_supported(d->r_k, d->r_v, proj->d_model)) {
    if (!lla::launch_encode_fused_kv(d->r_k, d->r_v, fa[0], fa[1], s)) return LLA_ERR_UNSUPPORTED;
  } else {
    for (int ax = 0; ax < 2; ++ax)
      if (!lla::launch_encode_fused(rs[ax], fa[ax], per_head, s)) return LLA_ERR_UNSUPPORTED;
  }
  return hip_status();
}

int32_t lla_decode_num_splits(const lla_dims* d, int32_t n_ctx, int32_t loop_count,
                              const lla_decode_opts* opts) {
  if (check_dims(d) != LLA_OK || n_ctx < 0 || loop_count < 1) return 0;
  return plan_splits(*d, n_ctx, loop_count, opts).S;
}

size_t lla_decode_workspace_bytes(const lla_dims* d, int32_t n_ctx, int32_t loop_count,
                                  const lla_decode_opts* opts) {
  if (check_dims(d) != LLA_OK || n_ctx < 0 || n_ctx > d->n_max || loop_count < 1) return 0;
  const Plan p = plan_splits(*d, n_ctx, loop_count, opts);
  const size_t bytes = static_cast<size_t>(d->batch) * d->H * loop_count * p.S * (2 + d->r_v) * 4;
  return (bytes + 255) / 256 * 256;
}

}  // extern "C"

// Every check of lla_decode_attn except those of the workspace; host-side only.
int32_t lla::check_decode_args(const lla_dims* d, const lla_codec* codec, const lla_cache* cache,
                               int32_t layer, int32_t n_ctx, const int32_t* ctx_lens,
                               const float* q, int32_t loop_begin, int32_t loop_count,
                               const float* out, const lla_decode_opts* opts) {
  const int32_t st = check_dims(d);
  if (st != LLA_OK) return st;
  if (codec == nullptr || cache == nullptr) return LLA_ERR_INVALID_ARG;
  if (layer < 0 || layer >= d->D) return LLA_ERR_INVALID_ARG;
  if (n_ctx < 0 || n_ctx > d->n_max) return LLA_ERR_INVALID_ARG;
  if (loop_begin < 0 || loop_count < 1 || static_cast<long long>(loop_begin) + loop_count > d->T)
    return LLA_ERR_INVALID_ARG;
  if (opts != nullptr && (opts->num_splits < 0 || opts->path < LLA_PATH_AUTO ||
                          opts->path > LLA_PATH_ROTARY_FOLD))
    return LLA_ERR_INVALID_ARG;
  const void* ptrs[] = {codec->mu_k, codec->w_up_k, codec->mu_v, codec->w_up_v, codec->rope_table,
                        cache->c_k, cache->c_v, q, out};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return LLA_ERR_INVALID_ARG;
  if (ctx_lens != nullptr && (reinterpret_cast<uintptr_t>(ctx_lens) & 3u) != 0) return LLA_ERR_INVALID_ARG;
  const int path = resolve_path(*d, opts);
  if (path == LLA_PATH_ROTARY_FOLD) {
    if (!fold_ok(*d)) return LLA_ERR_UNSUPPORTED;
  } else if (!lla::decode_reconstruct_supported(d->dtype, d->d_head, d->r_k, d->r_v)) {
    return LLA_ERR_UNSUPPORTED;
  }
  return LLA_OK;
}

extern "C" {

int32_t lla_decode_attn(const lla_dims* d, const lla_codec* codec, const lla_cache* cache,
                        int32_t layer, int32_t n_ctx, const int32_t* ctx_lens, const float* q,
                        int32_t loop_begin, int32_t loop_count, float* out, void* workspace,
                        size_t workspace_bytes, const lla_decode_opts* opts, void* stream) {
  int32_t st = lla::check_decode_args(d, codec, cache, layer, n_ctx, ctx_lens, q, loop_begin,
                                      loop_count, out, opts);
  if (st != LLA_OK) return st;
  if (workspace == nullptr || !aligned16(workspace)) return LLA_ERR_INVALID_ARG;
  if (workspace_bytes < lla_decode_workspace_bytes(d, n_ctx, loop_count, opts)) return LLA_ERR_WORKSPACE;
  const int path = resolve_path(*d, opts);

  const Plan p = plan_splits(*d, n_ctx, loop_count, opts);
  const size_t es = elem_bytes(*d);
  const int Hc = latent_heads(*d);
  const int K = d->T * d_in(*d);
  lla::DecodeArgs a;
  a.c_k = static_cast<const char*>(cache->c_k) +
          static_cast<size_t>(layer) * d->batch * Hc * static_cast<size_t>(d->n_max) * d->r_k * es;
  a.c_v = static_cast<const char*>(cache->c_v) +
          static_cast<size_t>(layer) * d->batch * Hc * static_cast<size_t>(d->n_max) * d->r_v * es;
  a.w_up_k = static_cast<const char*>(codec->w_up_k) +
             static_cast<size_t>(layer) * d->T * d->H * d->d_head * d->r_k * es;
  a.w_up_v = static_cast<const char*>(codec->w_up_v) +
             static_cast<size_t>(layer) * d->T * d->H * d->d_head * d->r_v * es;
  a.mu_k = static_cast<const char*>(codec->mu_k) + static_cast<size_t>(layer) * Hc * K * es;
  a.mu_v = static_cast<const char*>(codec->mu_v) + static_cast<size_t>(layer) * Hc * K * es;
  a.rope32 = static_cast<const float*>(codec->rope_table);
  a.rope16 = reinterpret_cast<const uint16_t*>(static_cast<const char*>(codec->rope_table) +
                                               static_cast<size_t>(d->n_max) * d->d_head * 4);
  a.q = q;
  a.ctx_lens = ctx_lens;
  a.part = static_cast<float*>(workspace);
  a.out = out;
  a.B = d->batch;
  a.H = d->H;
  a.Hc = Hc;
  a.T = d->T;
  a.L = loop_count;
  a.loop_begin = loop_begin;
  a.n_max = d->n_max;
  a.n_ctx = n_ctx;
  a.S = p.S;
  a.split_len = p.split_len;
  a.variant = d->variant;
  const double scale = d->scale > 0.f ? d->scale : 1.0 / std::sqrt(static_cast<double>(d->d_head));
  a.scale_log2e = static_cast<float>(scale * kLog2e);

  hipStream_t s = static_cast<hipStream_t>(stream);
  bool ok;
  if (path == LLA_PATH_ROTARY_FOLD) {
    ok = fold_kind(*d) == kFoldNarrow
             ? lla::launch_decode_rotary_fold(d->dtype, d->d_head, d->r_k, d->r_v, a, s)
             : (d->variant == LLA_2D &&
                lla::launch_decode_lla2d(d->dtype, d->d_head, d->r_k, d->r_v, a, s)) ||
                   lla::launch_decode_fold_wide(d->dtype, d->d_head, d->r_k, d->r_v,
                                                d->variant == LLA_2D, a, s);
  } else {
    ok = lla::launch_decode_reconstruct(d->dtype, d->d_head, d->r_k, d->r_v, a, s);
  }
  if (!ok) return LLA_ERR_UNSUPPORTED;
  st = hip_status();
  if (st != LLA_OK) return st;
  // The rotary-fold kernel finishes a single split itself (value up-projection in its
  // epilogue); everything else goes through the split merge.
  if (path == LLA_PATH_ROTARY_FOLD && p.S == 1) return LLA_OK;
  if (!lla::launch_combine(d->dtype, d->d_head, d->r_v, a, s)) return LLA_ERR_UNSUPPORTED;
  return hip_status();
}

size_t lla_decode_absorbed_workspace_bytes(const lla_dims* d, int32_t d_rope, int32_t n_ctx,
                                           int32_t loop_count, const lla_decode_opts* opts) {
  if (check_dims(d) != LLA_OK || n_ctx < 0 || n_ctx > d->n_max || loop_count < 1) return 0;
  if (d_rope < 16 || d_rope >= d->d_head || d_rope % 16 != 0) return 0;
  const Plan p = plan_absorbed(*d, n_ctx, loop_count, opts);
  const size_t part = static_cast<size_t>(d->batch) * d->H * loop_count * p.S * (2 + d->r_v) * 4;
  return (part + 255) / 256 * 256;
}

int32_t lla_decode_absorbed_supported(const lla_dims* d, int32_t d_rope) {
  if (check_dims(d) != LLA_OK) return 0;
  return lla::decode_absorbed_supported(d->dtype, d->d_head, d->r_k, d->r_v, d_rope) ? 1 : 0;
}

}  // extern "C"

namespace {

// Dense (pages == nullptr) and paged absorbed decode: validation, launch arguments, the
// kernel and the split merge.
int32_t absorbed_call(const lla_dims* d, const lla_codec* codec, const lla_cache* cache,
                      const lla_pages* pages, const void* k_rope, int32_t d_rope, int32_t layer,
                      int32_t n_ctx, const int32_t* ctx_lens, const float* q, int32_t loop_begin,
                      int32_t loop_count, float* out, void* workspace, size_t workspace_bytes,
                      const lla_decode_opts* opts, void* stream) {
  int32_t st = check_dims(d);
  if (st != LLA_OK) return st;
  if (pages != nullptr) {
    st = check_pages(*d, pages);
    if (st != LLA_OK) return st;
  }
  if (codec == nullptr || cache == nullptr) return LLA_ERR_INVALID_ARG;
  if (layer < 0 || layer >= d->D) return LLA_ERR_INVALID_ARG;
  if (n_ctx < 0 || n_ctx > d->n_max) return LLA_ERR_INVALID_ARG;
  if (loop_begin < 0 || loop_count < 1 || static_cast<long long>(loop_begin) + loop_count > d->T)
    return LLA_ERR_INVALID_ARG;
  if (d_rope < 16 || d_rope >= d->d_head || d_rope % 16 != 0) return LLA_ERR_INVALID_ARG;
  if (opts != nullptr && opts->num_splits < 0) return LLA_ERR_INVALID_ARG;
  const void* ptrs[] = {codec->mu_k, codec->w_up_k, codec->mu_v, codec->w_up_v,
                        cache->c_k, cache->c_v, k_rope, q, out, workspace};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return LLA_ERR_INVALID_ARG;
  if (ctx_lens != nullptr && (reinterpret_cast<uintptr_t>(ctx_lens) & 3u) != 0) return LLA_ERR_INVALID_ARG;
  if (!lla::decode_absorbed_supported(d->dtype, d->d_head, d->r_k, d->r_v, d_rope))
    return LLA_ERR_UNSUPPORTED;
  if (static_cast<long long>(d->n_max) * d_rope >= (1LL << 31)) return LLA_ERR_UNSUPPORTED;
  const size_t need = pages ? lla_decode_absorbed_paged_workspace_bytes(d, d_rope, n_ctx, loop_count, opts)
                            : lla_decode_absorbed_workspace_bytes(d, d_rope, n_ctx, loop_count, opts);
  if (workspace_bytes < need) return LLA_ERR_WORKSPACE;

  const Plan p = pages ? plan_absorbed_paged(*d, n_ctx, loop_count, opts)
                       : plan_absorbed(*d, n_ctx, loop_count, opts);
  const size_t es = elem_bytes(*d);
  const int Hc = latent_heads(*d);
  const int K = d->T * d_in(*d);
  // rows per layer: dense, batch x Hc planes of n_max rows; paged, the pool's pages
  const size_t lrows = pages ? static_cast<size_t>(pages->num_pages) * Hc * lla::kPage
                             : static_cast<size_t>(d->batch) * Hc * d->n_max;
  const size_t rrows = pages ? static_cast<size_t>(pages->num_pages) * d->H * lla::kPage
                             : static_cast<size_t>(d->batch) * d->H * d->n_max;
  lla::DecodeArgs a;
  a.c_k = static_cast<const char*>(cache->c_k) + static_cast<size_t>(layer) * lrows * d->r_k * es;
  a.c_v = static_cast<const char*>(cache->c_v) + static_cast<size_t>(layer) * lrows * d->r_v * es;
  a.w_up_k = static_cast<const char*>(codec->w_up_k) +
             static_cast<size_t>(layer) * d->T * d->H * d->d_head * d->r_k * es;
  a.w_up_v = static_cast<const char*>(codec->w_up_v) +
             static_cast<size_t>(layer) * d->T * d->H * d->d_head * d->r_v * es;
  a.mu_k = static_cast<const char*>(codec->mu_k) + static_cast<size_t>(layer) * Hc * K * es;
  a.mu_v = static_cast<const char*>(codec->mu_v) + static_cast<size_t>(layer) * Hc * K * es;
  a.rope32 = nullptr;
  a.rope16 = nullptr;
  a.q = q;
  a.ctx_lens = ctx_lens;
  a.part = static_cast<float*>(workspace);
  a.out = out;
  a.B = d->batch;
  a.H = d->H;
  a.Hc = Hc;
  a.T = d->T;
  a.L = loop_count;
  a.loop_begin = loop_begin;
  a.n_max = d->n_max;
  a.n_ctx = n_ctx;
  a.S = p.S;
  a.split_len = p.split_len;
  a.variant = d->variant;
  const double scale = d->scale > 0.f ? d->scale : 1.0 / std::sqrt(static_cast<double>(d->d_head));
  a.scale_log2e = static_cast<float>(scale * kLog2e);
  const char* kr = static_cast<const char*>(k_rope) + static_cast<size_t>(layer) * rrows * d_rope * es;

  hipStream_t s = static_cast<hipStream_t>(stream);
  bool ok;
  if (pages != nullptr) {
    const lla::PageArgs pg{pages->block_table, pages->max_blocks, pages->num_pages};
    ok = lla::launch_decode_absorbed_paged(d->dtype, d->d_head, d->r_k, d->r_v, d_rope, a, kr, pg, s);
  } else {
    ok = lla::launch_decode_absorbed(d->dtype, d->d_head, d->r_k, d->r_v, d_rope, a, kr, s);
  }
  if (!ok) return LLA_ERR_UNSUPPORTED;
  st = hip_status();
  if (st != LLA_OK) return st;
  if (p.S == 1) return LLA_OK;  // the kernel finished the single split itself
  if (!lla::launch_combine(d->dtype, d->d_head, d->r_v, a, s)) return LLA_ERR_UNSUPPORTED;
  return hip_status();
}

}  // namespace

extern "C" {

int32_t lla_decode_attn_absorbed(const lla_dims* d, const lla_codec* codec, const lla_cache* cache,
                                 const void* k_rope, int32_t d_rope, int32_t layer, int32_t n_ctx,
                                 const int32_t* ctx_lens, const float* q, int32_t loop_begin,
                                 int32_t loop_count, float* out, void* workspace,
                                 size_t workspace_bytes, const lla_decode_opts* opts, void* stream) {
  return absorbed_call(d, codec, cache, nullptr, k_rope, d_rope, layer, n_ctx, ctx_lens, q,
                       loop_begin, loop_count, out, workspace, workspace_bytes, opts, stream);
}

size_t lla_decode_absorbed_paged_workspace_bytes(const lla_dims* d, int32_t d_rope, int32_t n_ctx,
                                                 int32_t loop_count, const lla_decode_opts* opts) {
  if (check_dims(d) != LLA_OK || n_ctx < 0 || n_ctx > d->n_max || loop_count < 1) return 0;
  if (d_rope < 16 || d_rope >= d->d_head || d_rope % 16 != 0) return 0;
  const Plan p = plan_absorbed_paged(*d, n_ctx, loop_count, opts);
  const size_t part = static_cast<size_t>(d->batch) * d->H * loop_count * p.S * (2 + d->r_v) * 4;
  return (part + 255) / 256 * 256;
}

int32_t lla_decode_attn_absorbed_paged(const lla_dims* d, const lla_codec* codec,
                                       const lla_cache* cache, const lla_pages* pages,
                                       const void* k_rope, int32_t d_rope, int32_t layer,
                                       int32_t n_ctx, const int32_t* ctx_lens, const float* q,
                                       int32_t loop_begin, int32_t loop_count, float* out,
                                       void* workspace, size_t workspace_bytes,
                                       const lla_decode_opts* opts, void* stream) {
  if (pages == nullptr) return LLA_ERR_INVALID_ARG;
  return absorbed_call(d, codec, cache, pages, k_rope, d_rope, layer, n_ctx, ctx_lens, q,
                       loop_begin, loop_count, out, workspace, workspace_bytes, opts, stream);
}

size_t lla_decode_teacher_workspace_bytes(const lla_dims* d, int32_t n_ctx, int32_t loop_count,
                                          const lla_decode_opts* opts) {
  if (check_teacher_dims(d) != LLA_OK || n_ctx < 0 || n_ctx > d->n_max || loop_count < 1) return 0;
  const Plan p = plan_teacher(*d, n_ctx, loop_count, opts);
  if (p.S == 1) return 0;  // a single split writes the output itself
  const size_t part = static_cast<size_t>(d->batch) * d->H * loop_count * p.S * (2 + d->d_head) * 4;
  return (part + 255) / 256 * 256;
}

int32_t lla_decode_teacher_supported(const lla_dims* d) {
  return check_teacher_dims(d) == LLA_OK ? 1 : 0;
}

int32_t lla_decode_teacher_num_splits(const lla_dims* d, int32_t n_ctx, int32_t loop_count,
                                      const lla_decode_opts* opts) {
  if (check_teacher_dims(d) != LLA_OK || n_ctx < 0 || n_ctx > d->n_max || loop_count < 1) return 0;
  return plan_teacher(*d, n_ctx, loop_count, opts).S;
}

int32_t lla_decode_attn_teacher(const lla_dims* d, const void* k_cache, const void* v_cache,
                                int32_t layer, int32_t n_ctx, const int32_t* ctx_lens,
                                const float* q, int32_t loop_begin, int32_t loop_count,
                                float* out, void* workspace, size_t workspace_bytes,
                                const lla_decode_opts* opts, void* stream) {
  int32_t st = check_teacher_dims(d);
  if (st != LLA_OK) return st;
  if (layer < 0 || layer >= d->D) return LLA_ERR_INVALID_ARG;
  if (n_ctx < 0 || n_ctx > d->n_max) return LLA_ERR_INVALID_ARG;
  if (loop_begin < 0 || loop_count < 1 || static_cast<long long>(loop_begin) + loop_count > d->T)
    return LLA_ERR_INVALID_ARG;
  if (opts != nullptr && opts->num_splits < 0) return LLA_ERR_INVALID_ARG;
  const void* ptrs[] = {k_cache, v_cache, q, out};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return LLA_ERR_INVALID_ARG;
  if (ctx_lens != nullptr && (reinterpret_cast<uintptr_t>(ctx_lens) & 3u) != 0) return LLA_ERR_INVALID_ARG;
  const size_t need = lla_decode_teacher_workspace_bytes(d, n_ctx, loop_count, opts);
  if (need > 0 && (workspace == nullptr || !aligned16(workspace))) return LLA_ERR_INVALID_ARG;
  if (workspace_bytes < need) return LLA_ERR_WORKSPACE;

  const Plan p = plan_teacher(*d, n_ctx, loop_count, opts);
  const size_t es = elem_bytes(*d);
  const size_t layer_elems = static_cast<size_t>(d->T) * d->batch * d->H *
                             static_cast<size_t>(d->n_max) * d->d_head;
  lla::DecodeArgs a{};
  a.c_k = static_cast<const char*>(k_cache) + static_cast<size_t>(layer) * layer_elems * es;
  a.c_v = static_cast<const char*>(v_cache) + static_cast<size_t>(layer) * layer_elems * es;
  a.q = q;
  a.ctx_lens = ctx_lens;
  a.part = static_cast<float*>(workspace);
  a.out = out;
  a.B = d->batch;
  a.H = d->H;
  a.Hc = d->H;
  a.T = d->T;
  a.L = loop_count;
  a.loop_begin = loop_begin;
  a.n_max = d->n_max;
  a.n_ctx = n_ctx;
  a.S = p.S;
  a.split_len = p.split_len;
  const double scale = d->scale > 0.f ? d->scale : 1.0 / std::sqrt(static_cast<double>(d->d_head));
  a.scale_log2e = static_cast<float>(scale * kLog2e);

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!lla::launch_decode_teacher(d->dtype, d->d_head, a, s)) return LLA_ERR_UNSUPPORTED;
  st = hip_status();
  if (st != LLA_OK) return st;
  if (p.S == 1) return LLA_OK;
  if (!lla::launch_combine_identity(d->dtype, d->d_head, a, s)) return LLA_ERR_UNSUPPORTED;
  return hip_status();
}

int32_t lla_reconstruct(const lla_dims* d, const lla_codec* codec, const lla_cache* cache,
                        int32_t layer, int32_t loop_begin, int32_t loop_count, int32_t pos_start,
                        int32_t n_tok, void* k_out, void* v_out, void* stream) {
  const int32_t st = check_dims(d);
  if (st != LLA_OK) return st;
  if (codec == nullptr || cache == nullptr) return LLA_ERR_INVALID_ARG;
  if (layer < 0 || layer >= d->D) return LLA_ERR_INVALID_ARG;
  if (loop_begin < 0 || loop_count < 1 || static_cast<long long>(loop_begin) + loop_count > d->T)
    return LLA_ERR_INVALID_ARG;
  if (pos_start < 0 || n_tok < 0 || static_cast<long long>(pos_start) + n_tok > d->n_max)
    return LLA_ERR_INVALID_ARG;
  if (k_out == nullptr && v_out == nullptr) return LLA_ERR_INVALID_ARG;
  if (k_out != nullptr) {
    const void* ptrs[] = {codec->w_up_k, codec->mu_k, codec->rope_table, cache->c_k, k_out};
    for (const void* p : ptrs)
      if (p == nullptr || !aligned16(p)) return LLA_ERR_INVALID_ARG;
    if (!lla::reconstruct_supported(d->dtype, d->d_head, d->r_k)) return LLA_ERR_UNSUPPORTED;
  }
  if (v_out != nullptr) {
    const void* ptrs[] = {codec->w_up_v, codec->mu_v, cache->c_v, v_out};
    for (const void* p : ptrs)
      if (p == nullptr || !aligned16(p)) return LLA_ERR_INVALID_ARG;
    if (!lla::reconstruct_supported(d->dtype, d->d_head, d->r_v)) return LLA_ERR_UNSUPPORTED;
  }
  if (n_tok == 0) return LLA_OK;

  const size_t es = elem_bytes(*d);
  const int Hc = latent_heads(*d);
  const int K = d->T * d_in(*d);
  const size_t loop_elems = static_cast<size_t>(d->batch) * d->H * d->n_max * d->d_head;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int axis = 0; axis < 2; ++axis) {
    void* out = axis == 0 ? k_out : v_out;
    if (out == nullptr) continue;
    const int r = axis == 0 ? d->r_k : d->r_v;
    lla::ReconArgs a{};
    a.c = static_cast<const char*>(axis == 0 ? cache->c_k : cache->c_v) +
          static_cast<size_t>(layer) * d->batch * Hc * static_cast<size_t>(d->n_max) * r * es;
    a.w_up = static_cast<const char*>(axis == 0 ? codec->w_up_k : codec->w_up_v) +
             static_cast<size_t>(layer) * d->T * d->H * d->d_head * r * es;
    a.mu = static_cast<const char*>(axis == 0 ? codec->mu_k : codec->mu_v) +
           static_cast<size_t>(layer) * Hc * K * es;
    a.rope32 = axis == 0 ? static_cast<const float*>(codec->rope_table) : nullptr;
    a.B = d->batch;
    a.H = d->H;
    a.Hc = Hc;
    a.T = d->T;
    a.n_max = d->n_max;
    a.pos_start = pos_start;
    a.n_tok = n_tok;
    a.variant = d->variant;
    // Slots per workgroup: long chunks (up to 1024) amortise each wave's W_up load and keep
    // its stores streaming; shorter ones keep about 1024 workgroups for short ranges.
    const long long per_wg = static_cast<long long>(n_tok) * d->batch * d->H / 1024;
    const long long chunk = (per_wg + 15) / 16 * 16;
    a.chunk = static_cast<int>(chunk < 64 ? 64 : (chunk > 1024 ? 1024 : chunk));
    const int max_l = lla::reconstruct_max_loops(d->dtype, d->d_head, r);
    if (max_l < 1) return LLA_ERR_UNSUPPORTED;
    for (int lb = 0; lb < loop_count; lb += max_l) {
      a.L = loop_count - lb < max_l ? loop_count - lb : max_l;
      a.loop_begin = loop_begin + lb;
      a.out = static_cast<char*>(out) + static_cast<size_t>(lb) * loop_elems * es;
      if (!lla::launch_reconstruct(d->dtype, d->d_head, r, a, s)) return LLA_ERR_UNSUPPORTED;
      const int32_t hs = hip_status();
      if (hs != LLA_OK) return hs;
    }
  }
  return LLA_OK;
}

int32_t lla_encode_paged(const lla_dims* d, const lla_codec* codec, const lla_cache* cache,
                         const lla_pages* pages, int32_t layer, const void* x_k, const void* x_v,
                         int32_t pos_start, int32_t n_new, void* stream) {
  int32_t st = check_dims(d);
  if (st != LLA_OK) return st;
  st = check_pages(*d, pages);
  if (st != LLA_OK) return st;
  if (codec == nullptr || cache == nullptr) return LLA_ERR_INVALID_ARG;
  if (layer < 0 || layer >= d->D) return LLA_ERR_INVALID_ARG;
  if (n_new < 0 || pos_start < 0 || static_cast<long long>(pos_start) + n_new > d->n_max)
    return LLA_ERR_INVALID_ARG;
  const void* ptrs[] = {x_k, x_v, codec->w_down_k_t, codec->w_down_v_t, codec->mu_k, codec->mu_v,
                        cache->c_k, cache->c_v};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return LLA_ERR_INVALID_ARG;
  const int Hc = latent_heads(*d);
  const int K = d->T * d_in(*d);
  if (!lla::encode_supported(d->dtype, d->r_k, K) || !lla::encode_supported(d->dtype, d->r_v, K))
    return LLA_ERR_UNSUPPORTED;
  if (n_new == 0) return LLA_OK;
  if (static_cast<long long>(d->batch) * n_new >= (1LL << 31) - 64) return LLA_ERR_UNSUPPORTED;
  const size_t es = elem_bytes(*d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const lla::PageArgs pg{pages->block_table, pages->max_blocks, pages->num_pages};
  const int rs[2] = {d->r_k, d->r_v};
  const void* xs[2] = {x_k, x_v};
  const void* wds[2] = {codec->w_down_k_t, codec->w_down_v_t};
  const void* mus[2] = {codec->mu_k, codec->mu_v};
  void* cs[2] = {cache->c_k, cache->c_v};
  for (int ax = 0; ax < 2; ++ax) {
    const int r = rs[ax];
    lla::EncodeArgs a;
    a.x = xs[ax];
    a.w_down_t = static_cast<const char*>(wds[ax]) + static_cast<size_t>(layer) * Hc * r * K * es;
    a.mu = static_cast<const char*>(mus[ax]) + static_cast<size_t>(layer) * Hc * K * es;
    a.c = static_cast<char*>(cs[ax]) +
          static_cast<size_t>(layer) * pages->num_pages * Hc * static_cast<size_t>(lla::kPage) * r * es;
    a.B = d->batch;
    a.Hc = Hc;
    a.Kdim = K;
    a.n_new = n_new;
    a.pos_start = pos_start;
    a.n_max = d->n_max;
    if (!lla::launch_encode_paged(d->dtype, r, a, pg, s)) return LLA_ERR_UNSUPPORTED;
  }
  return hip_status();
}

size_t lla_decode_paged_workspace_bytes(const lla_dims* d, int32_t n_ctx, int32_t loop_count,
                                        const lla_decode_opts* opts) {
  if (check_dims(d) != LLA_OK || n_ctx < 0 || n_ctx > d->n_max || loop_count < 1) return 0;
  const Plan p = plan_paged(*d, n_ctx, loop_count, opts);
  const size_t bytes = static_cast<size_t>(d->batch) * d->H * loop_count * p.S * (2 + d->r_v) * 4;
  return (bytes + 255) / 256 * 256;
}

int32_t lla_decode_paged_num_splits(const lla_dims* d, int32_t n_ctx, int32_t loop_count,
                                    const lla_decode_opts* opts) {
  if (check_dims(d) != LLA_OK || n_ctx < 0 || n_ctx > d->n_max || loop_count < 1) return 0;
  return plan_paged(*d, n_ctx, loop_count, opts).S;
}

int32_t lla_decode_attn_paged(const lla_dims* d, const lla_codec* codec, const lla_cache* cache,
                              const lla_pages* pages, int32_t layer, int32_t n_ctx,
                              const int32_t* ctx_lens, const float* q, int32_t loop_begin,
                              int32_t loop_count, float* out, void* workspace,
                              size_t workspace_bytes, const lla_decode_opts* opts, void* stream) {
  int32_t st = check_dims(d);
  if (st != LLA_OK) return st;
  st = check_pages(*d, pages);
  if (st != LLA_OK) return st;
  if (codec == nullptr || cache == nullptr) return LLA_ERR_INVALID_ARG;
  if (layer < 0 || layer >= d->D) return LLA_ERR_INVALID_ARG;
  if (n_ctx < 0 || n_ctx > d->n_max) return LLA_ERR_INVALID_ARG;
  if (loop_begin < 0 || loop_count < 1 || static_cast<long long>(loop_begin) + loop_count > d->T)
    return LLA_ERR_INVALID_ARG;
  if (opts != nullptr && (opts->num_splits < 0 || opts->path < LLA_PATH_AUTO ||
                          opts->path > LLA_PATH_ROTARY_FOLD))
    return LLA_ERR_INVALID_ARG;
  const void* ptrs[] = {codec->mu_k, codec->w_up_k, codec->mu_v, codec->w_up_v, codec->rope_table,
                        cache->c_k, cache->c_v, q, out, workspace};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return LLA_ERR_INVALID_ARG;
  if (ctx_lens != nullptr && (reinterpret_cast<uintptr_t>(ctx_lens) & 3u) != 0) return LLA_ERR_INVALID_ARG;
  const int path = paged_path(*d, opts);
  if (path < 0) return LLA_ERR_UNSUPPORTED;
  if (path == LLA_PATH_RECONSTRUCT &&
      !lla::decode_reconstruct_supported(d->dtype, d->d_head, d->r_k, d->r_v))
    return LLA_ERR_UNSUPPORTED;
  if (workspace_bytes < lla_decode_paged_workspace_bytes(d, n_ctx, loop_count, opts))
    return LLA_ERR_WORKSPACE;

  const Plan p = plan_paged(*d, n_ctx, loop_count, opts);
  const size_t es = elem_bytes(*d);
  const int Hc = latent_heads(*d);
  const int K = d->T * d_in(*d);
  const size_t pool_rows = static_cast<size_t>(pages->num_pages) * Hc * lla::kPage;
  lla::DecodeArgs a;
  a.c_k = static_cast<const char*>(cache->c_k) + static_cast<size_t>(layer) * pool_rows * d->r_k * es;
  a.c_v = static_cast<const char*>(cache->c_v) + static_cast<size_t>(layer) * pool_rows * d->r_v * es;
  a.w_up_k = static_cast<const char*>(codec->w_up_k) +
             static_cast<size_t>(layer) * d->T * d->H * d->d_head * d->r_k * es;
  a.w_up_v = static_cast<const char*>(codec->w_up_v) +
             static_cast<size_t>(layer) * d->T * d->H * d->d_head * d->r_v * es;
  a.mu_k = static_cast<const char*>(codec->mu_k) + static_cast<size_t>(layer) * Hc * K * es;
  a.mu_v = static_cast<const char*>(codec->mu_v) + static_cast<size_t>(layer) * Hc * K * es;
  a.rope32 = static_cast<const float*>(codec->rope_table);
  a.rope16 = reinterpret_cast<const uint16_t*>(static_cast<const char*>(codec->rope_table) +
                                               static_cast<size_t>(d->n_max) * d->d_head * 4);
  a.q = q;
  a.ctx_lens = ctx_lens;
  a.part = static_cast<float*>(workspace);
  a.out = out;
  a.B = d->batch;
  a.H = d->H;
  a.Hc = Hc;
  a.T = d->T;
  a.L = loop_count;
  a.loop_begin = loop_begin;
  a.n_max = d->n_max;
  a.n_ctx = n_ctx;
  a.S = p.S;
  a.split_len = p.split_len;
  a.variant = d->variant;
  const double scale = d->scale > 0.f ? d->scale : 1.0 / std::sqrt(static_cast<double>(d->d_head));
  a.scale_log2e = static_cast<float>(scale * kLog2e);
  const lla::PageArgs pg{pages->block_table, pages->max_blocks, pages->num_pages};

  hipStream_t s = static_cast<hipStream_t>(stream);
  bool ok;
  if (path == LLA_PATH_ROTARY_FOLD) {
    ok = fold_kind(*d) == kFoldNarrow
             ? lla::launch_decode_rotary_fold_paged(d->dtype, d->d_head, d->r_k, d->r_v, a, pg, s)
             : (d->variant == LLA_2D &&
                lla::launch_decode_lla2d_paged(d->dtype, d->d_head, d->r_k, d->r_v, a, pg, s)) ||
                   lla::launch_decode_fold_wide_paged(d->dtype, d->d_head, d->r_k, d->r_v,
                                                      d->variant == LLA_2D, a, pg, s);
  } else {
    ok = lla::launch_decode_reconstruct_paged(d->dtype, d->d_head, d->r_k, d->r_v, a, pg, s);
  }
  if (!ok) return LLA_ERR_UNSUPPORTED;
  st = hip_status();
  if (st != LLA_OK) return st;
  if (path == LLA_PATH_ROTARY_FOLD && p.S == 1) return LLA_OK;
  if (!lla::launch_combine(d->dtype, d->d_head, d->r_v, a, s)) return LLA_ERR_UNSUPPORTED;
  return hip_status();
}

}  // extern "C"
