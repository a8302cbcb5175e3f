// Launch planning of the decode entry points: which kernel runs a call and how many
// context splits it uses. Included by lla_api.cpp only (its functions are file-local).
#pragma once

#include "lla.h"
#include "lla_kernels.h"

namespace {

struct Plan {
  int S;
  int split_len;
};

int waves_per_unit(const lla_dims& d, const lla_decode_opts* opts);

// Context splits: enough (sequence, head, loop, split) waves to fill the GPU, counting the
// waves the chosen kernel spends per head.
Plan plan_splits(const lla_dims& d, int n_ctx, int loop_count, const lla_decode_opts* opts) {
  Plan p{1, 16};
  if (n_ctx <= 0) return p;
  const long long units = static_cast<long long>(d.batch) * d.H * loop_count * waves_per_unit(d, opts);
  long long S;
  if (opts != nullptr && opts->num_splits > 0) {
    S = opts->num_splits;
  } else {
    const long long target = 2048;  // waves in flight wanted across 256 CUs
    S = (target + units - 1) / units;
    const long long max_by_len = (n_ctx + 255) / 256;  // keep splits >= 256 tokens
    if (S > max_by_len) S = max_by_len;
  }
  if (S < 1) S = 1;
  long long len = (n_ctx + S - 1) / S;
  len = (len + 15) / 16 * 16;
  p.split_len = static_cast<int>(len);
  p.S = static_cast<int>((n_ctx + len - 1) / len);
  return p;
}

// Rotary-fold kernels: narrow latents (one wave per head) for the per-head codec, and the
// wide kernel (a pair of waves per head) for wide latents and for LLA-2D.
enum FoldKind { kFoldNone = 0, kFoldNarrow = 1, kFoldWide = 2 };

int fold_kind(const lla_dims& d) {
  if (d.dtype != LLA_BF16) return kFoldNone;
  if (d.variant == LLA_PER_HEAD && d.H % lla::kFoldHeadsPerGroup == 0 &&
      lla::decode_rotary_fold_supported(d.dtype, d.d_head, d.r_k, d.r_v))
    return kFoldNarrow;
  if (lla::decode_fold_wide_supported(d.dtype, d.d_head, d.r_k, d.r_v) &&
      d.H % lla::fold_wide_heads_per_group(d.d_head, d.r_k, d.r_v, d.variant == LLA_2D) == 0)
    return kFoldWide;
  return kFoldNone;
}

bool fold_ok(const lla_dims& d) { return fold_kind(d) != kFoldNone; }

int resolve_path(const lla_dims& d, const lla_decode_opts* opts) {
  const int want = opts ? opts->path : LLA_PATH_AUTO;
  if (want == LLA_PATH_AUTO) {
    if (fold_ok(d))
      return LLA_PATH_ROTARY_FOLD;
    return LLA_PATH_RECONSTRUCT;
  }
  return want;
}

// Waves the chosen kernel spends per (sequence, head, loop, split): a pair for the wide
// fold kernel, one for the LLA-2D kernel and the others.
int waves_per_unit(const lla_dims& d, const lla_decode_opts* opts) {
  if (resolve_path(d, opts) == LLA_PATH_ROTARY_FOLD && fold_kind(d) == kFoldWide &&
      !(d.variant == LLA_2D && lla::decode_lla2d_supported(d.dtype, d.d_head, d.r_k, d.r_v, d.H)))
    return lla::fold_wide_waves_per_head();
  return 1;
}

// Absorbed decode: one wave per (sequence, head, loop, split).
Plan plan_absorbed(const lla_dims& d, int n_ctx, int loop_count, const lla_decode_opts* opts) {
  lla_decode_opts o{0, LLA_PATH_RECONSTRUCT};  // one wave per unit, like the reconstruct kernel
  if (opts != nullptr) o.num_splits = opts->num_splits;
  return plan_splits(d, n_ctx, loop_count, &o);
}

// One wave per (sequence, head, loop, split), as the reconstruct kernel.
Plan plan_teacher(const lla_dims& d, int n_ctx, int loop_count, const lla_decode_opts* opts) {
  lla_decode_opts o{0, LLA_PATH_RECONSTRUCT};
  if (opts != nullptr) o.num_splits = opts->num_splits;
  return plan_splits(d, n_ctx, loop_count, &o);  // reads batch and H only on this path
}

}  // namespace
