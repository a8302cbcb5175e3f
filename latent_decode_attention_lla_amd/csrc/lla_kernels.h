// Internal interface between the C ABI (lla_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lla_args.h"
#include "lla_page_args.h"
#include "lla_recon_args.h"

namespace lla {

// Launchers return false when no kernel is built for (dtype, d, r_k, r_v) on that path.
bool launch_decode_reconstruct(int dtype, int d, int r_k, int r_v, const DecodeArgs& a,
                               hipStream_t s);
bool launch_decode_rotary_fold(int dtype, int d, int r_k, int r_v, const DecodeArgs& a,
                               hipStream_t s);
// Paged cache (pg.table non-null): c_k / c_v of the args are the layer's page pools.
bool launch_decode_rotary_fold_paged(int dtype, int d, int r_k, int r_v, const DecodeArgs& a,
                                     const PageArgs& pg, hipStream_t s);
bool launch_decode_fold_wide_paged(int dtype, int d, int r_k, int r_v, bool shared,
                                   const DecodeArgs& a, const PageArgs& pg, hipStream_t s);
bool launch_decode_reconstruct_paged(int dtype, int d, int r_k, int r_v, const DecodeArgs& a,
                                     const PageArgs& pg, hipStream_t s);
bool launch_encode_paged(int dtype, int r, const EncodeArgs& a, const PageArgs& pg, hipStream_t s);
// Wide latents (r_k >= 64): a pair of waves per head; `shared` selects LLA-2D (all heads
// read one latent plane). H must be a multiple of fold_wide_heads_per_group(...).
// LLA-2D decode with the value side on the matrix cores, one wave per head (bfloat16; d 128
// with (r_k, r_v) of (96, 160) or (64, 64), H a multiple of the heads per
// workgroup); where it is not built the wide fold kernel runs LLA-2D.
bool decode_lla2d_supported(int dtype, int d, int r_k, int r_v, int H);
bool launch_decode_lla2d(int dtype, int d, int r_k, int r_v, const DecodeArgs& a, hipStream_t s);
bool launch_decode_lla2d_paged(int dtype, int d, int r_k, int r_v, const DecodeArgs& a,
                               const PageArgs& pg, hipStream_t s);
bool launch_decode_fold_wide(int dtype, int d, int r_k, int r_v, bool shared, const DecodeArgs& a,
                             hipStream_t s);
bool decode_fold_wide_supported(int dtype, int d, int r_k, int r_v);
int fold_wide_heads_per_group(int d, int r_k, int r_v, bool shared);
int fold_wide_waves_per_head();
bool launch_combine(int dtype, int d, int r_v, const DecodeArgs& a, hipStream_t s);
// Decoupled-RoPE absorbed decode: `k_rope` is the layer's rotary-key base.
bool launch_decode_absorbed(int dtype, int d, int r_k, int r_v, int d_rope, const DecodeArgs& a,
                            const void* k_rope, hipStream_t s);
bool decode_absorbed_supported(int dtype, int d, int r_k, int r_v, int d_rope);
// Paged instance: c_k, c_v and k_rope are the layer's pools (a chunk of 16 tokens is one
// page); at most kMaxSplitPages pages per split.
bool launch_decode_absorbed_paged(int dtype, int d, int r_k, int r_v, int d_rope,
                                  const DecodeArgs& a, const void* k_rope, const PageArgs& pg,
                                  hipStream_t s);
// Uncompressed decode: c_k / c_v of the args are the layer's per-loop key and value
// caches [T][B][H][n_max][d]; combine with `project` false merges its partials.
bool launch_decode_teacher(int dtype, int d, const DecodeArgs& a, hipStream_t s);
bool decode_teacher_supported(int dtype, int d);
bool launch_combine_identity(int dtype, int d, const DecodeArgs& a, hipStream_t s);
bool decode_reconstruct_supported(int dtype, int d, int r_k, int r_v);
bool decode_rotary_fold_supported(int dtype, int d, int r_k, int r_v);

// Materialised reconstruction of one axis: a.L loops per launch, at most
// reconstruct_max_loops(d, r) of them.
bool launch_reconstruct(int dtype, int d, int r, const ReconArgs& a, hipStream_t s);
bool reconstruct_supported(int dtype, int d, int r);
int reconstruct_max_loops(int dtype, int d, int r);

bool launch_encode(int dtype, int r, const EncodeArgs& a, hipStream_t s);
// Projection-fused encode of one loop and axis (bfloat16, d 128).
bool encode_fused_supported(int dtype, int d, int r);
bool launch_encode_fused(int r, const FusedArgs& a, bool per_head, hipStream_t s);
// Both axes in one launch (per-head codec; built (r_k, r_v) pairs, d_model a multiple of 64).
bool encode_fused_kv_supported(int r_k, int r_v, int d_model);
bool launch_encode_fused_kv(int r_k, int r_v, const FusedArgs& k, const FusedArgs& v, hipStream_t s);
bool encode_supported(int dtype, int r, int Kdim);

void launch_rope_table(int d, int n_max, double base, float* t32, uint16_t* t16, hipStream_t s);

}  // namespace lla

#include "lla.h"

namespace lla {

// Argument checks of lla_decode_attn other than its workspace (host only; lla_api.cpp).
int32_t check_decode_args(const lla_dims* d, const lla_codec* codec, const lla_cache* cache,
                          int32_t layer, int32_t n_ctx, const int32_t* ctx_lens, const float* q,
                          int32_t loop_begin, int32_t loop_count, const float* out,
                          const lla_decode_opts* opts);

}  // namespace lla
