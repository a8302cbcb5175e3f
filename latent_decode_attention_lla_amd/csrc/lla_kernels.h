// Internal interface between the C ABI (lla_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lla {

// Decode: one launch covers one layer and loops [loop_begin, loop_begin + L).
struct DecodeArgs {
  const void* c_k;      // layer base, [B][Hc][n_max][r_k]
  const void* c_v;      // layer base, [B][Hc][n_max][r_v]
  const void* w_up_k;   // layer base, [T][H][d][r_k]
  const void* w_up_v;   // layer base, [T][H][d][r_v]
  const void* mu_k;     // layer base, [Hc][T*d_in]
  const void* mu_v;
  const float* rope32;  // [n_max][d/2][2]  (cos, sin) interleaved per pair
  const uint16_t* rope16;  // [n_max][d] float16: cos of all pairs then sin of all pairs
  const float* q;       // [B][H][L][d]
  const int32_t* ctx_lens;  // [B] or null
  float* part;          // [B][H][L][S][2 + r_v]: (max, sum, acc[r_v]) per split
  float* out;           // [B][H][L][d]
  int B, H, Hc, T, L, loop_begin, n_max, n_ctx, S, split_len;
  int variant;          // 0 per head, 1 LLA-2D
  float scale_log2e;    // score scale times log2(e): scores live in the exp2 domain
};

struct EncodeArgs {
  const void* x;        // [B][n_new][Hc][T*d_in]
  const void* w_down_t; // layer base, [Hc][r][T*d_in]
  const void* mu;       // layer base, [Hc][T*d_in]
  void* c;              // layer base, [B][Hc][n_max][r]
  int B, Hc, Kdim, n_new, pos_start, n_max;
};

// Heads per workgroup of the rotary-fold kernel; H must be a multiple of it.
#ifndef LLA_FOLD_HPW
#define LLA_FOLD_HPW 4
#endif
constexpr int kFoldHeadsPerGroup = LLA_FOLD_HPW;

// Launchers return false when no kernel is built for (dtype, d, r_k, r_v) on that path.
bool launch_decode_reconstruct(int dtype, int d, int r_k, int r_v, const DecodeArgs& a,
                               hipStream_t s);
bool launch_decode_rotary_fold(int dtype, int d, int r_k, int r_v, const DecodeArgs& a,
                               hipStream_t s);
// Wide latents (r_k >= 64): a pair of waves per head; `shared` selects LLA-2D (all heads
// read one latent plane). H must be a multiple of fold_wide_heads_per_group(...).
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
// Uncompressed decode: c_k / c_v of the args are the layer's per-loop key and value
// caches [T][B][H][n_max][d]; combine with `project` false merges its partials.
bool launch_decode_teacher(int dtype, int d, const DecodeArgs& a, hipStream_t s);
bool decode_teacher_supported(int dtype, int d);
bool launch_combine_identity(int dtype, int d, const DecodeArgs& a, hipStream_t s);
bool decode_reconstruct_supported(int dtype, int d, int r_k, int r_v);
bool decode_rotary_fold_supported(int dtype, int d, int r_k, int r_v);

bool launch_encode(int dtype, int r, const EncodeArgs& a, hipStream_t s);
bool encode_supported(int dtype, int r, int Kdim);

void launch_rope_table(int d, int n_max, double base, float* t32, uint16_t* t16, hipStream_t s);

}  // namespace lla
