// Launch arguments shared by the C ABI (lla_api.cpp) and the gfx950 kernels, and the
// compile-time shape constants both sides must agree on.
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

// Projection-fused encode: loop `loop` of one layer and one axis (keys or values).
struct FusedArgs {
  const void* h;        // [Ntok][d_model], Ntok = B * n_new: the loop's projection input
  const void* w_proj;   // layer base, [H * d][d_model] (output features x input features)
  const void* w_down_t; // layer base, [Hc][r][T * d_in]
  const void* mu;       // layer base, [Hc][T * d_in]
  void* c;              // layer base, [B][Hc][n_max][r]
  float* acc;           // [Ntok][Hc][RT]: running sum over the loops, this axis at ao
  int Ntok, n_new, pos_start, n_max, H, Hc, T, d_in, d_model, loop, RT, ao;
};

// Heads per workgroup of the rotary-fold kernel; H must be a multiple of it.
#ifndef LLA_FOLD_HPW
#define LLA_FOLD_HPW 4
#endif
constexpr int kFoldHeadsPerGroup = LLA_FOLD_HPW;

}  // namespace lla
