// Launch arguments of the materialised reconstruction, shared by the C ABI and its kernel.
#pragma once

namespace lla {

// Materialised reconstruction: one launch covers one layer, one axis (keys or values)
// and loops [loop_begin, loop_begin + L).
struct ReconArgs {
  const void* c;        // layer base, [B][Hc][n_max][r]
  const void* w_up;     // layer base, [T][H][d][r]
  const void* mu;       // layer base, [Hc][T*d_in]
  const float* rope32;  // [n_max][d/2][2] (cos, sin) per pair, or null: no rotation
  void* out;            // [L][B][H][n_max][d], rows pos_start .. pos_start + n_tok - 1
  int B, H, Hc, T, L, loop_begin, n_max, pos_start, n_tok;
  int variant;          // 0 per head, 1 LLA-2D
  int chunk;            // tokens per wave (a multiple of 16)
};

}  // namespace lla
