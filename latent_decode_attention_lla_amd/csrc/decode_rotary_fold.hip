// Latent-store decode, rotary-fold path (gfx950). Placeholder until the kernel lands.
#include "lla_kernels.h"

namespace lla {

bool decode_rotary_fold_supported(int, int, int, int) { return false; }

bool launch_decode_rotary_fold(int, int, int, int, const DecodeArgs&, hipStream_t) { return false; }

}  // namespace lla
