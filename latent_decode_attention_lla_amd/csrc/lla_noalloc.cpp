// lla_decode_attn for callers that cannot allocate device memory: the split partials live
// in a fixed device array of this library instead of a caller-provided workspace. The
// decode itself is lla_decode_attn's (same validation, plan and kernels), so the results
// are bit-identical to a call with a workspace.
#include "lla.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "lla_kernels.h"

namespace {

// Split partials of one call, [batch][H][loops][splits][2 + r_v] float32. The runtime
// creates one copy per GPU when the code object is loaded there; it lives until the
// process ends. Every split writes its partial before the merge reads it, so nothing
// has to be cleared between calls.
static __device__ __align__(256) unsigned char scratch[LLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of the current device's copy of `scratch`, looked up once per
// device. Host code never passes `scratch` itself to a kernel: on the host that name
// is only a stand-in for the symbol.
int32_t scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return LLA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return LLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return LLA_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return LLA_OK;
}

}  // namespace

extern "C" int32_t lla_decode_attn_noalloc(const lla_dims* d, const lla_codec* codec,
                                           const lla_cache* cache, int32_t layer, int32_t n_ctx,
                                           const int32_t* ctx_lens, const float* q,
                                           int32_t loop_begin, int32_t loop_count, float* out,
                                           const lla_decode_opts* opts, void* stream) {
  // every argument is checked on the host before the first HIP call
  const int32_t chk = lla::check_decode_args(d, codec, cache, layer, n_ctx, ctx_lens, q,
                                             loop_begin, loop_count, out, opts);
  if (chk != LLA_OK) return chk;
  if (lla_decode_workspace_bytes(d, n_ctx, loop_count, opts) > LLA_NOALLOC_SCRATCH_BYTES)
    return LLA_ERR_WORKSPACE;
  void* ws = nullptr;
  const int32_t st = scratch_of_current_device(&ws);
  if (st != LLA_OK) return st;
  return lla_decode_attn(d, codec, cache, layer, n_ctx, ctx_lens, q, loop_begin, loop_count, out,
                         ws, LLA_NOALLOC_SCRATCH_BYTES, opts, stream);
}
