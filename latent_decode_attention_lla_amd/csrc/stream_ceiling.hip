// Plain streaming kernels that measure the HBM ceilings the decode and encode kernels are
// compared against (gfx950): a read-only pass, a copy (1:1), and 4:1 and 1:4 read:write
// mixes. Every lane moves 16-byte vectors with a grid-stride loop; nothing here belongs to
// the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lla_stream.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// mode 0: read n vectors of src, one xor-fold per workgroup into dst[block]
// mode 1: dst[i] = src[i]
// mode 2: dst[i] = src[i] ^ src[i + n] ^ src[i + 2n] ^ src[i + 3n]   (4 reads : 1 write)
// mode 3: dst[i + k n] = src[i] for k = 0 .. 3                         (1 read : 4 writes)
__global__ __launch_bounds__(256) void stream_kernel(int mode, const u32x4* __restrict__ src,
                                                     u32x4* __restrict__ dst, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (mode == 0) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(src + i);
    __shared__ u32x4 red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (static_cast<int>(threadIdx.x) < s) red[threadIdx.x] ^= red[threadIdx.x + s];
      __syncthreads();
    }
    if (threadIdx.x == 0) dst[blockIdx.x] = red[0];
  } else if (mode == 1) {
    for (; i < n; i += stride) dst[i] = __builtin_nontemporal_load(src + i);
  } else if (mode == 2) {
    for (; i < n; i += stride)
      dst[i] = __builtin_nontemporal_load(src + i) ^ __builtin_nontemporal_load(src + i + n) ^
               __builtin_nontemporal_load(src + i + 2 * n) ^ __builtin_nontemporal_load(src + i + 3 * n);
  } else {
    for (; i < n; i += stride) {
      const u32x4 v = __builtin_nontemporal_load(src + i);
      dst[i] = v;
      dst[i + n] = v;
      dst[i + 2 * n] = v;
      dst[i + 3 * n] = v;
    }
  }
}

}  // namespace

extern "C" int32_t lla_stream_ceiling(int32_t mode, const void* src, void* dst, size_t n_vectors,
                                      int32_t workgroups, void* stream) {
  if (mode < 0 || mode > 3 || src == nullptr || dst == nullptr || n_vectors == 0 || workgroups < 1)
    return -1;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) return -1;
  hipLaunchKernelGGL(stream_kernel, dim3(static_cast<unsigned>(workgroups)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), mode, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), n_vectors);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
