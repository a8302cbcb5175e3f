/*
 * lla_stream.h - measurement helper of liblla.so, not part of the method: plain streaming
 * kernels that give the HBM ceilings (a read-only pass, a copy, 4:1 and 1:4 read:write
 * mixes) the latent-store kernels are compared against on the same device.
 */
#ifndef LLA_STREAM_H_
#define LLA_STREAM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Stream n_vectors 16-byte vectors, asynchronously on `stream` (a hipStream_t):
 *   mode 0: read src[0 .. n), write one 16-byte xor-fold per workgroup to dst[0 .. workgroups)
 *   mode 1: dst[i] = src[i]                                            (1 read : 1 write)
 *   mode 2: dst[i] = src[i] ^ src[i + n] ^ src[i + 2n] ^ src[i + 3n]   (4 reads : 1 write)
 *   mode 3: dst[i + k n] = src[i], k = 0 .. 3                          (1 read : 4 writes)
 * src and dst are device pointers, 16-byte aligned, owned by the caller, large enough for
 * the mode (mode 2 reads 4n vectors, mode 3 writes 4n, mode 0 writes `workgroups`).
 * workgroups: 256-thread workgroups of the grid-stride loop.
 * Returns 0, -1 for invalid arguments (nothing enqueued), -4 when the launch failed. */
int32_t lla_stream_ceiling(int32_t mode, const void* src, void* dst, size_t n_vectors,
                           int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LLA_STREAM_H_ */
