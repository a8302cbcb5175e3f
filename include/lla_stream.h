/*
 * lla_stream.h - measurement helper of liblla.so, not part of the method: plain streaming
 * kernels that give the HBM ceilings (a read-only pass, a copy, 4:1 and 1:4 read:write
 * mixes, read-only passes through LDS or registers, and the narrow fold's row pattern)
 * the latent-store kernels are compared against on the same device.
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
 *   modes 4-6: read src[0 .. n) with every wave (4 per workgroup) streaming its own
 *           contiguous chunk of 1 KiB blocks: mode 4 through a ring of buffer loads to
 *           LDS, mode 5 through registers, mode 6 half through each; n must split into the
 *           same whole number of blocks per wave, a multiple of 16 and at least 32, each
 *           chunk under 2 GiB (else -1); nothing is written unless a checksum of the data
 *           hits one fixed value (then 16 bytes to dst[0]).
 *   mode 7: the latent-row pattern of the narrow fold kernel: read src[0 .. n) as 4 ·
 *           workgroups key planes of 32-byte rows (the first third) and as many value
 *           planes of 64-byte rows (the rest), every wave streaming one plane of each in
 *           16-row tiles (a 512-byte and a 1 KiB wave load per tile, 8 tiles in flight);
 *           n must be 96 vectors times the wave count times a multiple of 8 (else -1);
 *           writes as modes 4-6.
 * src and dst are device pointers, 16-byte aligned, owned by the caller, large enough for
 * the mode (mode 2 reads 4n vectors, mode 3 writes 4n, mode 0 writes `workgroups`).
 * workgroups: 256-thread workgroups of the grid (a grid-stride loop in modes 0-3).
 * Returns 0, -1 for invalid arguments (nothing enqueued), -4 when the launch failed. */
int32_t lla_stream_ceiling(int32_t mode, const void* src, void* dst, size_t n_vectors,
                           int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LLA_STREAM_H_ */
