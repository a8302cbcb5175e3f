// Helpers of the streaming decode kernels (the absorbed and the uncompressed decode,
// gfx950 wave64): a token's cache rows are read as 16-byte pieces by consecutive lanes,
// the pieces' partial dots are summed over those lanes with DPP.
#pragma once

#include <type_traits>

#include "lla_device.h"

#ifndef LLA_STREAM_NT
#define LLA_STREAM_NT 1  // stream the cache rows with nontemporal loads
#endif

namespace lla {
namespace stream {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ float load_scalar(const T* p) {
  if constexpr (std::is_same<T, float>::value) return *p;
  else return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[0]);
}

// v plus the lane that the constant DPP control CTRL selects for each lane.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over each aligned group of GP consecutive lanes, every lane of the group receiving
// the total. Lane bits 0 and 1 by quad permutations ([1,0,3,2], [2,3,0,1]); bit 2 by the
// half-row mirror (once quads are summed, lane i and lane 7 - i of a half row hold its two
// quads); bit 3 by a row rotation of 8; bits 4 and 5 by the permlane swaps.
template <int GP>
__device__ __forceinline__ float sum_lanes(float v) {
  static_assert(GP >= 2 && GP <= 64 && (GP & (GP - 1)) == 0, "power-of-two lane groups");
  v = dpp_add<0xB1>(v);
  if constexpr (GP >= 4) v = dpp_add<0x4E>(v);
  if constexpr (GP >= 8) v = dpp_add<0x141>(v);
  if constexpr (GP >= 16) v = dpp_add<0x128>(v);
  if constexpr (GP >= 32) v = sum_xor16(v);
  if constexpr (GP >= 64) v = sum_xor32(v);
  return v;
}

// Element e of a 16-byte piece of a row as float.
template <typename T>
__device__ __forceinline__ float elem16(const u32x4& w, int e) {
  if constexpr (std::is_same<T, float>::value) {
    return __uint_as_float(w[e]);
  } else {
    const uint32_t x = w[e >> 1];
    return (e & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
  }
}

__device__ __forceinline__ u32x4 load16(const char* p) {
#if LLA_STREAM_NT
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}

}  // namespace stream
}  // namespace lla
