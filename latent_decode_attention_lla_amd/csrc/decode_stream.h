// Helpers of the streaming decode kernels (the absorbed and the uncompressed decode,
// gfx950 wave64): a wave's 64 lanes are G groups of 64/G tokens, and each group takes
// every G-th 8-byte unit of a token's cache rows, so that one load instruction reads 8 G
// contiguous bytes of each row it touches.
#pragma once

#include <type_traits>

#include "lla_device.h"

#ifndef LLA_STREAM_NT
#define LLA_STREAM_NT 1  // stream the cache rows with nontemporal loads
#endif

namespace lla {
namespace stream {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A lane group's share of one row: the row is cut into 8-byte units and group g takes
// units g, g + G, g + 2 G, ..., so that one load instruction of the wave reads 8 G
// contiguous bytes of each of its rows. Kept as raw 32-bit words until used; local
// element e is row element ((e / EU) G + g) EU + e % EU, EU elements per unit.
template <typename T, int N>
struct Piece {
  static constexpr int BYTES = N * static_cast<int>(sizeof(T));
  static constexpr int WORDS = BYTES / 4;
  static constexpr int UNITS = BYTES / 8;
  uint32_t w[WORDS];
};

template <typename T>
struct Unit { static constexpr int EU = 8 / static_cast<int>(sizeof(T)); };

// row element of local element e for lane group g
template <typename T, int G>
__device__ __forceinline__ int row_elem(int e, int g) {
  constexpr int EU = Unit<T>::EU;
  return ((e / EU) * G + g) * EU + e % EU;
}

template <typename T, int N, int G>
__device__ __forceinline__ void load_piece(Piece<T, N>& p, const char* row, int g) {
  static_assert(Piece<T, N>::BYTES % 8 == 0, "whole 8-byte units");
#pragma unroll
  for (int k = 0; k < Piece<T, N>::UNITS; ++k) {
#if LLA_STREAM_NT
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(row) + k * G + g);
#else
    const u32x2 v = reinterpret_cast<const u32x2*>(row)[k * G + g];
#endif
    p.w[2 * k] = v.x; p.w[2 * k + 1] = v.y;
  }
}

// Element e of a piece as float.
template <typename T, int N>
__device__ __forceinline__ float elem(const Piece<T, N>& p, int e) {
  if constexpr (std::is_same<T, float>::value) {
    return __uint_as_float(p.w[e]);
  } else {
    const uint32_t w = p.w[e >> 1];
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
}

template <typename T>
__device__ __forceinline__ float load_scalar(const T* p) {
  if constexpr (std::is_same<T, float>::value) return *p;
  else return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[0]);
}

// v + (v of lane l ^ 8): rotate each 16-lane row by 8 (DPP row_ror:8)
__device__ __forceinline__ float sum_xor8(float v) {
  const int r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false);
  return v + __int_as_float(r);
}

template <int G>
__device__ __forceinline__ float sum_groups(float v) {
  static_assert(G == 4 || G == 8, "lane groups");
  if constexpr (G == 8) v = sum_xor8(v);
  return sum_xor32(sum_xor16(v));
}

// v plus lane (l ^ m) of v's DPP source pattern CTRL (a constant DPP control).
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
