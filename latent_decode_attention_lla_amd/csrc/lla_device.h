// Device-side helpers for the gfx950 kernels: storage types, conversions, MFMA
// fragments and cross-lane reductions. wave64 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lla {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// bfloat16 storage as raw 16-bit words.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f32(float x) { return x; }
};
template <>
struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(p->bits); }
};

// Load N consecutive elements starting at p (p aligned to N elements' worth when the
// vector width allows) and widen to float.
template <int N>
__device__ __forceinline__ void load_f32(const float* p, float* out) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      float4 v = *reinterpret_cast<const float4*>(p + i);
      out[i] = v.x; out[i + 1] = v.y; out[i + 2] = v.z; out[i + 3] = v.w;
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 2) {
      float2 v = *reinterpret_cast<const float2*>(p + i);
      out[i] = v.x; out[i + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = p[i];
  }
}

template <int N>
__device__ __forceinline__ void load_f32(const bf16_t* p, float* out) {
  const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
  if constexpr (N % 8 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 8) {
      uint4 v = *reinterpret_cast<const uint4*>(q + i);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        out[i + 2 * k] = __uint_as_float(w[k] << 16);
        out[i + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    }
  } else if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      uint2 v = *reinterpret_cast<const uint2*>(q + i);
      out[i] = __uint_as_float(v.x << 16);
      out[i + 1] = __uint_as_float(v.x & 0xffff0000u);
      out[i + 2] = __uint_as_float(v.y << 16);
      out[i + 3] = __uint_as_float(v.y & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = bf16_to_f32(q[i]);
  }
}

// ---------------------------------------------------------------------------
// MFMA 16x16 tiles, wave64. For a super-step of KS contraction indices, lane l holds
// E consecutive indices k = E * (l >> 4) + e (e < E) of row/column (l & 15) of the A
// and B operands; the 16x16 float result holds D[4 * (l >> 4) + v][l & 15] in
// element v of lane l.
//   float32 : four v_mfma_f32_16x16x4f32 per super-step (KS = 16, E = 4); sub-step e
//             contracts index E * (l >> 4) + e, so A and B see the same order.
//   bf16    : v_mfma_f32_16x16x32_bf16 (KS = 32, E = 8) or
//             v_mfma_f32_16x16x16bf16_1k (KS = 16, E = 4).
//   f16     : v_mfma_f32_16x16x32_f16 (KS = 32, E = 8).
// ---------------------------------------------------------------------------
template <typename T, int KS>
struct Mfma;

template <>
struct Mfma<float, 16> {
  static constexpr int E = 4;
  struct Frag { float v[4]; };
  static __device__ __forceinline__ Frag load(const float* p) {
    float4 x = *reinterpret_cast<const float4*>(p);
    return Frag{{x.x, x.y, x.z, x.w}};
  }
  static __device__ __forceinline__ Frag zero() { return Frag{{0.f, 0.f, 0.f, 0.f}}; }
  static __device__ __forceinline__ f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[0], b.v[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[1], b.v[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[2], b.v[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[3], b.v[3], c, 0, 0, 0);
    return c;
  }
};

template <>
struct Mfma<bf16_t, 32> {
  static constexpr int E = 8;
  struct Frag { bf16x8 v; };
  static __device__ __forceinline__ Frag load(const bf16_t* p) {
    return Frag{*reinterpret_cast<const bf16x8*>(p)};
  }
  static __device__ __forceinline__ Frag zero() {
    Frag f;
    for (int i = 0; i < 8; ++i) f.v[i] = static_cast<__bf16>(0.f);
    return f;
  }
  static __device__ __forceinline__ f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
  }
};

template <>
struct Mfma<bf16_t, 16> {
  static constexpr int E = 4;
  struct Frag { i16x4 v; };
  static __device__ __forceinline__ Frag load(const bf16_t* p) {
    return Frag{*reinterpret_cast<const i16x4*>(p)};
  }
  static __device__ __forceinline__ Frag zero() { return Frag{i16x4{0, 0, 0, 0}}; }
  static __device__ __forceinline__ f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, c, 0, 0, 0);
  }
};

// Contraction width per super-step for a latent of size R: 32 when it divides R for
// bf16, else 16.
template <typename T, int R>
struct KStep { static constexpr int value = 16; };
template <int R>
struct KStep<bf16_t, R> { static constexpr int value = (R % 32 == 0) ? 32 : 16; };

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// v + (v of lane l ^ 16) and v + (v of lane l ^ 32), with the gfx950 permlane swaps: a
// swap of a register with itself leaves the two row groups that are exchanged in the
// two results, so their sum is the butterfly sum without a trip through LDS.
__device__ __forceinline__ float sum_xor16(float v) {
  const unsigned u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const unsigned u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace lla
