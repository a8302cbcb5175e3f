// RoPE cos/sin tables for rebuilt keys (gfx950).
//
// "Looped Latent Attention" (arXiv 2607.15456v2), Section 3 "RoPE and reconstruction":
// a token's rotary phase is the same at every loop, so the model's RoPE is applied
// after reconstruction. RoPE follows RoFormer (which the paper cites): interleaved
// pairs (2i, 2i+1) rotated by p * theta_i, theta_i = base^(-2i/d).
//
// The angle, cosine and sine are evaluated in float64 and rounded once:
//   t32[p][i] = (cos, sin) as float32, pairs interleaved      (reconstruct path)
//   t16: CS_p[k] = cos(p theta_k) for k < d/2, sin(p theta_(k-d/2)) for k >= d/2, as
//        float16, stored in the order a 16x16x32 MFMA B fragment is read: position
//        p = 16 tile + j, index k = 32 ks + 8 g + e lives at
//        ((tile * (d/32) + ks) * 64 + j + 16 g) * 8 + e, so one wave reads a fragment
//        as 1 KiB of consecutive bytes. Positions are padded to a multiple of 16.
#include <math.h>

#include "lla_kernels.h"

namespace lla {

namespace {

// float64 -> float16 bits, nearest with ties to even, including half subnormals.
__device__ uint16_t f64_to_f16_bits(double x) {
  const double ax = fabs(x);
  double r;
  if (ax >= 6.103515625e-05) {  // 2^-14, smallest normal half
    int e;
    const double m = frexp(x, &e);        // x = m 2^e, 0.5 <= |m| < 1
    r = ldexp(rint(ldexp(m, 11)), e - 11);  // 11 significant bits
  } else {
    r = ldexp(rint(ldexp(x, 24)), -24);   // half subnormal spacing 2^-24
  }
  const _Float16 h = static_cast<_Float16>(static_cast<float>(r));  // exact
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ size_t frag_offset(int p, int k, int d) {
  const int tile = p >> 4, j = p & 15;
  const int ks = k >> 5, g = (k & 31) >> 3, e = k & 7;
  return ((static_cast<size_t>(tile) * (d / 32) + ks) * 64 + j + 16 * g) * 8 + e;
}

__global__ void rope_table_kernel(int d, int n_max, double base, float* t32, uint16_t* t16) {
  const int half = d / 2;
  const int n_pad = (n_max + 15) / 16 * 16;
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long long>(n_pad) * half) return;
  const int p = static_cast<int>(idx / half);
  const int i = static_cast<int>(idx - static_cast<long long>(p) * half);
  const double theta = pow(base, -2.0 * i / d);
  const double phi = static_cast<double>(p) * theta;
  const double c = cos(phi), s = sin(phi);
  if (p < n_max) {
    t32[(static_cast<size_t>(p) * half + i) * 2] = static_cast<float>(c);
    t32[(static_cast<size_t>(p) * half + i) * 2 + 1] = static_cast<float>(s);
  }
  t16[frag_offset(p, i, d)] = f64_to_f16_bits(c);
  t16[frag_offset(p, half + i, d)] = f64_to_f16_bits(s);
}

}  // namespace

void launch_rope_table(int d, int n_max, double base, float* t32, uint16_t* t16, hipStream_t s) {
  const long long total = static_cast<long long>((n_max + 15) / 16 * 16) * (d / 2);
  const int threads = 256;
  const int blocks = static_cast<int>((total + threads - 1) / threads);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(threads), 0, s, d, n_max, base, t32, t16);
}

}  // namespace lla
