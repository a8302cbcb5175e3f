// Split merge and value up-projection (gfx950).
//
// Each decode wave leaves (max, sum, acc[r_v]) for its context split, with acc the
// softmax-weighted sum of value latents in the exp2 domain of that split's max. This
// kernel merges the splits of one (b, h, t) by log-sum-exp, forms the normalised
// latent a = acc / sum, and applies the loop-specific value map once:
//   out = a W_up,v,t^T + mu_v,t
// which equals sum_j softmax_j V_t[j] because the weights sum to one
// ("Looped Latent Attention", Section 3 Eq. 3 and Appendix J "Absorbed attention").
// For a cache of uncompressed values the partials hold value rows and the merged row is
// the output itself (no projection). An empty context (every split empty) gives zeros.
#include "lla_device.h"
#include "lla_kernels.h"

namespace lla {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

constexpr int kLdsSplits = 32;  // partials of up to this many splits are staged in LDS

// One workgroup of 256 threads per (b, h, t). Everything the unit needs from memory (its
// split partials, its rows of W_up,v,t and mu_v,t) is requested at the start, so the
// kernel pays one memory round trip: thread k owns output i = k / TPR and the TPR-th
// slice of that row of W_up,v,t.
template <typename T, int D, int RV, bool PROJ>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  constexpr int TPR = 256 / D;      // threads per output row
  constexpr int RS = RV / TPR;      // row entries per thread
  static_assert(256 % D == 0 && RV % TPR == 0, "row slices");
  constexpr int PS = 2 + RV;        // floats per split partial
  __shared__ float part[kLdsSplits * PS];
  __shared__ float wsplit[kLdsSplits];
  __shared__ float abar[RV];
  __shared__ float red[2];

  const int tid = threadIdx.x;
  const int unit = blockIdx.x;  // (b * H + h) * L + li
  const int li = unit % a.L;
  const int h = (unit / a.L) % a.H;
  const int t = a.loop_begin + li;
  const int S = a.S;
  const float* p = a.part + static_cast<size_t>(unit) * S * PS;
  const bool staged = S <= kLdsSplits;

  // (1) every load of the unit
  if (staged) {
    for (int k = tid; k < S * PS; k += 256) part[k] = p[k];
  }
  const int i = tid / TPR, sub = tid % TPR;
  float w[RS];
  float mu1[1] = {0.f};
  if constexpr (PROJ) {
    const T* wv = static_cast<const T*>(a.w_up_v) + static_cast<size_t>(t * a.H + h) * D * RV +
                  static_cast<size_t>(i) * RV + sub * RS;
    load_f32<RS>(wv, w);
    const size_t mu_off = a.variant == 0 ? static_cast<size_t>(h * a.T + t) * D
                                         : static_cast<size_t>(t * a.H + h) * D;
    load_f32<1>(static_cast<const T*>(a.mu_v) + mu_off + i, mu1);
  }
  __syncthreads();

  // (2) log-sum-exp weights of the splits, then the normalised latent
  auto merge = [&](const float* src) {
    if (tid == 0) {
      float mx = kNegInf;
      for (int s = 0; s < S; ++s) mx = fmaxf(mx, src[s * PS]);
      float total = 0.f;
      if (mx != kNegInf) {
        for (int s = 0; s < S; ++s) {
          const float ms = src[s * PS];
          const float ws = ms != kNegInf ? fast_exp2(ms - mx) : 0.f;
          if (s < kLdsSplits) wsplit[s] = ws;
          total += src[s * PS + 1] * ws;
        }
      }
      red[0] = mx;
      red[1] = total;
    }
    __syncthreads();
    const float mx = red[0], total = red[1];
    const float inv = total > 0.f ? 1.f / total : 0.f;
    for (int r = tid; r < RV; r += 256) {
      float v = 0.f;
      for (int s = 0; s < S; ++s) {
        const float ms = src[s * PS];
        const float ws = s < kLdsSplits ? wsplit[s] : (ms != kNegInf ? fast_exp2(ms - mx) : 0.f);
        v += src[s * PS + 2 + r] * ws;
      }
      abar[r] = v * inv;
    }
    __syncthreads();
    return total;
  };
  const float total = staged ? merge(part) : merge(p);

  if constexpr (!PROJ) {  // the merged value itself (an uncompressed cache)
    for (int r = tid; r < RV; r += 256) a.out[static_cast<size_t>(unit) * D + r] = abar[r];
    return;
  }
  // (3) out = abar W_up,v,t^T + mu_v,t
  float o = 0.f;
#pragma unroll
  for (int e = 0; e < RS; ++e) o += abar[sub * RS + e] * w[e];
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) o += shfl_xor(o, m);
  if (sub == 0) a.out[static_cast<size_t>(unit) * D + i] = total > 0.f ? o + mu1[0] : 0.f;
}

template <typename T, int D, int RV, bool PROJ = true>
void launch(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((combine_kernel<T, D, RV, PROJ>), dim3(a.B * a.H * a.L), dim3(256), 0, s, a);
}

}  // namespace

#define LLA_COMBINE_SHAPES(X) X(64, 24) X(64, 32) X(64, 256) X(128, 32) X(128, 64) X(128, 160) X(128, 128)

bool launch_combine(int dtype, int d, int r_v, const DecodeArgs& a, hipStream_t s) {
#define X(D_, RV_)                               \
  if (d == D_ && r_v == RV_) {                   \
    if (dtype == 0) launch<float, D_, RV_>(a, s); \
    else launch<bf16_t, D_, RV_>(a, s);          \
    return true;                                 \
  }
  LLA_COMBINE_SHAPES(X)
#undef X
  return false;
}

// Merge the partials of an uncompressed decode (values of width d, no up-projection).
bool launch_combine_identity(int dtype, int d, const DecodeArgs& a, hipStream_t s) {
  (void)dtype;  // the partials are float whatever the cache type
#define X(D_)                               \
  if (d == D_) {                            \
    launch<float, D_, D_, false>(a, s);     \
    return true;                            \
  }
  X(64) X(128)
#undef X
  return false;
}

}  // namespace lla
