// Split merge and value up-projection (gfx950).
//
// Each decode wave leaves (max, sum, acc[r_v]) for its context split, with acc the
// softmax-weighted sum of value latents in the exp2 domain of that split's max. This
// kernel merges the splits of one (b, h, t) by log-sum-exp, forms the normalised
// latent a = acc / sum, and applies the loop-specific value map once:
//   out = a W_up,v,t^T + mu_v,t
// which equals sum_j softmax_j V_t[j] because the weights sum to one
// ("Looped Latent Attention", Section 3 Eq. 3 and Appendix J "Absorbed attention").
// An empty context (every split empty) gives zeros.
#include "lla_device.h"
#include "lla_kernels.h"

namespace lla {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

template <typename T, int D, int RV>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  __shared__ float abar[RV];
  const int unit = blockIdx.x;  // (b * H + h) * L + li
  const int li = unit % a.L;
  const int bh = unit / a.L;
  const int h = bh % a.H;
  const int t = a.loop_begin + li;
  const float* p = a.part + static_cast<size_t>(unit) * a.S * (2 + RV);

  float mx = kNegInf;
  for (int s = 0; s < a.S; ++s) mx = fmaxf(mx, p[s * (2 + RV)]);
  float total = 0.f;
  if (mx != kNegInf) {
    for (int s = 0; s < a.S; ++s) total += p[s * (2 + RV) + 1] * fast_exp2(p[s * (2 + RV)] - mx);
  }
  const float inv = total > 0.f ? 1.f / total : 0.f;
  for (int r = threadIdx.x; r < RV; r += blockDim.x) {
    float v = 0.f;
    if (mx != kNegInf) {
      for (int s = 0; s < a.S; ++s) {
        const float ms = p[s * (2 + RV)];
        if (ms != kNegInf) v += p[s * (2 + RV) + 2 + r] * fast_exp2(ms - mx);
      }
    }
    abar[r] = v * inv;
  }
  __syncthreads();

  const T* wv = static_cast<const T*>(a.w_up_v) + static_cast<size_t>(t * a.H + h) * D * RV;
  const size_t mu_off = a.variant == 0 ? static_cast<size_t>(h * a.T + t) * D
                                       : static_cast<size_t>(t * a.H + h) * D;
  const T* muv = static_cast<const T*>(a.mu_v) + mu_off;
  float* out = a.out + static_cast<size_t>(unit) * D;
  for (int i = threadIdx.x; i < D; i += blockDim.x) {
    float o = 0.f;
    if (total > 0.f) {
      static_assert(RV % 8 == 0, "r_v multiple of 8");
#pragma unroll 4
      for (int r0 = 0; r0 < RV; r0 += 8) {
        float w[8];
        load_f32<8>(wv + static_cast<size_t>(i) * RV + r0, w);
#pragma unroll
        for (int r = 0; r < 8; ++r) o += abar[r0 + r] * w[r];
      }
      float m1[1];
      load_f32<1>(muv + i, m1);
      o += m1[0];
    }
    out[i] = o;
  }
}

template <typename T, int D, int RV>
void launch(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((combine_kernel<T, D, RV>), dim3(a.B * a.H * a.L), dim3(D), 0, s, a);
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

}  // namespace lla
