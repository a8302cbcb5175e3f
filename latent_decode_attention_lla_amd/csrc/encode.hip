// Encode (gfx950): c = (x - mu) W_down for tokens whose T loops are finished
// ("Looped Latent Attention", Section 3 Eqs. 1-2; the latent of a token is written once,
// after its last loop).
//
// Computed transposed on the matrix cores, C^T (r x tokens) = W_down^T (r x K) X^T
// (K x tokens) with K = T * d_in, so that
//   * A fragments are rows of W_down^T and B fragments rows of x: both contiguous runs
//     of the contraction index;
//   * a lane ends up holding 4 consecutive latent entries of one token, stored as one
//     8-byte (bf16) or 16-byte (float32) write into the cache row.
// Centring: for float32 x - mu is formed before the MFMA; for bfloat16 the bias mu W_down
// is produced by the same MFMA with mu broadcast into every B column and subtracted
// from the float32 accumulator, so no intermediate is rounded to bfloat16. The result is
// rounded once (nearest, ties to even) into the storage type.
//
// One wave: 32 tokens (two 16-column tiles) of one latent head, all r. Tokens are taken
// over (sequence, new token) jointly, so appending one token to each of many sequences
// (the decode-time encode) fills the tiles as well as a long prompt does.
#include "lla_device.h"
#include "lla_kernels.h"

namespace lla {

namespace {

template <typename T>
struct KsOf { static constexpr int value = 16; };
template <>
struct KsOf<bf16_t> { static constexpr int value = 32; };

__device__ __forceinline__ void store4(float* p, f32x4 v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16_t* p, f32x4 v) {
  uint2 w;
  w.x = static_cast<uint32_t>(f32_to_bf16_rne(v[0])) | (static_cast<uint32_t>(f32_to_bf16_rne(v[1])) << 16);
  w.y = static_cast<uint32_t>(f32_to_bf16_rne(v[2])) | (static_cast<uint32_t>(f32_to_bf16_rne(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = w;
}

template <typename T, int R>
__global__ __launch_bounds__(64) void encode_kernel(EncodeArgs a) {
  constexpr int KS = KsOf<T>::value;
  using M = Mfma<T, KS>;
  constexpr int E = M::E;
  constexpr int NR = (R + 15) / 16;  // the last tile is partial when 16 does not divide R
  constexpr int NT = 2;
  constexpr bool kBias = !std::is_same<T, float>::value;

  const int lane = threadIdx.x;
  const int lo = lane & 15, hi = lane >> 4;
  const int j0 = blockIdx.x * (16 * NT);  // flattened (sequence, new token) index
  const int hc = blockIdx.y;
  const int K = a.Kdim;
  const int total = a.B * a.n_new;

  const T* w = static_cast<const T*>(a.w_down_t) + static_cast<size_t>(hc) * R * K;
  const T* mu = static_cast<const T*>(a.mu) + static_cast<size_t>(hc) * K;
  const T* xrow[NT];
  bool valid[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int tok = j0 + 16 * nt + lo;
    valid[nt] = tok < total;
    const int row = valid[nt] ? tok : total - 1;
    xrow[nt] = static_cast<const T*>(a.x) + (static_cast<size_t>(row) * a.Hc + hc) * K;
  }

  f32x4 acc[NT][NR];
  f32x4 bias[NR];
#pragma unroll
  for (int rt = 0; rt < NR; ++rt) {
    bias[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int k0 = 0; k0 < K; k0 += KS) {
    typename M::Frag xf[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) xf[nt] = M::load(xrow[nt] + k0 + hi * E);
    const typename M::Frag mf = M::load(mu + k0 + hi * E);
    if constexpr (!kBias) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < E; ++e) xf[nt].v[e] -= mf.v[e];
    }
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
      typename M::Frag wfr;
      if (R % 16 == 0 || 16 * rt + lo < R) {
        wfr = M::load(w + static_cast<size_t>(16 * rt + lo) * K + k0 + hi * E);
      } else {
        wfr = M::zero();
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt][rt] = M::mma(wfr, xf[nt], acc[nt][rt]);
      if constexpr (kBias) bias[rt] = M::mma(wfr, mf, bias[rt]);
    }
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (!valid[nt]) continue;
    const int tok = j0 + 16 * nt + lo;
    const int b = tok / a.n_new;
    const int j = tok - b * a.n_new;
    T* crow = static_cast<T*>(a.c) +
              (static_cast<size_t>(b * a.Hc + hc) * a.n_max + a.pos_start + j) * R;
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
      f32x4 v = acc[nt][rt];
      if constexpr (kBias) v = v - bias[rt];
      if (R % 16 == 0 || 16 * rt + 4 * hi < R) store4(crow + 16 * rt + 4 * hi, v);
    }
  }
}

template <typename T, int R>
void launch(const EncodeArgs& a, hipStream_t s) {
  const long long total = static_cast<long long>(a.B) * a.n_new;
  dim3 grid(static_cast<unsigned>((total + 31) / 32), a.Hc, 1);
  hipLaunchKernelGGL((encode_kernel<T, R>), grid, dim3(64), 0, s, a);
}

}  // namespace

#define LLA_ENCODE_RANKS(X) X(16) X(24) X(32) X(64) X(96) X(128) X(160) X(256)

bool encode_supported(int dtype, int r, int Kdim) {
  const int ks = dtype == 0 ? 16 : 32;
  if (Kdim % ks != 0) return false;
#define X(R_) if (r == R_) return true;
  LLA_ENCODE_RANKS(X)
#undef X
  return false;
}

bool launch_encode(int dtype, int r, const EncodeArgs& a, hipStream_t s) {
#define X(R_)                                  \
  if (r == R_) {                               \
    if (dtype == 0) launch<float, R_>(a, s);   \
    else launch<bf16_t, R_>(a, s);             \
    return true;                               \
  }
  LLA_ENCODE_RANKS(X)
#undef X
  return false;
}

}  // namespace lla
