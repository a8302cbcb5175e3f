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
// A workgroup covers 32 tokens (two 16-column tiles; tokens run over (sequence, new
// token) jointly) of one latent head and RG row tiles of 16 latent entries, with KSPLIT
// waves that each take a contiguous 1/KSPLIT of the contraction. Long prompts use one
// wave over all row tiles (x is read once); a few appended tokens use one row tile per
// workgroup and split the contraction, so the whole GPU shares the W_down read. Partial
// sums of the KSPLIT waves are added in LDS in a fixed order (deterministic). The
// contraction loop loads step k + 1 while it multiplies step k.
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

template <typename T, int R, int RG, int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) void encode_kernel(EncodeArgs a) {
  constexpr int KS = KsOf<T>::value;
  using M = Mfma<T, KS>;
  constexpr int E = M::E;
  constexpr int NR = (R + 15) / 16;  // the last row tile is partial when 16 does not divide R
  constexpr int NT = 2;
  constexpr bool kBias = !std::is_same<T, float>::value;
  constexpr int NACC = NT * RG + (kBias ? RG : 0);
  __shared__ f32x4 red[KSPLIT > 1 ? KSPLIT - 1 : 1][NACC][64];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, hi = lane >> 4;
  const int j0 = blockIdx.x * (16 * NT);  // flattened (sequence, new token) index
  const int rt0 = blockIdx.y * RG;        // first row tile
  const int hc = blockIdx.z;
  const int K = a.Kdim;
  const int total = a.B * a.n_new;
  const int kper = K / KSPLIT;
  const int kbeg = wave * kper, kend = kbeg + kper;

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
  const T* wrow[RG];
  bool wok[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int r = 16 * (rt0 + g) + lo;
    wok[g] = (rt0 + g < NR) && (R % 16 == 0 || r < R);
    wrow[g] = w + static_cast<size_t>(wok[g] ? r : 0) * K;
  }

  f32x4 acc[NT][RG];
  f32x4 bias[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    bias[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  typename M::Frag xf[NT], mf, wf[RG];
  auto load_step = [&](int k0, typename M::Frag (&x)[NT], typename M::Frag& m, typename M::Frag (&wv)[RG]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) x[nt] = M::load(xrow[nt] + k0 + hi * E);
    m = M::load(mu + k0 + hi * E);
#pragma unroll
    for (int g = 0; g < RG; ++g) wv[g] = wok[g] ? M::load(wrow[g] + k0 + hi * E) : M::zero();
  };
  load_step(kbeg, xf, mf, wf);
  for (int k0 = kbeg; k0 < kend; k0 += KS) {
    typename M::Frag xn[NT], mn, wn[RG];
    const bool more = k0 + KS < kend;
    if (more) load_step(k0 + KS, xn, mn, wn);
    if constexpr (!kBias) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < E; ++e) xf[nt].v[e] -= mf.v[e];
    }
#pragma unroll
    for (int g = 0; g < RG; ++g) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt][g] = M::mma(wf[g], xf[nt], acc[nt][g]);
      if constexpr (kBias) bias[g] = M::mma(wf[g], mf, bias[g]);
    }
    if (more) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) xf[nt] = xn[nt];
      mf = mn;
#pragma unroll
      for (int g = 0; g < RG; ++g) wf[g] = wn[g];
    }
  }

  if constexpr (KSPLIT > 1) {
    // waves 1.. publish their partial sums; wave 0 adds them in wave order
    if (wave > 0) {
      int i = 0;
#pragma unroll
      for (int g = 0; g < RG; ++g) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) red[wave - 1][i++][lane] = acc[nt][g];
        if constexpr (kBias) red[wave - 1][i++][lane] = bias[g];
      }
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int ws = 0; ws < KSPLIT - 1; ++ws) {
      int i = 0;
#pragma unroll
      for (int g = 0; g < RG; ++g) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][g] = acc[nt][g] + red[ws][i++][lane];
        if constexpr (kBias) bias[g] = bias[g] + red[ws][i++][lane];
      }
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
    for (int g = 0; g < RG; ++g) {
      const int r4 = 16 * (rt0 + g) + 4 * hi;
      if (rt0 + g >= NR || (R % 16 != 0 && r4 >= R)) continue;
      f32x4 v = acc[nt][g];
      if constexpr (kBias) v = v - bias[g];
      store4(crow + r4, v);
    }
  }
}

template <typename T, int R, int RG, int KSPLIT>
void launch(const EncodeArgs& a, hipStream_t s) {
  constexpr int NR = (R + 15) / 16;
  const long long total = static_cast<long long>(a.B) * a.n_new;
  dim3 grid(static_cast<unsigned>((total + 31) / 32), (NR + RG - 1) / RG, a.Hc);
  hipLaunchKernelGGL((encode_kernel<T, R, RG, KSPLIT>), grid, dim3(64 * KSPLIT), 0, s, a);
}

// Long prompts: one wave, every row tile (x read once). Few tokens: one row tile per
// workgroup and the contraction split over up to 8 waves.
template <typename T, int R>
void launch_shape(const EncodeArgs& a, hipStream_t s) {
  constexpr int NR = (R + 15) / 16;
  const long long total = static_cast<long long>(a.B) * a.n_new;
  const long long tiles = (total + 31) / 32;
  if (tiles * a.Hc >= 1024) {
    launch<T, R, NR, 1>(a, s);
  } else if (a.Kdim % (8 * KsOf<T>::value) == 0 && a.Kdim >= 8 * 256) {
    launch<T, R, 1, 8>(a, s);
  } else {
    launch<T, R, 1, 1>(a, s);
  }
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
#define X(R_)                                        \
  if (r == R_) {                                     \
    if (dtype == 0) launch_shape<float, R_>(a, s);   \
    else launch_shape<bf16_t, R_>(a, s);             \
    return true;                                     \
  }
  LLA_ENCODE_RANKS(X)
#undef X
  return false;
}

}  // namespace lla
