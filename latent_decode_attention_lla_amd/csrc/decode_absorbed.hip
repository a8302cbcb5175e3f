// Latent-store decode, decoupled-RoPE absorbed path (gfx950, wave64; bfloat16 or float32
// cache).
//
// "Looped Latent Attention", Appendix J "Absorbed attention": the score is bilinear, so the
// key up-projection moves to the query side, q . (c W_up^T + mu) = (W_up^T q) . c + q . mu,
// and the value side keeps the identity sum_j p_j (c_j W_up,v^T + mu_v) =
// (sum_j p_j c_j) W_up,v^T + mu_v for weights that sum to one. RoPE does not absorb, so the
// head is split: dimensions 0 .. d_rope-1 form a rotary branch whose key is stored per
// token (already rotated to its position, one for every loop of the token), and
// dimensions d_rope .. d-1 the content path that the latent reconstructs without RoPE.
// Per (sequence, head, loop):
//   q~ = W_up,k,t[content rows]^T q[content],   beta = q[content] . mu_k,t[content]
//   s_j = scale (q~ . c_j + beta + q[rotary] . k_rope,j)
// so attention reads only the c_k, k_rope and c_v rows and rebuilds no key.
//
// decode_absorbed_kernel: one wave per (sequence, head, loop, split). Its prologue folds
//   the query: q~, beta and the rotary query, scaled into the exp2 domain, go to LDS (the
//   unit's W_up,k,t rows are read from L2, shared by the unit's splits). Its 64 lanes are G
//   groups of 64/G: lane (j, g) takes token j of each (64/G)-token tile and every G-th
//   8-byte unit of each of its rows (c_k, k_rope, c_v), starting at unit g. G = 4 for narrow latents; G = 8 for
//   wide ones keeps a lane's share of the rows, the folded query and the value
//   accumulator within the registers of two waves per SIMD. The slice dots are summed over
//   the lane groups by butterflies (a DPP row rotation for 8, permlane swaps for 16 and
//   32). The per-column online softmax (max raised only past a 2^8 slack, exact) and the
//   value-latent accumulation follow the other decode kernels; one split finishes with the
//   value up-projection in the epilogue, more go through combine_kernel. The rows of the
//   next TPC tiles are loaded (non-temporal) while the current ones are computed, and
//   chunks wholly inside the context skip the clamping and masking.
#include <type_traits>

#include "decode_stream.h"
#include "lla_device.h"
#include "lla_kernels.h"

namespace lla {

namespace {

using namespace stream;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMaxInit = -1.0e30f;  // finite stand-in for -inf (see the fold kernels)
constexpr float kRescaleSlack = 8.0f;

// Folded query of one unit in LDS: q~ [RK], beta, then the rotary query [DR].
template <int RK, int DR>
struct QaLayout {
  static constexpr int BETA = RK;
  static constexpr int ROT = RK + 4;
  static constexpr int QS = RK + 4 + DR;
};

template <typename T, int D, int RK, int RV, int DR, int G, int TPC>
__global__ __launch_bounds__(64) void decode_absorbed_kernel(DecodeArgs a, const void* k_rope) {
  using L = QaLayout<RK, DR>;
  constexpr int TOK = 64 / G;                           // tokens per tile
  constexpr int NK = RK / G, NR = DR / G, NV = RV / G;  // row elements per lane group
  constexpr int ES = static_cast<int>(sizeof(T));
  static_assert((RK * ES) % (8 * G) == 0 && (DR * ES) % (8 * G) == 0 && (RV * ES) % (8 * G) == 0,
                "rows cut into whole 8-byte units per lane group");
  struct Rows {
    Piece<T, NK> k[TPC];
    Piece<T, NR> r[TPC];
    Piece<T, NV> v[TPC];
  };
  __shared__ float abar[RV];
  __shared__ float qs[QaLayout<RK, DR>::QS];

  const int lane = threadIdx.x;
  const int lo = lane % TOK, hi = lane / TOK;
  const int split = blockIdx.x;
  const int h = blockIdx.y / a.L;
  const int li = blockIdx.y - h * a.L;
  const int b = blockIdx.z;
  const int t = a.loop_begin + li;
  const int hc = a.variant == 0 ? h : 0;
  const size_t unit = static_cast<size_t>(b * a.H + h) * a.L + li;

  int len = a.n_ctx;
  if (a.ctx_lens != nullptr) len = max(0, min(a.ctx_lens[b], a.n_ctx));
  const int s0 = split * a.split_len;
  const int s1 = min(len, s0 + a.split_len);
  const int ntok = max(0, s1 - s0);
  const int nchunk = (ntok + TOK * TPC - 1) / (TOK * TPC);
  const int nfull = ntok / (TOK * TPC);

  // ---- fold the query: q~ = W_up,k,t[content]^T q[content], beta = q[content] . mu_k,t ----
  {
    const float* q = a.q + unit * D;
    const T* W = static_cast<const T*>(a.w_up_k) + static_cast<size_t>(t * a.H + h) * D * RK;
    const size_t mu_off = a.variant == 0 ? static_cast<size_t>(h * a.T + t) * D
                                         : static_cast<size_t>(t * a.H + h) * D;
    const T* mu = static_cast<const T*>(a.mu_k) + mu_off;
    const float sc = a.scale_log2e;
    for (int r = lane; r < RK; r += 64) {
      float acc = 0.f;
#pragma unroll 8
      for (int i = DR; i < D; ++i) acc += q[i] * load_scalar(W + static_cast<size_t>(i) * RK + r);
      qs[r] = acc * sc;
    }
    float bp = 0.f;
    for (int i = DR + lane; i < D; i += 64) bp += q[i] * load_scalar(mu + i);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) bp += shfl_xor(bp, m);
    if (lane == 0) qs[L::BETA] = bp * sc;
    for (int i = lane; i < DR; i += 64) qs[L::ROT + i] = q[i] * sc;
  }
  __syncthreads();
  // this lane's slice of the folded query, in its row-unit order
  const float* qv = qs;
  float qk[NK], qr[NR];
#pragma unroll
  for (int e = 0; e < NK; ++e) qk[e] = qv[row_elem<T, G>(e, hi)];
#pragma unroll
  for (int e = 0; e < NR; ++e) qr[e] = qv[L::ROT + row_elem<T, G>(e, hi)];
  const float beta = hi == 0 ? qv[L::BETA] : 0.f;  // added once per token

  const char* ck = static_cast<const char*>(a.c_k) + (static_cast<size_t>(b * a.Hc + hc) * a.n_max) * RK * ES;
  const char* kr = static_cast<const char*>(k_rope) + (static_cast<size_t>(b * a.H + h) * a.n_max) * DR * ES;
  const char* cv = static_cast<const char*>(a.c_v) + (static_cast<size_t>(b * a.Hc + hc) * a.n_max) * RV * ES;

  auto load_chunk = [&](Rows& R, int c) {
    const int tok0 = s0 + c * TPC * TOK;
    const bool clamp = c >= nfull;
#pragma unroll
    for (int tt = 0; tt < TPC; ++tt) {
      const int row0 = tok0 + TOK * tt + lo;
      const size_t row = static_cast<size_t>(clamp ? min(row0, s1 - 1) : row0);
      load_piece<T, NK, G>(R.k[tt], ck + row * (RK * ES), hi);
      load_piece<T, NR, G>(R.r[tt], kr + row * (DR * ES), hi);
      load_piece<T, NV, G>(R.v[tt], cv + row * (RV * ES), hi);
    }
  };

  float m_run = kMaxInit, l_run = 0.f;
  float acc[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) acc[e] = 0.f;

  auto compute_chunk = [&](int c, const Rows& R, auto full) {
    constexpr bool FULL = decltype(full)::value;
#pragma unroll
    for (int tt = 0; tt < TPC; ++tt) {
      float part = beta;
#pragma unroll
      for (int e = 0; e < NK; ++e) part += qk[e] * elem(R.k[tt], e);
#pragma unroll
      for (int e = 0; e < NR; ++e) part += qr[e] * elem(R.r[tt], e);
      part = sum_groups<G>(part);
      const int tok = s0 + (c * TPC + tt) * TOK + lo;
      const float s = (FULL || tok < s1) ? part : kNegInf;
      const bool raise = s > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = raise ? s : m_run;
        const float alpha = raise ? fast_exp2(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < NV; ++e) acc[e] *= alpha;
        m_run = m_new;
      }
      const float p = fast_exp2(s - m_run);
      l_run += p;
#pragma unroll
      for (int e = 0; e < NV; ++e) acc[e] += p * elem(R.v[tt], e);
    }
  };
  auto compute = [&](int c, const Rows& R) {
    if (c < nfull) compute_chunk(c, R, std::true_type{});
    else compute_chunk(c, R, std::false_type{});
  };

  // two row buffers used in turn: chunk c computes from one while chunk c + 1 loads
  Rows ra, rb;
  if (nchunk > 0) load_chunk(ra, 0);
  for (int c = 0; c < nchunk; c += 2) {
    if (c + 1 < nchunk) load_chunk(rb, c + 1);
    compute(c, ra);
    if (c + 1 >= nchunk) break;
    if (c + 2 < nchunk) load_chunk(ra, c + 2);
    compute(c + 1, rb);
  }

  // ---- merge the TOK token columns --------------------------------------------------
  float mx = m_run;
#pragma unroll
  for (int msk = 1; msk < TOK; msk <<= 1) mx = fmaxf(mx, shfl_xor(mx, msk));
  const float scl = fast_exp2(m_run - mx);
  float lsum = l_run * scl;
#pragma unroll
  for (int msk = 1; msk < TOK; msk <<= 1) lsum += shfl_xor(lsum, msk);
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    float v = acc[e] * scl;
#pragma unroll
    for (int msk = 1; msk < TOK; msk <<= 1) v += shfl_xor(v, msk);
    acc[e] = v;
  }

  if (a.S > 1) {
    float* out = a.part + (unit * a.S + split) * (2 + RV);
    if (lo == 0) {
#pragma unroll
      for (int e = 0; e < NV; ++e) out[2 + row_elem<T, G>(e, hi)] = acc[e];
      if (hi == 0) {
        out[0] = mx;
        out[1] = lsum;
      }
    }
    return;
  }

  // ---- single split: out = (acc / sum) W_up,v,t^T + mu_v,t -----------------------------
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  if (lo == 0) {
#pragma unroll
    for (int e = 0; e < NV; ++e) abar[row_elem<T, G>(e, hi)] = acc[e] * inv;
  }
  __syncthreads();
  const T* Wv = static_cast<const T*>(a.w_up_v) + static_cast<size_t>(t * a.H + h) * D * RV;
  const size_t muv_off = a.variant == 0 ? static_cast<size_t>(h * a.T + t) * D
                                        : static_cast<size_t>(t * a.H + h) * D;
  const T* muv = static_cast<const T*>(a.mu_v) + muv_off;
  float* out = a.out + unit * D;
#pragma unroll
  for (int k = 0; k < D / 64; ++k) {
    const int i = lane + 64 * k;
    float o = 0.f;
    if (lsum > 0.f) {
      const T* wrow = Wv + static_cast<size_t>(i) * RV;
#pragma unroll 4
      for (int r = 0; r < RV; ++r) o += abar[r] * load_scalar(wrow + r);
      o += load_scalar(muv + i);
    }
    out[i] = o;
  }
}

template <typename T, int D, int RK, int RV, int DR, int G, int TPC>
void launch(const DecodeArgs& a, const void* k_rope, hipStream_t s) {
  hipLaunchKernelGGL((decode_absorbed_kernel<T, D, RK, RV, DR, G, TPC>), dim3(a.S, a.H * a.L, a.B),
                     dim3(64), 0, s, a, k_rope);
}

}  // namespace

#ifndef LLA_ABS_WIDE_TPC
#define LLA_ABS_WIDE_TPC 2  // tiles per chunk for the wide (8 lane group) shapes
#endif

// (dtype, d, r_k, r_v, d_rope, lane groups, tiles per chunk)
#define LLA_ABSORBED_SHAPES(X)                        \
  X(bf16_t, 1, 128, 96, 160, 32, 8, LLA_ABS_WIDE_TPC) \
  X(bf16_t, 1, 128, 96, 160, 64, 8, LLA_ABS_WIDE_TPC) \
  X(bf16_t, 1, 128, 96, 160, 96, 8, LLA_ABS_WIDE_TPC) \
  X(bf16_t, 1, 128, 16, 32, 32, 4, 4)  \
  X(bf16_t, 1, 128, 16, 32, 64, 4, 2)  \
  X(bf16_t, 1, 64, 16, 32, 32, 4, 4)   \
  X(float, 0, 64, 16, 24, 16, 4, 2)    \
  X(float, 0, 64, 16, 24, 32, 4, 2)

bool decode_absorbed_supported(int dtype, int d, int r_k, int r_v, int d_rope) {
#define X(T_, DT_, D_, RK_, RV_, DR_, G_, TPC_) \
  if (dtype == DT_ && d == D_ && r_k == RK_ && r_v == RV_ && d_rope == DR_) return true;
  LLA_ABSORBED_SHAPES(X)
#undef X
  return false;
}

bool launch_decode_absorbed(int dtype, int d, int r_k, int r_v, int d_rope, const DecodeArgs& a,
                            const void* k_rope, hipStream_t s) {
#define X(T_, DT_, D_, RK_, RV_, DR_, G_, TPC_)                                    \
  if (dtype == DT_ && d == D_ && r_k == RK_ && r_v == RV_ && d_rope == DR_) {      \
    launch<T_, D_, RK_, RV_, DR_, G_, TPC_>(a, k_rope, s);                         \
    return true;                                                                   \
  }
  LLA_ABSORBED_SHAPES(X)
#undef X
  return false;
}

}  // namespace lla
