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
//   unit's W_up,k,t rows are read from L2, shared by the unit's splits). A token's c_v,
//   c_k and k_rope rows are cut into 16-byte pieces, numbered c_v first, then c_k, then
//   k_rope, and 16 consecutive lanes take the token's pieces j, j + 16, j + 32, ... (one
//   load instruction per round), so a round reads whole rows, or long runs of them, of 4
//   consecutive tokens. A lane's key pieces meet the matching slice of the folded query,
//   the 16 partial dots of a token are summed with DPP, and the per-token-slot online
//   softmax (max raised only past a 2^8 slack, exact) accumulates every piece with the
//   token's weight; only the value pieces are kept. One split finishes with the value
//   up-projection in the epilogue, more go through combine_kernel. The rows of the next
//   TPC tiles are loaded (non-temporal) while the current ones are computed, and chunks
//   wholly inside the context skip the clamping and masking. (Lanes that each took every
//   G-th 8-byte unit of a row read 8 G contiguous bytes per row and instruction and ran at
//   5.2 TB/s; whole rows per round run at 6.8 TB/s.)
//   With a paged cache a chunk (16 tokens) is one page: the latent rows and the rotary keys
//   of its tokens come from the page the block table names for it (the split's page
//   indices are read into LDS first), at the same offsets within the page as the dense
//   rows within a tile, so the arithmetic is the dense one.
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

// Row-piece layout: a token's c_v, c_k and k_rope rows are cut into 16-byte pieces,
// numbered c_v first, then c_k, then k_rope, and the token's 16 consecutive lanes take
// pieces j, j + 16, j + 32, ... (one load instruction per round). A round thus reads whole
// rows or long runs of them for 4 consecutive tokens, instead of 8 G contiguous bytes of
// each row. A lane's score pieces meet the matching slice of the folded query; the 16
// partial dots of a token are summed with DPP; every piece is also accumulated with the
// softmax weight, and only the value pieces are kept at the end.
template <typename T, int D, int RK, int RV, int DR, int TPC, bool PAGED>
__global__ __launch_bounds__(64) void decode_absorbed_kernel(DecodeArgs a, const void* k_rope,
                                                             PageArgs pg) {
  using L = QaLayout<RK, DR>;
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr int EPL = 16 / ES;                  // row elements per 16-byte piece
  constexpr int GP = 16, TOK = 64 / GP;         // lanes per token, tokens per tile
  constexpr int NPV = RV / EPL, NPK = RK / EPL, NPR = DR / EPL;
  constexpr int NP = NPV + NPK + NPR;
  constexpr int NRND = (NP + GP - 1) / GP;      // pieces per lane (rounds)
  static_assert(RV % EPL == 0 && RK % EPL == 0 && DR % EPL == 0, "whole 16-byte pieces");
  static_assert(!PAGED || TPC * TOK == kPage, "a chunk is one page");
  struct Rows {
    u32x4 x[TPC][NRND];
  };
  __shared__ float abar[RV];
  __shared__ float qs[QaLayout<RK, DR>::QS];
  __shared__ int split_pages[PAGED ? kMaxSplitPages : 1];  // page of each chunk of the split

  const int lane = threadIdx.x;
  const int tok = lane / GP, j = lane % GP;
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

  // ---- fold the query (as decode_absorbed_kernel) ----------------------------------------
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

  // ---- this lane's pieces: source, row stride and the query slice they meet --------------
  // dense: the (b, hc) latent plane and the (b, h) rotary-key plane; paged: the head's rows
  // within a page of the pool (a page holds Hc latent heads' and H rotary heads' 16 rows)
  const size_t lrow = PAGED ? static_cast<size_t>(hc) * kPage : static_cast<size_t>(b * a.Hc + hc) * a.n_max;
  const size_t rrow = PAGED ? static_cast<size_t>(h) * kPage : static_cast<size_t>(b * a.H + h) * a.n_max;
  const char* ck = static_cast<const char*>(a.c_k) + lrow * RK * ES;
  const char* kr = static_cast<const char*>(k_rope) + rrow * DR * ES;
  const char* cv = static_cast<const char*>(a.c_v) + lrow * RV * ES;
  const char* src[NRND];
  int stride[NRND];
  size_t pstep[NRND];  // bytes from one page of the pool to the next
  bool live[NRND];
  float qp[NRND][EPL];
#pragma unroll
  for (int u = 0; u < NRND; ++u) {
    const int p = j + GP * u;
    live[u] = p < NP;
    if (p < NPV) {
      src[u] = cv + p * 16;
      stride[u] = RV * ES;
      pstep[u] = static_cast<size_t>(a.Hc) * kPage * RV * ES;
    } else if (p < NPV + NPK) {
      src[u] = ck + (p - NPV) * 16;
      stride[u] = RK * ES;
      pstep[u] = static_cast<size_t>(a.Hc) * kPage * RK * ES;
    } else {
      src[u] = kr + (min(p, NP - 1) - NPV - NPK) * 16;
      stride[u] = DR * ES;
      pstep[u] = static_cast<size_t>(a.H) * kPage * DR * ES;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float qv = 0.f;
      if (p >= NPV && p < NPV + NPK) qv = qs[(p - NPV) * EPL + e];
      else if (p >= NPV + NPK && p < NP) qv = qs[L::ROT + (p - NPV - NPK) * EPL + e];
      qp[u][e] = qv;
    }
  }
  const float beta = j == 0 ? qs[L::BETA] : 0.f;  // added once per token

  if constexpr (PAGED) {
    for (int i = lane; i < min(nchunk, kMaxSplitPages); i += 64)
      split_pages[i] = page_of(pg, b, (s0 >> 4) + i);
    __syncthreads();
  }
  auto load_chunk = [&](Rows& R, int c) {
    const int tok0 = s0 + c * TPC * TOK;
    const bool clamp = c >= nfull;
    // paged: the chunk's page; rows are then counted from its first token
    const size_t page =
        PAGED ? static_cast<size_t>(__builtin_amdgcn_readfirstlane(split_pages[min(c, kMaxSplitPages - 1)])) : 0;
#pragma unroll
    for (int tt = 0; tt < TPC; ++tt) {
      const int row0 = tok0 + TOK * tt + tok;
      const int rc = clamp ? min(row0, s1 - 1) : row0;
      const size_t row = static_cast<size_t>(PAGED ? rc - tok0 : rc);
#pragma unroll
      for (int u = 0; u < NRND; ++u)
        R.x[tt][u] = live[u] ? load16(src[u] + page * pstep[u] + row * stride[u]) : u32x4{0u, 0u, 0u, 0u};
    }
  };

  float m_run = kMaxInit, l_run = 0.f;
  float acc[NRND][EPL];
#pragma unroll
  for (int u = 0; u < NRND; ++u)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[u][e] = 0.f;

  auto compute_chunk = [&](int c, const Rows& R, auto full) {
    constexpr bool FULL = decltype(full)::value;
#pragma unroll
    for (int tt = 0; tt < TPC; ++tt) {
      float part = beta;
#pragma unroll
      for (int u = 0; u < NRND; ++u)
#pragma unroll
        for (int e = 0; e < EPL; ++e) part += qp[u][e] * elem16<T>(R.x[tt][u], e);
      part = sum_lanes<GP>(part);
      const int tk = s0 + (c * TPC + tt) * TOK + tok;
      const float s = (FULL || tk < s1) ? part : kNegInf;
      const bool raise = s > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = raise ? s : m_run;
        const float alpha = raise ? fast_exp2(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int u = 0; u < NRND; ++u)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[u][e] *= alpha;
        m_run = m_new;
      }
      const float pw = fast_exp2(s - m_run);
      l_run += pw;
#pragma unroll
      for (int u = 0; u < NRND; ++u)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[u][e] += pw * elem16<T>(R.x[tt][u], e);
    }
  };
  auto compute = [&](int c, const Rows& R) {
    if (c < nfull) compute_chunk(c, R, std::true_type{});
    else compute_chunk(c, R, std::false_type{});
  };

  Rows ra, rb;
  if (nchunk > 0) load_chunk(ra, 0);
  for (int c = 0; c < nchunk; c += 2) {
    if (c + 1 < nchunk) load_chunk(rb, c + 1);
    compute(c, ra);
    if (c + 1 >= nchunk) break;
    if (c + 2 < nchunk) load_chunk(ra, c + 2);
    compute(c + 1, rb);
  }

  // ---- merge the TOK token slots -------------------------------------------------------
  float mx = m_run;
#pragma unroll
  for (int msk = GP; msk < 64; msk <<= 1) mx = fmaxf(mx, shfl_xor(mx, msk));
  const float scl = fast_exp2(m_run - mx);
  float lsum = l_run * scl;
#pragma unroll
  for (int msk = GP; msk < 64; msk <<= 1) lsum += shfl_xor(lsum, msk);
#pragma unroll
  for (int u = 0; u < NRND; ++u)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float v = acc[u][e] * scl;
#pragma unroll
      for (int msk = GP; msk < 64; msk <<= 1) v += shfl_xor(v, msk);
      acc[u][e] = v;
    }

  if (a.S > 1) {
    float* out = a.part + (unit * a.S + split) * (2 + RV);
    if (tok == 0) {
#pragma unroll
      for (int u = 0; u < NRND; ++u) {
        const int p = j + GP * u;
        if (p < NPV) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) out[2 + p * EPL + e] = acc[u][e];
        }
      }
      if (j == 0) {
        out[0] = mx;
        out[1] = lsum;
      }
    }
    return;
  }

  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  if (tok == 0) {
#pragma unroll
    for (int u = 0; u < NRND; ++u) {
      const int p = j + GP * u;
      if (p < NPV) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) abar[p * EPL + e] = acc[u][e] * inv;
      }
    }
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

#ifndef LLA_ABS_TPC
#define LLA_ABS_TPC 4  // tiles of 4 tokens per chunk; two chunks are in flight
#endif

template <typename T, int D, int RK, int RV, int DR, bool PAGED>
void launch(const DecodeArgs& a, const void* k_rope, const PageArgs& pg, hipStream_t s) {
  hipLaunchKernelGGL((decode_absorbed_kernel<T, D, RK, RV, DR, LLA_ABS_TPC, PAGED>),
                     dim3(a.S, a.H * a.L, a.B), dim3(64), 0, s, a, k_rope, pg);
}

}  // namespace

// (element type, dtype code, d, r_k, r_v, d_rope)
#define LLA_ABSORBED_SHAPES(X)          \
  X(bf16_t, 1, 128, 96, 160, 32)        \
  X(bf16_t, 1, 128, 96, 160, 64)        \
  X(bf16_t, 1, 128, 96, 160, 96)        \
  X(bf16_t, 1, 128, 16, 32, 32)         \
  X(bf16_t, 1, 128, 16, 32, 64)         \
  X(bf16_t, 1, 64, 16, 32, 32)          \
  X(float, 0, 64, 16, 24, 16)           \
  X(float, 0, 64, 16, 24, 32)

bool decode_absorbed_supported(int dtype, int d, int r_k, int r_v, int d_rope) {
#define X(T_, DT_, D_, RK_, RV_, DR_) \
  if (dtype == DT_ && d == D_ && r_k == RK_ && r_v == RV_ && d_rope == DR_) return true;
  LLA_ABSORBED_SHAPES(X)
#undef X
  return false;
}

bool launch_decode_absorbed(int dtype, int d, int r_k, int r_v, int d_rope, const DecodeArgs& a,
                            const void* k_rope, hipStream_t s) {
#define X(T_, DT_, D_, RK_, RV_, DR_)                                         \
  if (dtype == DT_ && d == D_ && r_k == RK_ && r_v == RV_ && d_rope == DR_) { \
    launch<T_, D_, RK_, RV_, DR_, false>(a, k_rope, PageArgs{}, s);           \
    return true;                                                              \
  }
  LLA_ABSORBED_SHAPES(X)
#undef X
  return false;
}

bool launch_decode_absorbed_paged(int dtype, int d, int r_k, int r_v, int d_rope,
                                  const DecodeArgs& a, const void* k_rope, const PageArgs& pg,
                                  hipStream_t s) {
  if (pg.table == nullptr) return false;
#define X(T_, DT_, D_, RK_, RV_, DR_)                                         \
  if (dtype == DT_ && d == D_ && r_k == RK_ && r_v == RV_ && d_rope == DR_) { \
    launch<T_, D_, RK_, RV_, DR_, true>(a, k_rope, pg, s);                    \
    return true;                                                              \
  }
  LLA_ABSORBED_SHAPES(X)
#undef X
  return false;
}

}  // namespace lla
