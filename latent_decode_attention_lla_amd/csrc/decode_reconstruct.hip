// Latent-store decode, reconstruct path (gfx950, wave64).
//
// "Looped Latent Attention" (arXiv 2607.15456v2): Section 3 Eq. 3 rebuilds loop t of a
// cached key as k_t = c W_up,t^T + mu_t; Section 3 "RoPE and reconstruction" rotates the
// rebuilt key with the model's RoPE; Figure 1: attention is otherwise unchanged;
// Appendix J "Absorbed attention": the value side is applied to the softmax-weighted
// latent, so V is never rebuilt per token.
//
// Both kernels below rebuild every key of the context on the matrix cores: K^T (d x 16
// tokens) = W_up,k,t (d x r_k) C^T (r_k x 16), the accumulators seeded with mu_k,t, then
// rotate the rebuilt key and take its dot with the query, and keep a per-column online
// softmax with the softmax-weighted value latent. At the end of a context split the 16
// token columns are merged (log-sum-exp) and (max, sum, acc[r_v]) go to the workspace;
// combine.hip merges splits and applies W_up,v,t and mu_v,t once per (b, h, t).
//
// bfloat16 cache (decode_reconstruct_bf16_kernel). A workgroup holds HPW heads of one
// (sequence, loop, context split), one wave each, walking the same tokens, TPC tiles of
// 16 per chunk; the next chunk's latent rows are loaded while the current one is
// computed. The rotation uses the float16 cos/sin table that lla_rope_table_build lays
// out in MFMA fragment order; each chunk's slice is staged once in LDS and read by all
// waves. The rows of each rebuilt 16-row tile are chosen so that the lane holding rebuilt
// rows (2i, 2i+1, 2i+2, 2i+3) of a token also holds, in the table's fragment order, the
// cosines and sines of pairs i and i+1 at that token's position. For a pair (k0, k1) of
// the rebuilt key rotated by angle phi and the query pair (q0, q1),
//   q . R(phi) k = q0 (cos k0 - sin k1) + q1 (sin k0 + cos k1)
//                = [q0, q1, q1, -q0] . [cos k0, cos k1, sin k0, sin k1],
// so each lane rounds its four rebuilt entries to float16, forms the eight products with
// cos and sin (four packed multiplies), and one v_mfma_f32_16x16x32_f16 per tile contracts
// them with a query fragment that holds [q0, q1, q1, -q0] per pair (scaled by
// scale * log2 e), the same in all 16 rows, so every row of the result is the score row
// and no cross-lane reduction is needed. The online softmax raises its running max only
// when a score exceeds it by more than 2^8 (exp2 domain), which is exact because the same
// max scales the running sum and the accumulator.
//
// float32 cache (decode_reconstruct_kernel): one wave per (sequence, head, loop, split),
// the rotation of each interleaved pair by j * theta_i from the float32 table and the dot
// with the query in float32 registers; the four lanes that share a token column finish
// the dot with two xor shuffles.
#include <type_traits>

#include "lla_device.h"
#include "lla_kernels.h"

namespace lla {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

template <typename T, int D, int RK, int RV, bool PAGED>
__global__ __launch_bounds__(64) void decode_reconstruct_kernel(DecodeArgs a, PageArgs pg) {
  constexpr int KS = KStep<T, RK>::value;
  using M = Mfma<T, KS>;
  constexpr int E = M::E;
  constexpr int NM = D / 16;   // 16-row tiles of K^T along the head dimension
  constexpr int NK = RK / KS;  // MFMA super-steps over the key latent
  constexpr int VS = RV / 4;   // value-latent entries accumulated per lane
  static_assert(D % 16 == 0 && RK % KS == 0 && RV % 4 == 0, "shape");

  const int lane = threadIdx.x;
  const int lo = lane & 15;  // token column of the tile / row of an A fragment
  const int hi = lane >> 4;  // which 4 rows (of 16) of each K^T tile this lane holds
  const int split = blockIdx.x;
  const int h = blockIdx.y / a.L;
  const int li = blockIdx.y - h * a.L;
  const int b = blockIdx.z;
  const int t = a.loop_begin + li;
  const int hc = a.variant == 0 ? h : 0;

  int len = a.n_ctx;
  if (a.ctx_lens != nullptr) len = max(0, min(a.ctx_lens[b], a.n_ctx));
  const int s0 = split * a.split_len;
  const int s1 = min(len, s0 + a.split_len);

  const T* wk = static_cast<const T*>(a.w_up_k) + static_cast<size_t>(t * a.H + h) * D * RK;
  const size_t mu_off = a.variant == 0 ? static_cast<size_t>(h * a.T + t) * D
                                       : static_cast<size_t>(t * a.H + h) * D;
  const T* muk = static_cast<const T*>(a.mu_k) + mu_off;
  const float* q = a.q + (static_cast<size_t>(b * a.H + h) * a.L + li) * D;

  // Loop-invariant operands: W_up,k,t as A fragments, mu_k,t as accumulator seeds, the
  // query entries matching this lane's accumulator rows.
  typename M::Frag wf[NM][NK];
  f32x4 mu4[NM];
  float qv[NM][4];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) wf[m][ks] = M::load(wk + (16 * m + lo) * RK + ks * KS + hi * E);
    float tmp[4];
    load_f32<4>(muk + 16 * m + 4 * hi, tmp);
    mu4[m] = f32x4{tmp[0], tmp[1], tmp[2], tmp[3]};
    load_f32<4>(q + 16 * m + 4 * hi, qv[m]);
  }

  // dense: this (sequence, latent head)'s plane; paged: its rows of page 0 of the pool
  const size_t plane = PAGED ? static_cast<size_t>(hc) * kPage : static_cast<size_t>(b * a.Hc + hc) * a.n_max;
  const T* ck = static_cast<const T*>(a.c_k) + plane * RK;
  const T* cv = static_cast<const T*>(a.c_v) + plane * RV;

  float m_run = kNegInf, l_run = 0.f;
  float acc[VS];
#pragma unroll
  for (int e = 0; e < VS; ++e) acc[e] = 0.f;

  for (int j0 = s0; j0 < s1; j0 += 16) {
    const int tok = j0 + lo;
    const bool valid = tok < s1;
    const int row = valid ? tok : s1 - 1;

    // a tile (j0 a multiple of 16) is one page; its clamped rows stay in it
    const T* ckt = ck;
    const T* cvt = cv;
    int prow = row;
    if constexpr (PAGED) {
      const size_t page = static_cast<size_t>(page_of(pg, b, __builtin_amdgcn_readfirstlane(j0 / kPage)));
      ckt = ck + page * a.Hc * kPage * RK;
      cvt = cv + page * a.Hc * kPage * RV;
      prow = row - j0;
    }
    typename M::Frag cf[NK];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) cf[ks] = M::load(ckt + static_cast<size_t>(prow) * RK + ks * KS + hi * E);
    float vv[VS];
    load_f32<VS>(cvt + static_cast<size_t>(prow) * RV + hi * VS, vv);

    const float* cs_row = a.rope32 + static_cast<size_t>(row) * D;  // (cos, sin) x D/2
    float part = 0.f;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      f32x4 kt = mu4[m];
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) kt = M::mma(wf[m][ks], cf[ks], kt);
      // rows 16m + 4hi + {0,1} form pair 8m + 2hi, rows {2,3} pair 8m + 2hi + 1
      const float4 cs = *reinterpret_cast<const float4*>(cs_row + 2 * (8 * m + 2 * hi));
      const float* qq = qv[m];
      part += cs.x * (qq[0] * kt[0] + qq[1] * kt[1]) + cs.y * (qq[1] * kt[0] - qq[0] * kt[1]);
      part += cs.z * (qq[2] * kt[2] + qq[3] * kt[3]) + cs.w * (qq[3] * kt[2] - qq[2] * kt[3]);
    }
    part += shfl_xor(part, 16);
    part += shfl_xor(part, 32);

    const float s = valid ? part * a.scale_log2e : kNegInf;
    const float m_new = fmaxf(m_run, s);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    const float p = fast_exp2(s - m_use);
    l_run = l_run * alpha + p;
#pragma unroll
    for (int e = 0; e < VS; ++e) acc[e] = acc[e] * alpha + p * vv[e];
    m_run = m_new;
  }

  // Merge the 16 token columns of each lane group (log-sum-exp).
  float mx = m_run;
#pragma unroll
  for (int msk = 1; msk < 16; msk <<= 1) mx = fmaxf(mx, shfl_xor(mx, msk));
  const float sc = (mx == kNegInf) ? 0.f : fast_exp2(m_run - mx);
  float lsum = l_run * sc;
#pragma unroll
  for (int msk = 1; msk < 16; msk <<= 1) lsum += shfl_xor(lsum, msk);
#pragma unroll
  for (int e = 0; e < VS; ++e) {
    float v = acc[e] * sc;
#pragma unroll
    for (int msk = 1; msk < 16; msk <<= 1) v += shfl_xor(v, msk);
    acc[e] = v;
  }
  float* out = a.part + ((static_cast<size_t>(b * a.H + h) * a.L + li) * a.S + split) * (2 + RV);
  if (lo == 0) {
#pragma unroll
    for (int e = 0; e < VS; ++e) out[2 + hi * VS + e] = acc[e];
    if (hi == 0) {
      out[0] = mx;
      out[1] = lsum;
    }
  }
}

// ---------------------------------------------------------------------------
// bfloat16 cache
// ---------------------------------------------------------------------------
constexpr float kMaxInit = -1.0e30f;  // finite stand-in for -inf as a starting running max
constexpr float kRescaleSlack = 8.0f;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#ifndef LLA_RECON_HPW
#define LLA_RECON_HPW 4    // heads (waves) per workgroup when H is a multiple of it
#endif
#ifndef LLA_RECON_TPC16
#define LLA_RECON_TPC16 4  // 16-token tiles per chunk for (d, r_k, r_v) = (128, 16, 32)
#endif
#ifndef LLA_RECON_WAVES_PER_EU
#define LLA_RECON_WAVES_PER_EU 0  // 0: let the compiler choose
#endif
#ifndef LLA_RECON_TAB_DMA
#define LLA_RECON_TAB_DMA 1  // 1: dense caches' cos/sin tiles go straight to LDS
#endif
#ifndef LLA_RECON_NT
#define LLA_RECON_NT 1  // 1: stream cache rows with non-temporal loads
#endif

template <typename V>
__device__ __forceinline__ V row_load(const V* p) {
#if LLA_RECON_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

// One lane's cache rows for a chunk of TPC tiles: the rebuild's B fragments of the key
// latent (NK super-steps of E entries) and the lane's VS value-latent entries, as raw
// bfloat16 pairs.
template <int NK, int E, int VS, int TPC>
struct ReconRows {
  uint32_t k[TPC][NK][E / 2];
  uint32_t v[TPC][VS / 2];
};

// Loads tile tt's rows for token row pointers krow (key latent) and vrow (value latent).
template <int KS, int NK, int E, int VS, int TPC>
__device__ __forceinline__ void load_recon_rows(ReconRows<NK, E, VS, TPC>& R, int tt,
                                                const uint16_t* krow, const uint16_t* vrow,
                                                int hi) {
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    const uint16_t* kp = krow + ks * KS + hi * E;
    if constexpr (E == 4) {
      const u32x2 x = row_load(reinterpret_cast<const u32x2*>(kp));
      R.k[tt][ks][0] = x.x;
      R.k[tt][ks][1] = x.y;
    } else {
      const u32x4 x = row_load(reinterpret_cast<const u32x4*>(kp));
#pragma unroll
      for (int i = 0; i < 4; ++i) R.k[tt][ks][i] = x[i];
    }
  }
  const uint16_t* vp = vrow + hi * VS;
  if constexpr (VS % 8 == 0) {
#pragma unroll
    for (int i = 0; i < VS / 8; ++i) {
      const u32x4 x = row_load(reinterpret_cast<const u32x4*>(vp + 8 * i));
#pragma unroll
      for (int j = 0; j < 4; ++j) R.v[tt][4 * i + j] = x[j];
    }
  } else if constexpr (VS % 4 == 0) {
#pragma unroll
    for (int i = 0; i < VS / 4; ++i) {
      const u32x2 x = row_load(reinterpret_cast<const u32x2*>(vp + 4 * i));
      R.v[tt][2 * i] = x.x;
      R.v[tt][2 * i + 1] = x.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < VS / 2; ++i) R.v[tt][i] = row_load(reinterpret_cast<const uint32_t*>(vp + 2 * i));
  }
}

template <int D, int RK, int RV, int HPW, int TPC, bool PAGED>
__global__ __launch_bounds__(64 * HPW)
#if LLA_RECON_WAVES_PER_EU
__attribute__((amdgpu_waves_per_eu(LLA_RECON_WAVES_PER_EU)))
#endif
void decode_reconstruct_bf16_kernel(DecodeArgs a, PageArgs pg) {
  constexpr int KS = KStep<bf16_t, RK>::value;
  using M = Mfma<bf16_t, KS>;
  constexpr int E = M::E;
  constexpr int NK = RK / KS;        // rebuild super-steps over the key latent
  constexpr int NM = D / 16;         // 16-row tiles of the rebuilt K^T
  constexpr int NCP = D / 64;        // cosine pieces (8 pairs each) per lane and tile
  constexpr int NKS = D / 32;        // table pieces per lane and tile: cosines, then sines
  constexpr int VS = RV / 4;         // value-latent entries per lane
  constexpr int NTHR = 64 * HPW;
  constexpr int TAB_CHUNK = TPC * NKS * 64;  // 16-byte table units per chunk
  constexpr int TPT = (TAB_CHUNK + NTHR - 1) / NTHR;
  constexpr bool kTabEven = TAB_CHUNK % NTHR == 0;
  static_assert(D % 64 == 0 && RK % KS == 0 && RV % 8 == 0, "shape");
  using Rows = ReconRows<NK, E, VS, TPC>;

  __shared__ u32x4 lds[2 * TAB_CHUNK];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, hi = lane >> 4;
  const int split = blockIdx.x;
  const int groups = a.H / HPW;
  const int li = blockIdx.y / groups;
  const int h = (blockIdx.y - li * groups) * HPW + wave;
  const int b = blockIdx.z;
  const int t = a.loop_begin + li;
  const int hc = a.variant == 0 ? h : 0;

  int len = a.n_ctx;
  if (a.ctx_lens != nullptr) len = max(0, min(a.ctx_lens[b], a.n_ctx));
  const int s0 = split * a.split_len;
  const int s1 = min(len, s0 + a.split_len);
  const int ntok = max(0, s1 - s0);
  const int nchunk = (ntok + 16 * TPC - 1) / (16 * TPC);
  const int nfull = ntok / (16 * TPC);  // chunks whose tokens are all in the context
  const int tile_max = (s1 > 0 ? (s1 - 1) >> 4 : 0);

  // ---- loop-invariant operands --------------------------------------------------------
  // Tile m (kap = m / 4, w = m % 4) holds, for lane group g, rebuilt rows
  // 64 kap + 16 g + 4 w + {0..3}: pairs p = 32 kap + 8 g + 2 w and p + 1, whose cosines
  // are the two float16 entries of dword w of the lane's cosine piece kap in the table
  // (sines: piece NCP + kap). Row r of the tile is head-dim row
  // 64 kap + 16 (r / 4) + 4 w + r % 4, which is what the A fragment loads.
  const bf16_t* wk = static_cast<const bf16_t*>(a.w_up_k) + static_cast<size_t>(t * a.H + h) * D * RK;
  const size_t mu_off = a.variant == 0 ? static_cast<size_t>(h * a.T + t) * D
                                       : static_cast<size_t>(t * a.H + h) * D;
  const bf16_t* muk = static_cast<const bf16_t*>(a.mu_k) + mu_off;
  const float* q = a.q + (static_cast<size_t>(b * a.H + h) * a.L + li) * D;
  const float sc = a.scale_log2e;
  typename M::Frag wf[NM][NK];
  f32x4 mu4[NM];
  f16x8 qa[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int kap = m >> 2, w = m & 3;
    const int arow = 64 * kap + 16 * (lo >> 2) + 4 * w + (lo & 3);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) wf[m][ks] = M::load(wk + static_cast<size_t>(arow) * RK + ks * KS + hi * E);
    const int r0 = 64 * kap + 16 * hi + 4 * w;
    float tmp[4];
    load_f32<4>(muk + r0, tmp);
    mu4[m] = f32x4{tmp[0], tmp[1], tmp[2], tmp[3]};
    const float4 qq = *reinterpret_cast<const float4*>(q + r0);
    const float q0 = qq.x * sc, q1 = qq.y * sc, q2 = qq.z * sc, q3 = qq.w * sc;
    qa[m] = f16x8{static_cast<_Float16>(q0), static_cast<_Float16>(q1),
                  static_cast<_Float16>(q2), static_cast<_Float16>(q3),
                  static_cast<_Float16>(q1), static_cast<_Float16>(-q0),
                  static_cast<_Float16>(q3), static_cast<_Float16>(-q2)};
  }

  // dense: this (sequence, latent head)'s plane; paged: its rows of page 0 of the pool
  const size_t plane = PAGED ? static_cast<size_t>(hc) * kPage : static_cast<size_t>(b * a.Hc + hc) * a.n_max;
  const uint16_t* ck = static_cast<const uint16_t*>(a.c_k) + plane * RK;
  const uint16_t* cv = static_cast<const uint16_t*>(a.c_v) + plane * RV;
  const u32x4* tab_g = reinterpret_cast<const u32x4*>(a.rope16);

  float m_run = kMaxInit, l_run = 0.f;
  float acc[VS];
#pragma unroll
  for (int e = 0; e < VS; ++e) acc[e] = 0.f;

  auto compute_chunk = [&](int c, const Rows& R, const u32x4* tcur, auto full) {
    constexpr bool FULL = decltype(full)::value;
#pragma unroll
    for (int tt = 0; tt < TPC; ++tt) {
      const int tok = s0 + (c * TPC + tt) * 16 + lo;
      uint32_t tp[NKS][4];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u32x4 x = tcur[(tt * NKS + ks) * 64 + lane];
        tp[ks][0] = x.x;
        tp[ks][1] = x.y;
        tp[ks][2] = x.z;
        tp[ks][3] = x.w;
      }
      f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = sa;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int kap = m >> 2, w = m & 3;
        f32x4 kt = mu4[m];
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          typename M::Frag cf;
          if constexpr (E == 4) cf.v = __builtin_bit_cast(i16x4, u32x2{R.k[tt][ks][0], R.k[tt][ks][1]});
          else cf.v = __builtin_bit_cast(bf16x8, u32x4{R.k[tt][ks][0], R.k[tt][ks][1], R.k[tt][ks][2], R.k[tt][ks][3]});
          kt = M::mma(wf[m][ks], cf, kt);
        }
        const f16x2 cw = __builtin_bit_cast(f16x2, tp[kap][w]);
        const f16x2 sw = __builtin_bit_cast(f16x2, tp[NCP + kap][w]);
        const f16x2 k01 = f16x2{static_cast<_Float16>(kt[0]), static_cast<_Float16>(kt[1])};
        const f16x2 k23 = f16x2{static_cast<_Float16>(kt[2]), static_cast<_Float16>(kt[3])};
        const f16x2 b01 = k01 * cw.xx, b23 = k23 * cw.yy;
        const f16x2 b45 = k01 * sw.xx, b67 = k23 * sw.yy;
        const f16x8 bf = f16x8{b01.x, b01.y, b23.x, b23.y, b45.x, b45.y, b67.x, b67.y};
        if (m & 1) sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[m], bf, sb, 0, 0, 0);
        else sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[m], bf, sa, 0, 0, 0);
      }
      const float s = (FULL || tok < s1) ? sa[0] + sb[0] : kNegInf;

      // online softmax for this lane's token column, lazily rescaled
      const bool raise = s > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = raise ? s : m_run;
        const float alpha = raise ? fast_exp2(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < VS; ++e) acc[e] *= alpha;
        m_run = m_new;
      }
      const float p = fast_exp2(s - m_run);
      l_run += p;
#pragma unroll
      for (int e = 0; e < VS / 2; ++e) {
        const uint32_t x = R.v[tt][e];
        acc[2 * e] += p * __uint_as_float(x << 16);
        acc[2 * e + 1] += p * __uint_as_float(x & 0xffff0000u);
      }
    }
  };

  // Paged: the pages of a chunk's tiles are looked up one chunk ahead of the rows that
  // need them (uniform over the workgroup; rows clamped to the context's last token lie
  // in the last tile's page).
  struct Pages {
    int p[TPC];
  };
  auto fetch_pages = [&](int c) {
    Pages P;
#pragma unroll
    for (int tt = 0; tt < TPC; ++tt) {
      const int ptile = min((s0 >> 4) + c * TPC + tt, tile_max);
      P.p[tt] = page_of(pg, b, __builtin_amdgcn_readfirstlane(ptile));
    }
    return P;
  };

  // CLAMP: rows past the context end re-read its last row (their weights are zero, and
  // the rows themselves may hold anything); full chunks skip the clamp.
  auto load_rows = [&](Rows& R, const Pages& P, int tile0, int tok0, auto clamp) {
    constexpr bool CLAMP = decltype(clamp)::value;
#pragma unroll
    for (int tt = 0; tt < TPC; ++tt) {
      const int row = CLAMP ? min(tok0 + 16 * tt + lo, s1 - 1) : tok0 + 16 * tt + lo;
      const uint16_t* krow;
      const uint16_t* vrow;
      if constexpr (PAGED) {
        const size_t prow = (static_cast<size_t>(P.p[tt]) * a.Hc) * kPage +
                            (row - min(tile0 + tt, tile_max) * kPage);
        krow = ck + prow * RK;
        vrow = cv + prow * RV;
      } else {
        krow = ck + static_cast<size_t>(row) * RK;
        vrow = cv + static_cast<size_t>(row) * RV;
      }
      load_recon_rows<KS>(R, tt, krow, vrow, hi);
    }
  };

  Rows ra, rb;
  u32x4* tab0 = lds;
  u32x4* tab1 = lds + TAB_CHUNK;
  // Dense caches: the chunk's table (TPC * NKS fragment blocks of 1 KiB, contiguous for
  // chunks inside the context) goes to LDS by direct-to-LDS loads dealt to the waves (lane
  // l: bytes 16 l .. 16 l + 15 of a block), complete once the barrier that follows them has
  // been passed. Paged caches stage it through registers (the transfers would queue behind
  // the page-dependent row loads).
  constexpr bool kTabDma = LLA_RECON_TAB_DMA && !PAGED;
  constexpr int TAB_BLOCKS = TPC * NKS;
  constexpr int NBW = (TAB_BLOCKS + HPW - 1) / HPW;  // blocks per wave (surplus ones repeat)
  auto issue_tab = [&](int c, u32x4* dst) {
    const int tile0 = (s0 >> 4) + c * TPC;
#pragma unroll
    for (int k = 0; k < NBW; ++k) {
      const int blk = min(wave + HPW * k, TAB_BLOCKS - 1);
      const int tile = min(tile0 + blk / NKS, tile_max);
      const char* src = reinterpret_cast<const char*>(tab_g) +
                        (static_cast<size_t>(tile) * NKS + blk % NKS) * 1024 + lane * 16;
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                       (void __attribute__((address_space(3)))*)(dst + blk * 64), 16, 0, 0);
    }
  };
  u32x4 tb[kTabDma ? 1 : TPT];
  u32x4* tab_next = tab1;  // where load_chunk puts the table of the chunk it loads
  auto load_chunk = [&](Rows& R, int c, const Pages& P) {
    const int tile0 = (s0 >> 4) + c * TPC;
    const int tok0 = s0 + c * TPC * 16;
    if constexpr (kTabDma) issue_tab(c, tab_next);
    if (c < nfull) {
      if constexpr (!kTabDma) {
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
          const int u = min(k * NTHR + static_cast<int>(threadIdx.x), TAB_CHUNK - 1);
          tb[k] = tab_g[static_cast<size_t>(tile0) * NKS * 64 + u];
        }
      }
      load_rows(R, P, tile0, tok0, std::false_type{});
    } else {
      if constexpr (!kTabDma) {
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
          const int u = min(k * NTHR + static_cast<int>(threadIdx.x), TAB_CHUNK - 1);
          const int tile = min(tile0 + u / (NKS * 64), tile_max);
          tb[k] = tab_g[static_cast<size_t>(tile) * NKS * 64 + (u % (NKS * 64))];
        }
      }
      load_rows(R, P, tile0, tok0, std::true_type{});
    }
  };
  auto store_tab = [&](u32x4* dst) {
    if constexpr (!kTabDma) {
#pragma unroll
      for (int k = 0; k < TPT; ++k) {
        const int u = k * NTHR + static_cast<int>(threadIdx.x);
        if (kTabEven || u < TAB_CHUNK) dst[u] = tb[k];
      }
    }
  };
  auto compute = [&](int c, const Rows& R, const u32x4* tcur) {
    if (c < nfull) compute_chunk(c, R, tcur, std::true_type{});
    else compute_chunk(c, R, tcur, std::false_type{});
  };

  Pages pa{}, pb{};
  if constexpr (PAGED) {
    pa = fetch_pages(0);
    pb = fetch_pages(1);
  }
  if (nchunk > 0) {
    tab_next = tab0;
    load_chunk(ra, 0, pa);
    store_tab(tab0);
  }
  __syncthreads();
  for (int c = 0; c < nchunk; c += 2) {
    // even chunk: compute from (ra, tab0), prefetch into (rb, tab1)
    const bool more1 = c + 1 < nchunk;
    tab_next = tab1;
    if (more1) load_chunk(rb, c + 1, pb);
    if constexpr (PAGED) pa = fetch_pages(c + 2);
    compute(c, ra, tab0);
    if (more1) store_tab(tab1);
    __syncthreads();
    if (!more1) break;
    // odd chunk: compute from (rb, tab1), prefetch into (ra, tab0)
    const bool more2 = c + 2 < nchunk;
    tab_next = tab0;
    if (more2) load_chunk(ra, c + 2, pa);
    if constexpr (PAGED) pb = fetch_pages(c + 3);
    compute(c + 1, rb, tab1);
    if (more2) store_tab(tab0);
    __syncthreads();
  }

  // ---- merge the 16 token columns of each lane group -----------------------------------
  float mx = m_run;
#pragma unroll
  for (int msk = 1; msk < 16; msk <<= 1) mx = fmaxf(mx, shfl_xor(mx, msk));
  const float scl = fast_exp2(m_run - mx);
  float lsum = l_run * scl;
#pragma unroll
  for (int msk = 1; msk < 16; msk <<= 1) lsum += shfl_xor(lsum, msk);
#pragma unroll
  for (int e = 0; e < VS; ++e) {
    float v = acc[e] * scl;
#pragma unroll
    for (int msk = 1; msk < 16; msk <<= 1) v += shfl_xor(v, msk);
    acc[e] = v;
  }
  float* out = a.part + ((static_cast<size_t>(b * a.H + h) * a.L + li) * a.S + split) * (2 + RV);
  if (lo == 0) {
#pragma unroll
    for (int e = 0; e < VS; ++e) out[2 + hi * VS + e] = acc[e];
    if (hi == 0) {
      out[0] = mx;
      out[1] = lsum;
    }
  }
}

template <typename T, int D, int RK, int RV, bool PAGED = false>
void launch_f32(const DecodeArgs& a, const PageArgs& pg, hipStream_t s) {
  dim3 grid(a.S, a.H * a.L, a.B);
  hipLaunchKernelGGL((decode_reconstruct_kernel<T, D, RK, RV, PAGED>), grid, dim3(64), 0, s, a, pg);
}

template <int D, int RK, int RV, int TPC, bool PAGED = false>
void launch_bf16(const DecodeArgs& a, const PageArgs& pg, hipStream_t s) {
  if (a.H % LLA_RECON_HPW == 0) {
    dim3 grid(a.S, (a.H / LLA_RECON_HPW) * a.L, a.B);
    hipLaunchKernelGGL((decode_reconstruct_bf16_kernel<D, RK, RV, LLA_RECON_HPW, TPC, PAGED>), grid,
                       dim3(64 * LLA_RECON_HPW), 0, s, a, pg);
  } else {
    dim3 grid(a.S, a.H * a.L, a.B);
    hipLaunchKernelGGL((decode_reconstruct_bf16_kernel<D, RK, RV, 1, TPC, PAGED>), grid, dim3(64), 0, s,
                       a, pg);
  }
}

}  // namespace

// Shapes built for the reconstruct path: (d, r_k, r_v, 16-token tiles per chunk of the
// bfloat16 kernel).
#define LLA_RECON_SHAPES(X) \
  X(64, 16, 24, 4)          \
  X(64, 16, 32, 4)          \
  X(64, 32, 32, 2)          \
  X(64, 256, 256, 1)        \
  X(128, 16, 32, LLA_RECON_TPC16) \
  X(128, 32, 64, 2)         \
  X(128, 96, 160, 1)        \
  X(128, 128, 128, 1)

bool decode_reconstruct_supported(int dtype, int d, int r_k, int r_v) {
#define X(D_, RK_, RV_, TPC_) \
  if (d == D_ && r_k == RK_ && r_v == RV_) return true;
  LLA_RECON_SHAPES(X)
#undef X
  (void)dtype;
  return false;
}

bool launch_decode_reconstruct(int dtype, int d, int r_k, int r_v, const DecodeArgs& a,
                               hipStream_t s) {
#define X(D_, RK_, RV_, TPC_)                                              \
  if (d == D_ && r_k == RK_ && r_v == RV_) {                               \
    if (dtype == 0) launch_f32<float, D_, RK_, RV_>(a, PageArgs{}, s);     \
    else launch_bf16<D_, RK_, RV_, TPC_>(a, PageArgs{}, s);                \
    return true;                                                           \
  }
  LLA_RECON_SHAPES(X)
#undef X
  return false;
}

bool launch_decode_reconstruct_paged(int dtype, int d, int r_k, int r_v, const DecodeArgs& a,
                                     const PageArgs& pg, hipStream_t s) {
  if (pg.table == nullptr) return false;
#define X(D_, RK_, RV_, TPC_)                                              \
  if (d == D_ && r_k == RK_ && r_v == RV_) {                               \
    if (dtype == 0) launch_f32<float, D_, RK_, RV_, true>(a, pg, s);       \
    else launch_bf16<D_, RK_, RV_, TPC_, true>(a, pg, s);                  \
    return true;                                                           \
  }
  LLA_RECON_SHAPES(X)
#undef X
  return false;
}

}  // namespace lla
