// Latent-store decode, reconstruct path (gfx950, wave64).
//
// "Looped Latent Attention" (arXiv 2607.15456v2): Section 3 Eq. 3 rebuilds loop t of a
// cached key as k_t = c W_up,t^T + mu_t; Section 3 "RoPE and reconstruction" rotates the
// rebuilt key with the model's RoPE; Figure 1: attention is otherwise unchanged;
// Appendix J "Absorbed attention": the value side is applied to the softmax-weighted
// latent, so V is never rebuilt per token.
//
// One wave owns one (sequence b, head h, loop t, context split). Per tile of 16 cached
// tokens it
//   1. loads the key latents straight into MFMA B fragments (a tile is one contiguous
//      run of 16 * r_k elements of the (b, h) plane) and the value-latent slice it
//      accumulates,
//   2. rebuilds K^T (d x 16) = W_up,k,t (d x r_k) C^T (r_k x 16) on the matrix cores,
//      seeding the accumulators with mu_k,t so the mean costs nothing,
//   3. rotates each interleaved pair of the rebuilt key by j * theta_i (cos/sin from
//      the float32 table) and dots it with the query in registers; the four lanes that
//      share a token column finish the dot with two xor shuffles,
//   4. keeps a per-column online softmax (running max, running sum, and the
//      softmax-weighted value latent), so no per-tile cross-column reduction is needed.
// At the end of the split the 16 columns are merged (log-sum-exp) and the wave writes
// (max, sum, acc[r_v]) to the workspace; combine.hip merges splits and applies
// W_up,v,t and mu_v,t once per (b, h, t).
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

template <typename T, int D, int RK, int RV, bool PAGED = false>
void launch(const DecodeArgs& a, const PageArgs& pg, hipStream_t s) {
  dim3 grid(a.S, a.H * a.L, a.B);
  hipLaunchKernelGGL((decode_reconstruct_kernel<T, D, RK, RV, PAGED>), grid, dim3(64), 0, s, a, pg);
}

}  // namespace

// Shapes built for the reconstruct path: (d, r_k, r_v).
#define LLA_RECON_SHAPES(X) \
  X(64, 16, 24)             \
  X(64, 16, 32)             \
  X(64, 32, 32)             \
  X(64, 256, 256)           \
  X(128, 16, 32)            \
  X(128, 32, 64)            \
  X(128, 96, 160)           \
  X(128, 128, 128)

bool decode_reconstruct_supported(int dtype, int d, int r_k, int r_v) {
#define X(D_, RK_, RV_) \
  if (d == D_ && r_k == RK_ && r_v == RV_) return true;
  LLA_RECON_SHAPES(X)
#undef X
  (void)dtype;
  return false;
}

bool launch_decode_reconstruct(int dtype, int d, int r_k, int r_v, const DecodeArgs& a,
                               hipStream_t s) {
#define X(D_, RK_, RV_)                                             \
  if (d == D_ && r_k == RK_ && r_v == RV_) {                        \
    if (dtype == 0) launch<float, D_, RK_, RV_>(a, PageArgs{}, s);  \
    else launch<bf16_t, D_, RK_, RV_>(a, PageArgs{}, s);            \
    return true;                                                    \
  }
  LLA_RECON_SHAPES(X)
#undef X
  return false;
}

bool launch_decode_reconstruct_paged(int dtype, int d, int r_k, int r_v, const DecodeArgs& a,
                                     const PageArgs& pg, hipStream_t s) {
  if (pg.table == nullptr) return false;
#define X(D_, RK_, RV_)                                             \
  if (d == D_ && r_k == RK_ && r_v == RV_) {                        \
    if (dtype == 0) launch<float, D_, RK_, RV_, true>(a, pg, s);    \
    else launch<bf16_t, D_, RK_, RV_, true>(a, pg, s);              \
    return true;                                                    \
  }
  LLA_RECON_SHAPES(X)
#undef X
  return false;
}

}  // namespace lla
