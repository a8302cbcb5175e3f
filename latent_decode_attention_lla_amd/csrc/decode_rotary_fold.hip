// Latent-store decode, rotary-fold path (gfx950, wave64, bfloat16 cache and codec).
//
// Computes exactly the scores of the reconstruct path ("Looped Latent Attention",
// Section 3: k_t = c W_up,t^T + mu_t, then RoPE; attention unchanged) through an exact
// rewrite that moves the rotation onto the matrix cores. For one rotary pair i of a key
// k rotated by angle j*theta_i, and a query q:
//   q . R(j theta_i) k = cos(j theta_i) (q_2i k_2i + q_2i+1 k_2i+1)
//                      + sin(j theta_i) (q_2i+1 k_2i - q_2i k_2i+1).
// Both brackets are linear in the latent c_j, so with
//   M[i][r]       = q_2i W[2i][r] + q_2i+1 W[2i+1][r]          (i <  d/2, cosine rows)
//   M[d/2+i][r]   = q_2i+1 W[2i][r] - q_2i W[2i+1][r]          (sine rows)
//   M[.][r_k]     = the same with mu_t in place of W[.][r]      (the mean's term)
// and CS_j = (cos(j theta_0..), sin(j theta_0..)), the score of token j is
//   s_j = sum_{r < r_k} c_j[r] G_j[r] + G_j[r_k],   G_j = CS_j M   (d x (r_k + 1)).
// CS is the same for every sequence, head and loop; M depends on (b, h, t) only.
// G^T = M^T CS^T runs on v_mfma_f32_16x16x32_f16 with M^T (scaled by scale*log2 e, in
// float16) held in registers for the whole context and CS^T tiles (float16, laid out in
// fragment order by lla_rope_table_build) staged once per workgroup in LDS and shared by
// its waves. The lane that holds G_j[4g .. 4g+3] also holds c_j[4g .. 4g+3] (the same
// layout as a 16x16x16 B fragment of the cache row), so the per-token dot is four FMAs
// and two cross-lane adds. The value side accumulates softmax-weighted value latents
// (Appendix J, "Absorbed attention") and applies W_up,v,t and mu_v,t once at the end.
//
// Workgroup: HPW waves = HPW heads of one (sequence, loop, context split); they walk the
// same token range in chunks of TPC tiles of 16 tokens. The ring instances (DA > 0) keep
// DA chunks of cache rows (registers) and table tiles (LDS) in flight per wave; the
// two-buffer instances (DA = 0) load the next chunk while the current one is computed.
// With a paged cache a 16-token tile is one page: its rows come from the page the block
// table names for it, and everything else (positions, the table of angles) follows the
// logical token index. Each lane keeps an online softmax for its token column; the
// running max is raised only when a score exceeds it by more than 2^8 (scores live in the
// exp2 domain), which is exact because the same max is used by the running sum and the
// accumulator.
#include <type_traits>

#include "lla_device.h"
#include "lla_kernels.h"

namespace lla {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
// Running maxima start at a finite stand-in for -inf: the first valid score always raises
// it (so exp2(s - m) never sees inf - inf), and columns or splits without a valid token
// keep a zero sum, so no per-token test for an empty column is needed.
constexpr float kMaxInit = -1.0e30f;
constexpr float kRescaleSlack = 8.0f;

// Launch-shape knobs (tuned on MI355X; overridable at build time).
#ifndef LLA_FOLD_HPW
#define LLA_FOLD_HPW 4          // heads (waves) per workgroup
#endif
#ifndef LLA_FOLD_TPC16
#define LLA_FOLD_TPC16 4        // 16-token tiles per chunk for r_k = 16
#endif
#ifndef LLA_FOLD_RING_TPC16
#define LLA_FOLD_RING_TPC16 2   // the same, dense caches (ring)
#endif
#ifndef LLA_FOLD_RING_DA16
#define LLA_FOLD_RING_DA16 3    // chunks in flight per wave, r_k = 16, dense caches
#endif
#ifndef LLA_FOLD_NT
#define LLA_FOLD_NT 1           // 1: stream cache rows with non-temporal loads
#endif
#ifndef LLA_FOLD_PERMLANE
#define LLA_FOLD_PERMLANE 1     // 1: cross-lane sums with permlane swaps, 0: LDS shuffles
#endif
#ifndef LLA_FOLD_WAVES_PER_EU
#define LLA_FOLD_WAVES_PER_EU 0  // 0: let the compiler choose
#endif
#ifndef LLA_FOLD_RING
#define LLA_FOLD_RING 1         // 1: dense caches keep several chunks in flight (a ring)
#endif
#ifndef LLA_FOLD_TAB_DMA
#define LLA_FOLD_TAB_DMA 1      // 1: dense caches' cos/sin tiles go straight to LDS
#endif

// Finishes this wave's LDS reads, then waits for the workgroup.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename V>
__device__ __forceinline__ V stream_load(const V* p) {
#if LLA_FOLD_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
// native 16-byte vector (HIP's uint4 is a struct whose copies go through memcpy)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_f16(const f16x8_t& a, const f16x8_t& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Cache rows of one chunk (TPC tiles of 16 tokens) for one lane.
template <int RK, int RV, int TPC>
struct Rows {
  uint2 k[TPC][RK / 16];  // c_k[tok][16 m + 4 g .. +3], bf16
  u32x4 v[TPC][RV / 32];  // c_v[tok][g RV/4 .. +RV/4), bf16, 16 bytes at a time
};

// CLAMP: rows past the context end re-read its last row (their weights are zero, and the
// rows themselves may hold anything); full chunks skip the clamp.
template <bool CLAMP, int RK, int RV, int TPC>
__device__ __forceinline__ void load_rows(Rows<RK, RV, TPC>& R, const uint16_t* ck, const uint16_t* cv,
                                          int tok0, int s1, int lo, int hi) {
#pragma unroll
  for (int tt = 0; tt < TPC; ++tt) {
    const int row = CLAMP ? min(tok0 + 16 * tt + lo, s1 - 1) : tok0 + 16 * tt + lo;
    const uint16_t* kp = ck + static_cast<size_t>(row) * RK + 4 * hi;
#pragma unroll
    for (int m = 0; m < RK / 16; ++m) {
      const u32x2 kk = stream_load(reinterpret_cast<const u32x2*>(kp + 16 * m));
      R.k[tt][m] = make_uint2(kk.x, kk.y);
    }
    const uint16_t* vp = cv + static_cast<size_t>(row) * RV + hi * (RV / 4);
#pragma unroll
    for (int m = 0; m < RV / 32; ++m) R.v[tt][m] = stream_load(reinterpret_cast<const u32x4*>(vp + 8 * m));
  }
}

// Paged: the rows of tile tt are those of the pool's page rows starting at element
// offsets koff[tt] / voff[tt] (wave-uniform), row r of the chunk's tile tt being row
// r - pt0[tt] of its page.
template <bool CLAMP, int RK, int RV, int TPC>
__device__ __forceinline__ void load_rows_paged(Rows<RK, RV, TPC>& R, const uint16_t* kpool,
                                                const uint16_t* vpool, const size_t* koff,
                                                const size_t* voff, const int* pt0, int tok0,
                                                int s1, int lo, int hi) {
#pragma unroll
  for (int tt = 0; tt < TPC; ++tt) {
    const int row = (CLAMP ? min(tok0 + 16 * tt + lo, s1 - 1) : tok0 + 16 * tt + lo) - pt0[tt];
    const uint16_t* kp = kpool + koff[tt] + row * RK + 4 * hi;
#pragma unroll
    for (int m = 0; m < RK / 16; ++m) {
      const u32x2 kk = stream_load(reinterpret_cast<const u32x2*>(kp + 16 * m));
      R.k[tt][m] = make_uint2(kk.x, kk.y);
    }
    const uint16_t* vp = vpool + voff[tt] + row * RV + hi * (RV / 4);
#pragma unroll
    for (int m = 0; m < RV / 32; ++m) R.v[tt][m] = stream_load(reinterpret_cast<const u32x4*>(vp + 8 * m));
  }
}

template <int D, int RK, int RV, int HPW, int TPC, int DA, bool PAGED>
__global__ __launch_bounds__(64 * HPW)
#if LLA_FOLD_WAVES_PER_EU
__attribute__((amdgpu_waves_per_eu(LLA_FOLD_WAVES_PER_EU)))
#endif
void decode_rotary_fold_kernel(DecodeArgs a, PageArgs pg) {
  constexpr int NKS = D / 32;        // k-steps of 32 over the cos|sin index
  constexpr int NMT = RK / 16 + 1;   // row tiles of M^T: r_k latent rows + the mean row
  constexpr int NCK = RK / 16;       // 8-byte key-latent pieces per lane per tile
  constexpr int VS = RV / 4;         // value-latent entries per lane
  constexpr int NTHR = 64 * HPW;
  constexpr int TAB_CHUNK = TPC * NKS * 64;  // 16-byte units of table per chunk
  constexpr int TAB_BLOCKS = TPC * NKS;      // 1 KiB table blocks (MFMA fragments) per chunk
  constexpr bool kRing = DA > 0;  // DA chunks in flight (else the two-buffer loop)
  constexpr int NBWR = (TAB_BLOCKS + HPW - 1) / HPW;  // table blocks per wave per chunk
  static_assert(RK % 16 == 0 && RV % 32 == 0 && D % 32 == 0, "shape");
  constexpr int TPT = (TAB_CHUNK + NTHR - 1) / NTHR;  // table units per thread per chunk
  constexpr bool kTabEven = TAB_CHUNK % NTHR == 0;
  constexpr int WT_STRIDE = D + 8;   // float16 row stride of the transposed W staging
  constexpr int STAGE_UNITS = HPW * 16 * WT_STRIDE * 2 / 16;
  constexpr int TAB_UNITS = (kRing ? DA + 1 : 2) * TAB_CHUNK;
  constexpr int LDS_UNITS = (TAB_UNITS > STAGE_UNITS) ? TAB_UNITS : STAGE_UNITS;
  static_assert(!kRing || DA >= 2, "ring depth");
  constexpr int DAR = kRing ? DA : 2;

  // the ring's paged instances keep the split's pages after the table stages
  constexpr int PAGE_UNITS = (kRing && PAGED) ? kMaxSplitPages / 4 : 0;
  __shared__ u32x4 lds[LDS_UNITS + PAGE_UNITS];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, hi = lane >> 4;
  const int split = blockIdx.x;
  const int groups = a.H / HPW;
  const int li = blockIdx.y / groups;
  const int h = (blockIdx.y - li * groups) * HPW + wave;
  const int b = blockIdx.z;
  const int t = a.loop_begin + li;

  int len = a.n_ctx;
  if (a.ctx_lens != nullptr) len = max(0, min(a.ctx_lens[b], a.n_ctx));
  const int s0 = split * a.split_len;
  const int s1 = min(len, s0 + a.split_len);
  const int ntok = max(0, s1 - s0);
  const int nchunk = (ntok + 16 * TPC - 1) / (16 * TPC);
  const int nfull = ntok / (16 * TPC);  // chunks whose tokens are all in the context

  // ---- M^T fragments (A operand), float16, scaled into the exp2 domain ----------------
  // For each 16-row tile of M^T the wave stages W_up,k,t[:, 16 mt .. 16 mt + 15] (or mu for
  // the mean row) transposed in LDS, then every lane reads the 16 consecutive entries of
  // its row that its 8 pairs need.
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.w_up_k) + static_cast<size_t>(t * a.H + h) * D * RK;
  const uint16_t* mu = reinterpret_cast<const uint16_t*>(a.mu_k) + static_cast<size_t>(h * a.T + t) * D;
  const float* q = a.q + (static_cast<size_t>(b * a.H + h) * a.L + li) * D;
  const float sc = a.scale_log2e;
  uint16_t* wt = reinterpret_cast<uint16_t*>(lds) + wave * 16 * WT_STRIDE;
  f16x8_t mf[NMT][NKS];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    // stage: lane handles head-dim rows c = lane + 64 k
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      const int c = lane + 64 * k;
      if (mt < NCK) {
        const uint4* src = reinterpret_cast<const uint4*>(W + static_cast<size_t>(c) * RK + 16 * mt);
        const uint4 x0 = src[0], x1 = src[1];
        const uint32_t w8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          wt[(2 * j) * WT_STRIDE + c] = static_cast<uint16_t>(w8[j] & 0xffffu);
          wt[(2 * j + 1) * WT_STRIDE + c] = static_cast<uint16_t>(w8[j] >> 16);
        }
      } else {
        wt[c] = mu[c];
#pragma unroll
        for (int j = 1; j < 16; ++j) wt[j * WT_STRIDE + c] = 0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks2 = 0; ks2 < NKS / 2; ++ks2) {
      const int p0 = 32 * ks2 + 8 * hi;  // first of this lane's 8 pairs
      const uint4* wrow = reinterpret_cast<const uint4*>(wt + lo * WT_STRIDE + 2 * p0);
      const uint4 y0 = wrow[0], y1 = wrow[1];
      const uint32_t wp[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};  // (W[2p], W[2p+1])
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x0 = __uint_as_float(wp[e] << 16);
        const float x1 = __uint_as_float(wp[e] & 0xffff0000u);
        const float2 qp = *reinterpret_cast<const float2*>(q + 2 * (p0 + e));
        mf[mt][ks2][e] = static_cast<_Float16>((qp.x * x0 + qp.y * x1) * sc);
        mf[mt][ks2 + NKS / 2][e] = static_cast<_Float16>((qp.y * x0 - qp.x * x1) * sc);
      }
    }
    __syncthreads();
  }

  // dense: this head's plane; paged: this head's rows of page 0 of the pool
  const size_t plane = PAGED ? static_cast<size_t>(h) * kPage : static_cast<size_t>(b * a.H + h) * a.n_max;
  const uint16_t* ck = reinterpret_cast<const uint16_t*>(a.c_k) + plane * RK;
  const uint16_t* cv = reinterpret_cast<const uint16_t*>(a.c_v) + plane * RV;
  const u32x4* tab_g = reinterpret_cast<const u32x4*>(a.rope16);
  const int tile_max = (s1 > 0 ? (s1 - 1) >> 4 : 0);

  float m_run = kMaxInit, l_run = 0.f;
  float acc[VS];
#pragma unroll
  for (int e = 0; e < VS; ++e) acc[e] = 0.f;

  // One chunk: TPC tiles of 16 tokens, from the rows in R and the table in LDS buffer tcur.
  // FULL: every token of the chunk is in the context (no masking).
  auto compute_chunk = [&](int c, const auto& R, const u32x4* tcur, auto full) {
    constexpr bool FULL = decltype(full)::value;
#pragma unroll
    for (int tt = 0; tt < TPC; ++tt) {
      const int tok = s0 + (c * TPC + tt) * 16 + lo;
      f32x4 g[NMT];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) g[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const f16x8_t bf = __builtin_bit_cast(f16x8_t, tcur[(tt * NKS + ks) * 64 + lane]);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) g[mt] = mfma_f16(mf[mt][ks], bf, g[mt]);
      }
      // element 0 of the mean tile is the mean row for hi = 0 and an all-zero padding row
      // of M^T (so exactly 0) for the other lane groups
      float part = g[NMT - 1][0];
#pragma unroll
      for (int m = 0; m < NCK; ++m) {
        const auto w = R.k[tt][m];
        part += __uint_as_float(w.x << 16) * g[m][0] + __uint_as_float(w.x & 0xffff0000u) * g[m][1] +
                __uint_as_float(w.y << 16) * g[m][2] + __uint_as_float(w.y & 0xffff0000u) * g[m][3];
      }
#if LLA_FOLD_PERMLANE
      part = sum_xor32(sum_xor16(part));
#else
      part += shfl_xor(part, 16);
      part += shfl_xor(part, 32);
#endif
      const float s = (FULL || tok < s1) ? part : kNegInf;

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
      for (int m = 0; m < RV / 32; ++m) {
        const u32x4 w = R.v[tt][m];
        acc[8 * m + 0] += p * __uint_as_float(w.x << 16);
        acc[8 * m + 1] += p * __uint_as_float(w.x & 0xffff0000u);
        acc[8 * m + 2] += p * __uint_as_float(w.y << 16);
        acc[8 * m + 3] += p * __uint_as_float(w.y & 0xffff0000u);
        acc[8 * m + 4] += p * __uint_as_float(w.z << 16);
        acc[8 * m + 5] += p * __uint_as_float(w.z & 0xffff0000u);
        acc[8 * m + 6] += p * __uint_as_float(w.w << 16);
        acc[8 * m + 7] += p * __uint_as_float(w.w & 0xffff0000u);
      }
    }
  };

  auto compute = [&](int c, const auto& R, const u32x4* tcur) {
    if (c < nfull) compute_chunk(c, R, tcur, std::true_type{});
    else compute_chunk(c, R, tcur, std::false_type{});
  };

  if constexpr (kRing) {
    // ---- DAR chunks in flight per wave (dense and paged caches) -----------------------
    // Rows go to registers, the chunk's cos/sin blocks to a ring of DAR + 1 LDS stages.
    // Chunk c's loads are issued DAR chunks ahead, at the end of chunk c - DAR's step (rows)
    // and right after its barrier (table); every wave issues the same count per chunk, the
    // chunks past the end included (their addresses clamp to the last row and tile), so a
    // single wait for "at most (DAR - 1) chunks outstanding" means chunk c has landed.
    // The table moves with buffer loads to LDS (MUBUF): a pending FLAT global_load_lds
    // would make the compiler wait for every load in flight before reading any register a
    // plain load wrote. The rows are inline-assembly loads the compiler neither counts
    // nor waits for; the explicit wait orders their use, and hold_rows ties the registers
    // to it (no instruction may touch them between the load and the marker: the built
    // assembly is checked for that).
    constexpr int NVL = RV / 32;
    constexpr int KRB = RK * 2, VRB = RV * 2;  // bytes per latent row
    constexpr int NLC = NBWR + TPC * (NCK + NVL);  // loads per chunk per wave
    static_assert((DAR - 1) * NLC <= 63, "vmcnt range");
    constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
    struct RowsR {
      u32x2 k[TPC][NCK];
      u32x4 v[TPC][NVL];
    };
    // the loads take a scalar base: the head's plane (paged: its rows in page 0 of the
    // pool), each tile's page and first row are formed from wave-uniform values held in
    // scalar registers
    const int hu = __builtin_amdgcn_readfirstlane(h);
    const size_t plane_u = PAGED ? static_cast<size_t>(hu) * kPage : static_cast<size_t>(b * a.H + hu) * a.n_max;
    const char* ckb = reinterpret_cast<const char*>(a.c_k) + plane_u * KRB;
    const char* cvb = reinterpret_cast<const char*>(a.c_v) + plane_u * VRB;
    const size_t kpage = static_cast<size_t>(a.H) * kPage * KRB;  // bytes per page (paged)
    const size_t vpage = static_cast<size_t>(a.H) * kPage * VRB;
    // paged: the pages of a chunk's tiles (rows past the context lie in the last tile's
    // page), looked up with scalar loads before the chunk's compute step and used after it
    struct PagesR {
      int p[TPC];
    };
    // The split's pages are read from the block table into LDS once (at most
    // kMaxSplitPages: the host caps a split's length to that many pages): a lookup is
    // then an LDS read, where a global load here would be a vector load (the inline
    // assembly below clobbers memory, so the compiler cannot use a scalar load) that the
    // compiler would wait for with a vmcnt counting only its own loads, draining the ring.
    int* split_pages = reinterpret_cast<int*>(lds + LDS_UNITS);
    if constexpr (PAGED) {
      const int ntiles = min(tile_max - (s0 >> 4) + 1, kMaxSplitPages);
      for (int i = threadIdx.x; i < ntiles; i += NTHR) split_pages[i] = page_of(pg, b, (s0 >> 4) + i);
      __syncthreads();
    }
    auto pages_of = [&](int c) {
      PagesR P{};
      if constexpr (PAGED) {
#pragma unroll
        for (int tt = 0; tt < TPC; ++tt) {
          const int i = min(min((s0 >> 4) + c * TPC + tt, tile_max) - (s0 >> 4), kMaxSplitPages - 1);
          P.p[tt] = __builtin_amdgcn_readfirstlane(split_pages[__builtin_amdgcn_readfirstlane(i)]);
        }
      }
      return P;
    };
    const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4*>(tab_g), 0, (tile_max + 1) * NKS * 1024, kRsrcWord3);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    auto issue_tab = [&](int c) {
      u32x4* st = lds + (c % (DAR + 1)) * TAB_CHUNK;
      const int tile0 = (s0 >> 4) + c * TPC;
#pragma unroll
      for (int k = 0; k < NBWR; ++k) {
        const int bi = min(wv + HPW * k, TAB_BLOCKS - 1);  // surplus blocks repeat
        const int tile = min(tile0 + bi / NKS, tile_max);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(trs, (__attribute__((address_space(3))) void*)(st + bi * 64), 16,
                                                 (bi % NKS) * 1024 + lane * 16, tile * NKS * 1024, 0, 0);
      }
    };
    auto load_rows_r = [&](RowsR& R, int c, const PagesR& P) {
#pragma unroll
      for (int tt = 0; tt < TPC; ++tt) {
        // the tile's first row (wave-uniform) and this lane's row from it; rows past the
        // context repeat its last one
        const int r0 = __builtin_amdgcn_readfirstlane(min(s0 + 16 * (c * TPC + tt), s1 - 1));
        const int rl = min(lo, s1 - 1 - r0);
        const char* kb = ckb + static_cast<size_t>(r0) * KRB;
        const char* vb = cvb + static_cast<size_t>(r0) * VRB;
        if constexpr (PAGED) {  // a tile is one page; r0 - 16 * tile is its row in the page
          const int pr = r0 - 16 * min((s0 >> 4) + c * TPC + tt, tile_max);
          kb = ckb + static_cast<size_t>(P.p[tt]) * kpage + pr * KRB;
          vb = cvb + static_cast<size_t>(P.p[tt]) * vpage + pr * VRB;
        }
        const uint32_t ko = static_cast<uint32_t>(rl * KRB + 8 * hi);
        const uint32_t vo = static_cast<uint32_t>(rl * VRB + hi * (RV / 2));
#pragma unroll
        for (int m = 0; m < NCK; ++m)
          asm volatile("global_load_dwordx2 %0, %1, %2 offset:%3 nt"
                       : "=v"(R.k[tt][m]) : "v"(ko), "s"(kb), "n"(32 * m) : "memory");
#pragma unroll
        for (int m = 0; m < NVL; ++m)
          asm volatile("global_load_dwordx4 %0, %1, %2 offset:%3 nt"
                       : "=v"(R.v[tt][m]) : "v"(vo), "s"(vb), "n"(16 * m) : "memory");
      }
    };
    auto hold_rows = [&](RowsR& R) {
#pragma unroll
      for (int tt = 0; tt < TPC; ++tt) {
#pragma unroll
        for (int m = 0; m < NCK; ++m) asm volatile("; keys %0" : "+v"(R.k[tt][m]));
#pragma unroll
        for (int m = 0; m < NVL; ++m) asm volatile("; keys %0" : "+v"(R.v[tt][m]));
      }
    };
    auto chunk_step = [&](int c, RowsR& R) {
      // chunk c's rows and table blocks (this wave's) have landed once at most the later
      // DAR - 1 chunks' loads are outstanding; the barrier then makes every wave's blocks
      // visible, and tells that every wave is done with chunk c - 1's stage, which takes
      // chunk c + DAR's table
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DAR - 1) * NLC) : "memory");
      hold_rows(R);
      ring_barrier();
      issue_tab(c + DAR);
      const PagesR P = pages_of(c + DAR);
      compute(c, R, lds + (c % (DAR + 1)) * TAB_CHUNK);
      load_rows_r(R, c + DAR, P);  // the buffer's next chunk, once its rows are used
    };
    if (nchunk > 0) {
      RowsR rr[DAR];
#pragma unroll
      for (int u = 0; u < DAR; ++u) {
        issue_tab(u);
        load_rows_r(rr[u], u, pages_of(u));
      }
      // whole rounds of DAR chunks (each buffer in a fixed place in the round), then the rest
      int c0 = 0;
      for (; c0 + DAR <= nchunk; c0 += DAR) {
#pragma unroll
        for (int u = 0; u < DAR; ++u) chunk_step(c0 + u, rr[u]);
      }
#pragma unroll
      for (int u = 0; u < DAR - 1; ++u) {
        if (c0 + u < nchunk) chunk_step(c0 + u, rr[u]);
      }
      // the requests past the end land before the LDS and the registers are reused
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int u = 0; u < DAR; ++u) hold_rows(rr[u]);
    }
    __syncthreads();
  } else {
  // Two row buffers used in turn: chunk c computes from one while chunk c + 1 loads into
  // the other; the table of chunk c + 1 goes into the other LDS half.
  // Paged rows: the pages of a chunk's tiles (uniform across the workgroup; rows clamped to
  // the context's last token lie in the last tile's page) are read with scalar loads one
  // chunk ahead of the rows that need them, so the lookup is off the loads' issue path.
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
  const int h_u = __builtin_amdgcn_readfirstlane(h);  // the wave's head, in a scalar register
  auto load_paged = [&](Rows<RK, RV, TPC>& R, const Pages& P, int tile0, int tok0, auto clamp) {
    size_t koff[TPC], voff[TPC];
    int pt0[TPC];
#pragma unroll
    for (int tt = 0; tt < TPC; ++tt) {
      const size_t rows = (static_cast<size_t>(P.p[tt]) * a.H + h_u) * kPage;  // page's first row
      koff[tt] = rows * RK;
      voff[tt] = rows * RV;
      pt0[tt] = min(tile0 + tt, tile_max) * kPage;
    }
    load_rows_paged<decltype(clamp)::value, RK, RV, TPC>(
        R, reinterpret_cast<const uint16_t*>(a.c_k), reinterpret_cast<const uint16_t*>(a.c_v), koff,
        voff, pt0, tok0, s1, lo, hi);
  };

  Rows<RK, RV, TPC> ra, rb;
  u32x4* tab0 = lds;
  u32x4* tab1 = lds + TAB_CHUNK;
  // Dense caches: the chunk's table is TPC * NKS blocks of 1 KiB (one MFMA fragment each),
  // contiguous in the table for chunks inside the context; each wave moves its share of the
  // blocks with direct-to-LDS loads (lane l: bytes 16 l .. 16 l + 15 of a block). The loads
  // are complete once the barrier that follows them has been passed (__syncthreads waits
  // for this wave's loads, and every wave reaches it). Paged caches stage the table through
  // registers (measured faster there: the transfers then do not queue behind the
  // page-dependent row loads).
  constexpr bool kTabDma = LLA_FOLD_TAB_DMA && !PAGED;
  constexpr int NBW = NBWR;  // blocks per wave (surplus ones repeat)
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
  auto load_chunk = [&](Rows<RK, RV, TPC>& R, int c, const Pages& P) {
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
      if constexpr (PAGED) load_paged(R, P, tile0, tok0, std::false_type{});
      else load_rows<false, RK, RV, TPC>(R, ck, cv, tok0, s1, lo, hi);
    } else {
      if constexpr (!kTabDma) {
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
          const int u = min(k * NTHR + static_cast<int>(threadIdx.x), TAB_CHUNK - 1);
          const int tile = min(tile0 + u / (NKS * 64), tile_max);
          tb[k] = tab_g[static_cast<size_t>(tile) * NKS * 64 + (u % (NKS * 64))];
        }
      }
      if constexpr (PAGED) load_paged(R, P, tile0, tok0, std::true_type{});
      else load_rows<true, RK, RV, TPC>(R, ck, cv, tok0, s1, lo, hi);
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
  }


  // ---- merge the 16 token columns of each lane group ---------------------------------
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

  const size_t unit = static_cast<size_t>(b * a.H + h) * a.L + li;
  if (a.S > 1) {
    float* out = a.part + (unit * a.S + split) * (2 + RV);
    if (lo == 0) {
#pragma unroll
      for (int e = 0; e < VS; ++e) out[2 + hi * VS + e] = acc[e];
      if (hi == 0) {
        out[0] = mx;
        out[1] = lsum;
      }
    }
    return;
  }

  // ---- single split: finish here, out = (acc / sum) W_up,v,t^T + mu_v,t ---------------
  float* abar = reinterpret_cast<float*>(lds) + wave * RV;
  static_assert(sizeof(lds) >= sizeof(float) * RV * HPW, "LDS reuse for the normalised latent");
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  if (lo == 0) {
#pragma unroll
    for (int e = 0; e < VS; ++e) abar[hi * VS + e] = acc[e] * inv;
  }
  __syncthreads();
  const uint16_t* Wv = reinterpret_cast<const uint16_t*>(a.w_up_v) + static_cast<size_t>(t * a.H + h) * D * RV;
  const uint16_t* muv = reinterpret_cast<const uint16_t*>(a.mu_v) + static_cast<size_t>(h * a.T + t) * D;
  float* out = a.out + unit * D;
#pragma unroll
  for (int k = 0; k < D / 64; ++k) {
    const int i = lane + 64 * k;
    float o = 0.f;
    if (lsum > 0.f) {
#pragma unroll
      for (int r0 = 0; r0 < RV; r0 += 8) {
        const uint4 w = *reinterpret_cast<const uint4*>(Wv + static_cast<size_t>(i) * RV + r0);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
          o += abar[r0 + 2 * k2] * __uint_as_float(ws[k2] << 16);
          o += abar[r0 + 2 * k2 + 1] * __uint_as_float(ws[k2] & 0xffff0000u);
        }
      }
      o += bf16_to_f32(muv[i]);
    }
    out[i] = o;
  }
}

template <int D, int RK, int RV, int HPW, int TPC, int DA, bool PAGED = false>
void launch(const DecodeArgs& a, const PageArgs& pg, hipStream_t s) {
  dim3 grid(a.S, (a.H / HPW) * a.L, a.B);
  hipLaunchKernelGGL((decode_rotary_fold_kernel<D, RK, RV, HPW, TPC, DA, PAGED>), grid, dim3(64 * HPW), 0,
                     s, a, pg);
}

// The ring pipeline, with RHPW heads per workgroup when H allows it (DA = 0: the
// two-buffer loop).
template <int D, int RK, int RV, int TPC, int RTPC, int DA, int RHPW, bool PAGED>
void launch_shape(const DecodeArgs& a, const PageArgs& pg, hipStream_t s) {
  if constexpr (!LLA_FOLD_RING || DA == 0) {
    launch<D, RK, RV, LLA_FOLD_HPW, TPC, 0, PAGED>(a, pg, s);
  } else {
    if (a.H % RHPW == 0) launch<D, RK, RV, RHPW, RTPC, DA, PAGED>(a, pg, s);
    else launch<D, RK, RV, LLA_FOLD_HPW, RTPC, DA, PAGED>(a, pg, s);
  }
}

}  // namespace

// (d, r_k, r_v, tiles per chunk of the two-buffer loop, then of the ring: tiles per
// chunk, chunks in flight (0: no ring, measured no faster for that shape) and heads per
// workgroup when H is a multiple of it); heads per workgroup is otherwise LLA_FOLD_HPW
// (H must be a multiple of it).
// Wider latents go to decode_fold_wide.hip (a pair of waves per head).
#define LLA_FOLD_SHAPES(X)                                                     \
  X(128, 16, 32, LLA_FOLD_TPC16, LLA_FOLD_RING_TPC16, LLA_FOLD_RING_DA16, 8)   \
  X(128, 32, 64, 2, 2, 0, 4)                                                   \
  X(64, 16, 32, 4, 2, 4, 8)                                                    \
  X(64, 32, 32, 2, 1, 4, 8)

bool decode_rotary_fold_supported(int dtype, int d, int r_k, int r_v) {
  if (dtype != 1) return false;
#define X(D_, RK_, RV_, TPC_, RTPC_, DA_, RHPW_) \
  if (d == D_ && r_k == RK_ && r_v == RV_) return true;
  LLA_FOLD_SHAPES(X)
#undef X
  return false;
}

bool launch_decode_rotary_fold(int dtype, int d, int r_k, int r_v, const DecodeArgs& a,
                               hipStream_t s) {
  if (dtype != 1 || a.H % LLA_FOLD_HPW != 0) return false;
#define X(D_, RK_, RV_, TPC_, RTPC_, DA_, RHPW_)                     \
  if (d == D_ && r_k == RK_ && r_v == RV_) {                          \
    launch_shape<D_, RK_, RV_, TPC_, RTPC_, DA_, RHPW_, false>(a, PageArgs{}, s); \
    return true;                                                      \
  }
  LLA_FOLD_SHAPES(X)
#undef X
  return false;
}

bool launch_decode_rotary_fold_paged(int dtype, int d, int r_k, int r_v, const DecodeArgs& a,
                                     const PageArgs& pg, hipStream_t s) {
  if (dtype != 1 || a.H % LLA_FOLD_HPW != 0 || pg.table == nullptr) return false;
#define X(D_, RK_, RV_, TPC_, RTPC_, DA_, RHPW_)                   \
  if (d == D_ && r_k == RK_ && r_v == RV_) {                       \
    launch_shape<D_, RK_, RV_, TPC_, RTPC_, DA_, RHPW_, true>(a, pg, s); \
    return true;                                                   \
  }
  LLA_FOLD_SHAPES(X)
#undef X
  return false;
}

}  // namespace lla
