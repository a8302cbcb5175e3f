// Latent-store decode for LLA-2D ("Looped Latent Attention", Section 3, "The LLA-2D
// variant"): one latent row per (sequence, token) serves every head, so the value side of
// attention is a true matrix product, P (heads x tokens) times the value latents (tokens x
// r_v), and runs on the matrix cores here (gfx950, wave64, bfloat16 cache and codec).
//
// Scores use the rotary-fold rewrite of the per-head kernels (Eq. 3 and "RoPE and
// reconstruction": RoPE of the reconstructed key at the slot index): for head h the score
// of token j is c_j . G_j + G_j[r_k], G_j = CS_j M_h, where M_h is built from q, W_up,k,(t,h)
// and the (t, h) slice of mu_k, and CS_j holds cos and sin of the slot's angles. G^T is an
// f16 MFMA product with all of M_h^T in one wave's registers (the value side needs only a
// few accumulator registers here), so a head's scores need no exchange between waves; the
// wave keeps one running max for its head.
//
// Value side (Appendix J, "Absorbed attention": the attention weights sum to one, so the
// weighted value latent can be up-projected once): per 16-token tile the softmax weights of
// the workgroup's heads are written to LDS as bfloat16, and acc[h][r] += sum_j p[h][j] c_v[j][r]
// is one v_mfma_f32_16x16x16_bf16 per 16 value entries, spread over the workgroup's waves.
// The running sum adds the same rounded weights, so the result is an exact weighted mean
// with weights rounded to bfloat16. The value product of tile c runs in the iteration of
// tile c + 1, after the barrier that publishes tile c + 1's rows, so each tile costs one
// workgroup barrier and the matrix-core work of one tile overlaps the vector work of the
// next.
//
// Workgroup: HG heads (one wave each) of one (sequence, loop, split). Cache rows and
// cos/sin tiles stream through a 4-stage direct-to-LDS ring two tiles ahead; the value
// rows of a stage are still read one iteration after its scores. Workgroups of one
// (sequence, loop, split) sit on the same XCD, so the shared latent rows come from HBM once.
// With a paged cache a 16-token tile is one page of the pool, named by the block table
// (the split's page indices are read into LDS before the ring starts); positions and the
// table of angles follow the logical token index, so the arithmetic is the dense one.
#include "lla_device.h"
#include "lla_kernels.h"

#ifndef LLA_2D_WAVES_PER_EU
#define LLA_2D_WAVES_PER_EU 2
#endif
#ifndef LLA_2D_ENABLE
#define LLA_2D_ENABLE 1  // 0 leaves dense LLA-2D to the wide fold kernel
#endif

namespace lla {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMaxInit = -1.0e30f;  // finite stand-in for -inf: the first valid score raises it
constexpr float kRescaleSlack = 8.0f;  // raise the running max only when exceeded by 2^8
constexpr int kXcds = 8;
constexpr int kStages = 4;  // ring depth: two tiles in flight, one computed, one read late

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_f16(const f16x8_t& a, const f16x8_t& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Barrier inside the ring loop: only this wave's LDS traffic has to be complete (the
// ring's direct-to-LDS loads are waited for explicitly with vmcnt), and a
// __syncthreads() fence would wait for every load in flight.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// max over the 16 lanes of each row group (DPP: swap neighbours, swap pairs, mirror
// halves of 8, mirror the 16)
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  const int o = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xf, 0xf, false);
  // med3(v, o, +inf) = max(v, o) for the finite and -inf scores here, without the NaN
  // quieting that fmaxf adds to each operand
  return __builtin_amdgcn_fmed3f(v, __int_as_float(o), __builtin_huge_valf());
}
__device__ __forceinline__ float max16(float v) {
  v = dpp_max<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_max<0x141>(v);  // row_half_mirror
  return dpp_max<0x140>(v);  // row_mirror
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [N - 3, N] (its loads of one tile): tile c has
// landed once only the n loads of tile c + 1 are outstanding
template <int N>
__device__ __forceinline__ void wait_loads(int n) {
  static_assert(N >= 3 && N <= 63, "vmcnt range");
  if (n >= N) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  else if (n == N - 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N - 1) : "memory");
  else if (n == N - 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N - 2) : "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N - 3) : "memory");
}

#ifndef LLA_2D_WAVE_SPECIALIZE
#define LLA_2D_WAVE_SPECIALIZE 1
#endif

// f(std::integral_constant<int, w>) for a wave-uniform w in [I, N): the tile loop compiled
// once per wave of the workgroup, so which ring blocks and value tiles a wave owns are
// compile-time constants
template <int I, int N, class F>
__device__ __forceinline__ void with_wave(int w, F& f) {
  if constexpr (I + 1 < N) {
    if (w == I) f(std::integral_constant<int, I>{});
    else with_wave<I + 1, N>(w, f);
  } else {
    f(std::integral_constant<int, I>{});
  }
}

template <int D, int RK, int RV, int HG, bool PAGED>
__global__ __launch_bounds__(64 * HG) __attribute__((amdgpu_waves_per_eu(LLA_2D_WAVES_PER_EU)))
void decode_lla2d_kernel(DecodeArgs a, PageArgs pg) {
  constexpr int NW = HG;                   // waves: one per head
  constexpr int NKS = D / 32;              // K steps of the score MFMA
  constexpr int NCK = RK / 16;             // latent row tiles of M^T
  constexpr int NT = NCK + 1;              // MFMA row tiles: the latent rows and the mean row
  constexpr int NRT = RV / 16;             // value tiles of 16 entries
  constexpr int VT = (NRT + NW - 1) / NW;  // value tiles per wave (wave w owns w, w + NW, ..)
  constexpr int WT_STRIDE = D + 8;
  // ring stage: key rows (16 x KSP slots of 16 B, one padding slot), value rows, cos/sin tile
  constexpr int KSL = RK / 8, KSP = KSL + 1;
  constexpr int VSL = RV / 8, VSP = VSL + 1;
  constexpr int NIK = (16 * KSP + 63) / 64;
  constexpr int NIV = (16 * VSP + 63) / 64;
  constexpr int STAGE_BLOCKS = NIK + NIV + NKS;  // 1 KiB blocks
  constexpr int RING_UNITS = kStages * STAGE_BLOCKS * 64;
  constexpr int P_UNITS = 2 * 16 * 16 * 2 / 16;
  constexpr int AL_UNITS = 2 * 16 * 4 / 16;
  constexpr int PAGE_UNITS = PAGED ? kMaxSplitPages * 4 / 16 : 0;  // the split's page indices
  constexpr int LDS_UNITS = RING_UNITS + P_UNITS + AL_UNITS + PAGE_UNITS;
  static_assert(NW * 16 * WT_STRIDE * 2 / 16 <= RING_UNITS, "prologue staging fits the ring");
  static_assert(HG * RV + 2 * HG <= RING_UNITS * 4, "epilogue staging fits the ring");
  static_assert(RK % 16 == 0 && RV % 16 == 0 && D % 32 == 0 && HG <= 16, "shape");
  static_assert((NIK + NW - 1) / NW + (NIV + NW - 1) / NW + (NKS + NW - 1) / NW <= 31, "vmcnt range");
  // the last wave issues the fewest loads per tile, NIK / NW + NIV / NW + NKS / NW, at
  // least NSLOT - 3 (the range wait_loads covers)
  static_assert((NIK + NW - 1) / NW + (NIV + NW - 1) / NW + (NKS + NW - 1) / NW -
                        (NIK / NW + NIV / NW + NKS / NW) <= 3, "load counts");

  __shared__ u32x4 lds[LDS_UNITS];
  uint16_t* ptile = reinterpret_cast<uint16_t*>(lds + RING_UNITS);                 // [2][16][16]
  float* alpha_buf = reinterpret_cast<float*>(lds + RING_UNITS + P_UNITS);           // [2][16]
  int* split_pages = reinterpret_cast<int*>(lds + RING_UNITS + P_UNITS + AL_UNITS);  // [pages]

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, hi = lane >> 4;
  const int hw = wave;  // head within the workgroup

  // (sequence, loop, split) units are dealt to XCDs round robin; the H / HG workgroups of
  // one unit take consecutive slots of the same XCD
  const int groups = a.H / HG;
  const int L = static_cast<int>(blockIdx.x);
  const int xcd = L % kXcds;
  const int slot = L / kXcds;
  const int unit = xcd + kXcds * (slot / groups);
  const int hg = slot % groups;
  const int split = unit % a.S;
  const int li = (unit / a.S) % a.L;
  const int b = unit / (a.S * a.L);
  if (b >= a.B) return;  // padding workgroups of the last round
  const int h = hg * HG + hw;
  const int t = a.loop_begin + li;

  int len = a.n_ctx;
  if (a.ctx_lens != nullptr) len = max(0, min(a.ctx_lens[b], a.n_ctx));
  const int s0 = split * a.split_len;
  const int s1 = min(len, s0 + a.split_len);
  const int ntok = max(0, s1 - s0);
  const int ntile = (ntok + 15) >> 4;
  const int nfull = ntok >> 4;

  // ---- M^T fragments of this head (scaled by scale * log2 e), via an LDS transpose ----
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.w_up_k) + static_cast<size_t>(t * a.H + h) * D * RK;
  const uint16_t* mu = reinterpret_cast<const uint16_t*>(a.mu_k) + static_cast<size_t>(t * a.H + h) * D;
  const float* q = a.q + (static_cast<size_t>(b * a.H + h) * a.L + li) * D;
  const float sc = a.scale_log2e;
  uint16_t* wt = reinterpret_cast<uint16_t*>(lds) + wave * 16 * WT_STRIDE;
  f16x8_t mf[NT][NKS];
#pragma unroll
  for (int i = 0; i < NT; ++i) {  // latent row tiles, then the mean row (tile NCK)
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      const int c = lane + 64 * k;  // model dimension
      if (i < NCK) {
        const u32x4* src = reinterpret_cast<const u32x4*>(W + static_cast<size_t>(c) * RK + 16 * i);
        const u32x4 x0 = src[0], x1 = src[1];
        const uint32_t w8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          wt[(2 * j) * WT_STRIDE + c] = static_cast<uint16_t>(w8[j] & 0xffffu);
          wt[(2 * j + 1) * WT_STRIDE + c] = static_cast<uint16_t>(w8[j] >> 16);
        }
      } else {
        // the mean row alone in its tile (row 0), the other rows zero
        wt[c] = mu[c];
#pragma unroll
        for (int j = 1; j < 16; ++j) wt[j * WT_STRIDE + c] = 0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks2 = 0; ks2 < NKS / 2; ++ks2) {
      const int p0 = 32 * ks2 + 8 * hi;  // rotary pair index
      const u32x4* wrow = reinterpret_cast<const u32x4*>(wt + lo * WT_STRIDE + 2 * p0);
      const u32x4 y0 = wrow[0], y1 = wrow[1];
      const uint32_t wp[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x0 = __uint_as_float(wp[e] << 16);
        const float x1 = __uint_as_float(wp[e] & 0xffff0000u);
        const float2 qp = *reinterpret_cast<const float2*>(q + 2 * (p0 + e));
        mf[i][ks2][e] = static_cast<_Float16>((qp.x * x0 + qp.y * x1) * sc);
        mf[i][ks2 + NKS / 2][e] = static_cast<_Float16>((qp.y * x0 - qp.x * x1) * sc);
      }
    }
    __syncthreads();
  }

  // ---- ring set-up: per block slot of this wave, its source and the step per tile ----
  // dense: the sequence's plane; paged: the pool (a page's 16 rows are contiguous, Hc = 1)
  const size_t plane = PAGED ? 0 : static_cast<size_t>(b) * a.n_max;
  const char* ck = reinterpret_cast<const char*>(a.c_k) + plane * RK * 2;
  const char* cv = reinterpret_cast<const char*>(a.c_v) + plane * RV * 2;
  const char* tab_g = reinterpret_cast<const char*>(a.rope16);
  const int tile_max = s1 > 0 ? (s1 - 1) >> 4 : 0;
  // Block slots of this wave by kind: NSK key, NSV value and NST table slots; slot j of a
  // kind loads block wave + NW j of it, if the kind has that many blocks (waves with fewer
  // blocks issue fewer loads per tile). Per slot this lane keeps the token row it loads and
  // its byte offset in the tile (row * row size + column).
  constexpr int NSK = (NIK + NW - 1) / NW, NSV = (NIV + NW - 1) / NW, NST = (NKS + NW - 1) / NW;
  constexpr int NSLOT = NSK + NSV + NST;
  int kblk[NSK], krow[NSK], vblk[NSV], vrow[NSV], tblk[NST];
  uint32_t koff[NSK], voff[NSV], toff[NST];
#pragma unroll
  for (int j = 0; j < NSK; ++j) {
    const int bi = min(wave + NW * j, NIK - 1);
    const int sidx = bi * 64 + lane;
    kblk[j] = bi;
    krow[j] = min(sidx / KSP, 15);
    koff[j] = static_cast<uint32_t>(krow[j] * (RK * 2) + min(sidx % KSP, KSL - 1) * 16);
  }
#pragma unroll
  for (int j = 0; j < NSV; ++j) {
    const int bi = min(wave + NW * j, NIV - 1);
    const int sidx = bi * 64 + lane;
    vblk[j] = NIK + bi;
    vrow[j] = min(sidx / VSP, 15);
    voff[j] = static_cast<uint32_t>(vrow[j] * (RV * 2) + min(sidx % VSP, VSL - 1) * 16);
  }
#pragma unroll
  for (int j = 0; j < NST; ++j) {
    const int bi = min(wave + NW * j, NKS - 1);
    tblk[j] = NIK + NIV + bi;
    toff[j] = static_cast<uint32_t>(bi * 1024 + lane * 16);
  }
  auto dma = [&](const char* src, u32x4* dst) {
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                     (void __attribute__((address_space(3)))*)dst, 16, 0, 0);
  };
  if constexpr (PAGED) {
    for (int i = static_cast<int>(threadIdx.x); i < ntile; i += 64 * NW)
      split_pages[i] = page_of(pg, b, (s0 >> 4) + i);
    __syncthreads();
  }
  // page of tile tl of the split (tiles past the last use the last one's)
  auto page_for = [&](int tl) {
    return PAGED ? __builtin_amdgcn_readfirstlane(split_pages[min(tl, ntile - 1)]) : 0;
  };
  int page_next = PAGED && ntile > 0 ? page_for(0) : 0;  // read one issue ahead
  // Sources are a wave-uniform base plus this lane's 32-bit offset. Tiles past the last
  // (the ring's run-out) load the last tile's rows again.
  auto issue = [&](auto wc, int tl) {
    const int W = wc;
    auto has = [&](int j, int blocks) { return W + NW * j < blocks; };
    u32x4* stage = lds + (tl % kStages) * STAGE_BLOCKS * 64;
    const char* tb = tab_g + static_cast<size_t>(min((s0 >> 4) + tl, tile_max)) * (NKS * 1024);
#pragma unroll
    for (int j = 0; j < NST; ++j)
      if (has(j, NKS)) dma(tb + toff[j], stage + tblk[j] * 64);
    // first row of the tile (tiles past the last: of the last tile) in the sequence's plane,
    // or the first row of the tile's page in the pool
    const int tlc = min(tl, ntile - 1);
    const size_t row0 = PAGED ? static_cast<size_t>(16) * page_next : static_cast<size_t>(s0 + 16 * tlc);
    const char* kb = ck + row0 * (RK * 2);
    const char* vb = cv + row0 * (RV * 2);
    if (tl < nfull) {
#pragma unroll
      for (int j = 0; j < NSK; ++j)
        if (has(j, NIK)) dma(kb + koff[j], stage + kblk[j] * 64);
#pragma unroll
      for (int j = 0; j < NSV; ++j)
        if (has(j, NIV)) dma(vb + voff[j], stage + vblk[j] * 64);
    } else {  // rows past the context end clamp to its last token (they get zero weight)
      const int t0 = s0 + 16 * tlc;
#pragma unroll
      for (int j = 0; j < NSK; ++j) {
        const int d = min(t0 + krow[j], s1 - 1) - t0 - krow[j];  // <= 0 rows
        if (has(j, NIK))
          dma(kb + static_cast<uint32_t>(static_cast<int>(koff[j]) + d * (RK * 2)), stage + kblk[j] * 64);
      }
#pragma unroll
      for (int j = 0; j < NSV; ++j) {
        const int d = min(t0 + vrow[j], s1 - 1) - t0 - vrow[j];
        if (has(j, NIV))
          dma(vb + static_cast<uint32_t>(static_cast<int>(voff[j]) + d * (RV * 2)), stage + vblk[j] * 64);
      }
    }
    if constexpr (PAGED) page_next = page_for(tl + 1);
  };

  float m_run = kMaxInit;  // this head's running max (exp2 domain), the same in every lane
  float l_run = 0.f;       // this lane's token column's share of the running sum
  f32x4 vacc[VT];          // acc[heads 4 hi .. 4 hi + 3][value entry 16 rt + lo]
#pragma unroll
  for (int k = 0; k < VT; ++k) vacc[k] = f32x4{0.f, 0.f, 0.f, 0.f};

  // value product of tile cc: rescale by the tile's alphas, then acc += P(cc) C_v(cc)
  auto value_step = [&](auto wc, int cc) {
    const int W = wc;
    const char* vreg = reinterpret_cast<const char*>(lds + (cc % kStages) * STAGE_BLOCKS * 64 + NIK * 64);
    const f32x4 al = *reinterpret_cast<const f32x4*>(alpha_buf + (cc & 1) * 16 + 4 * hi);
    const i16x4 pa = *reinterpret_cast<const i16x4*>(ptile + (cc & 1) * 256 + lo * 16 + 4 * hi);
    // all of this wave's value fragments are read before the first product (a value tile
    // past the last reads the last one and is not used)
    i16x4 vb[VT];
#pragma unroll
    for (int k = 0; k < VT; ++k) {
      const char* col = vreg + (16 * min(W + NW * k, NRT - 1) + lo) * 2 + 4 * hi * (VSP * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) vb[k][i] = *reinterpret_cast<const short*>(col + i * (VSP * 16));
    }
#pragma unroll
    for (int k = 0; k < VT; ++k) {
      if (W + NW * k < NRT) {
        f32x4 acc = vacc[k];
        acc[0] *= al[0];
        acc[1] *= al[1];
        acc[2] *= al[2];
        acc[3] *= al[3];
        vacc[k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb[k], acc, 0, 0, 0);
      }
    }
  };

  // scores of tile c for this head, softmax weights into the P tile
  auto score_step = [&](int c) {
    const u32x4* st = lds + (c % kStages) * STAGE_BLOCKS * 64;
    const char* kreg = reinterpret_cast<const char*>(st);
    const u32x4* treg = st + (NIK + NIV) * 64;
    f32x4 g[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) g[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const f16x8_t bf = __builtin_bit_cast(f16x8_t, treg[ks * 64 + lane]);
#pragma unroll
      for (int i = 0; i < NT; ++i) g[i] = mfma_f16(mf[i][ks], bf, g[i]);
    }
    // element 0 of the last tile: the mean row for hi = 0, a zero row elsewhere
    float pp = g[NT - 1][0];
#pragma unroll
    for (int m = 0; m < NCK; ++m) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(kreg + lo * (KSP * 16) + 32 * m + 8 * hi);
      pp += __uint_as_float(w.x << 16) * g[m][0] + __uint_as_float(w.x & 0xffff0000u) * g[m][1] +
            __uint_as_float(w.y << 16) * g[m][2] + __uint_as_float(w.y & 0xffff0000u) * g[m][3];
    }
    const float full = sum_xor32(sum_xor16(pp));
    const float s = lo < s1 - s0 - 16 * c ? full : kNegInf;
    float alpha = 1.f;
    // the head's max is raised (to the tile's max) only when a score exceeds it by 2^8;
    // every lane of the wave holds the same head, so the branch is uniform
    if (__builtin_amdgcn_ballot_w64(s > m_run + kRescaleSlack) != 0) {
      const float mt = max16(s);
      alpha = fast_exp2(m_run - mt);
      l_run *= alpha;
      m_run = mt;
    }
    const uint16_t pb = __builtin_bit_cast(uint16_t, static_cast<__bf16>(fast_exp2(s - m_run)));
    l_run += bf16_to_f32(pb);
    if (hi == 0) ptile[(c & 1) * 256 + hw * 16 + lo] = pb;
    if (lane == 0) alpha_buf[(c & 1) * 16 + hw] = alpha;
  };

  // heads past HG: unit alphas and zero weights, so their accumulator rows stay zero
  if (threadIdx.x < 32) alpha_buf[threadIdx.x] = 1.f;
  for (int i = static_cast<int>(threadIdx.x); i < 2 * (16 - HG) * 16; i += 64 * HG)
    ptile[(i / ((16 - HG) * 16)) * 256 + HG * 16 + i % ((16 - HG) * 16)] = 0;
  auto ring_loop = [&](auto wc) {
    const int W = wc;
    int nl = 0;  // this wave's loads per tile
#pragma unroll
    for (int j = 0; j < NSK; ++j) nl += W + NW * j < NIK;
#pragma unroll
    for (int j = 0; j < NSV; ++j) nl += W + NW * j < NIV;
#pragma unroll
    for (int j = 0; j < NST; ++j) nl += W + NW * j < NKS;
    issue(wc, 0);
    issue(wc, 1);
    for (int c = 0; c <= ntile; ++c) {
        // tile c has landed once only tile c + 1's loads are outstanding; the barrier then
        // publishes every wave's blocks of tile c and the weights of tile c - 1, and tells
        // that tile c - 2's stage is free for tile c + 2
        wait_loads<NSLOT>(nl);
        ring_barrier();
        issue(wc, c + 2);
        if (c > 0) value_step(wc, c - 1);
        if (c < ntile) score_step(c);
    }
  };
  if (ntile > 0) {
#if LLA_2D_WAVE_SPECIALIZE
    with_wave<0, NW>(wave, ring_loop);
#else
    ring_loop(wave);
#endif
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may land in the reused LDS
  __syncthreads();

  // ---- epilogue: the head's sum, the accumulated latent through LDS ----
  float lsum = l_run;
#pragma unroll
  for (int msk = 1; msk < 16; msk <<= 1) lsum += shfl_xor(lsum, msk);
  float* abar = reinterpret_cast<float*>(lds);  // [HG][RV]
  float* stats = abar + HG * RV;                // [HG][2]: max, sum
#pragma unroll
  for (int k = 0; k < VT; ++k) {
    const int rt = wave + NW * k;
    if (rt < NRT) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * hi + i < HG) abar[(4 * hi + i) * RV + 16 * rt + lo] = vacc[k][i];
    }
  }
  if (lane == 0) {
    stats[2 * hw] = m_run;
    stats[2 * hw + 1] = lsum;
  }
  __syncthreads();
  const float* arow = abar + hw * RV;
  const size_t uidx = static_cast<size_t>(b * a.H + h) * a.L + li;
  if (a.S > 1) {
    float* out = a.part + (uidx * a.S + split) * (2 + RV);
    for (int r = lane; r < RV; r += 64) out[2 + r] = arow[r];
    if (lane == 0) {
      out[0] = stats[2 * hw];
      out[1] = stats[2 * hw + 1];
    }
    return;
  }
  // single split: out = (acc / sum) W_up,v,(t,h)^T + mu_v,(t,h)
  const float l_tot = stats[2 * hw + 1];
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const uint16_t* Wv = reinterpret_cast<const uint16_t*>(a.w_up_v) + static_cast<size_t>(t * a.H + h) * D * RV;
  const uint16_t* muv = reinterpret_cast<const uint16_t*>(a.mu_v) + static_cast<size_t>(t * a.H + h) * D;
  float* out = a.out + uidx * D;
  for (int i = lane; i < D; i += 64) {
    float o = 0.f;
    if (l_tot > 0.f) {
#pragma unroll 4
      for (int r0 = 0; r0 < RV; r0 += 8) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(Wv + static_cast<size_t>(i) * RV + r0);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
          o += arow[r0 + 2 * k2] * __uint_as_float(ws[k2] << 16);
          o += arow[r0 + 2 * k2 + 1] * __uint_as_float(ws[k2] & 0xffff0000u);
        }
      }
      o = o * inv + bf16_to_f32(muv[i]);
    }
    out[i] = o;
  }
}

template <int D, int RK, int RV, int HG, bool PAGED>
void launch(const DecodeArgs& a, const PageArgs& pg, hipStream_t s) {
  const long long units = static_cast<long long>(a.B) * a.L * a.S;
  const long long rounds = (units + kXcds - 1) / kXcds;
  const long long blocks = rounds * kXcds * (a.H / HG);
  hipLaunchKernelGGL((decode_lla2d_kernel<D, RK, RV, HG, PAGED>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * HG), 0, s, a, pg);
}

}  // namespace

// Heads per workgroup: LLA_2D_HG when H is a multiple of it (one workgroup per CU, the
// stage's rows shared by more heads), else LLA_2D_HG_MIN, which H must be a multiple of.
#ifndef LLA_2D_HG
#define LLA_2D_HG 8
#endif
#ifndef LLA_2D_HG_MIN
#define LLA_2D_HG_MIN 4
#endif
// M^T of (r_k + 16) x d float16 stays in one wave's registers: r_k <= 96 at d = 128
#define LLA_2D_SHAPES(X) \
  X(128, 96, 160)        \
  X(128, 64, 64)

bool decode_lla2d_supported(int dtype, int d, int r_k, int r_v, int H) {
  if (!LLA_2D_ENABLE || dtype != 1 || H % LLA_2D_HG_MIN != 0) return false;
#define X(D_, RK_, RV_) \
  if (d == D_ && r_k == RK_ && r_v == RV_) return true;
  LLA_2D_SHAPES(X)
#undef X
  return false;
}

bool launch_decode_lla2d(int dtype, int d, int r_k, int r_v, const DecodeArgs& a, hipStream_t s) {
  if (a.variant != 1 || !decode_lla2d_supported(dtype, d, r_k, r_v, a.H)) return false;
#define X(D_, RK_, RV_)                                      \
  if (d == D_ && r_k == RK_ && r_v == RV_) {                 \
    if (a.H % LLA_2D_HG == 0)                                \
      launch<D_, RK_, RV_, LLA_2D_HG, false>(a, PageArgs{}, s); \
    else                                                     \
      launch<D_, RK_, RV_, LLA_2D_HG_MIN, false>(a, PageArgs{}, s); \
    return true;                                             \
  }
  LLA_2D_SHAPES(X)
#undef X
  return false;
}

bool launch_decode_lla2d_paged(int dtype, int d, int r_k, int r_v, const DecodeArgs& a,
                               const PageArgs& pg, hipStream_t s) {
  if (a.variant != 1 || pg.table == nullptr || !decode_lla2d_supported(dtype, d, r_k, r_v, a.H))
    return false;
#define X(D_, RK_, RV_)                                \
  if (d == D_ && r_k == RK_ && r_v == RV_) {           \
    if (a.H % LLA_2D_HG == 0)                          \
      launch<D_, RK_, RV_, LLA_2D_HG, true>(a, pg, s); \
    else                                               \
      launch<D_, RK_, RV_, LLA_2D_HG_MIN, true>(a, pg, s); \
    return true;                                       \
  }
  LLA_2D_SHAPES(X)
#undef X
  return false;
}

}  // namespace lla
