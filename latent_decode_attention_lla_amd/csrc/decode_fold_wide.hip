// Latent-store decode, rotary-fold path for wide latents (r_k >= 64), per-head and
// LLA-2D (gfx950, wave64, bfloat16 cache and codec).
//
// Same exact rewrite as decode_rotary_fold.hip ("Looped Latent Attention", Section 3
// Eq. 3 and "RoPE and reconstruction"; the value identity of Appendix J "Absorbed
// attention"): the score of token j is c_j . G_j + G_j[r_k] with G_j = CS_j M, M built from
// q, W_up,k,t and mu_k,t; the value side accumulates softmax-weighted value latents and
// applies W_up,v,t and mu_v,t once.
//
// Wide latents do not fit one wave's registers (M alone is (r_k + 1) x d float16), so each
// head is served by a pair of waves that split the latent dimension:
//   half 0: M rows of the first NR0 row tiles,          value entries 0 .. r_v/2-1
//   half 1: M rows of the other row tiles + mean row,  value entries r_v/2 .. r_v-1
// Per tile of 16 tokens both halves compute their partial scores, swap them through LDS,
// and then run the same online softmax on the full scores (so both hold identical maxima
// and sums) while accumulating their own half of the value latent.
//
// Two kernels:
// - decode_fold_head_kernel (per head): each wave loads its key entries into registers
//   two tiles ahead; value rows and cos/sin tiles come through a direct-to-LDS ring.
// - decode_fold_wide_kernel (LLA-2D, Section 3, "The LLA-2D variant", at the ranks the
//   LLA-2D kernel is not built for): every head reads the same latent plane of its
//   sequence, so key and value rows both come through the ring, read once for all heads
//   of the workgroup; mu_t of head h is the (t, h) slice of the stacked mean. Workgroups
//   that share a (sequence, split) are placed on the same XCD (blocks are dealt to the 8
//   XCDs round robin), so the shared rows are read from HBM once into that XCD's L2.
#include <type_traits>

#include "lla_device.h"
#include "lla_kernels.h"

namespace lla {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
// Running maxima start at a finite stand-in for -inf: the first valid score always raises
// it, and columns or splits without a valid token keep a zero sum.
constexpr float kMaxInit = -1.0e30f;
constexpr float kRescaleSlack = 8.0f;
constexpr int kXcds = 8;

#ifndef LLA_WIDE_MAX_STAGES
#define LLA_WIDE_MAX_STAGES 4  // deepest direct-to-LDS ring (tiles in flight + 1)
#endif

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_f16(const f16x8_t& a, const f16x8_t& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Workgroup barrier for the ring loop. __syncthreads() also fences memory, and the
// compiler implements that fence by waiting for every outstanding direct-to-LDS load
// (vmcnt(0)), which would drain the ring at each barrier. The ring's loads are waited for
// explicitly (vmcnt(n) before the barrier that publishes a stage); this barrier only
// needs this wave's own LDS reads and writes to be complete, and the "memory" clobber
// keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D, int RK, int RV, int HPW, int NH, bool PAGED = false>
__global__ __launch_bounds__(64 * NH * HPW) __attribute__((amdgpu_waves_per_eu(NH == 2 ? 2 : 1)))
void decode_fold_wide_kernel(DecodeArgs a, PageArgs pg) {
  constexpr int NKS = D / 32;
  constexpr int NCK = RK / 16;            // latent row tiles of M^T
  // NH == 2: half 0 owns latent row tiles [0, NR0), half 1 owns [NR0, NCK) and the mean row.
  // NH == 1: the single wave owns every row tile and the mean row.
  constexpr int NR0 = NH == 2 ? (NCK + 2) / 2 : NCK;
  constexpr int NT0 = NH == 2 ? NR0 : NCK + 1;  // MFMA row tiles of half 0
  constexpr int NT1 = NCK - NR0 + 1;            // MFMA row tiles of half 1 (last is the mean)
  constexpr int NTMAX = NT0 > NT1 ? NT0 : NT1;
  constexpr int RVH = RV / NH;            // value entries per half
  constexpr int VSH = RVH / 4;            // value entries per lane
  constexpr int WT_STRIDE = D + 8;
  constexpr int STAGE_UNITS = NH * HPW * 16 * WT_STRIDE * 2 / 16;
  constexpr int NIK = RK / 32, NIV = RV / 32;         // 1 KiB blocks of a plane's 16 rows
  constexpr int NPL = 1;                              // latent planes per stage (shared)
  constexpr int STAGE_BLOCKS = NPL * (NIK + NIV) + NKS;  // 1 KiB blocks
  constexpr int XCH_UNITS = NH == 2 ? (NH * HPW * 16 + 3) / 4 : 0;  // the pairs' partial scores
  constexpr int PAGE_UNITS = PAGED ? kMaxSplitPages * 4 / 16 : 0;  // the split's page indices
  // Ring depth: as many stages as keep the workgroup within 80 KiB (two per CU), at least 3.
  constexpr int NB_FIT = (80 * 1024 / 16 - XCH_UNITS - PAGE_UNITS) / (STAGE_BLOCKS * 64);
  constexpr int NB = NB_FIT < 3 ? 3 : (NB_FIT > LLA_WIDE_MAX_STAGES ? LLA_WIDE_MAX_STAGES : NB_FIT);
  constexpr int LDS_UNITS_RING = NB * STAGE_BLOCKS * 64 + XCH_UNITS;
  constexpr int LDS_UNITS = LDS_UNITS_RING + PAGE_UNITS > STAGE_UNITS ? LDS_UNITS_RING + PAGE_UNITS
                                                                      : STAGE_UNITS;
  static_assert(RK % 32 == 0 && RV % 32 == 0 && VSH % 4 == 0 && D % 32 == 0, "shape");

  __shared__ u32x4 lds[LDS_UNITS];

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, hi = lane >> 4;
  const int half = NH == 2 ? (wave & 1) : 0;
  const int hw = NH == 2 ? (wave >> 1) : wave;  // head within the workgroup

  // Block placement: a flat grid where the H / HPW head groups of one (sequence, loop,
  // split) sit on the same XCD.
  const int groups = a.H / HPW;
  const int L = static_cast<int>(blockIdx.x);
  const int xcd = L % kXcds;
  const int slot_ = L / kXcds;
  const int unit_ = xcd + kXcds * (slot_ / groups);  // (b, li, split) index
  const int hg = slot_ % groups;
  const int split = unit_ % a.S;
  const int li = (unit_ / a.S) % a.L;
  const int b = unit_ / (a.S * a.L);
  if (b >= a.B) return;  // padding blocks of the last XCD round (whole workgroup exits)
  const int h = hg * HPW + hw;
  const int t = a.loop_begin + li;

  int len = a.n_ctx;
  if (a.ctx_lens != nullptr) len = max(0, min(a.ctx_lens[b], a.n_ctx));
  const int s0 = split * a.split_len;
  const int s1 = min(len, s0 + a.split_len);
  const int ntok = max(0, s1 - s0);

  // dense: the sequence's latent plane; paged: the pool (pages are added per tile)
  const size_t plane = PAGED ? 0 : static_cast<size_t>(b) * a.n_max;
  const char* ck = reinterpret_cast<const char*>(a.c_k) + plane * RK * 2;
  const char* cv = reinterpret_cast<const char*>(a.c_v) + plane * RV * 2;
  const char* tab_g = reinterpret_cast<const char*>(a.rope16);
  const int tile_max = (s1 > 0 ? (s1 - 1) >> 4 : 0);
  constexpr int NCKH0 = NR0, NCKH1 = NH == 2 ? NCK - NR0 : 0;
  const int ntile = (ntok + 15) >> 4;
  const int nfull = ntok >> 4;  // tiles whose 16 tokens all lie in the context

  // ---- the ring: per stage one tile of 16 tokens --------------------------------------
  // For every latent plane of the stage a key region (16 rows of KSL 16-byte slots) and a
  // value region (VSL slots per row), then the NKS 1 KiB blocks of the cos/sin tile. Every
  // region is filled by 1 KiB direct-to-LDS loads (global_load_lds_dwordx4: lane l writes
  // bytes 16 l .. 16 l + 15 of the block). Row r keeps its slots XOR-permuted within each
  // aligned group of four by (r >> 2) & 3: the rows are 64-byte multiples long, so without
  // it rows r and r + 4 would start in the same bank, and with it the 16 rows of a read
  // cover all 64 banks once.
  constexpr int KSL = RK / 8;
  constexpr int VSL = RV / 8;
  constexpr int PLB = NIK + NIV;                    // 1 KiB blocks per plane
  static_assert(16 * KSL == 64 * NIK && 16 * VSL == 64 * NIV, "ring shape");
  constexpr int NW = NH * HPW;
  constexpr int NIW = (STAGE_BLOCKS + NW - 1) / NW;  // blocks each wave loads per stage
  static_assert(NB >= 2 && (NB - 2) * NIW <= 63, "vmcnt range");
  // the W_up staging fits the ring's last stage, so the first tiles can be requested first
  constexpr bool kEarly = NB >= 3 && STAGE_UNITS <= STAGE_BLOCKS * 64;
  static_assert(LDS_UNITS_RING + PAGE_UNITS <= 80 * 1024 / 16 || NB == 3, "ring size");
  u32x4* ring = lds;
  float* xch = reinterpret_cast<float*>(lds + NB * STAGE_BLOCKS * 64);  // [wave][16] (LLA-2D)

  // Per block slot of this wave: the block index in the stage, this lane's source address
  // for the next tile to be issued, and the byte step from one tile to the next. Tiles
  // wholly inside the context advance the address by the step; the last, partial tile (and
  // the ring's run-out past the end) recomputes it with the token clamped to the last one
  // in the context (the clamped rows get zero weight) and the table tile to the last used.
  int blk[NIW], srow[NIW];
  const char* nxt[NIW];
  const char* sbase[NIW];  // slot's source at tile 0 minus its row offset (rows clamp)
  int rbytes[NIW];         // bytes per source row (0 marks a table block)
  size_t step[NIW];        // bytes from one tile's source to the next
#pragma unroll
  for (int k = 0; k < NIW; ++k) {
    int bi = wave + NW * k;
    if (bi >= STAGE_BLOCKS) bi = wave;  // even out the per-wave count with a repeat
    blk[k] = bi;
    if (bi >= NPL * PLB) {
      const int ks = bi - NPL * PLB;
      rbytes[k] = 0;
      srow[k] = 0;
      step[k] = static_cast<size_t>(NKS) * 1024;
      sbase[k] = tab_g + static_cast<size_t>(ks) * 1024 + lane * 16;
      nxt[k] = sbase[k] + static_cast<size_t>(s0 >> 4) * NKS * 1024;
    } else {
      const int pl = bi / PLB, r = bi - pl * PLB;
      const bool isk = r < NIK;
      const int sl = isk ? KSL : VSL;
      const int slot = (isk ? r : r - NIK) * 64 + lane;  // physical slot in the region
      const int row = slot / sl;
      const int col = ((slot % sl) ^ ((row >> 2) & 3)) * 16;  // its row's logical slot
      (void)pl;  // one plane
      rbytes[k] = isk ? RK * 2 : RV * 2;
      srow[k] = row;
      step[k] = PAGED ? static_cast<size_t>(a.Hc) * kPage * rbytes[k]  // one page
                      : static_cast<size_t>(16) * rbytes[k];
      sbase[k] = (isk ? ck : cv) + col;
      nxt[k] = sbase[k] + static_cast<size_t>(PAGED ? row : s0 + row) * rbytes[k];
    }
  }

  auto dma = [&](const char* src, u32x4* dst) {
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                     (void __attribute__((address_space(3)))*)dst, 16, 0, 0);
  };
  // Paged: the pages of the split's tiles are read into LDS once, before the ring starts
  // (a vector load inside the ring would wait for every transfer issued before it).
  int* split_pages = reinterpret_cast<int*>(lds + LDS_UNITS_RING);
  if constexpr (PAGED) {
    for (int i = static_cast<int>(threadIdx.x); i < ntile; i += 64 * NW)
      split_pages[i] = page_of(pg, b, (s0 >> 4) + i);
    __syncthreads();
  }
  auto page_for = [&](int tl) {
    return PAGED ? __builtin_amdgcn_readfirstlane(split_pages[min(tl, ntile - 1)]) : 0;
  };
  int page_next = ntile > 0 ? page_for(0) : 0;
  auto issue = [&](int tl) {
    u32x4* stage = ring + (tl % NB) * STAGE_BLOCKS * 64;
    if constexpr (PAGED) {
      const size_t page = static_cast<size_t>(page_next);
      if (tl < nfull) {  // rows unclamped: the slot's row within the page is its own
#pragma unroll
        for (int k = 0; k < NIW; ++k) {
          if (rbytes[k] == 0) {
            dma(nxt[k], stage + blk[k] * 64);
            nxt[k] += step[k];
          } else {
            dma(nxt[k] + page * step[k], stage + blk[k] * 64);
          }
        }
      } else {
        const int ptok0 = min((s0 >> 4) + tl, tile_max) * kPage;  // the page's first token
#pragma unroll
        for (int k = 0; k < NIW; ++k) {
          const char* src;
          if (rbytes[k] == 0) {
            src = sbase[k] + static_cast<size_t>(min((s0 >> 4) + tl, tile_max)) * NKS * 1024;
          } else {
            const int tok = min(s0 + 16 * tl + srow[k], s1 - 1);
            src = sbase[k] + page * step[k] + static_cast<size_t>(tok - ptok0) * rbytes[k];
          }
          dma(src, stage + blk[k] * 64);
        }
      }
      page_next = page_for(tl + 1);
      return;
    }
    if (tl < nfull) {
#pragma unroll
      for (int k = 0; k < NIW; ++k) {
        dma(nxt[k], stage + blk[k] * 64);
        nxt[k] += step[k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < NIW; ++k) {
        const char* src =
            rbytes[k] == 0 ? sbase[k] + static_cast<size_t>(min((s0 >> 4) + tl, tile_max)) * NKS * 1024
                           : sbase[k] + static_cast<size_t>(min(s0 + 16 * tl + srow[k], s1 - 1)) * rbytes[k];
        dma(src, stage + blk[k] * 64);
      }
    }
  };

  // ---- this half's M^T fragments, through a per-wave LDS transpose of W_up,k,t ----
  // Every W_up,k,t row this wave needs is requested at once (one memory round trip), and
  // with kEarly the ring's first tiles are already in flight: the staging then sits in the
  // ring's last stage, which the prologue does not fill.
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.w_up_k) + static_cast<size_t>(t * a.H + h) * D * RK;
  const uint16_t* mu = reinterpret_cast<const uint16_t*>(a.mu_k) + static_cast<size_t>(t * a.H + h) * D;
  const float* q = a.q + (static_cast<size_t>(b * a.H + h) * a.L + li) * D;
  const float sc = a.scale_log2e;
  uint16_t* wt = reinterpret_cast<uint16_t*>(lds + (kEarly ? (NB - 1) * STAGE_BLOCKS * 64 : 0)) +
                 wave * 16 * WT_STRIDE;
  u32x4 wpre[NTMAX][D / 64][2];
  uint16_t mpre[D / 64];
#pragma unroll
  for (int i = 0; i < NTMAX; ++i) {
    const int tile = half == 0 ? i : NR0 + i;
    const bool active = half == 0 ? (i < NT0) : (i < NT1);
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      if (active && tile < NCK) {
        const u32x4* src = reinterpret_cast<const u32x4*>(W + static_cast<size_t>(lane + 64 * k) * RK + 16 * tile);
        wpre[i][k][0] = src[0];
        wpre[i][k][1] = src[1];
      } else {
        wpre[i][k][0] = u32x4{0u, 0u, 0u, 0u};
        wpre[i][k][1] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
#pragma unroll
  for (int k = 0; k < D / 64; ++k) mpre[k] = mu[lane + 64 * k];
  if (kEarly && ntile > 0) {
#pragma unroll
    for (int tl = 0; tl < NB - 1; ++tl) issue(tl);
  }
  f16x8_t mf[NTMAX][NKS];
#pragma unroll
  for (int i = 0; i < NTMAX; ++i) {
    const int tile = half == 0 ? i : NR0 + i;  // latent row tile; NCK is the mean row
    const bool active = half == 0 ? (i < NT0) : (i < NT1);
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      const int c = lane + 64 * k;
      if (active && tile < NCK) {
        const u32x4 x0 = wpre[i][k][0], x1 = wpre[i][k][1];
        const uint32_t w8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          wt[(2 * j) * WT_STRIDE + c] = static_cast<uint16_t>(w8[j] & 0xffffu);
          wt[(2 * j + 1) * WT_STRIDE + c] = static_cast<uint16_t>(w8[j] >> 16);
        }
      } else {
        wt[c] = (active && tile == NCK) ? mpre[k] : static_cast<uint16_t>(0);
#pragma unroll
        for (int j = 1; j < 16; ++j) wt[j * WT_STRIDE + c] = 0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks2 = 0; ks2 < NKS / 2; ++ks2) {
      const int p0 = 32 * ks2 + 8 * hi;
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
  if (!kEarly && ntile > 0) {
#pragma unroll
    for (int tl = 0; tl < NB - 1; ++tl) issue(tl);
  }

  float m_run = kMaxInit, l_run = 0.f;
  float acc[VSH];
#pragma unroll
  for (int e = 0; e < VSH; ++e) acc[e] = 0.f;

  constexpr int mypl = 0;
  const int swz = ((lo >> 2) & 3) << 4;  // byte XOR of this lane's token row (row lo)

  // The tile loop, compiled once per half so that which row tiles, latent rows and value
  // entries a wave owns are compile-time constants (no branches inside the loop).
  auto run = [&](auto half_c) {
    constexpr int HALF = decltype(half_c)::value;
    constexpr int NT = HALF == 0 ? NT0 : NT1;          // MFMA row tiles of this half
    constexpr int NCKh = HALF == 0 ? NCKH0 : NCKH1;    // latent row tiles of this half
    constexpr int KT0 = HALF == 0 ? 0 : NR0;           // its first latent row tile
    constexpr bool MEAN = NH == 1 || HALF == 1;        // its last MFMA tile holds the mean row
    for (int c = 0; c < ntile; ++c) {
      // this wave's blocks of tile c have landed once at most the later (NB - 2) tiles'
      // are outstanding; the barrier then makes every wave's blocks visible, and also tells
      // that every wave is done with tile c - 1, whose stage the next issue overwrites
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NB - 2) * NIW) : "memory");
      ring_barrier();
      const u32x4* st = ring + (c % NB) * STAGE_BLOCKS * 64;
      const char* kreg = reinterpret_cast<const char*>(st + (mypl * PLB) * 64);
      const char* vreg = reinterpret_cast<const char*>(st + (mypl * PLB + NIK) * 64);
      const u32x4* treg = st + (NPL * PLB) * 64;
      const char* krow = kreg + lo * (KSL * 16);
      const char* vrow = vreg + lo * (VSL * 16);

      // Every LDS operand of the tile is requested at once, before the next tile's loads
      // are issued, so that their latencies overlap instead of adding up.
      f16x8_t bfr[NKS];
      u32x2 kw[NCKh > 0 ? NCKh : 1];
      u32x2 vw[VSH / 4];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) bfr[ks] = __builtin_bit_cast(f16x8_t, treg[ks * 64 + lane]);
#pragma unroll
      for (int m = 0; m < NCKh; ++m)
        kw[m] = *reinterpret_cast<const u32x2*>(krow + ((32 * (KT0 + m) + 8 * hi) ^ swz));
#pragma unroll
      for (int m = 0; m < VSH / 4; ++m)
        vw[m] = *reinterpret_cast<const u32x2*>(vrow + ((2 * (HALF * RVH + hi * VSH) + 8 * m) ^ swz));
      issue(c + NB - 1);

      // (1) this half's partial score for the 16 tokens, published to LDS
      f32x4 g[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) g[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int i = 0; i < NT; ++i) g[i] = mfma_f16(mf[i][ks], bfr[ks], g[i]);
      }
      // element 0 of the mean tile: the mean row for hi = 0, an all-zero padding row of
      // M^T (so exactly 0) for the other lane groups
      float pp = MEAN ? g[NT - 1][0] : 0.f;
#pragma unroll
      for (int m = 0; m < NCKh; ++m) {
        const u32x2 w = kw[m];
        pp += __uint_as_float(w.x << 16) * g[m][0] + __uint_as_float(w.x & 0xffff0000u) * g[m][1] +
              __uint_as_float(w.y << 16) * g[m][2] + __uint_as_float(w.y & 0xffff0000u) * g[m][3];
      }
      const float part = sum_xor32(sum_xor16(pp));
      float full = part;
      if constexpr (NH == 2) {
        if (hi == 0) xch[wave * 16 + lo] = part;
        ring_barrier();
        const float other = xch[(wave ^ 1) * 16 + lo];
        full = HALF == 0 ? part + other : other + part;  // same order in both halves
      }

      // (2) full score, online softmax, this half's value update
      const float s = (c < nfull || s0 + 16 * c + lo < s1) ? full : kNegInf;
      const bool raise = s > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = raise ? s : m_run;
        const float alpha = raise ? fast_exp2(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < VSH; ++e) acc[e] *= alpha;
        m_run = m_new;
      }
      const float p = fast_exp2(s - m_run);
      l_run += p;
#pragma unroll
      for (int m = 0; m < VSH / 4; ++m) {
        const u32x2 w = vw[m];
        acc[4 * m + 0] += p * __uint_as_float(w.x << 16);
        acc[4 * m + 1] += p * __uint_as_float(w.x & 0xffff0000u);
        acc[4 * m + 2] += p * __uint_as_float(w.y << 16);
        acc[4 * m + 3] += p * __uint_as_float(w.y & 0xffff0000u);
      }
    }
  };
  if constexpr (NH == 2) {
    if (half == 0) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, 0>{});
  }
  // no direct-to-LDS load may land after this point (the LDS is reused below and at exit)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ---- merge the 16 token columns (identical maxima and sums in both halves) ----
  float mx = m_run;
#pragma unroll
  for (int msk = 1; msk < 16; msk <<= 1) mx = fmaxf(mx, shfl_xor(mx, msk));
  const float scl = fast_exp2(m_run - mx);
  float lsum = l_run * scl;
#pragma unroll
  for (int msk = 1; msk < 16; msk <<= 1) lsum += shfl_xor(lsum, msk);
#pragma unroll
  for (int e = 0; e < VSH; ++e) {
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
      for (int e = 0; e < VSH; ++e) out[2 + half * RVH + hi * VSH + e] = acc[e];
      if (hi == 0 && half == 0) {
        out[0] = mx;
        out[1] = lsum;
      }
    }
    return;
  }

  // ---- single split: out = (acc / sum) W_up,v,t^T + mu_v,t; the pair shares the work ----
  float* abar = reinterpret_cast<float*>(lds) + hw * RV;
  static_assert(sizeof(lds) >= sizeof(float) * RV * HPW, "LDS reuse for the normalised latent");
  static_assert(NH == 1 || NH == 2, "one or two waves per head");
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  if (lo == 0) {
#pragma unroll
    for (int e = 0; e < VSH; ++e) abar[half * RVH + hi * VSH + e] = acc[e] * inv;
  }
  __syncthreads();
  const uint16_t* Wv = reinterpret_cast<const uint16_t*>(a.w_up_v) + static_cast<size_t>(t * a.H + h) * D * RV;
  const uint16_t* muv = reinterpret_cast<const uint16_t*>(a.mu_v) + static_cast<size_t>(t * a.H + h) * D;
  float* out = a.out + unit * D;
  for (int i = half * (D / NH) + lane; i < (half + 1) * (D / NH); i += 64) {
    float o = 0.f;
    if (lsum > 0.f) {
#pragma unroll 4
      for (int r0 = 0; r0 < RV; r0 += 8) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(Wv + static_cast<size_t>(i) * RV + r0);
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

template <int D, int RK, int RV, int HPW, int NH, bool PAGED = false>
void launch(const DecodeArgs& a, const PageArgs& pg, hipStream_t s) {
  // (b, loop, split) units dealt to XCDs so that one unit's head groups share an XCD
  const long long units = static_cast<long long>(a.B) * a.L * a.S;
  const long long rounds = (units + kXcds - 1) / kXcds;
  const long long blocks = rounds * kXcds * (a.H / HPW);
  hipLaunchKernelGGL((decode_fold_wide_kernel<D, RK, RV, HPW, NH, PAGED>),
                     dim3(static_cast<unsigned>(blocks)), dim3(64 * NH * HPW), 0, s, a, pg);
}

// ---- per-head instance: keys into registers, values through the ring -----------------
// Direct-to-LDS loads (which need no registers for the prefetch depth) stream measurably
// slower from HBM than plain loads on gfx950 when they carry all of a kernel's bytes, and
// a wave that mixes the two reaches the plain loads' rate. So each wave of a head's pair
// loads the key entries it works on straight into registers, LLA_HEAD_AHEAD tiles ahead
// in rotating buffers, while the value rows and the cos/sin tiles come through a
// direct-to-LDS ring as deep.
//
// Key side: the latent row tiles a half owns are taken in pairs. For a pair covering
// latent entries E .. E + 31, the MFMA rows of its first tile are entries E + 8 g + e and
// those of its second E + 8 g + 4 + e (g, e = 0..3), so that the lane holding score rows
// 4 hi .. 4 hi + 3 of both tiles needs the 8 consecutive entries E + 8 hi .. E + 8 hi + 7
// of its token: one 16-byte load. An odd last tile keeps the natural order (entries
// 16 kt + 4 hi + e, one 8-byte load).
#ifndef LLA_HEAD_AHEAD
#define LLA_HEAD_AHEAD 2  // tiles requested ahead of the one being computed
#endif

template <int D, int RK, int RV, int HPW, bool PAGED>
__global__ __launch_bounds__(128 * HPW) __attribute__((amdgpu_waves_per_eu(2)))
void decode_fold_head_kernel(DecodeArgs a, PageArgs pg) {
  constexpr int NKS = D / 32;
  constexpr int NCK = RK / 16;              // latent row tiles of M^T
  constexpr int NR0 = (NCK + 2) / 2;        // half 0: row tiles [0, NR0); half 1 the rest + mean
  constexpr int NT0 = NR0;
  constexpr int NT1 = NCK - NR0 + 1;
  constexpr int NTMAX = NT0 > NT1 ? NT0 : NT1;
  constexpr int RVH = RV / 2;               // value entries per half
  constexpr int VSH = RVH / 4;              // value entries per lane
  constexpr int WT_STRIDE = D + 8;
  constexpr int NW = 2 * HPW;
  constexpr int DA = LLA_HEAD_AHEAD;
  constexpr int NB = DA + 1;                // ring stages
  // ring stage: per head the 16 value rows (VSL 16-byte slots each, XOR-permuted within
  // aligned groups of four by (row >> 2) & 3 so that a read's 16 rows cover the 64 banks
  // once), then the NKS 1 KiB blocks of the cos/sin tile
  constexpr int VSL = RV / 8;
  constexpr int NIV = RV / 32;              // 1 KiB blocks of a head's 16 value rows
  constexpr int STAGE_BLOCKS = HPW * NIV + NKS;
  constexpr int NIW = (STAGE_BLOCKS + NW - 1) / NW;  // blocks each wave loads per tile
  constexpr int RING_UNITS = NB * STAGE_BLOCKS * 64;
  constexpr int XCH_UNITS = (NW * 16 + 3) / 4;
  constexpr int STAGING_UNITS = NW * 16 * WT_STRIDE * 2 / 16;
  constexpr int PAGE_UNITS = PAGED ? kMaxSplitPages * 4 / 16 : 0;
  constexpr int LDS_UNITS = RING_UNITS + XCH_UNITS + STAGING_UNITS + PAGE_UNITS;
  static_assert(RK % 32 == 0 && RV % 32 == 0 && VSH % 4 == 0 && D % 64 == 0, "shape");
  static_assert(DA >= 1 && 16 * VSL == 64 * NIV, "ring shape");
  static_assert(LDS_UNITS * 16 <= 160 * 1024, "LDS");
  static_assert(static_cast<size_t>(LDS_UNITS) * 16 >= sizeof(float) * RV * HPW, "LDS reuse");

  __shared__ u32x4 lds[LDS_UNITS];
  u32x4* ring = lds;
  float* xch = reinterpret_cast<float*>(lds + RING_UNITS);
  uint16_t* wt_all = reinterpret_cast<uint16_t*>(lds + RING_UNITS + XCH_UNITS);
  int* split_pages = reinterpret_cast<int*>(lds + RING_UNITS + XCH_UNITS + STAGING_UNITS);

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, hi = lane >> 4;
  const int half = wave & 1;
  const int hw = wave >> 1;  // head within the workgroup

  const int groups = a.H / HPW;
  const int split = blockIdx.x;
  const int li = blockIdx.y / groups;
  const int hg = blockIdx.y - li * groups;
  const int b = blockIdx.z;
  const int h = hg * HPW + hw;
  const int t = a.loop_begin + li;

  int len = a.n_ctx;
  if (a.ctx_lens != nullptr) len = max(0, min(a.ctx_lens[b], a.n_ctx));
  const int s0 = split * a.split_len;
  const int s1 = min(len, s0 + a.split_len);
  const int ntok = max(0, s1 - s0);
  const int ntile = (ntok + 15) >> 4;
  const int nfull = ntok >> 4;  // tiles whose 16 tokens all lie in the context
  const int tile_max = s1 > 0 ? (s1 - 1) >> 4 : 0;

  if constexpr (PAGED) {
    for (int i = static_cast<int>(threadIdx.x); i < ntile; i += 64 * NW)
      split_pages[i] = page_of(pg, b, (s0 >> 4) + i);
    __syncthreads();
  }
  auto page_for = [&](int tl) {
    return PAGED ? __builtin_amdgcn_readfirstlane(split_pages[min(tl, ntile - 1)]) : 0;
  };

  // ---- latent planes: dense, head h's plane; paged, the pool (pages added per tile) ----
  constexpr int KRB = RK * 2, VRB = RV * 2;  // bytes per latent row
  const char* ck;
  const char* cv;
  if constexpr (PAGED) {  // head h's rows of a page start h * kPage rows into it
    ck = reinterpret_cast<const char*>(a.c_k) + static_cast<size_t>(h) * kPage * KRB;
    cv = reinterpret_cast<const char*>(a.c_v);
  } else {
    const size_t plane = static_cast<size_t>(b * a.H + h) * a.n_max;
    ck = reinterpret_cast<const char*>(a.c_k) + plane * KRB;
    cv = reinterpret_cast<const char*>(a.c_v) + (plane - static_cast<size_t>(hw) * a.n_max) * VRB;
  }
  const size_t kpage = static_cast<size_t>(a.Hc) * kPage * KRB;  // bytes per page (paged)
  const size_t vpage = static_cast<size_t>(a.Hc) * kPage * VRB;

  // ---- ring slots of this wave: value blocks of the workgroup's heads, cos/sin blocks ----
  // The ring is filled with buffer loads to LDS (MUBUF): unlike the FLAT-encoded
  // global_load_lds, a pending one does not make the compiler wait for every load in
  // flight before it reads a register loaded by a plain load (the keys). Per slot: the
  // block index in the stage, a buffer resource over the slot's source (a head's value
  // plane, or the cos/sin table; paged: rebuilt per tile over the tile's page), and this
  // lane's byte offset in it for tile 0 (a wave-uniform offset adds the tile). The last,
  // partial tile and the run-out past the end clamp the token to the last one in the
  // context (the clamped rows get zero weight) and the table tile to the last used.
  const char* tab_g = reinterpret_cast<const char*>(a.rope16);
  constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
  int blk[NIW], srow[NIW], scol[NIW], spl[NIW];
  bool istab[NIW];
  __amdgpu_buffer_rsrc_t rs[NIW];
  uint32_t voff[NIW];
#pragma unroll
  for (int k = 0; k < NIW; ++k) {
    const int bi = (wave + NW * k) % STAGE_BLOCKS;  // repeats even out the per-wave count
    blk[k] = bi;
    if (bi >= HPW * NIV) {
      const int ks = bi - HPW * NIV;
      istab[k] = true;
      srow[k] = scol[k] = spl[k] = 0;
      rs[k] = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(tab_g), 0, (tile_max + 1) * NKS * 1024, kRsrcWord3);
      voff[k] = static_cast<uint32_t>(ks * 1024 + lane * 16);
    } else {
      const int pl = bi / NIV, r = bi - pl * NIV;
      const int slot = r * 64 + lane;  // physical slot in the head's value region
      const int row = slot / VSL;
      const int col = ((slot % VSL) ^ ((row >> 2) & 3)) * 16;  // its row's logical slot
      istab[k] = false;
      srow[k] = row;
      scol[k] = col;
      spl[k] = pl;
      // dense: head (hg * HPW + pl)'s plane (cv points at head hg * HPW's)
      rs[k] = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(cv + (PAGED ? 0 : static_cast<size_t>(pl) * a.n_max * VRB)), 0,
          PAGED ? 0 : a.n_max * VRB, kRsrcWord3);
      voff[k] = static_cast<uint32_t>(row * VRB + col);
    }
  }
  auto dma = [&](__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so, u32x4* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, vo, so, 0, 0);
  };
  auto issue = [&](int tl) {
    u32x4* stage = ring + (tl % NB) * STAGE_BLOCKS * 64;
    const int ttab = min((s0 >> 4) + tl, tile_max);  // the table tile (clamped)
    const uint32_t tsoff = static_cast<uint32_t>(ttab * NKS * 1024);
    if constexpr (PAGED) {
      const size_t page = static_cast<size_t>(page_for(tl));
      const int ptok0 = ttab * kPage;  // the page's first token
#pragma unroll
      for (int k = 0; k < NIW; ++k) {
        if (istab[k]) {
          dma(rs[k], voff[k], tsoff, stage + blk[k] * 64);
        } else {
          // head (hg * HPW + pl)'s 16 rows of the page
          const char* pb = cv + page * vpage + static_cast<size_t>(hg * HPW + spl[k]) * kPage * VRB;
          const int tok = min(s0 + 16 * tl + srow[k], s1 - 1);
          dma(__builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(pb), 0, kPage * VRB, kRsrcWord3),
              static_cast<uint32_t>((tok - ptok0) * VRB + scol[k]), 0u, stage + blk[k] * 64);
        }
      }
      return;
    }
    if (tl < nfull) {
      const uint32_t vsoff = static_cast<uint32_t>((s0 + 16 * tl) * VRB);
#pragma unroll
      for (int k = 0; k < NIW; ++k) dma(rs[k], voff[k], istab[k] ? tsoff : vsoff, stage + blk[k] * 64);
    } else {
#pragma unroll
      for (int k = 0; k < NIW; ++k) {
        if (istab[k]) {
          dma(rs[k], voff[k], tsoff, stage + blk[k] * 64);
        } else {
          const int tok = min(s0 + 16 * tl + srow[k], s1 - 1);
          dma(rs[k], static_cast<uint32_t>(tok * VRB + scol[k]), 0u, stage + blk[k] * 64);
        }
      }
    }
  };

  // ---- M^T fragments through a per-wave LDS transpose of W_up,k,t ----
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.w_up_k) + static_cast<size_t>(t * a.H + h) * D * RK;
  const uint16_t* mu = reinterpret_cast<const uint16_t*>(a.mu_k) + static_cast<size_t>(h * a.T + t) * D;
  const float* q = a.q + (static_cast<size_t>(b * a.H + h) * a.L + li) * D;
  const float sc = a.scale_log2e;
  uint16_t* wt = wt_all + wave * 16 * WT_STRIDE;
  const int kt0 = half == 0 ? 0 : NR0;                  // the half's first latent row tile
  const int nckh = half == 0 ? NR0 : NCK - NR0;          // its latent row tiles
  const int npair = nckh / 2;
  // first latent entry of row group g (4 rows) of the half's row tile i
  auto ent0 = [&](int i, int g) {
    return i < 2 * npair ? 16 * (kt0 + 2 * (i / 2)) + 8 * g + 4 * (i % 2) : 16 * (kt0 + i) + 4 * g;
  };
  u32x2 wpre[NTMAX][D / 64][4];
  uint16_t mpre[D / 64];
#pragma unroll
  for (int i = 0; i < NTMAX; ++i) {
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (i < nckh)
          wpre[i][k][g] = *reinterpret_cast<const u32x2*>(W + static_cast<size_t>(lane + 64 * k) * RK + ent0(i, g));
        else
          wpre[i][k][g] = u32x2{0u, 0u};
      }
    }
  }
#pragma unroll
  for (int k = 0; k < D / 64; ++k) mpre[k] = mu[lane + 64 * k];
  f16x8_t mf[NTMAX][NKS];
#pragma unroll
  for (int i = 0; i < NTMAX; ++i) {
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      const int c = lane + 64 * k;
      if (i < nckh) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 x = wpre[i][k][g];
          wt[(4 * g + 0) * WT_STRIDE + c] = static_cast<uint16_t>(x.x & 0xffffu);
          wt[(4 * g + 1) * WT_STRIDE + c] = static_cast<uint16_t>(x.x >> 16);
          wt[(4 * g + 2) * WT_STRIDE + c] = static_cast<uint16_t>(x.y & 0xffffu);
          wt[(4 * g + 3) * WT_STRIDE + c] = static_cast<uint16_t>(x.y >> 16);
        }
      } else {
        // the mean row (row 0 of half 1's last tile), zero rows otherwise
        wt[c] = (half == 1 && i == nckh) ? mpre[k] : static_cast<uint16_t>(0);
#pragma unroll
        for (int j = 1; j < 16; ++j) wt[j * WT_STRIDE + c] = 0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks2 = 0; ks2 < NKS / 2; ++ks2) {
      const int p0 = 32 * ks2 + 8 * hi;
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

  float m_run = kMaxInit, l_run = 0.f;
  float acc[VSH];
#pragma unroll
  for (int e = 0; e < VSH; ++e) acc[e] = 0.f;
  const int swz = ((lo >> 2) & 3) << 4;  // byte XOR of this lane's token row (row lo)

  auto run = [&](auto half_c) {
    constexpr int HALF = decltype(half_c)::value;
    constexpr int NT = HALF == 0 ? NT0 : NT1;         // MFMA row tiles of this half
    constexpr int NCKh = HALF == 0 ? NR0 : NCK - NR0;  // latent row tiles of this half
    constexpr int KT0 = HALF == 0 ? 0 : NR0;
    constexpr int NP = NCKh / 2, NS = NCKh % 2;        // key loads: pairs (16 B), single (8 B)
    constexpr bool MEAN = HALF == 1;
    constexpr int NKL = NP + NS;                       // key loads per tile
    static_assert((DA - 1) * (NIW + NKL) <= 63, "vmcnt range");
    struct Keys {
      u32x4 kp[NP > 0 ? NP : 1];
      u32x2 ks[NS > 0 ? NS : 1];
    };
    const int koff = 32 * KT0 + 16 * hi;               // pair p at + 64 p
    const int ksoff = 32 * (KT0 + 2 * NP) + 8 * hi;    // the single tile
    // A tile's key rows: a wave-uniform base (its first row, or its page) plus a per-lane
    // 32-bit offset, so the loads take the scalar-base form.
    auto load_keys = [&](Keys& K, int tl) {
      const char* kb;
      int rl;  // this lane's row from the base (rows past the context repeat the last token)
      if constexpr (PAGED) {
        const int tile = min((s0 >> 4) + tl, tile_max);
        kb = ck + static_cast<size_t>(page_for(tl)) * kpage;
        rl = min(s0 + 16 * tl + lo, s1 - 1) - 16 * tile;
      } else {
        const int r0 = min(s0 + 16 * tl, s1 - 1);
        kb = ck + static_cast<size_t>(r0) * KRB;
        rl = min(lo, s1 - 1 - r0);
      }
      const uint32_t ko = static_cast<uint32_t>(rl * KRB + koff);
      // Issued as inline assembly: the compiler then neither counts these loads nor waits
      // for them (it would otherwise wait for nearly every load in flight, since it does
      // not count the ring's loads to LDS). tile_step's explicit vmcnt wait, which counts
      // them in issue order with the ring's loads, orders their use; hold_keys ties the
      // registers to that wait.
#pragma unroll
      for (int p = 0; p < NP; ++p)
        asm volatile("global_load_dwordx4 %0, %1, %2 offset:%3 nt" : "=v"(K.kp[p]) : "v"(ko), "s"(kb), "n"(64 * p) : "memory");
      if constexpr (NS > 0)
        asm volatile("global_load_dwordx2 %0, %1, %2 nt"
                     : "=v"(K.ks[0]) : "v"(static_cast<uint32_t>(rl * KRB + ksoff)), "s"(kb) : "memory");
    };
    auto hold_keys = [&](Keys& K) {
#pragma unroll
      for (int p = 0; p < NP; ++p) asm volatile("; keys %0" : "+v"(K.kp[p]));
      if constexpr (NS > 0) asm volatile("; keys %0" : "+v"(K.ks[0]));
    };

    Keys kl[DA];
#pragma unroll
    for (int tl = 0; tl < DA; ++tl) {
      issue(tl);
      load_keys(kl[tl], tl);
    }

    auto tile_step = [&](int c, Keys& K) {
      // tile c's ring blocks and keys (this wave's) have landed once at most the later
      // DA - 1 tiles' loads are outstanding; the barrier then makes every wave's blocks
      // visible, and tells that every wave is done with tile c - 1's stage
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DA - 1) * (NIW + NKL)) : "memory");
      hold_keys(K);
      ring_barrier();
      const u32x4* st = ring + (c % NB) * STAGE_BLOCKS * 64;
      const char* vrow = reinterpret_cast<const char*>(st + hw * NIV * 64) + lo * (VSL * 16);
      const u32x4* treg = st + HPW * NIV * 64;
      // every LDS operand of the tile is requested at once, before the next loads
      f16x8_t bfr[NKS];
      u32x2 vw[VSH / 4];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) bfr[ks] = __builtin_bit_cast(f16x8_t, treg[ks * 64 + lane]);
#pragma unroll
      for (int m = 0; m < VSH / 4; ++m)
        vw[m] = *reinterpret_cast<const u32x2*>(vrow + ((2 * (HALF * RVH + hi * VSH) + 8 * m) ^ swz));
      issue(c + DA);

      // (1) this half's partial score for the 16 tokens
      f32x4 g[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) g[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int i = 0; i < NT; ++i) g[i] = mfma_f16(mf[i][ks], bfr[ks], g[i]);
      }
      // element 0 of the mean tile: the mean row for hi = 0, an all-zero row of M^T (so
      // exactly 0) for the other lane groups
      float pp = MEAN ? g[NT - 1][0] : 0.f;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const u32x4 w = K.kp[p];
        pp += __uint_as_float(w.x << 16) * g[2 * p][0] + __uint_as_float(w.x & 0xffff0000u) * g[2 * p][1] +
              __uint_as_float(w.y << 16) * g[2 * p][2] + __uint_as_float(w.y & 0xffff0000u) * g[2 * p][3];
        pp += __uint_as_float(w.z << 16) * g[2 * p + 1][0] + __uint_as_float(w.z & 0xffff0000u) * g[2 * p + 1][1] +
              __uint_as_float(w.w << 16) * g[2 * p + 1][2] + __uint_as_float(w.w & 0xffff0000u) * g[2 * p + 1][3];
      }
      if constexpr (NS > 0) {
        const u32x2 w = K.ks[0];
        pp += __uint_as_float(w.x << 16) * g[2 * NP][0] + __uint_as_float(w.x & 0xffff0000u) * g[2 * NP][1] +
              __uint_as_float(w.y << 16) * g[2 * NP][2] + __uint_as_float(w.y & 0xffff0000u) * g[2 * NP][3];
      }
      // the buffer's next tile, requested once its keys are used
      load_keys(K, c + DA);
      const float part = sum_xor32(sum_xor16(pp));
      if (hi == 0) xch[wave * 16 + lo] = part;
      ring_barrier();
      const float other = xch[(wave ^ 1) * 16 + lo];
      const float full = HALF == 0 ? part + other : other + part;  // same order in both halves

      // (2) full score, online softmax, this half's value update
      const float s = (c < nfull || s0 + 16 * c + lo < s1) ? full : kNegInf;
      const bool raise = s > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = raise ? s : m_run;
        const float alpha = raise ? fast_exp2(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < VSH; ++e) acc[e] *= alpha;
        m_run = m_new;
      }
      const float p = fast_exp2(s - m_run);
      l_run += p;
#pragma unroll
      for (int m = 0; m < VSH / 4; ++m) {
        const u32x2 w = vw[m];
        acc[4 * m + 0] += p * __uint_as_float(w.x << 16);
        acc[4 * m + 1] += p * __uint_as_float(w.x & 0xffff0000u);
        acc[4 * m + 2] += p * __uint_as_float(w.y << 16);
        acc[4 * m + 3] += p * __uint_as_float(w.y & 0xffff0000u);
      }
    };

    // whole rounds of DA tiles (each key buffer in a fixed place in the round), then the
    // remaining tiles
    int c0 = 0;
    for (; c0 + DA <= ntile; c0 += DA) {
#pragma unroll
      for (int u = 0; u < DA; ++u) tile_step(c0 + u, kl[u]);
    }
#pragma unroll
    for (int u = 0; u < DA - 1; ++u) {
      if (c0 + u < ntile) tile_step(c0 + u, kl[u]);
    }
    // the last requests (past the end) land before their registers can be reused
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int u = 0; u < DA; ++u) hold_keys(kl[u]);
  };
  if (ntile > 0) {
    if (half == 0) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
  }
  // no load may land after this point (the LDS is reused below and at exit)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ---- merge the 16 token columns (identical maxima and sums in both halves) ----
  float mx = m_run;
#pragma unroll
  for (int msk = 1; msk < 16; msk <<= 1) mx = fmaxf(mx, shfl_xor(mx, msk));
  const float scl = fast_exp2(m_run - mx);
  float lsum = l_run * scl;
#pragma unroll
  for (int msk = 1; msk < 16; msk <<= 1) lsum += shfl_xor(lsum, msk);
#pragma unroll
  for (int e = 0; e < VSH; ++e) {
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
      for (int e = 0; e < VSH; ++e) out[2 + half * RVH + hi * VSH + e] = acc[e];
      if (hi == 0 && half == 0) {
        out[0] = mx;
        out[1] = lsum;
      }
    }
    return;
  }

  // ---- single split: out = (acc / sum) W_up,v,t^T + mu_v,t; the pair shares the work ----
  float* abar = reinterpret_cast<float*>(lds) + hw * RV;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  if (lo == 0) {
#pragma unroll
    for (int e = 0; e < VSH; ++e) abar[half * RVH + hi * VSH + e] = acc[e] * inv;
  }
  __syncthreads();
  const uint16_t* Wv = reinterpret_cast<const uint16_t*>(a.w_up_v) + static_cast<size_t>(t * a.H + h) * D * RV;
  const uint16_t* muv = reinterpret_cast<const uint16_t*>(a.mu_v) + static_cast<size_t>(h * a.T + t) * D;
  float* out = a.out + unit * D;
  for (int i = half * (D / 2) + lane; i < (half + 1) * (D / 2); i += 64) {
    float o = 0.f;
    if (lsum > 0.f) {
#pragma unroll 4
      for (int r0 = 0; r0 < RV; r0 += 8) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(Wv + static_cast<size_t>(i) * RV + r0);
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

template <int D, int RK, int RV, int HPW, bool PAGED>
void launch_head(const DecodeArgs& a, const PageArgs& pg, hipStream_t s) {
  dim3 grid(a.S, (a.H / HPW) * a.L, a.B);
  hipLaunchKernelGGL((decode_fold_head_kernel<D, RK, RV, HPW, PAGED>), grid, dim3(128 * HPW), 0, s, a, pg);
}

}  // namespace

// Per shape: (d, r_k, r_v, heads per LLA-2D workgroup). The per-head kernel takes 4 heads
// per workgroup (one workgroup per CU) when H allows, else 2; its ring is
// LLA_HEAD_AHEAD + 1 stages. The LLA-2D ring takes as many stages (3 ..
// LLA_WIDE_MAX_STAGES) as keep a workgroup within 80 KiB of LDS.
#ifndef LLA_WIDE_HPW_2D
#define LLA_WIDE_HPW_2D 2
#endif
#define LLA_WIDE_SHAPES(X)             \
  X(128, 96, 160, LLA_WIDE_HPW_2D)     \
  X(128, 128, 128, LLA_WIDE_HPW_2D)    \
  X(128, 64, 64, LLA_WIDE_HPW_2D)      \
  X(64, 256, 256, 2)

bool decode_fold_wide_supported(int dtype, int d, int r_k, int r_v) {
  if (dtype != 1) return false;
#define X(D_, RK_, RV_, H2_) \
  if (d == D_ && r_k == RK_ && r_v == RV_) return true;
  LLA_WIDE_SHAPES(X)
#undef X
  return false;
}

int fold_wide_waves_per_head() { return 2; }

int fold_wide_heads_per_group(int d, int r_k, int r_v, bool shared) {
#define X(D_, RK_, RV_, H2_) \
  if (d == D_ && r_k == RK_ && r_v == RV_) return shared ? H2_ : 2;
  LLA_WIDE_SHAPES(X)
#undef X
  return 1 << 30;
}

bool launch_decode_fold_wide(int dtype, int d, int r_k, int r_v, bool shared, const DecodeArgs& a,
                             hipStream_t s) {
  if (dtype != 1 || a.H % fold_wide_heads_per_group(d, r_k, r_v, shared) != 0) return false;
#define X(D_, RK_, RV_, H2_)                                                     \
  if (d == D_ && r_k == RK_ && r_v == RV_) {                                     \
    if (shared) launch<D_, RK_, RV_, H2_, 2>(a, PageArgs{}, s);                  \
    else if (a.H % 4 == 0) launch_head<D_, RK_, RV_, 4, false>(a, PageArgs{}, s); \
    else launch_head<D_, RK_, RV_, 2, false>(a, PageArgs{}, s);                  \
    return true;                                                                 \
  }
  LLA_WIDE_SHAPES(X)
#undef X
  return false;
}

bool launch_decode_fold_wide_paged(int dtype, int d, int r_k, int r_v, bool shared,
                                   const DecodeArgs& a, const PageArgs& pg, hipStream_t s) {
  if (dtype != 1 || pg.table == nullptr ||
      a.H % fold_wide_heads_per_group(d, r_k, r_v, shared) != 0)
    return false;
#define X(D_, RK_, RV_, H2_)                                             \
  if (d == D_ && r_k == RK_ && r_v == RV_) {                             \
    if (shared) launch<D_, RK_, RV_, H2_, 2, true>(a, pg, s);            \
    else if (a.H % 4 == 0) launch_head<D_, RK_, RV_, 4, true>(a, pg, s); \
    else launch_head<D_, RK_, RV_, 2, true>(a, pg, s);                   \
    return true;                                                         \
  }
  LLA_WIDE_SHAPES(X)
#undef X
  return false;
}

}  // namespace lla
