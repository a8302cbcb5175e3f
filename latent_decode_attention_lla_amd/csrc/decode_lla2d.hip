// Latent-store decode for LLA-2D ("Looped Latent Attention", Section 3, "The LLA-2D
// variant"): one latent row per (sequence, token) serves every head, so the value side of
// attention is a true matrix product, P (heads x tokens) times the value latents (tokens x
// r_v), and runs on the matrix cores here (gfx950, wave64, bfloat16 cache and codec).
//
// Scores use the rotary-fold rewrite of the per-head kernels (Eq. 3 and "RoPE and
// reconstruction": RoPE of the reconstructed key at the slot index): for head h the score
// of token j is c_j . G_j + G_j[r_k], G_j = CS_j M_h, where M_h is built from q, W_up,k,(t,h)
// and the (t, h) slice of mu_k, and CS_j holds cos and sin of the slot's angles. G^T is an
// f16 MFMA product with all of M_h^T in one wave's registers, so a head's scores need no
// exchange between waves; the wave keeps one running max for its head.
//
// Value side (Appendix J, "Absorbed attention": the attention weights sum to one, so the
// weighted value latent can be up-projected once): per 16-token tile the softmax weights of
// the workgroup's heads are written to LDS as bfloat16, and acc[h][r] += sum_j p[h][j] c_v[j][r]
// is one v_mfma_f32_16x16x16_bf16 per 16 value entries, spread over the workgroup's waves.
// The running sum adds the same rounded weights, so the result is an exact weighted mean
// with weights rounded to bfloat16.
//
// Workgroup: HG heads (one wave each) of one (sequence, loop, split). Cache rows and cos/sin
// tiles stream through a direct-to-LDS ring of kStages stages, kAhead tiles ahead (5 with 8
// heads, one workgroup per CU; 3 with 4 heads, so that two workgroups share a CU). Each wave
// runs its tiles as a three-deep software pipeline, one workgroup barrier per tile:
//   iteration c:  score MFMAs and latent dot of tile c (operands read in iteration c - 1)
//                 softmax of tile c - 1 (its score carried in a register), P tile c - 1 out
//                 value product of tile c - 2 (every head's weights published by the barrier)
//                 operands of tile c + 1 read from LDS into registers
// so the matrix-core chain of one tile, the vector tail of the previous one and the LDS
// latency of the next one overlap inside a wave instead of following one another. Keys sit
// in LDS as [row-tile pair][entry group][token] 16-byte units and the rows of M^T are
// ordered to match, so a wave's key reads are linear 1 KiB runs. Workgroups of one (sequence, loop, split) sit on the same XCD,
// so the shared latent rows come from HBM once. With a paged cache a 16-token tile is one
// page of the pool, named by the block table (the split's page indices are read into LDS
// first); positions and the angles follow the logical token index, so the arithmetic is
// the dense one.
#include "lla_device.h"
#include "lla_kernels.h"

#ifndef LLA_2D_ENABLE
#define LLA_2D_ENABLE 1  // 0 leaves dense LLA-2D to the wide fold kernel
#endif

namespace lla {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMaxInit = -1.0e30f;   // finite stand-in for -inf: the first valid score raises it
constexpr float kRescaleSlack = 8.0f;  // raise the running max only when exceeded by 2^8
constexpr int kXcds = 8;
#ifndef LLA_2D_AHEAD
#define LLA_2D_AHEAD 5      // ring lookahead with 8 heads per workgroup (one per CU)
#endif
#ifndef LLA_2D_AHEAD_SMALL
#define LLA_2D_AHEAD_SMALL 3  // with fewer heads per workgroup (two workgroups per CU)
#endif
// tile c + ahead is requested in iteration c; tiles c - 2 .. c + ahead live in iteration c,
// and an even stage count keeps the P buffer parity a function of the stage index
template <int HG>
struct Ring {
  static constexpr int kAhead = HG >= 8 ? LLA_2D_AHEAD : LLA_2D_AHEAD_SMALL;
  static constexpr int kStages = (kAhead + 4) / 2 * 2;
};

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_f16(const f16x8_t& a, const f16x8_t& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Barrier inside the ring loop. The ring's direct-to-LDS loads are waited for explicitly
// with vmcnt before it, and every LDS write another wave reads after it (the P tile, the
// rescale factors) is waited for right after it is made, so LDS reads of the next tile's
// operands may still be in flight here; a __syncthreads() fence would also wait for every
// load in flight.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// LDS written by this wave's lanes is read back by other lanes of the same wave: the
// wave's LDS operations complete in order, so waiting for its own writes is enough.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
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

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D, int RK, int RV, int HG>
struct Shape {
  static constexpr int NW = HG;                   // waves: one per head
  static constexpr int NKS = D / 32;              // K steps of the score MFMA
  static constexpr int NCK = RK / 16;             // latent row tiles of M^T
  static constexpr int NT = NCK + 1;              // MFMA row tiles: the latent rows and the mean row
  static constexpr int NRT = RV / 16;             // value tiles of 16 entries
  static constexpr int VT = (NRT + NW - 1) / NW;  // value tiles per wave (wave w: w, w + NW, ..)
  // stage layout, in 16-byte units: keys by (row-tile pair, entry group, token), values
  // row-major, then the cos/sin tile (NKS fragments of 1 KiB). A value row is padded to VSP
  // units with VSP % 8 in {2, 6}, so the four token rows one lane group reads start 8 or
  // 24 banks apart.
  static constexpr int KEY_UNITS = NCK * 32;      // [row-tile pair][4 entry groups][token]
  static constexpr int VSL = RV / 8;
  static constexpr int VSP = (VSL + 1) % 8 == 2 || (VSL + 1) % 8 == 6 ? VSL + 1
                             : (VSL + 2) % 8 == 2 || (VSL + 2) % 8 == 6 ? VSL + 2
                             : (VSL + 3) % 8 == 2 || (VSL + 3) % 8 == 6 ? VSL + 3 : VSL + 4;
  static constexpr int VAL_UNITS = 16 * VSP;
  static constexpr int KEY_BLOCKS = (KEY_UNITS + 63) / 64;
  static constexpr int VAL_BLOCKS = (VAL_UNITS + 63) / 64;
  static constexpr int BLOCKS = KEY_BLOCKS + VAL_BLOCKS + NKS;  // 1 KiB DMA blocks per tile
  static constexpr int STAGE_UNITS = BLOCKS * 64;
  static constexpr int VAL_OFF = KEY_BLOCKS * 64;               // units
  static constexpr int TAB_OFF = (KEY_BLOCKS + VAL_BLOCKS) * 64;
  // DMA blocks per wave and tile, the same for every wave: slot j of wave w loads block
  // min(w + NW j, BLOCKS - 1), so surplus slots re-load the last block into the same bytes
  static constexpr int NSLOT = (BLOCKS + NW - 1) / NW;
  static constexpr int WT_STRIDE = D + 8;                       // float16 row stride of the W staging
  static constexpr int STAGING_UNITS = NW * 16 * WT_STRIDE * 2 / 16;
  static_assert(RK % 32 == 0, "row tiles come in pairs");
  static_assert(RK % 16 == 0 && RV % 16 == 0 && D % 64 == 0 && HG <= 16, "shape");
};

template <int D, int RK, int RV, int HG, bool PAGED>
__global__ __launch_bounds__(64 * HG) __attribute__((amdgpu_waves_per_eu(2)))
void decode_lla2d_kernel(DecodeArgs a, PageArgs pg) {
  using S = Shape<D, RK, RV, HG>;
  constexpr int NW = S::NW, NKS = S::NKS, NCK = S::NCK, NT = S::NT, NRT = S::NRT, VT = S::VT;
  constexpr int kAhead = Ring<HG>::kAhead;
  constexpr int kStages = Ring<HG>::kStages;
  constexpr int RING_UNITS = kStages * S::STAGE_UNITS;
  // The W_up transpose staging of the prologue sits in ring stages kAhead.. when it fits
  // there (the prologue fills stages 0 .. kAhead - 1 only, and the first barrier of the
  // tile loop comes before any load into stage kAhead); else after the ring.
  constexpr bool kStagingInRing = (kStages - kAhead) * S::STAGE_UNITS >= S::STAGING_UNITS;
  constexpr int STAGING_EXTRA = kStagingInRing ? 0 : S::STAGING_UNITS;
  constexpr int P_UNITS = (2 * 16 * 16 + 64) * 2 / 16;  // two P tiles of bf16, 64 spare slots
  constexpr int AL_UNITS = (2 * 16 + 64) * 4 / 16;       // two rows of rescale factors, spares
  constexpr int PAGE_UNITS = PAGED ? kMaxSplitPages * 4 / 16 : 0;
  constexpr int LDS_UNITS = RING_UNITS + STAGING_EXTRA + P_UNITS + AL_UNITS + PAGE_UNITS;
  static_assert(HG * RV + 2 * HG <= RING_UNITS * 4, "epilogue staging fits the ring");

  __shared__ u32x4 lds[LDS_UNITS];
  uint16_t* staging = reinterpret_cast<uint16_t*>(lds + (kStagingInRing ? kAhead * S::STAGE_UNITS : RING_UNITS));
  // P tiles [2][token / 4][16 heads][token % 4]: a lane's 4 weights of one head are 8 bytes
  uint16_t* ptile = reinterpret_cast<uint16_t*>(lds + RING_UNITS + STAGING_EXTRA);
  float* alpha_buf = reinterpret_cast<float*>(lds + RING_UNITS + STAGING_EXTRA + P_UNITS);  // [2][16]
  int* split_pages = reinterpret_cast<int*>(lds + RING_UNITS + STAGING_EXTRA + P_UNITS + AL_UNITS);

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
  const int tile_max = s1 > 0 ? (s1 - 1) >> 4 : 0;

  // ---- this head's codec rows and query, requested before the ring's first tiles -------
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.w_up_k) + static_cast<size_t>(t * a.H + h) * D * RK;
  const uint16_t* mu = reinterpret_cast<const uint16_t*>(a.mu_k) + static_cast<size_t>(t * a.H + h) * D;
  const float* q = a.q + (static_cast<size_t>(b * a.H + h) * a.L + li) * D;
  // Row r of M^T's row tile m holds latent entry 32 (m / 2) + 8 (r / 4) + 4 (m % 2) + r % 4,
  // so the 4 rows of tile m in lane group hi and those of tile m ^ 1 are 8 consecutive
  // entries of one token: one 16-byte key unit per lane and tile pair.
  u32x2 wreg[NCK][D / 64][4];  // W[lane + 64 k][entries of tile m's rows 4 g .. 4 g + 3]
#pragma unroll
  for (int i = 0; i < NCK; ++i)
#pragma unroll
    for (int k = 0; k < D / 64; ++k)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        wreg[i][k][g4] = *reinterpret_cast<const u32x2*>(
            W + static_cast<size_t>(lane + 64 * k) * RK + 32 * (i / 2) + 8 * g4 + 4 * (i % 2));
  // this lane's 8 rotary pairs of each half: p0 = 32 ks2 + 8 hi
  float4 qreg[NKS / 2][4];
#pragma unroll
  for (int ks2 = 0; ks2 < NKS / 2; ++ks2)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      qreg[ks2][e] = *reinterpret_cast<const float4*>(q + 2 * (32 * ks2 + 8 * hi) + 4 * e);
  u32x4 mreg[NKS / 2][2];  // mu[2 p0 .. 2 p0 + 15] (used by the lanes holding the mean row)
#pragma unroll
  for (int ks2 = 0; ks2 < NKS / 2; ++ks2) {
    const u32x4* src = reinterpret_cast<const u32x4*>(mu + 2 * (32 * ks2 + 8 * hi));
    mreg[ks2][0] = src[0];
    mreg[ks2][1] = src[1];
  }

  // ---- ring: per DMA slot of this wave, the lane's byte offset in the tile and its row ----
  // block k of a stage is issued by wave k % NW; keys: block P, lane (hi, lo) -> entries
  // 32 P + 8 hi .. + 7 of token lo; values: unit u -> row u / VSP, slot u % VSP (the padding
  // slot re-reads the row's last slot); table: fragment k - KEY_BLOCKS - VAL_BLOCKS.
  const size_t plane = PAGED ? 0 : static_cast<size_t>(b) * a.n_max;
  const char* ck = reinterpret_cast<const char*>(a.c_k) + plane * RK * 2;
  const char* cv = reinterpret_cast<const char*>(a.c_v) + plane * RV * 2;
  const char* tab_g = reinterpret_cast<const char*>(a.rope16);
  int srow[S::NSLOT];
  uint32_t soff[S::NSLOT];
  int skind[S::NSLOT];  // 0 keys, 1 values, 2 table (wave-uniform)
#pragma unroll
  for (int j = 0; j < S::NSLOT; ++j) {
    const int blk = min(wave + NW * j, S::BLOCKS - 1);
    skind[j] = blk < S::KEY_BLOCKS ? 0 : (blk < S::KEY_BLOCKS + S::VAL_BLOCKS ? 1 : 2);
    const int u = blk * 64 + lane;
    if (blk < S::KEY_BLOCKS) {  // block = row-tile pair P, lane = (entry group hi, token lo)
      srow[j] = lo;
      soff[j] = static_cast<uint32_t>(lo * RK * 2 + (32 * blk + 8 * hi) * 2);
    } else if (blk < S::KEY_BLOCKS + S::VAL_BLOCKS) {
      const int uv = u - S::VAL_OFF;
      const int row = min(uv / S::VSP, 15);
      srow[j] = row;
      soff[j] = static_cast<uint32_t>(row * RV * 2 + min(uv % S::VSP, S::VSL - 1) * 16);
    } else {
      srow[j] = 0;
      soff[j] = static_cast<uint32_t>((blk - S::KEY_BLOCKS - S::VAL_BLOCKS) * 1024 + lane * 16);
    }
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
  // Tile tl of the split into stage stg; tiles past the last load the last tile again.
  // Tiles wholly inside the context take sources from a wave-uniform base plus the lane's
  // fixed offset; the others clamp rows past the context end to its last row.
  auto issue = [&](int tl, int stg) {
    u32x4* stage = lds + stg * S::STAGE_UNITS;
    if (tl < nfull) {
      size_t row0;
      if constexpr (PAGED) row0 = static_cast<size_t>(16) * __builtin_amdgcn_readfirstlane(split_pages[tl]);
      else row0 = static_cast<size_t>(s0 + 16 * tl);
      const char* base[3] = {ck + row0 * (RK * 2), cv + row0 * (RV * 2),
                             tab_g + static_cast<size_t>((s0 >> 4) + tl) * (NKS * 1024)};
#pragma unroll
      for (int j = 0; j < S::NSLOT; ++j)
        dma(base[skind[j]] + soff[j], stage + min(wave + NW * j, S::BLOCKS - 1) * 64);
      return;
    }
    const int tlc = min(tl, ntile - 1);
    const char* tb = tab_g + static_cast<size_t>(min((s0 >> 4) + tl, tile_max)) * (NKS * 1024);
    size_t row0;
    if constexpr (PAGED) row0 = static_cast<size_t>(16) * __builtin_amdgcn_readfirstlane(split_pages[tlc]);
    else row0 = static_cast<size_t>(s0 + 16 * tlc);
    const char* kb = ck + row0 * (RK * 2);
    const char* vb = cv + row0 * (RV * 2);
    const int rmax = s1 - 1 - (s0 + 16 * tlc);  // rows past the context end re-read its last row
#pragma unroll
    for (int j = 0; j < S::NSLOT; ++j) {
      u32x4* dst = stage + min(wave + NW * j, S::BLOCKS - 1) * 64;
      const int d = min(srow[j], rmax) - srow[j];
      if (skind[j] == 0)
        dma(kb + static_cast<uint32_t>(static_cast<int>(soff[j]) + d * (RK * 2)), dst);
      else if (skind[j] == 1)
        dma(vb + static_cast<uint32_t>(static_cast<int>(soff[j]) + d * (RV * 2)), dst);
      else
        dma(tb + soff[j], dst);
    }
  };

  // ---- M^T fragments of this head (scaled by scale * log2 e), via a wave-local transpose --
  const float sc = a.scale_log2e;
  uint16_t* wt = staging + wave * 16 * S::WT_STRIDE;
  f16x8_t mf[NT][NKS];
  auto fold_row = [&](const u32x4 (&wp)[2], int ks2, int tile) {
    // wp holds (W[2p], W[2p + 1]) for this lane's 8 pairs p0 .. p0 + 7 of half ks2
    const uint32_t w8[8] = {wp[0].x, wp[0].y, wp[0].z, wp[0].w, wp[1].x, wp[1].y, wp[1].z, wp[1].w};
    const float qf[16] = {qreg[ks2][0].x, qreg[ks2][0].y, qreg[ks2][0].z, qreg[ks2][0].w,
                          qreg[ks2][1].x, qreg[ks2][1].y, qreg[ks2][1].z, qreg[ks2][1].w,
                          qreg[ks2][2].x, qreg[ks2][2].y, qreg[ks2][2].z, qreg[ks2][2].w,
                          qreg[ks2][3].x, qreg[ks2][3].y, qreg[ks2][3].z, qreg[ks2][3].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x0 = __uint_as_float(w8[e] << 16);
      const float x1 = __uint_as_float(w8[e] & 0xffff0000u);
      mf[tile][ks2][e] = static_cast<_Float16>((qf[2 * e] * x0 + qf[2 * e + 1] * x1) * sc);
      mf[tile][ks2 + NKS / 2][e] = static_cast<_Float16>((qf[2 * e + 1] * x0 - qf[2 * e] * x1) * sc);
    }
  };

  auto prologue_and_loop = [&]() {
    constexpr int NL = S::NSLOT;  // DMA loads per wave and tile
    static_assert(NL * (kAhead - 2) <= 63, "vmcnt range");
#pragma unroll
    for (int k = 0; k < kAhead; ++k) issue(k, k);

#pragma unroll
    for (int i = 0; i < NCK; ++i) {
#pragma unroll
      for (int k = 0; k < D / 64; ++k) {
        const int c = lane + 64 * k;
        const uint32_t w8[8] = {wreg[i][k][0].x, wreg[i][k][0].y, wreg[i][k][1].x, wreg[i][k][1].y,
                                wreg[i][k][2].x, wreg[i][k][2].y, wreg[i][k][3].x, wreg[i][k][3].y};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          wt[(2 * j) * S::WT_STRIDE + c] = static_cast<uint16_t>(w8[j] & 0xffffu);
          wt[(2 * j + 1) * S::WT_STRIDE + c] = static_cast<uint16_t>(w8[j] >> 16);
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int ks2 = 0; ks2 < NKS / 2; ++ks2) {
        const u32x4* wrow = reinterpret_cast<const u32x4*>(wt + lo * S::WT_STRIDE + 2 * (32 * ks2 + 8 * hi));
        const u32x4 wp[2] = {wrow[0], wrow[1]};
        fold_row(wp, ks2, i);
      }
      wave_lds_sync();  // the reads are done before the next row tile overwrites the staging
    }
    // the mean row: row 0 of its tile is mu, the other 15 rows are zero
#pragma unroll
    for (int ks2 = 0; ks2 < NKS / 2; ++ks2) {
      fold_row(mreg[ks2], ks2, NCK);
      if (lo != 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          mf[NCK][ks2][e] = static_cast<_Float16>(0.f);
          mf[NCK][ks2 + NKS / 2][e] = static_cast<_Float16>(0.f);
        }
      }
    }

    // ---- the pipelined tile loop ----
    float m_run = kMaxInit;  // this head's running max (exp2 domain), the same in every lane
    float l_run = 0.f;       // this lane's token column's share of the running sum
    f32x4 vacc[VT];          // acc[heads 4 hi .. 4 hi + 3][value entry 16 rt + lo]
#pragma unroll
    for (int k = 0; k < VT; ++k) vacc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    f16x8_t bq[NKS];   // cos/sin fragments of the next tile to score
    u32x4 kq[NCK / 2]; // its key latents: entries 32 P + 8 hi .. + 7 of token lo
    float s_prev = kNegInf;  // the previous tile's score of token lo (exp2 domain)

    auto read_operands = [&](int stg) {
      const u32x4* st = lds + stg * S::STAGE_UNITS;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) bq[ks] = __builtin_bit_cast(f16x8_t, st[S::TAB_OFF + ks * 64 + lane]);
#pragma unroll
      for (int pr = 0; pr < NCK / 2; ++pr) kq[pr] = st[pr * 64 + lane];
    };
    // score of tile c from the operands in registers; the value returned is the full score
    // of token lo in every lane (or -inf past the context end)
    auto score = [&](int c) {
      f32x4 g[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) g[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int i = 0; i < NT; ++i) g[i] = mfma_f16(mf[i][ks], bq[ks], g[i]);
      // element 0 of the last tile: the mean row for hi = 0, a zero row elsewhere
      float pp = g[NT - 1][0];
#pragma unroll
      for (int m = 0; m < NCK; ++m) {
        const u32x2 w = (m % 2 == 0) ? u32x2{kq[m / 2].x, kq[m / 2].y} : u32x2{kq[m / 2].z, kq[m / 2].w};
        pp += __uint_as_float(w.x << 16) * g[m][0] + __uint_as_float(w.x & 0xffff0000u) * g[m][1] +
              __uint_as_float(w.y << 16) * g[m][2] + __uint_as_float(w.y & 0xffff0000u) * g[m][3];
      }
      const float full = sum_xor32(sum_xor16(pp));
      return lo < s1 - s0 - 16 * c ? full : kNegInf;
    };
    // softmax weights of tile c from its scores, into P tile c and its rescale factor
    auto tail = [&](int par, float s) {
      // The head's max is raised (to the tile's max) only when a score exceeds it by 2^8;
      // every lane of the wave holds the same head, so the choice is uniform. It is made
      // without a branch (the tile max is formed every time), and every lane writes (the
      // lanes that hold no P entry or rescale factor write to a spare slot), so the tail
      // shares one basic block with the next tile's matrix-core work.
      const bool raise = __builtin_amdgcn_ballot_w64(s > m_run + kRescaleSlack) != 0;
      const float m_new = raise ? max16(s) : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      const uint16_t pb = __builtin_bit_cast(uint16_t, static_cast<__bf16>(fast_exp2(s - m_run)));
      l_run += bf16_to_f32(pb);
      ptile[hi == 0 ? par * 256 + (lo >> 2) * 64 + hw * 4 + (lo & 3) : 512 + lane] = pb;
      alpha_buf[lane == 0 ? par * 16 + hw : 32 + lane] = alpha;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // visible to the next barrier's readers
    };
    // value product of tile c: rescale by the tile's alphas, then acc += P(c) C_v(c)
    auto value_step = [&](int stg, int par) {
      const char* vreg = reinterpret_cast<const char*>(lds + stg * S::STAGE_UNITS + S::VAL_OFF);
      const f32x4 al = *reinterpret_cast<const f32x4*>(alpha_buf + par * 16 + 4 * hi);
      const i16x4 pa = *reinterpret_cast<const i16x4*>(ptile + par * 256 + hi * 64 + lo * 4);
      // B fragment (tokens 4 hi .. 4 hi + 3 of entry 16 rt + lo) by a transposing read: lane
      // (hi, 4 k + j) names entries 16 rt + 4 j .. + 3 of token 4 hi + k, and lane (hi, lo)
      // receives short lo % 4 of the chunks lanes (hi, 4 k + lo / 4) name, k = 0 .. 3
      i16x4 vb[VT];
#pragma unroll
      for (int k = 0; k < VT; ++k) {
        const char* chunk = vreg + (4 * hi + (lo >> 2)) * (S::VSP * 16) +
                            (16 * min(wave + NW * k, NRT - 1) + 4 * (lo & 3)) * 2;
        vb[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(chunk));
      }
#pragma unroll
      for (int k = 0; k < VT; ++k) {
        if (wave + NW * k < NRT) {
          f32x4 acc = vacc[k];
          acc[0] *= al[0];
          acc[1] *= al[1];
          acc[2] *= al[2];
          acc[3] *= al[3];
          vacc[k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb[k], acc, 0, 0, 0);
        }
      }
    };

    // One pipeline step for tile c whose stage is K (a compile-time constant in the
    // unrolled steady loop, where K = c % kStages and the P buffers alternate with c).
    auto step = [&](int c, int K) {
      wait_vmcnt<NL * (kAhead - 2)>();
      ring_barrier();
      issue(c + kAhead, (K + kAhead) % kStages);
      const float s_cur = score(c);
      tail((K + 1) & 1, s_prev);                      // tile c - 1
      value_step((K + kStages - 2) % kStages, K & 1);  // tile c - 2
      read_operands((K + 1) % kStages);                // tile c + 1
      s_prev = s_cur;
    };
    static_assert(kStages % 2 == 0, "P buffer parity follows the stage index");

    // tiles 0 and 1 have landed once only tiles 2 .. kAhead - 1 are outstanding
    wait_vmcnt<NL * (kAhead - 2)>();
    ring_barrier();
    read_operands(0);
    // c = 0
    issue(kAhead, kAhead % kStages);
    float s_cur = score(0);
    if (ntile > 1) read_operands(1);
    s_prev = s_cur;
    if (ntile > 1) {
      // c = 1: no value product yet
      wait_vmcnt<NL * (kAhead - 2)>();
      ring_barrier();
      issue(1 + kAhead, (1 + kAhead) % kStages);
      s_cur = score(1);
      tail(0, s_prev);
      read_operands(2);
      s_prev = s_cur;
      // steady state, unrolled by the ring depth so that every stage index is a constant
      int c = 2;
      for (; c + kStages <= ntile; c += kStages) {
#pragma unroll
        for (int k = 0; k < kStages; ++k) step(c + k, (2 + k) % kStages);
      }
      for (; c < ntile; ++c) step(c, c % kStages);
    }
    // drain: the softmax of the last tile, then the last value products
    ring_barrier();
    tail((ntile - 1) & 1, s_prev);
    if (ntile > 1) value_step((ntile - 2) % kStages, (ntile - 2) & 1);
    ring_barrier();
    value_step((ntile - 1) % kStages, (ntile - 1) & 1);

    // ---- epilogue: the head's sum, the accumulated latent through LDS ----
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may land in the reused LDS
    __syncthreads();
    float* abar = reinterpret_cast<float*>(lds);  // [HG][RV]
#pragma unroll
    for (int k = 0; k < VT; ++k) {
      const int rt = wave + NW * k;
      if (rt < NRT) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * hi + i < HG) abar[(4 * hi + i) * RV + 16 * rt + lo] = vacc[k][i];
      }
    }
    float lsum = l_run;
#pragma unroll
    for (int msk = 1; msk < 16; msk <<= 1) lsum += shfl_xor(lsum, msk);
    float* stats = abar + HG * RV;  // [HG][2]: max, sum
    if (lane == 0) {
      stats[2 * hw] = m_run;
      stats[2 * hw + 1] = lsum;
    }
  };

  // heads past HG: unit alphas and zero weights, so their accumulator rows stay zero
  if (threadIdx.x < 32) alpha_buf[threadIdx.x] = 1.f;
  for (int i = static_cast<int>(threadIdx.x); i < 2 * (16 - HG) * 16; i += 64 * HG) {
    const int par = i / ((16 - HG) * 16), rem = i % ((16 - HG) * 16);
    const int hd = HG + rem / 16, tok = rem % 16;
    ptile[par * 256 + (tok >> 2) * 64 + hd * 4 + (tok & 3)] = 0;
  }
  // an empty split leaves a zero accumulator and sum
  if (ntile <= 0) {
    float* abar = reinterpret_cast<float*>(lds);
    for (int i = lane; i < RV; i += 64) abar[hw * RV + i] = 0.f;
    if (lane == 0) {
      abar[HG * RV + 2 * hw] = kMaxInit;
      abar[HG * RV + 2 * hw + 1] = 0.f;
    }
  } else {
    __syncthreads();  // the P padding rows and alphas are set before any wave reads them
    prologue_and_loop();
  }
  __syncthreads();

  const float* abar = reinterpret_cast<const float*>(lds);
  const float* stats = abar + HG * RV;
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
