// Projection-fused, loop-incremental encode (gfx950): the latents of Eq. 2 formed while
// a looped layer's key (value) projection runs, one loop at a time, so a prompt's per-loop
// keys and values are never stored ("Looped Latent Attention", Appendix J, "Eviction and
// long-context prefill"; Section 3, Eqs. 1-2). Eq. 2 is linear in the stacked vector:
//   c = sum_t (x_t - mu_t) W_down[block t],   x_t = h_t W_proj,
// with block t the rows of loop t (t d_in .. t d_in + d_in - 1; within it, head h's keys at
// h d for LLA-2D). Each call handles loop t of one layer: x_t = h_t W_proj on the matrix
// cores (bfloat16 inputs, float32 accumulation), then, without leaving registers, mu_t is
// subtracted and (x_t - mu_t) W_down[block t] is added to a float32 accumulator the caller
// keeps between the loops; the call of the last loop rounds the sum once to the cache
// dtype and writes the cache rows.
//
// Workgroup: 4 waves and TPW tokens per wave (64 per head, 32 for LLA-2D, whose latent is
// shared by all heads and is kept in registers while the workgroup runs through them). For
// each head it covers, the workgroup computes X^T = W_proj[head]^T h^T (128 columns x
// 4 TPW tokens, K = d_model) with W_proj^T (the weight as a linear layer stores it, rows =
// output columns) and h staged through a 3-stage direct-to-LDS ring, 32 values of K per
// stage. Both operands are rows of 64 bytes read as 16-byte fragments; the 16-byte slots of
// each row are XOR-swizzled by the row index so that 16 consecutive rows fall in distinct
// banks. The projection's output columns are loaded in a permuted order: M row
// 16 ct + 4 j + i of the product holds column 32 (ct / 2) + 8 j + 4 (ct % 2) + i, so the 8
// values a lane holds for one token in tiles 2 s and 2 s + 1 are the consecutive columns
// 32 s + 8 j .. + 7. That is the A operand of the second product with K in natural order;
// its B operand (W_down^T rows) and mu_t then come as single 16-byte loads. x - mu enters
// that product split into bfloat16 hi and lo parts (about 16 significant bits).
//
// Launch order: loops 0 .. T-1 of one layer on one stream, with the same accumulator.
// Loop 0 writes it, later loops read and update it, and loop T-1 writes the cache.
#include <type_traits>

#include "lla_device.h"
#include "lla_kernels.h"

namespace lla {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kD = 128;        // head width the fused kernel is built for
constexpr int kKc = 32;        // K values per ring stage
constexpr int kStages = 3;
constexpr int kXcds = 8;

__device__ __forceinline__ f32x4 mfma_bf16_k32(const i16x8& a, const i16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Physical 16-byte slot of logical slot `sl` (0..3) in LDS row `row`. A 16-byte LDS read
// on gfx950 is served in four passes of 16 lanes: lane bit 5 and the parity of lane bits
// 2-4 select the pass, and a pass is conflict-free when its lanes touch 16 distinct 16-byte
// bank groups (address / 16 mod 16). Fragment reads put row 16 k + (lane & 15) in a lane
// and logical slot lane >> 4; with this swizzle, (row & 3, physical slot) is distinct over
// every pass.
__device__ __forceinline__ int swz(int row, int sl) { return sl ^ (((row >> 2) & 1) << 1); }

// Head column held by M row q of the projection tile (see the header comment).
__device__ __forceinline__ int perm_col(int q) {
  const int b = q >> 5, m = q & 31;
  return 32 * b + 8 * ((m >> 2) & 3) + 4 * (m >> 4) + (m & 3);
}

template <int R, bool PER_HEAD>
__global__ __launch_bounds__(256, PER_HEAD ? 2 : 1) void encode_fused_kernel(FusedArgs a) {
  constexpr int TPW = PER_HEAD ? 64 : 32;   // tokens per wave
  constexpr int TT = TPW / 16;              // token tiles per wave
  constexpr int TOKWG = 4 * TPW;
  constexpr int NCT = kD / 16;              // column tiles of one head
  constexpr int NLT = R / 16;               // latent tiles
  constexpr int NS2 = kD / 32;              // K chunks of the second product
  constexpr int W_UNITS = kD * 4;           // [128 rows][4 slots] of 16 bytes
  constexpr int H_UNITS = TOKWG * 4;        // [TOKWG rows][4 slots]
  constexpr int STAGE = W_UNITS + H_UNITS;
  constexpr int NBLK = STAGE / 64;          // 1 KiB DMA blocks per stage
  constexpr int BPW = NBLK / 4;             // blocks per wave
  static_assert(NBLK % 4 == 0, "whole blocks per wave");
  static_assert(!PER_HEAD || 4 * NLT <= 2 * NBLK, "W_down fragments fit two stages");
  __shared__ u32x4 lds[kStages * STAGE];

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, hi = lane >> 4;

  // token blocks are dealt to XCDs round robin; the latent heads of one block share an XCD
  const int heads_y = PER_HEAD ? a.Hc : 1;
  const int L = static_cast<int>(blockIdx.x);
  const int xcd = L % kXcds, slot = L / kXcds;
  const int tb = xcd + kXcds * (slot / heads_y);
  const int hc = slot % heads_y;
  const int ntb = (a.Ntok + TOKWG - 1) / TOKWG;
  if (tb >= ntb) return;  // padding workgroups of the last round
  const int tok0 = tb * TOKWG;
  const int nk = a.d_model / kKc;
  const int h_begin = PER_HEAD ? hc : 0;
  const int nh = PER_HEAD ? 1 : a.H;
  const int nsteps = nh * nk;
  const int K = a.T * a.d_in;

  const char* hbase = static_cast<const char*>(a.h);
  const char* wbase = static_cast<const char*>(a.w_proj);
  // DMA slots: wave w loads blocks BPW w .. BPW w + BPW - 1 of a stage. A block's lane l
  // writes LDS unit 64 blk + l = (row, physical slot l % 4) and fetches the logical slot
  // that lands there. Blocks 0-7 are W_proj^T rows (M row q from head column perm_col(q));
  // the rest are h rows of the workgroup's tokens (rows past the end repeat the last).
  uint32_t dofs[BPW];
  bool dw[BPW];
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int blk = BPW * wave + j;
    const int u = 64 * blk + lane;
    if (blk < W_UNITS / 64) {
      const int q = u >> 2, sl = swz(q, u & 3);  // swz is an involution in sl
      dw[j] = true;
      dofs[j] = static_cast<uint32_t>((perm_col(q) * a.d_model + 8 * sl) * 2);
    } else {
      const int t = (u - W_UNITS) >> 2, sl = swz(t, u & 3);
      const int tok = min(tok0 + t, a.Ntok - 1);
      dw[j] = false;
      dofs[j] = static_cast<uint32_t>((static_cast<size_t>(tok - tok0) * a.d_model + 8 * sl) * 2);
    }
  }
  auto dma = [&](const char* src, u32x4* dst) {
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                     (void __attribute__((address_space(3)))*)dst, 16, 0, 0);
  };
  // step s = (head index) * nk + K chunk
  auto issue = [&](int s) {
    const int hh = h_begin + s / nk, kc = s % nk;
    u32x4* stage = lds + (s % kStages) * STAGE;
    const char* wsrc = wbase + (static_cast<size_t>(hh) * kD * a.d_model + kc * kKc) * 2;
    const char* hsrc = hbase + (static_cast<size_t>(tok0) * a.d_model + kc * kKc) * 2;
#pragma unroll
    for (int j = 0; j < BPW; ++j) dma((dw[j] ? wsrc : hsrc) + dofs[j], stage + (BPW * wave + j) * 64);
  };

  // per-lane LDS units of the fragments (stage-relative)
  int aunit[NCT], bunit[TT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) aunit[ct] = (16 * ct + lo) * 4 + swz(16 * ct + lo, hi);
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int t = TPW * wave + 16 * tt + lo;
    bunit[tt] = W_UNITS + t * 4 + swz(t, hi);
  }

  f32x4 lat[PER_HEAD ? 1 : TT][PER_HEAD ? 1 : NLT];
  if constexpr (!PER_HEAD) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int lt = 0; lt < NLT; ++lt) lat[tt][lt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  f32x4 x[NCT][TT];
  const bool first = a.loop == 0, last = a.loop == a.T - 1;
  uint16_t* cache = static_cast<uint16_t*>(a.c);

  // Second product for head h_begin + hi_: x[2 s2 + g][tt] lane (lo, hi) element i is
  // token 16 tt + lo of the wave and head column 32 s2 + 8 hi + 4 g + i.
  auto second = [&](int hi_) {
    const int hh = h_begin + hi_;

    const size_t kbase = static_cast<size_t>(a.loop) * a.d_in + (PER_HEAD ? 0 : hh * kD);
    const uint16_t* wdg = static_cast<const uint16_t*>(a.w_down_t) + static_cast<size_t>(hc) * R * K +
                          kbase + 8 * hi;
    const uint16_t* mut = static_cast<const uint16_t*>(a.mu) + static_cast<size_t>(hc) * K + kbase + 8 * hi;
    if constexpr (PER_HEAD) {  // the W_down fragments have landed for every wave
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      asm volatile("s_barrier" ::: "memory");
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      i16x8 fh[NS2], fl[NS2];
#pragma unroll
      for (int s2 = 0; s2 < NS2; ++s2) {
        const i16x8 mu8 = __builtin_bit_cast(i16x8, *reinterpret_cast<const u32x4*>(mut + 32 * s2));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = x[2 * s2 + e / 4][tt][e % 4] - bf16_to_f32(static_cast<uint16_t>(mu8[e]));
          const uint16_t vh = f32_to_bf16_rne(v);
          fh[s2][e] = static_cast<short>(vh);
          fl[s2][e] = static_cast<short>(f32_to_bf16_rne(v - bf16_to_f32(vh)));
        }
      }
#pragma unroll(PER_HEAD ? 2 : NLT)
      for (int lt = 0; lt < NLT; ++lt) {
        i16x8 bw[NS2];
#pragma unroll
        for (int s2 = 0; s2 < NS2; ++s2) {
          if constexpr (PER_HEAD) {
            const int fb = 4 * lt + s2;
            const u32x4* src = fb < NBLK ? lds + (nsteps % kStages) * STAGE + 64 * fb
                                         : lds + ((nsteps + 1) % kStages) * STAGE + 64 * (fb - NBLK);
            bw[s2] = __builtin_bit_cast(i16x8, src[lane]);
          } else {
            bw[s2] = __builtin_bit_cast(
                i16x8, *reinterpret_cast<const u32x4*>(wdg + static_cast<size_t>(16 * lt + lo) * K + 32 * s2));
          }
        }
        f32x4 acc4;
        if constexpr (PER_HEAD) acc4 = f32x4{0.f, 0.f, 0.f, 0.f};
        else acc4 = lat[tt][lt];
#pragma unroll
        for (int s2 = 0; s2 < NS2; ++s2) {
          acc4 = mfma_bf16_k32(fh[s2], bw[s2], acc4);
          acc4 = mfma_bf16_k32(fl[s2], bw[s2], acc4);
        }
        if constexpr (!PER_HEAD) {
          lat[tt][lt] = acc4;
        } else {
          // acc4 lane (lo, hi): token 16 tt + 4 hi + i of the wave, entry 16 lt + lo
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = tok0 + TPW * wave + 16 * tt + 4 * hi + i;
            if (tok >= a.Ntok) continue;
            const int e = 16 * lt + lo;
            float* arow = a.acc + (static_cast<size_t>(tok) * a.Hc + hc) * a.RT + a.ao;
            float v = acc4[i];
            if (!first) v += arow[e];
            if (last) {
              const int b = tok / a.n_new, jj = tok - b * a.n_new;
              cache[((static_cast<size_t>(b) * a.Hc + hc) * a.n_max + a.pos_start + jj) * R + e] =
                  f32_to_bf16_rne(v);
            } else {
              arow[e] = v;
            }
          }
        }
      }
    }
  };

  issue(0);
  if (nsteps > 1) issue(1);
  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps) {
      if constexpr (BPW == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    asm volatile("s_barrier" ::: "memory");
    if (s + 2 < nsteps) issue(s + 2);
    const int kc = s % nk;
    if constexpr (PER_HEAD) {
      // Last step: the head's W_down rows of this loop go, in fragment order, into the two
      // stages no step reads any more (fragment block fb = 4 lt + s2, lane (lo, hi) holds
      // W_down^T[16 lt + lo][kbase + 32 s2 + 8 hi .. + 7]).
      if (s == nsteps - 1) {
        const uint16_t* wd = static_cast<const uint16_t*>(a.w_down_t) +
                             (static_cast<size_t>(hc) * R + lo) * K + static_cast<size_t>(a.loop) * a.d_in + 8 * hi;
#pragma unroll
        for (int j = 0; j < NLT; ++j) {
          const int fb = 4 * j + wave;  // lt = j, s2 = wave
          u32x4* dst = fb < NBLK ? lds + (nsteps % kStages) * STAGE + 64 * fb
                                 : lds + ((nsteps + 1) % kStages) * STAGE + 64 * (fb - NBLK);
          dma(reinterpret_cast<const char*>(wd + static_cast<size_t>(16 * j) * K + 32 * wave), dst);
        }
      }
    }
    if (kc == 0) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) x[ct][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const u32x4* stage = lds + (s % kStages) * STAGE;
    i16x8 bfr[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) bfr[tt] = __builtin_bit_cast(i16x8, stage[bunit[tt]]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const i16x8 afr = __builtin_bit_cast(i16x8, stage[aunit[ct]]);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) x[ct][tt] = mfma_bf16_k32(afr, bfr[tt], x[ct][tt]);
    }
    if constexpr (!PER_HEAD) {
      if (kc == nk - 1) second(s / nk);
    }
  }
  if constexpr (PER_HEAD) second(0);

  if constexpr (!PER_HEAD) {
    // lat[tt][lt] lane (lo, hi): token 16 tt + 4 hi + i of the wave, entry 16 lt + lo
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tok0 + TPW * wave + 16 * tt + 4 * hi + i;
        if (tok >= a.Ntok) continue;
        float* arow = a.acc + static_cast<size_t>(tok) * a.RT + a.ao;
        const int b = tok / a.n_new, jj = tok - b * a.n_new;
        uint16_t* crow = cache + (static_cast<size_t>(b) * a.n_max + a.pos_start + jj) * R;
#pragma unroll
        for (int lt = 0; lt < NLT; ++lt) {
          const int e = 16 * lt + lo;
          float v = lat[tt][lt][i];
          if (!first) v += arow[e];
          if (last) crow[e] = f32_to_bf16_rne(v);
          else arow[e] = v;
        }
      }
    }
  }
}

// Physical 16-byte slot of logical slot `sl` (0..7) in a 128-byte LDS row `row`: with
// fragment reads putting row 16 k + (lane & 15) in a lane and slot 4 kh + (lane >> 4),
// (row & 1, physical slot) is distinct over every 16-lane pass of a 16-byte read.
__device__ __forceinline__ int swz8(int row, int sl) {
  return sl ^ ((((row >> 2) & 1) << 1) | (((row >> 1) & 1) << 2));
}

template <int SLOTS>
__device__ __forceinline__ int swz_rows(int row, int sl) {
  static_assert(SLOTS == 4 || SLOTS == 8, "64- or 128-byte rows");
  if constexpr (SLOTS == 4) return swz(row, sl);
  else return swz8(row, sl);
}

#ifndef LLA_FUSED_KC
#define LLA_FUSED_KC 64
#endif
#ifndef LLA_FUSED_NST
#define LLA_FUSED_NST 2
#endif
#ifndef LLA_FUSED_GROUP
#define LLA_FUSED_GROUP 1
#endif

// Both axes of one loop for the per-head codec in one launch. A workgroup of 8 waves takes
// 256 tokens and one head: its product tile is the head's 128 key columns and 128 value
// columns against the 256 tokens, so the hidden-state tile is loaded once for both
// projections. Wave w computes axis w / 4 (keys, values) for tokens 64 (w % 4) .. + 63.
// K advances KC2 values per stage (KC2 = 64: 128-byte rows, whole cache lines per request)
// through an NST-stage direct-to-LDS ring (NST - 1 stages in flight). During the last step
// both axes' W_down rows of this loop are staged, in fragment order, into the stages no
// step reads any more; each wave then runs the second product of its axis from there.
template <int RK, int RV, int KC2, int NST>
__global__ __launch_bounds__(512) void encode_fused_kv_kernel(FusedArgs ka, FusedArgs va) {
  constexpr int SLOTS = KC2 * 2 / 16;       // 16-byte slots per LDS row
  constexpr int NKH = KC2 / 32;             // MFMA K chunks per stage
  constexpr int TPW = 64, TT = TPW / 16, TOKWG = 4 * TPW;
  constexpr int NCT = kD / 16, NS2 = kD / 32;
  constexpr int W_UNITS = 2 * kD * SLOTS;   // key rows then value rows of the head
  constexpr int H_UNITS = TOKWG * SLOTS;
  constexpr int STAGE = W_UNITS + H_UNITS;  // 64 KiB
  constexpr int NBLK = STAGE / 64;
  constexpr int BPW = NBLK / 8;
  constexpr int NLTK = RK / 16, NLTV = RV / 16;
  constexpr int NFB = 4 * (NLTK + NLTV);    // W_down fragment blocks of both axes
  static_assert(NST >= 2 && (NST >= 3 || NFB <= NBLK) && NFB <= (NST - 1) * NBLK,
                "both W_down blocks fit the stages the last step does not read");
  static_assert(BPW * 8 == NBLK && W_UNITS % 64 == 0, "whole DMA blocks per wave");
  static_assert(NST * STAGE * 16 <= 160 * 1024, "LDS");
  // one token tile of both axes' running sums is staged in the stages the W_down rows do
  // not use: (nk - 1) % NST and, for two-stage tiles, (nk - 2) % NST
  static_assert(NFB <= NBLK || NST >= 4, "running-sum tile fits the free stages");
  __shared__ u32x4 lds[NST * STAGE];

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, hi = lane >> 4;
  const int tg = wave & 3, ax = wave >> 2;
  const FusedArgs& a = ka;  // fields shared by both axes (no run-time choice between ka and va
                            // by reference: that would put both in scratch memory)

  const int L = static_cast<int>(blockIdx.x);
  const int xcd = L % kXcds, slot = L / kXcds;
#if LLA_FUSED_GROUP
  // consecutive slots of an XCD (the workgroups it runs together) cover GT token blocks x
  // GH heads, so both the hidden-state tiles and the projection rows are shared in L2
  const int GH = a.Hc % 8 == 0 ? 8 : (a.Hc % 4 == 0 ? 4 : (a.Hc % 2 == 0 ? 2 : 1));
  const int GT = 32 / GH;
  const int grp = slot / 32, g = slot % 32;
  const int hgroups = a.Hc / GH;
  const int tb = xcd + kXcds * ((grp / hgroups) * GT + g / GH);
  const int hc = (grp % hgroups) * GH + g % GH;
#else
  const int tb = xcd + kXcds * (slot / a.Hc);
  const int hc = slot % a.Hc;
#endif
  const int ntb = (a.Ntok + TOKWG - 1) / TOKWG;
  if (tb >= ntb) return;  // padding workgroups of the last round
  const int tok0 = tb * TOKWG;
  const int nk = a.d_model / KC2;
  const int K = a.T * a.d_in;

  // DMA: wave w loads blocks BPW w .. BPW w + BPW - 1 of a stage; blocks below
  // W_UNITS / 64 / 2 are key rows, then value rows, then h rows. A lane writes unit
  // 64 blk + lane = (row, physical slot lane % 8) and fetches the logical slot landing there.
  uint32_t dofs[BPW];
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int u = 64 * (BPW * wave + j) + lane;
    if (u < W_UNITS) {
      const int row = u / SLOTS, sl = swz_rows<SLOTS>(row, u % SLOTS);
      dofs[j] = static_cast<uint32_t>((perm_col(row % kD) * a.d_model + 8 * sl) * 2);
    } else {
      const int t = (u - W_UNITS) / SLOTS, sl = swz_rows<SLOTS>(t, u % SLOTS);
      const int tok = min(tok0 + t, a.Ntok - 1);
      dofs[j] = static_cast<uint32_t>((static_cast<size_t>(tok - tok0) * a.d_model + 8 * sl) * 2);
    }
  }
  auto dma = [&](const void* src, u32x4* dst) __attribute__((always_inline)) {
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                     (void __attribute__((address_space(3)))*)dst, 16, 0, 0);
  };
  // each wave's blocks come from one source: waves 0-1 key rows, 2-3 value rows, 4-7 h
  static_assert(W_UNITS / 64 == 4 * BPW, "four waves load the projection rows");
  const size_t wrow = static_cast<size_t>(hc) * kD * a.d_model * 2;
  const uint64_t src_base =
      wave < 2 ? reinterpret_cast<uint64_t>(ka.w_proj) + wrow
               : (wave < 4 ? reinterpret_cast<uint64_t>(va.w_proj) + wrow
                           : reinterpret_cast<uint64_t>(a.h) + static_cast<size_t>(tok0) * a.d_model * 2);
  const char* srcw = reinterpret_cast<const char*>(src_base);
  auto issue = [&](int s) __attribute__((always_inline)) {
    u32x4* stage = lds + (s % NST) * STAGE + 64 * BPW * wave;
    const char* src = srcw + static_cast<size_t>(s) * KC2 * 2;
#pragma unroll
    for (int j = 0; j < BPW; ++j) dma(src + dofs[j], stage + 64 * j);
  };

  // fragment units: row 16 k + lo, logical slot 4 kh + hi; swz8 depends on row bits 1-2 only
  int fu[NKH];
#pragma unroll
  for (int kh = 0; kh < NKH; ++kh) fu[kh] = lo * SLOTS + swz_rows<SLOTS>(lo, 4 * kh + hi);
  const int arow0 = ax * kD, brow0 = TPW * tg;

  f32x4 x[NCT][TT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) x[ct][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // W_down fragment block fb lives in stage (nk + fb / NBLK) % NST, which the last step
  // does not read
  auto region = [&](int fb) __attribute__((always_inline)) {
    return lds + ((nk + fb / NBLK) % NST) * STAGE + 64 * (fb % NBLK);
  };
#pragma unroll
  for (int t = 0; t < NST - 1; ++t)
    if (t < nk) issue(t);
  for (int s = 0; s < nk; ++s) {
    // stages s + 1 .. s + NST - 2 may stay in flight
    const int ahead = min(NST - 2, nk - 1 - s);
    if constexpr (NST >= 4) {
      if (ahead >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * BPW) : "memory");
      else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(BPW) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else if constexpr (NST == 3) {
      if (ahead >= 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(BPW) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    asm volatile("s_barrier" ::: "memory");
    if (s + NST - 1 < nk) {
      issue(s + NST - 1);
    } else if (s == nk - 1) {
      // last step: this loop's W_down rows of both axes into the stage no step reads any
      // more (fragment block fb: axis, latent tile lt, K chunk s2; lane (lo, hi) holds
      // W_down^T[16 lt + lo][loop d_in + 32 s2 + 8 hi .. + 7])
      const size_t wdo = static_cast<size_t>(lo) * K + static_cast<size_t>(a.loop) * a.d_in + 8 * hi;
      const uint16_t* wdk = static_cast<const uint16_t*>(ka.w_down_t) + static_cast<size_t>(hc) * RK * K + wdo;
      const uint16_t* wdv = static_cast<const uint16_t*>(va.w_down_t) + static_cast<size_t>(hc) * RV * K + wdo;
#pragma unroll
      for (int j = 0; j < (NFB + 7) / 8; ++j) {
        const int fb = 8 * j + wave;
        if (fb < NFB) {
          if (fb < 4 * NLTK) {
            dma(wdk + (static_cast<size_t>(16 * (fb >> 2)) * K + 32 * (fb & 3)), region(fb));
          } else {
            const int f = fb - 4 * NLTK;
            dma(wdv + (static_cast<size_t>(16 * (f >> 2)) * K + 32 * (f & 3)), region(fb));
          }
        }
      }
    }
    // Fragment reads run one column-tile pair ahead of the MFMAs that use them (and the B
    // fragments of the next K chunk one pair before they are needed), issued right after
    // the current pair's first MFMA, with scheduler fences keeping that order, so LDS
    // latency hides behind the pair's other seven MFMAs.
    const u32x4* stage = lds + (s % NST) * STAGE;
    auto rd_b = [&](int kh, i16x8* b) __attribute__((always_inline)) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        b[tt] = __builtin_bit_cast(i16x8, stage[W_UNITS + (brow0 + 16 * tt) * SLOTS + fu[kh]]);
    };
    auto rd_a = [&](int kh, int ct) __attribute__((always_inline)) {
      return __builtin_bit_cast(i16x8, stage[(arow0 + 16 * ct) * SLOTS + fu[kh]]);
    };
    constexpr int NPAIR = NKH * NCT / 2;
    i16x8 bq[NKH][TT];
    i16x8 ap[2][2];
    rd_b(0, bq[0]);
    ap[0][0] = rd_a(0, 0);
    ap[0][1] = rd_a(0, 1);
#pragma unroll
    for (int q = 0; q < NPAIR; ++q) {
      const int kh = q / (NCT / 2), ct = 2 * (q % (NCT / 2));
      // the pair's first MFMA (waiting for its operands), then the next pair's reads, then
      // the other seven MFMAs of this pair while those reads are in flight
      x[ct][0] = mfma_bf16_k32(ap[q & 1][0], bq[kh][0], x[ct][0]);
      __builtin_amdgcn_sched_barrier(0);
      if (q + 1 < NPAIR) {
        const int kn = (q + 1) / (NCT / 2), cn = 2 * ((q + 1) % (NCT / 2));
        ap[(q + 1) & 1][0] = rd_a(kn, cn);
        ap[(q + 1) & 1][1] = rd_a(kn, cn + 1);
        if (kn != kh) rd_b(kn, bq[kn]);
      }
      __builtin_amdgcn_sched_barrier(0);
      x[ct + 1][0] = mfma_bf16_k32(ap[q & 1][1], bq[kh][0], x[ct + 1][0]);
#pragma unroll
      for (int tt = 1; tt < TT; ++tt) {
        x[ct][tt] = mfma_bf16_k32(ap[q & 1][0], bq[kh][tt], x[ct][tt]);
        x[ct + 1][tt] = mfma_bf16_k32(ap[q & 1][1], bq[kh][tt], x[ct + 1][tt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  asm volatile("s_barrier" ::: "memory");

  // Second product of the wave's axis: x[2 s2 + g][tt] lane (lo, hi) element i is token
  // 16 tt + lo of the wave and head column 32 s2 + 8 hi + 4 g + i.
  const bool first = a.loop == 0, last = a.loop == a.T - 1;
  // The accumulator of this workgroup is kept in fragment order: for the axis at entry
  // offset ao, block (tg, tt, lt) holds 256 floats, lane l's 4 values at 4 l .. 4 l + 3
  // (tokens 16 tt + 4 (l / 16) + i of the wave, entry 16 lt + l % 16). Loads and stores
  // are contiguous 16-byte lanes. For each token tile a wave first copies its blocks of
  // the running sum into its own slice of the stage the last step read (direct-to-LDS, so
  // the latency overlaps the hi / lo split), then reads them back per latent tile.
  const int sbase = ax == 0 ? tg * NLTK : 4 * NLTK + tg * NLTV;  // the wave's staging blocks
  auto acc_region = [&](int b) __attribute__((always_inline)) {
    return lds + (((nk - 1 - b / NBLK) % NST + NST) % NST) * STAGE + 64 * (b % NBLK);
  };
  auto second = [&](auto rtag, const void* mu, void* c, int ao, int fb0) __attribute__((always_inline)) {
    constexpr int R = decltype(rtag)::value;
    constexpr int NLT = R / 16;
    const uint16_t* mut = static_cast<const uint16_t*>(mu) + static_cast<size_t>(hc) * K +
                          static_cast<size_t>(a.loop) * a.d_in + 8 * hi;
    uint16_t* cache = static_cast<uint16_t*>(c);
    float* accw = a.acc + (static_cast<size_t>(tb) * a.Hc + hc) * a.RT * TOKWG +
                  static_cast<size_t>(ao) * TOKWG + static_cast<size_t>(tg) * TT * NLT * 256 + 4 * lane;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if (!first) {
#pragma unroll
        for (int lt = 0; lt < NLT; ++lt) dma(accw + (tt * NLT + lt) * 256, acc_region(sbase + lt));
      }
      i16x8 fh[NS2], fl[NS2];
#pragma unroll
      for (int s2 = 0; s2 < NS2; ++s2) {
        const i16x8 mu8 = __builtin_bit_cast(i16x8, *reinterpret_cast<const u32x4*>(mut + 32 * s2));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = x[2 * s2 + e / 4][tt][e % 4] - bf16_to_f32(static_cast<uint16_t>(mu8[e]));
          const uint16_t vh = f32_to_bf16_rne(v);
          fh[s2][e] = static_cast<short>(vh);
          fl[s2][e] = static_cast<short>(f32_to_bf16_rne(v - bf16_to_f32(vh)));
        }
      }
      if (!first) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's slice landed
#pragma unroll 2
      for (int lt = 0; lt < NLT; ++lt) {
        f32x4 acc4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < NS2; ++s2) {
          const i16x8 bw = __builtin_bit_cast(i16x8, region(fb0 + 4 * lt + s2)[lane]);
          acc4 = mfma_bf16_k32(fh[s2], bw, acc4);
          acc4 = mfma_bf16_k32(fl[s2], bw, acc4);
        }
        if (!first) acc4 += __builtin_bit_cast(f32x4, acc_region(sbase + lt)[lane]);
        if (!last) {
          *reinterpret_cast<f32x4*>(accw + (tt * NLT + lt) * 256) = acc4;
        } else {
          // acc4 lane (lo, hi): token 16 tt + 4 hi + i of the wave, entry 16 lt + lo
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = tok0 + brow0 + 16 * tt + 4 * hi + i;
            if (tok >= a.Ntok) continue;
            const int b = tok / a.n_new, jj = tok - b * a.n_new;
            cache[((static_cast<size_t>(b) * a.Hc + hc) * a.n_max + a.pos_start + jj) * R + 16 * lt + lo] =
                f32_to_bf16_rne(acc4[i]);
          }
        }
      }
      // the slice is refilled for the next tile only after every read of it above
      if (!first) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  };
  if (ax == 0) second(std::integral_constant<int, RK>{}, ka.mu, ka.c, ka.ao, 0);
  else second(std::integral_constant<int, RV>{}, va.mu, va.c, va.ao, 4 * NLTK);
}

template <int RK, int RV>
void launch_kv(const FusedArgs& k, const FusedArgs& v, hipStream_t s) {
  constexpr int KC2 = LLA_FUSED_KC, NST = LLA_FUSED_NST;
  const int ntb = (k.Ntok + 255) / 256;
#if LLA_FUSED_GROUP
  const int GH = k.Hc % 8 == 0 ? 8 : (k.Hc % 4 == 0 ? 4 : (k.Hc % 2 == 0 ? 2 : 1));
  const long long per_xcd = (ntb + kXcds - 1) / kXcds;          // token blocks per XCD
  const long long tgroups = (per_xcd + 32 / GH - 1) / (32 / GH);  // token groups per XCD
  const unsigned blocks = static_cast<unsigned>(tgroups * (k.Hc / GH) * 32 * kXcds);
#else
  const long long rounds = (ntb + kXcds - 1) / kXcds;
  const unsigned blocks = static_cast<unsigned>(rounds * kXcds * k.Hc);
#endif
  hipLaunchKernelGGL((encode_fused_kv_kernel<RK, RV, KC2, NST>), dim3(blocks), dim3(512), 0, s, k, v);
}

template <int R>
void launch_axis(const FusedArgs& a, bool per_head, hipStream_t s) {
  const int tokwg = per_head ? 256 : 128;
  const int ntb = (a.Ntok + tokwg - 1) / tokwg;
  const int heads_y = per_head ? a.Hc : 1;
  const long long rounds = (ntb + kXcds - 1) / kXcds;
  const unsigned blocks = static_cast<unsigned>(rounds * kXcds * heads_y);
  if (per_head)
    hipLaunchKernelGGL((encode_fused_kernel<R, true>), dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((encode_fused_kernel<R, false>), dim3(blocks), dim3(256), 0, s, a);
}

}  // namespace

// Latent sizes the fused encode is built for (d_head 128, bfloat16).
#define LLA_FUSED_RANKS(X) X(16) X(32) X(64) X(96) X(128) X(160)

bool encode_fused_supported(int dtype, int d, int r) {
  if (dtype != 1 || d != kD) return false;
#define X(R_) \
  if (r == R_) return true;
  LLA_FUSED_RANKS(X)
#undef X
  return false;
}

// (r_k, r_v) pairs with a two-axis per-head kernel (r_k + r_v <= 256).
#define LLA_FUSED_KV_PAIRS(X) X(16, 32) X(32, 64) X(64, 64) X(96, 160) X(128, 128)

bool encode_fused_kv_supported(int r_k, int r_v, int d_model) {
  if (d_model % LLA_FUSED_KC != 0) return false;
#define X(K_, V_) \
  if (r_k == K_ && r_v == V_) return true;
  LLA_FUSED_KV_PAIRS(X)
#undef X
  return false;
}

bool launch_encode_fused_kv(int r_k, int r_v, const FusedArgs& k, const FusedArgs& v, hipStream_t s) {
#define X(K_, V_)                      \
  if (r_k == K_ && r_v == V_) {        \
    launch_kv<K_, V_>(k, v, s);        \
    return true;                       \
  }
  LLA_FUSED_KV_PAIRS(X)
#undef X
  return false;
}

bool launch_encode_fused(int r, const FusedArgs& a, bool per_head, hipStream_t s) {
#define X(R_)                          \
  if (r == R_) {                       \
    launch_axis<R_>(a, per_head, s);   \
    return true;                       \
  }
  LLA_FUSED_RANKS(X)
#undef X
  return false;
}

}  // namespace lla
