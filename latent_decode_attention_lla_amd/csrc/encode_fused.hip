// Projection-fused, loop-incremental encode (gfx950): the latents of Eq. 2 formed while
// a looped layer's key (value) projection runs, one loop at a time, so a prompt's per-loop
// keys and values are never stored ("Looped Latent Attention", Appendix J, "Eviction and
// long-context prefill"; Section 3, Eqs. 1-2). Eq. 2 is linear in the stacked vector:
//   c = sum_t x_t W_down[block t] - mu W_down,   x_t = h_t W_proj,
// with block t the rows of loop t (t d_in .. t d_in + d_in - 1; within it, head h's keys at
// h d for LLA-2D). Each call handles loop t of one layer: x_t = h_t W_proj on the matrix
// cores (bfloat16 inputs, float32 accumulation), then, without leaving registers,
// x_t W_down[block t] is added to a float32 accumulator the caller keeps between the
// loops; the call of the last loop subtracts mu W_down, rounds once to the cache dtype and
// writes the cache rows.
//
// Workgroup: 4 waves and 128 tokens (32 per wave) of one latent head (per-head codec) or of
// all heads (LLA-2D, whose latent row is shared by the heads). For each head it covers,
// the workgroup computes X^T = W_proj[:, head]^T h^T (128 columns x 128 tokens, K = d_model)
// with W and h staged through a 3-stage direct-to-LDS ring, 32 values of K per stage; the
// W^T operand comes from transposing LDS reads (W rows are XOR-swizzled in 16-byte slots
// so the reads avoid bank conflicts). A wave's result lanes hold 4 consecutive columns of
// one token, which is the A operand of the second product with a permuted K order: x
// (split into bfloat16 hi and lo parts, so x enters with about 16 significant bits) times
// W_down[block t] from W_down^T's rows in the same order.
//
// Launch order: loops 0 .. T-1 of one layer on one stream, with the same accumulator.
// Loop 0 writes it, later loops read and update it, and loop T-1 writes the cache.
#include "lla_device.h"
#include "lla_kernels.h"

namespace lla {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kD = 128;        // head width the fused kernel is built for
constexpr int kTokWg = 128;    // tokens per workgroup
constexpr int kKc = 32;        // K values per ring stage
constexpr int kStages = 3;
constexpr int kXcds = 8;

__device__ __forceinline__ f32x4 mfma_bf16_k32(const i16x8& a, const i16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16-byte slot of column chunk c (8 columns) in W stage row r
__device__ __forceinline__ int w_slot(int r, int c) { return c ^ (((r & 3) << 1) ^ (((r >> 3) & 1) << 3)); }

__device__ __forceinline__ uint16_t bf16_rne(float f) { return f32_to_bf16_rne(f); }

template <int R, bool PER_HEAD>
__global__ __launch_bounds__(256) void encode_fused_kernel(FusedArgs a) {
  constexpr int NCT = kD / 16;   // column tiles of one head
  constexpr int NLT = R / 16;    // latent tiles
  constexpr int TT = 2;          // token tiles per wave
  constexpr int W_UNITS = kKc * 16;            // [32 rows][16 slots] of 16 bytes
  constexpr int H_UNITS = kTokWg * kKc * 2 / 16;  // [128 tokens][4 slots]
  constexpr int STAGE = W_UNITS + H_UNITS;     // 16-byte units: 16 blocks of 1 KiB
  static_assert(STAGE == 16 * 64, "4 DMA blocks per wave and stage");
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
  const int ntb = (a.Ntok + kTokWg - 1) / kTokWg;
  if (tb >= ntb) return;  // padding workgroups of the last round
  const int tok0 = tb * kTokWg;
  const int ldw = a.H * kD;
  const int nk = a.d_model / kKc;
  const int h_begin = PER_HEAD ? hc : 0;
  const int nh = PER_HEAD ? 1 : a.H;
  const int nsteps = nh * nk;

  const char* hbase = static_cast<const char*>(a.h);
  const char* wbase = static_cast<const char*>(a.w_proj);
  // DMA slots: wave w loads blocks 4 w .. 4 w + 3 of a stage; blocks 0-7 hold W rows
  // 4 i .. 4 i + 3 (a lane: one 16-byte slot of one row), blocks 8-15 the h rows of tokens
  // 16 (i - 8) .. + 15 (a lane: 16 bytes of one token's 32 K values)
  uint32_t dofs[4];
  int dkind[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int blk = 4 * wave + j;
    if (blk < 8) {
      const int r = 4 * blk + lane / 16, sl = lane % 16;
      dkind[j] = 0;
      dofs[j] = static_cast<uint32_t>((r * ldw + 8 * w_slot(r, sl)) * 2);  // w_slot is an involution
    } else {
      const int tok = min(tok0 + 16 * (blk - 8) + lane / 4, a.Ntok - 1);  // past the end: last row
      dkind[j] = 1;
      dofs[j] = static_cast<uint32_t>(static_cast<size_t>(tok - tok0) * a.d_model * 2 + (lane % 4) * 16);
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
    const char* wsrc = wbase + (static_cast<size_t>(kc) * kKc * ldw + hh * kD) * 2;
    const char* hsrc = hbase + (static_cast<size_t>(tok0) * a.d_model + kc * kKc) * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma((dkind[j] == 0 ? wsrc : hsrc) + dofs[j], stage + (4 * wave + j) * 64);
  };

  f32x4 lat[TT][NLT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt) lat[tt][lt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 x[NCT][TT];

  issue(0);
  if (nsteps > 1) issue(1);
  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
    if (s + 2 < nsteps) issue(s + 2);
    const int kc = s % nk;
    if (kc == 0) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) x[ct][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const u32x4* stage = lds + (s % kStages) * STAGE;
    const char* wst = reinterpret_cast<const char*>(stage);
    const u32x4* hst = stage + W_UNITS;
    // B operands: h^T of this wave's two token tiles (token 16 tt + lo, K 8 hi .. 8 hi + 7)
    i16x8 bfr[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
      bfr[tt] = __builtin_bit_cast(i16x8, hst[(32 * wave + 16 * tt + lo) * 4 + hi]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      // A operand W^T of column tile ct: lane (hi, lo) holds W[8 hi + e][16 ct + lo], e = 0..7,
      // from two transposing reads: lane (hi, 4 k + j) names W[8 hi + 4 half + k][16 ct + 4 j .. + 3]
      i16x4 part[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int r = 8 * hi + 4 * half + (lo >> 2);
        const int c = 2 * ct + ((lo & 3) >> 1);
        const char* p = wst + r * 256 + w_slot(r, c) * 16 + (lo & 1) * 8;
        part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
      }
      const i16x8 afr = {part[0][0], part[0][1], part[0][2], part[0][3],
                         part[1][0], part[1][1], part[1][2], part[1][3]};
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) x[ct][tt] = mfma_bf16_k32(afr, bfr[tt], x[ct][tt]);
    }
    if (kc == nk - 1) {
      // x[ct][tt] lane (lo, hi): x_t[token 16 tt + lo][column 16 ct + 4 hi + i] of head hh.
      // Second product with K = the head's 128 columns, 32 per step s2, in the order: lane
      // group hi's element e is column 32 s2 + 4 hi + e (e < 4) or 32 s2 + 16 + 4 hi + e - 4.
      const int hh = h_begin + s / nk;
      const size_t kbase = static_cast<size_t>(a.loop) * a.d_in + (PER_HEAD ? 0 : hh * kD);
      const uint16_t* wd = static_cast<const uint16_t*>(a.w_down_t) +
                           static_cast<size_t>(hc) * R * (a.T * a.d_in) + kbase;
      const uint16_t* mut = static_cast<const uint16_t*>(a.mu) +
                            static_cast<size_t>(hc) * (a.T * a.d_in) + kbase + 4 * hi;
#pragma unroll
      for (int s2 = 0; s2 < kD / 32; ++s2) {
        // mu_t of this lane's 8 columns (4 hi + e of tiles 2 s2 and 2 s2 + 1)
        const u32x2 m0 = *reinterpret_cast<const u32x2*>(mut + 32 * s2);
        const u32x2 m1 = *reinterpret_cast<const u32x2*>(mut + 32 * s2 + 16);
        const u32x4 mm = {m0.x, m0.y, m1.x, m1.y};
        const i16x8 mu8 = __builtin_bit_cast(i16x8, mm);
        i16x8 ahi[TT], alo[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = x[2 * s2 + e / 4][tt][e % 4] - bf16_to_f32(static_cast<uint16_t>(mu8[e]));
            const uint16_t vh = bf16_rne(v);
            ahi[tt][e] = static_cast<short>(vh);
            alo[tt][e] = static_cast<short>(bf16_rne(v - bf16_to_f32(vh)));
          }
        }
#pragma unroll
        for (int lt = 0; lt < NLT; ++lt) {
          const uint16_t* row = wd + static_cast<size_t>(16 * lt + lo) * (a.T * a.d_in) + 32 * s2 + 4 * hi;
          const u32x2 b0 = *reinterpret_cast<const u32x2*>(row);
          const u32x2 b1 = *reinterpret_cast<const u32x2*>(row + 16);
          const u32x4 bb = {b0.x, b0.y, b1.x, b1.y};
          const i16x8 bfrag = __builtin_bit_cast(i16x8, bb);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            lat[tt][lt] = mfma_bf16_k32(ahi[tt], bfrag, lat[tt][lt]);
            lat[tt][lt] = mfma_bf16_k32(alo[tt], bfrag, lat[tt][lt]);
          }
        }
      }
    }
  }

  // lat[tt][lt] lane (lo, hi): the loop's term for token 32 w + 16 tt + 4 hi + i, entry 16 lt + lo
  const bool first = a.loop == 0, last = a.loop == a.T - 1;
  uint16_t* cache = static_cast<uint16_t*>(a.c);
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tok0 + 32 * wave + 16 * tt + 4 * hi + i;
      if (tok >= a.Ntok) continue;
      float* arow = a.acc + (static_cast<size_t>(tok) * a.Hc + hc) * a.RT + a.ao;
      const int b = tok / a.n_new, j = tok - b * a.n_new;
      uint16_t* crow = cache + ((static_cast<size_t>(b) * a.Hc + hc) * a.n_max + a.pos_start + j) * R;
#pragma unroll
      for (int lt = 0; lt < NLT; ++lt) {
        const int e = 16 * lt + lo;
        float v = lat[tt][lt][i];
        if (!first) v += arow[e];
        if (last) crow[e] = bf16_rne(v);
        else arow[e] = v;
      }
    }
  }
}

template <int R>
void launch_axis(const FusedArgs& a, bool per_head, hipStream_t s) {
  const int ntb = (a.Ntok + kTokWg - 1) / kTokWg;
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
