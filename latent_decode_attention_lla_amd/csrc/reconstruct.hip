// Materialised reconstruction (gfx950, wave64; bfloat16 or float32 latents).
//
// Rebuilds loop t's keys or values of a range of cache slots from one layer's latents,
//   x_t[j] = c[j] W_up,t^T + mu_t   ("Looped Latent Attention", Section 3 Eq. 3),
// and rotates the keys at their slot index (Section 3, "RoPE and reconstruction"). This
// is what the latent-store decoder's two-pass prefill feeds its second pass, one layer
// at a time so that no layer's full-width K/V outlives its use (Appendix A, "Decoding and
// caching"; Appendix J, "Eviction and long-context prefill"); the rebuilt rows use the
// layout of the uncompressed cache, so they can also be attended directly.
//
// A workgroup owns one (sequence, head) and a chunk of slots, with one wave per (loop,
// group of MS row tiles of the head dimension). A wave keeps its rows of W_up,t as MFMA A
// fragments and mu_t as accumulator seeds, and per 16-slot tile computes
// X^T (16 MS rows x 16 slots) = W_up,t C^T + mu_t on the matrix cores, loading the next
// tile's latents while it multiplies the current one. The waves of a workgroup read the
// same latent tiles, so the chunk is read from HBM once and served to the loops from the
// CU's cache. The MFMA leaves a lane 4 consecutive entries of one slot's row; the wave
// passes its tile through LDS (float32) so that in the copy-out each lane owns a 16-byte
// piece of one row in the storage type: consecutive lanes cover consecutive row pieces,
// the RoPE angles are read contiguously (and once per tile, by angle addition), and each
// store instruction writes whole rows
// (a direct store of the MFMA layout writes 16 separate short pieces per instruction, at
// about a third of the bandwidth). bfloat16 results are rounded once, to nearest even.
#include "lla_device.h"
#include "lla_kernels.h"

namespace lla {

namespace {

constexpr int kMaxWaves = 8;  // waves per workgroup (loops x row-tile groups)

#ifndef LLA_RECON_WFRAGS
#define LLA_RECON_WFRAGS 24  // W_up fragments a wave keeps in registers (4 registers each)
#endif

// Row tiles of the head dimension per wave: as many as keep the W_up fragments within
// about 96 registers.
template <typename T, int D, int R>
struct ReconShape {
  static constexpr int KS = KStep<T, R>::value;
  static constexpr int NK = (R + KS - 1) / KS;  // the last super-step is zero-padded
  static constexpr int NM = D / 16;
  static constexpr int MS0 = LLA_RECON_WFRAGS / NK < 1 ? 1 : LLA_RECON_WFRAGS / NK;
  // at least 2 in bfloat16, so that a row piece of the copy-out is 16 bytes
  static constexpr int MSF = MS0 >= NM ? NM : (MS0 >= 4 ? 4 : (MS0 >= 2 ? 2 : 1));
  static constexpr int MS = (sizeof(T) == 2 && MSF < 2) ? 2 : MSF;
  static constexpr int NMG = NM / MS;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <typename T, int D, int R>
__global__ __launch_bounds__(64 * kMaxWaves) void reconstruct_kernel(ReconArgs a) {
  using S = ReconShape<T, D, R>;
  constexpr int KS = S::KS, NK = S::NK, MS = S::MS, NMG = S::NMG;
  using M = Mfma<T, KS>;
  constexpr int E = M::E;
  static_assert(R % E == 0, "a lane's fragment is wholly inside or outside the latent");

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, hi = lane >> 4;
  const int li = wave / NMG, mg = wave - li * NMG;
  const int chunk = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int t = a.loop_begin + li;
  const int hc = a.variant == 0 ? h : 0;

  const int j0 = a.pos_start + chunk * a.chunk;
  const int j1 = min(a.pos_start + a.n_tok, j0 + a.chunk);

  // Loop-invariant operands: this wave's rows of W_up,t (A fragments, zero past R) and
  // mu_t (accumulator seeds).
  const T* w = static_cast<const T*>(a.w_up) + static_cast<size_t>(t * a.H + h) * D * R;
  const size_t mu_off = a.variant == 0 ? static_cast<size_t>(h * a.T + t) * D
                                       : static_cast<size_t>(t * a.H + h) * D;
  const T* mu = static_cast<const T*>(a.mu) + mu_off;
  typename M::Frag wf[MS][NK];
  f32x4 mu4[MS];
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    const int row = 16 * (mg * MS + m);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int k0 = ks * KS + hi * E;
      wf[m][ks] = k0 < R ? M::load(w + (row + lo) * R + k0) : M::zero();
    }
    float tmp[4];
    load_f32<4>(mu + row + 4 * hi, tmp);
    mu4[m] = f32x4{tmp[0], tmp[1], tmp[2], tmp[3]};
  }

  const T* c = static_cast<const T*>(a.c) + static_cast<size_t>(b * a.Hc + hc) * a.n_max * R;
  T* out = static_cast<T*>(a.out) + (static_cast<size_t>(li * a.B + b) * a.H + h) * a.n_max * D;

  auto load_tile = [&](typename M::Frag* cf, int tile) {
    const int row = min(tile + lo, j1 - 1);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int k0 = ks * KS + hi * E;
      cf[ks] = k0 < R ? M::load(c + static_cast<size_t>(row) * R + k0) : M::zero();
    }
  };

  // This wave's staging tile: 16 slots x (16 MS) float32 entries, rows padded by 16 bytes
  // so the 16 slots of a write start in different banks. The copy-out gives each lane
  // EPL consecutive entries of one slot (one 16-byte store in the storage type), rotates
  // their pairs with one contiguous read of the slot's table row, rounds and stores.
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr int EPL = 16 / ES;             // output entries per lane in the copy-out
  constexpr int ROWP = 16 * MS * 4 + 16;   // padded LDS row (bytes)
  constexpr int LPR = 16 * MS / EPL;       // lanes per slot row in the copy-out
  constexpr int RPI = 64 / LPR;            // slot rows per store instruction
  static_assert(64 % LPR == 0 && 16 % RPI == 0, "copy-out shape");
  extern __shared__ __attribute__((aligned(16))) char lds_dyn[];
  char* stage = lds_dyn + wave * (16 * ROWP);
  const int cl = lane % LPR, cr = lane / LPR;  // copy-out: piece cl of slot row cr + RPI i
  const int d0 = 16 * mg * MS + cl * EPL;      // first head-dimension entry of that piece

  // The table's first 16 rows (the angles of slot offsets 0 .. 15), shared by every tile of
  // the workgroup, are kept in LDS.
  __shared__ __attribute__((aligned(16))) float rope_lo[16 * D];
  if (a.rope32 != nullptr) {
    const int nrow = min(16, a.n_max);
    for (int i = threadIdx.x; i < 16 * D; i += blockDim.x)
      rope_lo[i] = i < nrow * D ? a.rope32[i] : 0.f;
  }
  __syncthreads();

  typename M::Frag ca[NK], cb[NK];
  auto compute = [&](const typename M::Frag* cf, int tile) {
    // the angles of the tile's first slot, requested before the matrix work
    float4 base4[EPL / 4];
    if (a.rope32 != nullptr) {
#pragma unroll
      for (int q4 = 0; q4 < EPL; q4 += 4)
        base4[q4 / 4] = *reinterpret_cast<const float4*>(a.rope32 + static_cast<size_t>(tile) * D + d0 + q4);
    }
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      f32x4 x = mu4[m];
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) x = M::mma(wf[m][ks], cf[ks], x);
      *reinterpret_cast<f32x4*>(stage + lo * ROWP + (16 * m + 4 * hi) * 4) = x;
    }
    lds_wait();
#pragma unroll
    for (int i = 0; i < 16 / RPI; ++i) {
      const int r = cr + RPI * i;
      const int tk = tile + r;
      float v[EPL];
#pragma unroll
      for (int q4 = 0; q4 < EPL; q4 += 4) {
        const f32x4 f = *reinterpret_cast<const f32x4*>(stage + r * ROWP + (cl * EPL + q4) * 4);
        v[q4] = f[0]; v[q4 + 1] = f[1]; v[q4 + 2] = f[2]; v[q4 + 3] = f[3];
      }
      if (a.rope32 != nullptr) {
        // The angle of slot tile + r is the sum of those of slots tile and r: its (cos, sin)
        // come from the table row of the tile's first slot (read once per tile) and one of
        // the table's first 16 rows (in LDS). Pair p of the piece is entries 2p, 2p + 1.
        const float* cd = rope_lo + r * D + d0;
#pragma unroll
        for (int q4 = 0; q4 < EPL; q4 += 4) {
          const float4 b4 = base4[q4 / 4];
          const float4 d4 = *reinterpret_cast<const float4*>(cd + q4);
          const float c0 = b4.x * d4.x - b4.y * d4.y, s0 = b4.y * d4.x + b4.x * d4.y;
          const float c1 = b4.z * d4.z - b4.w * d4.w, s1 = b4.w * d4.z + b4.z * d4.w;
          const float x0 = v[q4], x1 = v[q4 + 1], x2 = v[q4 + 2], x3 = v[q4 + 3];
          v[q4] = x0 * c0 - x1 * s0;
          v[q4 + 1] = x0 * s0 + x1 * c0;
          v[q4 + 2] = x2 * c1 - x3 * s1;
          v[q4 + 3] = x2 * s1 + x3 * c1;
        }
      }
      if (tk < j1) {  // one 16-byte store per lane
        u32x4 pk;
        if constexpr (ES == 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) pk[e] = __float_as_uint(v[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pk[e] = static_cast<uint32_t>(f32_to_bf16_rne(v[2 * e])) |
                    (static_cast<uint32_t>(f32_to_bf16_rne(v[2 * e + 1])) << 16);
        }
        // written once and read by a later kernel: stream it past the caches
        __builtin_nontemporal_store(pk, reinterpret_cast<u32x4*>(out + static_cast<size_t>(tk) * D + d0));
      }
    }
    lds_wait();  // the next tile's writes into the staging tile come after these reads
  };

  if (j0 >= j1) return;
  load_tile(ca, j0);
  for (int tile = j0; tile < j1; tile += 32) {
    if (tile + 16 < j1) load_tile(cb, tile + 16);
    compute(ca, tile);
    if (tile + 16 >= j1) break;
    if (tile + 32 < j1) load_tile(ca, tile + 32);
    compute(cb, tile + 16);
  }
}

template <typename T, int D, int R>
void launch(const ReconArgs& a, hipStream_t s) {
  using S = ReconShape<T, D, R>;
  const int nchunk = (a.n_tok + a.chunk - 1) / a.chunk;
  const int waves = a.L * S::NMG;
  const size_t lds = static_cast<size_t>(waves) * 16 * (16 * S::MS * 4 + 16);
  hipLaunchKernelGGL((reconstruct_kernel<T, D, R>), dim3(nchunk, a.H, a.B), dim3(64 * waves), lds,
                     s, a);
}

}  // namespace

#define LLA_RECON_SHAPES(X)                                                         \
  X(64, 16) X(64, 24) X(64, 32) X(64, 64) X(64, 96) X(64, 128) X(64, 160) X(64, 256) \
  X(128, 16) X(128, 24) X(128, 32) X(128, 64) X(128, 96) X(128, 128) X(128, 160) X(128, 256)

bool reconstruct_supported(int dtype, int d, int r) {
  (void)dtype;
#define X(D_, R_) \
  if (d == D_ && r == R_) return true;
  LLA_RECON_SHAPES(X)
#undef X
  return false;
}

// Loops one workgroup covers: at most kMaxWaves waves and 64 KiB of staging tiles.
template <typename T, int D, int R>
int max_loops() {
  using S = ReconShape<T, D, R>;
  const int by_waves = kMaxWaves / S::NMG;
  const int by_lds = (64 * 1024) / (16 * (16 * S::MS * 4 + 16) * S::NMG);
  return by_waves < by_lds ? by_waves : by_lds;
}

int reconstruct_max_loops(int dtype, int d, int r) {
#define X(D_, R_)                                                                   \
  if (d == D_ && r == R_)                                                           \
    return dtype == 0 ? max_loops<float, D_, R_>() : max_loops<bf16_t, D_, R_>();
  LLA_RECON_SHAPES(X)
#undef X
  return 0;
}

bool launch_reconstruct(int dtype, int d, int r, const ReconArgs& a, hipStream_t s) {
#define X(D_, R_)                                   \
  if (d == D_ && r == R_) {                         \
    if (dtype == 0) launch<float, D_, R_>(a, s);    \
    else launch<bf16_t, D_, R_>(a, s);              \
    return true;                                    \
  }
  LLA_RECON_SHAPES(X)
#undef X
  return false;
}

}  // namespace lla
