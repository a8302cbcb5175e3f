// Encode (gfx950): c = (x - mu) W_down for tokens whose T loops are finished
// ("Looped Latent Attention", Section 3 Eqs. 1-2; the latent of a token is written once,
// after its last loop).
//
// Computed transposed on the matrix cores, C^T (r x tokens) = W_down^T (r x K) X^T
// (K x tokens) with K = T * d_in, so that
//   * A fragments are rows of W_down^T and B fragments rows of x: both contiguous runs
//     of the contraction index;
//   * a lane ends up holding 4 consecutive latent entries of one token, stored as one
//     8-byte (bf16) or 16-byte (float32) write into the cache row.
// Centring: for float32 x - mu is formed before the MFMA; for bfloat16 the bias mu W_down
// is produced by the same MFMA with mu broadcast into every B column and subtracted
// from the float32 accumulator, so no intermediate is rounded to bfloat16. The result is
// rounded once (nearest, ties to even) into the storage type.
//
// A workgroup covers 32 tokens (two 16-column tiles; tokens run over (sequence, new
// token) jointly) of one latent head and RG row tiles of 16 latent entries, with KSPLIT
// waves that each take a contiguous 1/KSPLIT of the contraction. Long prompts use one
// wave over all row tiles (x is read once); a few appended tokens use one row tile per
// workgroup and split the contraction, so the whole GPU shares the W_down read. Partial
// sums of the KSPLIT waves are added in LDS in a fixed order (deterministic). The
// contraction loop loads step k + 1 while it multiplies step k.
#include "lla_device.h"
#include "lla_kernels.h"

namespace lla {

namespace {

template <typename T>
struct KsOf { static constexpr int value = 16; };
template <>
struct KsOf<bf16_t> { static constexpr int value = 32; };

__device__ __forceinline__ void store4(float* p, f32x4 v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16_t* p, f32x4 v) {
  uint2 w;
  w.x = static_cast<uint32_t>(f32_to_bf16_rne(v[0])) | (static_cast<uint32_t>(f32_to_bf16_rne(v[1])) << 16);
  w.y = static_cast<uint32_t>(f32_to_bf16_rne(v[2])) | (static_cast<uint32_t>(f32_to_bf16_rne(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = w;
}

template <typename T, int R, int RG, int KSPLIT, bool PAGED = false>
__global__ __launch_bounds__(64 * KSPLIT) void encode_kernel(EncodeArgs a, PageArgs pg) {
  constexpr int KS = KsOf<T>::value;
  using M = Mfma<T, KS>;
  constexpr int E = M::E;
  constexpr int NR = (R + 15) / 16;  // the last row tile is partial when 16 does not divide R
  constexpr int NT = 2;
  constexpr bool kBias = !std::is_same<T, float>::value;
  constexpr int NACC = NT * RG + (kBias ? RG : 0);
  __shared__ f32x4 red[KSPLIT > 1 ? KSPLIT - 1 : 1][NACC][64];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, hi = lane >> 4;
  const int j0 = blockIdx.x * (16 * NT);  // flattened (sequence, new token) index
  const int rt0 = blockIdx.y * RG;        // first row tile
  const int hc = blockIdx.z;
  const int K = a.Kdim;
  const int total = a.B * a.n_new;
  const int kper = K / KSPLIT;
  const int kbeg = wave * kper, kend = kbeg + kper;

  const T* w = static_cast<const T*>(a.w_down_t) + static_cast<size_t>(hc) * R * K;
  const T* mu = static_cast<const T*>(a.mu) + static_cast<size_t>(hc) * K;
  const T* xrow[NT];
  bool valid[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int tok = j0 + 16 * nt + lo;
    valid[nt] = tok < total;
    const int row = valid[nt] ? tok : total - 1;
    xrow[nt] = static_cast<const T*>(a.x) + (static_cast<size_t>(row) * a.Hc + hc) * K;
  }
  const T* wrow[RG];
  bool wok[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int r = 16 * (rt0 + g) + lo;
    wok[g] = (rt0 + g < NR) && (R % 16 == 0 || r < R);
    wrow[g] = w + static_cast<size_t>(wok[g] ? r : 0) * K;
  }

  f32x4 acc[NT][RG];
  f32x4 bias[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    bias[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  typename M::Frag xf[NT], mf, wf[RG];
  auto load_step = [&](int k0, typename M::Frag (&x)[NT], typename M::Frag& m, typename M::Frag (&wv)[RG]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) x[nt] = M::load(xrow[nt] + k0 + hi * E);
    m = M::load(mu + k0 + hi * E);
#pragma unroll
    for (int g = 0; g < RG; ++g) wv[g] = wok[g] ? M::load(wrow[g] + k0 + hi * E) : M::zero();
  };
  load_step(kbeg, xf, mf, wf);
  for (int k0 = kbeg; k0 < kend; k0 += KS) {
    typename M::Frag xn[NT], mn, wn[RG];
    const bool more = k0 + KS < kend;
    if (more) load_step(k0 + KS, xn, mn, wn);
    if constexpr (!kBias) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < E; ++e) xf[nt].v[e] -= mf.v[e];
    }
#pragma unroll
    for (int g = 0; g < RG; ++g) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt][g] = M::mma(wf[g], xf[nt], acc[nt][g]);
      if constexpr (kBias) bias[g] = M::mma(wf[g], mf, bias[g]);
    }
    if (more) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) xf[nt] = xn[nt];
      mf = mn;
#pragma unroll
      for (int g = 0; g < RG; ++g) wf[g] = wn[g];
    }
  }

  if constexpr (KSPLIT > 1) {
    // waves 1.. publish their partial sums; wave 0 adds them in wave order
    if (wave > 0) {
      int i = 0;
#pragma unroll
      for (int g = 0; g < RG; ++g) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) red[wave - 1][i++][lane] = acc[nt][g];
        if constexpr (kBias) red[wave - 1][i++][lane] = bias[g];
      }
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int ws = 0; ws < KSPLIT - 1; ++ws) {
      int i = 0;
#pragma unroll
      for (int g = 0; g < RG; ++g) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][g] = acc[nt][g] + red[ws][i++][lane];
        if constexpr (kBias) bias[g] = bias[g] + red[ws][i++][lane];
      }
    }
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (!valid[nt]) continue;
    const int tok = j0 + 16 * nt + lo;
    const int b = tok / a.n_new;
    const int j = tok - b * a.n_new;
    const int pos = a.pos_start + j;
    T* crow;
    if constexpr (PAGED) {  // row pos % 16 of the page the block table names for it
      const size_t page = static_cast<size_t>(page_of(pg, b, pos / kPage));
      crow = static_cast<T*>(a.c) + ((page * a.Hc + hc) * kPage + pos % kPage) * R;
    } else {
      crow = static_cast<T*>(a.c) + (static_cast<size_t>(b * a.Hc + hc) * a.n_max + pos) * R;
    }
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const int r4 = 16 * (rt0 + g) + 4 * hi;
      if (rt0 + g >= NR || (R % 16 != 0 && r4 >= R)) continue;
      f32x4 v = acc[nt][g];
      if constexpr (kBias) v = v - bias[g];
      store4(crow + r4, v);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Long prompts, general shapes. A workgroup of LLA_EP_WAVES waves covers 32 tokens per
// wave (two 16-token tiles) and every latent row tile of one latent head. Per contraction
// step the workgroup's x fragments (one 1 KiB block per token tile), W_down^T fragments
// (one block per row tile) and the mean fragment (one block) stream through a ring of
// LLA_EP_STAGES LDS stages with direct-to-LDS loads (global_load_lds_dwordx4: lane l
// writes bytes 16 l .. 16 l + 15 of a block), laid out so that every MFMA operand is one
// conflict-free 1 KiB LDS read. W_down^T is read once per workgroup's tokens, and the bias
// mu W_down once per workgroup (wave w takes the row tiles w, w + NW, ... and publishes
// them through LDS at the end).
// ---------------------------------------------------------------------------------------
#ifndef LLA_EP_STAGES
#define LLA_EP_STAGES 3
#endif
#ifndef LLA_EP_WAVES
#define LLA_EP_WAVES 8
#endif
#ifndef LLA_EP_HEADS_FAST
#define LLA_EP_HEADS_FAST 1
#endif
#ifndef LLA_EP_CPOL
#define LLA_EP_CPOL 0
#endif

typedef uint32_t ep_u32x4 __attribute__((ext_vector_type(4)));

// A plain workgroup barrier: the ring's loads are waited for explicitly (vmcnt), while a
// fenced __syncthreads() would make the compiler wait for every one of them.
__device__ __forceinline__ void ep_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename T, int R>
__global__ __launch_bounds__(64 * LLA_EP_WAVES) void encode_prefill_kernel(EncodeArgs a) {
  constexpr int KS = KsOf<T>::value;
  using M = Mfma<T, KS>;
  constexpr int E = M::E;                    // E * sizeof(T) == 16 bytes per lane
  static_assert(E * sizeof(T) == 16, "one 16-byte piece per lane per fragment");
  constexpr int NR = (R + 15) / 16;
  constexpr int NW = LLA_EP_WAVES;
  constexpr int NTT = 2 * NW;                // token tiles (16 tokens) per workgroup
  constexpr int BLK = NTT + NR + 1;          // blocks per stage: x tiles, W tiles, mean
  constexpr int NIW = (BLK + NW - 1) / NW;   // blocks each wave loads per stage
  constexpr int NB = LLA_EP_STAGES;
  constexpr bool kBias = !std::is_same<T, float>::value;
  constexpr int NBT = (NR + NW - 1) / NW;    // bias row tiles per wave
  static_assert(NB >= 2 && (NB - 2) * NIW <= 63, "vmcnt range");
  constexpr int LDS_UNITS = NB * BLK * 64;
  __shared__ ep_u32x4 lds[LDS_UNITS > NR * 64 ? LDS_UNITS : NR * 64];

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, hi = lane >> 4;
  // one-dimensional grid over (token block, latent head)
#if LLA_EP_HEADS_FAST
  const int hc = blockIdx.x % a.Hc;
  const int tok0 = (blockIdx.x / a.Hc) * (16 * NTT);
#else
  const int ntb = (a.B * a.n_new + 16 * NTT - 1) / (16 * NTT);
  const int hc = blockIdx.x / ntb;
  const int tok0 = (blockIdx.x % ntb) * (16 * NTT);
#endif
  const int K = a.Kdim;
  const int nsteps = K / KS;
  const int total = a.B * a.n_new;

  const T* x = static_cast<const T*>(a.x);
  const T* w = static_cast<const T*>(a.w_down_t) + static_cast<size_t>(hc) * R * K;
  const T* mu = static_cast<const T*>(a.mu) + static_cast<size_t>(hc) * K;
  // this lane's source for each of the wave's block slots, at contraction step 0
  const T* src[NIW];
  int blk[NIW];
#pragma unroll
  for (int k = 0; k < NIW; ++k) {
    int bi = wave + NW * k;
    if (bi >= BLK) bi = wave;  // even out the per-wave count with a repeat
    blk[k] = bi;
    if (bi < NTT) {
      const int token = min(tok0 + 16 * bi + lo, total - 1);
      src[k] = x + (static_cast<size_t>(token) * a.Hc + hc) * K + hi * E;
    } else if (bi < NTT + NR) {
      const int r = min(16 * (bi - NTT) + lo, R - 1);
      src[k] = w + static_cast<size_t>(r) * K + hi * E;
    } else {
      src[k] = mu + hi * E;
    }
  }
  auto issue = [&](int st) {
    const int step = min(st, nsteps - 1);  // past the end: reload the last step (unused)
    const int stage = st % NB;
#pragma unroll
    for (int k = 0; k < NIW; ++k) {
      const T* g = src[k] + static_cast<size_t>(step) * KS;
      ep_u32x4* d = lds + (stage * BLK + blk[k]) * 64;
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)g,
                                       (void __attribute__((address_space(3)))*)d, 16, 0,
                                       LLA_EP_CPOL);
    }
  };

  f32x4 acc[2][NR];
  f32x4 bias[NBT];
#pragma unroll
  for (int rt = 0; rt < NR; ++rt) acc[0][rt] = acc[1][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < NBT; ++b) bias[b] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < NB - 1; ++st) issue(st);
  for (int st = 0; st < nsteps; ++st) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NB - 2) * NIW) : "memory");
    ep_barrier();
    issue(st + NB - 1);
    const ep_u32x4* sb = lds + (st % NB) * BLK * 64;
    typename M::Frag xf[2], mf;
#pragma unroll
    for (int t = 0; t < 2; ++t) xf[t] = M::load(reinterpret_cast<const T*>(sb + (2 * wave + t) * 64 + lane));
    mf = M::load(reinterpret_cast<const T*>(sb + (NTT + NR) * 64 + lane));
    if constexpr (!kBias) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < E; ++e) xf[t].v[e] -= mf.v[e];
    }
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
      const typename M::Frag wf = M::load(reinterpret_cast<const T*>(sb + (NTT + rt) * 64 + lane));
      acc[0][rt] = M::mma(wf, xf[0], acc[0][rt]);
      acc[1][rt] = M::mma(wf, xf[1], acc[1][rt]);
      if constexpr (kBias) {
        if (rt % NW == wave) bias[rt / NW] = M::mma(wf, mf, bias[rt / NW]);
      }
    }
  }
  // every direct-to-LDS load has landed before the LDS is reused or the wave exits
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f32x4* bl = reinterpret_cast<f32x4*>(lds);
  if constexpr (kBias) {
#pragma unroll
    for (int b = 0; b < NBT; ++b) {
      const int rt = wave + NW * b;
      if (rt < NR) bl[rt * 64 + lane] = bias[b];
    }
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int tok = tok0 + 32 * wave + 16 * t + lo;
    if (tok >= total) continue;
    const int b = tok / a.n_new;
    const int j = tok - b * a.n_new;
    T* crow = static_cast<T*>(a.c) + (static_cast<size_t>(b * a.Hc + hc) * a.n_max + a.pos_start + j) * R;
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
      const int r4 = 16 * rt + 4 * hi;
      if (R % 16 != 0 && r4 >= R) continue;
      f32x4 v = acc[t][rt];
      if constexpr (kBias) v = v - bl[rt * 64 + lane];
      store4(crow + r4, v);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Long prompts, per-head bfloat16 with a short contraction (K = T d_in of 256 or 512).
// W_down^T of one latent head stays in registers: wave w holds row tiles
// NRW w .. NRW w + NRW - 1 for every contraction step, and the bias mu W_down of those rows,
// both loaded once per workgroup. The workgroup then walks a contiguous run of 16-token
// tiles; each tile's x (16 tokens x K, all contraction steps) is one ring stage of NS
// 1 KiB blocks filled with direct-to-LDS loads, so every token's K values are requested
// together and read from HBM exactly once. Each wave multiplies its row tiles against the
// stage (one conflict-free LDS read per contraction step) and stores its latents.
// ---------------------------------------------------------------------------------------
#ifndef LLA_ES_STAGES
#define LLA_ES_STAGES 4
#endif
#ifndef LLA_ES_NRW
#define LLA_ES_NRW 3
#endif
#ifndef LLA_ES_WG_TARGET
#define LLA_ES_WG_TARGET 1024
#endif

template <int R>
struct EsShape {
  static constexpr int NR = (R + 15) / 16;
  static constexpr int NRW = NR < LLA_ES_NRW ? NR : LLA_ES_NRW;  // row tiles per wave
  static constexpr int NW = (NR + NRW - 1) / NRW;                  // waves per workgroup
};

template <int R, int NS>
__global__ __launch_bounds__(64 * EsShape<R>::NW) void encode_stream_kernel(EncodeArgs a,
                                                                              int tiles_per_wg) {
  using T = bf16_t;
  using M = Mfma<T, 32>;
  constexpr int E = M::E;
  constexpr int NR = EsShape<R>::NR, NRW = EsShape<R>::NRW, NW = EsShape<R>::NW;
  constexpr int NB = LLA_ES_STAGES;
  constexpr int NIW = (NS + NW - 1) / NW;  // blocks each wave loads per stage
  static_assert(NW <= NS, "every wave owns at least one block of a stage");
  static_assert(NB >= 2, "a ring needs two stages");
  // loads of later stages allowed in flight (the counter holds 63 at most; fewer is safe)
  constexpr int kWait = (NB - 2) * NIW < 63 ? (NB - 2) * NIW : 63;
  __shared__ ep_u32x4 lds[NB * NS * 64];

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int lo = lane & 15, hi = lane >> 4;
  const int hc = blockIdx.x % a.Hc;
  const int total = a.B * a.n_new;
  const int ntiles = (total + 15) / 16;
  const int t_begin = (blockIdx.x / a.Hc) * tiles_per_wg;
  const int nt = min(t_begin + tiles_per_wg, ntiles) - t_begin;
  if (nt <= 0) return;  // uniform over the workgroup
  constexpr int K = NS * 32;

  const T* w = static_cast<const T*>(a.w_down_t) + static_cast<size_t>(hc) * R * K;
  const T* mu = static_cast<const T*>(a.mu) + static_cast<size_t>(hc) * K;
  const T* x = static_cast<const T*>(a.x);

  // this lane's block slots: contraction step of each (repeats even out the count)
  int step[NIW];
#pragma unroll
  for (int k = 0; k < NIW; ++k) step[k] = (wave + NW * k < NS) ? wave + NW * k : wave;
  auto issue = [&](int rel) {
    const int tile = t_begin + min(rel, nt - 1);  // past the end: reload the last tile (unused)
    const int token = min(tile * 16 + lo, total - 1);
    const T* src = x + (static_cast<size_t>(token) * a.Hc + hc) * K + hi * E;
    ep_u32x4* base = lds + (rel % NB) * NS * 64;
#pragma unroll
    for (int k = 0; k < NIW; ++k)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(src + step[k] * 32),
                                       (void __attribute__((address_space(3)))*)(base + step[k] * 64),
                                       16, 0, 0);
  };
#pragma unroll
  for (int st = 0; st < NB - 1; ++st) issue(st);

  // resident operands: W_down^T fragments of this wave's row tiles and their bias
  typename M::Frag wf[NRW][NS];
  f32x4 bias[NRW];
#pragma unroll
  for (int i = 0; i < NRW; ++i) {
    const int r = min(16 * (wave * NRW + i) + lo, R - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s) wf[i][s] = M::load(w + static_cast<size_t>(r) * K + s * 32 + hi * E);
    bias[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const typename M::Frag mf = M::load(mu + s * 32 + hi * E);
#pragma unroll
    for (int i = 0; i < NRW; ++i) bias[i] = M::mma(wf[i][s], mf, bias[i]);
  }

  for (int rel = 0; rel < nt; ++rel) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWait) : "memory");
    ep_barrier();
    issue(rel + NB - 1);
    const ep_u32x4* sb = lds + (rel % NB) * NS * 64;
    f32x4 acc[NRW];
#pragma unroll
    for (int i = 0; i < NRW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const typename M::Frag xf = M::load(reinterpret_cast<const T*>(sb + s * 64 + lane));
#pragma unroll
      for (int i = 0; i < NRW; ++i) acc[i] = M::mma(wf[i][s], xf, acc[i]);
    }
    const int tok = (t_begin + rel) * 16 + lo;
    if (tok < total) {
      const int b = tok / a.n_new;
      const int j = tok - b * a.n_new;
      T* crow = static_cast<T*>(a.c) + (static_cast<size_t>(b * a.Hc + hc) * a.n_max + a.pos_start + j) * R;
#pragma unroll
      for (int i = 0; i < NRW; ++i) {
        const int rt = wave * NRW + i;
        const int r4 = 16 * rt + 4 * hi;
        if (rt < NR && (R % 16 == 0 || r4 < R)) store4(crow + r4, acc[i] - bias[i]);
      }
    }
  }
  // every direct-to-LDS load has landed before the wave exits
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int R, int NS>
void launch_stream(const EncodeArgs& a, hipStream_t s) {
  const long long ntiles = (static_cast<long long>(a.B) * a.n_new + 15) / 16;
  const long long nch = std::max<long long>(1, (LLA_ES_WG_TARGET + a.Hc - 1) / a.Hc);
  const int per = static_cast<int>((ntiles + nch - 1) / nch);
  const long long groups = (ntiles + per - 1) / per;
  hipLaunchKernelGGL((encode_stream_kernel<R, NS>), dim3(static_cast<unsigned>(groups * a.Hc)),
                     dim3(64 * EsShape<R>::NW), 0, s, a, per);
}

template <typename T, int R, int RG, int KSPLIT, bool PAGED = false>
void launch(const EncodeArgs& a, hipStream_t s, const PageArgs& pg = PageArgs{}) {
  constexpr int NR = (R + 15) / 16;
  const long long total = static_cast<long long>(a.B) * a.n_new;
  dim3 grid(static_cast<unsigned>((total + 31) / 32), (NR + RG - 1) / RG, a.Hc);
  hipLaunchKernelGGL((encode_kernel<T, R, RG, KSPLIT, PAGED>), grid, dim3(64 * KSPLIT), 0, s, a, pg);
}

// Paged cache: the few-token kernel for any token count (its rows are addressed per token).
template <typename T, int R>
void launch_shape_paged(const EncodeArgs& a, const PageArgs& pg, hipStream_t s) {
  constexpr int NR = (R + 15) / 16;
  const long long tiles = (static_cast<long long>(a.B) * a.n_new + 31) / 32;
  if (tiles * a.Hc >= 1024) {
    launch<T, R, NR, 1, true>(a, s, pg);
  } else if (a.Kdim % (8 * KsOf<T>::value) == 0 && a.Kdim >= 8 * 256) {
    launch<T, R, 1, 8, true>(a, s, pg);
  } else {
    launch<T, R, 1, 1, true>(a, s, pg);
  }
}

// Long prompts: the register-resident W_down^T stream for per-head bfloat16 with a short
// contraction, else the ring kernel. Few tokens: one row tile per workgroup and
// the contraction split over up to 8 waves (or one wave over all row tiles when there are
// enough token tiles to fill the GPU).
template <typename T, int R>
void launch_shape(const EncodeArgs& a, hipStream_t s) {
  constexpr int NR = (R + 15) / 16;
  const long long total = static_cast<long long>(a.B) * a.n_new;
  const long long tiles = (total + 31) / 32;
  if constexpr (!std::is_same<T, float>::value) {
    const long long ntiles = (total + 15) / 16;
    if (ntiles * a.Hc >= 4096 && (a.Kdim == 256 || a.Kdim == 512)) {
      if (a.Kdim == 256) launch_stream<R, 8>(a, s);
      else launch_stream<R, 16>(a, s);
      return;
    }
  }
  constexpr int kTokWG = 32 * LLA_EP_WAVES;
  const long long tblocks = (total + kTokWG - 1) / kTokWG;
  if (tblocks * a.Hc >= 512 && tblocks * a.Hc < (1LL << 24) && a.Kdim % KsOf<T>::value == 0) {
    const dim3 grid(static_cast<unsigned>(tblocks * a.Hc));
    hipLaunchKernelGGL((encode_prefill_kernel<T, R>), grid, dim3(64 * LLA_EP_WAVES), 0, s, a);
  } else if (tiles * a.Hc >= 1024) {
    launch<T, R, NR, 1>(a, s);
  } else if (a.Kdim % (8 * KsOf<T>::value) == 0 && a.Kdim >= 8 * 256) {
    launch<T, R, 1, 8>(a, s);
  } else {
    launch<T, R, 1, 1>(a, s);
  }
}

}  // namespace

#define LLA_ENCODE_RANKS(X) X(16) X(24) X(32) X(64) X(96) X(128) X(160) X(256)

bool encode_supported(int dtype, int r, int Kdim) {
  const int ks = dtype == 0 ? 16 : 32;
  if (Kdim % ks != 0) return false;
#define X(R_) if (r == R_) return true;
  LLA_ENCODE_RANKS(X)
#undef X
  return false;
}

bool launch_encode_paged(int dtype, int r, const EncodeArgs& a, const PageArgs& pg, hipStream_t s) {
  if (pg.table == nullptr) return false;
#define X(R_)                                                \
  if (r == R_) {                                             \
    if (dtype == 0) launch_shape_paged<float, R_>(a, pg, s); \
    else launch_shape_paged<bf16_t, R_>(a, pg, s);           \
    return true;                                             \
  }
  LLA_ENCODE_RANKS(X)
#undef X
  return false;
}

bool launch_encode(int dtype, int r, const EncodeArgs& a, hipStream_t s) {
#define X(R_)                                        \
  if (r == R_) {                                     \
    if (dtype == 0) launch_shape<float, R_>(a, s);   \
    else launch_shape<bf16_t, R_>(a, s);             \
    return true;                                     \
  }
  LLA_ENCODE_RANKS(X)
#undef X
  return false;
}

}  // namespace lla
