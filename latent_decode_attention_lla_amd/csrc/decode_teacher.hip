// Uncompressed decode over the loop-indexed cache (gfx950, wave64; bfloat16 or float32).
//
// The teacher of "Looped Latent Attention" keeps keys and values for every loop t of every
// layer (Section 3, "Teacher cache"; Section 7, Table 5's teacher column). This is the
// decode that reads that cache directly, the baseline the latent store is compared with:
//   out[b][h][t] = softmax_j(scale q . K_t[j]) V_t[j]   over j < len_b,
// with K_t stored already rotated to its positions.
//
// decode_teacher_kernel: one wave per (sequence, head, loop, split). A token's key (and
// value) row is read as 16-byte pieces by GP consecutive lanes, so each load instruction
// of the wave covers 64 / GP whole consecutive rows, one contiguous KiB. The partial dots
// are summed over a row's lanes with DPP, and a per-row-slot online softmax (max raised
// only past a 2^8 slack, exact) accumulates the weighted value pieces. Two chunks of rows
// are in flight: chunk c + 1 loads while chunk c is computed; chunks wholly inside the
// context skip the clamping and masking. One split writes the normalised output; more
// write (max, sum, acc[d]) partials that combine_kernel merges without an up-projection.
#include <type_traits>

#include "decode_stream.h"
#include "lla_device.h"
#include "lla_kernels.h"

namespace lla {

namespace {

using namespace stream;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMaxInit = -1.0e30f;  // finite stand-in for -inf (see the fold kernels)
constexpr float kRescaleSlack = 8.0f;

template <typename T, int D, int TPC>
__global__ __launch_bounds__(64) void decode_teacher_kernel(DecodeArgs a) {
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr int EPL = 16 / ES;   // row elements per lane: one 16-byte load
  constexpr int GP = D / EPL;    // lanes per row
  constexpr int TOK = 64 / GP;   // rows per tile
  static_assert(D % EPL == 0 && GP >= 2 && 64 % GP == 0, "whole rows per wave");
  struct Rows {
    u32x4 k[TPC];
    u32x4 v[TPC];
  };

  const int lane = threadIdx.x;
  const int tok = lane / GP, grp = lane % GP;
  const int split = blockIdx.x;
  const int h = blockIdx.y / a.L;
  const int li = blockIdx.y - h * a.L;
  const int b = blockIdx.z;
  const int t = a.loop_begin + li;
  const size_t unit = static_cast<size_t>(b * a.H + h) * a.L + li;

  int len = a.n_ctx;
  if (a.ctx_lens != nullptr) len = max(0, min(a.ctx_lens[b], a.n_ctx));
  const int s0 = split * a.split_len;
  const int s1 = min(len, s0 + a.split_len);
  const int ntok = max(0, s1 - s0);
  const int nchunk = (ntok + TOK * TPC - 1) / (TOK * TPC);
  const int nfull = ntok / (TOK * TPC);

  const float* qg = a.q + unit * D + grp * EPL;
  float qs[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qs[e] = qg[e] * a.scale_log2e;

  const size_t plane = (static_cast<size_t>(t * a.B + b) * a.H + h) * a.n_max;
  const char* kc = static_cast<const char*>(a.c_k) + plane * D * ES + grp * 16;
  const char* vc = static_cast<const char*>(a.c_v) + plane * D * ES + grp * 16;

  auto load_chunk = [&](Rows& R, int c) {
    const int tok0 = s0 + c * TPC * TOK;
    const bool clamp = c >= nfull;
#pragma unroll
    for (int tt = 0; tt < TPC; ++tt) {
      const int row0 = tok0 + TOK * tt + tok;
      const size_t row = static_cast<size_t>(clamp ? min(row0, s1 - 1) : row0);
      R.k[tt] = load16(kc + row * (D * ES));
      R.v[tt] = load16(vc + row * (D * ES));
    }
  };

  float m_run = kMaxInit, l_run = 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

  auto compute_chunk = [&](int c, const Rows& R, auto full) {
    constexpr bool FULL = decltype(full)::value;
#pragma unroll
    for (int tt = 0; tt < TPC; ++tt) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) part += qs[e] * elem16<T>(R.k[tt], e);
      part = sum_lanes<GP>(part);
      const int tk = s0 + (c * TPC + tt) * TOK + tok;
      const float s = (FULL || tk < s1) ? part : kNegInf;
      const bool raise = s > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = raise ? s : m_run;
        const float alpha = raise ? fast_exp2(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
        m_run = m_new;
      }
      const float p = fast_exp2(s - m_run);
      l_run += p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += p * elem16<T>(R.v[tt], e);
    }
  };
  auto compute = [&](int c, const Rows& R) {
    if (c < nfull) compute_chunk(c, R, std::true_type{});
    else compute_chunk(c, R, std::false_type{});
  };

  Rows ra, rb;
  if (nchunk > 0) load_chunk(ra, 0);
  for (int c = 0; c < nchunk; c += 2) {
    if (c + 1 < nchunk) load_chunk(rb, c + 1);
    compute(c, ra);
    if (c + 1 >= nchunk) break;
    if (c + 2 < nchunk) load_chunk(ra, c + 2);
    compute(c + 1, rb);
  }

  // ---- merge the TOK row slots (lane bits above the row's lanes) ----------------------
  float mx = m_run;
#pragma unroll
  for (int msk = GP; msk < 64; msk <<= 1) mx = fmaxf(mx, shfl_xor(mx, msk));
  const float scl = fast_exp2(m_run - mx);
  float lsum = l_run * scl;
#pragma unroll
  for (int msk = GP; msk < 64; msk <<= 1) lsum += shfl_xor(lsum, msk);
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    float v = acc[e] * scl;
#pragma unroll
    for (int msk = GP; msk < 64; msk <<= 1) v += shfl_xor(v, msk);
    acc[e] = v;
  }

  if (tok != 0) return;
  if (a.S > 1) {
    float* out = a.part + (unit * a.S + split) * (2 + D);
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[2 + grp * EPL + e] = acc[e];
    if (grp == 0) {
      out[0] = mx;
      out[1] = lsum;
    }
    return;
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  float* out = a.out + unit * D + grp * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[e] = acc[e] * inv;
}

#ifndef LLA_TEACHER_TPC
#define LLA_TEACHER_TPC 2  // tiles of TOK rows per chunk; two chunks are in flight
#endif

template <typename T, int D>
void launch(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((decode_teacher_kernel<T, D, LLA_TEACHER_TPC>), dim3(a.S, a.H * a.L, a.B),
                     dim3(64), 0, s, a);
}

}  // namespace

// (element type, dtype code, d_head)
#define LLA_TEACHER_SHAPES(X) \
  X(bf16_t, 1, 128)           \
  X(bf16_t, 1, 64)            \
  X(float, 0, 64)             \
  X(float, 0, 128)

bool decode_teacher_supported(int dtype, int d) {
#define X(T_, DT_, D_) \
  if (dtype == DT_ && d == D_) return true;
  LLA_TEACHER_SHAPES(X)
#undef X
  return false;
}

bool launch_decode_teacher(int dtype, int d, const DecodeArgs& a, hipStream_t s) {
#define X(T_, DT_, D_)           \
  if (dtype == DT_ && d == D_) { \
    launch<T_, D_>(a, s);        \
    return true;                 \
  }
  LLA_TEACHER_SHAPES(X)
#undef X
  return false;
}

}  // namespace lla
