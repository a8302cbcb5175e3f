"""Seeded synthetic inputs for the LLA latent-store decode path.

This module only draws random numbers and lays them out; it holds none of the method's
arithmetic. The HIP path (through the binding) and the fp64 oracle (in tests) are fed
the same tensors from here.

Workloads (shapes from "Looped Latent Attention", Section 5 setup and Appendix A:
Ouro-1.4B has D=24 layers, H=16 heads, d_head=128, T=4 loops; ranks from Table 8 and
Table 5):

* ``tiny_f32``     T=4, D=1, H=2, d=64, (r_k, r_v)=(16, 24), fp32, batch 1, context 128
* ``ouro_layer_4x`` T=4, D=1, H=16, d=128, (96, 160), bf16, batch 32, context 4096
* ``capacity_21x``  T=4, D=24, H=16, d=128, (16, 32), bf16, batch 768, context 4096
* ``encode_heavy``  T=4, D=1, H=16, d=128, (96, 160), bf16, batch 8, context 8192
* ``lla2d_long``    LLA-2D, T=4, D=24, H=16, d=128, shared (96, 160), bf16, batch 16,
                    context 16384
* ``absorbed_4x``   the Ouro-1.4B 4x geometry, T=4, D=24, H=16, d=128, (96, 160), bf16,
                    decoupled decode with a 64-wide rotary branch (Appendix J, Table 14's
                    d_rope), batch 8, context 32768 (Table 13's shortest context)
* ``prefill_64k``   the two-pass prefill of one 65536-token prompt at the Ouro-1.4B 4x
                    geometry (T=4, D=24, H=16, d=128, (96, 160), bf16, hidden size 2048):
                    pass 1 encodes while the looped stack runs (the K/V projections fused
                    with the latent accumulation, loop by loop), pass 2 rebuilds each
                    layer's K/V for all loops (Appendix J's 64k passkey cells; Table 12)
* ``paged_21x``     ``capacity_21x`` stored in a paged cache: 16-token pages of each
                    layer's pool in a random order, found through a block table
* ``paged_ouro_4x`` the Ouro-1.4B 4x geometry (96, 160) for all 24 layers, 32 sequences at
                    context 4096, in a paged cache (the wide fold kernel)
* ``paged_absorbed_4x`` ``absorbed_4x`` over a paged cache: latents and rotary keys in
                    shuffled 16-token pages under one block table per sequence
* ``teacher_4k``    the uncompressed loop-indexed cache the latent store replaces (Section
                    3 "Teacher cache"; Table 5's teacher column): T=4, D=24, H=16, d=128,
                    bf16 keys and values for every loop, batch 32 (the teacher's measured
                    capacity at 4k), context 4096

Distributions: latents, queries and pre-RoPE K/V ~ N(0, 1); W_up,t ~ N(0, 1/r)
(variance 1/r, so rebuilt keys have about unit variance); mu ~ N(0, 0.1) (variance).
Encode-side codecs: ``orthonormal`` (QR of a Gaussian; W_up,t are the loop slices
of W_down, the structure the SVD initialisation produces) or Gaussian.

Memory layouts (all row-major, shared with the C ABI):
  c_k  [D][B][Hc][n_max][r_k]     c_v  [D][B][Hc][n_max][r_v]
  k_rope [D][B][H][n_max][d_rope] (rotary keys of the decoupled decode, ~ N(0, 1))
  k_cache, v_cache [D][T][B][H][n_max][d] (the uncompressed cache, ~ N(0, 1); keys
                  already rotated)
  w_down_k_t [D][Hc][r_k][T*d_in] (W_down transposed)   mu_k [D][Hc][T*d_in]
  w_up_k [D][T][H][d][r_k]        (same for v)
  q    [D][T][B][H][d]  (post-RoPE queries for every layer and loop)
  x_k, x_v [B][n_new][Hc][T][d_in]  (pre-RoPE per-loop keys/values to encode)
Hc = H and d_in = d for the per-head codec; Hc = 1 and d_in = H*d for LLA-2D.
"""

from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    D: int
    H: int
    d: int
    r_k: int
    r_v: int
    batch: int
    n: int
    variant: str = "per_head"      # "per_head" or "2d"
    dtype: str = "bf16"            # "f32" or "bf16" (latents and codec weights)
    rope_base: float = 10000.0
    scale: float = 0.0             # score scale; 0 selects 1/sqrt(d)
    d_rope: int = 0                # rotary-branch width of the decoupled (absorbed) decode
    teacher: bool = False          # an uncompressed per-loop cache (no codec)
    stream_prefill: bool = False   # a step is the layer-by-layer two-pass prefill
    paged: bool = False            # latents in shuffled 16-token pages (a block table)
    d_model: int = 0               # hidden size entering the K/V projections (fused encode)

    @property
    def Hc(self) -> int:
        return self.H if self.variant == "per_head" else 1

    @property
    def d_in(self) -> int:
        return self.d if self.variant == "per_head" else self.H * self.d

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", T=4, D=1, H=2, d=64, r_k=16, r_v=24, batch=1, n=128,
                         dtype="f32"),
    "ouro_layer_4x": Workload("ouro_layer_4x", T=4, D=1, H=16, d=128, r_k=96, r_v=160,
                              batch=32, n=4096),
    "capacity_21x": Workload("capacity_21x", T=4, D=24, H=16, d=128, r_k=16, r_v=32,
                             batch=768, n=4096),
    "encode_heavy": Workload("encode_heavy", T=4, D=1, H=16, d=128, r_k=96, r_v=160,
                             batch=8, n=8192),
    "lla2d_long": Workload("lla2d_long", T=4, D=24, H=16, d=128, r_k=96, r_v=160,
                           batch=16, n=16384, variant="2d"),
    "absorbed_4x": Workload("absorbed_4x", T=4, D=24, H=16, d=128, r_k=96, r_v=160,
                            batch=8, n=32768, d_rope=64),
    "paged_21x": Workload("paged_21x", T=4, D=24, H=16, d=128, r_k=16, r_v=32, batch=768,
                          n=4096, paged=True),
    "paged_ouro_4x": Workload("paged_ouro_4x", T=4, D=24, H=16, d=128, r_k=96, r_v=160,
                              batch=32, n=4096, paged=True),
    "paged_absorbed_4x": Workload("paged_absorbed_4x", T=4, D=24, H=16, d=128, r_k=96,
                                  r_v=160, batch=8, n=32768, d_rope=64, paged=True),
    "prefill_64k": Workload("prefill_64k", T=4, D=24, H=16, d=128, r_k=96, r_v=160, batch=1,
                            n=65536, stream_prefill=True, d_model=2048),
    "teacher_4k": Workload("teacher_4k", T=4, D=24, H=16, d=128, r_k=0, r_v=0, batch=32,
                           n=4096, teacher=True),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, std, dtype, g, device):
    """N(0, std^2) drawn in float32 then stored in ``dtype``."""
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def decode_inputs(w: Workload, seed: int, device="cpu", n_alloc: int | None = None,
                  with_q: bool = True):
    """Random latent cache, decode-side codec and queries for every layer and loop.
    ``n_alloc`` (>= w.n) sets the cache capacity n_max; rows beyond w.n are drawn
    too, so a kernel that reads past its context changes the result."""
    n_max = n_alloc or w.n
    g = _gen(seed, device)
    dt = w.torch_dtype
    out = {
        "c_k": _randn((w.D, w.batch, w.Hc, n_max, w.r_k), 1.0, dt, g, device),
        "c_v": _randn((w.D, w.batch, w.Hc, n_max, w.r_v), 1.0, dt, g, device),
        "w_up_k": _randn((w.D, w.T, w.H, w.d, w.r_k), 1.0 / math.sqrt(w.r_k), dt, g, device),
        "w_up_v": _randn((w.D, w.T, w.H, w.d, w.r_v), 1.0 / math.sqrt(w.r_v), dt, g, device),
        "mu_k": _randn((w.D, w.Hc, w.T * w.d_in), math.sqrt(0.1), dt, g, device),
        "mu_v": _randn((w.D, w.Hc, w.T * w.d_in), math.sqrt(0.1), dt, g, device),
    }
    if with_q:
        out["q"] = _randn((w.D, w.T, w.batch, w.H, w.d), 1.0, torch.float32, g, device)
    if w.d_rope > 0:  # drawn last, so the tensors above do not depend on it
        out["k_rope"] = _randn((w.D, w.batch, w.H, n_max, w.d_rope), 1.0, dt, g, device)
    return out


def paged_decode_inputs(w: Workload, seed: int, device="cpu"):
    """decode_inputs with the latents drawn straight into page pools [D][P][Hc][16][r]
    (P = batch * ceil(n / 16) pages) and a block table [batch][ceil(n / 16)] int32 that
    deals the pages out in a random order; with a rotary branch, its keys in a pool
    [D][P][H][16][d_rope] under the same table."""
    npg = (w.n + 15) // 16
    P = w.batch * npg
    g = _gen(seed, device)
    dt = w.torch_dtype
    out = {
        "c_k": _randn((w.D, P, w.Hc, 16, w.r_k), 1.0, dt, g, device),
        "c_v": _randn((w.D, P, w.Hc, 16, w.r_v), 1.0, dt, g, device),
        "w_up_k": _randn((w.D, w.T, w.H, w.d, w.r_k), 1.0 / math.sqrt(w.r_k), dt, g, device),
        "w_up_v": _randn((w.D, w.T, w.H, w.d, w.r_v), 1.0 / math.sqrt(w.r_v), dt, g, device),
        "mu_k": _randn((w.D, w.Hc, w.T * w.d_in), math.sqrt(0.1), dt, g, device),
        "mu_v": _randn((w.D, w.Hc, w.T * w.d_in), math.sqrt(0.1), dt, g, device),
        "q": _randn((w.D, w.T, w.batch, w.H, w.d), 1.0, torch.float32, g, device),
    }
    perm = torch.randperm(P, generator=g, device=device)
    out["block_table"] = perm.reshape(w.batch, npg).to(torch.int32)
    if w.d_rope > 0:  # rotary keys of the decoupled decode, paged like the latents
        out["k_rope"] = _randn((w.D, P, w.H, 16, w.d_rope), 1.0, dt, g, device)
    return out


def teacher_inputs(w: Workload, seed: int, device="cpu", n_alloc: int | None = None,
                   with_q: bool = True):
    """Random uncompressed per-loop key and value caches and queries. Drawn one layer at a
    time (each layer's float32 draw is converted to the storage dtype before the next), so a
    full-size cache needs no float32 copy of itself."""
    n_max = n_alloc or w.n
    g = _gen(seed, device)
    dt = w.torch_dtype
    shape = (w.D, w.T, w.batch, w.H, n_max, w.d)
    out = {"k_cache": torch.empty(shape, dtype=dt, device=device),
           "v_cache": torch.empty(shape, dtype=dt, device=device)}
    for name in ("k_cache", "v_cache"):
        for layer in range(w.D):
            out[name][layer].copy_(_randn(shape[1:], 1.0, dt, g, device))
    if with_q:
        out["q"] = _randn((w.D, w.T, w.batch, w.H, w.d), 1.0, torch.float32, g, device)
    return out


def orthonormal_columns(rows: int, cols: int, seed: int) -> torch.Tensor:
    """A rows x cols float64 matrix with orthonormal columns (QR of a seeded
    Gaussian, signs fixed so the R factor has a positive diagonal)."""
    g = _gen(seed, "cpu")
    a = torch.randn(rows, cols, generator=g, dtype=torch.float64)
    q, r = torch.linalg.qr(a)
    return q * torch.sign(torch.diagonal(r))[None, :]


def encode_codec_orthonormal(w: Workload, seed: int):
    """Codec whose W_down has orthonormal columns and whose W_up,t are the loop slices
    of W_down (float64, CPU). Returns dict with w_down_k [D][Hc][T*d_in][r_k] (not
    transposed), w_up_k [D][T][H][d][r_k], mu_k [D][Hc][T*d_in] and the same for v."""
    g = _gen(seed + 7919, "cpu")
    out = {}
    for ax, r in (("k", w.r_k), ("v", w.r_v)):
        wd = torch.empty(w.D, w.Hc, w.T * w.d_in, r, dtype=torch.float64)
        for l in range(w.D):
            for hc in range(w.Hc):
                wd[l, hc] = orthonormal_columns(w.T * w.d_in, r, seed * 1000 + l * 37 + hc
                                                + (0 if ax == "k" else 500))
        # loop slices: per head, rows t*d..(t+1)*d of that head's W_down; for 2D the
        # rows of (t, h) are t*H*d + h*d ..
        wu = torch.empty(w.D, w.T, w.H, w.d, r, dtype=torch.float64)
        for t in range(w.T):
            for h in range(w.H):
                if w.variant == "per_head":
                    wu[:, t, h] = wd[:, h, t * w.d:(t + 1) * w.d, :]
                else:
                    wu[:, t, h] = wd[:, 0, (t * w.H + h) * w.d:(t * w.H + h + 1) * w.d, :]
        mu = torch.randn(w.D, w.Hc, w.T * w.d_in, generator=g, dtype=torch.float64) \
            * math.sqrt(0.1)
        out["w_down_" + ax] = wd
        out["w_up_" + ax] = wu
        out["mu_" + ax] = mu
    return out


def encode_x(w: Workload, n_new: int, seed: int, device="cpu", correlated: bool = False,
             batch: int | None = None):
    """Pre-RoPE per-loop keys and values to encode, [B][n_new][Hc][T][d_in] in the
    workload dtype. ``correlated``: x_1 ~ N(0, I) and x_t = x_1 + 0.3 * t * eps_t for
    t = 2..T with eps_t ~ N(0, I) (the loop-correlated recipe); else iid N(0, 1)."""
    B = batch or w.batch
    g = _gen(seed, device)
    out = []
    for _ in range(2):
        x = torch.randn(B, n_new, w.Hc, w.T, w.d_in, generator=g, device=device,
                        dtype=torch.float32)
        if correlated:
            eps = torch.randn(B, n_new, w.Hc, w.T, w.d_in, generator=g, device=device,
                              dtype=torch.float32)
            for t in range(1, w.T):
                x[:, :, :, t] = x[:, :, :, 0] + 0.3 * (t + 1) * eps[:, :, :, t]
        out.append(x.to(w.torch_dtype))
    return out[0], out[1]


def fused_encode_inputs(w: Workload, n_new: int, d_model: int, seed: int, device="cpu",
                        batch: int | None = None):
    """Inputs of the projection-fused encode, in the workload dtype: the hidden states
    that enter a layer's key and value projections at each loop, h [T][B][n_new][d_model]
    ~ N(0, 1), and the projections of every layer as linear-layer weights (output
    features x input features), w_k and w_v [D][H*d][d_model] ~ N(0, 1/d_model) (so the
    per-loop keys and values have about unit variance, like the per-loop K/V drawn by
    encode_x)."""
    B = batch or w.batch
    g = _gen(seed, device)
    dt = w.torch_dtype
    h = _randn((w.T, B, n_new, d_model), 1.0, dt, g, device)
    w_k = _randn((w.D, w.H * w.d, d_model), 1.0 / math.sqrt(d_model), dt, g, device)
    w_v = _randn((w.D, w.H * w.d, d_model), 1.0 / math.sqrt(d_model), dt, g, device)
    return h, w_k, w_v


def gaussian_encode_codec(w: Workload, seed: int, device="cpu"):
    """Encode-side codec with W_down ~ N(0, 1/K) (K = T*d_in), stored transposed
    [D][Hc][r][K], and mu ~ N(0, 0.1) [D][Hc][K], in the workload dtype."""
    g = _gen(seed, device)
    dt = w.torch_dtype
    K = w.T * w.d_in
    return {
        "w_down_k_t": _randn((w.D, w.Hc, w.r_k, K), 1.0 / math.sqrt(K), dt, g, device),
        "w_down_v_t": _randn((w.D, w.Hc, w.r_v, K), 1.0 / math.sqrt(K), dt, g, device),
        "mu_k": _randn((w.D, w.Hc, K), math.sqrt(0.1), dt, g, device),
        "mu_v": _randn((w.D, w.Hc, K), math.sqrt(0.1), dt, g, device),
    }
