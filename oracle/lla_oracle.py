"""fp64 CPU oracle for the Looped Latent Attention (LLA) latent-store decode path.

TEST INFRASTRUCTURE ONLY. This module is the slow, plainly written definition that
the HIP path is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. It shares no code with the HIP
path and imports nothing from ``latent_decode_attention_lla_amd``.

Source: "Looped Latent Attention: Cross-Loop KV Compression for Looped Transformers"
(arXiv 2607.15456v2), Section 3 (Eqs. 1-4, "RoPE and reconstruction", "The LLA-2D
variant", "Initialization and conversion"), Section 7 and Appendix J.

Everything is computed in float64 with nothing factored: the keys and values of every
cached token are rebuilt explicitly, RoPE is applied to the rebuilt keys, and textbook
softmax attention follows. Readings taken where the pages are silent:

* RoPE pairs are interleaved, (2i, 2i+1), rotated counter-clockwise by p*theta_i with
  theta_i = base**(-2i/d) (RoFormer, which the LLA paper cites for RoPE).
* A cached token's position is its slot index j in [0, n).
* Queries arrive already rotated (the model rotates q as usual); only keys rebuilt
  from latents are rotated here.
* Score scale defaults to 1/sqrt(d_head).
* Attention over an empty context returns zeros.
* LLA-2D stacks its input (t, h, d) with the loop index outermost.
* Projection-fused encode (Appendix J, "Eviction and long-context prefill"; Eq. 2): the
  keys (values) of loop t are x_t = h_t W_proj with the layer's projection shared by
  every loop, taken exactly (the fused path never stores x_t, so it is not rounded).
* Decoupled (absorbed) decode, Appendix J: dimensions 0 .. d_rope-1 of a head are the
  rotary branch (one stored, already rotated key per token, shared by every loop), the
  rest the content path (the loop's reconstructed key without RoPE); scale 1/sqrt(d).

Parity: every function here is pinned by ``tests/test_oracle_pins.py`` (closed forms
printed on the pages, the full-rank special case against textbook attention, RoPE
invariants, softmax special cases, a scalar brute-force re-derivation, the LLA-2D
block-diagonal reduction and the Eckart-Young property of the SVD initialisation;
the decoupled decode against textbook attention on the original keys and values, a
scalar brute force, and its reduction to the full-RoPE decode; the uncompressed decode
against textbook attention and against the latent decode of the same cache; the
materialised reconstruction by a full-rank round trip, a scalar brute force and by
feeding the uncompressed decode; the paged cache by identity and permuted block tables,
and eviction by textbook attention over the kept keys at their new positions).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "compression_ratio",
    "teacher_scalars_per_token_layer",
    "latent_scalars_per_token_layer",
    "cache_bytes_per_token",
    "stack_loops",
    "encode",
    "reconstruct",
    "rope_theta",
    "apply_rope",
    "softmax",
    "attention",
    "decode",
    "absorbed_scale",
    "absorbed_keys",
    "decode_absorbed",
    "teacher_rows",
    "decode_teacher",
    "reconstruct_cache",
    "PAGE",
    "gather_pages",
    "decode_paged",
    "window_pages",
    "svd_init",
    "round_bf16",
    "encode_stored",
    "encode_fused",
]


# ---------------------------------------------------------------------------
# Closed forms: Section 3, Eq. 4 and the paragraph before it; Section 7, Table 5.
# ---------------------------------------------------------------------------

def teacher_scalars_per_token_layer(T: int, H: int, d_head: int) -> int:
    """Uncompressed loop-indexed cache: K and V for every loop and head (Section 3,
    "Teacher cache")."""
    return 2 * T * H * d_head


def latent_scalars_per_token_layer(H: int, r_k: int, r_v: int, variant: str = "per_head") -> int:
    """Latent cache: (r_k + r_v) per head (Section 3, "Cross-loop codec"), or one
    shared latent of r_k + r_v for LLA-2D (Section 3, "The LLA-2D variant")."""
    if variant == "per_head":
        return (r_k + r_v) * H
    if variant == "2d":
        return r_k + r_v
    raise ValueError(variant)


def compression_ratio(T: int, d_head: int, r_k: int, r_v: int, H: int = 1,
                      variant: str = "per_head") -> float:
    """rho = teacher scalars / latent scalars (Section 3, Eq. 4). For the per-head
    codec H cancels and rho = 2 T d_head / (r_k + r_v)."""
    return (teacher_scalars_per_token_layer(T, H, d_head)
            / latent_scalars_per_token_layer(H, r_k, r_v, variant))


def cache_bytes_per_token(D: int, H: int, r_k: int, r_v: int, bytes_per_scalar: int,
                          variant: str = "per_head") -> int:
    """Bytes one token occupies across all D layers (Section 7, Table 5 row
    "KV / token")."""
    return D * latent_scalars_per_token_layer(H, r_k, r_v, variant) * bytes_per_scalar


# ---------------------------------------------------------------------------
# Codec: Section 3, Eqs. 1-3.
# ---------------------------------------------------------------------------

def stack_loops(x_loops: np.ndarray) -> np.ndarray:
    """Eq. 1: stack the T per-loop vectors [..., T, d] into x = [x_1; ...; x_T]
    of length T*d, loop index outermost."""
    x_loops = np.asarray(x_loops, dtype=np.float64)
    return x_loops.reshape(*x_loops.shape[:-2], x_loops.shape[-2] * x_loops.shape[-1])


def encode(x: np.ndarray, mu: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """Eq. 2: c = (x - mu) W_down. x: [..., T*d], mu: [T*d], W_down: [T*d, r]."""
    x = np.asarray(x, dtype=np.float64)
    return (x - np.asarray(mu, dtype=np.float64)) @ np.asarray(w_down, dtype=np.float64)


def reconstruct(c: np.ndarray, w_up_t: np.ndarray, mu_t: np.ndarray) -> np.ndarray:
    """Eq. 3: x_hat_t = c W_up,t^T + mu_t (row-vector convention). c: [..., r],
    W_up,t: [d, r], mu_t: [d]."""
    c = np.asarray(c, dtype=np.float64)
    return c @ np.asarray(w_up_t, dtype=np.float64).T + np.asarray(mu_t, dtype=np.float64)


# ---------------------------------------------------------------------------
# RoPE after reconstruction: Section 3, "RoPE and reconstruction".
# ---------------------------------------------------------------------------

def rope_theta(d: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d), i = 0 .. d/2-1 (RoFormer frequencies)."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / d)


def apply_rope(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotate each interleaved pair (x_2i, x_2i+1) of x [..., n, d] by angle
    p * theta_i, p = positions[n]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    phi = np.asarray(positions, dtype=np.float64)[:, None] * rope_theta(d, base)[None, :]
    cos, sin = np.cos(phi), np.sin(phi)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * cos - x1 * sin
    y[..., 1::2] = x0 * sin + x1 * cos
    return y


# ---------------------------------------------------------------------------
# Attention itself is unchanged by LLA (Section 3, Figure 1 caption).
# ---------------------------------------------------------------------------

def softmax(s: np.ndarray) -> np.ndarray:
    """Two-pass softmax over the last axis."""
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Textbook single-query attention: q [d], k [n, d], v [n, d_v] -> [d_v].
    An empty context (n == 0) returns zeros."""
    if k.shape[0] == 0:
        return np.zeros(v.shape[-1], dtype=np.float64)
    a = softmax(scale * (k @ q))
    return a @ v


# ---------------------------------------------------------------------------
# Latent-store decode: Section 7 ("caches only the latent and reconstructs on read")
# with the codec of Eqs. 2-3, RoPE after reconstruction, and LLA-2D.
# ---------------------------------------------------------------------------

def _mu_slice(mu: np.ndarray, variant: str, t: int, h: int, H: int, d: int) -> np.ndarray:
    """mu_t for one head. Per-head: mu[h] has length T*d, loop t is its t-th block.
    LLA-2D: mu[0] has length T*H*d stacked (t, h, d)."""
    if variant == "per_head":
        return mu[h, t * d:(t + 1) * d]
    return mu[0, (t * H + h) * d:(t * H + h + 1) * d]


def decode(c_k: np.ndarray, c_v: np.ndarray,
           w_up_k: np.ndarray, mu_k: np.ndarray,
           w_up_v: np.ndarray, mu_v: np.ndarray,
           q: np.ndarray, loop_begin: int = 0,
           ctx_lens=None, rope_base: float = 10000.0, scale: float | None = None,
           variant: str = "per_head") -> np.ndarray:
    """Decode attention for one layer over the latent cache.

    c_k [B, Hc, n, r_k], c_v [B, Hc, n, r_v] : cached latents (Hc = H per head, 1 for 2D)
    w_up_k [T, H, d, r_k], w_up_v [T, H, d, r_v] : loop-specific up-projections
    mu_k, mu_v [Hc, T*d] (per head) or [1, T*H*d] (2D) : calibration means
    q [B, H, L, d] : post-RoPE queries for loops loop_begin .. loop_begin+L-1
    ctx_lens [B] or None : tokens 0 .. ctx_lens[b]-1 are attended (default all n)
    returns out [B, H, L, d] float64
    """
    c_k = np.asarray(c_k)
    c_v = np.asarray(c_v)
    B, Hc, n, _ = c_k.shape
    L = q.shape[2]
    H = q.shape[1]
    d = q.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if ctx_lens is None:
        ctx_lens = [n] * B
    out = np.zeros((B, H, L, d), dtype=np.float64)
    for b in range(B):
        nb = int(ctx_lens[b])
        pos = np.arange(nb)
        for h in range(H):
            hc = h if variant == "per_head" else 0
            ck = np.asarray(c_k[b, hc, :nb], dtype=np.float64)
            cv = np.asarray(c_v[b, hc, :nb], dtype=np.float64)
            for li in range(L):
                t = loop_begin + li
                k_hat = reconstruct(ck, w_up_k[t, h], _mu_slice(mu_k, variant, t, h, H, d))
                v_hat = reconstruct(cv, w_up_v[t, h], _mu_slice(mu_v, variant, t, h, H, d))
                k_rot = apply_rope(k_hat, pos, rope_base)
                out[b, h, li] = attention(np.asarray(q[b, h, li], dtype=np.float64),
                                          k_rot, v_hat, scale)
    return out


# ---------------------------------------------------------------------------
# Absorbed decode with a decoupled rotary branch: Appendix J, "Absorbed attention"
# (an MLA-style content path without RoPE plus a small explicit rotary branch that every
# loop of a token shares). The pages give no formulas for the split; the reading taken
# here: the first d_rope dimensions of every head are the rotary branch, whose key is
# stored per (sequence, head, token) already rotated to the token's position; the other
# d - d_rope dimensions are the content path, whose key is the loop-t reconstruction
# (Eq. 3) without RoPE. The score scale stays 1/sqrt(d).
# ---------------------------------------------------------------------------

def absorbed_scale(d: int, d_rope: int) -> float:
    """Default score scale of the decoupled decode: 1/sqrt(d) of the whole head."""
    return 1.0 / math.sqrt(d)


def absorbed_keys(k_rope: np.ndarray, k_hat: np.ndarray, d_rope: int) -> np.ndarray:
    """Key rows of the decoupled decode: rotary branch in dimensions 0 .. d_rope-1,
    content (the reconstructed key, no RoPE) in d_rope .. d-1. k_rope [n, d_rope],
    k_hat [n, d] -> [n, d]."""
    return np.concatenate([np.asarray(k_rope, dtype=np.float64).reshape(k_hat.shape[0], d_rope),
                           k_hat[:, d_rope:]], axis=1)


def decode_absorbed(c_k: np.ndarray, c_v: np.ndarray, k_rope: np.ndarray,
                    w_up_k: np.ndarray, mu_k: np.ndarray,
                    w_up_v: np.ndarray, mu_v: np.ndarray,
                    q: np.ndarray, d_rope: int, loop_begin: int = 0,
                    ctx_lens=None, scale: float | None = None,
                    variant: str = "per_head") -> np.ndarray:
    """Decode attention for one layer with the decoupled key, written out explicitly:
    keys [k_rope ; K_t content], values V_t, both reconstructed per token (Eq. 3).

    k_rope [B, H, n, d_rope] : rotary keys, rotated to their positions, one per token
                               for all loops
    q [B, H, L, d]           : queries; entries 0 .. d_rope-1 are the rotated rotary part
    other arguments as in `decode`; returns out [B, H, L, d] float64
    """
    c_k = np.asarray(c_k)
    c_v = np.asarray(c_v)
    B, Hc, n, _ = c_k.shape
    L = q.shape[2]
    H = q.shape[1]
    d = q.shape[3]
    if scale is None:
        scale = absorbed_scale(d, d_rope)
    if ctx_lens is None:
        ctx_lens = [n] * B
    out = np.zeros((B, H, L, d), dtype=np.float64)
    for b in range(B):
        nb = int(ctx_lens[b])
        for h in range(H):
            hc = h if variant == "per_head" else 0
            ck = np.asarray(c_k[b, hc, :nb], dtype=np.float64)
            cv = np.asarray(c_v[b, hc, :nb], dtype=np.float64)
            kr = np.asarray(k_rope[b, h, :nb], dtype=np.float64)
            for li in range(L):
                t = loop_begin + li
                k_hat = reconstruct(ck, w_up_k[t, h], _mu_slice(mu_k, variant, t, h, H, d))
                v_hat = reconstruct(cv, w_up_v[t, h], _mu_slice(mu_v, variant, t, h, H, d))
                out[b, h, li] = attention(np.asarray(q[b, h, li], dtype=np.float64),
                                          absorbed_keys(kr, k_hat, d_rope), v_hat, scale)
    return out


# ---------------------------------------------------------------------------
# Uncompressed decode: the teacher's loop-indexed cache (Section 3, "Problem setup":
# every loop t keeps its own keys and values; Section 7, Table 5's "teacher" column).
# ---------------------------------------------------------------------------

def teacher_rows(cache: np.ndarray, t: int, b: int, h: int, nb: int) -> np.ndarray:
    """The first nb cached rows of loop t, sequence b, head h: [nb, d] float64."""
    return np.asarray(cache[t, b, h, :nb], dtype=np.float64)


def decode_teacher(k_cache: np.ndarray, v_cache: np.ndarray, q: np.ndarray,
                   loop_begin: int = 0, ctx_lens=None, scale: float | None = None) -> np.ndarray:
    """Decode attention over the uncompressed per-loop cache.

    k_cache [T, B, H, n, d] : keys of every loop, already rotated to their positions
    v_cache [T, B, H, n, d] : values of every loop
    q [B, H, L, d]          : rotated queries for loops loop_begin .. loop_begin+L-1
    returns out [B, H, L, d] float64 (zeros for an empty context)
    """
    T, B, H, n, d = k_cache.shape
    L = q.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if ctx_lens is None:
        ctx_lens = [n] * B
    out = np.zeros((B, H, L, d), dtype=np.float64)
    for b in range(B):
        nb = int(ctx_lens[b])
        for h in range(H):
            for li in range(L):
                t = loop_begin + li
                out[b, h, li] = attention(np.asarray(q[b, h, li], dtype=np.float64),
                                          teacher_rows(k_cache, t, b, h, nb),
                                          teacher_rows(v_cache, t, b, h, nb), scale)
    return out


# ---------------------------------------------------------------------------
# Materialised reconstruction for the streamed two-pass prefill: Appendix A, "Decoding
# and caching" (pass 2 re-forwards with the codec's reconstruction, which the latent-
# store decoder streams layer by layer) and Appendix J, "Eviction and long-context
# prefill" (one layer's K/V rebuilt and freed at a time). Eq. 3 for every token of a
# range, then RoPE on the keys at the slot index (Section 3, "RoPE and reconstruction").
# ---------------------------------------------------------------------------

def reconstruct_cache(c_k: np.ndarray, c_v: np.ndarray,
                      w_up_k: np.ndarray, mu_k: np.ndarray,
                      w_up_v: np.ndarray, mu_v: np.ndarray,
                      loop_begin: int, loop_count: int, pos_start: int, n_tok: int,
                      rope_base: float = 10000.0, variant: str = "per_head"):
    """Keys and values of loops loop_begin .. loop_begin+loop_count-1 for the tokens in
    slots pos_start .. pos_start+n_tok-1 of one layer's latent cache.

    c_k [B, Hc, n, r_k], c_v [B, Hc, n, r_v]; w_up_* [T, H, d, r]; mu_* as in decode.
    returns (k [L, B, H, n_tok, d], v [L, B, H, n_tok, d]) float64: k rotated by RoPE at
    its slot index, v as rebuilt.
    """
    B = c_k.shape[0]
    _, H, d, _ = np.asarray(w_up_k).shape
    pos = np.arange(pos_start, pos_start + n_tok)
    k = np.zeros((loop_count, B, H, n_tok, d), dtype=np.float64)
    v = np.zeros((loop_count, B, H, n_tok, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            hc = h if variant == "per_head" else 0
            ck = np.asarray(c_k[b, hc, pos_start:pos_start + n_tok], dtype=np.float64)
            cv = np.asarray(c_v[b, hc, pos_start:pos_start + n_tok], dtype=np.float64)
            for li in range(loop_count):
                t = loop_begin + li
                k_hat = reconstruct(ck, w_up_k[t, h], _mu_slice(mu_k, variant, t, h, H, d))
                k[li, b, h] = apply_rope(k_hat, pos, rope_base)
                v[li, b, h] = reconstruct(cv, w_up_v[t, h], _mu_slice(mu_v, variant, t, h, H, d))
    return k, v


# ---------------------------------------------------------------------------
# Paged latent cache with token eviction: Appendix D (Table 9, StreamingLLM/H2O-style
# eviction to a sink plus a recent window) and Appendix J, "Eviction and long-context
# prefill" (the sequence axis composes with the loop axis; a 1024-token budget caps the
# 1M-context cache). Readings: the cache is stored in pages of PAGE tokens listed per
# sequence by a block table in logical order; what eviction keeps is the sink pages plus
# the most recent pages; positions for RoPE are the logical slots of the kept cache (the
# StreamingLLM convention, free here because latents are stored before RoPE).
# ---------------------------------------------------------------------------

PAGE = 16


def gather_pages(pool: np.ndarray, block_table: np.ndarray, n: int) -> np.ndarray:
    """Logical latent rows of every sequence: token j of sequence b is row j % PAGE of
    page block_table[b][j // PAGE]. pool [P, Hc, PAGE, r] -> [B, Hc, n, r] float64."""
    pool = np.asarray(pool)
    block_table = np.asarray(block_table)
    B = block_table.shape[0]
    Hc, r = pool.shape[1], pool.shape[3]
    out = np.zeros((B, Hc, n, r), dtype=np.float64)
    for b in range(B):
        for j in range(n):
            out[b, :, j] = pool[int(block_table[b][j // PAGE]), :, j % PAGE]
    return out


def decode_paged(pool_k: np.ndarray, pool_v: np.ndarray, block_table: np.ndarray,
                 w_up_k: np.ndarray, mu_k: np.ndarray, w_up_v: np.ndarray, mu_v: np.ndarray,
                 q: np.ndarray, loop_begin: int = 0, ctx_lens=None, n_ctx: int | None = None,
                 rope_base: float = 10000.0, scale: float | None = None,
                 variant: str = "per_head") -> np.ndarray:
    """Decode attention over a paged latent cache: the latent decode of the logical rows
    the block table lists (RoPE at the logical slot)."""
    if n_ctx is None:
        n_ctx = np.asarray(block_table).shape[1] * PAGE
    c_k = gather_pages(pool_k, block_table, n_ctx)
    c_v = gather_pages(pool_v, block_table, n_ctx)
    return decode(c_k, c_v, w_up_k, mu_k, w_up_v, mu_v, q, loop_begin, ctx_lens, rope_base,
                  scale, variant)


def decode_absorbed_paged(pool_k: np.ndarray, pool_v: np.ndarray, pool_rope: np.ndarray,
                          block_table: np.ndarray, w_up_k: np.ndarray, mu_k: np.ndarray,
                          w_up_v: np.ndarray, mu_v: np.ndarray, q: np.ndarray, d_rope: int,
                          loop_begin: int = 0, ctx_lens=None, n_ctx: int | None = None,
                          scale: float | None = None, variant: str = "per_head") -> np.ndarray:
    """Decoupled-RoPE decode over a paged cache: the latent rows and the rotary keys
    (pool_rope [P, H, PAGE, d_rope]) of the logical tokens the block table lists, then the
    decode of `decode_absorbed`."""
    if n_ctx is None:
        n_ctx = np.asarray(block_table).shape[1] * PAGE
    c_k = gather_pages(pool_k, block_table, n_ctx)
    c_v = gather_pages(pool_v, block_table, n_ctx)
    k_rope = gather_pages(pool_rope, block_table, n_ctx)
    return decode_absorbed(c_k, c_v, k_rope, w_up_k, mu_k, w_up_v, mu_v, q, d_rope, loop_begin,
                           ctx_lens, scale, variant)


def window_pages(n_pages_written: int, sink_pages: int, window_pages: int) -> list:
    """Logical pages eviction keeps once n_pages_written pages exist: the first sink_pages
    pages and the window_pages most recent ones, in order (all of them while they fit)."""
    if n_pages_written <= sink_pages + window_pages:
        return list(range(n_pages_written))
    return list(range(sink_pages)) + list(range(n_pages_written - window_pages, n_pages_written))


# ---------------------------------------------------------------------------
# SVD initialisation: Section 3, "Initialization and conversion"; Appendix A.
# ---------------------------------------------------------------------------

def svd_init(x: np.ndarray, r: int, T: int, d: int):
    """Codec from calibration activations x [N, T*d] (stacked loops, pre-RoPE):
    centre by the per-loop mean, take the top-r right singular vectors of the centred
    stacked-loop matrix as W_down [T*d, r]; the initial W_up,t are its loop slices
    [d, r]. Returns (mu [T*d], W_down, W_up [T, d, r])."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=0)
    _, _, vh = np.linalg.svd(x - mu, full_matrices=False)
    w_down = vh[:r].T.copy()
    w_up = np.stack([w_down[t * d:(t + 1) * d, :] for t in range(T)])
    return mu, w_down, w_up


# ---------------------------------------------------------------------------
# Storage rounding (latents are stored in the cache dtype).
# ---------------------------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits), ties to
    even, returned as float64. Normal range only (no overflow or bf16 subnormals are
    generated by the tests)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def encode_stored(x: np.ndarray, mu: np.ndarray, w_down: np.ndarray, dtype: str) -> np.ndarray:
    """Eq. 2 followed by rounding to the storage dtype ("f32" or "bf16"), both from
    the exact fp64 value."""
    c = encode(x, mu, w_down)
    if dtype == "bf16":
        return round_bf16(c)
    if dtype == "f32":
        return c.astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Projection-fused encode: Appendix J, "Eviction and long-context prefill" (stream the
# prefill so that no layer holds its per-loop keys and values longer than needed);
# Section 3, Eqs. 1-2.
# ---------------------------------------------------------------------------

def encode_fused(h_loops: np.ndarray, w_proj: np.ndarray, mu: np.ndarray, w_down: np.ndarray,
                 H: int, d: int, variant: str = "per_head") -> np.ndarray:
    """Latents of N tokens from the hidden states that enter one layer's key (or value)
    projection at each loop: x_t = h_t W_proj for t = 1 .. T (one projection shared by
    every loop of the looped layer), the per-loop vectors stacked as in Eq. 1, then Eq. 2.

    h_loops [T, N, d_model]; w_proj [d_model, H*d] (head h owns columns h*d .. h*d+d-1);
    mu [Hc, T*d_in]; w_down [Hc, T*d_in, r] (Hc = H, d_in = d per head; Hc = 1, d_in = H*d
    for LLA-2D, stacked (t, h, d)). Returns c [N, Hc, r] float64, unrounded."""
    h_loops = np.asarray(h_loops, dtype=np.float64)
    T, N, _ = h_loops.shape
    x = np.stack([h_loops[t] @ np.asarray(w_proj, dtype=np.float64) for t in range(T)])  # [T, N, H*d]
    Hc = mu.shape[0]
    out = np.empty((N, Hc, w_down.shape[-1]))
    for hc in range(Hc):
        if variant == "per_head":
            xs = stack_loops(np.transpose(x[:, :, hc * d:(hc + 1) * d], (1, 0, 2)))  # [N, T*d]
        else:
            xs = stack_loops(np.transpose(x, (1, 0, 2)))  # [N, T*H*d], (t, h, d)
        out[:, hc] = encode(xs, mu[hc], w_down[hc])
    return out

