"""The oracle against its pins, and a mutation check: a plausible mistake planted in
the oracle (on the CPU) must move at least one pin past its tolerance."""

import numpy as np
import pytest

from oracle import lla_oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("name", list(P.ALL_PINS))
def test_pin(name):
    fn, tol = P.ALL_PINS[name]
    err = fn()
    assert err <= tol, f"pin {name}: deviation {err} > {tol}"


def _mut_rope_sign(x, positions, base):
    return _ORIG["apply_rope"](x, -np.asarray(positions), base)


def _mut_rope_halfsplit(x, positions, base):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    phi = np.asarray(positions, dtype=np.float64)[:, None] * O.rope_theta(d, base)[None, :]
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def _mut_theta(d, base):
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(base), -i / d)


def _mut_recon_no_mu(c, w_up_t, mu_t):
    return np.asarray(c, dtype=np.float64) @ np.asarray(w_up_t, dtype=np.float64).T


def _mut_recon_transposed_pairs(c, w_up_t, mu_t):
    out = _ORIG["reconstruct"](c, w_up_t, mu_t)
    d = out.shape[-1]
    return out.reshape(*out.shape[:-1], d // 2, 2)[..., ::-1].reshape(out.shape)


def _mut_encode_no_center(x, mu, w_down):
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_down, dtype=np.float64)


def _mut_attention_no_scale(q, k, v, scale):
    return _ORIG["attention"](q, k, v, 1.0)


def _mut_attention_softmax_over_wrong_axis(q, k, v, scale):
    if k.shape[0] == 0:
        return np.zeros(v.shape[-1])
    s = scale * (k @ q)
    a = np.exp(s) / np.exp(s).sum() if s.size < 2 else np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    return a[::-1] @ v


def _mut_attention_no_max_shift(q, k, v, scale):
    """Softmax without subtracting the largest score: overflows for large scores."""
    if k.shape[0] == 0:
        return np.zeros(v.shape[-1])
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(scale * (k @ q))
        return (e / e.sum()) @ v


def _mut_mu_slice_2d_head_major(mu, variant, t, h, H, d):
    if variant == "per_head":
        return mu[h, t * d:(t + 1) * d]
    T = mu.shape[1] // (H * d)
    return mu[0, (h * T + t) * d:(h * T + t + 1) * d]


def _mut_mu_slice_wrong_loop(mu, variant, t, h, H, d):
    T = mu.shape[1] // (d if variant == "per_head" else H * d)
    return _ORIG["_mu_slice"](mu, variant, (t + 1) % T, h, H, d)


def _mut_svd_no_center(x, r, T, d):
    x = np.asarray(x, dtype=np.float64)
    _, _, vh = np.linalg.svd(x, full_matrices=False)
    w = vh[:r].T.copy()
    return x.mean(axis=0), w, np.stack([w[t * d:(t + 1) * d] for t in range(T)])


def _mut_ratio_no_two(T, d_head, r_k, r_v, H=1, variant="per_head"):
    return T * d_head / (r_k + r_v)


def _mut_round_truncate(x):
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.trunc(m * 256.0), e - 8)


def _mut_absorbed_rotary_last(k_rope, k_hat, d_rope):
    n, d = k_hat.shape
    return np.concatenate([k_hat[:, :d - d_rope],
                           np.asarray(k_rope, dtype=np.float64).reshape(n, d_rope)], axis=1)


def _mut_absorbed_drops_rotary(k_rope, k_hat, d_rope):
    return np.concatenate([np.zeros((k_hat.shape[0], d_rope)), k_hat[:, d_rope:]], axis=1)


def _mut_absorbed_content_rotated(k_rope, k_hat, d_rope):
    return _ORIG["absorbed_keys"](k_rope, O.apply_rope(k_hat, np.arange(k_hat.shape[0]), 10000.0),
                                  d_rope)


def _mut_absorbed_scale_content_only(d, d_rope):
    return 1.0 / np.sqrt(max(d - d_rope, 1))


def _mut_teacher_next_loop(cache, t, b, h, nb):
    return np.asarray(cache[(t + 1) % cache.shape[0], b, h, :nb], dtype=np.float64)


def _mut_reconstruct_cache_positions_from_zero(c_k, c_v, w_up_k, mu_k, w_up_v, mu_v, loop_begin,
                                               loop_count, pos_start, n_tok, rope_base=10000.0,
                                               variant="per_head"):
    """Rotates the rebuilt keys as if the range started at slot 0."""
    k, v = _ORIG["reconstruct_cache"](c_k, c_v, w_up_k, mu_k, w_up_v, mu_v, loop_begin,
                                      loop_count, pos_start, n_tok, rope_base, variant)
    d = k.shape[-1]
    phi = pos_start * O.rope_theta(d, rope_base)
    back = np.empty_like(k)  # rotate every pair back by pos_start * theta
    back[..., 0::2] = k[..., 0::2] * np.cos(phi) + k[..., 1::2] * np.sin(phi)
    back[..., 1::2] = -k[..., 0::2] * np.sin(phi) + k[..., 1::2] * np.cos(phi)
    return back, v


def _mut_reconstruct_cache_rotates_values(c_k, c_v, w_up_k, mu_k, w_up_v, mu_v, loop_begin,
                                          loop_count, pos_start, n_tok, rope_base=10000.0,
                                          variant="per_head"):
    k, v = _ORIG["reconstruct_cache"](c_k, c_v, w_up_k, mu_k, w_up_v, mu_v, loop_begin,
                                      loop_count, pos_start, n_tok, rope_base, variant)
    return k, O.apply_rope(v, np.arange(pos_start, pos_start + n_tok), rope_base)


def _mut_gather_pages_next_page(pool, block_table, n):
    """Reads page j // PAGE + 1 of the table (wrapping)."""
    pool = np.asarray(pool)
    bt = np.asarray(block_table)
    out = np.zeros((bt.shape[0], pool.shape[1], n, pool.shape[3]))
    for b in range(bt.shape[0]):
        for j in range(n):
            out[b, :, j] = pool[int(bt[b][(j // O.PAGE + 1) % bt.shape[1]]), :, j % O.PAGE]
    return out


def _mut_absorbed_paged_rope_unrouted(pool_k, pool_v, pool_rope, block_table, w_up_k, mu_k,
                                      w_up_v, mu_v, q, d_rope, loop_begin=0, ctx_lens=None,
                                      n_ctx=None, scale=None, variant="per_head"):
    """Takes the rotary keys from pages in logical order, bypassing the block table."""
    bt = np.asarray(block_table)
    if n_ctx is None:
        n_ctx = bt.shape[1] * O.PAGE
    ident = np.arange(bt.size).reshape(bt.shape)
    c_k = O.gather_pages(pool_k, bt, n_ctx)
    c_v = O.gather_pages(pool_v, bt, n_ctx)
    k_rope = O.gather_pages(pool_rope, ident, n_ctx)
    return O.decode_absorbed(c_k, c_v, k_rope, w_up_k, mu_k, w_up_v, mu_v, q, d_rope, loop_begin,
                             ctx_lens, scale, variant)


def _mut_window_keeps_oldest(n_pages_written, sink_pages, window_pages):
    if n_pages_written <= sink_pages + window_pages:
        return list(range(n_pages_written))
    return list(range(sink_pages + window_pages))


def _mut_fused_loops_reversed(h_loops, w_proj, mu, w_down, H, d, variant="per_head"):
    """Stacks the loops in reverse order."""
    return _ORIG["encode_fused"](np.asarray(h_loops)[::-1], w_proj, mu, w_down, H, d, variant)


def _mut_fused_next_head(h_loops, w_proj, mu, w_down, H, d, variant="per_head"):
    """Takes each head's keys from the next head's projection columns."""
    w = np.roll(np.asarray(w_proj), -d, axis=1)
    return _ORIG["encode_fused"](h_loops, w, mu, w_down, H, d, variant)


def _mut_fused_no_centering(h_loops, w_proj, mu, w_down, H, d, variant="per_head"):
    return _ORIG["encode_fused"](h_loops, w_proj, np.zeros_like(mu), w_down, H, d, variant)


_ORIG = {name: getattr(O, name) for name in
         ("apply_rope", "reconstruct", "attention", "_mu_slice", "rope_theta", "absorbed_keys",
          "reconstruct_cache", "encode_fused")}

MUTANTS = {
    "rope_sign": ("apply_rope", _mut_rope_sign),
    "rope_halfsplit": ("apply_rope", _mut_rope_halfsplit),
    "rope_theta_exponent": ("rope_theta", _mut_theta),
    "reconstruct_drops_mu": ("reconstruct", _mut_recon_no_mu),
    "reconstruct_swaps_pair": ("reconstruct", _mut_recon_transposed_pairs),
    "encode_no_centering": ("encode", _mut_encode_no_center),
    "attention_no_scale": ("attention", _mut_attention_no_scale),
    "attention_reversed_weights": ("attention", _mut_attention_softmax_over_wrong_axis),
    "attention_no_max_shift": ("attention", _mut_attention_no_max_shift),
    "mu_2d_head_major": ("_mu_slice", _mut_mu_slice_2d_head_major),
    "mu_wrong_loop": ("_mu_slice", _mut_mu_slice_wrong_loop),
    "svd_no_centering": ("svd_init", _mut_svd_no_center),
    "rho_missing_factor_two": ("compression_ratio", _mut_ratio_no_two),
    "bf16_truncates": ("round_bf16", _mut_round_truncate),
    "absorbed_rotary_last": ("absorbed_keys", _mut_absorbed_rotary_last),
    "absorbed_drops_rotary": ("absorbed_keys", _mut_absorbed_drops_rotary),
    "absorbed_content_rotated": ("absorbed_keys", _mut_absorbed_content_rotated),
    "absorbed_scale_content_only": ("absorbed_scale", _mut_absorbed_scale_content_only),
    "teacher_next_loop": ("teacher_rows", _mut_teacher_next_loop),
    "reconstruct_cache_positions_from_zero": ("reconstruct_cache", _mut_reconstruct_cache_positions_from_zero),
    "reconstruct_cache_rotates_values": ("reconstruct_cache", _mut_reconstruct_cache_rotates_values),
    "gather_pages_next_page": ("gather_pages", _mut_gather_pages_next_page),
    "window_keeps_oldest": ("window_pages", _mut_window_keeps_oldest),
    "absorbed_paged_rope_unrouted": ("decode_absorbed_paged", _mut_absorbed_paged_rope_unrouted),
    "fused_loops_reversed": ("encode_fused", _mut_fused_loops_reversed),
    "fused_next_head": ("encode_fused", _mut_fused_next_head),
    "fused_no_centering": ("encode_fused", _mut_fused_no_centering),
}


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_planted_mistake_is_caught(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for name, (pin, tol) in P.ALL_PINS.items():
        try:
            err = pin()
        except Exception:  # a crash also counts as caught
            err = float("inf")
        if not err <= tol:
            caught.append(name)
    assert caught, f"mutant {mutant} passed every pin"
