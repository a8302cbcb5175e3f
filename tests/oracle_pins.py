"""Pins for the fp64 oracle: each check ties ``oracle/lla_oracle.py`` to something other
than itself (values printed on the pages, closed forms, a textbook routine, invariants,
a scalar brute force). Each returns the largest deviation it saw (0 when exact) so
that the mutation test can show that a planted mistake moves at least one of them.

All references are to "Looped Latent Attention: Cross-Loop KV Compression for Looped
Transformers" (arXiv 2607.15456v2) unless another page is named.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from oracle import lla_oracle as O
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _orthonormal(n, r, seed):
    a = _rng(seed).standard_normal((n, r))
    q, rr = np.linalg.qr(a)
    return q * np.sign(np.diag(rr))[None, :]


# ---------------------------------------------------------------------------
# Closed forms printed on the pages (Eq. 4, Table 5, Table 8, Table 3, slides).
# ---------------------------------------------------------------------------

def pin_closed_forms() -> float:
    g = _load("compression_closed_forms.json")
    err = 0.0
    w = g["worked_example"]
    err = max(err, abs(O.compression_ratio(w["T"], w["d_head"], w["r_k"], w["r_v"]) - w["rho"]))
    err = max(err, abs(O.teacher_scalars_per_token_layer(w["T"], 1, w["d_head"]) - w["numerator"]))
    err = max(err, abs(O.latent_scalars_per_token_layer(1, w["r_k"], w["r_v"]) - w["denominator"]))
    for r_k, r_v, rho in g["table8_ranks"]["rows"]:
        got = O.compression_ratio(4, 128, r_k, r_v)
        err = max(err, abs(round(got, 2) - rho))
    t5 = g["table5_memory"]
    H, d, T, bps = t5["H"], t5["d_head"], t5["T"], t5["bytes_per_scalar"]
    for D, key in ((24, "kv_per_token_kib_1p4b"), (48, "kv_per_token_kib_2p6b")):
        tab = t5[key]
        teacher = D * O.teacher_scalars_per_token_layer(T, H, d) * bps / 1024
        err = max(err, abs(teacher - tab["teacher"]))
        err = max(err, abs(O.cache_bytes_per_token(D, H, 96, 160, bps) / 1024 - tab["lla_4x"]))
        err = max(err, abs(O.cache_bytes_per_token(D, H, 16, 32, bps) / 1024 - tab["lla_21x"]))
    gib = t5["kv_1m_context_gib_1p4b"]
    err = max(err, abs(O.cache_bytes_per_token(24, H, 96, 160, bps) * 2**20 / 2**30 - gib["lla_4x"]))
    err = max(err, abs(O.cache_bytes_per_token(24, H, 16, 32, bps) * 2**20 / 2**30 - gib["lla_21x"]))
    err = max(err, abs(round(O.compression_ratio(4, 128, 16, 32), 1) - t5["lla_21x_rho_printed"]))
    ev = g["eviction_budget"]
    err = max(err, abs(O.cache_bytes_per_token(24, H, 16, 32, bps) * ev["kept_tokens"] / 2**20
                       - ev["mib_total"]))
    # Huginn (Table 3): every printed (rho, r_k, r_v) implies the same d_head via Eq. 4.
    hu = g["huginn_table3"]
    implied = [rho * (rk + rv) / (2 * hu["T"]) for rho, rk, rv in hu["rows"]]
    for rho, rk, rv in hu["rows"]:
        err = max(err, abs(O.compression_ratio(hu["T"], implied[0], rk, rv) - rho))
    return err


# ---------------------------------------------------------------------------
# RoPE: the RoFormer rotation, applied after reconstruction (Section 3).
# ---------------------------------------------------------------------------

def pin_rope() -> float:
    err = 0.0
    # theta_i = base^(-2i/d): d=4, base=10000 gives (1, 1/100).
    err = max(err, float(np.max(np.abs(O.rope_theta(4, 10000.0) - np.array([1.0, 0.01])))))
    # d=2 has theta_0 = 1 for any base: a counter-clockwise rotation by the position.
    for p in (0, 1, 3, 17):
        y = O.apply_rope(np.array([[1.0, 0.0], [0.0, 1.0]])[None], np.array([p]), 500.0)[0]
        err = max(err, abs(y[0, 0] - math.cos(p)), abs(y[0, 1] - math.sin(p)),
                  abs(y[1, 0] + math.sin(p)), abs(y[1, 1] - math.cos(p)))
    # Interleaved pairs: dims (0, 1) form pair 0 at theta_0 = 1 and dims (2, 3) pair 1.
    y = O.apply_rope(np.array([[[0.0, 0.0, 1.0, 0.0]]]), np.array([5]), 10000.0)[0, 0]
    err = max(err, abs(y[0]), abs(y[1]), abs(y[2] - math.cos(0.05)), abs(y[3] - math.sin(0.05)))
    # Position 0 is the identity, norms are preserved, and scores depend on the
    # position difference only.
    rng = _rng(3)
    x = rng.standard_normal((1, 6, 16))
    err = max(err, float(np.max(np.abs(O.apply_rope(x, np.zeros(6), 10000.0) - x))))
    pos = np.array([0, 1, 7, 100, 2047, 4095])
    y = O.apply_rope(x, pos, 10000.0)
    err = max(err, float(np.max(np.abs(np.linalg.norm(y, axis=-1) - np.linalg.norm(x, axis=-1)))))
    q, k = rng.standard_normal(16), rng.standard_normal(16)
    for a, b, shift in ((3, 10, 55), (0, 4000, 77), (120, 7, 1000)):
        s1 = O.apply_rope(q[None, None], np.array([a]), 10000.0)[0, 0] @ \
            O.apply_rope(k[None, None], np.array([b]), 10000.0)[0, 0]
        s2 = O.apply_rope(q[None, None], np.array([a + shift]), 10000.0)[0, 0] @ \
            O.apply_rope(k[None, None], np.array([b + shift]), 10000.0)[0, 0]
        err = max(err, abs(s1 - s2))
    return err


# ---------------------------------------------------------------------------
# Codec round trips and the SVD initialisation (Section 3, Eqs. 2-3).
# ---------------------------------------------------------------------------

def pin_codec() -> float:
    err = 0.0
    T, d = 2, 4
    rng = _rng(11)
    x = rng.standard_normal((9, T * d))
    mu = rng.standard_normal(T * d)
    # Full rank, orthonormal W_down, W_up,t its loop slices: exact round trip.
    w = _orthonormal(T * d, T * d, 5)
    c = O.encode(x, mu, w)
    for t in range(T):
        xt = O.reconstruct(c, w[t * d:(t + 1) * d], mu[t * d:(t + 1) * d])
        err = max(err, float(np.max(np.abs(xt - x[:, t * d:(t + 1) * d]))))
    # Scalar brute force of Eq. 2.
    wl = _orthonormal(T * d, 3, 6)
    cb = [brute.brute_encode_one(list(xi), list(mu), wl.tolist()) for xi in x]
    err = max(err, float(np.max(np.abs(O.encode(x, mu, wl) - np.array(cb)))))
    # Low rank with tied weights: reconstruction is the orthogonal projection of x - mu
    # onto span(W_down): idempotent, residual orthogonal to the span.
    c = O.encode(x, mu, wl)
    xh = np.concatenate([O.reconstruct(c, wl[t * d:(t + 1) * d], mu[t * d:(t + 1) * d])
                         for t in range(T)], axis=1)
    c2 = O.encode(xh, mu, wl)
    err = max(err, float(np.max(np.abs(c2 - c))))
    err = max(err, float(np.max(np.abs((x - xh) @ wl))))
    return err


def pin_svd_init() -> float:
    err = 0.0
    T, d, r = 3, 4, 5
    rng = _rng(21)
    n = 200
    base = rng.standard_normal((n, r)) @ rng.standard_normal((r, T * d))
    mu_true = rng.standard_normal(T * d)
    # Data of exact rank r after centring is reproduced exactly.
    x = base - base.mean(axis=0) + mu_true
    mu, wd, wu = O.svd_init(x, r, T, d)
    err = max(err, float(np.max(np.abs(mu - x.mean(axis=0)))))
    c = O.encode(x, mu, wd)
    for t in range(T):
        xt = O.reconstruct(c, wu[t], mu[t * d:(t + 1) * d])
        err = max(err, float(np.max(np.abs(xt - x[:, t * d:(t + 1) * d]))))
        err = max(err, float(np.max(np.abs(wu[t] - wd[t * d:(t + 1) * d]))))
    # Eckart-Young: with noise added, the residual energy equals the sum of the
    # discarded eigenvalues of the centred scatter matrix (computed with eigvalsh).
    xn = x + 0.3 * rng.standard_normal(x.shape)
    mu, wd, wu = O.svd_init(xn, r, T, d)
    c = O.encode(xn, mu, wd)
    xh = np.concatenate([O.reconstruct(c, wu[t], mu[t * d:(t + 1) * d]) for t in range(T)], 1)
    xc = xn - xn.mean(axis=0)
    ev = np.sort(np.linalg.eigvalsh(xc.T @ xc))[::-1]
    resid = float(np.sum((xn - xh) ** 2))
    err = max(err, abs(resid - float(np.sum(ev[r:]))) / max(1.0, resid))
    return err


# ---------------------------------------------------------------------------
# Whole decode: full-rank special case against textbook attention, special cases,
# the scalar brute force, and the LLA-2D reduction.
# ---------------------------------------------------------------------------

def _textbook_rope_complex(x: torch.Tensor, pos: torch.Tensor, base: float) -> torch.Tensor:
    """RoPE as complex multiplication: pairs (x_2i, x_2i+1) -> x_2i + i x_2i+1 times
    exp(i p theta_i)."""
    d = x.shape[-1]
    theta = base ** (-(torch.arange(0, d, 2, dtype=torch.float64)) / d)
    rot = torch.polar(torch.ones(pos.shape[0], d // 2, dtype=torch.float64),
                      pos[:, None].double() * theta[None, :])
    z = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous())
    return torch.view_as_real(z * rot).reshape(x.shape)


def pin_full_rank_textbook() -> float:
    """r = T*d, orthonormal W_down, W_up,t its loop slices: the latent decode must equal
    ordinary attention on the original per-loop keys and values (torch SDPA, fp64)."""
    T, H, d, n, B = 4, 2, 8, 13, 2
    rng = _rng(31)
    xk = rng.standard_normal((B, H, n, T, d))
    xv = rng.standard_normal((B, H, n, T, d))
    q = rng.standard_normal((B, H, T, d))
    r = T * d
    ck = np.empty((B, H, n, r))
    cv = np.empty((B, H, n, r))
    wuk = np.empty((T, H, d, r))
    wuv = np.empty((T, H, d, r))
    muk = rng.standard_normal((H, T * d))
    muv = rng.standard_normal((H, T * d))
    for h in range(H):
        wk = _orthonormal(r, r, 100 + h)
        wv = _orthonormal(r, r, 200 + h)
        ck[:, h] = O.encode(O.stack_loops(xk[:, h]), muk[h], wk)
        cv[:, h] = O.encode(O.stack_loops(xv[:, h]), muv[h], wv)
        for t in range(T):
            wuk[t, h] = wk[t * d:(t + 1) * d]
            wuv[t, h] = wv[t * d:(t + 1) * d]
    got = O.decode(ck, cv, wuk, muk, wuv, muv, q, 0, None, 10000.0)
    pos = torch.arange(n)
    err = 0.0
    for t in range(T):
        k = _textbook_rope_complex(torch.from_numpy(xk[:, :, :, t]), pos, 10000.0)
        v = torch.from_numpy(xv[:, :, :, t])
        qt = torch.from_numpy(q[:, :, t])[:, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v)[:, :, 0]
        err = max(err, float(np.max(np.abs(got[:, :, t] - ref.numpy()))))
    return err


def _tiny(seed, T=2, H=2, d=4, n=5, r_k=3, r_v=4, B=2, variant="per_head"):
    rng = _rng(seed)
    Hc = H if variant == "per_head" else 1
    din = d if variant == "per_head" else H * d
    return dict(
        c_k=rng.standard_normal((B, Hc, n, r_k)),
        c_v=rng.standard_normal((B, Hc, n, r_v)),
        w_up_k=rng.standard_normal((T, H, d, r_k)) / math.sqrt(r_k),
        mu_k=rng.standard_normal((Hc, T * din)) * 0.3,
        w_up_v=rng.standard_normal((T, H, d, r_v)) / math.sqrt(r_v),
        mu_v=rng.standard_normal((Hc, T * din)) * 0.3,
        q=rng.standard_normal((B, H, T, d)),
    )


def pin_brute_force() -> float:
    err = 0.0
    for variant, seed, base, ctx in (("per_head", 41, 10000.0, [5, 3]), ("per_head", 42, 7.0, [5, 5]),
                                     ("2d", 43, 100.0, [4, 5])):
        a = _tiny(seed, variant=variant)
        T, H, d = a["w_up_k"].shape[0], a["w_up_k"].shape[1], a["w_up_k"].shape[2]
        got = O.decode(a["c_k"], a["c_v"], a["w_up_k"], a["mu_k"], a["w_up_v"], a["mu_v"],
                       a["q"], 0, ctx, base, None, variant)
        for b in range(a["q"].shape[0]):
            for h in range(H):
                hc = h if variant == "per_head" else 0
                for t in range(T):
                    if variant == "per_head":
                        mk = a["mu_k"][h][t * d:(t + 1) * d]
                        mv = a["mu_v"][h][t * d:(t + 1) * d]
                    else:
                        mk = a["mu_k"][0][(t * H + h) * d:(t * H + h + 1) * d]
                        mv = a["mu_v"][0][(t * H + h) * d:(t * H + h + 1) * d]
                    ref = brute.brute_decode_one(
                        a["c_k"][b, hc, :ctx[b]].tolist(), a["c_v"][b, hc, :ctx[b]].tolist(),
                        a["w_up_k"][t, h].tolist(), list(mk), a["w_up_v"][t, h].tolist(), list(mv),
                        list(a["q"][b, h, t]), base, 1.0 / math.sqrt(d))
                    err = max(err, float(np.max(np.abs(got[b, h, t] - np.array(ref)))))
    return err


def pin_special_cases() -> float:
    err = 0.0
    a = _tiny(51, n=6)
    T, H, d = 2, 2, 4
    # q = 0: uniform weights, so the output is the mean latent pushed through W_up,v
    # plus mu_v (the V-side identity of Appendix J, "Absorbed attention").
    q0 = np.zeros_like(a["q"])
    got = O.decode(a["c_k"], a["c_v"], a["w_up_k"], a["mu_k"], a["w_up_v"], a["mu_v"], q0)
    for b in range(2):
        for h in range(H):
            for t in range(T):
                ref = a["c_v"][b, h].mean(axis=0) @ a["w_up_v"][t, h].T + a["mu_v"][h, t * d:(t + 1) * d]
                err = max(err, float(np.max(np.abs(got[b, h, t] - ref))))
    # n = 1: the output is that token's rebuilt value, whatever the query.
    got = O.decode(a["c_k"][:, :, :1], a["c_v"][:, :, :1], a["w_up_k"], a["mu_k"],
                   a["w_up_v"], a["mu_v"], a["q"] * 50.0)
    for b in range(2):
        for h in range(H):
            for t in range(T):
                ref = a["c_v"][b, h, 0] @ a["w_up_v"][t, h].T + a["mu_v"][h, t * d:(t + 1) * d]
                err = max(err, float(np.max(np.abs(got[b, h, t] - ref))))
    # Empty context: zeros (the reading taken for attention over no tokens).
    got = O.decode(a["c_k"], a["c_v"], a["w_up_k"], a["mu_k"], a["w_up_v"], a["mu_v"], a["q"],
                   0, [0, 6])
    err = max(err, float(np.max(np.abs(got[0]))))
    # Loop offset: decoding loops 1.. with loop_begin=1 equals the same slice of a
    # decode over all loops.
    full = O.decode(a["c_k"], a["c_v"], a["w_up_k"], a["mu_k"], a["w_up_v"], a["mu_v"], a["q"])
    part = O.decode(a["c_k"], a["c_v"], a["w_up_k"], a["mu_k"], a["w_up_v"], a["mu_v"],
                    a["q"][:, :, 1:], 1)
    err = max(err, float(np.max(np.abs(full[:, :, 1:] - part))))
    return err


def pin_large_alpha_limit() -> float:
    """q = alpha * K~_t[j*] for a late token j*: as alpha grows the softmax concentrates on
    j*, so the output tends to that token's rebuilt value V_t[j*] (attention is unchanged,
    Figure 1 caption; the value side of Eq. 3). The scores are formed here independently
    (explicit reconstruction, RoPE by complex multiplication); the oracle's output must lie
    within the bound (1 - a_j*) max_j |V_t[j] - V_t[j*]| <= sum_{j != j*} exp(s_j - s_j*)
    max_j |V_t[j] - V_t[j*]| of V_t[j*], and at alpha = 32 it must equal V_t[j*] to 1e-9.
    The largest scores are then several hundred, so the pin also needs a softmax that does
    not overflow."""
    worst = 0.0
    for variant, seed in (("per_head", 57), ("2d", 58)):
        a = _tiny(seed, T=2, H=2, d=16, n=40, r_k=6, r_v=5, B=2, variant=variant)
        T, H, d = 2, 2, 16
        n = a["c_k"].shape[2]
        scale = 1.0 / math.sqrt(d)
        pos = torch.arange(n)
        for alpha in (8.0, 32.0):
            q = np.zeros_like(a["q"])
            expect = np.zeros_like(a["q"])
            bound = np.zeros(a["q"].shape[:3])
            for b in range(2):
                for h in range(H):
                    hc = h if variant == "per_head" else 0
                    for t in range(T):
                        if variant == "per_head":
                            mk, mv = a["mu_k"][h][t * d:(t + 1) * d], a["mu_v"][h][t * d:(t + 1) * d]
                        else:
                            mk = a["mu_k"][0][(t * H + h) * d:(t * H + h + 1) * d]
                            mv = a["mu_v"][0][(t * H + h) * d:(t * H + h + 1) * d]
                        k_hat = a["c_k"][b, hc] @ a["w_up_k"][t, h].T + mk
                        v_hat = a["c_v"][b, hc] @ a["w_up_v"][t, h].T + mv
                        k_rot = _textbook_rope_complex(torch.from_numpy(k_hat), pos, 10000.0).numpy()
                        # j*: among the last 8 tokens, the one whose own score beats every
                        # other token's by the widest margin
                        gram = k_rot @ k_rot.T
                        cand = range(n - 8, n)
                        margin = [min(gram[j, j] - gram[i, j] for i in range(n) if i != j) for j in cand]
                        js = list(cand)[int(np.argmax(margin))]
                        assert max(margin) > 0.0
                        q[b, h, t] = alpha * k_rot[js]
                        s = scale * (k_rot @ q[b, h, t])
                        rest = np.exp(np.delete(s, js) - s[js]).sum()
                        spread = np.max(np.abs(v_hat - v_hat[js]))
                        expect[b, h, t] = v_hat[js]
                        bound[b, h, t] = rest * spread + 1e-12
            got = O.decode(a["c_k"], a["c_v"], a["w_up_k"], a["mu_k"], a["w_up_v"], a["mu_v"], q,
                           0, None, 10000.0, None, variant)
            dev = np.max(np.abs(got - expect), axis=-1)
            if not np.all(np.isfinite(dev)):
                return float("inf")
            worst = max(worst, float(np.max(dev - bound)))
            if alpha == 32.0:  # the limit is reached: o_t equals V_t[j*] to 1e-9
                worst = max(worst, float(np.max(dev)) - 1e-9)
    return max(worst, 0.0)


def pin_lla2d_block_diagonal() -> float:
    """LLA-2D with a block-diagonal codec (head h owns latent columns h*r_h ..) must equal
    per-head LLA with rank r_h (Section 3, "The LLA-2D variant": one latent per token
    and layer reconstructing all heads). Covers both encode and decode."""
    T, H, d, n, B, rk, rv = 2, 3, 4, 6, 2, 2, 3
    rng = _rng(61)
    xk = rng.standard_normal((B, n, H, T, d))
    xv = rng.standard_normal((B, n, H, T, d))
    q = rng.standard_normal((B, H, T, d))
    wdk = rng.standard_normal((H, T * d, rk))
    wdv = rng.standard_normal((H, T * d, rv))
    muk = rng.standard_normal((H, T * d))
    muv = rng.standard_normal((H, T * d))
    wuk = rng.standard_normal((T, H, d, rk))
    wuv = rng.standard_normal((T, H, d, rv))
    # per-head latents
    ck = np.stack([O.encode(xk[:, :, h].reshape(B, n, T * d), muk[h], wdk[h]) for h in range(H)], 1)
    cv = np.stack([O.encode(xv[:, :, h].reshape(B, n, T * d), muv[h], wdv[h]) for h in range(H)], 1)
    ref = O.decode(ck, cv, wuk, muk, wuv, muv, q, 0, None, 10000.0)
    # 2D: input stacked (t, h, d) with t outermost.
    x2k = np.transpose(xk, (0, 1, 3, 2, 4)).reshape(B, n, T * H * d)
    x2v = np.transpose(xv, (0, 1, 3, 2, 4)).reshape(B, n, T * H * d)

    def blockdiag(wd, r):
        out = np.zeros((T * H * d, H * r))
        for h in range(H):
            for t in range(T):
                out[(t * H + h) * d:(t * H + h + 1) * d, h * r:(h + 1) * r] = wd[h, t * d:(t + 1) * d]
        return out

    def restack(mu):
        out = np.zeros(T * H * d)
        for h in range(H):
            for t in range(T):
                out[(t * H + h) * d:(t * H + h + 1) * d] = mu[h, t * d:(t + 1) * d]
        return out

    def upembed(wu, r):
        out = np.zeros((T, H, d, H * r))
        for h in range(H):
            out[:, h, :, h * r:(h + 1) * r] = wu[:, h]
        return out

    mu2k, mu2v = restack(muk), restack(muv)
    c2k = O.encode(x2k, mu2k, blockdiag(wdk, rk))[:, None]
    c2v = O.encode(x2v, mu2v, blockdiag(wdv, rv))[:, None]
    err = float(np.max(np.abs(c2k[:, 0].reshape(B, n, H, rk) - np.transpose(ck, (0, 2, 1, 3)))))
    got = O.decode(c2k, c2v, upembed(wuk, rk), mu2k[None], upembed(wuv, rv), mu2v[None], q, 0,
                   None, 10000.0, None, "2d")
    return max(err, float(np.max(np.abs(got - ref))))


def pin_round_bf16() -> float:
    """Round-to-nearest-even to 8 significant bits, checked against torch's float32 ->
    bfloat16 conversion on values exact in float32, and on explicit ties."""
    rng = _rng(71)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    err = float(np.max(np.abs(O.round_bf16(x.astype(np.float64)) - ref) / np.abs(ref)))
    # Explicit ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 (goes to 1, the even
    # mantissa); 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6 (goes to 1 + 2^-6);
    # 0.5 + 3*2^-9 lies halfway between 0.5 + 2^-8 and 0.5 + 2^-7 (goes to 0.5 + 2^-7).
    ties = np.array([1 + 2.0**-8, 1 + 3 * 2.0**-8, -(1 + 2.0**-8), 0.5 + 3 * 2.0**-9])
    want = np.array([1.0, 1 + 2.0**-6, -1.0, 0.5 + 2.0**-7])
    err = max(err, float(np.max(np.abs(O.round_bf16(ties) - want))))
    return err


def pin_absorbed_textbook() -> float:
    """Decoupled decode with a full-rank codec (r = T*d, orthonormal W_down, W_up,t its
    loop slices, so Eq. 3 gives back the original per-loop keys and values): it must equal
    ordinary attention (torch SDPA, fp64) whose keys are the stored rotary keys in
    dimensions < d_rope and the original keys elsewhere, with scale 1/sqrt(d). Covers
    d_rope = 0 (content only), a mixed split and d_rope = d (rotary only)."""
    T, H, d, n, B = 2, 2, 8, 11, 2
    rng = _rng(61)
    xk = rng.standard_normal((B, H, n, T, d))
    xv = rng.standard_normal((B, H, n, T, d))
    q = rng.standard_normal((B, H, T, d))
    r = T * d
    ck = np.empty((B, H, n, r))
    cv = np.empty((B, H, n, r))
    wuk = np.empty((T, H, d, r))
    wuv = np.empty((T, H, d, r))
    muk = rng.standard_normal((H, T * d))
    muv = rng.standard_normal((H, T * d))
    for h in range(H):
        wk = _orthonormal(r, r, 300 + h)
        wv = _orthonormal(r, r, 400 + h)
        ck[:, h] = O.encode(O.stack_loops(xk[:, h]), muk[h], wk)
        cv[:, h] = O.encode(O.stack_loops(xv[:, h]), muv[h], wv)
        for t in range(T):
            wuk[t, h] = wk[t * d:(t + 1) * d]
            wuv[t, h] = wv[t * d:(t + 1) * d]
    err = 0.0
    for d_rope in (0, 4, d):
        kr = rng.standard_normal((B, H, n, d_rope))
        got = O.decode_absorbed(ck, cv, kr, wuk, muk, wuv, muv, q, d_rope)
        for t in range(T):
            k = torch.from_numpy(np.concatenate([kr, xk[:, :, :, t, d_rope:]], axis=-1))
            v = torch.from_numpy(xv[:, :, :, t])
            qt = torch.from_numpy(q[:, :, t])[:, :, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v, scale=1.0 / math.sqrt(d))[:, :, 0]
            err = max(err, float(np.max(np.abs(got[:, :, t] - ref.numpy()))))
    return err


def pin_absorbed_brute_force() -> float:
    """Decoupled decode against the scalar re-derivation, low-rank codec, ragged
    contexts, per head and LLA-2D."""
    err = 0.0
    for variant, seed, ctx, d_rope in (("per_head", 71, [5, 2], 2), ("2d", 72, [4, 5], 2),
                                       ("per_head", 73, [5, 5], 4)):
        a = _tiny(seed, variant=variant)
        T, H, d = a["w_up_k"].shape[0], a["w_up_k"].shape[1], a["w_up_k"].shape[2]
        B, n = a["q"].shape[0], a["c_k"].shape[2]
        kr = _rng(seed + 100).standard_normal((B, H, n, d_rope))
        got = O.decode_absorbed(a["c_k"], a["c_v"], kr, a["w_up_k"], a["mu_k"], a["w_up_v"],
                                a["mu_v"], a["q"], d_rope, 0, ctx, None, variant)
        for b in range(B):
            for h in range(H):
                hc = h if variant == "per_head" else 0
                for t in range(T):
                    if variant == "per_head":
                        mk = a["mu_k"][h][t * d:(t + 1) * d]
                        mv = a["mu_v"][h][t * d:(t + 1) * d]
                    else:
                        mk = a["mu_k"][0][(t * H + h) * d:(t * H + h + 1) * d]
                        mv = a["mu_v"][0][(t * H + h) * d:(t * H + h + 1) * d]
                    ref = brute.brute_decode_absorbed_one(
                        a["c_k"][b, hc, :ctx[b]].tolist(), a["c_v"][b, hc, :ctx[b]].tolist(),
                        kr[b, h, :ctx[b]].tolist(), a["w_up_k"][t, h].tolist(), list(mk),
                        a["w_up_v"][t, h].tolist(), list(mv), list(a["q"][b, h, t]), d_rope,
                        1.0 / math.sqrt(d))
                    err = max(err, float(np.max(np.abs(got[b, h, t] - np.array(ref)))))
    return err


def pin_absorbed_equals_full_rope() -> float:
    """With a single loop, d_rope = d and the rotary keys set to the rotated
    reconstructions (computed here by complex multiplication), the decoupled decode is
    the full-RoPE latent decode."""
    a = _tiny(81, T=1, n=6)
    B, H, n = a["q"].shape[0], a["q"].shape[1], a["c_k"].shape[2]
    d = a["w_up_k"].shape[2]
    kr = np.empty((B, H, n, d))
    for b in range(B):
        for h in range(H):
            k_hat = a["c_k"][b, h] @ a["w_up_k"][0, h].T + a["mu_k"][h][:d]
            kr[b, h] = _textbook_rope_complex(torch.from_numpy(k_hat), torch.arange(n), 10000.0).numpy()
    got = O.decode_absorbed(a["c_k"], a["c_v"], kr, a["w_up_k"], a["mu_k"], a["w_up_v"],
                            a["mu_v"], a["q"], d)
    ref = O.decode(a["c_k"], a["c_v"], a["w_up_k"], a["mu_k"], a["w_up_v"], a["mu_v"], a["q"])
    return float(np.max(np.abs(got - ref)))


def pin_teacher_textbook() -> float:
    """Uncompressed decode against torch SDPA (fp64) on the same per-loop caches, ragged
    contexts included (a masked tail)."""
    T, B, H, n, d = 3, 2, 2, 9, 8
    rng = _rng(91)
    k = rng.standard_normal((T, B, H, n, d))
    v = rng.standard_normal((T, B, H, n, d))
    q = rng.standard_normal((B, H, T, d))
    lens = [9, 4]
    got = O.decode_teacher(k, v, q, 0, lens)
    err = 0.0
    for t in range(T):
        for b in range(B):
            kk = torch.from_numpy(k[t, b, :, :lens[b]])[None]
            vv = torch.from_numpy(v[t, b, :, :lens[b]])[None]
            qq = torch.from_numpy(q[b, :, t])[None, :, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[0, :, 0]
            err = max(err, float(np.max(np.abs(got[b, :, t] - ref.numpy()))))
    return err


def pin_teacher_equals_latent_decode() -> float:
    """The latent decode is the teacher's attention over the keys and values that the
    codec rebuilds: materialise K_t = RoPE(c_k W_up,k,t^T + mu_k,t) (complex RoPE here)
    and V_t, and the uncompressed decode of them equals the latent decode."""
    a = _tiny(92, T=3, n=7)
    T, H, d = a["w_up_k"].shape[0], a["w_up_k"].shape[1], a["w_up_k"].shape[2]
    B, n = a["q"].shape[0], a["c_k"].shape[2]
    k = np.empty((T, B, H, n, d))
    v = np.empty((T, B, H, n, d))
    for t in range(T):
        for b in range(B):
            for h in range(H):
                kh = a["c_k"][b, h] @ a["w_up_k"][t, h].T + a["mu_k"][h][t * d:(t + 1) * d]
                k[t, b, h] = _textbook_rope_complex(torch.from_numpy(kh), torch.arange(n), 10000.0).numpy()
                v[t, b, h] = a["c_v"][b, h] @ a["w_up_v"][t, h].T + a["mu_v"][h][t * d:(t + 1) * d]
    lens = [7, 3]
    got = O.decode_teacher(k, v, a["q"], 0, lens)
    ref = O.decode(a["c_k"], a["c_v"], a["w_up_k"], a["mu_k"], a["w_up_v"], a["mu_v"], a["q"], 0, lens)
    return float(np.max(np.abs(got - ref)))


def pin_reconstruct_round_trip() -> float:
    """Full-rank orthonormal codec (r = T*d, W_up,t the loop slices of W_down): the
    materialised reconstruction of a slot range gives back the original per-loop keys
    (rotated by complex multiplication at their slots) and values exactly."""
    T, H, d, n, B = 3, 2, 4, 9, 2
    rng = _rng(93)
    xk = rng.standard_normal((B, H, n, T, d))
    xv = rng.standard_normal((B, H, n, T, d))
    r = T * d
    ck, cv = np.empty((B, H, n, r)), np.empty((B, H, n, r))
    wuk, wuv = np.empty((T, H, d, r)), np.empty((T, H, d, r))
    muk, muv = rng.standard_normal((H, T * d)), rng.standard_normal((H, T * d))
    for h in range(H):
        wk, wv = _orthonormal(r, r, 300 + h), _orthonormal(r, r, 400 + h)
        ck[:, h] = O.encode(O.stack_loops(xk[:, h]), muk[h], wk)
        cv[:, h] = O.encode(O.stack_loops(xv[:, h]), muv[h], wv)
        for t in range(T):
            wuk[t, h], wuv[t, h] = wk[t * d:(t + 1) * d], wv[t * d:(t + 1) * d]
    p0, nt, lb, lc = 3, 5, 1, 2
    k, v = O.reconstruct_cache(ck, cv, wuk, muk, wuv, muv, lb, lc, p0, nt, 10000.0)
    err = 0.0
    for li in range(lc):
        t = lb + li
        kr = _textbook_rope_complex(torch.from_numpy(xk[:, :, p0:p0 + nt, t]),
                                    torch.arange(p0, p0 + nt), 10000.0).numpy()
        err = max(err, float(np.max(np.abs(k[li] - kr))),
                  float(np.max(np.abs(v[li] - xv[:, :, p0:p0 + nt, t]))))
    return err


def pin_reconstruct_brute_force() -> float:
    """Element by element against oracle/brute.py (scalar codec, complex RoPE), per head
    and LLA-2D, a slot range that starts inside the cache."""
    err = 0.0
    for variant, seed, base in (("per_head", 94, 10000.0), ("2d", 95, 100.0)):
        a = _tiny(seed, T=3, n=7, variant=variant)
        T, H, d = a["w_up_k"].shape[0], a["w_up_k"].shape[1], a["w_up_k"].shape[2]
        p0, nt = 2, 4
        k, v = O.reconstruct_cache(a["c_k"], a["c_v"], a["w_up_k"], a["mu_k"], a["w_up_v"],
                                   a["mu_v"], 0, T, p0, nt, base, variant)
        for b in range(a["c_k"].shape[0]):
            for h in range(H):
                hc = h if variant == "per_head" else 0
                for t in range(T):
                    if variant == "per_head":
                        mk = a["mu_k"][h][t * d:(t + 1) * d]
                        mv = a["mu_v"][h][t * d:(t + 1) * d]
                    else:
                        mk = a["mu_k"][0][(t * H + h) * d:(t * H + h + 1) * d]
                        mv = a["mu_v"][0][(t * H + h) * d:(t * H + h + 1) * d]
                    for j in range(nt):
                        kb = brute.brute_reconstruct_key_one(list(a["c_k"][b, hc, p0 + j]),
                                                             a["w_up_k"][t, h].tolist(), list(mk),
                                                             p0 + j, base)
                        vb = brute.brute_reconstruct_value_one(list(a["c_v"][b, hc, p0 + j]),
                                                               a["w_up_v"][t, h].tolist(), list(mv))
                        err = max(err, float(np.max(np.abs(k[t, b, h, j] - np.array(kb)))),
                                  float(np.max(np.abs(v[t, b, h, j] - np.array(vb)))))
    return err


def pin_reconstruct_feeds_teacher() -> float:
    """The full-memory path: reconstruct every slot, then the uncompressed decode of the
    rebuilt cache equals the latent decode (both oracle functions, different routes)."""
    a = _tiny(96, T=3, n=8)
    T = a["w_up_k"].shape[0]
    n = a["c_k"].shape[2]
    k, v = O.reconstruct_cache(a["c_k"], a["c_v"], a["w_up_k"], a["mu_k"], a["w_up_v"],
                               a["mu_v"], 0, T, 0, n, 10000.0)
    lens = [8, 5]
    got = O.decode_teacher(k, v, a["q"], 0, lens)
    ref = O.decode(a["c_k"], a["c_v"], a["w_up_k"], a["mu_k"], a["w_up_v"], a["mu_v"], a["q"], 0, lens)
    return float(np.max(np.abs(got - ref)))


def pin_paged_permuted() -> float:
    """A dense latent cache scattered into pages in a random order (the pool built here by
    reshaping, not by the oracle's gather): the paged decode equals the dense decode, per
    head and LLA-2D, ragged contexts included."""
    err = 0.0
    for variant, seed in (("per_head", 97), ("2d", 98)):
        a = _tiny(seed, T=2, n=48, variant=variant)
        B, Hc, n, _ = a["c_k"].shape
        npg = n // O.PAGE
        rng = _rng(seed + 1)
        perm = rng.permutation(B * npg + 3)[:B * npg]  # physical page of (b, p), spares unused
        table = perm.reshape(B, npg)
        pools = []
        for key in ("c_k", "c_v"):
            x = a[key]
            pool = rng.standard_normal((B * npg + 3, Hc, O.PAGE, x.shape[3]))  # junk in spares
            pages = x.reshape(B, Hc, npg, O.PAGE, x.shape[3]).transpose(0, 2, 1, 3, 4)
            pool[table.reshape(-1)] = pages.reshape(B * npg, Hc, O.PAGE, x.shape[3])
            pools.append(pool)
        lens = [48, 21]
        got = O.decode_paged(pools[0], pools[1], table, a["w_up_k"], a["mu_k"], a["w_up_v"],
                             a["mu_v"], a["q"], 0, lens, None, 10000.0, None, variant)
        ref = O.decode(a["c_k"], a["c_v"], a["w_up_k"], a["mu_k"], a["w_up_v"], a["mu_v"], a["q"],
                       0, lens, 10000.0, None, variant)
        err = max(err, float(np.max(np.abs(got - ref))))
    return err


def pin_absorbed_paged_permuted() -> float:
    """The decoupled decode over a cache scattered into shuffled pages (latents and rotary
    keys, pools built here by reshaping, junk in spare pages) equals the dense decoupled
    decode, per head and LLA-2D, ragged contexts included."""
    err = 0.0
    for variant, seed, d_rope in (("per_head", 91, 2), ("2d", 92, 4)):
        a = _tiny(seed, T=2, n=48, variant=variant)
        B, Hc, n, _ = a["c_k"].shape
        H = a["w_up_k"].shape[1]
        npg = n // O.PAGE
        rng = _rng(seed + 1)
        kr = rng.standard_normal((B, H, n, d_rope))
        table = rng.permutation(B * npg + 2)[:B * npg].reshape(B, npg)
        pools = []
        for x in (a["c_k"], a["c_v"], kr):
            X = x.shape[1]
            pool = rng.standard_normal((B * npg + 2, X, O.PAGE, x.shape[3]))
            pages = x.reshape(B, X, npg, O.PAGE, x.shape[3]).transpose(0, 2, 1, 3, 4)
            pool[table.reshape(-1)] = pages.reshape(B * npg, X, O.PAGE, x.shape[3])
            pools.append(pool)
        lens = [48, 19]
        got = O.decode_absorbed_paged(pools[0], pools[1], pools[2], table, a["w_up_k"], a["mu_k"],
                                      a["w_up_v"], a["mu_v"], a["q"], d_rope, 0, lens, None, None,
                                      variant)
        ref = O.decode_absorbed(a["c_k"], a["c_v"], kr, a["w_up_k"], a["mu_k"], a["w_up_v"],
                                a["mu_v"], a["q"], d_rope, 0, lens, None, variant)
        err = max(err, float(np.max(np.abs(got - ref))))
    return err


def pin_eviction_window() -> float:
    """StreamingLLM-style eviction: window_pages against hand-listed cases, then, with a
    full-rank orthonormal codec, the paged decode over the kept pages (sink page plus the
    newest pages) equals textbook attention (torch SDPA, fp64) over the kept tokens'
    original keys and values, the keys rotated at their positions in the kept cache."""
    err = 0.0
    for args, want in (((3, 1, 4), [0, 1, 2]), ((5, 1, 4), [0, 1, 2, 3, 4]),
                       ((10, 1, 4), [0, 6, 7, 8, 9]), ((9, 2, 3), [0, 1, 6, 7, 8])):
        if O.window_pages(*args) != want:
            err = max(err, 1.0)
    T, H, d, B = 2, 2, 4, 1
    r = T * d
    written = 9  # pages written; kept: page 0 and pages 6..8
    n_all = written * O.PAGE
    rng = _rng(99)
    xk = rng.standard_normal((B, H, n_all, T, d))
    xv = rng.standard_normal((B, H, n_all, T, d))
    muk, muv = rng.standard_normal((H, T * d)), rng.standard_normal((H, T * d))
    wuk, wuv = np.empty((T, H, d, r)), np.empty((T, H, d, r))
    pool_k = np.zeros((written + 2, H, O.PAGE, r))
    pool_v = np.zeros((written + 2, H, O.PAGE, r))
    phys = rng.permutation(written + 2)[:written]  # physical page of each logical page
    for h in range(H):
        wk, wv = _orthonormal(r, r, 500 + h), _orthonormal(r, r, 600 + h)
        ck = O.encode(O.stack_loops(xk[0, h]), muk[h], wk)
        cv = O.encode(O.stack_loops(xv[0, h]), muv[h], wv)
        for pg in range(written):
            pool_k[phys[pg], h] = ck[pg * O.PAGE:(pg + 1) * O.PAGE]
            pool_v[phys[pg], h] = cv[pg * O.PAGE:(pg + 1) * O.PAGE]
        for t in range(T):
            wuk[t, h], wuv[t, h] = wk[t * d:(t + 1) * d], wv[t * d:(t + 1) * d]
    kept = O.window_pages(written, 1, 3)
    table = np.array([[phys[pg] for pg in kept]])
    toks = np.concatenate([np.arange(pg * O.PAGE, (pg + 1) * O.PAGE) for pg in kept])
    n_kept = len(toks) - 5  # the newest page only partly filled
    toks = toks[:n_kept]
    q = rng.standard_normal((B, H, T, d))
    got = O.decode_paged(pool_k, pool_v, table, wuk, muk, wuv, muv, q, 0, [n_kept], None)
    pos = torch.arange(n_kept)
    for t in range(T):
        k = _textbook_rope_complex(torch.from_numpy(xk[:, :, toks, t]), pos, 10000.0)
        v = torch.from_numpy(xv[:, :, toks, t])
        qt = torch.from_numpy(q[:, :, t])[:, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v)[:, :, 0]
        err = max(err, float(np.max(np.abs(got[:, :, t] - ref.numpy()))))
    return err


def pin_encode_fused() -> float:
    """Projection-fused encode: (1) a scalar brute force (oracle/brute.py) on tiny inputs,
    per head and LLA-2D; (2) full rank: r = T*d, orthonormal W_down, W_up,t its loop slices,
    so rebuilding loop t gives back h_t W_proj (head slice, by torch.matmul) exactly; (3)
    the oracle's encode of captures materialised by torch.matmul, stacked by reshaping."""
    err = 0.0
    rng = _rng(71)
    T, H, d, dm, N = 2, 2, 4, 6, 3
    for variant in ("per_head", "2d"):
        Hc = H if variant == "per_head" else 1
        din = d if variant == "per_head" else H * d
        r = 3
        h = rng.standard_normal((T, N, dm))
        wp = rng.standard_normal((dm, H * d)) / math.sqrt(dm)
        mu = rng.standard_normal((Hc, T * din)) * 0.3
        wd = rng.standard_normal((Hc, T * din, r)) / math.sqrt(T * din)
        got = O.encode_fused(h, wp, mu, wd, H, d, variant)
        for n in range(N):
            for hc in range(Hc):
                ref = brute.brute_encode_fused_one(h[:, n].tolist(), wp.tolist(), mu[hc].tolist(),
                                                   wd[hc].tolist(), hc, H, d, variant == "per_head")
                err = max(err, float(np.max(np.abs(got[n, hc] - np.array(ref)))))
        # (3) captures by a library matmul, stacked by reshaping [N, T, H, d]
        x = torch.matmul(torch.from_numpy(h), torch.from_numpy(wp)).numpy()  # [T, N, H*d]
        xs = np.transpose(x.reshape(T, N, H, d), (1, 2, 0, 3))  # [N, H, T, d]
        for hc in range(Hc):
            stacked = xs[:, hc].reshape(N, T * d) if variant == "per_head" else \
                np.transpose(xs, (0, 2, 1, 3)).reshape(N, T * H * d)
            err = max(err, float(np.max(np.abs(got[:, hc] - O.encode(stacked, mu[hc], wd[hc])))))
    # (2) full-rank round trip, per head
    r = T * d
    h = rng.standard_normal((T, N, dm))
    wp = rng.standard_normal((dm, H * d))
    mu = rng.standard_normal((H, T * d))
    wd = np.stack([_orthonormal(r, r, 300 + hh) for hh in range(H)])
    c = O.encode_fused(h, wp, mu, wd, H, d, "per_head")
    x = torch.matmul(torch.from_numpy(h), torch.from_numpy(wp)).numpy()
    for hh in range(H):
        for t in range(T):
            back = O.reconstruct(c[:, hh], wd[hh][t * d:(t + 1) * d], mu[hh, t * d:(t + 1) * d])
            err = max(err, float(np.max(np.abs(back - x[t][:, hh * d:(hh + 1) * d]))))
    return err


ALL_PINS = {
    "closed_forms": (pin_closed_forms, 1e-9),
    "rope": (pin_rope, 1e-12),
    "codec": (pin_codec, 1e-12),
    "svd_init": (pin_svd_init, 1e-9),
    "full_rank_textbook": (pin_full_rank_textbook, 1e-12),
    "brute_force": (pin_brute_force, 1e-12),
    "special_cases": (pin_special_cases, 1e-12),
    "large_alpha_limit": (pin_large_alpha_limit, 1e-12),
    "lla2d_block_diagonal": (pin_lla2d_block_diagonal, 1e-12),
    "round_bf16": (pin_round_bf16, 0.0),
    "absorbed_textbook": (pin_absorbed_textbook, 1e-12),
    "absorbed_brute_force": (pin_absorbed_brute_force, 1e-12),
    "absorbed_equals_full_rope": (pin_absorbed_equals_full_rope, 1e-12),
    "teacher_textbook": (pin_teacher_textbook, 1e-12),
    "teacher_equals_latent_decode": (pin_teacher_equals_latent_decode, 1e-12),
    "reconstruct_round_trip": (pin_reconstruct_round_trip, 1e-12),
    "reconstruct_brute_force": (pin_reconstruct_brute_force, 1e-12),
    "reconstruct_feeds_teacher": (pin_reconstruct_feeds_teacher, 1e-12),
    "paged_permuted": (pin_paged_permuted, 1e-12),
    "eviction_window": (pin_eviction_window, 1e-12),
    "absorbed_paged_permuted": (pin_absorbed_paged_permuted, 1e-12),
    "encode_fused": (pin_encode_fused, 1e-12),
}
