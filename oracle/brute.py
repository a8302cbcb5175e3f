"""Scalar brute-force re-derivation of LLA latent decode, for tiny inputs.

TEST INFRASTRUCTURE ONLY: used by ``tests/`` to pin ``oracle/lla_oracle.py``.

Written independently of the NumPy oracle and in a different form: plain Python
floats and lists, RoPE as multiplication of the complex number x_2i + i x_2i+1 by
exp(i p theta_i) (the complex form of the RoFormer rotation), a max-shifted softmax
summed with ``math.fsum``, and the codec of "Looped Latent Attention" Section 3
(Eqs. 2-3) written out element by element. Intended for n <= 8, d <= 8, r <= 8.
"""

from __future__ import annotations

import cmath
import math


def _row_times_matT(c, w):
    """c [r] times w^T where w is [d][r] -> [d]."""
    return [math.fsum(c[k] * w[i][k] for k in range(len(c))) for i in range(len(w))]


def brute_decode_one(c_k, c_v, w_up_k_t, mu_k_t, w_up_v_t, mu_v_t, q, base, scale):
    """One (sequence, head, loop): c_k [n][r_k], c_v [n][r_v], W_up [d][r], mu [d],
    q [d]. Returns the attention output [d] as a list of floats."""
    n = len(c_k)
    d = len(q)
    if n == 0:
        return [0.0] * d
    scores = []
    for j in range(n):
        k = [a + b for a, b in zip(_row_times_matT(c_k[j], w_up_k_t), mu_k_t)]
        s = 0.0
        for i in range(d // 2):
            theta = base ** (-(2.0 * i) / d)
            z = complex(k[2 * i], k[2 * i + 1]) * cmath.exp(1j * (j * theta))
            s += q[2 * i] * z.real + q[2 * i + 1] * z.imag
        scores.append(scale * s)
    m = max(scores)
    e = [math.exp(s - m) for s in scores]
    tot = math.fsum(e)
    out = [0.0] * d
    for j in range(n):
        v = [a + b for a, b in zip(_row_times_matT(c_v[j], w_up_v_t), mu_v_t)]
        w = e[j] / tot
        for i in range(d):
            out[i] += w * v[i]
    return out


def brute_encode_one(x, mu, w_down):
    """Eq. 2 for one vector: x [T*d], mu [T*d], W_down [T*d][r] -> c [r]."""
    r = len(w_down[0])
    return [math.fsum((x[i] - mu[i]) * w_down[i][k] for i in range(len(x))) for k in range(r)]


def brute_decode_absorbed_one(c_k, c_v, k_rope, w_up_k_t, mu_k_t, w_up_v_t, mu_v_t, q, d_rope,
                              scale):
    """One (head, loop) of the decoupled decode with scalar loops: for every token the
    score is the rotary dot over dimensions i < d_rope (stored rotated key) plus the
    content dot over i >= d_rope of the reconstructed key (Eq. 3, no rotation)."""
    d = len(q)
    scores = []
    for j in range(len(c_k)):
        k_hat = _row_times_matT(c_k[j], w_up_k_t)
        s = [q[i] * k_rope[j][i] for i in range(d_rope)]
        s += [q[i] * (k_hat[i] + mu_k_t[i]) for i in range(d_rope, d)]
        scores.append(scale * math.fsum(s))
    if not scores:
        return [0.0] * d
    m = max(scores)
    w = [math.exp(x - m) for x in scores]
    tot = math.fsum(w)
    out = []
    for i in range(d):
        out.append(math.fsum(w[j] * (_row_times_matT(c_v[j], w_up_v_t)[i] + mu_v_t[i])
                             for j in range(len(c_v))) / tot)
    return out


def brute_reconstruct_key_one(c, w_up_t, mu_t, pos, base):
    """One rebuilt key at slot `pos`: c [r], W_up,t [d][r], mu_t [d]; the pairs rotated
    as complex numbers. Returns [d] as a list of floats."""
    k = [a + b for a, b in zip(_row_times_matT(c, w_up_t), mu_t)]
    d = len(k)
    out = [0.0] * d
    for i in range(d // 2):
        theta = base ** (-(2.0 * i) / d)
        z = complex(k[2 * i], k[2 * i + 1]) * cmath.exp(1j * (pos * theta))
        out[2 * i], out[2 * i + 1] = z.real, z.imag
    return out


def brute_reconstruct_value_one(c, w_up_t, mu_t):
    """One rebuilt value: c [r], W_up,t [d][r], mu_t [d] -> [d]."""
    return [a + b for a, b in zip(_row_times_matT(c, w_up_t), mu_t)]


def brute_encode_fused_one(h_loops, w_proj, mu, w_down, head, H, d, per_head):
    """Latent of one token and latent head by scalar loops: h_loops [T][d_model], w_proj
    [d_model][H*d], mu [T*d_in], w_down [T*d_in][r]. Loop t's projection is summed term
    by term and placed at stacked offset t*d_in (+ h*d within LLA-2D's (t, h, d) order)."""
    T = len(h_loops)
    heads = [head] if per_head else list(range(H))
    d_in = d * len(heads)
    x = [0.0] * (T * d_in)
    for t in range(T):
        for k, hh in enumerate(heads):
            for i in range(d):
                col = hh * d + i
                x[t * d_in + k * d + i] = math.fsum(h_loops[t][m] * w_proj[m][col]
                                                    for m in range(len(h_loops[t])))
    r = len(w_down[0])
    return [math.fsum((x[a] - mu[a]) * w_down[a][j] for a in range(len(x))) for j in range(r)]

