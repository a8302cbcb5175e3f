"""Decode inputs that drive attention into its large-score regimes, shared by the GPU
parity tests (tests/test_gpu_softmax_regimes.py) and the CPU check that those inputs are
strong enough to expose a kernel that forgets to rescale its running softmax state
(tests/test_softmax_regimes.py).

Attention itself is unchanged by the codec ("Looped Latent Attention", Figure 1 caption),
so every decode must follow the textbook softmax also where scores spread over tens of
nats and the running maximum rises late in the context. Regimes:

* ``spread``  : queries alpha * N(0, 1) with alpha = 8; scores then have a standard
                deviation of about 8 (score spreads of 40-60 over a 1000-token context).
* ``planted`` : one late token j* per (sequence, head, loop) with q = beta * K~_t[j*] /
                |K~_t[j*]| + 0.5 N(0, 1), beta = 40: its score beats the others by about
                30, so the output is essentially V_t[j*] (the large-alpha limit of the
                oracle's pins), and a running maximum is raised at j* with live state.
* ``scale``   : an explicit score scale 0.3 (not 1/sqrt(d)) with queries 2 * N(0, 1).
* ``base1e6`` : RoPE base 1e6 (the Ouro family's setting on the Ragged-KV page) with the
                ``spread`` queries.

All inputs are drawn on the CPU (``inputs.decode_inputs`` / ``teacher_inputs``), the
queries of the layer under test are replaced here, and the GPU tests copy the tensors to
the device, so the CPU check sees exactly the GPU's inputs. The key rows used to plant a
query come from the oracle (tests may use it); nothing here comes from the HIP path.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from latent_decode_attention_lla_amd.inputs import Workload, decode_inputs, teacher_inputs
from oracle import lla_oracle as O

REGIMES = ("spread", "planted", "scale", "base1e6")
LOG2E = 1.4426950408889634


def regime_workload(w: Workload, regime: str) -> Workload:
    if regime == "scale":
        return w.replace(scale=0.3)
    if regime == "base1e6":
        return w.replace(rope_base=1.0e6)
    return w


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def key_rows(w: Workload, t: dict, layer: int, loop: int, b: int, h: int, n: int) -> np.ndarray:
    """The keys loop ``loop`` of head h attends over, [n][d] float64: rebuilt and rotated
    latents (Eq. 3 and RoPE), the decoupled key [k_rope ; content] of the absorbed decode,
    or the uncompressed cache's rows."""
    if w.teacher:
        return _f64(t["k_cache"][layer, loop, b, h, :n])
    variant = "per_head" if w.variant == "per_head" else "2d"
    hc = h if variant == "per_head" else 0
    mu = O._mu_slice(_f64(t["mu_k"][layer]), variant, loop, h, w.H, w.d)
    k_hat = O.reconstruct(_f64(t["c_k"][layer, b, hc, :n]), _f64(t["w_up_k"][layer, loop, h]), mu)
    if w.d_rope > 0:
        return O.absorbed_keys(_f64(t["k_rope"][layer, b, h, :n]), k_hat, w.d_rope)
    return O.apply_rope(k_hat, np.arange(n), w.rope_base)


def score_scale(w: Workload) -> float:
    return w.scale if w.scale != 0.0 else 1.0 / math.sqrt(w.d)


def build(w: Workload, regime: str, seed: int, layer: int = 0, loop_begin: int = 0,
          loop_count: int | None = None):
    """CPU tensors for ``regime`` (the workload already passed through regime_workload),
    with the queries of loops loop_begin .. of ``layer`` replaced. Returns (tensors,
    planted) where planted[(b, h, loop)] = j* for the planted regime."""
    L = w.T - loop_begin if loop_count is None else loop_count
    t = teacher_inputs(w, seed, "cpu") if w.teacher else decode_inputs(w, seed, "cpu")
    q = t["q"][layer, loop_begin:loop_begin + L]  # [L][B][H][d] view
    alpha = {"spread": 8.0, "base1e6": 8.0, "scale": 2.0, "planted": 0.5}[regime]
    q.mul_(alpha)
    planted = {}
    if regime == "planted":
        rng = np.random.default_rng(seed)
        for li in range(L):
            for b in range(w.batch):
                for h in range(w.H):
                    keys = key_rows(w, t, layer, loop_begin + li, b, h, w.n)
                    js = int(rng.integers(int(0.75 * w.n), w.n))
                    u = keys[js] / np.linalg.norm(keys[js])
                    q[li, b, h] += torch.from_numpy(40.0 * u).to(torch.float32)
                    planted[(b, h, loop_begin + li)] = js
    return t, planted


def scores_exp2(w: Workload, t: dict, layer: int, loop: int, b: int, h: int, n: int) -> np.ndarray:
    """Scores of every token in the exp2 domain (scale * log2 e * q . k), float64."""
    keys = key_rows(w, t, layer, loop, b, h, n)
    q = _f64(t["q"][layer, loop, b, h])
    return score_scale(w) * LOG2E * (keys @ q)


def value_rows(w: Workload, t: dict, layer: int, loop: int, b: int, h: int, n: int) -> np.ndarray:
    """Rebuilt values V_t (Eq. 3) or the uncompressed cache's value rows, [n][d]."""
    if w.teacher:
        return _f64(t["v_cache"][layer, loop, b, h, :n])
    variant = "per_head" if w.variant == "per_head" else "2d"
    hc = h if variant == "per_head" else 0
    mu = O._mu_slice(_f64(t["mu_v"][layer]), variant, loop, h, w.H, w.d)
    return O.reconstruct(_f64(t["c_v"][layer, b, hc, :n]), _f64(t["w_up_v"][layer, loop, h]), mu)
