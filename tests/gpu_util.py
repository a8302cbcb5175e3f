"""Helpers shared by the GPU parity tests: build-if-missing, host copies in float64, the
oracle on a sample of sequences, and error measures."""

from __future__ import annotations

import math
import os
import sys

import numpy as np
import torch

from latent_decode_attention_lla_amd import lla
from oracle import lla_oracle as O

BF16_TOL = 2e-2   # decode outputs from bfloat16-stored latents and weights
F32_TOL = 1e-5    # decode outputs from float32 latents and weights


def ensure_built():
    if not os.path.exists(lla.LIB_PATH):
        from latent_decode_attention_lla_amd import build
        build.build()
    lla.load()


def announce(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def oracle_scale(w):
    """The score scale a workload asks for (None: the oracle's default 1/sqrt(d))."""
    return None if w.scale == 0.0 else float(w.scale)


def oracle_decode(store, layer: int, loop_begin: int, loop_count: int, seqs, n_ctx: int,
                  ctx_lens=None, q=None):
    """fp64 oracle on sequences ``seqs`` of a DeviceLatentStore's cache (stored values)."""
    t = store.t
    w = store.w
    idx = torch.as_tensor(list(seqs), device=t["c_k"].device)
    ck = f64(t["c_k"][layer].index_select(0, idx)[:, :, :n_ctx])
    cv = f64(t["c_v"][layer].index_select(0, idx)[:, :, :n_ctx])
    if q is None:
        qq = t["q"][layer, loop_begin:loop_begin + loop_count].permute(1, 2, 0, 3)
    else:
        qq = q
    qq = f64(qq.index_select(0, idx))
    lens = None if ctx_lens is None else [int(ctx_lens[i]) for i in seqs]
    return O.decode(ck, cv, f64(t["w_up_k"][layer]), f64(t["mu_k"][layer]), f64(t["w_up_v"][layer]),
                    f64(t["mu_v"][layer]), qq, loop_begin, lens, w.rope_base, oracle_scale(w),
                    "per_head" if w.variant == "per_head" else "2d")


def oracle_decode_absorbed(store, layer: int, loop_begin: int, loop_count: int, seqs, n_ctx: int,
                           ctx_lens=None, q=None):
    """fp64 oracle of the decoupled (absorbed) decode on sequences ``seqs``."""
    t = store.t
    w = store.w
    idx = torch.as_tensor(list(seqs), device=t["c_k"].device)
    ck = f64(t["c_k"][layer].index_select(0, idx)[:, :, :n_ctx])
    cv = f64(t["c_v"][layer].index_select(0, idx)[:, :, :n_ctx])
    kr = f64(t["k_rope"][layer].index_select(0, idx)[:, :, :n_ctx])
    qq = t["q"][layer, loop_begin:loop_begin + loop_count].permute(1, 2, 0, 3) if q is None else q
    qq = f64(qq.index_select(0, idx))
    lens = None if ctx_lens is None else [int(ctx_lens[i]) for i in seqs]
    return O.decode_absorbed(ck, cv, kr, f64(t["w_up_k"][layer]), f64(t["mu_k"][layer]),
                             f64(t["w_up_v"][layer]), f64(t["mu_v"][layer]), qq, w.d_rope,
                             loop_begin, lens, oracle_scale(w),
                             "per_head" if w.variant == "per_head" else "2d")


def oracle_decode_teacher(cache, layer: int, loop_begin: int, loop_count: int, seqs, n_ctx: int,
                          ctx_lens=None, q=None, heads=None):
    """fp64 oracle of the uncompressed decode on sequences ``seqs`` (and ``heads``, all by
    default) of a DeviceTeacherCache. Returns [len(seqs)][len(heads)][loop_count][d]."""
    t = cache.t
    dev = t["k_cache"].device
    idx = torch.as_tensor(list(seqs), device=dev)
    hs = torch.as_tensor(list(range(cache.w.H)) if heads is None else list(heads), device=dev)
    kc = t["k_cache"][layer].index_select(1, idx).index_select(2, hs)[:, :, :, :n_ctx]
    vc = t["v_cache"][layer].index_select(1, idx).index_select(2, hs)[:, :, :, :n_ctx]
    qq = t["q"][layer, loop_begin:loop_begin + loop_count].permute(1, 2, 0, 3) if q is None else q
    qq = qq.index_select(0, idx).index_select(1, hs)
    lens = None if ctx_lens is None else [int(ctx_lens[i]) for i in seqs]
    return O.decode_teacher(f64(kc), f64(vc), f64(qq), loop_begin, lens, oracle_scale(cache.w))


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |x| (8 significant bits); tiny for x == 0."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 7), 2.0 ** -133)


def seed_everything(seed: int):
    torch.manual_seed(seed)
    np.random.seed(seed)
    return seed


def rel_note(err: float, tol: float) -> str:
    return f"max-abs {err:.3e} (tolerance {tol:.0e}, {err / tol:.1%} of it)" if tol > 0 else f"{err:.3e}"


__all__ = ["BF16_TOL", "F32_TOL", "ensure_built", "announce", "f64", "oracle_decode",
           "oracle_decode_absorbed", "oracle_decode_teacher", "max_abs",
           "bf16_ulp", "seed_everything", "rel_note", "math"]
