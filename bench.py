"""Throughput of the LLA latent-store decode path on one MI355X.

One step = one decode step of a looped model (T loops x D layers) over the latent cache
("Looped Latent Attention", Section 7: the latent-store decoder caches only latents and
rebuilds K/V on read; Appendix A "Decoding and caching"):
  1. write the new token's latents for every layer (lla_encode, n_new = 1 per sequence),
  2. decode attention for every (loop, layer) in the model's order, one lla_decode_attn
     call per (loop, layer) with loop_count = 1.
Default workload: 21.3x compression at capacity (T=4, D=24, H=16, d_head=128,
(r_k, r_v) = (16, 32), bfloat16, 768 sequences, context 4096), synthetic seeded data
resident in HBM before the timed region.

Prints one JSON line. ``value`` is decode tokens/s for the whole step (batch / step time).
``roofline`` is for the dominant kernel (the decode call), with algorithmic bytes per call
divided by the average call duration measured with HIP events on the launch stream over
the timed region. ``cpu_baseline`` times the fp64 oracle on a bounded sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


# Sources whose compiled code (or launch plan) a kernel's measured traffic depends on:
# device helpers, launch arguments, split planning, and each call's kernels (host-side
# validation and dispatch in lla_api.cpp do not change what a kernel reads).
_COMMON_SOURCES = ("lla_device.h", "lla_args.h", "lla_plan.h")
KERNEL_SOURCES = {
    "decode": _COMMON_SOURCES + ("decode_rotary_fold.hip", "decode_fold_wide.hip", "decode_lla2d.hip",
                                 "decode_reconstruct.hip", "combine.hip", "rope_table.hip"),
    "absorbed": _COMMON_SOURCES + ("decode_absorbed.hip", "decode_stream.h", "combine.hip"),
    "encode": _COMMON_SOURCES + ("encode.hip",),
    "encode_fused": _COMMON_SOURCES + ("encode_fused.hip",),
    "teacher": _COMMON_SOURCES + ("decode_teacher.hip", "decode_stream.h", "combine.hip"),
    "reconstruct": _COMMON_SOURCES + ("reconstruct.hip", "lla_recon_args.h"),
    "paged": _COMMON_SOURCES + ("decode_rotary_fold.hip", "decode_fold_wide.hip", "decode_lla2d.hip",
                                "decode_reconstruct.hip", "combine.hip", "lla_page_args.h"),
}


# The decode kernels' own sources, by a substring of their kernel names: a summary taken
# on one of them depends on its file only, not on the other decode kernels'.
_DECODE_KERNEL_FILES = {"decode_rotary_fold": "decode_rotary_fold.hip",
                        "decode_fold_wide": "decode_fold_wide.hip",
                        "decode_fold_head": "decode_fold_wide.hip",
                        "decode_lla2d": "decode_lla2d.hip",
                        "decode_reconstruct": "decode_reconstruct.hip"}


def kernel_sources(kind: str, kernel=None) -> tuple:
    """Sources behind a call kind; for the decode calls, when the measured kernel name(s)
    are given, only the decode kernel file(s) those names come from."""
    files = KERNEL_SOURCES[kind]
    if kernel and kind in ("decode", "paged"):
        names = kernel if isinstance(kernel, (list, tuple)) else [kernel]
        used = {f for k, f in _DECODE_KERNEL_FILES.items() if any(k in n for n in names)}
        if used:
            files = tuple(f for f in files if f not in _DECODE_KERNEL_FILES.values() or f in used)
    return files


def kernel_source_hash(kind: str, kernel=None) -> str:
    """Hash of the HIP/C++ sources behind one call kind (a key of KERNEL_SOURCES; with
    `kernel`, the measured decode kernel's sources only) with comments and whitespace
    removed, and of their compile flags: it changes when that call's compiled code or
    launch plan can change, not when a comment or another kernel's sources do."""
    import re
    csrc = os.path.join(ROOT, "latent_decode_attention_lla_amd", "csrc")
    h = hashlib.sha256()
    names = sorted(kernel_sources(kind, kernel))
    files = [os.path.join(csrc, f) for f in names]
    from latent_decode_attention_lla_amd import build as _build  # the compile flags
    # flags with include paths relative to the repository, so the hash does not depend on
    # where the checkout lives
    root = os.path.realpath(ROOT)
    flags = [os.path.relpath(os.path.realpath(f), root) if os.path.isabs(f) else f
             for f in _build.HIP_FLAGS]
    file_flags = sorted((f, v) for f, v in _build.FILE_FLAGS.items() if f in names)
    h.update(repr((_build.ARCH, flags, file_flags)).encode())
    for path in files:
        f = os.path.basename(path)
        with open(path) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        src = re.sub(r"\s+", " ", src)
        h.update(f.encode() + src.encode())
    return h.hexdigest()[:16]


def _profile_stem(kind: str, workload: str, path: str) -> str:
    """File stem of a call's committed summaries; a forced decode path gets its own."""
    return f"{kind}_{workload}" + ("" if path == "auto" else f"_{path}")


def traffic_file(kind: str, workload: str, path: str = "auto") -> str:
    return os.path.join(ROOT, "profiles", f"{_profile_stem(kind, workload, path)}_traffic.json")


def measured_traffic(kind: str, workload: str, path: str):
    """HBM bytes per call from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, or
    None when there is none or the call's sources have changed since it was taken."""
    try:
        with open(traffic_file(kind, workload, path)) as f:
            tr = json.load(f)
    except (OSError, ValueError):
        return None
    if tr.get("kernel_source_hash") == kernel_source_hash(kind, tr.get("kernel")) and tr.get("path") == path \
            and tr.get("workload") == workload:
        return tr.get("hbm_bytes_per_launch")
    return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="capacity_21x")
    p.add_argument("--path", default="auto", choices=["auto", "reconstruct", "rotary_fold"])
    p.add_argument("--splits", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-reference-calls", action="store_true",
                   help="skip timing the full-RoPE paths beside the absorbed decode")
    p.add_argument("--cpu-sample-seqs", type=int, default=1)
    p.add_argument("--cpu-sample-tokens", type=int, default=16384,
                   help="prompt tokens of the oracle's sample for the streamed-prefill workload")
    p.add_argument("--prefill-encode", default="fused", choices=["fused", "captures"],
                   help="streamed-prefill workload: pass 1 through the projection-fused encode "
                        "(loop by loop, no per-loop K/V stored) or lla_encode of stored captures")
    p.add_argument("--ceiling-gib", type=float, default=0.0,
                   help="time plain streaming passes over buffers of this size (read-only, "
                        "copy, 4:1 and 1:4 read:write; per-wave chunks through LDS, registers "
                        "or both) and print their HBM rates instead")
    p.add_argument("--copy-calibration-gib", type=float, default=0.0,
                   help="only run a plain device copy of this size (for counter scaling)")
    return p.parse_args()


def stream_ceilings(gib: float):
    """HBM ceilings on this device from plain 16-byte-per-lane streaming passes
    (include/lla_stream.h) over `gib` GiB of reads (the 1:4 mix: of writes): the rates the
    decode (read-only), encode (4:1) and reconstruction (1:4) kernels compare against."""
    import torch
    from latent_decode_attention_lla_amd import lla
    lla.load()
    n = int(gib * 2**30) // 16
    n -= n % (64 * 4 * 512 * 16)  # whole 16-block runs of 1 KiB per wave at 512 workgroups
    src = torch.empty(n * 16, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n * 16, dtype=torch.uint8, device="cuda")
    src.random_(0, 255)
    # (mode, vectors per pass, bytes read, bytes written)
    modes = {"read": (0, n, n * 16, 0), "copy_1to1": (1, n // 2, n // 2 * 16, n // 2 * 16),
             "mix_4to1": (2, n // 4, n * 16, n // 4 * 16), "mix_1to4": (3, n // 4, n // 4 * 16, n * 16)}
    # per-wave contiguous chunks at 2 workgroups of 4 waves per CU: the same reads through
    # direct-to-LDS loads, through registers, and half through each
    wave_modes = {"read_wave_lds": (4, n, n * 16, 0), "read_wave_regs": (5, n, n * 16, 0),
                  "read_wave_mixed": (6, n, n * 16, 0)}
    # the narrow fold's latent-row pattern (mode 7: per wave one key and one value row plane
    # in 16-row tiles, 8 in flight) at 16 and 32 waves per CU
    n7 = {wg: n - n % (96 * 4 * wg * 8) for wg in (1024, 2048)}
    row_modes = {f"read_rows_fold_{wg // 64}w": (wg, (7, n7[wg], n7[wg] * 16, 0)) for wg in n7}
    res = {}
    runs = [(wg, m) for wg in (1024, 2048, 4096, 8192) for m in modes.items()]
    runs += [(512, m) for m in wave_modes.items()]
    runs += [(wg, (name, m)) for name, (wg, m) in row_modes.items()]
    for wg, (name, (mode, nv, rd, wr)) in runs:
        for _ in range(2):
            lla.lla_stream_ceiling(mode, src, dst, nv, wg)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        reps = 10
        ev[0].record()
        for _ in range(reps):
            lla.lla_stream_ceiling(mode, src, dst, nv, wg)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        tbs = (rd + wr) / (ms * 1e-3) / 1e12
        best = res.get(name)
        if best is None or tbs > best["tb_per_s"]:
            res[name] = {"tb_per_s": round(tbs, 3), "ms": round(ms, 4), "workgroups": wg,
                         "bytes_read": rd, "bytes_written": wr,
                         "frac_of_8tbs": round(tbs / (HBM_PEAK_GBS / 1e3), 4)}
    print(json.dumps({"stream_ceilings": res, "buffer_gib": gib}))


def copy_calibration(gib: float):
    import torch
    n = int(gib * 2**30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "launches": 3}))


def cpu_baseline(w, seqs: int):
    """The fp64 oracle (as it stands) on `seqs` sequences of the same workload: every head,
    layer and loop of one decode step, same shapes and distributions (CPU inputs)."""
    import numpy as np
    from latent_decode_attention_lla_amd.inputs import decode_inputs
    from oracle import lla_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    # the decoupled decode's oracle rebuilds a 32768-token context per (head, loop), and
    # the uncompressed cache of one sequence is 1.6 GB at 24 layers: a few layers are
    # timed and the step scaled by D
    layers = 1 if w.d_rope > 0 else (2 if w.teacher else w.D)
    sw = w.replace(batch=seqs, D=layers)
    if w.teacher:
        from latent_decode_attention_lla_amd.inputs import teacher_inputs
        t = teacher_inputs(sw, seed=12345, device="cpu")
    elif w.paged:
        from latent_decode_attention_lla_amd.inputs import paged_decode_inputs
        t = paged_decode_inputs(sw, seed=12345, device="cpu")
    else:
        t = decode_inputs(sw, seed=12345, device="cpu")
    t = {k: v.float().numpy().astype(np.float64) for k, v in t.items()}
    variant = "per_head" if w.variant == "per_head" else "2d"
    t0 = time.perf_counter()
    for loop in range(w.T):
        for layer in range(layers):
            q = t["q"][layer, loop:loop + 1].transpose(1, 2, 0, 3)
            if w.teacher:
                O.decode_teacher(t["k_cache"][layer], t["v_cache"][layer], q, loop)
            elif w.paged and w.d_rope > 0:
                O.decode_absorbed_paged(t["c_k"][layer], t["c_v"][layer], t["k_rope"][layer],
                                        t["block_table"], t["w_up_k"][layer], t["mu_k"][layer],
                                        t["w_up_v"][layer], t["mu_v"][layer], q, w.d_rope, loop,
                                        None, w.n, None, variant)
            elif w.paged:
                O.decode_paged(t["c_k"][layer], t["c_v"][layer], t["block_table"], t["w_up_k"][layer],
                               t["mu_k"][layer], t["w_up_v"][layer], t["mu_v"][layer], q, loop, None,
                               w.n, w.rope_base, None, variant)
            elif w.d_rope > 0:
                O.decode_absorbed(t["c_k"][layer], t["c_v"][layer], t["k_rope"][layer],
                                  t["w_up_k"][layer], t["mu_k"][layer], t["w_up_v"][layer],
                                  t["mu_v"][layer], q, w.d_rope, loop, None, None, variant)
            else:
                O.decode(t["c_k"][layer], t["c_v"][layer], t["w_up_k"][layer], t["mu_k"][layer],
                         t["w_up_v"][layer], t["mu_v"][layer], q, loop, None, w.rope_base, None,
                         variant)
    dt = time.perf_counter() - t0
    step_s = dt * w.D / layers
    scaled = "" if layers == w.D else f", timed on {layers} layer(s) and scaled by {w.D // layers}"
    return {"value": seqs / step_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{seqs} sequence(s) x {w.H} heads x {layers} layer(s) x {w.T} loops at "
                      f"context {w.n} (a decode step for {seqs} of the {w.batch} sequences{scaled}), "
                      f"fp64 NumPy, {dt:.1f} s; host os.cpu_count()={os.cpu_count()}"}


def step_shape(w):
    """(prefill, tokens encoded per sequence, layers) of one step of workload ``w``."""
    prefill = w.name in ("ouro_layer_4x", "encode_heavy")
    if w.teacher:  # the uncompressed cache has no encode
        return False, 0, w.D
    if w.stream_prefill:  # every layer encodes the whole prompt
        return True, w.n, w.D
    return prefill, (w.n if prefill else 1), (1 if prefill else w.D)


def algorithmic(w, kind: str, L: int = 1, n_new: int = 0):
    """Algorithmic HBM bytes and matrix-core flops of one call.
    decode: every cached latent read once, q and out, one loop's W_up and mu slices;
            flops are those of rebuilding the keys, 2 r_k d per (token, head) (LLA-2D adds
            the shared-latent value accumulation, 2 r_v per (token, head)).
    encode: x_k and x_v read once, latents written once, W_down and mu read once;
            flops 2 T d_in (r_k + r_v) per (token, latent head)."""
    es = 2 if w.dtype == "bf16" else 4
    if kind == "encode_fused":
        # one (loop, layer) call, averaged over the T loops of a layer: the hidden states
        # and both projections read once, the loop's W_down rows and mu slice, the float32
        # accumulator written by loop 0, read and written by the middle loops and read by
        # the last, which writes the latents; flops of both projections and the loop's
        # share of Eq. 2, 2 d_in (r_k + r_v) per (token, latent head)
        tok = w.batch * n_new
        ent = tok * w.Hc * (w.r_k + w.r_v)
        nbytes = (tok * w.d_model * es + 2 * w.d_model * w.H * w.d * es
                  + w.Hc * (w.r_k + w.r_v) * w.d_in * es + 2 * w.Hc * w.d_in * es
                  + (ent * 8 * (w.T - 1) + ent * es) / w.T)
        flops = 2.0 * tok * w.d_model * w.H * w.d * 2 + 2.0 * tok * w.Hc * w.d_in * (w.r_k + w.r_v)
        return nbytes, flops
    if kind == "reconstruct":
        # every latent of the range read once, L loops of keys and values written once,
        # W_up and mu slices; flops of rebuilding both axes on the matrix cores
        tok = w.batch * n_new
        nbytes = (tok * w.Hc * (w.r_k + w.r_v) * es + 2 * L * tok * w.H * w.d * es
                  + L * w.H * w.d * (w.r_k + w.r_v) * es + 2 * L * w.H * w.d * es)
        return nbytes, 2.0 * L * tok * w.H * w.d * (w.r_k + w.r_v)
    if kind == "decode" and w.teacher:
        # uncompressed decode: one loop's key and value rows read once, q and out;
        # 4 d flop per (token, head) for the score and the weighted value
        nbytes = 2 * w.batch * w.H * w.n * w.d * es + 2 * w.batch * w.H * L * w.d * 4
        return nbytes, 4.0 * w.batch * w.H * w.n * L * w.d
    if kind == "decode":
        tok = w.batch * w.Hc * w.n
        nbytes = (tok * (w.r_k + w.r_v) * es + 2 * w.batch * w.H * L * w.d * 4
                  + L * w.H * w.d * (w.r_k + w.r_v) * es + 2 * L * w.H * w.d * es)
        if w.d_rope > 0:
            # decoupled decode: the rotary keys are read too; scores and values on the
            # vector ALU, 2 (r_k + d_rope + r_v) flop per (token, head)
            nbytes += w.batch * w.H * w.n * w.d_rope * es
            return nbytes, 2.0 * w.batch * w.H * w.n * L * (w.r_k + w.d_rope + w.r_v)
        if w.variant == "per_head":
            flops = 2.0 * w.batch * w.H * w.n * L * w.r_k * w.d
        else:
            flops = 2.0 * w.batch * w.n * w.H * L * (w.r_k * w.d + w.r_v)
        return nbytes, flops
    K = w.T * w.d_in
    toks = w.batch * n_new * w.Hc
    nbytes = (2 * toks * K * es + toks * (w.r_k + w.r_v) * es + w.Hc * (w.r_k + w.r_v) * K * es
              + 2 * w.Hc * K * es)
    return nbytes, 2.0 * toks * K * (w.r_k + w.r_v)


def cpu_baseline_prefill(w, tokens: int):
    """The fp64 oracle's encode (Eq. 2) and materialised reconstruction of `tokens`
    prompt tokens of one layer (every head, all T loops), scaled to the whole prompt and
    all D layers."""
    import numpy as np
    from oracle import lla_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    rng = np.random.default_rng(12345)
    K = w.T * w.d_in
    x = rng.standard_normal((tokens, w.Hc, K))
    wd = [rng.standard_normal((w.Hc, K, r)) / math.sqrt(K) for r in (w.r_k, w.r_v)]
    mu = [rng.standard_normal((w.Hc, K)) * math.sqrt(0.1) for _ in range(2)]
    wu = [rng.standard_normal((w.T, w.H, w.d, r)) / math.sqrt(r) for r in (w.r_k, w.r_v)]
    t0 = time.perf_counter()
    c = []
    for axis in range(2):
        c.append(np.stack([O.encode(x[:, hc], mu[axis][hc], wd[axis][hc]) for hc in range(w.Hc)])[None])
    O.reconstruct_cache(c[0], c[1], wu[0], mu[0], wu[1], mu[1], 0, w.T, 0, tokens, w.rope_base,
                        "per_head" if w.variant == "per_head" else "2d")
    dt = time.perf_counter() - t0
    scale = (w.batch * w.n / tokens) * w.D
    return {"value": w.batch * w.n / (dt * scale), "unit": "prompt tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{tokens} prompt tokens x {w.H} heads x 1 layer (encode of both axes, then "
                      f"K/V rebuilt for all {w.T} loops), fp64 NumPy, {dt:.1f} s, scaled by "
                      f"{scale:g} to the {w.n}-token prompt and {w.D} layers; host "
                      f"os.cpu_count()={os.cpu_count()}"}


def cpu_baseline_prefill_fused(w, tokens: int):
    """The fp64 oracle's projection-fused encode (all T loops, both axes) and materialised
    reconstruction of `tokens` prompt tokens of one layer, scaled to the whole prompt and
    all D layers."""
    import numpy as np
    from oracle import lla_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    rng = np.random.default_rng(12345)
    K = w.T * w.d_in
    variant = "per_head" if w.variant == "per_head" else "2d"
    h = rng.standard_normal((w.T, tokens, w.d_model))
    wp = [rng.standard_normal((w.d_model, w.H * w.d)) / math.sqrt(w.d_model) for _ in range(2)]
    wd = [rng.standard_normal((w.Hc, K, r)) / math.sqrt(K) for r in (w.r_k, w.r_v)]
    mu = [rng.standard_normal((w.Hc, K)) * math.sqrt(0.1) for _ in range(2)]
    wu = [rng.standard_normal((w.T, w.H, w.d, r)) / math.sqrt(r) for r in (w.r_k, w.r_v)]
    t0 = time.perf_counter()
    c = [np.transpose(O.encode_fused(h, wp[a], mu[a], wd[a], w.H, w.d, variant), (1, 0, 2))[None]
         for a in range(2)]
    O.reconstruct_cache(c[0], c[1], wu[0], mu[0], wu[1], mu[1], 0, w.T, 0, tokens, w.rope_base,
                        variant)
    dt = time.perf_counter() - t0
    scale = (w.batch * w.n / tokens) * w.D
    return {"value": w.batch * w.n / (dt * scale), "unit": "prompt tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{tokens} prompt tokens x {w.H} heads x 1 layer (projection-fused encode of "
                      f"both axes over {w.T} loops from hidden size {w.d_model}, then K/V rebuilt "
                      f"for all {w.T} loops), fp64 NumPy, {dt:.1f} s, scaled by {scale:g} to the "
                      f"{w.n}-token prompt and {w.D} layers; host os.cpu_count()={os.cpu_count()}"}


def prefill_working_sets(w, n: int, acc_bytes_layer: int):
    """GiB held by the prefill's cache-side buffers at pass 1's peak (when the last loop
    starts): the latent cache, the pass-1 state, and one layer's rebuilt K/V of pass 2.
    Pass 1 of a looped stack runs every layer at every loop, so a layer's per-loop K/V
    captures (or its accumulator) live until the last loop reaches that layer."""
    es = 2 if w.dtype == "bf16" else 4
    lat = w.D * w.batch * w.Hc * n * (w.r_k + w.r_v) * es
    kv = 2 * w.T * w.batch * w.H * n * w.d * es
    cap = w.D * (w.T - 1) * 2 * w.batch * n * w.H * w.d  # elements of loops 0 .. T-2
    acc = w.D * acc_bytes_layer
    g = 2.0 ** 30
    return {"latents": round(lat / g, 2), "rebuilt_kv_one_layer": round(kv / g, 2),
            "pass1_fused_accumulators": round(acc / g, 2),
            "pass1_captures_bf16": round(cap * 2 / g, 2),
            "pass1_captures_f32": round(cap * 4 / g, 2),
            "fused_total": round((lat + acc + kv) / g, 2),
            "captures_bf16_total": round((lat + cap * 2 + kv) / g, 2),
            "one_shot_f32_total": round((lat + w.D * w.T * 2 * w.batch * n * w.H * w.d * 4
                                         + w.D * kv) / g, 2)}


def main_stream_prefill_fused(args, w):
    """One step = the two-pass prefill of a prompt with the projection-fused encode.
    Pass 1 runs the looped stack loop by loop: at loop t, every layer's key and value
    projections of that loop's hidden states go through lla_encode_fused, which adds the
    loop's share of Eq. 2 to the layer's float32 accumulator (no per-loop K/V is stored);
    loop T-1 writes the latents. Pass 2, layer by layer, rebuilds the layer's K/V for all
    loops with lla_reconstruct (its buffer is reused). One seeded hidden-state buffer
    stands in for every (loop, layer) input."""
    import torch
    from latent_decode_attention_lla_amd import lla
    from latent_decode_attention_lla_amd.harness import DeviceLatentStore
    from latent_decode_attention_lla_amd.inputs import fused_encode_inputs, gaussian_encode_codec
    dev = torch.device("cuda:0")
    n = w.n
    st = DeviceLatentStore(w, seed=3, device=dev, with_q=False)
    ct = gaussian_encode_codec(w, seed=4, device=dev)
    st.t.update(ct)
    st.codec = lla.make_codec(ct["w_down_k_t"], ct["mu_k"], st.t["w_up_k"], ct["w_down_v_t"],
                              ct["mu_v"], st.t["w_up_v"], st.rope)
    h, w_k, w_v = fused_encode_inputs(w.replace(T=1), n, w.d_model, seed=5, device=dev)
    h = h[0, 0]
    proj = lla.make_proj(w_k, w_v, w.d_model)
    acc_bytes = lla.lla_encode_fused_acc_bytes(st.dims, n)
    ws = prefill_working_sets(w, n, acc_bytes)
    print(f"[bench] allocating {w.name}: latents {ws['latents']} GiB, accumulators "
          f"{ws['pass1_fused_accumulators']} GiB", file=sys.stderr, flush=True)
    acc = torch.empty(w.D, acc_bytes // 4, dtype=torch.float32, device=dev)
    kv = [torch.empty(w.T, w.batch, w.H, n, w.d, dtype=w.torch_dtype, device=dev) for _ in range(2)]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    steps = max(args.steps, 1)
    ev = {"encode_fused": [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                           for _ in range(w.T * w.D * steps)],
          "reconstruct": [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                          for _ in range(w.D * steps)]}

    def step(record):
        for t in range(w.T):
            for layer in range(w.D):
                e = None if record is None else ev["encode_fused"][(record * w.T + t) * w.D + layer]
                if e is not None:
                    e[0].record(stream)
                lla.lla_encode_fused(st.dims, st.codec, proj, st.cache, layer, t, h, 0, n, acc[layer],
                                     acc_bytes, sp)
                if e is not None:
                    e[1].record(stream)
        for layer in range(w.D):
            e = None if record is None else ev["reconstruct"][record * w.D + layer]
            if e is not None:
                e[0].record(stream)
            lla.lla_reconstruct(st.dims, st.codec, st.cache, layer, 0, w.T, 0, n, kv[0], kv[1], sp)
            if e is not None:
                e[1].record(stream)

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for s_ in range(args.steps):
        step(s_)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    calls = {}
    counts = {"encode_fused": w.T * w.D, "reconstruct": w.D}
    for kind in ("encode_fused", "reconstruct"):
        xs = sorted(a.elapsed_time(b) for a, b in ev[kind][:counts[kind] * args.steps])
        ms = sum(xs) / len(xs)
        nb, fl = (algorithmic(w, "encode_fused", n_new=n) if kind == "encode_fused"
                  else algorithmic(w, "reconstruct", L=w.T, n_new=n))
        calls[kind] = {"avg_ms": round(ms, 5), "median_ms": round(xs[len(xs) // 2], 5),
                       "per_step": counts[kind], "algorithmic_bytes": nb, "algorithmic_flops": fl,
                       "roofline": roofline(nb, fl, ms, measured_traffic(kind, w.name, "auto"),
                                            measured_counters(kind, w.name, "auto"))}
    dominant = max(calls, key=lambda k: calls[k]["avg_ms"] * calls[k]["per_step"])
    cpu = None if args.no_cpu_baseline else cpu_baseline_prefill_fused(w, args.cpu_sample_tokens)
    res = {
        "metric": "LLA two-pass prefill with the projection-fused encode, prompt tokens/s (pass 1: "
                  "per loop and layer, K/V projections fused with the latent accumulation; pass 2: "
                  "per layer, K/V rebuilt for all loops), 1 GPU",
        "value": round(w.batch * n / (ms_step * 1e-3), 1),
        "unit": "prompt tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian hidden states, projections and codec maps; no model "
                "weights)",
        "config": {"workload": w.name, "T": w.T, "D": w.D, "H": w.H, "d_head": w.d, "r_k": w.r_k,
                   "r_v": w.r_v, "variant": w.variant, "batch": w.batch, "prompt": n,
                   "d_model": w.d_model, "prefill_encode": "fused",
                   "step": f"{w.T} loops x {w.D} layers of lla_encode_fused ({n} tokens), then "
                           f"{w.D} x lla_reconstruct of {w.T} loops",
                   "working_set_gib": ws,
                   "device_peak_allocated_gib": round(torch.cuda.max_memory_allocated(dev) / 2**30, 2)},
        "roofline": calls[dominant]["roofline"],
        "roofline_kernel": "lla_" + dominant,
        "cpu_baseline": cpu,
        "encode_fused_call": calls["encode_fused"],
        "reconstruct_call": calls["reconstruct"],
        "wall_s_timed": round(wall, 3),
        "kernel_source_hash": {k: kernel_source_hash(k) for k in KERNEL_SOURCES},
    }
    print(json.dumps(res))


def main_stream_prefill(args, w):
    """One step = the streamed two-pass prefill of a prompt: for every layer in turn,
    lla_encode of the prompt's per-loop K/V (the capture buffer is reused by every layer),
    then lla_reconstruct of that layer's K/V for all T loops (the second pass's input; its
    buffer is reused too). Peak memory is the latent cache plus one layer's captures and
    one layer's rebuilt K/V."""
    import torch
    from latent_decode_attention_lla_amd import lla
    from latent_decode_attention_lla_amd.harness import DeviceLatentStore
    dev = torch.device("cuda:0")
    es = 2 if w.dtype == "bf16" else 4
    n = w.n
    print(f"[bench] allocating {w.name}: latents "
          f"{w.D * w.batch * w.Hc * n * (w.r_k + w.r_v) * es / 2**30:.1f} GiB", file=sys.stderr,
          flush=True)
    st = DeviceLatentStore(w, seed=3, device=dev, with_q=False)
    g = torch.Generator(device=dev).manual_seed(4)
    K = w.T * w.d_in
    dt = w.torch_dtype
    st.t["w_down_k_t"] = (torch.randn(w.D, w.Hc, w.r_k, K, generator=g, device=dev) / math.sqrt(K)).to(dt)
    st.t["w_down_v_t"] = (torch.randn(w.D, w.Hc, w.r_v, K, generator=g, device=dev) / math.sqrt(K)).to(dt)
    st.codec = lla.make_codec(st.t["w_down_k_t"], st.t["mu_k"], st.t["w_up_k"], st.t["w_down_v_t"],
                              st.t["mu_v"], st.t["w_up_v"], st.rope)
    x = [torch.randn(w.batch, n, w.Hc, w.T, w.d_in, generator=g, device=dev).to(dt) for _ in range(2)]
    kv = [torch.empty(w.T, w.batch, w.H, n, w.d, dtype=dt, device=dev) for _ in range(2)]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    steps = max(args.steps, 1)
    ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(w.D * steps)] for k in ("encode", "reconstruct")}

    def step(record):
        for layer in range(w.D):
            if record is not None:
                ev["encode"][record * w.D + layer][0].record(stream)
            lla.lla_encode(st.dims, st.codec, st.cache, layer, x[0], x[1], 0, n, sp)
            if record is not None:
                ev["encode"][record * w.D + layer][1].record(stream)
                ev["reconstruct"][record * w.D + layer][0].record(stream)
            lla.lla_reconstruct(st.dims, st.codec, st.cache, layer, 0, w.T, 0, n, kv[0], kv[1], sp)
            if record is not None:
                ev["reconstruct"][record * w.D + layer][1].record(stream)

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for s_ in range(args.steps):
        step(s_)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    calls = {}
    for kind in ("encode", "reconstruct"):
        xs = sorted(a.elapsed_time(b) for a, b in ev[kind][:w.D * args.steps])
        ms = sum(xs) / len(xs)
        nb, fl = (algorithmic(w, "encode", n_new=n) if kind == "encode"
                  else algorithmic(w, "reconstruct", L=w.T, n_new=n))
        calls[kind] = {"avg_ms": round(ms, 5), "median_ms": round(xs[len(xs) // 2], 5),
                       "algorithmic_bytes": nb, "algorithmic_flops": fl,
                       "roofline": roofline(nb, fl, ms, measured_traffic(kind, w.name, "auto"),
                                            measured_counters(kind, w.name, "auto"))}
    dominant = max(calls, key=lambda k: calls[k]["avg_ms"])
    cpu = None if args.no_cpu_baseline else cpu_baseline_prefill(w, args.cpu_sample_tokens)
    # a looped stack's pass 1 would hold every layer's captures of loops 0 .. T-2; this
    # bench reuses one layer's capture buffer, so it times the encode, not that peak
    ws = prefill_working_sets(w, n, lla.lla_encode_fused_acc_bytes(st.dims, n))
    res = {
        "metric": "LLA streamed two-pass prefill, prompt tokens/s (per layer in turn: encode of "
                  "the prompt's per-loop K/V, then K/V rebuilt for all loops), 1 GPU; HBM GB/s of "
                  "the dominant kernel and fraction of peak",
        "value": round(w.batch * n / (ms_step * 1e-3), 1),
        "unit": "prompt tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian per-loop K/V and codec maps; no model weights)",
        "config": {"workload": w.name, "T": w.T, "D": w.D, "H": w.H, "d_head": w.d, "r_k": w.r_k,
                   "r_v": w.r_v, "variant": w.variant, "batch": w.batch, "prompt": n,
                   "prefill_encode": "captures",
                   "step": f"{w.D} x (lla_encode of {n} tokens, lla_reconstruct of {w.T} loops)",
                   "working_set_gib": ws,
                   "device_peak_allocated_gib": round(torch.cuda.max_memory_allocated(dev) / 2**30, 2)},
        "roofline": calls[dominant]["roofline"],
        "roofline_kernel": "lla_" + dominant,
        "cpu_baseline": cpu,
        "encode_call": calls["encode"],
        "reconstruct_call": calls["reconstruct"],
        "wall_s_timed": round(wall, 3),
        "kernel_source_hash": {k: kernel_source_hash(k) for k in KERNEL_SOURCES},
    }
    print(json.dumps(res))


def counters_file(kind: str, workload: str, path: str = "auto") -> str:
    return os.path.join(ROOT, "profiles", f"{_profile_stem(kind, workload, path)}_counters.json")


def measured_counters(kind: str, workload: str, path: str):
    """Wave-state counters of the call's dominant kernel from the committed rocprofv3 --pmc
    summary (wait and issue-wait fractions, instructions per wave), or None when there is
    none or the call's sources have changed since it was taken."""
    try:
        with open(counters_file(kind, workload, path)) as f:
            ct = json.load(f)
    except (OSError, ValueError):
        return None
    if ct.get("kernel_source_hash") == kernel_source_hash(kind, ct.get("kernel")) and ct.get("path") == path \
            and ct.get("workload") == workload:
        return {k: ct[k] for k in ("kernel", "wave_wait_frac", "wave_issue_wait_frac",
                                   "valu_insts_per_wave", "mfma_insts_per_wave",
                                   "salu_insts_per_wave", "lds_bank_conflict_pct",
                                   "lds_conflicts_per_access", "mfma_busy_frac")
                if k in ct}
    return None


NEAR_ROOF = 0.5  # a call reaching half of a roof's peak is taken as bound by that roof


def roofline(nbytes, flops, ms, traffic=None, counters=None):
    """Both fractions of peak for one call: HBM (algorithmic bytes, and the measured
    traffic when a current summary exists) and bf16 MFMA (algorithmic flops). `bound` is
    the roof the call is closer to, and `frac` is quoted against it. `binding` names what
    limits the call: that roof when the call reaches NEAR_ROOF of it, else "issue" (neither
    HBM nor the matrix cores near their peaks: instruction issue, dependency latency and
    waits bound the call), with the committed wave-state counters as evidence."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    tfs = flops / (ms * 1e-3) / 1e12
    hbm_frac = gbs / HBM_PEAK_GBS
    mfma_frac = tfs / MFMA_BF16_PEAK_TFLOPS
    meas_frac = None if traffic is None else traffic / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    hbm_best = max(hbm_frac, meas_frac or 0.0)
    if mfma_frac > hbm_best:
        r = {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": round(mfma_frac, 4), "traffic": traffic}
    else:
        r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(hbm_frac, 4), "traffic": traffic}
    r["hbm_frac"] = round(hbm_frac, 4)
    r["measured_hbm_frac"] = None if meas_frac is None else round(meas_frac, 4)
    r["mfma_frac"] = round(mfma_frac, 4)
    r["binding"] = r["bound"] if max(hbm_best, mfma_frac) >= NEAR_ROOF else "issue"
    r["counters"] = counters
    return r


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration_gib > 0:
        copy_calibration(args.copy_calibration_gib)
        return
    if args.ceiling_gib > 0:
        stream_ceilings(args.ceiling_gib)
        return

    from latent_decode_attention_lla_amd import lla
    from latent_decode_attention_lla_amd.harness import DeviceLatentStore, DeviceTeacherCache
    from latent_decode_attention_lla_amd.inputs import WORKLOADS

    if not os.path.exists(lla.LIB_PATH):
        from latent_decode_attention_lla_amd import build as _b
        _b.build()
    lla.load()

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if w.stream_prefill and args.prefill_encode == "fused":
        main_stream_prefill_fused(args, w)
        return
    if w.stream_prefill:
        main_stream_prefill(args, w)
        return
    # Step shape: "append" workloads decode over an existing cache after appending one new
    # token per sequence; "prefill" workloads encode a whole prompt of n tokens per
    # sequence for one layer, then take one decode step over all loops of that layer.
    prefill, n_new, layers = step_shape(w)
    pos = 0 if prefill else w.n - 1
    es = 2 if w.dtype == "bf16" else 4
    teacher = w.teacher  # the uncompressed per-loop cache, no codec
    cache_gib = (2 * w.D * w.T * w.batch * w.H * w.n * w.d * es if teacher else
                 w.D * w.batch * w.Hc * w.n * (w.r_k + w.r_v) * es) / 2**30
    print(f"[bench] allocating {args.workload}: {'K/V cache' if teacher else 'latents'} "
          f"{cache_gib:.1f} GiB", file=sys.stderr, flush=True)
    path = {"auto": lla.LLA_PATH_AUTO, "reconstruct": lla.LLA_PATH_RECONSTRUCT,
            "rotary_fold": lla.LLA_PATH_ROTARY_FOLD}[args.path]
    opts = lla.make_opts(args.splits, path)
    absorbed = w.d_rope > 0  # the decoupled-RoPE absorbed decode (one wave per head)
    if teacher:
        st = DeviceTeacherCache(w, seed=3, device=dev)
        x_new = None
    else:
        if w.paged:  # latents in shuffled pages of each layer's pool, a block table per sequence
            from latent_decode_attention_lla_amd.inputs import paged_decode_inputs
            st = DeviceLatentStore(w, seed=3, device=dev, tensors=paged_decode_inputs(w, 3, dev))
            st.block_table = st.t["block_table"]
            st.pages = lla.make_pages(st.block_table, st.block_table.shape[1],
                                      st.t["c_k"].shape[1])
        else:
            st = DeviceLatentStore(w, seed=3, device=dev)
        # Encode-side codec and the finished per-loop K/V to encode for every layer used.
        g = torch.Generator(device=dev).manual_seed(4)
        K = w.T * w.d_in
        dt = w.torch_dtype
        st.t["w_down_k_t"] = (torch.randn(w.D, w.Hc, w.r_k, K, generator=g, device=dev) / math.sqrt(K)).to(dt)
        st.t["w_down_v_t"] = (torch.randn(w.D, w.Hc, w.r_v, K, generator=g, device=dev) / math.sqrt(K)).to(dt)
        st.codec = lla.make_codec(st.t["w_down_k_t"], st.t["mu_k"], st.t["w_up_k"], st.t["w_down_v_t"],
                                  st.t["mu_v"], st.t["w_up_v"], st.rope)
        x_new = [torch.randn(layers, w.batch, n_new, w.Hc, w.T, w.d_in, generator=g, device=dev).to(dt)
                 for _ in range(2)]
    if teacher:
        S = lla.lla_decode_teacher_num_splits(st.dims, w.n, 1, opts)
        ws = st.workspace(w.n, 1, opts)
    elif absorbed:
        # the workspace holds one (max, sum, r_v accumulators) partial per split
        nb = (lla.lla_decode_absorbed_paged_workspace_bytes if w.paged else
              lla.lla_decode_absorbed_workspace_bytes)(st.dims, w.d_rope, w.n, 1, opts)
        S = nb // (w.batch * w.H * (2 + w.r_v) * 4)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
    elif w.paged:
        S = lla.lla_decode_paged_num_splits(st.dims, w.n, 1, opts)
        ws = torch.empty(max(lla.lla_decode_paged_workspace_bytes(st.dims, w.n, 1, opts), 256),
                         dtype=torch.uint8, device=dev)
    else:
        S = lla.lla_decode_num_splits(st.dims, w.n, 1, opts)
        ws = st.workspace(w.n, 1, opts)
    out = torch.empty(w.batch, w.H, 1, w.d, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    n_dec = layers * w.T
    n_enc = 0 if teacher else layers
    steps = max(args.steps, 1)
    ev_dec = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_dec * steps)]
    ev_enc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_enc * steps)]

    def step(record):
        for layer in range(n_enc):
            if record is not None:
                ev_enc[record * n_enc + layer][0].record(stream)
            if w.paged:
                lla.lla_encode_paged(st.dims, st.codec, st.cache, st.pages, layer, x_new[0][layer],
                                     x_new[1][layer], pos, n_new, sp)
            else:
                lla.lla_encode(st.dims, st.codec, st.cache, layer, x_new[0][layer],
                               x_new[1][layer], pos, n_new, sp)
            if record is not None:
                ev_enc[record * n_enc + layer][1].record(stream)
        k = 0
        for loop in range(w.T):
            for layer in range(layers):
                q = st.t["q"][layer, loop]
                if record is not None:
                    ev_dec[record * n_dec + k][0].record(stream)
                if teacher:
                    lla.lla_decode_attn_teacher(st.dims, st.t["k_cache"], st.t["v_cache"], layer, w.n,
                                                None, q, loop, 1, out, ws, ws.numel(), opts, sp)
                elif w.paged and absorbed:
                    lla.lla_decode_attn_absorbed_paged(st.dims, st.codec, st.cache, st.pages,
                                                       st.t["k_rope"], w.d_rope, layer, w.n, None,
                                                       q, loop, 1, out, ws, ws.numel(), opts, sp)
                elif w.paged:
                    lla.lla_decode_attn_paged(st.dims, st.codec, st.cache, st.pages, layer, w.n,
                                              None, q, loop, 1, out, ws, ws.numel(), opts, sp)
                elif absorbed:
                    lla.lla_decode_attn_absorbed(st.dims, st.codec, st.cache, st.t["k_rope"], w.d_rope,
                                                 layer, w.n, None, q, loop, 1, out, ws, ws.numel(),
                                                 opts, sp)
                else:
                    lla.lla_decode_attn(st.dims, st.codec, st.cache, layer, w.n, None, q, loop, 1,
                                        out, ws, ws.numel(), opts, sp)
                if record is not None:
                    ev_dec[record * n_dec + k][1].record(stream)
                k += 1

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        step(s)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps

    def avg(evs):
        xs = sorted(a.elapsed_time(b) for a, b in evs[:len(evs)])
        return sum(xs) / len(xs), xs[len(xs) // 2]

    dec_kind = "teacher" if teacher else ("absorbed" if absorbed else ("paged" if w.paged else "decode"))
    dec_ms, dec_med = avg(ev_dec[:n_dec * args.steps])
    dec_bytes, dec_flops = algorithmic(w, "decode")
    dec_roof = roofline(dec_bytes, dec_flops, dec_ms, measured_traffic(dec_kind, args.workload, args.path),
                        measured_counters(dec_kind, args.workload, args.path))
    if n_enc > 0:
        enc_ms, enc_med = avg(ev_enc[:n_enc * args.steps])
        enc_bytes, enc_flops = algorithmic(w, "encode", n_new=n_new)
        enc_roof = roofline(enc_bytes, enc_flops, enc_ms,
                            measured_traffic("encode", args.workload, args.path),
                            measured_counters("encode", args.workload, args.path))
    dominant = "decode" if n_enc == 0 or dec_ms * n_dec >= enc_ms * n_enc else "encode"

    reference = None
    if absorbed and not args.no_reference_calls:
        # the same call shape on the full-RoPE paths, for the ratio the pages report
        reference = {}
        for name, pth in (("rotary_fold_full_rope", lla.LLA_PATH_AUTO), ("reconstruct", lla.LLA_PATH_RECONSTRUCT)):
            o = lla.make_opts(0, pth)
            q = st.t["q"][0, 0]
            if w.paged:
                wsr = torch.empty(max(lla.lla_decode_paged_workspace_bytes(st.dims, w.n, 1, o), 256),
                                  dtype=torch.uint8, device=dev)
            else:
                wsr = st.workspace(w.n, 1, o)

            def ref_call():
                if w.paged:
                    lla.lla_decode_attn_paged(st.dims, st.codec, st.cache, st.pages, 0, w.n, None,
                                              q, 0, 1, out, wsr, wsr.numel(), o, sp)
                else:
                    lla.lla_decode_attn(st.dims, st.codec, st.cache, 0, w.n, None, q, 0, 1, out,
                                        wsr, wsr.numel(), o, sp)
            for _ in range(2):
                ref_call()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(5):
                ref_call()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 5
            reference[name] = {"avg_ms": round(ms, 5), "absorbed_speedup": round(ms / dec_ms, 3)}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_sample_seqs)

    value = w.batch / (ms_step * 1e-3)
    step_desc = (f"encode a {n_new}-token prompt per sequence for one layer, then {w.T} decode calls"
                 if prefill else
                 f"encode the new token for {w.D} layers, then {w.D} x {w.T} decode calls")
    if w.paged:
        step_desc += " over a paged cache (16-token pages in a random order, block table per sequence)"
    if teacher:
        step_desc = (f"{w.D} x {w.T} uncompressed decode calls over the per-loop K/V cache (the "
                     f"new token's K/V rows, {w.batch * w.T * w.H * w.d * 2 * es // 1024} KiB per "
                     f"layer, are not written)")
    if absorbed:
        step_desc += f" (decoupled-RoPE absorbed decode, rotary branch {w.d_rope} wide)"
    res = {
        "metric": ("uncompressed (teacher) decode tokens/s (D layers x T loops of attention over "
                   "the per-loop K/V cache), 1 GPU, the reference for the latent store's ratio"
                   if teacher else
                   "LLA decode tokens/s (one decode step of the looped model over the latent "
                   "cache: the new token's encode plus D layers x T loops of latent-store "
                   "attention), 1 GPU; HBM GB/s or MFMA TFLOP/s of the dominant kernel and "
                   "fraction of peak"),
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian latents, codec maps and queries; no model weights)",
        "config": {"workload": w.name, "T": w.T, "D": w.D, "H": w.H, "d_head": w.d,
                   **({"cache": "uncompressed per-loop K/V"} if teacher else
                      {"r_k": w.r_k, "r_v": w.r_v, "variant": w.variant}),
                   "batch": w.batch, "context": w.n,
                   "path": args.path, "splits": S, "step": step_desc,
                   "decode_calls_per_step": n_dec, "encode_calls_per_step": n_enc,
                   **({"d_rope": w.d_rope} if absorbed else {})},
        "roofline": dec_roof if dominant == "decode" else enc_roof,
        "roofline_kernel": ("lla_decode_attn_absorbed_paged" if absorbed and w.paged else
                            {"teacher": "lla_decode_attn_teacher", "absorbed": "lla_decode_attn_absorbed",
                             "paged": "lla_decode_attn_paged", "decode": "lla_decode_attn"}[dec_kind])
                           if dominant == "decode" else "lla_encode",
        "cpu_baseline": cpu,
        "decode_call": {"avg_ms": round(dec_ms, 5), "median_ms": round(dec_med, 5),
                        "algorithmic_bytes": dec_bytes, "algorithmic_flops": dec_flops,
                        "loop_step_tokens_per_s": round(w.batch / (dec_ms * 1e-3), 1),
                        "roofline": dec_roof},
        "encode_call": None if n_enc == 0 else
                       {"avg_ms": round(enc_ms, 5), "median_ms": round(enc_med, 5),
                        "tokens": w.batch * n_new, "algorithmic_bytes": enc_bytes,
                        "algorithmic_flops": enc_flops,
                        "tokens_per_s": round(w.batch * n_new / (enc_ms * 1e-3), 1),
                        "roofline": enc_roof},
        **({"reference_calls": reference} if reference is not None else {}),
        "wall_s_timed": round(wall, 3),
        "kernel_source_hash": {k: kernel_source_hash(k) for k in KERNEL_SOURCES},
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
