"""GPU parity of lla_decode_attn_teacher (decode over the uncompressed loop-indexed cache
that "Looped Latent Attention" compresses: Section 3 "Teacher cache", Table 5's teacher
column) against the fp64 oracle, through the C ABI. Small cases are checked on every
output; the full-size launch (Ouro-1.4B geometry, batch 32 at context 4096, all 24
layers resident) on a sample of sequences."""

import numpy as np
import pytest
import torch

from latent_decode_attention_lla_amd import lla
from latent_decode_attention_lla_amd.harness import DeviceTeacherCache
from latent_decode_attention_lla_amd.inputs import WORKLOADS
from tests.gpu_util import (BF16_TOL, F32_TOL, announce, ensure_built, f64, max_abs,
                            oracle_decode_teacher, rel_note)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def _w(**kw):
    return WORKLOADS["teacher_4k"].replace(**kw)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_f32_every_output(d, splits):
    w = _w(D=2, H=2, d=d, batch=2, n=200, dtype="f32")
    tc = DeviceTeacherCache(w, seed=41)
    for layer in (0, 1):
        out = tc.decode(layer, 0, 4, opts=lla.make_opts(splits))
        ref = oracle_decode_teacher(tc, layer, 0, 4, range(w.batch), w.n)
        err = max_abs(f64(out), ref)
        announce(f"teacher f32 d={d} splits={splits} layer={layer}: {rel_note(err, F32_TOL)}")
        assert err <= F32_TOL


@pytest.mark.parametrize("d,batch,n,splits", [
    (128, 3, 517, 0),
    (128, 3, 517, 5),
    (128, 2, 1, 0),
    (128, 1, 64, 1),
    (128, 2, 2049, 0),
    (64, 3, 300, 0),
    (64, 2, 1000, 7),
])
def test_bf16_every_output(d, batch, n, splits):
    w = _w(D=2, H=4, d=d, batch=batch, n=n)
    announce(f"teacher bf16 d={d} B={batch} n={n} splits={splits}")
    tc = DeviceTeacherCache(w, seed=42)
    for layer, lb, lc in ((0, 0, 4), (1, 1, 2), (1, 3, 1)):
        out = tc.decode(layer, lb, lc, opts=lla.make_opts(splits))
        ref = oracle_decode_teacher(tc, layer, lb, lc, range(batch), n)
        err = max_abs(f64(out), ref)
        announce(f"  layer {layer} loops {lb}..{lb + lc - 1}: {rel_note(err, BF16_TOL)}")
        assert err <= BF16_TOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_contexts_and_poisoned_tail(dtype):
    """Per-sequence lengths over rows that hold NaN past each length, in keys and values
    of every loop: no kernel may read them. An empty context gives zeros."""
    w = _w(D=1, H=2, batch=4, n=160, dtype=dtype)
    tc = DeviceTeacherCache(w, seed=43, n_alloc=192)
    lens = [160, 77, 1, 0]
    for b, n_b in enumerate(lens):
        for key in ("k_cache", "v_cache"):
            tc.t[key][0, :, b, :, n_b:] = float("nan")
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    tol = F32_TOL if dtype == "f32" else BF16_TOL
    for splits in (0, 1, 3):
        out = tc.decode(0, 0, 4, n_ctx=160, ctx_lens=ctx, opts=lla.make_opts(splits))
        got = f64(out)
        assert np.isfinite(got).all()
        assert np.all(got[3] == 0.0)
        ref = oracle_decode_teacher(tc, 0, 0, 4, range(3), 160, ctx_lens=lens)
        err = max_abs(got[:3], ref)
        announce(f"teacher ragged {dtype} splits={splits}: {rel_note(err, tol)}")
        assert err <= tol


def test_empty_context_gives_zeros():
    w = _w(D=1, H=2, batch=2, n=64)
    tc = DeviceTeacherCache(w, seed=44)
    out = tc.decode(0, 0, 4, n_ctx=0)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_teacher_4k_full_launch_sampled():
    """Batch 32 at context 4096 with every layer's keys and values resident (the whole
    uncompressed cache, about 103 GB), one (layer, loop) per call as the bench times it;
    sampled sequences of the first and last layer against the oracle."""
    w = _w()
    announce("teacher_4k full cache, B=32 n=4096 D=24")
    tc = DeviceTeacherCache(w, seed=45)
    for layer, loop in ((0, 0), (23, 3)):
        out = tc.decode(layer, loop, 1)
        torch.cuda.synchronize()
        seqs = [0, 17, 31]
        ref = oracle_decode_teacher(tc, layer, loop, 1, seqs, w.n)
        err = max_abs(f64(out[seqs]), ref)
        announce(f"  layer {layer} loop {loop}: {rel_note(err, BF16_TOL)}")
        assert err <= BF16_TOL
        assert torch.isfinite(out).all()
    del tc
    torch.cuda.empty_cache()


def test_unsupported_and_invalid_arguments():
    w = _w(D=1, H=2, batch=1, n=32)
    tc = DeviceTeacherCache(w, seed=46)
    assert lla.lla_decode_teacher_supported(tc.dims)
    out = torch.empty(1, w.H, 1, w.d, device="cuda")
    q = tc.t["q"][0, 0]
    kc, vc = tc.t["k_cache"], tc.t["v_cache"]
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")

    def call(dims=tc.dims, k=kc, layer=0, n_ctx=w.n, lb=0, lc=1, o=out, wsb=ws.numel(), opts=None):
        return lla.lla_decode_attn_teacher_status(dims, k, vc, layer, n_ctx, None, q, lb, lc, o,
                                                  ws, wsb, opts)

    assert call() == lla.LLA_OK
    d96 = lla.make_dims(w.T, w.D, w.H, 96, 0, 0, 1, w.n, lla.LLA_PER_HEAD, lla.LLA_BF16,
                        10000.0, 0.0)
    assert not lla.lla_decode_teacher_supported(d96)
    assert call(dims=d96) == lla.LLA_ERR_UNSUPPORTED
    assert call(k=kc.data_ptr() + 2) == lla.LLA_ERR_INVALID_ARG
    assert call(k=0) == lla.LLA_ERR_INVALID_ARG
    assert call(layer=1) == lla.LLA_ERR_INVALID_ARG
    assert call(n_ctx=w.n + 1) == lla.LLA_ERR_INVALID_ARG
    assert call(lb=3, lc=2) == lla.LLA_ERR_INVALID_ARG
    forced = lla.make_opts(2)
    need = lla.lla_decode_teacher_workspace_bytes(tc.dims, w.n, 1, forced)
    assert need > 0
    assert call(opts=forced, wsb=need - 1) == lla.LLA_ERR_WORKSPACE
    assert call(opts=forced, wsb=need) == lla.LLA_OK
    torch.cuda.synchronize()
