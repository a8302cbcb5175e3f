"""GPU parity of lla_decode_attn_absorbed (the decoupled-RoPE absorbed decode of "Looped
Latent Attention", Appendix J "Absorbed attention") against the fp64 oracle, through the
C ABI. Small cases are checked on every output; the full-size launch of the Ouro-1.4B 4x
geometry at context 32768 on a seeded sample of sequences."""

import numpy as np
import pytest
import torch

from latent_decode_attention_lla_amd import lla
from latent_decode_attention_lla_amd.harness import DeviceLatentStore
from latent_decode_attention_lla_amd.inputs import WORKLOADS
from tests.gpu_util import (BF16_TOL, F32_TOL, announce, ensure_built, f64, max_abs,
                            oracle_decode_absorbed, rel_note)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


@pytest.mark.parametrize("d_rope", [16, 32])
@pytest.mark.parametrize("splits", [0, 3])
def test_tiny_f32_every_output(d_rope, splits):
    w = WORKLOADS["tiny_f32"].replace(batch=2, d_rope=d_rope)
    st = DeviceLatentStore(w, seed=21)
    out = st.decode_absorbed(0, 0, 4, opts=lla.make_opts(splits))
    torch.cuda.synchronize()
    ref = oracle_decode_absorbed(st, 0, 0, 4, range(w.batch), w.n)
    err = max_abs(f64(out), ref)
    announce(f"absorbed tiny_f32 d_rope={d_rope} splits={splits}: {rel_note(err, F32_TOL)}")
    assert err <= F32_TOL


@pytest.mark.parametrize("name,d_rope,batch,n,splits", [
    ("ouro_layer_4x", 32, 2, 300, 0),
    ("ouro_layer_4x", 64, 2, 300, 0),
    ("ouro_layer_4x", 96, 2, 300, 5),
    ("ouro_layer_4x", 64, 3, 77, 1),
    ("ouro_layer_4x", 64, 1, 8, 1),
    ("capacity_21x", 32, 3, 517, 0),
    ("capacity_21x", 64, 3, 517, 4),
    ("capacity_21x", 32, 2, 1, 1),
])
def test_bf16_small_every_output(name, d_rope, batch, n, splits):
    w = WORKLOADS[name].replace(batch=batch, n=n, D=2, d_rope=d_rope)
    announce(f"absorbed {name} d_rope={d_rope} B={batch} n={n} splits={splits}")
    st = DeviceLatentStore(w, seed=22)
    for layer in (0, 1):
        out = st.decode_absorbed(layer, 0, 4, opts=lla.make_opts(splits))
        ref = oracle_decode_absorbed(st, layer, 0, 4, range(batch), n)
        err = max_abs(f64(out), ref)
        announce(f"  layer {layer}: {rel_note(err, BF16_TOL)}")
        assert err <= BF16_TOL


@pytest.mark.parametrize("name", ["ouro_layer_4x", "capacity_21x"])
def test_ragged_contexts_and_poisoned_tail(name):
    """Per-sequence lengths over rows that hold NaN past each length, in the latents and
    the rotary keys: no kernel may read them. Empty contexts give zeros."""
    w = WORKLOADS[name].replace(batch=4, n=160, D=1, d_rope=64)
    st = DeviceLatentStore(w, seed=23, n_alloc=192)
    lens = [160, 77, 1, 0]
    for b, n_b in enumerate(lens):
        for key in ("c_k", "c_v", "k_rope"):
            st.t[key][0, b, :, n_b:] = float("nan")
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for splits in (0, 3):
        out = st.decode_absorbed(0, 0, 4, n_ctx=160, ctx_lens=ctx, opts=lla.make_opts(splits))
        got = f64(out)
        assert np.isfinite(got).all()
        assert np.all(got[3] == 0.0)
        ref = oracle_decode_absorbed(st, 0, 0, 4, range(3), 160, ctx_lens=lens)
        err = max_abs(got[:3], ref)
        announce(f"absorbed ragged {name} splits={splits}: {rel_note(err, BF16_TOL)}")
        assert err <= BF16_TOL


def test_lla2d_latents():
    """The decoupled decode over an LLA-2D latent (one per token for all heads; the rotary
    keys stay per head)."""
    w = WORKLOADS["lla2d_long"].replace(batch=2, n=200, D=1, d_rope=64)
    st = DeviceLatentStore(w, seed=24)
    out = st.decode_absorbed(0, 0, 4)
    ref = oracle_decode_absorbed(st, 0, 0, 4, range(w.batch), w.n)
    err = max_abs(f64(out), ref)
    announce(f"absorbed lla2d: {rel_note(err, BF16_TOL)}")
    assert err <= BF16_TOL


def test_absorbed_4x_full_launch_sampled():
    """The 4x geometry with a 64-wide rotary branch at batch 8 and context 32768, one
    (layer, loop) per call; a seeded sample of sequences against the oracle."""
    w = WORKLOADS["absorbed_4x"].replace(D=1)
    announce("absorbed_4x full launch, B=8 n=32768 d_rope=64")
    st = DeviceLatentStore(w, seed=25)
    for loop in (0, 3):
        out = st.decode_absorbed(0, loop, 1)
        torch.cuda.synchronize()
        seqs = [1, 6]
        ref = oracle_decode_absorbed(st, 0, loop, 1, seqs, w.n)
        err = max_abs(f64(out[seqs]), ref)
        announce(f"  loop {loop}: {rel_note(err, BF16_TOL)}")
        assert err <= BF16_TOL
        assert torch.isfinite(out).all()


def test_unsupported_and_invalid_arguments():
    w = WORKLOADS["ouro_layer_4x"].replace(batch=1, n=32, D=1, d_rope=64)
    st = DeviceLatentStore(w, seed=26)
    assert lla.lla_decode_absorbed_supported(st.dims, 64)
    assert not lla.lla_decode_absorbed_supported(st.dims, 48)
    out = torch.empty(1, w.H, 1, w.d, device="cuda")
    ws = st.absorbed_workspace(w.n, 1)
    q = st.t["q"][0, 0]
    for d_rope, want in ((48, lla.LLA_ERR_UNSUPPORTED), (8, lla.LLA_ERR_INVALID_ARG),
                         (128, lla.LLA_ERR_INVALID_ARG)):
        got = lla.lla_decode_attn_absorbed_status(st.dims, st.codec, st.cache, st.t["k_rope"], d_rope,
                                                  0, w.n, None, q, 0, 1, out, ws, ws.numel())
        assert got == want, (d_rope, got)
    small = lla.lla_decode_absorbed_workspace_bytes(st.dims, 64, w.n, 1) - 256
    got = lla.lla_decode_attn_absorbed_status(st.dims, st.codec, st.cache, st.t["k_rope"], 64, 0,
                                              w.n, None, q, 0, 1, out, ws, small)
    assert got == lla.LLA_ERR_WORKSPACE
