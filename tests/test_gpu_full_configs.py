"""The Ouro-1.4B layer at 4x (batch 32, context 4096) and the encode-heavy prefill (batch
8, context 8192, SVD codec) checked in full against the fp64 oracle, through the C ABI:
the GPU encodes every prompt token once and runs one decode step over all 4 loops; every
stored latent is checked against Eq. 2 ("Looped Latent Attention", Section 3) and every
decode output against the oracle's attention over the reconstructed keys and values
(Eq. 3, RoPE at the slot) of the stored latents. Shapes are Appendix A's Ouro-1.4B
geometry at Table 5's 4x ranks. The checks run over blocks of sequences so that each
test's oracle work stays at a few seconds."""

import numpy as np
import pytest
import torch

from latent_decode_attention_lla_amd.inputs import WORKLOADS, encode_codec_orthonormal, encode_x
from tests.gpu_util import BF16_TOL, announce, ensure_built, f64, max_abs, oracle_decode, rel_note
from tests.test_gpu_encode import _check_latents, _oracle_latents, _store_for_encode, _svd_codec

pytestmark = pytest.mark.gpu

OURO_BLOCK = 8    # sequences per check of the Ouro layer (4 blocks)
HEAVY_BLOCK = 2   # sequences per check of the encode-heavy prefill (4 blocks)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


@pytest.fixture(scope="module")
def ouro_full():
    """Encode 32 x 4096 tokens (Gaussian per-loop K/V, orthonormal codec), then one
    decode step over all 4 loops in one call."""
    w = WORKLOADS["ouro_layer_4x"]
    announce("ouro_layer_4x in full: encode 32x4096, decode 4 loops")
    st = _store_for_encode(w, encode_codec_orthonormal(w, seed=8), seed=8)
    xk, xv = encode_x(w, w.n, seed=9, device="cuda")
    st.encode(0, xk, xv, 0, w.n)
    out = st.decode(0, 0, 4)
    torch.cuda.synchronize()
    return w, st, xk, xv, f64(out)


@pytest.fixture(scope="module")
def heavy_full():
    """Encode 8 x 8192 loop-correlated tokens with the SVD codec of a calibration
    subsample, then one decode step over all 4 loops at context 8192."""
    w = WORKLOADS["encode_heavy"]
    announce("encode_heavy in full: SVD codec, encode 8x8192, decode 4 loops")
    xk, xv = encode_x(w, w.n, seed=10, device="cuda", correlated=True)
    st = _store_for_encode(w, _svd_codec(w, xk, xv, seed=10), seed=10)
    st.encode(0, xk, xv, 0, w.n)
    out = st.decode(0, 0, 4)
    torch.cuda.synchronize()
    return w, st, xk, xv, f64(out)


def _latents(case, seqs):
    w, st, xk, xv, _ = case
    worst = 0.0
    for axis, x in (("k", xk), ("v", xv)):
        got = f64(st.t[f"c_{axis}"][0][seqs])
        worst = max(worst, _check_latents(got, _oracle_latents(st, 0, x[seqs], axis, "bf16"), "bf16"))
    return worst


def _outputs(case, seqs):
    w, st, _, _, out = case
    ref = oracle_decode(st, 0, 0, 4, seqs, w.n)
    assert np.all(np.isfinite(out[seqs]))
    return max_abs(out[seqs], ref)


@pytest.mark.parametrize("block", range(32 // OURO_BLOCK))
def test_ouro_layer_4x_every_latent(ouro_full, block):
    seqs = list(range(OURO_BLOCK * block, OURO_BLOCK * (block + 1)))
    worst = _latents(ouro_full, seqs)
    announce(f"ouro_layer_4x latents of sequences {seqs[0]}..{seqs[-1]}: within one bf16 "
             f"spacing (+ float32 bound), worst {worst:.3f} spacings")


@pytest.mark.parametrize("block", range(32 // OURO_BLOCK))
def test_ouro_layer_4x_every_output(ouro_full, block):
    seqs = list(range(OURO_BLOCK * block, OURO_BLOCK * (block + 1)))
    err = _outputs(ouro_full, seqs)
    announce(f"ouro_layer_4x outputs of sequences {seqs[0]}..{seqs[-1]}, 16 heads x 4 loops: "
             f"{rel_note(err, BF16_TOL)}")
    assert err <= BF16_TOL


@pytest.mark.parametrize("block", range(8 // HEAVY_BLOCK))
def test_encode_heavy_every_latent(heavy_full, block):
    seqs = list(range(HEAVY_BLOCK * block, HEAVY_BLOCK * (block + 1)))
    worst = _latents(heavy_full, seqs)
    announce(f"encode_heavy latents of sequences {seqs[0]}..{seqs[-1]}: within one bf16 "
             f"spacing (+ float32 bound), worst {worst:.3f} spacings")


@pytest.mark.parametrize("block", range(8 // HEAVY_BLOCK))
def test_encode_heavy_every_output(heavy_full, block):
    seqs = list(range(HEAVY_BLOCK * block, HEAVY_BLOCK * (block + 1)))
    err = _outputs(heavy_full, seqs)
    announce(f"encode_heavy outputs of sequences {seqs[0]}..{seqs[-1]}, 16 heads x 4 loops: "
             f"{rel_note(err, BF16_TOL)}")
    assert err <= BF16_TOL
