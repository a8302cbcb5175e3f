"""GPU parity of lla_reconstruct (the materialised reconstruction that the latent-store
decoder's two-pass prefill feeds its second pass, one layer at a time: "Looped Latent
Attention", Section 3 Eq. 3 and "RoPE and reconstruction"; Appendix A "Decoding and
caching"; Appendix J "Eviction and long-context prefill") against the fp64 oracle,
through the C ABI. float32 outputs to 1e-5; bfloat16 outputs, rounded once, to one
bfloat16 ulp of the exact value (the rounding plus float32 accumulation that can move a
value across a rounding midpoint)."""

import numpy as np
import pytest
import torch

from latent_decode_attention_lla_amd import lla
from latent_decode_attention_lla_amd.harness import DeviceLatentStore, DeviceTeacherCache
from latent_decode_attention_lla_amd.inputs import WORKLOADS
from oracle import lla_oracle as O
from tests.gpu_util import (BF16_TOL, F32_TOL, announce, bf16_ulp, ensure_built, f64, max_abs,
                            rel_note)

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def _oracle(st, layer, loop_begin, loop_count, pos_start, n_tok):
    t, w = st.t, st.w
    return O.reconstruct_cache(f64(t["c_k"][layer]), f64(t["c_v"][layer]), f64(t["w_up_k"][layer]),
                               f64(t["mu_k"][layer]), f64(t["w_up_v"][layer]), f64(t["mu_v"][layer]),
                               loop_begin, loop_count, pos_start, n_tok, w.rope_base,
                               "per_head" if w.variant == "per_head" else "2d")


def _excess(got, ref, dtype):
    """Largest error beyond the allowed bound (<= 0 passes) and the max-abs error."""
    err = np.abs(got - ref)
    bound = F32_TOL if dtype == "f32" else bf16_ulp(ref) + 1e-6
    return float(np.max(err - bound)), float(np.max(err))


def _check_range(st, layer, lb, lc, p0, nt, label):
    shape = (lc, st.w.batch, st.w.H, st.n_max, st.w.d)
    k_out = torch.full(shape, SENTINEL, dtype=st.w.torch_dtype, device="cuda")
    v_out = torch.full(shape, SENTINEL, dtype=st.w.torch_dtype, device="cuda")
    st.reconstruct(layer, lb, lc, p0, nt, k_out, v_out)
    torch.cuda.synchronize()
    kr, vr = _oracle(st, layer, lb, lc, p0, nt)
    kg, vg = f64(k_out), f64(v_out)
    for name, g, r in (("K", kg, kr), ("V", vg, vr)):
        over, err = _excess(g[:, :, :, p0:p0 + nt], r, st.w.dtype)
        announce(f"reconstruct {label} {name}: max-abs {err:.3e}, worst excess over bound {over:.3e}")
        assert over <= 0.0
        outside = np.concatenate([g[:, :, :, :p0].ravel(), g[:, :, :, p0 + nt:].ravel()])
        assert np.all(outside == SENTINEL), "rows outside the slot range were written"


@pytest.mark.parametrize("p0,nt", [(0, 128), (37, 61), (127, 1)])
def test_tiny_f32(p0, nt):
    w = WORKLOADS["tiny_f32"].replace(batch=2)
    st = DeviceLatentStore(w, seed=61)
    _check_range(st, 0, 0, 4, p0, nt, f"tiny_f32 p0={p0} n={nt}")


@pytest.mark.parametrize("name,r_k,r_v,H", [
    ("ouro_layer_4x", 96, 160, 4),
    ("capacity_21x", 16, 32, 4),
    ("ouro_layer_4x", 256, 256, 2),
    ("ouro_layer_4x", 128, 128, 2),
    ("ouro_layer_4x", 64, 24, 2),
])
def test_bf16_ranks(name, r_k, r_v, H):
    w = WORKLOADS[name].replace(batch=2, n=300, D=2, H=H, r_k=r_k, r_v=r_v)
    st = DeviceLatentStore(w, seed=62)
    _check_range(st, 1, 0, 4, 5, 290, f"{name} ({r_k},{r_v}) H={H}")
    _check_range(st, 0, 1, 2, 0, 17, f"{name} ({r_k},{r_v}) loops 1-2")


@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f32"), (64, "f32")])
def test_other_head_widths_and_float32(d, dtype):
    w = WORKLOADS["ouro_layer_4x"].replace(batch=2, n=100, D=1, H=2, d=d, r_k=32, r_v=64,
                                           dtype=dtype)
    st = DeviceLatentStore(w, seed=63)
    _check_range(st, 0, 0, 4, 3, 90, f"d={d} {dtype}")


def test_lla2d():
    w = WORKLOADS["lla2d_long"].replace(batch=2, n=200, D=1)
    st = DeviceLatentStore(w, seed=64)
    _check_range(st, 0, 0, 4, 10, 150, "lla2d")


def test_full_memory_path_feeds_the_uncompressed_decode():
    """Reconstruct every slot of a layer, attend over it with lla_decode_attn_teacher, and
    compare with the oracle's uncompressed decode of the same (rounded) rows and with the
    oracle's latent decode."""
    w = WORKLOADS["ouro_layer_4x"].replace(batch=2, n=700, D=1)
    st = DeviceLatentStore(w, seed=65)
    k, v = st.reconstruct(0, 0, 4)
    tw = WORKLOADS["teacher_4k"].replace(batch=2, n=700, D=1, H=w.H, d=w.d, T=4)
    q = st.t["q"][0]  # [T][B][H][d]
    tc = DeviceTeacherCache(tw, seed=0, tensors={"k_cache": k[None], "v_cache": v[None], "q": q[None]})
    out = tc.decode(0, 0, 4)
    torch.cuda.synchronize()
    got = f64(out)
    ref_teacher = O.decode_teacher(f64(k), f64(v), f64(q.permute(1, 2, 0, 3)), 0, None)
    err_t = max_abs(got, ref_teacher)
    ref_latent = O.decode(f64(st.t["c_k"][0]), f64(st.t["c_v"][0]), f64(st.t["w_up_k"][0]),
                          f64(st.t["mu_k"][0]), f64(st.t["w_up_v"][0]), f64(st.t["mu_v"][0]),
                          f64(q.permute(1, 2, 0, 3)), 0, None, w.rope_base)
    err_l = max_abs(got, ref_latent)
    announce(f"full-memory path: vs uncompressed oracle {rel_note(err_t, BF16_TOL)}; "
             f"vs latent oracle {rel_note(err_l, BF16_TOL)}")
    assert err_t <= BF16_TOL and err_l <= BF16_TOL


def test_prefill_64k_full_layer_sampled():
    """One layer of a 65536-token prompt at the Ouro-1.4B 4x geometry: all four loops'
    keys and values rebuilt in one call (2.1 GB), sampled slots against the oracle."""
    w = WORKLOADS["ouro_layer_4x"].replace(batch=1, n=65536, D=1)
    announce("reconstruct 65536 slots x 16 heads x 4 loops")
    st = DeviceLatentStore(w, seed=66)
    k, v = st.reconstruct(0, 0, 4)
    torch.cuda.synchronize()
    rng = np.random.default_rng(66)
    worst = 0.0
    for j in sorted(rng.choice(65536, size=12, replace=False).tolist()) + [0, 65535]:
        kr, vr = _oracle(st, 0, 0, 4, j, 1)
        for g, r in ((k, kr), (v, vr)):
            over, err = _excess(f64(g[:, :, :, j:j + 1]), r, "bf16")
            worst = max(worst, err)
            assert over <= 0.0, j
    announce(f"  sampled slots: max-abs {worst:.3e}")
    assert torch.isfinite(k).all() and torch.isfinite(v).all()


def test_invalid_arguments():
    w = WORKLOADS["ouro_layer_4x"].replace(batch=1, n=64, D=1, H=2)
    st = DeviceLatentStore(w, seed=67)
    k = torch.empty(4, 1, 2, 64, 128, dtype=torch.bfloat16, device="cuda")

    def call(lb=0, lc=4, p0=0, nt=64, ko=k, vo=k, layer=0):
        return lla.lla_reconstruct_status(st.dims, st.codec, st.cache, layer, lb, lc, p0, nt, ko, vo)

    assert call() == lla.LLA_OK
    assert call(nt=0) == lla.LLA_OK
    assert call(p0=1) == lla.LLA_ERR_INVALID_ARG        # past n_max
    assert call(p0=-1, nt=1) == lla.LLA_ERR_INVALID_ARG
    assert call(lb=3, lc=2) == lla.LLA_ERR_INVALID_ARG
    assert call(layer=1) == lla.LLA_ERR_INVALID_ARG
    assert call(ko=None, vo=None) == lla.LLA_ERR_INVALID_ARG
    assert call(ko=k.data_ptr() + 2) == lla.LLA_ERR_INVALID_ARG
    w48 = w.replace(r_k=48)
    st48 = DeviceLatentStore(w48, seed=68)
    assert lla.lla_reconstruct_status(st48.dims, st48.codec, st48.cache, 0, 0, 4, 0, 64, k, None) \
        == lla.LLA_ERR_UNSUPPORTED
    assert lla.lla_reconstruct_status(st48.dims, st48.codec, st48.cache, 0, 0, 4, 0, 64, None, k) \
        == lla.LLA_OK
    torch.cuda.synchronize()
