"""GPU parity of lla_decode_attn against the fp64 oracle, through the C ABI.

Workloads are the seeded synthetic recipes of latent_decode_attention_lla_amd.inputs
(Ouro-1.4B shapes from "Looped Latent Attention", Appendix A; ranks from Tables 5
and 8). Small cases are checked element by element over every output; the full-size
launch configurations are checked on a seeded sample of sequences (all heads, the
loops named), which the oracle computes one by one.
"""

import numpy as np
import pytest
import torch

from latent_decode_attention_lla_amd import lla
from latent_decode_attention_lla_amd.harness import DeviceLatentStore
from latent_decode_attention_lla_amd.inputs import WORKLOADS
from tests.gpu_util import (BF16_TOL, F32_TOL, announce, ensure_built, f64, max_abs,
                            oracle_decode, rel_note)

pytestmark = pytest.mark.gpu

RECON = lla.LLA_PATH_RECONSTRUCT
FOLD = lla.LLA_PATH_ROTARY_FOLD
BF16_PATHS = [pytest.param(RECON, id="reconstruct"), pytest.param(FOLD, id="rotary_fold")]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


# ---------------------------------------------------------------------------
# tiny float32 workload: T=4, H=2, d=64, (16, 24), batch 1, context 128
# ---------------------------------------------------------------------------

def test_tiny_f32_all_loops_one_call():
    w = WORKLOADS["tiny_f32"]
    announce(f"tiny_f32 all loops, seed 1")
    st = DeviceLatentStore(w, seed=1)
    out = st.decode(0, 0, 4, opts=lla.make_opts(0, RECON))
    torch.cuda.synchronize()
    ref = oracle_decode(st, 0, 0, 4, range(w.batch), w.n)
    err = max_abs(f64(out), ref)
    announce(f"tiny_f32 4 loops: {rel_note(err, F32_TOL)}")
    assert err <= F32_TOL


@pytest.mark.parametrize("loop", [0, 1, 2, 3])
def test_tiny_f32_per_loop_calls(loop):
    w = WORKLOADS["tiny_f32"]
    st = DeviceLatentStore(w, seed=1)
    out = st.decode(0, loop, 1, opts=lla.make_opts(0, RECON))
    ref = oracle_decode(st, 0, loop, 1, range(w.batch), w.n)
    assert max_abs(f64(out), ref) <= F32_TOL


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 8])
def test_tiny_f32_split_invariance(splits):
    """Any split count gives the oracle's answer (the log-sum-exp merge is exact up to
    rounding); splits of a 128-token context are at most 8 tiles of 16."""
    w = WORKLOADS["tiny_f32"].replace(batch=2)
    st = DeviceLatentStore(w, seed=2)
    opts = lla.make_opts(splits, RECON)
    eff = lla.lla_decode_num_splits(st.dims, w.n, 4, opts)
    assert 1 <= eff <= splits
    announce(f"tiny_f32 requested {splits} splits, planned {eff}")
    out = st.decode(0, 0, 4, opts=opts)
    ref = oracle_decode(st, 0, 0, 4, range(w.batch), w.n)
    assert max_abs(f64(out), ref) <= F32_TOL


def test_tiny_f32_ragged_contexts_and_poisoned_tail():
    """Per-sequence lengths (a full one, a ragged one, one token, none) over a cache whose
    rows past each length hold NaN: the kernels must never read them."""
    w = WORKLOADS["tiny_f32"].replace(batch=4, n=128)
    st = DeviceLatentStore(w, seed=3, n_alloc=160)
    lens = [128, 77, 1, 0]
    for b, n_b in enumerate(lens):
        st.t["c_k"][0, b, :, n_b:] = float("nan")
        st.t["c_v"][0, b, :, n_b:] = float("nan")
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for splits in (0, 3):
        out = st.decode(0, 0, 4, n_ctx=128, ctx_lens=ctx, opts=lla.make_opts(splits, RECON))
        got = f64(out)
        assert np.isfinite(got).all()
        assert np.all(got[3] == 0.0)  # empty context -> zeros
        # oracle on clean copies of the attended rows only
        ref = oracle_decode(st, 0, 0, 4, range(3), 128, ctx_lens=lens)
        assert max_abs(got[:3], ref) <= F32_TOL


def test_tiny_f32_zero_query_and_single_token():
    w = WORKLOADS["tiny_f32"]
    st = DeviceLatentStore(w, seed=4)
    q0 = torch.zeros(w.batch, w.H, 4, w.d, device="cuda")
    out = st.decode(0, 0, 4, q=q0, opts=lla.make_opts(0, RECON))
    ref = oracle_decode(st, 0, 0, 4, range(w.batch), w.n, q=q0)
    assert max_abs(f64(out), ref) <= F32_TOL
    out1 = st.decode(0, 0, 4, n_ctx=1, opts=lla.make_opts(0, RECON))
    ref1 = oracle_decode(st, 0, 0, 4, range(w.batch), 1)
    assert max_abs(f64(out1), ref1) <= F32_TOL


def test_empty_context_gives_zeros():
    w = WORKLOADS["tiny_f32"]
    st = DeviceLatentStore(w, seed=5)
    out = st.decode(0, 0, 4, n_ctx=0, opts=lla.make_opts(0, RECON))
    assert torch.all(out == 0)


def test_rope_base_one_million():
    """RoPE base is an argument (Ouro-family models use 1e6 per the Ragged-KV page)."""
    w = WORKLOADS["tiny_f32"].replace(rope_base=1.0e6)
    st = DeviceLatentStore(w, seed=6)
    out = st.decode(0, 0, 4, opts=lla.make_opts(0, RECON))
    ref = oracle_decode(st, 0, 0, 4, range(w.batch), w.n)
    assert max_abs(f64(out), ref) <= F32_TOL


def test_determinism_bitwise():
    w = WORKLOADS["ouro_layer_4x"].replace(batch=2, n=300)
    st = DeviceLatentStore(w, seed=7)
    a = st.decode(0, 0, 4).clone()
    b = st.decode(0, 0, 4).clone()
    assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# bfloat16 per-head workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", BF16_PATHS)
@pytest.mark.parametrize("name,batch,n,splits", [
    ("ouro_layer_4x", 2, 300, 0),
    ("ouro_layer_4x", 2, 300, 5),
    ("capacity_21x", 3, 517, 0),
    ("capacity_21x", 3, 517, 1),
    ("capacity_21x", 3, 517, 4),
    ("capacity_21x", 2, 16, 1),
    ("capacity_21x", 2, 1, 1),
    ("ouro_layer_4x", 3, 77, 1),
    ("ouro_layer_4x", 1, 16, 1),
])
def test_bf16_small_every_output(name, batch, n, splits, path):
    w = WORKLOADS[name].replace(batch=batch, n=n, D=2)
    announce(f"{name} B={batch} n={n} splits={splits} path={path}")
    st = DeviceLatentStore(w, seed=11)
    for layer in (0, 1):
        out = st.decode(layer, 0, 4, opts=lla.make_opts(splits, path))
        ref = oracle_decode(st, layer, 0, 4, range(batch), n)
        err = max_abs(f64(out), ref)
        announce(f"  layer {layer}: {rel_note(err, BF16_TOL)}")
        assert err <= BF16_TOL


@pytest.mark.parametrize("path", BF16_PATHS)
def test_capacity_21x_full_launch_sampled(path):
    """The 21.3x capacity point at its real launch shape: 768 sequences x 16 heads,
    context 4096, one (layer, loop) per call. One layer is resident (the call shape does
    not depend on D); a seeded sample of sequences is checked against the oracle."""
    w = WORKLOADS["capacity_21x"].replace(D=1)
    announce(f"capacity_21x full launch, B=768 n=4096 path={path}")
    st = DeviceLatentStore(w, seed=3)
    rng = np.random.default_rng(3)
    seqs = sorted(rng.choice(w.batch, size=4, replace=False).tolist()) + [w.batch - 1]
    for loop in (0, 3):
        out = st.decode(0, loop, 1, opts=lla.make_opts(0, path))
        torch.cuda.synchronize()
        ref = oracle_decode(st, 0, loop, 1, seqs, w.n)
        got = f64(out[seqs])
        err = max_abs(got, ref)
        announce(f"  loop {loop}: {rel_note(err, BF16_TOL)}")
        assert err <= BF16_TOL
        assert torch.isfinite(out).all()


@pytest.mark.parametrize("path", BF16_PATHS)
def test_lla2d_full_launch_sampled(path):
    """LLA-2D (one latent per token shared by 16 heads), batch 16, context 16384."""
    w = WORKLOADS["lla2d_long"].replace(D=1)
    announce(f"lla2d_long full launch, B=16 n=16384 path={path}")
    st = DeviceLatentStore(w, seed=5)
    out = st.decode(0, 2, 1, opts=lla.make_opts(0, path))
    torch.cuda.synchronize()
    seqs = [0, 9, 15]
    ref = oracle_decode(st, 0, 2, 1, seqs, w.n)
    err = max_abs(f64(out[seqs]), ref)
    announce(f"  lla2d loop 2: {rel_note(err, BF16_TOL)}")
    assert err <= BF16_TOL


@pytest.mark.parametrize("path", BF16_PATHS)
@pytest.mark.parametrize("H,batch,n,splits", [
    (16, 2, 200, 0), (16, 2, 200, 1), (16, 2, 200, 3), (16, 3, 17, 1), (16, 9, 64, 2),
    # H not a multiple of 8: the LLA-2D kernel's 4-heads-per-workgroup instance, one and
    # three splits (H = 12: three workgroups per (sequence, loop, split))
    (4, 2, 200, 1), (4, 2, 200, 3), (12, 2, 200, 1), (12, 3, 200, 3)])
def test_lla2d_small_every_output(path, H, batch, n, splits):
    w = WORKLOADS["lla2d_long"].replace(D=1, batch=batch, n=n, H=H)
    st = DeviceLatentStore(w, seed=6)
    out = st.decode(0, 0, 4, opts=lla.make_opts(splits, path))
    ref = oracle_decode(st, 0, 0, 4, range(batch), n)
    err = max_abs(f64(out), ref)
    announce(f"lla2d H={H} B={batch} n={n} splits={splits} path={path}: {rel_note(err, BF16_TOL)}")
    assert err <= BF16_TOL


@pytest.mark.parametrize("path", BF16_PATHS)
@pytest.mark.parametrize("H", [16, 4, 12])
def test_lla2d_ragged_poisoned(path, H):
    w = WORKLOADS["lla2d_long"].replace(D=1, batch=4, n=150, H=H)
    st = DeviceLatentStore(w, seed=7, n_alloc=160)
    lens = [150, 33, 1, 0]
    for b, n_b in enumerate(lens):
        st.t["c_k"][0, b, :, n_b:] = float("nan")
        st.t["c_v"][0, b, :, n_b:] = float("nan")
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for splits in (1, 2):
        got = f64(st.decode(0, 1, 2, n_ctx=150, ctx_lens=ctx, opts=lla.make_opts(splits, path)))
        assert np.isfinite(got).all() and np.all(got[3] == 0.0)
        ref = oracle_decode(st, 0, 1, 2, range(3), 150, ctx_lens=lens)
        assert max_abs(got[:3], ref) <= BF16_TOL


@pytest.mark.parametrize("H", [2, 6])
@pytest.mark.parametrize("d,r_k,r_v", [(128, 96, 160), (128, 64, 64), (128, 128, 128), (64, 256, 256)])
def test_bf16_wide_fold_two_heads_per_workgroup(d, r_k, r_v, H):
    """The per-head wide fold with a head count that is not a multiple of 4, so that its
    workgroups take 2 heads instead of 4: every shape, a ragged tail tile, one and three
    splits, all 4 loops, every output against the oracle."""
    w = WORKLOADS["ouro_layer_4x"].replace(D=1, batch=2, n=93, d=d, r_k=r_k, r_v=r_v, H=H)
    st = DeviceLatentStore(w, seed=23)
    for splits in (1, 3):
        out = st.decode(0, 0, 4, opts=lla.make_opts(splits, FOLD))
        ref = oracle_decode(st, 0, 0, 4, range(w.batch), w.n)
        err = max_abs(f64(out), ref)
        announce(f"wide fold H={H} d={d} ranks=({r_k}, {r_v}) splits={splits}: {rel_note(err, BF16_TOL)}")
        assert err <= BF16_TOL


@pytest.mark.parametrize("H", [4, 12, 16])
@pytest.mark.parametrize("d,r_k,r_v", [(128, 16, 32), (128, 32, 64), (64, 16, 32), (64, 32, 32)])
def test_bf16_narrow_fold_every_shape_and_head_group(d, r_k, r_v, H):
    """The narrow fold over a dense cache keeps several chunks of rows in flight per wave,
    with 8 heads per workgroup where the shape and H allow it and 4 otherwise: every shape
    it is built for, head counts that take each grouping, contexts that end inside the
    first chunk, on a round boundary and past several rounds with a ragged tail, one and
    three splits, all 4 loops, every output against the oracle."""
    for n in (16, 93, 517):
        w = WORKLOADS["capacity_21x"].replace(D=1, batch=2, n=n, d=d, r_k=r_k, r_v=r_v, H=H)
        st = DeviceLatentStore(w, seed=29)
        for splits in (1, 3):
            out = st.decode(0, 0, 4, opts=lla.make_opts(splits, FOLD))
            ref = oracle_decode(st, 0, 0, 4, range(w.batch), w.n)
            err = max_abs(f64(out), ref)
            announce(f"narrow fold H={H} d={d} ranks=({r_k}, {r_v}) n={n} splits={splits}: "
                     f"{rel_note(err, BF16_TOL)}")
            assert err <= BF16_TOL


@pytest.mark.parametrize("variant", ["per_head", "lla2d"])
@pytest.mark.parametrize("d,r_k,r_v", [(128, 64, 64), (128, 128, 128), (64, 256, 256)])
def test_bf16_table8_ranks_every_output(d, r_k, r_v, variant):
    """The other rank points the fold kernels are built for (Table 8's ranks, and a
    64-wide head with wide latents), per head and LLA-2D, on the folded path: a ragged
    tail tile, one and several splits, all 4 loops."""
    base = WORKLOADS["lla2d_long" if variant == "lla2d" else "ouro_layer_4x"]
    w = base.replace(D=1, batch=2, n=200, d=d, r_k=r_k, r_v=r_v, H=16 if variant == "lla2d" else 4)
    st = DeviceLatentStore(w, seed=21)
    for splits in (1, 3):
        out = st.decode(0, 0, 4, opts=lla.make_opts(splits, FOLD))
        ref = oracle_decode(st, 0, 0, 4, range(w.batch), w.n)
        err = max_abs(f64(out), ref)
        announce(f"{variant} d={d} ranks=({r_k}, {r_v}) splits={splits}: {rel_note(err, BF16_TOL)}")
        assert err <= BF16_TOL


@pytest.mark.parametrize("name", ["capacity_21x", "ouro_layer_4x", "lla2d_long"])
@pytest.mark.parametrize("T", [2, 8])
def test_bf16_other_loop_counts(name, T):
    """Loop counts other than Ouro's 4 (the codec's stacked contraction is T d_in long
    and W_up, mu are sliced per loop): every loop in one call, folded path, two splits."""
    w = WORKLOADS[name].replace(D=1, batch=2, n=150, T=T, H=4)
    st = DeviceLatentStore(w, seed=31)
    out = st.decode(0, 0, T, opts=lla.make_opts(2, FOLD))
    ref = oracle_decode(st, 0, 0, T, range(w.batch), w.n)
    err = max_abs(f64(out), ref)
    announce(f"{name} T={T}: {rel_note(err, BF16_TOL)}")
    assert err <= BF16_TOL


@pytest.mark.parametrize("path", BF16_PATHS)
def test_bf16_ragged_contexts_poisoned_tail(path):
    """Ragged per-sequence lengths with NaN in every cache row past a sequence's length."""
    w = WORKLOADS["capacity_21x"].replace(D=1, batch=5, n=300)
    st = DeviceLatentStore(w, seed=12, n_alloc=320)
    lens = [300, 257, 17, 1, 0]
    for b, n_b in enumerate(lens):
        st.t["c_k"][0, b, :, n_b:] = float("nan")
        st.t["c_v"][0, b, :, n_b:] = float("nan")
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for splits in (1, 0, 3):
        out = st.decode(0, 0, 4, n_ctx=300, ctx_lens=ctx, opts=lla.make_opts(splits, path))
        got = f64(out)
        assert np.isfinite(got).all()
        assert np.all(got[4] == 0.0)
        ref = oracle_decode(st, 0, 0, 4, range(4), 300, ctx_lens=lens)
        assert max_abs(got[:4], ref) <= BF16_TOL


@pytest.mark.parametrize("path", BF16_PATHS)
def test_bf16_ouro_layer_full_sampled(path):
    """Ouro-1.4B layer at 4x, batch 32, context 4096, all 4 loops in one call."""
    w = WORKLOADS["ouro_layer_4x"]
    st = DeviceLatentStore(w, seed=13)
    out = st.decode(0, 0, 4, opts=lla.make_opts(0, path))
    seqs = [0, 31]
    ref = oracle_decode(st, 0, 0, 4, seqs, w.n)
    err = max_abs(f64(out[seqs]), ref)
    announce(f"ouro_layer_4x full path={path}: {rel_note(err, BF16_TOL)}")
    assert err <= BF16_TOL


def test_fold_and_reconstruct_agree_at_scale():
    """Both paths compute the same scores; their outputs over a whole 768 x 16 launch
    agree to the float16 rounding of the folded operands."""
    w = WORKLOADS["capacity_21x"].replace(D=1, batch=96)
    st = DeviceLatentStore(w, seed=14)
    a = f64(st.decode(0, 1, 1, opts=lla.make_opts(0, RECON)))
    b = f64(st.decode(0, 1, 1, opts=lla.make_opts(0, FOLD)))
    err = max_abs(a, b)
    announce(f"fold vs reconstruct over 96 x 16 outputs: max-abs {err:.3e}")
    assert err <= BF16_TOL


@pytest.mark.parametrize("variant", ["per_head", "lla2d"])
@pytest.mark.parametrize("H", [4, 6])
@pytest.mark.parametrize("d,r_k,r_v", [(64, 16, 24), (64, 16, 32), (64, 32, 32), (64, 256, 256),
                                       (128, 16, 32), (128, 32, 64), (128, 96, 160), (128, 128, 128)])
def test_bf16_reconstruct_every_shape(d, r_k, r_v, H, variant):
    """The literal rebuild-then-rotate kernel for bfloat16 caches at every shape it is built
    for, per head and LLA-2D, with 4 heads per workgroup (H = 4) and one (H = 6), a
    ragged tail tile, one and three splits, all 4 loops, every output against the oracle.
    (64, 16, 24) is the one shape whose value-latent slice per lane (6 entries) is read as
    single dwords."""
    base = WORKLOADS["lla2d_long" if variant == "lla2d" else "ouro_layer_4x"]
    w = base.replace(D=1, batch=2, n=77, d=d, r_k=r_k, r_v=r_v, H=H)
    st = DeviceLatentStore(w, seed=41)
    for splits in (1, 3):
        out = st.decode(0, 0, 4, opts=lla.make_opts(splits, RECON))
        ref = oracle_decode(st, 0, 0, 4, range(w.batch), w.n)
        err = max_abs(f64(out), ref)
        announce(f"reconstruct {variant} d={d} ranks=({r_k}, {r_v}) H={H} splits={splits}: "
                 f"{rel_note(err, BF16_TOL)}")
        assert err <= BF16_TOL
