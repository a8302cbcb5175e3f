"""GPU parity of the paged latent cache (lla_encode_paged, lla_decode_attn_paged) and of
sink-plus-window eviction over it ("Looped Latent Attention", Appendix D Table 9 and
Appendix J "Eviction and long-context prefill") against the fp64 oracle, through the C
ABI. The paged kernels do the dense kernels' arithmetic on rows found through the block
table, so a shuffled pool must also give bit-identical results to the dense cache."""

import numpy as np
import pytest
import torch

from latent_decode_attention_lla_amd import lla
from latent_decode_attention_lla_amd.harness import DeviceLatentStore
from latent_decode_attention_lla_amd.inputs import WORKLOADS, encode_codec_orthonormal, encode_x
from oracle import lla_oracle as O
from tests.gpu_util import (BF16_TOL, F32_TOL, announce, ensure_built, f64, max_abs, rel_note)
from tests.test_gpu_encode import _check_latents, _oracle_latents, _store_for_encode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def _oracle_paged(st, layer, loop_begin, loop_count, seqs, n_ctx, ctx_lens=None):
    t, w = st.t, st.w
    idx = torch.as_tensor(list(seqs), device=st.device)
    table = st.block_table.index_select(0, idx).cpu().numpy()
    q = t["q"][layer, loop_begin:loop_begin + loop_count].permute(1, 2, 0, 3).index_select(0, idx)
    lens = None if ctx_lens is None else [int(ctx_lens[i]) for i in seqs]
    return O.decode_paged(f64(t["c_k"][layer]), f64(t["c_v"][layer]), table, f64(t["w_up_k"][layer]),
                          f64(t["mu_k"][layer]), f64(t["w_up_v"][layer]), f64(t["mu_v"][layer]),
                          f64(q), loop_begin, lens, n_ctx, w.rope_base, None,
                          "per_head" if w.variant == "per_head" else "2d")


@pytest.mark.parametrize("name,over,path,splits", [
    ("capacity_21x", {}, lla.LLA_PATH_AUTO, 0),            # rotary fold, r_k = 16
    ("capacity_21x", {}, lla.LLA_PATH_AUTO, 3),
    ("capacity_21x", {"r_k": 32, "r_v": 64}, lla.LLA_PATH_AUTO, 0),
    ("capacity_21x", {}, lla.LLA_PATH_RECONSTRUCT, 0),
    ("capacity_21x", {"H": 6}, lla.LLA_PATH_RECONSTRUCT, 2),  # one head per workgroup
    ("capacity_21x", {"H": 6, "d": 64, "r_v": 24}, lla.LLA_PATH_RECONSTRUCT, 0),
    ("ouro_layer_4x", {}, lla.LLA_PATH_AUTO, 2),            # wide fold, a pair of waves per head
    ("ouro_layer_4x", {}, lla.LLA_PATH_AUTO, 0),
    ("ouro_layer_4x", {}, lla.LLA_PATH_RECONSTRUCT, 2),
    ("tiny_f32", {}, lla.LLA_PATH_AUTO, 0),                # float32: reconstruct path
    ("lla2d_long", {}, lla.LLA_PATH_AUTO, 0),               # LLA-2D kernel, 4 heads per workgroup
    ("lla2d_long", {}, lla.LLA_PATH_AUTO, 3),
    ("lla2d_long", {}, lla.LLA_PATH_RECONSTRUCT, 0),
    ("lla2d_long", {"H": 16}, lla.LLA_PATH_AUTO, 1),        # LLA-2D kernel, 8 heads per workgroup
    ("lla2d_long", {"H": 16}, lla.LLA_PATH_AUTO, 3),
    ("lla2d_long", {"H": 12}, lla.LLA_PATH_AUTO, 3),        # 4 heads per workgroup, 3 groups
    ("lla2d_long", {"r_k": 64, "r_v": 64}, lla.LLA_PATH_AUTO, 2),     # LLA-2D kernel, other ranks
    ("lla2d_long", {"r_k": 128, "r_v": 128}, lla.LLA_PATH_AUTO, 0),   # wide fold, shared plane
    ("ouro_layer_4x", {"r_k": 64, "r_v": 64}, lla.LLA_PATH_AUTO, 3),  # wide fold, per head
    ("ouro_layer_4x", {"H": 6}, lla.LLA_PATH_AUTO, 2),      # wide fold, 2 heads per workgroup
    ("ouro_layer_4x", {"H": 8}, lla.LLA_PATH_AUTO, 0),      # wide fold, 4 heads per workgroup, 2 groups
])
def test_shuffled_pool_matches_dense_and_oracle(name, over, path, splits):
    """The dense and paged decodes run the same kernel (narrow fold, wide fold or
    reconstruct) on the same rows, so they must agree bit for bit."""
    heads = {} if name == "tiny_f32" or "H" in over else {"H": 4}
    w = WORKLOADS[name].replace(batch=3, n=300, D=2, **heads, **over)
    st = DeviceLatentStore(w, seed=71)
    lens = [300, 133, 1]
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    opts = lla.make_opts(splits, path)
    dense = st.decode(1, 0, w.T, ctx_lens=ctx, opts=opts).clone()
    st.paginate(seed=72, spare_pages=5)
    paged = st.decode_paged(1, 0, w.T, ctx_lens=ctx, opts=opts)
    torch.cuda.synchronize()
    ref = _oracle_paged(st, 1, 0, w.T, range(3), w.n, lens)
    tol = F32_TOL if w.dtype == "f32" else BF16_TOL
    err = max_abs(f64(paged), ref)
    same = torch.equal(paged, dense)
    announce(f"paged {name} {over} path={path} splits={splits}: {rel_note(err, tol)}; "
             f"bit-identical to dense: {same}")
    assert err <= tol
    assert same


@pytest.mark.parametrize("H", [16, 4])
def test_paged_narrow_fold_split_spans_at_most_256_pages(H):
    """A fold kernel keeps a split's page indices in LDS, 256 at most, so the host splits a
    paged context into spans of at most 4096 tokens: at 4500 tokens the auto plan takes two
    splits, the first filling every slot. Both the paged decode and the dense one match the
    oracle (their split boundaries differ, so they need not agree bit for bit)."""
    w = WORKLOADS["capacity_21x"].replace(batch=2, n=4500, D=1, H=H)
    st = DeviceLatentStore(w, seed=73)
    lens = [4500, 4100]
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    opts = lla.make_opts(0, lla.LLA_PATH_ROTARY_FOLD)
    n_split = lla.lla_decode_paged_num_splits(st.dims, w.n, w.T, opts)
    assert n_split >= 2
    dense = st.decode(0, 0, w.T, ctx_lens=ctx, opts=opts).clone()
    st.paginate(seed=74, spare_pages=3)
    paged = st.decode_paged(0, 0, w.T, ctx_lens=ctx, opts=opts)
    torch.cuda.synchronize()
    ref = _oracle_paged(st, 0, 0, w.T, range(2), w.n, lens)
    for label, got in (("paged", paged), ("dense", dense)):
        err = max_abs(f64(got), ref)
        announce(f"narrow fold H={H} n=4500 {label} ({n_split} paged splits): {rel_note(err, BF16_TOL)}")
        assert err <= BF16_TOL


@pytest.mark.parametrize("name", ["capacity_21x", "ouro_layer_4x", "lla2d_long"])
def test_pages_past_the_context_are_not_read(name):
    """Pages of the pool the table does not name for a token below len_b hold NaN (spares
    and the rows past each length): outputs stay finite; an empty context gives zeros."""
    w = WORKLOADS[name].replace(batch=4, n=160, D=1, H=4)
    st = DeviceLatentStore(w, seed=73)
    lens = [160, 77, 1, 0]
    for b, n_b in enumerate(lens):
        for key in ("c_k", "c_v"):
            st.t[key][0, b, :, n_b:] = float("nan")
    st.paginate(seed=74, spare_pages=7)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for path in (lla.LLA_PATH_AUTO, lla.LLA_PATH_RECONSTRUCT):
        for splits in (0, 2):
            out = st.decode_paged(0, 0, 4, ctx_lens=ctx, opts=lla.make_opts(splits, path))
            got = f64(out)
            assert np.isfinite(got).all()
            assert np.all(got[3] == 0.0)
            ref = _oracle_paged(st, 0, 0, 4, range(3), w.n, lens[:3])
            err = max_abs(got[:3], ref)
            announce(f"paged NaN tails {name} path={path} splits={splits}: {rel_note(err, BF16_TOL)}")
            assert err <= BF16_TOL


@pytest.mark.parametrize("name,n_new", [("capacity_21x", 1), ("capacity_21x", 37),
                                        ("tiny_f32", 20), ("ouro_layer_4x", 50)])
def test_paged_encode_matches_dense_encode(name, n_new):
    w = WORKLOADS[name].replace(batch=3, n=128, D=1)
    codec = encode_codec_orthonormal(w, seed=75)
    dense = _store_for_encode(w, codec, seed=75, sentinel=0.0)
    paged = _store_for_encode(w, codec, seed=75, sentinel=0.0)
    paged.paginate(seed=76, spare_pages=3)
    xk, xv = encode_x(w, n_new, seed=77, device="cuda")
    pos = 40
    dense.encode(0, xk, xv, pos, n_new)
    lla.lla_encode_paged(paged.dims, paged.codec, paged.cache, paged.pages, 0, xk, xv, pos, n_new)
    torch.cuda.synchronize()
    table = paged.block_table.cpu().numpy()
    for axis, x in (("k", xk), ("v", xv)):
        got = O.gather_pages(f64(paged.t[f"c_{axis}"][0]), table, w.n)
        ratio = _check_latents(got[:, :, pos:pos + n_new], _oracle_latents(paged, 0, x, axis, w.dtype),
                               w.dtype)
        want = f64(dense.t[f"c_{axis}"][0])
        if n_new <= 64:  # the dense path runs the same few-token kernel
            assert np.array_equal(got[:, :, pos:pos + n_new], want[:, :, pos:pos + n_new])
        announce(f"paged encode {name} n_new={n_new} {axis}: worst {ratio:.3g} (ulp or abs)")


@pytest.mark.parametrize("name", ["capacity_21x", "ouro_layer_4x", "lla2d_long"])
def test_streaming_eviction_sink_and_window(name):
    """A sequence grows page by page through lla_encode_paged; once sink + window pages
    are full, the oldest window page is evicted and its physical page reused. The block
    table then lists O.window_pages' logical pages, the stored latents are those of the
    kept tokens, and lla_decode_attn_paged over them (positions = slots of the kept cache)
    matches the oracle: narrow fold, wide fold and the LLA-2D kernel."""
    w = WORKLOADS[name].replace(batch=2, n=16 * 6, D=1, H=4)
    sink, window, written_pages = 1, 4, 11
    codec = encode_codec_orthonormal(w, seed=78)
    st = _store_for_encode(w, codec, seed=78, sentinel=0.0)
    cap_pages = sink + window + 1                 # room for the page being filled
    num_pages = w.batch * cap_pages
    pool = {k: torch.zeros(w.D, num_pages, w.Hc, 16, r, dtype=w.torch_dtype, device="cuda")
            for k, r in (("c_k", w.r_k), ("c_v", w.r_v))}
    st.t.update(pool)
    st.cache = lla.make_cache(pool["c_k"], pool["c_v"])
    free = list(range(num_pages))
    logical = [[] for _ in range(w.batch)]        # kept logical page ids, in order
    phys = [[] for _ in range(w.batch)]           # their physical pages
    table = torch.zeros(w.batch, cap_pages, dtype=torch.int32, device="cuda")
    xs = []
    for pg in range(written_pages):
        xk, xv = encode_x(w, 16, seed=1000 + pg, device="cuda")
        xs.append((xk, xv))
        for b in range(w.batch):
            if len(phys[b]) == sink + window:     # evict the oldest window page
                free.append(phys[b].pop(sink))
                logical[b].pop(sink)
            phys[b].append(free.pop(0))
            logical[b].append(pg)
            table[b, :len(phys[b])] = torch.tensor(phys[b], dtype=torch.int32)
        st.block_table = table
        st.pages = lla.make_pages(table, cap_pages, num_pages)
        pos = 16 * (len(phys[0]) - 1)             # the new page's first logical slot
        lla.lla_encode_paged(st.dims, st.codec, st.cache, st.pages, 0, xk, xv, pos, 16)
    torch.cuda.synchronize()
    for b in range(w.batch):
        assert logical[b] == O.window_pages(written_pages, sink, window)
    n_kept = 16 * len(phys[0])
    tab = table.cpu().numpy()
    for axis, ai in (("k", 0), ("v", 1)):
        x_kept = torch.cat([xs[pg][ai] for pg in logical[0]], 1)
        got = O.gather_pages(f64(st.t[f"c_{axis}"][0]), tab, n_kept)
        _check_latents(got, _oracle_latents(st, 0, x_kept, axis, w.dtype), w.dtype)
    ctx = torch.tensor([n_kept, n_kept - 5], dtype=torch.int32, device="cuda")
    out = st.decode_paged(0, 0, 4, n_ctx=n_kept, ctx_lens=ctx)
    ref = _oracle_paged(st, 0, 0, 4, range(w.batch), n_kept, [n_kept, n_kept - 5])
    err = max_abs(f64(out), ref)
    announce(f"streaming eviction {name} (sink {sink}, window {window} pages, {written_pages} written): "
             f"{rel_note(err, BF16_TOL)}")
    assert err <= BF16_TOL


@pytest.mark.parametrize("name,seqs", [("capacity_21x", [0, 383, 767]), ("ouro_layer_4x", [0, 31]),
                                       ("lla2d_long", [0, 15])])
def test_full_launch_paged_sampled(name, seqs):
    """The 21.3x capacity shape (768 x 4096, narrow fold), the Ouro-1.4B 4x layer
    (32 x 4096, wide fold) and LLA-2D at 16 x 16384 (LLA-2D kernel) with shuffled pages:
    one (layer, loop) call as the bench times it; bit-identical to the dense cache,
    sampled sequences against the oracle."""
    w = WORKLOADS[name].replace(D=1)
    announce(f"paged {name} full launch, B={w.batch} n={w.n}")
    st = DeviceLatentStore(w, seed=79)
    dense = st.decode(0, 2, 1).clone()
    st.paginate(seed=80)
    del st.dense
    torch.cuda.empty_cache()
    out = st.decode_paged(0, 2, 1)
    torch.cuda.synchronize()
    assert torch.equal(out, dense)
    ref = _oracle_paged(st, 0, 2, 1, seqs, w.n)
    err = max_abs(f64(out[seqs]), ref)
    announce(f"  sampled: {rel_note(err, BF16_TOL)}")
    assert err <= BF16_TOL


def test_invalid_arguments():
    w = WORKLOADS["capacity_21x"].replace(batch=2, n=64, D=1, H=4)
    st = DeviceLatentStore(w, seed=81)
    st.paginate(seed=82)
    out = torch.empty(2, 4, 1, w.d, device="cuda")
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    q = st.t["q"][0, 0]

    def call(pages=st.pages, opts=None):
        return lla.lla_decode_attn_paged_status(st.dims, st.codec, st.cache, pages, 0, w.n, None, q,
                                                0, 1, out, ws, ws.numel(), opts)

    assert call() == lla.LLA_OK
    assert call(lla.make_pages(st.block_table, 3, st.pages.num_pages)) == lla.LLA_ERR_INVALID_ARG
    assert call(lla.make_pages(0, 4, st.pages.num_pages)) == lla.LLA_ERR_INVALID_ARG
    assert call(lla.make_pages(st.block_table.data_ptr() + 2, 4, 8)) == lla.LLA_ERR_INVALID_ARG
    assert call(lla.make_pages(st.block_table, 4, 0)) == lla.LLA_ERR_INVALID_ARG
    w4 = WORKLOADS["tiny_f32"].replace(batch=1, n=64, D=1)  # float32: no fold kernel
    s4 = DeviceLatentStore(w4, seed=83)
    s4.paginate(seed=84)
    o4 = torch.empty(1, w4.H, 1, w4.d, device="cuda")
    got = lla.lla_decode_attn_paged_status(s4.dims, s4.codec, s4.cache, s4.pages, 0, w4.n, None,
                                           s4.t["q"][0, 0], 0, 1, o4, ws, ws.numel(),
                                           lla.make_opts(0, lla.LLA_PATH_ROTARY_FOLD))
    assert got == lla.LLA_ERR_UNSUPPORTED
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# decoupled-RoPE absorbed decode over a paged cache (latents and rotary keys in pages)
# ---------------------------------------------------------------------------

def _oracle_absorbed_paged(st, layer, loop_begin, loop_count, seqs, n_ctx, ctx_lens=None):
    t, w = st.t, st.w
    idx = torch.as_tensor(list(seqs), device=st.device)
    table = st.block_table.index_select(0, idx).cpu().numpy()
    q = t["q"][layer, loop_begin:loop_begin + loop_count].permute(1, 2, 0, 3).index_select(0, idx)
    lens = None if ctx_lens is None else [int(ctx_lens[i]) for i in seqs]
    return O.decode_absorbed_paged(f64(t["c_k"][layer]), f64(t["c_v"][layer]), f64(t["k_rope"][layer]),
                                   table, f64(t["w_up_k"][layer]), f64(t["mu_k"][layer]),
                                   f64(t["w_up_v"][layer]), f64(t["mu_v"][layer]), f64(q), w.d_rope,
                                   loop_begin, lens, n_ctx, None,
                                   "per_head" if w.variant == "per_head" else "2d")


@pytest.mark.parametrize("name,d_rope,splits", [
    ("ouro_layer_4x", 64, 0),
    ("ouro_layer_4x", 32, 3),
    ("capacity_21x", 32, 0),
    ("capacity_21x", 64, 2),
    ("tiny_f32", 16, 0),
    ("tiny_f32", 32, 3),
    ("lla2d_long", 64, 2),
])
def test_absorbed_shuffled_pool_matches_dense_and_oracle(name, d_rope, splits):
    """The dense and paged absorbed decodes run the same arithmetic on the same rows (the
    rotary keys through the same pages as the latents): bit for bit equal, and equal to
    the oracle's decode over the gathered pages. Ragged contexts, NaN in spare pages."""
    w = WORKLOADS[name].replace(batch=3, n=300, D=2, d_rope=d_rope,
                                **({"H": 4} if name != "tiny_f32" else {}))
    st = DeviceLatentStore(w, seed=81)
    lens = [300, 141, 1]
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    opts = lla.make_opts(splits)
    dense = st.decode_absorbed(1, 0, w.T, ctx_lens=ctx, opts=opts).clone()
    st.paginate(seed=82, spare_pages=4)
    paged = st.decode_absorbed_paged(1, 0, w.T, ctx_lens=ctx, opts=opts)
    torch.cuda.synchronize()
    ref = _oracle_absorbed_paged(st, 1, 0, w.T, range(3), w.n, lens)
    tol = F32_TOL if w.dtype == "f32" else BF16_TOL
    err = max_abs(f64(paged), ref)
    same = torch.equal(paged, dense)
    announce(f"absorbed paged {name} d_rope={d_rope} splits={splits}: {rel_note(err, tol)}; "
             f"bit-identical to dense: {same}")
    assert err <= tol
    assert same


def test_absorbed_full_launch_paged_matches_dense():
    """The absorbed 4x launch (8 x 16 heads, context 32768, 64-wide rotary branch) on a
    shuffled pool equals the dense cache bit for bit; one sequence against the oracle."""
    w = WORKLOADS["absorbed_4x"].replace(D=1)
    announce("absorbed_4x paged full launch, B=8 n=32768")
    st = DeviceLatentStore(w, seed=83)
    dense = st.decode_absorbed(0, 2, 1).clone()
    st.paginate(seed=84, spare_pages=3)
    paged = st.decode_absorbed_paged(0, 2, 1)
    torch.cuda.synchronize()
    same = torch.equal(paged, dense)
    ref = _oracle_absorbed_paged(st, 0, 2, 1, [5], w.n)
    err = max_abs(f64(paged[[5]]), ref)
    announce(f"  bit-identical to dense: {same}; sequence 5: {rel_note(err, BF16_TOL)}")
    assert same
    assert err <= BF16_TOL


def test_absorbed_paged_invalid_arguments():
    w = WORKLOADS["ouro_layer_4x"].replace(batch=2, n=64, D=1, H=4, d_rope=64)
    st = DeviceLatentStore(w, seed=85)
    st.paginate(seed=86)
    out = torch.empty(w.batch, w.H, 1, w.d, device="cuda")
    nb = lla.lla_decode_absorbed_paged_workspace_bytes(st.dims, 64, w.n, 1)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    q = st.t["q"][0, 0]
    args = (st.dims, st.codec, st.cache)
    tail = (st.t["k_rope"], 64, 0, w.n, None, q, 0, 1, out, ws, ws.numel())
    assert lla.lla_decode_attn_absorbed_paged_status(*args, st.pages, *tail) == lla.LLA_OK
    assert lla.lla_decode_attn_absorbed_paged_status(*args, None, *tail) == lla.LLA_ERR_INVALID_ARG
    bad = lla.make_pages(st.block_table, 1, st.pages.num_pages)  # max_blocks * 16 < n_max
    assert lla.lla_decode_attn_absorbed_paged_status(*args, bad, *tail) == lla.LLA_ERR_INVALID_ARG
    tail48 = (st.t["k_rope"], 48) + tail[2:]
    assert lla.lla_decode_attn_absorbed_paged_status(*args, st.pages, *tail48) == lla.LLA_ERR_UNSUPPORTED
    small = (st.t["k_rope"], 64, 0, w.n, None, q, 0, 1, out, ws, nb - 256)
    if nb >= 256:
        assert lla.lla_decode_attn_absorbed_paged_status(*args, st.pages, *small) == lla.LLA_ERR_WORKSPACE
