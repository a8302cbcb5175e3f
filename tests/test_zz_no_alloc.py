"""lla_decode_attn_noalloc: lla_decode_attn with its split partials in the library's fixed
device array instead of a caller's workspace, for callers that cannot allocate. Its
results must be those of lla_decode_attn (the same kernels on the same plan), on
consecutive calls whose second one is smaller (the array keeps the first call's
contents), and sizes beyond the array are refused before anything runs."""

import numpy as np
import pytest
import torch

from latent_decode_attention_lla_amd import lla
from latent_decode_attention_lla_amd.harness import DeviceLatentStore
from latent_decode_attention_lla_amd.inputs import WORKLOADS
from tests.gpu_util import (BF16_TOL, F32_TOL, announce, ensure_built, f64, max_abs,
                            oracle_decode, rel_note)

RECON = lla.LLA_PATH_RECONSTRUCT


def _call_noalloc(st, layer, loop_begin, loop_count, n_ctx, ctx_lens, opts):
    w = st.w
    q = st.t["q"][layer, loop_begin:loop_begin + loop_count].permute(1, 2, 0, 3).contiguous()
    out = torch.full((w.batch, w.H, loop_count, w.d), float("nan"), device=st.device)
    lla.lla_decode_attn_noalloc(st.dims, st.codec, st.cache, layer, n_ctx, ctx_lens, q,
                                loop_begin, loop_count, out, opts)
    return out


# (workload, overrides for the first and the second, smaller, call, splits, path)
CASES = {
    "narrow_fold": ("capacity_21x", dict(batch=6, n=1000), dict(batch=2, n=300), 3, 0),
    "wide_fold": ("ouro_layer_4x", dict(batch=4, n=900, H=4), dict(batch=1, n=77, H=4), 2, 0),
    "lla2d": ("lla2d_long", dict(batch=3, n=1000), dict(batch=2, n=200), 3, 0),
    "reconstruct_f32": ("tiny_f32", dict(batch=3, n=128), dict(batch=1, n=40), 1, RECON),
}


@pytest.mark.gpu
@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_matches_decode_with_workspace(case):
    ensure_built()
    name, first, second, splits, path = CASES[case]
    for k, over in enumerate((first, second)):
        w = WORKLOADS[name].replace(D=1, **over)
        announce(f"noalloc {case} call {k + 1}: B={w.batch} H={w.H} n={w.n} splits={splits}")
        st = DeviceLatentStore(w, seed=91 + k, n_alloc=w.n + 16)
        lens = [w.n - 5 * b for b in range(w.batch)]
        ctx = torch.tensor(lens, dtype=torch.int32, device=st.device)
        opts = lla.make_opts(splits, path)
        ref_ws = st.decode(0, 0, w.T, n_ctx=w.n, ctx_lens=ctx, opts=opts)
        got = _call_noalloc(st, 0, 0, w.T, w.n, ctx, opts)
        torch.cuda.synchronize()
        tol = F32_TOL if w.dtype == "f32" else BF16_TOL
        err = max_abs(f64(got), oracle_decode(st, 0, 0, w.T, range(w.batch), w.n, ctx_lens=lens))
        same = torch.equal(got, ref_ws)
        announce(f"  {rel_note(err, tol)}; identical to the workspace call: {same}")
        assert err <= tol
        assert same


def test_noalloc_refuses_sizes_beyond_its_array():
    """Partials larger than the array give LLA_ERR_WORKSPACE; invalid arguments give the
    decode's own status. Both are decided on the host, before any HIP call."""
    lla.load()
    w = WORKLOADS["ouro_layer_4x"].replace(batch=64, n=8192)
    dims = lla.make_dims(w.T, w.D, w.H, w.d, w.r_k, w.r_v, w.batch, w.n, lla.LLA_PER_HEAD,
                         lla.LLA_BF16, w.rope_base, 0.0)
    opts = lla.make_opts(32, 0)
    need = lla.lla_decode_workspace_bytes(dims, w.n, 4, opts)
    assert need > lla.LLA_NOALLOC_SCRATCH_BYTES
    fake = 1 << 20  # never dereferenced: the call is refused first
    codec = lla.make_codec(fake, fake, fake, fake, fake, fake, fake)
    cache = lla.make_cache(fake, fake)
    with pytest.raises(lla.LLAError) as e:
        lla.lla_decode_attn_noalloc(dims, codec, cache, 0, w.n, None, fake, 0, 4, fake, opts, 0)
    assert e.value.status == lla.LLA_ERR_WORKSPACE
    with pytest.raises(lla.LLAError) as e:
        lla.lla_decode_attn_noalloc(dims, codec, cache, 5, w.n, None, fake, 0, 4, fake, opts, 0)
    assert e.value.status == lla.LLA_ERR_INVALID_ARG
