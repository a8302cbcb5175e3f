"""The decode entry points under HIP graph capture: every kernel they launch goes to the
caller's stream, they allocate nothing and clear nothing with a memset, so a captured
call replays to the same result. Each case captures one call (with several context splits,
so the split kernel and the merge are both in the graph), replays it three times with the
program's own eager work and synchronisations in between, and compares every replay with
the eager result bit for bit."""

import pytest
import torch

from latent_decode_attention_lla_amd import lla
from latent_decode_attention_lla_amd.harness import DeviceLatentStore
from latent_decode_attention_lla_amd.inputs import WORKLOADS
from tests.gpu_util import announce, ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


@pytest.mark.parametrize("name,kind", [
    ("capacity_21x", "fold"),        # narrow rotary fold
    ("ouro_layer_4x", "fold"),       # wide rotary fold
    ("lla2d_long", "fold"),          # LLA-2D kernel
    ("capacity_21x", "reconstruct"),
    ("ouro_layer_4x", "absorbed"),
    ("capacity_21x", "paged"),
    ("lla2d_long", "paged"),
])
def test_graph_replay_matches_eager(name, kind):
    over = {"d_rope": 64} if kind == "absorbed" else {}
    w = WORKLOADS[name].replace(D=2, batch=4, n=700, H=4, **over)
    st = DeviceLatentStore(w, seed=91)
    if kind == "paged":
        st.paginate(seed=92, spare_pages=2)
    out = torch.empty(w.batch, w.H, 1, w.d, dtype=torch.float32, device="cuda")
    path = lla.LLA_PATH_RECONSTRUCT if kind == "reconstruct" else lla.LLA_PATH_AUTO
    opts = lla.make_opts(3, path)

    def call():
        if kind == "absorbed":
            st.decode_absorbed(1, 2, 1, opts=opts, out=out)
        elif kind == "paged":
            st.decode_paged(1, 2, 1, opts=opts, out=out)
        else:
            st.decode(1, 2, 1, opts=opts, out=out)

    call()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as graph capture expects
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(out, ref)
        announce(f"graph replay {rep} {name} {kind}: bit-identical to eager: {same}")
        assert same
