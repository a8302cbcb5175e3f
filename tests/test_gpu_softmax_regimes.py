"""GPU parity of every decode kernel in the large-score regimes of tests/softmax_regimes.py
(score spreads of 30-70, a running maximum raised late with live state, an explicit score
scale, RoPE base 1e6), through the C ABI, every output against the fp64 oracle at the
bfloat16 bar. Attention is unchanged by the codec ("Looped Latent Attention", Figure 1
caption), so these regimes must hold to the same bar as unit-scale queries.

Kernels: the narrow and wide rotary folds, the wide fold on an LLA-2D shape, the LLA-2D
kernel (8 heads per workgroup at H = 16, 4 at H = 4 and 12), the reconstruct path, the
decoupled-RoPE absorbed decode and the uncompressed decode; one and three context splits;
the paged instances must also reproduce the dense results bit for bit. The CPU test
tests/test_softmax_regimes.py shows that on these inputs a kernel without the rescale
would miss the oracle by far more than the bar."""

import numpy as np
import pytest
import torch

from latent_decode_attention_lla_amd import lla
from latent_decode_attention_lla_amd.harness import DeviceLatentStore, DeviceTeacherCache
from latent_decode_attention_lla_amd.inputs import WORKLOADS
from tests import softmax_regimes as R
from tests.gpu_util import (BF16_TOL, announce, ensure_built, f64, max_abs, oracle_decode,
                            oracle_decode_absorbed, oracle_decode_teacher, rel_note)

pytestmark = pytest.mark.gpu

FOLD = lla.LLA_PATH_ROTARY_FOLD
RECON = lla.LLA_PATH_RECONSTRUCT


def _w(name, **kw):
    return WORKLOADS[name].replace(D=1, batch=2, n=1000, **kw)


# kernel id -> (workload, decode kind, path, paged instance to compare)
KERNELS = {
    "narrow_fold": (_w("capacity_21x", H=8), "latent", FOLD, True),
    "narrow_fold_h4": (_w("capacity_21x", H=4), "latent", FOLD, False),
    "wide_fold": (_w("ouro_layer_4x", H=4), "latent", FOLD, True),
    "wide_fold_2d": (_w("lla2d_long", H=16, r_k=128, r_v=128), "latent", FOLD, False),
    "lla2d_h16": (_w("lla2d_long", H=16), "latent", FOLD, True),
    "lla2d_h4": (_w("lla2d_long", H=4), "latent", FOLD, True),
    "lla2d_h12": (_w("lla2d_long", H=12), "latent", FOLD, False),
    "reconstruct": (_w("capacity_21x", H=4), "latent", RECON, False),
    "reconstruct_2d": (_w("lla2d_long", H=4), "latent", RECON, False),
    "absorbed": (_w("ouro_layer_4x", H=4, d_rope=64), "absorbed", None, True),
    "teacher": (_w("teacher_4k", H=4), "teacher", None, False),
}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


@pytest.mark.parametrize("regime", R.REGIMES)
@pytest.mark.parametrize("kernel", list(KERNELS))
def test_large_score_regime_every_output(kernel, regime):
    base, kind, path, check_paged = KERNELS[kernel]
    w = R.regime_workload(base, regime)
    announce(f"{kernel} {regime}: B={w.batch} H={w.H} n={w.n} ranks=({w.r_k}, {w.r_v}) "
             f"scale={w.scale} base={w.rope_base:g}")
    t, planted = R.build(w, regime, seed=401)
    spread = float(np.ptp(R.scores_exp2(w, t, 0, 0, 0, 0, w.n))) / R.LOG2E
    if kind == "teacher":
        st = DeviceTeacherCache(w, seed=0, tensors=t)
        ref = oracle_decode_teacher(st, 0, 0, w.T, range(w.batch), w.n)
    else:
        st = DeviceLatentStore(w, seed=0, tensors=t)
        oracle = oracle_decode_absorbed if kind == "absorbed" else oracle_decode
        ref = oracle(st, 0, 0, w.T, range(w.batch), w.n)
    if planted:  # the planted token holds nearly all the weight: the output is near V_t[j*]
        for (b, h, loop), js in list(planted.items())[:4]:
            v = R.value_rows(w, t, 0, loop, b, h, w.n)[js]
            assert np.max(np.abs(ref[b, h, loop] - v)) < 0.1
    dense = {}
    for splits in (1, 3):
        opts = lla.make_opts(splits, path if path is not None else lla.LLA_PATH_AUTO)
        if kind == "absorbed":
            out = st.decode_absorbed(0, 0, w.T, opts=opts)
        else:
            out = st.decode(0, 0, w.T, opts=opts)
        torch.cuda.synchronize()
        got = f64(out)
        err = max_abs(got, ref)
        announce(f"  splits={splits}: spread {spread:.1f}, {rel_note(err, BF16_TOL)}")
        assert np.isfinite(got).all()
        assert err <= BF16_TOL
        dense[splits] = out.clone()
    if check_paged:
        st.paginate(seed=402, spare_pages=3)
        for splits in (1, 3):
            opts = lla.make_opts(splits, path if path is not None else lla.LLA_PATH_AUTO)
            if kind == "absorbed":
                paged = st.decode_absorbed_paged(0, 0, w.T, opts=opts)
            else:
                paged = st.decode_paged(0, 0, w.T, opts=opts)
            torch.cuda.synchronize()
            assert torch.equal(paged, dense[splits]), f"paged {kernel} splits={splits} differs from dense"
