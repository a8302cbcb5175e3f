"""The large-score decode inputs of tests/softmax_regimes.py are strong enough to catch a
kernel that forgets to rescale.

The decode kernels keep an online softmax whose running maximum is raised lazily: per
token column of a 16-token tile (the narrow and wide folds, the absorbed and uncompressed
decodes) or per head over a whole tile (the LLA-2D kernel), and only when a score beats
it by more than 8 in the exp2 domain. Raising the maximum must rescale the running sum
and the accumulator. With queries ~ N(0, 1) such a raise almost never meets live state,
so a kernel without the rescale would still pass. Here the same schedule is simulated in
float64 on the regime inputs: with the rescale it must equal the oracle, and without it
it must miss the oracle by far more than the 2e-2 bar, after raises with live state.
CPU only; the GPU parity on the same inputs is tests/test_gpu_softmax_regimes.py."""

import numpy as np
import pytest

from latent_decode_attention_lla_amd.inputs import WORKLOADS
from oracle import lla_oracle as O
from tests import softmax_regimes as R

SLACK = 8.0


def lazy_online_softmax(s2, v, per_tile: bool, rescale: bool):
    """Weighted mean of the rows of v under softmax weights of the exp2-domain scores s2,
    by a lazily raised running maximum per token column (or per tile), merged at the end.
    Returns (output, raises that met a non-zero running sum)."""
    cols = 1 if per_tile else 16
    m = np.full(cols, -1.0e30)
    l = np.zeros(cols)
    acc = np.zeros((cols, v.shape[1]))
    live = 0
    for j0 in range(0, len(s2), 16):
        tile = s2[j0:j0 + 16]
        for c in range(cols):
            top = tile.max() if per_tile else (tile[c] if c < len(tile) else -np.inf)
            if top > m[c] + SLACK:
                live += int(l[c] > 0)
                if rescale:
                    alpha = np.exp2(m[c] - top)
                    l[c] *= alpha
                    acc[c] *= alpha
                m[c] = top
        for i, s in enumerate(tile):
            c = 0 if per_tile else i
            p = np.exp2(s - m[c])
            l[c] += p
            acc[c] += p * v[j0 + i]
    mx = m.max()
    w = np.exp2(m - mx)
    return (w @ acc) / (w @ l), live


CASES = {
    "narrow_fold_shape": WORKLOADS["capacity_21x"].replace(D=1, batch=2, n=1000, H=8),
    "wide_fold_shape": WORKLOADS["ouro_layer_4x"].replace(D=1, batch=2, n=1000, H=4),
    "lla2d_shape": WORKLOADS["lla2d_long"].replace(D=1, batch=2, n=1000, H=16),
    "absorbed_shape": WORKLOADS["ouro_layer_4x"].replace(D=1, batch=2, n=1000, H=4, d_rope=64),
    "teacher_shape": WORKLOADS["teacher_4k"].replace(D=1, batch=2, n=1000, H=4),
}


@pytest.mark.parametrize("regime", ["spread", "planted"])
@pytest.mark.parametrize("case", list(CASES))
def test_forgotten_rescale_fails_on_regime_inputs(case, regime):
    w = R.regime_workload(CASES[case], regime)
    t, planted = R.build(w, regime, seed=301)
    per_tile = case == "lla2d_shape"
    good_err, bad_err, live = 0.0, 0.0, 0
    for h in (0, w.H - 1):
        for loop in range(w.T):
            s2 = R.scores_exp2(w, t, 0, loop, 0, h, w.n)
            v = R.value_rows(w, t, 0, loop, 0, h, w.n)
            a = np.exp2(s2 - s2.max())
            ref = (a / a.sum()) @ v  # textbook softmax over the oracle's key and value rows
            good, n_live = lazy_online_softmax(s2, v, per_tile, True)
            bad, _ = lazy_online_softmax(s2, v, per_tile, False)
            good_err = max(good_err, float(np.max(np.abs(good - ref))))
            bad_err = max(bad_err, float(np.max(np.abs(bad - ref))))
            live += n_live
            if regime == "planted":  # near the large-alpha limit: j* takes the weight
                assert a[planted[(0, h, loop)]] / a.sum() > 0.99
    spread = float(np.ptp(R.scores_exp2(w, t, 0, 0, 0, 0, w.n))) / R.LOG2E
    print(f"{case} {regime}: score spread {spread:.1f}, live raises {live}, "
          f"with rescale {good_err:.1e}, without {bad_err:.2e}")
    assert 30.0 <= spread <= 80.0
    assert live > 0
    assert good_err < 1e-9
    assert bad_err > 0.1  # five times the 2e-2 bar


def test_regime_outputs_match_oracle_decode():
    """The textbook softmax above equals oracle.decode on the same inputs (so the regime
    helpers read the rows the oracle reads)."""
    w = R.regime_workload(CASES["narrow_fold_shape"], "scale")
    t, _ = R.build(w, "scale", seed=302)
    f = R._f64
    out = O.decode(f(t["c_k"][0, :1]), f(t["c_v"][0, :1]), f(t["w_up_k"][0]), f(t["mu_k"][0]),
                   f(t["w_up_v"][0]), f(t["mu_v"][0]),
                   f(t["q"][0].permute(1, 2, 0, 3)[:1]), 0, None, w.rope_base, w.scale)
    for h in (0, 5):
        for loop in range(w.T):
            s2 = R.scores_exp2(w, t, 0, loop, 0, h, w.n)
            a = np.exp2(s2 - s2.max())
            ref = (a / a.sum()) @ R.value_rows(w, t, 0, loop, 0, h, w.n)
            assert np.max(np.abs(out[0, h, loop] - ref)) < 1e-12
