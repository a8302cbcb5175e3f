"""GPU parity of lla_encode_fused (the projection-fused, loop-incremental encode: Section 3,
Eqs. 1-2 of "Looped Latent Attention"; Appendix J, "Eviction and long-context prefill")
against the fp64 oracle's encode_fused.

Bound for stored latents. Per loop t the GPU forms x~_t = h_t W_proj with float32
accumulation over d_model products of bfloat16 values (exact products), subtracts mu_t in
float32, splits v = x~ - mu into bfloat16 hi + lo parts (v - hi is exact; lo drops at most
2^-16 |v|), and accumulates (hi + lo) W_down over the loop's columns, then over the loops,
in float32; the last loop rounds once to bfloat16. With u = 2^-24, K = T d_in, for every
latent entry e
  |y - c| <= delta = sum_k |W_down[k, e]| ((d_model + 2) u S_k + (2^-16 + (2K + T + 4) u) |x_k - mu_k|) * 1.01,
where S_k = sum_m |h_m W_proj[m, k]| bounds the projection's float32 error, the second
term the centering, the split and the second product's accumulation (standard float
dot-product bounds), and 1.01 covers the second-order terms. The stored value then
differs from the oracle's rounded latent by at most one bfloat16 spacing plus delta.
"""

import numpy as np
import pytest
import torch

from latent_decode_attention_lla_amd import lla
from latent_decode_attention_lla_amd.harness import dims_for
from latent_decode_attention_lla_amd.inputs import (WORKLOADS, Workload, fused_encode_inputs,
                                                    gaussian_encode_codec)
from oracle import lla_oracle as O
from tests.gpu_util import announce, bf16_ulp, ensure_built, f64

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


class Fused:
    """Device tensors of one fused-encode problem and the T calls of a layer."""

    def __init__(self, w: Workload, d_model: int, n_new: int, n_max: int, seed: int):
        dev = torch.device("cuda")
        self.w, self.d_model, self.n_new, self.n_max = w, d_model, n_new, n_max
        self.h, self.w_k, self.w_v = fused_encode_inputs(w, n_new, d_model, seed, device=dev)
        self.codec_t = gaussian_encode_codec(w, seed + 1, device=dev)
        dt = w.torch_dtype
        self.c_k = torch.full((w.D, w.batch, w.Hc, n_max, w.r_k), SENTINEL, dtype=dt, device=dev)
        self.c_v = torch.full((w.D, w.batch, w.Hc, n_max, w.r_v), SENTINEL, dtype=dt, device=dev)
        self.dims = dims_for(w, n_max=n_max)
        ct = self.codec_t
        self.codec = lla.make_codec(ct["w_down_k_t"], ct["mu_k"], None, ct["w_down_v_t"], ct["mu_v"])
        self.proj = lla.make_proj(self.w_k, self.w_v, d_model)
        self.cache = lla.make_cache(self.c_k, self.c_v)
        self.acc_bytes = lla.lla_encode_fused_acc_bytes(self.dims, n_new)
        self.acc = torch.empty(max(self.acc_bytes, 256) // 4, dtype=torch.float32, device=dev)

    def call(self, layer: int, loop: int, pos_start: int):
        lla.lla_encode_fused(self.dims, self.codec, self.proj, self.cache, layer, loop,
                             self.h[loop], pos_start, self.n_new, self.acc, self.acc_bytes)

    def encode_layer(self, layer: int, pos_start: int, check_untouched: bool = False):
        for t in range(self.w.T):
            if check_untouched and t == self.w.T - 1:
                torch.cuda.synchronize()
                for c in (self.c_k, self.c_v):
                    assert bool((c[layer] == SENTINEL).all()), "cache written before the last loop"
            self.call(layer, t, pos_start)
        torch.cuda.synchronize()

    def oracle(self, layer: int, axis: str, b: int, toks=None):
        """(rounded latents [n][Hc][r], bound delta) of sequence b's new tokens `toks` (all
        when None) from the oracle."""
        w = self.w
        hb = self.h[:, b] if toks is None else self.h[:, b][:, torch.as_tensor(toks, device=self.h.device)]
        hl = f64(hb)  # [T][n][d_model]
        wp = f64((self.w_k if axis == "k" else self.w_v)[layer]).T  # [d_model][H d]
        wd = f64(self.codec_t[f"w_down_{axis}_t"][layer]).transpose(0, 2, 1)  # [Hc][K][r]
        mu = f64(self.codec_t[f"mu_{axis}"][layer])
        variant = "per_head" if w.variant == "per_head" else "2d"
        c = O.encode_fused(hl, wp, mu, wd, w.H, w.d, variant)
        # error bound (needs |x - mu| and S per stacked column; x itself from the same fp64
        # products the bound is about, not an expected value)
        T, n = hl.shape[:2]
        x = np.stack([hl[t] @ wp for t in range(T)])            # [T][n][H d]
        s = np.stack([np.abs(hl[t]) @ np.abs(wp) for t in range(T)])
        K = w.T * w.d_in
        u = 2.0 ** -24
        delta = np.empty_like(c)
        for hc in range(w.Hc):
            if variant == "per_head":
                xs, ss = x[:, :, hc * w.d:(hc + 1) * w.d], s[:, :, hc * w.d:(hc + 1) * w.d]
            else:
                xs, ss = x, s
            xs = np.transpose(xs, (1, 0, 2)).reshape(n, K)     # (t, column) stacking
            ss = np.transpose(ss, (1, 0, 2)).reshape(n, K)
            term = (self.d_model + 2) * u * ss + (2.0 ** -16 + (2 * K + T + 4) * u) * np.abs(xs - mu[hc])
            delta[:, hc] = 1.01 * (term @ np.abs(wd[hc]))
        return O.round_bf16(c), delta

    def check(self, layer: int, pos_start: int, seqs=None, toks=None):
        w = self.w
        worst = 0.0
        for axis, cache in (("k", self.c_k), ("v", self.c_v)):
            got_all = f64(cache[layer])  # [B][Hc][n_max][r]
            for b in (range(w.batch) if seqs is None else seqs):
                ref, delta = self.oracle(layer, axis, b, toks)
                rows = (np.arange(pos_start, pos_start + self.n_new) if toks is None
                        else pos_start + np.asarray(toks))
                got = got_all[b][:, rows].transpose(1, 0, 2)
                err = np.abs(got - ref)
                allowed = bf16_ulp(ref) + delta
                bad = err > allowed * (1 + 1e-12)
                assert not bad.any(), (f"{axis} seq {b}: {int(bad.sum())} latents beyond one "
                                       f"bf16 spacing + delta (max excess "
                                       f"{float(np.max(err - allowed)):.3e})")
                worst = max(worst, float(np.max(err / bf16_ulp(ref))))
                if toks is not None:
                    continue
                rest = np.concatenate([got_all[b][:, :pos_start], got_all[b][:, pos_start + self.n_new:]],
                                      axis=1)
                assert np.all(rest == SENTINEL), f"{axis} seq {b}: rows outside the range written"
        return worst


def _wl(name, **kw) -> Workload:
    return WORKLOADS[name].replace(**kw)


@pytest.mark.parametrize("w,d_model,n_new,pos_start", [
    # Ouro-1.4B 4x geometry, hidden 2048: two sequences whose 300 new tokens straddle
    # the 128-token blocks (the third block holds both sequences and a ragged tail)
    (_wl("ouro_layer_4x", D=2, batch=2, n=340), 2048, 300, 20),
    # capacity_21x ranks (16, 32)
    (_wl("capacity_21x", D=2, batch=1, n=200), 2048, 131, 7),
    # LLA-2D at the 4x geometry (K = 8192 stacked columns)
    (_wl("lla2d_long", D=2, batch=1, n=160), 2048, 150, 3),
])
def test_fused_encode_matches_oracle(w, d_model, n_new, pos_start):
    announce(f"fused encode {w.name} {w.variant} ({w.r_k},{w.r_v}) B={w.batch} n_new={n_new} "
             f"d_model={d_model}")
    f = Fused(w, d_model, n_new, w.n, seed=11)
    f.encode_layer(1, pos_start, check_untouched=True)
    assert bool((f.c_k[0] == SENTINEL).all()) and bool((f.c_v[0] == SENTINEL).all())
    ulps = f.check(1, pos_start)
    announce(f"  max {ulps:.2f} bf16 spacings")


@pytest.mark.parametrize("r_k,r_v,d_model,variant,H", [
    (16, 32, 32, "per_head", 2),     # one K chunk per head
    (64, 128, 64, "per_head", 2),    # two K chunks (ring shorter than its depth)
    (160, 96, 96, "per_head", 3),    # three chunks, odd head count
    # pairs with a two-axis kernel (d_model a multiple of 64): an odd and an even number
    # of 64-wide K steps, so the W_down rows land in either ring stage
    (32, 64, 192, "per_head", 2),
    (64, 64, 128, "per_head", 3),
    (128, 128, 64, "per_head", 1),
    (32, 16, 64, "2d", 2),
    (128, 64, 160, "2d", 3),
])
def test_fused_encode_ranks_and_short_projections(r_k, r_v, d_model, variant, H):
    w = Workload("fused_small", T=4, D=1, H=H, d=128, r_k=r_k, r_v=r_v, batch=2, n=300,
                 variant=variant)
    announce(f"fused encode ranks ({r_k},{r_v}) {variant} H={H} d_model={d_model}")
    f = Fused(w, d_model, 257, 300, seed=13)
    f.encode_layer(0, 40)
    f.check(0, 40)


@pytest.mark.parametrize("T,n_new", [(1, 45), (2, 1), (7, 129)])
def test_fused_encode_loop_counts_and_single_token(T, n_new):
    """T = 1 (the first call is also the last), one new token (one block, 127 padded
    rows), and 7 loops."""
    w = Workload("fused_loops", T=T, D=1, H=4, d=128, r_k=96, r_v=160, batch=3, n=n_new + 5)
    announce(f"fused encode T={T} n_new={n_new}")
    f = Fused(w, 256, n_new, n_new + 5, seed=17)
    f.encode_layer(0, 5)
    f.check(0, 5)


def test_fused_encode_accumulator_reuse_and_zero_tokens():
    """The accumulator carries no state between layers (loop 0 overwrites it), and
    n_new = 0 writes nothing."""
    w = Workload("fused_reuse", T=4, D=3, H=2, d=128, r_k=96, r_v=160, batch=1, n=200)
    f = Fused(w, 128, 200, 200, seed=19)
    f.acc.fill_(float("nan"))
    for layer in (2, 0):
        f.encode_layer(layer, 0)
    f.check(2, 0)
    f.check(0, 0)
    assert bool((f.c_k[1] == SENTINEL).all()) and bool((f.c_v[1] == SENTINEL).all())
    lla.lla_encode_fused(f.dims, f.codec, f.proj, f.cache, 1, 0, f.h[0], 0, 0, f.acc, 0)
    torch.cuda.synchronize()
    assert bool((f.c_k[1] == SENTINEL).all())


def test_fused_encode_prefill_64k_full_size_sampled():
    """The streamed-prefill workload at full size in the launch configuration the
    benchmark times: 65536 prompt tokens, hidden size 2048, the last of 24 layers, all
    four loops; 96 sampled tokens (both ends, block edges, random) against the oracle."""
    w = WORKLOADS["prefill_64k"]
    announce(f"fused encode prefill_64k full size: {w.n} tokens, layer {w.D - 1}")
    f = Fused(w, w.d_model, w.n, w.n, seed=23)
    f.encode_layer(w.D - 1, 0)
    rng = np.random.default_rng(23)
    toks = sorted(set([0, 1, 127, 128, 129, 4095, 4096, w.n - 129, w.n - 128, w.n - 1]
                      + rng.choice(w.n, size=86, replace=False).tolist()))
    ulps = f.check(w.D - 1, 0, toks=toks)
    announce(f"  max {ulps:.2f} bf16 spacings over {len(toks)} tokens x {w.H} heads")
    for c in (f.c_k, f.c_v):  # the other layers stay untouched
        assert bool((c[: w.D - 1] == SENTINEL).all())
