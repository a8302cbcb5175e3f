"""Host logic of bench.py, on the CPU: the algorithmic bytes and flops per call (closed
forms of the workloads' shapes), the roofline choice, the committed HBM-traffic summaries
(each must still match the sources of the call it measured), and the one-GPU guard."""

import glob
import json
import os
import subprocess
import sys

import pytest

import bench
from latent_decode_attention_lla_amd.inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_headline_decode_bytes_and_flops():
    """768 x 16 heads x 4096 tokens of (16 + 32) bf16 latents, float32 q and out per
    (sequence, head), one loop's W_up,k / W_up,v slices and mu slices; 2 r_k d matrix-core
    flops per (token, head) to rebuild the keys."""
    w = WORKLOADS["capacity_21x"]
    nbytes, flops = bench.algorithmic(w, "decode")
    tok = 768 * 16 * 4096
    assert nbytes == tok * 48 * 2 + 2 * 768 * 16 * 128 * 4 + 16 * 128 * 48 * 2 + 2 * 16 * 128 * 2
    assert nbytes == 4_844_625_920
    assert flops == 2.0 * tok * 16 * 128


def test_lla2d_flops_count_the_shared_value_product():
    w = WORKLOADS["lla2d_long"]
    nbytes, flops = bench.algorithmic(w, "decode")
    assert nbytes == 16 * 16384 * 256 * 2 + 2 * 16 * 16 * 128 * 4 + 16 * 128 * 256 * 2 + 2 * 16 * 128 * 2
    assert flops == 2.0 * 16 * 16384 * 16 * (96 * 128 + 160)


def test_absorbed_bytes_include_the_rotary_keys():
    w = WORKLOADS["absorbed_4x"]
    plain, _ = bench.algorithmic(w.replace(d_rope=0), "decode")
    nbytes, flops = bench.algorithmic(w, "decode")
    assert nbytes - plain == 8 * 16 * 32768 * 64 * 2
    assert flops == 2.0 * 8 * 16 * 32768 * (96 + 64 + 160)


def test_encode_bytes():
    """x_k and x_v read once, latents written once, W_down and mu read once."""
    w = WORKLOADS["ouro_layer_4x"]
    nbytes, flops = bench.algorithmic(w, "encode", n_new=4096)
    toks = 32 * 4096 * 16
    K = 4 * 128
    assert nbytes == 2 * toks * K * 2 + toks * 256 * 2 + 16 * 256 * K * 2 + 2 * 16 * K * 2
    assert flops == 2.0 * toks * K * 256


def test_roofline_reports_both_fractions_and_the_binding_resource():
    # 8 GB in 1 ms is the HBM peak: HBM-bound, whatever the flops
    r = bench.roofline(8e9, 8e9 * 300, 1.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["binding"] == "hbm"
    assert r["achieved"] == pytest.approx(8000.0) and r["frac"] == pytest.approx(1.0)
    assert r["mfma_frac"] == pytest.approx(0.96)
    # 1.5 PFLOP/s of bf16 MFMA: matrix-core bound
    r = bench.roofline(1e9, 1.5e12, 1.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["binding"] == "mfma"
    assert r["frac"] == pytest.approx(0.6) and r["hbm_frac"] == pytest.approx(0.125)
    # neither roof within half of its peak: issue-bound, quoted against the nearer roof, and
    # the measured traffic counts toward the HBM fraction
    ctr = {"wave_wait_frac": 0.35}
    r = bench.roofline(1e9, 6.5e11, 1.0, traffic=2e9, counters=ctr)
    assert r["bound"] == "mfma" and r["frac"] == pytest.approx(0.26)
    assert r["measured_hbm_frac"] == pytest.approx(0.25) and r["binding"] == "issue"
    assert r["counters"] == ctr
    r = bench.roofline(1e9, 1e11, 1.0, traffic=4.5e9)
    assert r["bound"] == "hbm" and r["binding"] == "hbm"  # measured traffic reaches the roof


def test_source_hash_is_stable_and_covers_every_kind():
    for kind in bench.KERNEL_SOURCES:
        for f in bench.KERNEL_SOURCES[kind]:
            assert os.path.exists(os.path.join(ROOT, "latent_decode_attention_lla_amd", "csrc", f)), f
        assert bench.kernel_source_hash(kind) == bench.kernel_source_hash(kind)
    assert len({bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES}) == len(bench.KERNEL_SOURCES)


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json"))),
                         ids=lambda p: os.path.basename(p))
def test_committed_traffic_is_reported_only_while_current(path):
    """A committed FETCH_SIZE / WRITE_SIZE summary is reported by bench.py exactly while it
    was taken on the sources the call has now (a changed kernel reports no traffic until
    it is re-taken); and its bytes are close to the algorithmic bytes."""
    tr = json.load(open(path))
    kind, workload = tr["call"], tr["workload"]
    assert path == bench.traffic_file(kind, workload, tr["path"])
    got = bench.measured_traffic(kind, workload, tr["path"])
    if tr["kernel_source_hash"] == bench.kernel_source_hash(kind, tr["kernel"]):
        assert got == tr["hbm_bytes_per_launch"]
    else:
        assert got is None
    assert 0.99 < tr["traffic_over_algorithmic"] < 2.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_source_hash_does_not_depend_on_where_the_checkout_lives(monkeypatch, tmp_path):
    """The compile flags enter the hash with include paths relative to the repository, so
    a copy of the tree elsewhere (or reached through a symlink) hashes the same."""
    from latent_decode_attention_lla_amd import build as B
    before = {k: bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES}
    link = tmp_path / "checkout"
    link.symlink_to(bench.ROOT)
    monkeypatch.setattr(B, "HIP_FLAGS", [f.replace(bench.ROOT, str(link)) if f.startswith(bench.ROOT) else f
                                         for f in B.HIP_FLAGS])
    assert any(str(link) in f for f in B.HIP_FLAGS)
    assert {k: bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES} == before


def test_decode_summary_hash_follows_the_measured_kernel_only():
    """A decode summary taken on one decode kernel hashes that kernel's file (and the shared
    sources), so an edit to another decode kernel leaves it current; the full call hash
    still covers every decode kernel."""
    fold = bench.kernel_sources("decode", "decode_rotary_fold_kernel<128, 16, 32, 4, 4, false>")
    assert "decode_rotary_fold.hip" in fold and "decode_reconstruct.hip" not in fold
    assert "combine.hip" in fold and "lla_plan.h" in fold
    both = bench.kernel_sources("decode", ["decode_reconstruct_bf16_kernel<...>", "combine_kernel<...>"])
    assert "decode_reconstruct.hip" in both and "decode_fold_wide.hip" not in both
    assert bench.kernel_sources("decode") == bench.KERNEL_SOURCES["decode"]
    assert bench.kernel_sources("decode", "some_other_kernel") == bench.KERNEL_SOURCES["decode"]
    assert bench.kernel_source_hash("decode", "decode_lla2d_kernel") != bench.kernel_source_hash("decode")
    # non-decode calls ignore the kernel name
    assert bench.kernel_source_hash("encode", "decode_lla2d_kernel") == bench.kernel_source_hash("encode")
