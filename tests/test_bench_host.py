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


def test_roofline_bound_follows_the_ridge():
    # below the bf16 ridge (2.5e15 / 8e12 = 312.5 flop/B): HBM; above it: matrix cores
    r = bench.roofline(8e9, 8e9 * 300, 1.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(8000.0) and r["frac"] == pytest.approx(1.0)
    r = bench.roofline(1e9, 1e9 * 400, 1.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(400.0) and r["frac"] == pytest.approx(0.16)


def test_source_hash_is_stable_and_covers_every_kind():
    for kind in bench.KERNEL_SOURCES:
        for f in bench.KERNEL_SOURCES[kind]:
            assert os.path.exists(os.path.join(ROOT, "latent_decode_attention_lla_amd", "csrc", f)), f
        assert bench.kernel_source_hash(kind) == bench.kernel_source_hash(kind)
    assert len({bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES}) == len(bench.KERNEL_SOURCES)


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json"))),
                         ids=lambda p: os.path.basename(p))
def test_committed_traffic_matches_current_sources(path):
    """Every committed FETCH_SIZE / WRITE_SIZE summary was taken on the sources the call
    has now, so bench.py reports it; and its bytes are close to the algorithmic bytes."""
    tr = json.load(open(path))
    kind, workload = tr["call"], tr["workload"]
    assert os.path.basename(path) == f"{kind}_{workload}_traffic.json"
    assert tr["kernel_source_hash"] == bench.kernel_source_hash(kind), \
        f"{path} is stale: re-take it for the changed {kind} sources"
    assert bench.measured_traffic(kind, workload, tr["path"]) == tr["hbm_bytes_per_launch"]
    assert 0.99 < tr["traffic_over_algorithmic"] < 2.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
