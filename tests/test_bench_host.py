"""Host checks of bench.py's arithmetic: algorithmic bytes and roofline floors.

The byte counts are the method's own traffic for one step (bf16 weights and
KV read once, the tree rows' embeddings, the fp32 hidden state, and in
exact mode the head logits written and read back for drafting), worked out
by hand below for each workload from its shape.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import WORKLOADS  # noqa: E402


def _by_hand(d, V, K, B, H, Dh, T, L_total, exact=False):
    w = 2
    heads = w * (K * d * d + K * V * d)                 # W1, W2
    verifier = w * (V * d + 4 * d * d)                  # W_lm; W_qkv (3 d^2) + W_o (d^2)
    kv = w * 2 * H * Dh * L_total
    emb = w * d * B * T
    hidden = 4 * d * B
    logits = 2 * 4 * K * V * B if exact else 0
    return heads + verifier + kv + emb + hidden + logits


@pytest.mark.parametrize("name,T,L_total,expect", [
    ("vicuna7b_typical", 46, 2048, 1_908_801_536),
    ("vicuna13b_typical", 137, 4096, 2_523_248_640),
    ("vicuna7b_exact", 46, 4096, 1_943_635_968),
])
def test_algorithmic_bytes_single_sequence(name, T, L_total, expect):
    w = WORKLOADS[name]
    got = bench.algorithmic_bytes(w, T, L_total)
    assert got == expect
    assert got == _by_hand(w.d, w.V, w.K, w.B, w.H, w.Dh, T, L_total, w.mode == "exact")


def test_algorithmic_bytes_batch8_is_affine_in_prefix():
    w = WORKLOADS["vicuna7b_batch8_ragged"]
    base = bench.algorithmic_bytes(w, 46, 0)
    assert base == 1_877_999_616
    for L in (0, 512 * 8, 18_432, 4096 * 8):
        assert bench.algorithmic_bytes(w, 46, L) == base + 16_384 * L


def test_w2_launch_bytes():
    assert bench.w2_kernel_bytes(WORKLOADS["vicuna7b_typical"]) == 1_310_801_920
    # exact mode adds the fp32 head logits the launch writes
    ex = WORKLOADS["vicuna7b_exact"]
    assert bench.w2_kernel_bytes(ex) == 1_310_801_920 + 4 * ex.K * ex.V


def test_combined_floor():
    # single sequences: every stage is below the MFMA ridge, so the combined
    # floor is the HBM floor
    for name, T, L in (("vicuna7b_typical", 46, 2048), ("vicuna13b_typical", 137, 4096),
                       ("vicuna7b_exact", 46, 4096)):
        w = WORKLOADS[name]
        hbm_us = bench.algorithmic_bytes(w, T, L) / (bench.HBM_PEAK_GBS * 1e9) * 1e6
        assert abs(bench.combined_roofline_us(w, T, L) - hbm_us) < 0.5
    # eight sequences: the LM head (96.5 GFLOP) and the QKV projection sit
    # above the ridge, adding ~8 us at the expected prefix total
    w = WORKLOADS["vicuna7b_batch8_ragged"]
    hbm_us = bench.algorithmic_bytes(w, 46, 18_432) / 8e12 * 1e6
    comb = bench.combined_roofline_us(w, 46, 18_432)
    assert abs(hbm_us - 272.5) < 0.5
    assert abs(comb - 280.9) < 0.5
    lm_flops = 2 * 8 * 46 * w.V * w.d
    assert abs(lm_flops / 1e9 - 96.5) < 0.1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
