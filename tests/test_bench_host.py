"""Host-side logic of bench.py (CPU only): the refusal of several GPUs, the
pair count behind the effective FLOPs, the roofline arithmetic and the HBM
byte counts of the memory-bound kernels."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
import oracle
import sas_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_pair_count_matches_the_oracle():
    """Effective work: 64*64 pairs per kept block plus the 64*65/2 causal
    pairs of the current block, per query head."""
    g = np.random.default_rng(0)
    s = g.standard_normal((2, 3, 40, 40))
    _, cnt, _, _ = oracle.select(s, 5)
    for G in (1, 4, 5):
        assert bench.pair_count(cnt, G) == G * oracle.selected_pairs(cnt)
    # closed form for K >= every row's history: pairs = G * B * Hkv * sum_i (64*64*i + 2080)
    _, cnt_all, _, _ = oracle.select(s, 40)
    nb = 40
    per_row = sum(64 * 64 * i + 64 * 65 // 2 for i in range(nb))
    assert bench.pair_count(cnt_all, 4) == 4 * 2 * 3 * per_row


def test_roofline_arithmetic():
    w = si.WORKLOADS[3]
    pairs = 2_112_356_352
    res = dict(w=w, pairs=pairs, per_kernel={
        "sas_fwd_mfma_kernel": dict(avg_ms=1.2, launches=5),
        "sas_bwd_dq_kernel": dict(avg_ms=1.8, launches=5),
        "sas_bwd_dkdv_kernel": dict(avg_ms=2.8, launches=5),
        "sas_select_kernel": dict(avg_ms=0.02, launches=5)})
    r = bench.roofline_for(res)
    assert r["kernel"] == "sas_bwd_dkdv_kernel" and r["bound"] == "mfma"
    flops = 8 * w.d * pairs
    assert r["flop_per_launch"] == flops
    assert abs(r["achieved"] - flops / 2.8e-3 / 1e12) < 0.01
    assert abs(r["frac"] - r["achieved"] / 2500.0) < 1e-4


def test_hbm_kernel_bytes():
    w = si.WORKLOADS[3]
    res = dict(w=w, per_kernel={"sas_pool_means_kernel": dict(avg_ms=0.05),
                                "sas_pool_dot_kernel": dict(avg_ms=0.03),
                                "sas_select_kernel": dict(avg_ms=0.02)})
    h = bench.hbm_kernels(res)
    nb = w.nqb
    qk = (w.Hq + w.Hkv) * w.n * w.d * 2                     # bf16 q and k, read once
    means = 2 * w.Hkv * nb * w.d * 4                         # fp32 block means
    assert h["pool"]["bytes"] == qk + 2 * means + w.Hkv * nb * nb * 4
    hist = w.Hkv * nb * (nb - 1) // 2 * 4                    # scores m < i
    assert h["select"]["bytes"] == hist + w.Hkv * nb * (w.topk * 8 + 8)
    assert abs(h["pool"]["frac"] - h["pool"]["GBs"] / 8000.0) < 1e-3


def test_backward_pass_bytes_and_dq_flops():
    """The dZ-tile backward's memory-bound passes: the statistics (o and dO
    read, lse read, 128 floats per (head, block) written) and dq from the
    tiles (one 8 KB dZ tile per head and kept or own block, K read once, dq
    written); its dq kernel counts one contraction (2d FLOP per pair)."""
    import torch
    w = si.WORKLOADS[3]
    g = np.random.default_rng(1)
    cnt = np.minimum(np.arange(w.nqb), w.topk)[None, None, :].repeat(w.Hkv, axis=1)
    cnt = cnt.astype(np.int32) - (g.random(cnt.shape) < 0.1)     # some rows keep fewer
    cnt = np.maximum(cnt, 0).astype(np.int32)
    res = dict(w=w, sel={"cnt": torch.from_numpy(cnt)}, pairs=10**9,
               per_kernel={"sas_revidx_stats_kernel": dict(avg_ms=0.09, launches=5),
                           "sas_bwd_dqz_kernel": dict(avg_ms=1.0, launches=5),
                           "sas_bwd_dkdv_kernel": dict(avg_ms=3.0, launches=5)})
    h = bench.hbm_kernels(res)
    qsize = w.Hq * w.n * w.d * 2
    assert h["bwd_stats"]["bytes"] == 2 * qsize + w.Hq * w.n * 4 + w.Hq * w.nqb * 128 * 4
    tiles = int((cnt.astype(np.int64) + 1).sum()) * (w.Hq // w.Hkv)
    assert h["bwd_dqz"]["bytes"] == tiles * 8192 + w.Hkv * w.n * w.d * 2 + qsize
    # the dq-from-tiles kernel, when it dominates, counts 2d per pair
    res["per_kernel"]["sas_bwd_dqz_kernel"]["avg_ms"] = 9.0
    r = bench.roofline_for(res)
    assert r["kernel"] == "sas_bwd_dqz_kernel" and r["flop_per_launch"] == 2 * w.d * 10**9
