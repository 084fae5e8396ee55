"""Pins for the oracle's forward (CPU only).

The forward follows the SAS review page (paper.oopus.info) §2.3 equation
o = softmax(q K_S^T + log g_S) V_S, with §2.4's g_0 = 1 on the always-kept
current block and §2.6's masking of unselected blocks."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.sas_oracle import BLOCK


def _rand(seed, B, Hq, Hkv, n, d, NQB=None):
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, Hq, n, d))
    k = g.standard_normal((B, Hkv, n, d))
    v = g.standard_normal((B, Hkv, n, d))
    nb = n // BLOCK
    s = g.standard_normal((B, Hkv, nb, nb))
    return q, k, v, s


def _sdpa(q, k, v, mask, scale):
    """torch's reference attention in float64 on the CPU (library routine)."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=t(mask), scale=scale).numpy()


def test_k0_is_block_local_causal_attention():
    B, Hq, Hkv, n, d = 1, 2, 1, 256, 32
    q, k, v, s = _rand(0, B, Hq, Hkv, n, d)
    idx, cnt, lg, _ = oracle.select(s, 0)
    o, lse = oracle.fwd_dense(q, k, v, idx, cnt, lg)
    t = np.arange(n)
    mask = (t[None, :] <= t[:, None]) & (t[None, :] // BLOCK == t[:, None] // BLOCK)
    for h in range(Hq):
        ref = _sdpa(q[0, h], k[0, 0], v[0, 0], mask, 1 / math.sqrt(d))
        np.testing.assert_allclose(o[0, h], ref, rtol=1e-12, atol=1e-12)


def test_constant_scores_full_budget_is_causal_with_log_i_bias():
    B, Hq, Hkv, n, d = 1, 1, 1, 320, 16
    q, k, v, _ = _rand(1, B, Hq, Hkv, n, d)
    nb = n // BLOCK
    s = np.full((1, 1, nb, nb), -0.7)
    idx, cnt, lg, _ = oracle.select(s, nb)
    o, _ = oracle.fwd_dense(q, k, v, idx, cnt, lg, scale=0.3)
    t = np.arange(n)
    bt, bj = t[:, None] // BLOCK, t[None, :] // BLOCK
    bias = np.where(bj == bt, 0.0, -np.log(np.maximum(bt, 1)).astype(float))
    bias = np.where((t[None, :] <= t[:, None]), bias, -np.inf)
    ref = _sdpa(q[0, 0], k[0, 0], v[0, 0], bias, 0.3)
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-12, atol=1e-12)


def test_first_block_is_plain_causal():
    q, k, v, s = _rand(2, 1, 2, 2, 192, 16)
    idx, cnt, lg, _ = oracle.select(s, 2)
    o, _ = oracle.fwd_gather(q, k, v, idx, cnt, lg)
    t = np.arange(BLOCK)
    for h in range(2):
        ref = _sdpa(q[0, h, :BLOCK], k[0, h, :BLOCK], v[0, h, :BLOCK],
                    t[None, :] <= t[:, None], 0.25)
        np.testing.assert_allclose(o[0, h, :BLOCK], ref, rtol=1e-12, atol=1e-12)


def test_zero_query_closed_form():
    """q = 0: every logit equals its bias, so row t of q-block i is
    (sum_{m in S} g_m sum_{j in m} v_j + sum_{j<=t, j in i} v_j) /
    (64 sum_{m in S} g_m + (t - 64 i + 1))."""
    n, d, K = 384, 8, 2
    _, k, v, s = _rand(3, 1, 1, 1, n, d)
    q = np.zeros((1, 1, n, d))
    idx, cnt, lg, _ = oracle.select(s, K)
    o, _ = oracle.fwd_dense(q, k, v, idx, cnt, lg)
    for i in range(n // BLOCK):
        sel = [int(m) for m in idx[0, 0, i, :cnt[0, 0, i]]]
        gates = np.exp(lg[0, 0, i, :cnt[0, 0, i]])
        hist_num = sum(g * v[0, 0, m * BLOCK:(m + 1) * BLOCK].sum(axis=0) for g, m in zip(gates, sel))
        hist_den = BLOCK * gates.sum()
        for r in range(BLOCK):
            t = i * BLOCK + r
            num = hist_num + v[0, 0, i * BLOCK:t + 1].sum(axis=0)
            np.testing.assert_allclose(o[0, 0, t], num / (hist_den + r + 1), rtol=1e-12, atol=1e-13)


def test_history_permutation_invariance_last_block():
    n, d, K = 512, 16, 3
    q, k, v, s = _rand(4, 1, 2, 1, n, d)
    nb = n // BLOCK
    i = nb - 1
    idx, cnt, lg, _ = oracle.select(s, K)
    o, _ = oracle.fwd_gather(q, k, v, idx, cnt, lg, blocks=[(0, 0, i)])
    perm = np.random.default_rng(9).permutation(i)    # block m -> perm[m]
    k2, v2, s2 = k.copy(), v.copy(), s.copy()
    for m in range(i):
        k2[0, 0, perm[m] * BLOCK:(perm[m] + 1) * BLOCK] = k[0, 0, m * BLOCK:(m + 1) * BLOCK]
        v2[0, 0, perm[m] * BLOCK:(perm[m] + 1) * BLOCK] = v[0, 0, m * BLOCK:(m + 1) * BLOCK]
    s2[0, 0, i, perm] = s[0, 0, i, :i]
    idx2, cnt2, lg2, _ = oracle.select(s2, K)
    o2, _ = oracle.fwd_gather(q, k2, v2, idx2, cnt2, lg2, blocks=[(0, 0, i)])
    r = slice(i * BLOCK, n)
    np.testing.assert_allclose(o2[0, :, r], o[0, :, r], rtol=1e-12, atol=1e-12)


def test_shift_invariance_in_scores():
    q, k, v, s = _rand(5, 1, 2, 2, 256, 16)
    idx, cnt, lg, _ = oracle.select(s, 2)
    o, lse = oracle.fwd_dense(q, k, v, idx, cnt, lg)
    idx2, cnt2, lg2, _ = oracle.select(s - 11.5, 2)
    o2, lse2 = oracle.fwd_dense(q, k, v, idx2, cnt2, lg2)
    np.testing.assert_allclose(o2, o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=1e-11, atol=1e-11)


def test_gqa_equals_mha_with_repeated_kv():
    B, Hq, Hkv, n, d = 1, 4, 2, 256, 16
    q, k, v, s = _rand(6, B, Hq, Hkv, n, d)
    G = Hq // Hkv
    idx, cnt, lg, _ = oracle.select(s, 2)
    o, lse = oracle.fwd_dense(q, k, v, idx, cnt, lg)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    o2, lse2 = oracle.fwd_dense(q, kr, vr, np.repeat(idx, G, axis=1), np.repeat(cnt, G, axis=1),
                                np.repeat(lg, G, axis=1))
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("K", [0, 1, 3, 8])
def test_dense_equals_gather(K):
    q, k, v, s = _rand(7 + K, 2, 3, 1, 448, 16)
    idx, cnt, lg, _ = oracle.select(s, K)
    o, lse = oracle.fwd_dense(q, k, v, idx, cnt, lg, scale=0.2)
    o2, lse2 = oracle.fwd_gather(q, k, v, idx, cnt, lg, scale=0.2)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=1e-12)


def test_lse_matches_library_logsumexp():
    from scipy.special import logsumexp
    n, d = 256, 16
    q, k, v, s = _rand(8, 1, 1, 1, n, d)
    idx, cnt, lg, _ = oracle.select(s, 1)
    o, lse = oracle.fwd_dense(q, k, v, idx, cnt, lg)
    A = oracle.bias_matrix(n, idx[0, 0], cnt[0, 0], lg[0, 0])
    Z = q[0, 0] @ k[0, 0].T / math.sqrt(d) + A
    np.testing.assert_allclose(lse[0, 0], logsumexp(Z, axis=1), rtol=1e-13)
