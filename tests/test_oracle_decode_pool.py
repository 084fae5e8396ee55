"""Pins for the oracle's decode and block-score pooling (CPU only)."""
import math

import numpy as np
import torch

import oracle
from oracle.sas_oracle import BLOCK


def test_decode_equals_forward_row():
    """Decode of token T equals row T of the training forward when q-block
    blk(T) sees the same score row (the forward's causal rule j <= T covers
    exactly the tokens [64 blk(T), T])."""
    g = np.random.default_rng(0)
    Hq, Hkv, d, K = 4, 2, 16, 3
    for L in (1, 17, 64):
        i = 5
        T = i * BLOCK + L - 1
        n = (i + 1) * BLOCK
        q = g.standard_normal((1, Hq, n, d))
        k = g.standard_normal((1, Hkv, n, d))
        v = g.standard_normal((1, Hkv, n, d))
        s = g.standard_normal((1, Hkv, n // BLOCK, n // BLOCK))
        idx, cnt, lg, _ = oracle.select(s, K)
        o, _ = oracle.fwd_dense(q, k, v, idx, cnt, lg)
        cap = n + 2 * BLOCK
        kc = np.concatenate([k, g.standard_normal((1, Hkv, cap - n, d))], axis=2)
        vc = np.concatenate([v, g.standard_normal((1, Hkv, cap - n, d))], axis=2)
        # the decode score row of kv-group kv is the forward's row i
        sd = np.concatenate([s[:, :, i, :], g.standard_normal((1, Hkv, cap // BLOCK - n // BLOCK))],
                            axis=2)
        od, idd = oracle.decode(q[:, :, T, :], kc, vc, np.array([T + 1]), sd, K)
        np.testing.assert_allclose(od[0], o[0, :, T, :], rtol=1e-12, atol=1e-12)
        assert np.array_equal(idd[0], idx[0, :, i, :])


def test_decode_k0_is_attention_over_partial_block():
    g = np.random.default_rng(1)
    B, Hq, Hkv, d, cap = 3, 2, 1, 16, 512
    q = g.standard_normal((B, Hq, d))
    kc = g.standard_normal((B, Hkv, cap, d))
    vc = g.standard_normal((B, Hkv, cap, d))
    s = g.standard_normal((B, Hkv, cap // BLOCK))
    lens = np.array([1, 130, 512], dtype=np.int32)
    o, idx = oracle.decode(q, kc, vc, lens, s, 0)
    assert np.all(idx == -1) or idx.size == 0
    for b in range(B):
        i = (lens[b] - 1) // BLOCK
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
        for h in range(Hq):
            ref = torch.nn.functional.scaled_dot_product_attention(
                t(q[b, h][None]), t(kc[b, 0, i * BLOCK:lens[b]]), t(vc[b, 0, i * BLOCK:lens[b]]),
                scale=1 / math.sqrt(d)).numpy()[0]
            np.testing.assert_allclose(o[b, h], ref, rtol=1e-12, atol=1e-12)


def test_pool_constant_blocks_closed_form():
    """Rows of q-block i all equal a_i (every head) and rows of key block m all
    equal c_m: then s[i, m] = a_i . c_m / sqrt(d)."""
    g = np.random.default_rng(2)
    Hq, Hkv, nb, d = 4, 2, 5, 8
    a = g.standard_normal((Hkv, nb, d))
    c = g.standard_normal((Hkv, nb, d))
    q = np.zeros((1, Hq, nb * BLOCK, d))
    k = np.zeros((1, Hkv, nb * BLOCK, d))
    for h in range(Hq):
        q[0, h] = np.repeat(a[h // 2], BLOCK, axis=0)
    for kv in range(Hkv):
        k[0, kv] = np.repeat(c[kv], BLOCK, axis=0)
    s = oracle.pool_scores(q, k, Hkv)
    np.testing.assert_allclose(s[0], np.einsum("kid,kmd->kim", a, c) / math.sqrt(d), rtol=1e-12, atol=1e-14)


def test_pool_brute_force_loops():
    g = np.random.default_rng(3)
    Hq, Hkv, nb, d = 2, 1, 3, 4
    q = g.standard_normal((1, Hq, nb * BLOCK, d))
    k = g.standard_normal((1, Hkv, nb * BLOCK, d))
    s = oracle.pool_scores(q, k, Hkv)
    for i in range(nb):
        for m in range(nb):
            qs = [0.0] * d
            ks = [0.0] * d
            for h in range(Hq):
                for r in range(BLOCK):
                    for e in range(d):
                        qs[e] += q[0, h, i * BLOCK + r, e]
            for r in range(BLOCK):
                for e in range(d):
                    ks[e] += k[0, 0, m * BLOCK + r, e]
            dot = sum((qs[e] / (Hq * BLOCK)) * (ks[e] / BLOCK) for e in range(d))
            assert abs(s[0, 0, i, m] - dot / math.sqrt(d)) < 1e-13


def test_selected_pairs_count():
    cnt = np.array([[[0, 1, 2, 2]]])
    assert oracle.selected_pairs(cnt) == 5 * 64 * 64 + 4 * 64 * 65 // 2
