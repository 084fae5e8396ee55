"""Pins for the oracle's analytic backward and gate Jacobian (CPU only).

The backward differentiates o = softmax(tau q K_S^T + log g_S) V_S (SAS review
page, paper.oopus.info, §2.3) with log g_m = s_m - LSE(s_H) (§2.4); the
per-block gate gradient is the sum of the logit gradients inside the block
(§2.6).  Top-K itself carries no gradient (gitee README, figure caption (b))."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.sas_oracle import BLOCK


def _problem(seed, B=1, Hq=2, Hkv=1, n=256, d=16):
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, Hq, n, d))
    k = g.standard_normal((B, Hkv, n, d))
    v = g.standard_normal((B, Hkv, n, d))
    do = g.standard_normal((B, Hq, n, d))
    nb = n // BLOCK
    s = g.standard_normal((B, Hkv, nb, nb)) * 1.3
    return q, k, v, do, s


def _loss(q, k, v, do, s, K, idx_ref=None):
    idx, cnt, lg, _ = oracle.select(s, K)
    if idx_ref is not None:
        assert np.array_equal(idx, idx_ref), "selection changed under the perturbation"
    o, _ = oracle.fwd_gather(q, k, v, idx, cnt, lg)
    return float(np.sum(do * o))


@pytest.mark.parametrize("seed,K,Hq,Hkv", [(0, 2, 2, 1), (1, 1, 3, 1), (2, 3, 4, 2)])
def test_finite_differences(seed, K, Hq, Hkv):
    """Central differences in float64, directional, h = 1e-6."""
    q, k, v, do, s = _problem(seed, Hq=Hq, Hkv=Hkv)
    res = oracle.sas_forward_backward(q, k, v, do, s, K)
    g = np.random.default_rng(100 + seed)
    h = 1e-6
    hist = np.tril(np.ones(s.shape[-2:]), -1).astype(bool)   # only m < i is read
    for name, x, grad in (("q", q, res["dq"]), ("k", k, res["dk"]),
                          ("v", v, res["dv"]), ("s", s, res["ds"])):
        u = g.standard_normal(x.shape)
        if name == "s":
            u = u * hist
        args = dict(q=q, k=k, v=v, s=s)
        args[name] = x + h * u
        lp = _loss(args["q"], args["k"], args["v"], do, args["s"], K, res["idx"])
        args[name] = x - h * u
        lm = _loss(args["q"], args["k"], args["v"], do, args["s"], K, res["idx"])
        fd = (lp - lm) / (2 * h)
        an = float(np.sum(grad * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def _torch_dense_forward(q, k, v, s, idx, cnt, scale):
    """A torch float64 forward written from the review page's equations, used
    only to obtain autograd gradients of the same function."""
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    nb = n // BLOCK
    outs = []
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            rows = []
            for i in range(nb):
                z = scale * q[b, h, i * BLOCK:(i + 1) * BLOCK] @ k[b, kv].T
                bias = torch.full((BLOCK, n), -math.inf, dtype=torch.float64)
                if i > 0:
                    lse = torch.logsumexp(s[b, kv, i, :i], 0)
                    for sl in range(int(cnt[b, kv, i])):
                        m = int(idx[b, kv, i, sl])
                        bias[:, m * BLOCK:(m + 1) * BLOCK] = (s[b, kv, i, m] - lse)
                cur = torch.triu(torch.full((BLOCK, BLOCK), -math.inf, dtype=torch.float64), 1)
                bias[:, i * BLOCK:(i + 1) * BLOCK] = cur
                rows.append(torch.softmax(z + bias, dim=-1) @ v[b, kv])
            outs.append(torch.cat(rows))
    return torch.stack(outs).reshape(B, Hq, n, d)


def test_against_torch_autograd():
    q, k, v, do, s = _problem(3, Hq=4, Hkv=2, n=320)
    K, tau = 2, 0.21
    res = oracle.sas_forward_backward(q, k, v, do, s, K, scale=tau)
    tq, tk, tv, ts = (torch.tensor(x, requires_grad=True) for x in (q, k, v, s))
    o = _torch_dense_forward(tq, tk, tv, ts, res["idx"], res["cnt"], tau)
    np.testing.assert_allclose(o.detach().numpy(), res["o"], rtol=1e-12, atol=1e-12)
    (o * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(res["dq"], tq.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(res["dk"], tk.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(res["dv"], tv.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(res["ds"], ts.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_dense_equals_gather_backward():
    q, k, v, do, s = _problem(4, B=2, Hq=4, Hkv=2, n=384)
    for K in (0, 2, 5):
        idx, cnt, lg, _ = oracle.select(s, K)
        a = oracle.bwd_dense(q, k, v, do, idx, cnt, lg, 0.3)
        b = oracle.bwd_gather(q, k, v, do, idx, cnt, lg, 0.3)
        for x, y in zip(a, b):
            np.testing.assert_allclose(y, x, rtol=1e-11, atol=1e-11)


def test_ds_rows_sum_to_zero_and_upper_triangle_zero():
    q, k, v, do, s = _problem(5, Hq=2, Hkv=1, n=512)
    res = oracle.sas_forward_backward(q, k, v, do, s, 3)
    ds = res["ds"]
    np.testing.assert_allclose(ds.sum(axis=-1), 0.0, atol=1e-12)
    nb = ds.shape[-1]
    assert np.all(ds[..., np.triu(np.ones((nb, nb), dtype=bool))] == 0.0)


def test_gate_gradient_row_identity():
    """Each row of dZ sums to zero, so the gate gradients of a q-block equal
    minus the dZ mass on its own current block: sum_slots dlg[i] =
    -sum_{h, t in i, j in i, j <= t} dZ[t, j]."""
    q, k, v, do, s = _problem(6, Hq=2, Hkv=1, n=320)
    idx, cnt, lg, _ = oracle.select(s, 2)
    _, _, _, dlg = oracle.bwd_dense(q, k, v, do, idx, cnt, lg)
    n, d = q.shape[2], q.shape[3]
    tau = 1 / math.sqrt(d)
    A = oracle.bias_matrix(n, idx[0, 0], cnt[0, 0], lg[0, 0])
    cur_mass = np.zeros(n // BLOCK)
    for h in range(2):
        Z = tau * q[0, h] @ k[0, 0].T + A
        P = np.exp(Z - Z.max(1, keepdims=True))
        P /= P.sum(1, keepdims=True)
        O = P @ v[0, 0]
        dZ = P * (do[0, h] @ v[0, 0].T - np.sum(do[0, h] * O, 1, keepdims=True))
        np.testing.assert_allclose(dZ.sum(1), 0.0, atol=1e-12)
        for i in range(n // BLOCK):
            r = slice(i * BLOCK, (i + 1) * BLOCK)
            cur_mass[i] += dZ[r, r].sum()
    np.testing.assert_allclose(dlg[0, 0].sum(-1), -cur_mass, atol=1e-11)


def test_kv_block_sampler_matches_full_backward():
    q, k, v, do, s = _problem(7, Hq=2, Hkv=1, n=512)
    idx, cnt, lg, _ = oracle.select(s, 2)
    _, dk, dv, _ = oracle.bwd_gather(q, k, v, do, idx, cnt, lg)
    for m in (0, 3, 7):
        dkm, dvm = oracle.bwd_kv_block(q, k, v, do, idx, cnt, lg, 0, 0, m)
        np.testing.assert_allclose(dkm, dk[0, 0, m * BLOCK:(m + 1) * BLOCK], atol=1e-12)
        np.testing.assert_allclose(dvm, dv[0, 0, m * BLOCK:(m + 1) * BLOCK], atol=1e-12)
