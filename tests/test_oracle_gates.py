"""Pins for the oracle's gate variants (CPU only).

The review page (paper.oopus.info) compares the method's gate with three
alternatives in its ablations: a gate outside the softmax that only scales
the values (§2.3), sigmoid instead of softmax normalisation (§2.4), and a
hard gate trained with a straight-through estimator (§2.5).  The readings
(module header of the oracle) are pinned here against an independent dense
torch formulation differentiated by autograd, against finite differences
where the gradient is exact, and against special cases that reduce to the
method's own gate or to plain masked attention."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.sas_oracle import BLOCK

GATES = ("softmax", "sigmoid", "hard", "external")


def _problem(seed, B=1, Hq=2, Hkv=1, n=256, d=16):
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, Hq, n, d))
    k = g.standard_normal((B, Hkv, n, d))
    v = g.standard_normal((B, Hkv, n, d))
    do = g.standard_normal((B, Hq, n, d))
    nb = n // BLOCK
    s = g.standard_normal((B, Hkv, nb, nb)) * 1.3
    return q, k, v, do, s


def _torch_forward(q, k, v, s, idx, cnt, scale, gate):
    """Dense float64 torch forward, one row block at a time, written from the
    gate definitions; used only for its autograd gradients."""
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
                w = torch.zeros(n, dtype=torch.float64)
                for sl in range(int(cnt[b, kv, i])):
                    m = int(idx[b, kv, i, sl])
                    soft = s[b, kv, i, m] - torch.logsumexp(s[b, kv, i, :i], 0)
                    cols = slice(m * BLOCK, (m + 1) * BLOCK)
                    if gate == "softmax":
                        bias[:, cols] = soft
                    elif gate == "sigmoid":
                        bias[:, cols] = torch.nn.functional.logsigmoid(s[b, kv, i, m])
                    elif gate == "hard":     # value 0, gradient of the soft log-gate
                        bias[:, cols] = soft - soft.detach()
                    else:                    # external: mask only, values scaled
                        bias[:, cols] = 0.0
                        w = w.index_put((torch.arange(m * BLOCK, (m + 1) * BLOCK),),
                                        torch.exp(soft).expand(BLOCK))
                cur = slice(i * BLOCK, (i + 1) * BLOCK)
                bias[:, cur] = torch.triu(torch.full((BLOCK, BLOCK), -math.inf,
                                                     dtype=torch.float64), 1)
                p = torch.softmax(z + bias, dim=-1)
                if gate == "external":
                    w = w.index_put((torch.arange(i * BLOCK, (i + 1) * BLOCK),),
                                    torch.ones(BLOCK, dtype=torch.float64))
                    rows.append(p @ (w[:, None] * v[b, kv]))
                else:
                    rows.append(p @ v[b, kv])
            outs.append(torch.cat(rows))
    return torch.stack(outs).reshape(B, Hq, n, d)


@pytest.mark.parametrize("gate", GATES)
@pytest.mark.parametrize("mode", ["gather", "dense"])
def test_against_torch_autograd(gate, mode):
    q, k, v, do, s = _problem(7, Hq=4, Hkv=2, n=320)
    K, tau = 2, 0.23
    res = oracle.sas_forward_backward(q, k, v, do, s, K, scale=tau, mode=mode, gate=gate)
    tq, tk, tv, ts = (torch.tensor(x, requires_grad=True) for x in (q, k, v, s))
    o = _torch_forward(tq, tk, tv, ts, res["idx"], res["cnt"], tau, gate)
    np.testing.assert_allclose(res["o"], o.detach().numpy(), rtol=1e-12, atol=1e-12)
    (o * torch.from_numpy(do)).sum().backward()
    for name, ref in (("dq", tq), ("dk", tk), ("dv", tv), ("ds", ts)):
        np.testing.assert_allclose(res[name], ref.grad.numpy(), rtol=1e-10, atol=1e-11,
                                   err_msg=f"{gate} {name}")


def _loss(q, k, v, do, s, K, gate, idx_ref):
    idx, cnt, lg, _ = oracle.select(s, K, gate)
    assert np.array_equal(idx, idx_ref), "selection changed under the perturbation"
    o, _ = oracle.fwd_gather(q, k, v, idx, cnt, lg, gate=gate)
    return float(np.sum(do * o))


@pytest.mark.parametrize("gate", ["sigmoid", "external"])
def test_finite_differences(gate):
    """Both variants are differentiable functions of s on a fixed selection:
    central differences in float64 (h = 1e-6) match every gradient."""
    q, k, v, do, s = _problem(11, Hq=3, Hkv=1)
    K = 2
    res = oracle.sas_forward_backward(q, k, v, do, s, K, gate=gate)
    g = np.random.default_rng(12)
    h = 1e-6
    hist = np.tril(np.ones(s.shape[-2:]), -1).astype(bool)
    for name, x, grad in (("q", q, res["dq"]), ("k", k, res["dk"]),
                          ("v", v, res["dv"]), ("s", s, res["ds"])):
        u = g.standard_normal(x.shape)
        if name == "s":
            u = u * hist
        args = dict(q=q, k=k, v=v, s=s)
        args[name] = x + h * u
        lp = _loss(args["q"], args["k"], args["v"], do, args["s"], K, gate, res["idx"])
        args[name] = x - h * u
        lm = _loss(args["q"], args["k"], args["v"], do, args["s"], K, gate, res["idx"])
        fd = (lp - lm) / (2 * h)
        an = float(np.sum(grad * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (gate, name, fd, an)


def test_hard_forward_is_block_masked_attention():
    """With g = 1 on every kept block the forward is plain attention under a
    block mask: torch SDPA with a boolean mask."""
    q, k, v, _, s = _problem(13, Hq=2, Hkv=1, n=384)
    K = 3
    idx, cnt, lg, _ = oracle.select(s, K, "hard")
    assert np.all(lg[np.isfinite(lg)] == 0.0)
    o, _ = oracle.fwd_gather(q, k, v, idx, cnt, lg, gate="hard")
    n = q.shape[2]
    allow = np.zeros((n, n), dtype=bool)
    for i in range(n // BLOCK):
        r = slice(i * BLOCK, (i + 1) * BLOCK)
        for sl in range(int(cnt[0, 0, i])):
            m = int(idx[0, 0, i, sl])
            allow[r, m * BLOCK:(m + 1) * BLOCK] = True
        allow[r, r] = np.tril(np.ones((BLOCK, BLOCK), dtype=bool))
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    for h in range(2):
        ref = torch.nn.functional.scaled_dot_product_attention(
            t(q[0, h]), t(k[0, 0]), t(v[0, 0]), attn_mask=t(allow), scale=1 / math.sqrt(16))
        np.testing.assert_allclose(o[0, h], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_sigmoid_saturates_to_the_hard_forward():
    """log sigmoid(s) -> 0 as s -> +inf: shifted far up, the sigmoid gate's
    forward equals the hard gate's (the selection is shift invariant)."""
    q, k, v, _, s = _problem(14)
    K = 2
    a = oracle.select(s + 60.0, K, "sigmoid")
    b = oracle.select(s, K, "hard")
    assert np.array_equal(a[0], b[0])
    oa, _ = oracle.fwd_gather(q, k, v, a[0], a[1], a[2], gate="sigmoid")
    ob, _ = oracle.fwd_gather(q, k, v, b[0], b[1], b[2], gate="hard")
    np.testing.assert_allclose(oa, ob, rtol=1e-12, atol=1e-12)


def test_sigmoid_log_gate_values():
    """log sigmoid against scipy's expit, over a wide range of scores."""
    from scipy.special import expit
    s = np.array([[[[0.0] * 6, [-700.0] + [0.0] * 5, [3.0, -40.0] + [0.0] * 4,
                    [0.5, 1.5, 30.0] + [0.0] * 3, [-2.0, 0.25, -0.5, 7.0, 0, 0],
                    [1, 2, 3, 4, 5, 0.0]]]])
    idx, cnt, lg, _ = oracle.select(s, 6, "sigmoid")
    for i in range(6):
        for sl in range(int(cnt[0, 0, i])):
            x = s[0, 0, i, idx[0, 0, i, sl]]
            ref = -np.logaddexp(0.0, -x)    # log expit(x), stable
            assert lg[0, 0, i, sl] == pytest.approx(ref, rel=1e-14, abs=1e-300)
            if x > -30:
                assert lg[0, 0, i, sl] == pytest.approx(math.log(expit(x)), rel=1e-12)


def test_external_without_history_is_the_method():
    """K = 0 keeps no block, so no gate is applied anywhere: the external
    gate's forward and gradients equal the method's."""
    q, k, v, do, s = _problem(15, Hq=2, Hkv=2)
    a = oracle.sas_forward_backward(q, k, v, do, s, 0, gate="external")
    b = oracle.sas_forward_backward(q, k, v, do, s, 0)
    for key in ("o", "dq", "dk", "dv", "ds"):
        np.testing.assert_array_equal(a[key], b[key])


def test_external_uniform_scores_closed_form():
    """Constant scores over i history blocks, all kept: each kept block has
    g = 1/i.  One query row that sees every key equally (q = 0): the unbiased
    weights are uniform over the 64*i history keys and the t+1 visible
    current keys, and the output is their mean with the history values
    scaled by 1/i."""
    g = np.random.default_rng(16)
    n, d, i = 320, 8, 4
    q = np.zeros((1, 1, n, d))
    k = g.standard_normal((1, 1, n, d))
    v = g.standard_normal((1, 1, n, d))
    s = np.zeros((1, 1, n // BLOCK, n // BLOCK))
    idx, cnt, lg, _ = oracle.select(s, 8, "external")
    o, _ = oracle.fwd_gather(q, k, v, idx, cnt, lg, gate="external")
    for t in (0, 17, 63):
        row = i * BLOCK + t
        hist = v[0, 0, :i * BLOCK].sum(axis=0) / i
        cur = v[0, 0, i * BLOCK:row + 1].sum(axis=0)
        ref = (hist + cur) / (i * BLOCK + t + 1)
        np.testing.assert_allclose(o[0, 0, row], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("gate", GATES)
def test_decode_equals_forward_row(gate):
    g = np.random.default_rng(17)
    Hq, Hkv, d, K, i, L = 4, 2, 16, 3, 5, 23
    T = i * BLOCK + L - 1
    n = (i + 1) * BLOCK
    q = g.standard_normal((1, Hq, n, d))
    k = g.standard_normal((1, Hkv, n, d))
    v = g.standard_normal((1, Hkv, n, d))
    s = g.standard_normal((1, Hkv, n // BLOCK, n // BLOCK))
    idx, cnt, lg, _ = oracle.select(s, K, gate)
    o, _ = oracle.fwd_dense(q, k, v, idx, cnt, lg, gate=gate)
    od, idd = oracle.decode(q[:, :, T, :], k, v, np.array([T + 1]), s[:, :, i, :], K, gate=gate)
    np.testing.assert_allclose(od[0], o[0, :, T, :], rtol=1e-12, atol=1e-12)
    assert np.array_equal(idd[0], idx[0, :, i, :])
