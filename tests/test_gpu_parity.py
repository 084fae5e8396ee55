"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (tests/parity_bars.py): selected block indices and counts bit-exact; bf16
workloads o within max-abs 1e-2 plus the exact bf16 half-ulp of the oracle's
value (the storage rounding), dq, dk, dv, ds relative-L2 <= 2e-2; the float32
workloads 1e-5 for both.  lse / log_gate / s_lse tolerances follow from float32
accumulation.  Each check records its worst error as a fraction of its bar.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import sas_inputs as si
import parity_bars as pb
from parity_bars import assert_maxabs, assert_o, assert_rel
from sas_run import BLOCK, dev, host, rel_l2, run_layer, tdtype

pytestmark = pytest.mark.gpu

TOL = {dt: dict(o=pb.O_ABS[dt], grad=pb.GRAD_REL[dt], lse=pb.LSE_ABS[dt]) for dt in ("f32", "bf16")}


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_block_sparse_select_amd as m
    return m


def _check_select(res, s_host, topk, gate="softmax"):
    idx, cnt, lg, lse = oracle.select(s_host, topk, gate)
    assert np.array_equal(host(res["cnt"]), cnt)
    assert np.array_equal(host(res["idx"]), idx)
    g_lg, g_lse = host(res["log_gate"]), host(res["s_lse"])
    assert np.array_equal(np.isneginf(g_lg), np.isneginf(lg))
    fin = np.isfinite(lg)
    np.testing.assert_allclose(g_lg[fin], lg[fin], rtol=1e-5, atol=1e-5)
    assert np.array_equal(np.isneginf(g_lse), np.isneginf(lse))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(g_lse[fin], lse[fin], rtol=1e-5, atol=1e-5)
    return idx, cnt, lg, lse


# ---------------------------------------------------------------- selection
@pytest.mark.parametrize("case", ["normal", "ties", "k0", "kall", "gumbel"])
def test_select_bitexact(api, case):
    g = np.random.default_rng(11)
    B, Hkv, nb, K = 2, 3, 300, 7
    s = g.standard_normal((B, Hkv, nb, nb)).astype(np.float32)
    if case == "ties":
        s = np.round(s * 2).astype(np.float32)
        z = s == 0
        s[z] = np.where(g.random(z.sum()) < 0.5, np.float32(-0.0), np.float32(0.0))
    if case == "k0":
        K = 0
    if case == "kall":
        K = nb
    if case == "gumbel":
        s = (-3 * np.log(-np.log(g.random(s.shape)))).astype(np.float32)
    sh = api.make_shape(B, 4 * Hkv, Hkv, nb * BLOCK, 128, K, torch.bfloat16)
    st = torch.from_numpy(s).cuda()
    sel = api.alloc_select(sh)
    api.sas_select(sh, st, sel["idx"], sel["cnt"], sel["log_gate"], sel["s_lse"])
    torch.cuda.synchronize()
    _check_select(sel, s, K)


@pytest.mark.parametrize("nb,K", [(100, 3), (1000, 40), (1999, 7)])
def test_select_row_lengths(api, nb, K):
    """Rows of every register layout of the selection (2, 16 and 32
    candidates per lane), with ties, -0.0 and -inf scores mixed in."""
    g = np.random.default_rng(nb)
    B, Hkv = 1, 2
    s = np.round(g.standard_normal((B, Hkv, nb, nb)) * 3).astype(np.float32)
    s[s == 0] = np.float32(-0.0)
    s[g.random(s.shape) < 0.05] = -np.inf
    sh = api.make_shape(B, 2 * Hkv, Hkv, nb * BLOCK, 64, K, torch.bfloat16)
    sel = api.alloc_select(sh)
    api.sas_select(sh, torch.from_numpy(s).cuda(), sel["idx"], sel["cnt"], sel["log_gate"],
                   sel["s_lse"])
    torch.cuda.synchronize()
    _check_select(sel, s, K)


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_select_full_size(api, cfg):
    w = si.WORKLOADS[cfg]
    s = si.make_scores(w)
    sh = api.make_shape(w.B, w.Hq, w.Hkv, w.n, w.d, w.topk, tdtype(w.dtype))
    sel = api.alloc_select(sh)
    api.sas_select(sh, torch.from_numpy(s).cuda(), sel["idx"], sel["cnt"], sel["log_gate"],
                   sel["s_lse"])
    torch.cuda.synchronize()
    _check_select(sel, s, w.topk)


def test_mask_documents_bitexact(api):
    g = np.random.default_rng(12)
    B, Hkv, nb = 3, 2, 200
    s = g.standard_normal((B, Hkv, nb, nb)).astype(np.float32)
    df = np.stack([si.doc_first_of(si.packed_doc_blocks(12, b, nb)) for b in range(B)])
    df[2, ::7] = np.where(np.arange(0, nb, 7) % 2, -3, nb + 5)   # clamped into [0, i]
    sh = api.make_shape(B, 2 * Hkv, Hkv, nb * BLOCK, 128, 4, torch.bfloat16)
    st = torch.from_numpy(s).cuda()
    api.sas_mask_documents(sh, torch.from_numpy(df).cuda(), st)
    torch.cuda.synchronize()
    ref = oracle.mask_documents(s, df).astype(np.float32)
    assert np.array_equal(host(st), ref)


# ---------------------------------------------------------------- pooling
@pytest.mark.parametrize("cfg,small", [(3, True), (3, False)])
def test_pool_parity(api, cfg, small):
    w = si.WORKLOADS[cfg]
    if small:
        w = si.custom_workload(33, 1, 8, 2, 2048, 128, 4, "bf16")
    q, k, _, _ = si.make_qkv(w, with_do=False)
    sh = api.make_shape(w.B, w.Hq, w.Hkv, w.n, w.d, w.topk, tdtype(w.dtype))
    s = torch.empty((w.B, w.Hkv, w.nqb, w.nqb), dtype=torch.float32, device="cuda")
    ws = api.alloc_workspace(api.sas_pool_workspace_bytes(sh))
    api.sas_pool_scores(sh, dev(q, tdtype(w.dtype)), dev(k, tdtype(w.dtype)), s, ws)
    torch.cuda.synchronize()
    ref = oracle.pool_scores(q, k, w.Hkv)
    got = host(s)
    assert_rel(got, ref, 1e-5, "s_pool")
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))


# ---------------------------------------------------------------- training layer, full oracle
SMALL_CASES = {
    "cfg1_fp32": (si.WORKLOADS[1], None),
    "bf16_gqa4_d128": (si.custom_workload(101, 2, 8, 2, 1024, 128, 4, "bf16"), None),
    "bf16_gqa5_d64": (si.custom_workload(102, 1, 5, 1, 640, 64, 3, "bf16"), None),
    "bf16_single_block": (si.custom_workload(103, 1, 4, 1, 64, 128, 2, "bf16"), None),
    "bf16_k0": (si.custom_workload(104, 1, 4, 2, 512, 128, 0, "bf16"), None),
    "bf16_kall": (si.custom_workload(105, 1, 2, 1, 512, 128, 8, "bf16"), None),
    "bf16_mha_d128": (si.custom_workload(106, 1, 1, 1, 768, 128, 5, "bf16"), None),
    "bf16_heavy_gumbel": (si.custom_workload(107, 1, 4, 1, 1024, 128, 6, "bf16",
                                             s_kind="gumbel3"), None),
    "fp32_gqa2_d128": (si.custom_workload(108, 1, 4, 2, 384, 128, 2, "f32"), None),
    # 16 query heads per kv-head: four head chunks in the forward and dq
    "bf16_gqa16_d128": (si.custom_workload(109, 1, 16, 1, 512, 128, 3, "bf16"), None),
    # packed documents (scores of earlier documents masked to -inf on the device)
    "bf16_packed_gqa4_d128": (si.custom_workload(110, 2, 8, 2, 1536, 128, 4, "bf16",
                                                 packed=True), None),
    "fp32_packed_d64": (si.custom_workload(111, 1, 2, 1, 1024, 64, 3, "f32", packed=True), None),
}


def _scores(w):
    """(device scores as the library should receive them, doc_first on the
    device or None, host scores after the oracle's document mask)."""
    s = si.make_scores(w)
    df = si.make_doc_first(w)
    if df is None:
        return torch.from_numpy(s).cuda(), None, s
    return (torch.from_numpy(s).cuda(), torch.from_numpy(df).cuda(),
            oracle.mask_documents(s, df).astype(np.float32))


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_fwd_parity_full(api, name):
    w, _ = SMALL_CASES[name]
    q, k, v, _ = si.make_qkv(w, with_do=False)
    sd, df, s = _scores(w)
    dt = tdtype(w.dtype)
    res = run_layer(api, dev(q, dt), dev(k, dt), dev(v, dt), None, sd, w.topk, dt, bwd=False,
                    doc_first=df)
    assert np.array_equal(host(res["s"]), s)
    idx, cnt, lg, _ = _check_select(res, s, w.topk)
    o, lse = oracle.fwd_gather(q, k, v, idx, cnt, lg)
    tol = TOL[w.dtype]
    assert_o(host(res["o"]), o, w.dtype)
    assert_maxabs(host(res["lse"]), lse, tol["lse"], ("lse",))


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_layer_parity_full(api, name):
    w, _ = SMALL_CASES[name]
    q, k, v, do = si.make_qkv(w)
    sd, df, s = _scores(w)
    dt = tdtype(w.dtype)
    res = run_layer(api, dev(q, dt), dev(k, dt), dev(v, dt), dev(do, dt), sd, w.topk, dt,
                    doc_first=df)
    idx, cnt, lg, _ = _check_select(res, s, w.topk)
    ref = oracle.sas_forward_backward(q, k, v, do, s, w.topk)
    tol = TOL[w.dtype]
    assert_o(host(res["o"]), ref["o"], w.dtype)
    assert_maxabs(host(res["lse"]), ref["lse"], tol["lse"], ("lse",))
    for nm in ("dq", "dk", "dv", "ds"):
        assert_rel(host(res[nm]), ref[nm], tol["grad"], nm)
    if df is not None:   # no gradient reaches another document's blocks
        ds_g = host(res["ds"])
        assert np.all(ds_g[np.isneginf(s)] == 0.0)


# ---------------------------------------------------------------- gate variants
RECOMPUTE_CASES = ["bf16_gqa4_d128", "bf16_gqa5_d64", "bf16_k0", "bf16_kall", "bf16_gqa16_d128",
                   "bf16_packed_gqa4_d128"]


@pytest.mark.parametrize("name", RECOMPUTE_CASES)
def test_layer_parity_recompute_path(api, name):
    """The backward with only the minimum workspace: dq recomputes S and dP
    per tile instead of reading the dZ tiles the key-outer pass stores.  Both
    paths against the oracle, and against each other."""
    w, _ = SMALL_CASES[name]
    q, k, v, do = si.make_qkv(w)
    sd, df, s = _scores(w)
    dt = tdtype(w.dtype)
    args = (dev(q, dt), dev(k, dt), dev(v, dt), dev(do, dt))
    res = run_layer(api, *args, sd.clone(), w.topk, dt, doc_first=df, min_ws=True)
    fast = run_layer(api, *args, sd.clone(), w.topk, dt, doc_first=df)
    _check_select(res, s, w.topk)
    ref = oracle.sas_forward_backward(q, k, v, do, s, w.topk)
    tol = TOL[w.dtype]
    for nm in ("dq", "dk", "dv", "ds"):
        assert_rel(host(res[nm]), ref[nm], tol["grad"], nm)
        assert_rel(host(res[nm]), host(fast[nm]), tol["grad"], nm + " (paths)")


GATE_CASES = {
    "bf16_gqa4_d128": si.custom_workload(120, 2, 8, 2, 1024, 128, 4, "bf16"),
    "bf16_gqa5_d64_kall": si.custom_workload(121, 1, 5, 1, 512, 64, 8, "bf16", s_std=2.0),
    "fp32_gqa2_d64": si.custom_workload(122, 1, 4, 2, 384, 64, 2, "f32"),
}


@pytest.mark.parametrize("gate", ["sigmoid", "hard", "external"])
@pytest.mark.parametrize("name", list(GATE_CASES))
def test_gate_variant_layer_parity(api, gate, name):
    """The ablation gates through the whole layer against the oracle."""
    w = GATE_CASES[name]
    q, k, v, do = si.make_qkv(w)
    s = si.make_scores(w)
    dt = tdtype(w.dtype)
    res = run_layer(api, dev(q, dt), dev(k, dt), dev(v, dt), dev(do, dt),
                    torch.from_numpy(s).cuda(), w.topk, dt, gate=gate)
    _check_select(res, s, w.topk, gate)
    ref = oracle.sas_forward_backward(q, k, v, do, s, w.topk, gate=gate)
    tol = TOL[w.dtype]
    assert_o(host(res["o"]), ref["o"], w.dtype)
    assert_maxabs(host(res["lse"]), ref["lse"], tol["lse"], ("lse",))
    for nm in ("dq", "dk", "dv", "ds"):
        assert_rel(host(res[nm]), ref[nm], tol["grad"], nm)


@pytest.mark.parametrize("gate", ["sigmoid", "hard", "external"])
def test_gate_variant_packed_documents(api, gate):
    """Ablation gates on a packed batch: rows near a document's start keep
    fewer blocks (or none), and no gradient crosses documents."""
    w = si.custom_workload(123, 2, 8, 2, 1536, 128, 4, "bf16", packed=True)
    q, k, v, do = si.make_qkv(w)
    sd, df, s = _scores(w)
    dt = tdtype(w.dtype)
    res = run_layer(api, dev(q, dt), dev(k, dt), dev(v, dt), dev(do, dt), sd, w.topk, dt,
                    doc_first=df, gate=gate)
    _check_select(res, s, w.topk, gate)
    ref = oracle.sas_forward_backward(q, k, v, do, s, w.topk, gate=gate)
    tol = TOL[w.dtype]
    assert_o(host(res["o"]), ref["o"], w.dtype)
    for nm in ("dq", "dk", "dv", "ds"):
        assert_rel(host(res[nm]), ref[nm], tol["grad"], nm)
    assert np.all(host(res["ds"])[np.isneginf(s)] == 0.0)


@pytest.mark.parametrize("gate", ["sigmoid", "external"])
def test_gate_variant_full_size_sampled(api, gate):
    """The 8K Qwen3-4B layer with an ablation gate, sampled blocks."""
    w = si.WORKLOADS[2]
    q, k, v, do = si.make_qkv(w)
    s = si.make_scores(w)
    dt = tdtype(w.dtype)
    res = run_layer(api, dev(q, dt), dev(k, dt), dev(v, dt), dev(do, dt),
                    torch.from_numpy(s).cuda(), w.topk, dt, gate=gate)
    idx, cnt, lg, s_lse = _check_select(res, s, w.topk, gate)
    G = w.Hq // w.Hkv
    tol = TOL[w.dtype]
    o_g, dq_g, ds_g = host(res["o"]), host(res["dq"]), host(res["ds"])
    for (b, kv, i) in _sample_blocks(w, np.random.default_rng(31)):
        r = slice(i * BLOCK, (i + 1) * BLOCK)
        hs = slice(kv * G, (kv + 1) * G)
        ob, _ = oracle.fwd_gather_block(q, k, v, idx, cnt, lg, b, kv, i, gate=gate)
        assert_o(o_g[b, hs, r], ob, w.dtype, ("o", b, kv, i))
        dqb, _, _, _, dlg = oracle.bwd_gather_block(q, k, v, do, idx, cnt, lg, b, kv, i, gate=gate)
        assert_rel(dq_g[b, hs, r], dqb, tol["grad"], ("dq", b, kv, i))
        if i > 0:
            dlg_full = np.zeros((1, 1, w.nqb, w.topk))
            dlg_full[0, 0, i] = dlg
            dsr = oracle.gate_jacobian(s[b:b + 1, kv:kv + 1], s_lse[b:b + 1, kv:kv + 1],
                                       idx[b:b + 1, kv:kv + 1], cnt[b:b + 1, kv:kv + 1],
                                       dlg_full, gate)[0, 0, i]
            assert_rel(ds_g[b, kv, i], dsr, tol["grad"], ("ds", b, kv, i))
    dk_g, dv_g = host(res["dk"]), host(res["dv"])
    for (b, kv, m) in [(0, 0, 0), (0, w.Hkv - 1, w.nqb // 2), (0, 1, w.nqb - 1)]:
        dkm, dvm = oracle.bwd_kv_block(q, k, v, do, idx, cnt, lg, b, kv, m, gate=gate)
        r = slice(m * BLOCK, (m + 1) * BLOCK)
        assert_rel(dk_g[b, kv, r], dkm, tol["grad"], ("dk", b, kv, m))
        assert_rel(dv_g[b, kv, r], dvm, tol["grad"], ("dv", b, kv, m))


# ---------------------------------------------------------------- head-chunk mixes
# Groups of G heads run as workgroups of 4, 2 and 1 heads: G = 2, 3, 6, 7 use
# the two-head and one-head workgroups in every combination; K beyond the
# history, the longest history a row can have, and each gate kind appear.
CHUNK_CASES = [
    # seed, B, Hq, Hkv, n, d, K, gate
    (160, 1, 4, 2, 640, 128, 3, "softmax"),     # G = 2: one two-head chunk
    (161, 2, 3, 1, 512, 64, 5, "external"),     # G = 3: 2 + 1
    (162, 1, 12, 2, 448, 128, 2, "sigmoid"),    # G = 6: 4 + 2
    (163, 1, 7, 1, 576, 128, 20, "hard"),       # G = 7: 4 + 2 + 1, K > every history
    (164, 1, 14, 2, 320, 64, 1, "softmax"),     # G = 7 with d = 64
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: f"G{c[2] // c[3]}_d{c[5]}_K{c[6]}_{c[7]}")
def test_head_chunk_mixes(api, case):
    seed, B, Hq, Hkv, n, d, K, gate = case
    w = si.custom_workload(seed, B, Hq, Hkv, n, d, K, "bf16")
    q, k, v, do = si.make_qkv(w)
    s = si.make_scores(w)
    dt = tdtype(w.dtype)
    res = run_layer(api, dev(q, dt), dev(k, dt), dev(v, dt), dev(do, dt),
                    torch.from_numpy(s).cuda(), w.topk, dt, gate=gate)
    _check_select(res, s, w.topk, gate)
    ref = oracle.sas_forward_backward(q, k, v, do, s, w.topk, gate=gate)
    tol = TOL[w.dtype]
    assert_o(host(res["o"]), ref["o"], w.dtype)
    assert_maxabs(host(res["lse"]), ref["lse"], tol["lse"], ("lse",))
    for nm in ("dq", "dk", "dv", "ds"):
        assert_rel(host(res[nm]), ref[nm], tol["grad"], nm)


# ---------------------------------------------------------------- full-size sampled checks
def _sample_blocks(w, rng, n_blocks=5):
    picks = {(0, 0, 0), (0, w.Hkv - 1, w.nqb - 1), (0, w.Hkv // 2, min(w.topk, w.nqb - 1))}
    while len(picks) < n_blocks:
        picks.add((int(rng.integers(w.B)), int(rng.integers(w.Hkv)), int(rng.integers(w.nqb))))
    return sorted(picks)


@pytest.mark.parametrize("cfg,min_ws", [(2, False), (3, False), (4, False), (10, False),
                                        (9, False), (3, True)],
                         ids=["2", "3", "4", "10", "9", "3-recompute"])
def test_layer_parity_full_size_sampled(api, cfg, min_ws):
    """Full-size layers on sampled blocks; min_ws runs the backward with its
    minimum workspace (dq recomputes the logits, no dZ tiles)."""
    w = si.WORKLOADS[cfg]
    q, k, v, do = si.make_qkv(w)
    dt = tdtype(w.dtype)
    qd, kd, vd, dod = dev(q, dt), dev(k, dt), dev(v, dt), dev(do, dt)
    df = None
    if w.s_kind == "pool":
        res = run_layer(api, qd, kd, vd, dod, None, w.topk, dt, pool=True, min_ws=min_ws)
        s = host(res["s"])      # selection parity is defined on the device scores
    else:
        sd, df, s = _scores(w)
        res = run_layer(api, qd, kd, vd, dod, sd, w.topk, dt, doc_first=df, min_ws=min_ws)
        assert np.array_equal(host(res["s"]), s)
    idx, cnt, lg, s_lse = _check_select(res, s, w.topk)
    rng = np.random.default_rng(cfg)
    G = w.Hq // w.Hkv
    tol = TOL[w.dtype]
    o_g, lse_g, dq_g, ds_g = host(res["o"]), host(res["lse"]), host(res["dq"]), host(res["ds"])
    picks = _sample_blocks(w, rng)
    if df is not None:
        # a document's first block (no candidates) and the block after it
        starts = [i for i in range(1, w.nqb) if df[0, i] == i and i + 1 < w.nqb]
        picks += [(0, 1, starts[0]), (0, 2, starts[0] + 1), (0, 3, starts[-1])]
        assert np.all(ds_g[np.isneginf(s)] == 0.0)
    for (b, kv, i) in picks:
        ob, lb = oracle.fwd_gather_block(q, k, v, idx, cnt, lg, b, kv, i)
        r = slice(i * BLOCK, (i + 1) * BLOCK)
        hs = slice(kv * G, (kv + 1) * G)
        assert_o(o_g[b, hs, r], ob, w.dtype, ("o", b, kv, i))
        assert_maxabs(lse_g[b, hs, r], lb, tol["lse"], ("lse", b, kv, i))
        dqb, _, _, _, dlg = oracle.bwd_gather_block(q, k, v, do, idx, cnt, lg, b, kv, i)
        assert_rel(dq_g[b, hs, r], dqb, tol["grad"], ("dq", b, kv, i))
        if i > 0:
            dlg_full = np.zeros((1, 1, w.nqb, w.topk))
            dlg_full[0, 0, i] = dlg
            dsr = oracle.gate_jacobian(s[b:b + 1, kv:kv + 1], s_lse[b:b + 1, kv:kv + 1],
                                       idx[b:b + 1, kv:kv + 1], cnt[b:b + 1, kv:kv + 1],
                                       dlg_full)[0, 0, i]
            assert_rel(ds_g[b, kv, i], dsr, tol["grad"], ("ds", b, kv, i))
    dk_g, dv_g = host(res["dk"]), host(res["dv"])
    kv_picks = [(0, 0, 0), (0, w.Hkv - 1, w.nqb // 2), (0, 1, w.nqb - 1)]
    if w.topk >= w.nqb:   # full range: key block 0 is read by every row (slow in the oracle)
        kv_picks[0] = (0, 0, w.nqb // 2 + 17)
    for (b, kv, m) in kv_picks:
        dkm, dvm = oracle.bwd_kv_block(q, k, v, do, idx, cnt, lg, b, kv, m)
        r = slice(m * BLOCK, (m + 1) * BLOCK)
        assert_rel(dk_g[b, kv, r], dkm, tol["grad"], ("dk", b, kv, m))
        assert_rel(dv_g[b, kv, r], dvm, tol["grad"], ("dv", b, kv, m))


def test_layer_parity_max_length(api):
    """The longest sequence the ABI accepts (n = 131072, 2048 blocks): selection
    on every row, sampled q-blocks and key blocks against the oracle."""
    w = si.custom_workload(130, 1, 4, 1, 64 * 2048, 64, 16, "bf16")
    q, k, v, do = si.make_qkv(w)
    s = si.make_scores(w)
    dt = tdtype(w.dtype)
    res = run_layer(api, dev(q, dt), dev(k, dt), dev(v, dt), dev(do, dt),
                    torch.from_numpy(s).cuda(), w.topk, dt)
    idx, cnt, lg, s_lse = _check_select(res, s, w.topk)
    tol = TOL[w.dtype]
    o_g, dq_g, ds_g = host(res["o"]), host(res["dq"]), host(res["ds"])
    for i in (0, 1, 777, 2047):
        r = slice(i * BLOCK, (i + 1) * BLOCK)
        ob, _ = oracle.fwd_gather_block(q, k, v, idx, cnt, lg, 0, 0, i)
        assert_o(o_g[0, :, r], ob, w.dtype, ("o", i))
        dqb, _, _, _, dlg = oracle.bwd_gather_block(q, k, v, do, idx, cnt, lg, 0, 0, i)
        assert_rel(dq_g[0, :, r], dqb, tol["grad"], ("dq", i))
        if i > 0:
            dlg_full = np.zeros((1, 1, w.nqb, w.topk))
            dlg_full[0, 0, i] = dlg
            dsr = oracle.gate_jacobian(s, s_lse, idx, cnt, dlg_full)[0, 0, i]
            assert_rel(ds_g[0, 0, i], dsr, tol["grad"], ("ds", i))
    dk_g, dv_g = host(res["dk"]), host(res["dv"])
    for m in (1500, 2047):
        dkm, dvm = oracle.bwd_kv_block(q, k, v, do, idx, cnt, lg, 0, 0, m)
        r = slice(m * BLOCK, (m + 1) * BLOCK)
        assert_rel(dk_g[0, 0, r], dkm, tol["grad"], ("dk", m))
        assert_rel(dv_g[0, 0, r], dvm, tol["grad"], ("dv", m))


# ---------------------------------------------------------------- decode
def _decode_run(api, w, q, kc, vc, lens, s, gate="softmax"):
    dt = tdtype(w.dtype)
    sh = api.make_decode_shape(w.B, w.Hq, w.Hkv, w.cap, w.d, w.topk, dt, gate=gate)
    o = torch.empty_like(q)
    idx = torch.empty((w.B, w.Hkv, w.topk), dtype=torch.int32, device="cuda")
    ws = api.alloc_workspace(api.sas_decode_workspace_bytes(sh))
    api.sas_decode(sh, q, kc, vc, torch.from_numpy(lens).cuda(), torch.from_numpy(s).cuda(), o,
                   idx, ws)
    torch.cuda.synchronize()
    return o, idx


@pytest.mark.parametrize("dtype,G,d,cap,K", [("bf16", 4, 128, 1024, 5), ("bf16", 5, 64, 512, 3),
                                             ("f32", 2, 64, 768, 2), ("bf16", 1, 128, 256, 0),
                                             ("bf16", 12, 128, 512, 4), ("f32", 4, 128, 640, 3)])
def test_decode_parity_small(api, dtype, G, d, cap, K):
    w = si.DecodeWorkload(200 + G, 5, 2 * G, 2, cap, d, K, dtype, hist_blocks=cap // BLOCK - 1)
    q, kc, vc, lens, s = si.make_decode_small(w)
    lens = np.array([1, 64, 65, cap - 3, cap][:w.B], dtype=np.int32)
    dt = tdtype(dtype)
    o, idx = _decode_run(api, w, dev(q, dt), dev(kc, dt), dev(vc, dt), lens, s)
    ref_o, ref_idx = oracle.decode(q, kc, vc, lens, s, K)
    assert np.array_equal(host(idx), ref_idx)
    assert_o(host(o), ref_o, dtype)


@pytest.mark.parametrize("ties,K,nkb", [(False, 48, 64), (True, 64, 64), (True, 100, 128)])
def test_decode_parity_fused_wide_k(api, ties, K, nkb):
    """512 rows (batch 64 x 8 kv-heads: one workgroup per row, whose four
    waves select) with K > 32: into 64-slot segments for K <= 64, by the
    workgroup search beyond; some rows hold fewer history blocks than K, one
    only its current block; with ties, equal scores straddle the waves'
    shares."""
    w = si.DecodeWorkload(296 + K, 64, 8, 8, nkb * BLOCK, 64, K, "bf16", hist_blocks=nkb - 1)
    q, kc, vc, lens, s = si.make_decode_small(w)
    lens[::7] = (K - 8) * BLOCK + 5
    lens[1] = 1
    if ties:
        s = np.round(s * 2).astype(np.float32)
    dt = tdtype(w.dtype)
    o, idx = _decode_run(api, w, dev(q, dt), dev(kc, dt), dev(vc, dt), lens, s)
    ref_o, ref_idx = oracle.decode(q, kc, vc, lens, s, K)
    assert np.array_equal(host(idx), ref_idx)
    assert_o(host(o), ref_o, "bf16")


def test_decode_parity_max_cache(api):
    """A contiguous cache of the longest size the ABI accepts (131072 tokens,
    rows of up to 2047 history blocks selected by one wave)."""
    w = si.DecodeWorkload(290, 3, 8, 2, 64 * 2048, 64, 24, "bf16", hist_blocks=2047)
    q, kc, vc, lens, s = si.make_decode_small(w)
    lens = np.array([64 * 2048, 64 * 1500 + 7, 1], dtype=np.int32)
    dt = tdtype(w.dtype)
    o, idx = _decode_run(api, w, dev(q, dt), dev(kc, dt), dev(vc, dt), lens, s)
    ref_o, ref_idx = oracle.decode(q, kc, vc, lens, s, w.topk)
    assert np.array_equal(host(idx), ref_idx)
    assert_o(host(o), ref_o, "bf16")


def test_decode_parity_full_size(api):
    w = si.DECODE_WORKLOAD
    q, s = si.decode_q_and_scores(w)
    lens = si.decode_seq_lens(w)
    kc, vc = si.decode_cache_device(w, "cuda")
    o, idx = _decode_run(api, w, dev(q, torch.bfloat16), kc, vc, lens, s)
    rows = [(0, 0), (7, 3), (31, 7), (63, 5), (40, 1)]

    class _Cache:
        def __init__(self, t):
            self.t = t

        def __getitem__(self, bk):
            return self.t[bk[0], bk[1]].float().cpu().numpy()

    ref_o, ref_idx = oracle.decode(q, _Cache(kc), _Cache(vc), lens, s, w.topk, rows=rows)
    # selection for every row (cheap) and outputs on the sampled rows
    idx_h = host(idx)
    for b in range(w.B):
        for kv in range(w.Hkv):
            ch, _, _ = oracle.select_row(s[b, kv], (int(lens[b]) - 1) // BLOCK, w.topk)
            assert list(idx_h[b, kv, :len(ch)]) == ch
    o_h = host(o)
    G = w.Hq // w.Hkv
    for (b, kv) in rows:
        assert_o(o_h[b, kv * G:(kv + 1) * G], ref_o[b, kv * G:(kv + 1) * G], "bf16")


# ---------------------------------------------------------------- paged decode
class _PagedRows:
    """[b, kv] -> sequence b's [cap, d] cache seen through its page table, with
    out-of-range entries clipped into the pool as the library specifies (an
    input view for the oracle, which itself only knows contiguous caches)."""

    def __init__(self, pages, table):
        self.pages = pages
        self.table = np.clip(table, 0, pages.shape[0] - 1)

    def __getitem__(self, bk):
        b, kv = bk
        pages, pt = self.pages, self.table[b]

        class _Rows:
            def __getitem__(self, cols):
                cols = np.asarray(cols)
                return pages[pt[cols // BLOCK], kv, cols % BLOCK]

        return _Rows()


def _decode_paged_run(api, dtype, q, kp, vp, table, lens, s, K, gate="softmax"):
    B, Hq, d = q.shape
    num_pages, Hkv = kp.shape[:2]
    max_blocks = table.shape[1]
    dt = tdtype(dtype)
    shp = api.make_decode_paged_shape(B, Hq, Hkv, max_blocks, num_pages, d, K, dt, gate=gate)
    qd = dev(q, dt)
    o = torch.empty_like(qd)
    idx = torch.full((B, Hkv, K), -7, dtype=torch.int32, device="cuda")
    ws = api.alloc_workspace(api.sas_decode_paged_workspace_bytes(shp))
    api.sas_decode_paged(shp, qd, dev(kp, dt), dev(vp, dt), torch.from_numpy(table).cuda(),
                         torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda(),
                         torch.from_numpy(s).cuda(), o, idx, ws)
    torch.cuda.synchronize()
    return host(o), host(idx)


@pytest.mark.parametrize("dtype,G,d,max_blocks,num_pages,K", [
    ("bf16", 4, 128, 40, 400, 5),    # a page of its own for every block
    ("bf16", 2, 64, 24, 30, 3),      # blocks share pages
    ("f32", 2, 64, 16, 64, 2),
    ("bf16", 5, 128, 20, 100, 0),
    ("bf16", 4, 64, 1500, 2000, 16)])   # rows of 513..2048 blocks: one wave, 32 candidates per lane
def test_decode_paged_parity_small(api, dtype, G, d, max_blocks, num_pages, K):
    B, Hkv = 4, 2
    q, kp, vp, table, lens, s = si.make_decode_paged(400 + max_blocks, B, G * Hkv, Hkv, max_blocks,
                                                     num_pages, d, dtype)
    lens[0], lens[1] = 1, BLOCK * max_blocks          # shortest and longest rows
    table[2, :] = np.where(np.arange(max_blocks) % 3 == 0, -5, table[2, :])
    table[3, 1] = num_pages + 7                       # entries outside the pool are clamped
    o, idx = _decode_paged_run(api, dtype, q, kp, vp, table, lens, s, K)
    ref_o, ref_idx = oracle.decode(q, _PagedRows(kp, table), _PagedRows(vp, table), lens, s, K)
    assert np.array_equal(idx, ref_idx)
    assert_o(o, ref_o, dtype)


@pytest.mark.parametrize("ties,K", [(False, 32), (True, 32), (False, 0), (True, 2048), (False, 64),
                                    (True, 40)])
def test_decode_paged_long_context(api, ties, K):
    """Rows of up to 8191 history blocks (512K tokens), selected by the whole
    workgroup; with ties, equal scores straddle the waves' candidate ranges."""
    B, Hq, Hkv, d = 3, 4, 2, 64
    max_blocks, num_pages = 8192, 4096
    lens = [BLOCK * max_blocks, 300000, 1000]
    q, kp, vp, table, lens, s = si.make_decode_paged(450 + K, B, Hq, Hkv, max_blocks, num_pages, d,
                                                     "bf16", seq_lens=lens)
    if ties:
        s = np.round(s * 2).astype(np.float32)
    o, idx = _decode_paged_run(api, "bf16", q, kp, vp, table, lens, s, K)
    ref_o, ref_idx = oracle.decode(q, _PagedRows(kp, table), _PagedRows(vp, table), lens, s, K)
    assert np.array_equal(idx, ref_idx)
    assert_o(o, ref_o, "bf16")


def _mask_history(s, g, first):
    """-inf on the blocks before first[b] (an earlier document) and on a
    random tenth of the rest."""
    s = s.copy()
    for b in range(s.shape[0]):
        s[b, :, :first[b]] = -np.inf
    s[g.random(s.shape) < 0.1] = -np.inf
    return s


def test_decode_masked_scores(api):
    """Decode rows whose history holds non-candidate (-inf) blocks, one row
    with none left (only the current block is attended)."""
    w = si.DecodeWorkload(260, 5, 8, 2, 1024, 128, 5, "bf16", hist_blocks=15)
    q, kc, vc, lens, s = si.make_decode_small(w)
    g = np.random.default_rng(260)
    s = _mask_history(s, g, [0, 3, 9, 15, 1])
    s[4] = -np.inf
    dt = tdtype(w.dtype)
    o, idx = _decode_run(api, w, dev(q, dt), dev(kc, dt), dev(vc, dt), lens, s)
    ref_o, ref_idx = oracle.decode(q, kc, vc, lens, s, w.topk)
    assert np.array_equal(host(idx), ref_idx)
    assert np.all(host(idx)[4] == -1)
    assert_o(host(o), ref_o, "bf16")


def test_decode_paged_masked_long_context(api):
    """The workgroup selection over up to 8191 history blocks with -inf
    blocks: fewer candidates than K in one row, none in another."""
    B, Hq, Hkv, d, K = 4, 4, 2, 64, 32
    max_blocks, num_pages = 8192, 4096
    lens = [BLOCK * max_blocks, 300000, 200000, 5000]
    q, kp, vp, table, lens, s = si.make_decode_paged(470, B, Hq, Hkv, max_blocks, num_pages, d,
                                                     "bf16", seq_lens=lens)
    g = np.random.default_rng(470)
    s = _mask_history(s, g, [4000, 0, 3120, 0])
    s[1, :, :4680] = -np.inf                     # row 1: at most 7 candidates left (< K)
    s[1, :, 4680:4692] = g.standard_normal((Hkv, 12)).astype(np.float32)
    s[3] = -np.inf                               # row 3: no candidate
    o, idx = _decode_paged_run(api, "bf16", q, kp, vp, table, lens, s, K)
    ref_o, ref_idx = oracle.decode(q, _PagedRows(kp, table), _PagedRows(vp, table), lens, s, K)
    assert np.array_equal(idx, ref_idx)
    assert np.all(idx[3] == -1)
    assert_o(o, ref_o, "bf16")


@pytest.mark.parametrize("gate", ["sigmoid", "hard", "external"])
@pytest.mark.parametrize("dtype,nsplit_b", [("bf16", 3), ("f32", 3), ("bf16", 256)])
def test_decode_gate_variants(api, gate, dtype, nsplit_b):
    """Decode with the ablation gates; 3 sequences (6 rows) split their tiles
    over several workgroups, 256 sequences (512 rows) use one per row."""
    w = si.DecodeWorkload(280, nsplit_b, 8, 2, 512, 128, 5, dtype, hist_blocks=7)
    q, kc, vc, lens, s = si.make_decode_small(w)
    dt = tdtype(dtype)
    o, idx = _decode_run(api, w, dev(q, dt), dev(kc, dt), dev(vc, dt), lens, s, gate)
    ref_o, ref_idx = oracle.decode(q, kc, vc, lens, s, w.topk, gate=gate)
    assert np.array_equal(host(idx), ref_idx)
    assert_o(host(o), ref_o, dtype)


@pytest.mark.parametrize("gate", ["sigmoid", "external"])
def test_decode_paged_gate_variants_long_context(api, gate):
    B, Hq, Hkv, d, K = 2, 4, 2, 64, 32
    max_blocks, num_pages = 8192, 4096
    lens = [BLOCK * max_blocks, 200000]
    q, kp, vp, table, lens, s = si.make_decode_paged(490, B, Hq, Hkv, max_blocks, num_pages, d,
                                                     "bf16", seq_lens=lens)
    s = s * 3.0   # a wide spread of gates
    o, idx = _decode_paged_run(api, "bf16", q, kp, vp, table, lens, s, K, gate)
    ref_o, ref_idx = oracle.decode(q, _PagedRows(kp, table), _PagedRows(vp, table), lens, s, K,
                                   gate=gate)
    assert np.array_equal(idx, ref_idx)
    assert_o(o, ref_o, "bf16")


# ---------------------------------------------------------------- determinism
def test_run_twice_bitwise(api):
    w = si.custom_workload(300, 1, 8, 2, 2048, 128, 8, "bf16")
    q, k, v, do = si.make_qkv(w)
    s = torch.from_numpy(si.make_scores(w)).cuda()
    args = [dev(x, torch.bfloat16) for x in (q, k, v, do)]
    a = run_layer(api, *args, s, w.topk, torch.bfloat16)
    b = run_layer(api, *args, s, w.topk, torch.bfloat16)
    for nm in ("idx", "cnt", "log_gate", "s_lse", "o", "lse", "dq", "dk", "dv", "ds"):
        assert torch.equal(a[nm], b[nm]), nm


# ---------------------------------------------------------------- packed documents of any length
# Documents of any token length packed into one sequence: each is cut into
# 64-token blocks from its own first token (the last block partial) through
# the block table; outputs are compared on the documents' tokens only.
VARLEN_CASES = {
    # seed, B, Hq, Hkv, n, d, K, dtype, tail
    "bf16_gqa4_d128": (140, 1, 8, 2, 1000, 128, 3, "bf16", 0),
    "bf16_b2_gqa4_d64_tail": (141, 2, 8, 2, 700, 64, 2, "bf16", 23),   # padding blocks, tail rows
    "bf16_gqa5_d128_kall": (142, 1, 5, 1, 600, 128, 20, "bf16", 0),
    "bf16_gqa16_d128": (143, 1, 16, 1, 400, 128, 2, "bf16", 0),
    "fp32_gqa2_d64": (144, 1, 4, 2, 500, 64, 2, "f32", 5),
}


def _varlen_inputs(api, w):
    lens = [si.doc_token_lens(w, b) for b in range(w.B)]
    geom, first = oracle.packed_geometry(lens)
    blocks, doc_first = api.blocks_from_cu_seqlens([si.cu_seqlens_of(x) for x in lens])
    # the library's block cut is integer work: bit-exact against the oracle's
    assert np.array_equal(blocks.numpy(), geom) and np.array_equal(doc_first.numpy(), first)
    return lens, geom, first, blocks.cuda(), doc_first.cuda()


def _doc_rows(geom, b):
    return np.concatenate([np.arange(a, a + L) for a, L in geom[b] if L > 0])


@pytest.mark.parametrize("gate", ["softmax", "external", "softmax_min_ws"])
@pytest.mark.parametrize("name", list(VARLEN_CASES))
def test_varlen_layer_parity(api, name, gate):
    min_ws = gate.endswith("_min_ws")
    gate = gate.removesuffix("_min_ws")
    seed, B, Hq, Hkv, n, d, K, dtype, tail = VARLEN_CASES[name]
    w = si.custom_workload(seed, B, Hq, Hkv, n, d, K, dtype, varlen=True, tail=tail)
    q, k, v, do = si.make_qkv(w)
    s = si.make_scores(w)
    lens, geom, first, blocks, doc_first = _varlen_inputs(api, w)
    dt = tdtype(w.dtype)
    res = run_layer(api, dev(q, dt), dev(k, dt), dev(v, dt), dev(do, dt),
                    torch.from_numpy(s).cuda(), w.topk, dt, doc_first=doc_first, blocks=blocks,
                    gate=gate, min_ws=min_ws)
    sm = oracle.mask_documents(s, first).astype(np.float32)
    assert np.array_equal(host(res["s"]), sm)
    _check_select(res, sm, w.topk, gate)
    ref = oracle.sas_forward_backward(q, k, v, do, sm, w.topk, gate=gate, geom=geom)
    tol = TOL[w.dtype]
    got = {nm: host(res[nm]) for nm in ("o", "lse", "dq", "dk", "dv")}
    for b in range(w.B):
        r = _doc_rows(geom, b)
        assert_o(got["o"][b][:, r], ref["o"][b][:, r], w.dtype, "o")
        assert_maxabs(got["lse"][b][:, r], ref["lse"][b][:, r], tol["lse"], "lse")
        for nm in ("dq", "dk", "dv"):
            assert_rel(got[nm][b][:, r], ref[nm][b][:, r], tol["grad"], nm)
    assert_rel(host(res["ds"]), ref["ds"], tol["grad"], "ds")
    assert np.all(host(res["ds"])[np.isneginf(sm)] == 0.0)


def test_varlen_pool_parity(api):
    """Mean pooling over each block's own tokens (partial last blocks, empty
    padding blocks)."""
    w = si.custom_workload(145, 2, 8, 2, 900, 128, 4, "bf16", varlen=True, tail=11)
    q, k, _, _ = si.make_qkv(w, with_do=False)
    lens, geom, first, blocks, _ = _varlen_inputs(api, w)
    nb = geom.shape[1]
    sh = api.make_shape(w.B, w.Hq, w.Hkv, w.n, w.d, w.topk, torch.bfloat16, blocks=blocks)
    s = torch.empty((w.B, w.Hkv, nb, nb), dtype=torch.float32, device="cuda")
    ws = api.alloc_workspace(api.sas_pool_workspace_bytes(sh))
    api.sas_pool_scores(sh, dev(q, torch.bfloat16), dev(k, torch.bfloat16), s, ws)
    torch.cuda.synchronize()
    ref = oracle.pool_scores(q, k, w.Hkv, geom)
    assert_rel(host(s), ref, 1e-5, "s_pool")


def test_varlen_full_size_sampled(api):
    """The 32K Qwen3-8B layer holding documents of any length (the packed
    bench line's workload): selection on every row, sampled q-blocks (a
    document's first and partial last blocks among them) and key blocks."""
    w = si.WORKLOADS[7]
    q, k, v, do = si.make_qkv(w)
    s = si.make_scores(w)
    lens, geom, first, blocks, doc_first = _varlen_inputs(api, w)
    dt = tdtype(w.dtype)
    res = run_layer(api, dev(q, dt), dev(k, dt), dev(v, dt), dev(do, dt),
                    torch.from_numpy(s).cuda(), w.topk, dt, doc_first=doc_first, blocks=blocks)
    sm = oracle.mask_documents(s, first).astype(np.float32)
    idx, cnt, lg, s_lse = _check_select(res, sm, w.topk)
    G = w.Hq // w.Hkv
    tol = TOL[w.dtype]
    nb = geom.shape[1]
    partial = [i for i in range(nb) if 0 < geom[0, i, 1] < BLOCK]
    starts = [i for i in range(1, nb) if first[0, i] == i]
    picks = sorted({(0, 0, 0), (0, 1, partial[0]), (0, 2, partial[-1]), (0, 3, starts[0]),
                    (0, 5, starts[-1] + 1), (0, w.Hkv - 1, nb - 1), (0, 4, nb // 2)})
    o_g, dq_g, ds_g = host(res["o"]), host(res["dq"]), host(res["ds"])
    for (b, kv, i) in picks:
        r = slice(int(geom[b, i, 0]), int(geom[b, i, 0] + geom[b, i, 1]))
        hs = slice(kv * G, (kv + 1) * G)
        ob, _ = oracle.fwd_gather_block(q, k, v, idx, cnt, lg, b, kv, i, geom=geom)
        assert_o(o_g[b, hs, r], ob, w.dtype, ("o", b, kv, i))
        dqb, _, _, _, dlg = oracle.bwd_gather_block(q, k, v, do, idx, cnt, lg, b, kv, i, geom=geom)
        assert_rel(dq_g[b, hs, r], dqb, tol["grad"], ("dq", b, kv, i))
        if cnt[b, kv, i] > 0:
            dlg_full = np.zeros((1, 1, nb, w.topk))
            dlg_full[0, 0, i] = dlg
            dsr = oracle.gate_jacobian(sm[b:b + 1, kv:kv + 1], s_lse[b:b + 1, kv:kv + 1],
                                       idx[b:b + 1, kv:kv + 1], cnt[b:b + 1, kv:kv + 1],
                                       dlg_full)[0, 0, i]
            assert_rel(ds_g[b, kv, i], dsr, tol["grad"], ("ds", b, kv, i))
    assert np.all(ds_g[np.isneginf(sm)] == 0.0)
    dk_g, dv_g = host(res["dk"]), host(res["dv"])
    for (b, kv, m) in [(0, 0, partial[0]), (0, 1, starts[-1]), (0, 6, nb // 3)]:
        dkm, dvm = oracle.bwd_kv_block(q, k, v, do, idx, cnt, lg, b, kv, m, geom=geom)
        r = slice(int(geom[b, m, 0]), int(geom[b, m, 0] + geom[b, m, 1]))
        assert_rel(dk_g[b, kv, r], dkm, tol["grad"], ("dk", b, kv, m))
        assert_rel(dv_g[b, kv, r], dvm, tol["grad"], ("dv", b, kv, m))
