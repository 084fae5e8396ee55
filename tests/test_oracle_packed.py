"""Pins for packed training batches (CPU only).

Several documents, each a whole number of 64-token blocks, share one
sequence.  Attention never crosses a document: a q-block selects among, and
normalises its gate over, the earlier blocks of its own document only (SAS
review page, paper.oopus.info, §2.2 and §2.4, applied per document).  The
scores carry that mask: s[i, m] = -inf for blocks m of an earlier document,
and the selection treats a -inf score as "not a candidate".  The pins do not
retype that rule; they check its consequences: a packed run must give, block
for block, what separate runs over the documents give, and cross-document
gradients must vanish."""
import numpy as np
import pytest

import oracle
import sas_inputs as si
from oracle.sas_oracle import BLOCK, NEG_INF


@pytest.mark.parametrize("doc_blocks,K,Hq,Hkv", [([5, 8, 3], 3, 2, 1), ([1, 6, 2, 7], 2, 4, 2),
                                                 ([16], 4, 2, 1), ([4, 4], 8, 2, 2)])
def test_packed_documents_match_separate_runs(doc_blocks, K, Hq, Hkv):
    g = np.random.default_rng(sum(doc_blocks) * 7 + K)
    nb = sum(doc_blocks)
    n, d, B = nb * BLOCK, 16, 1
    q = g.standard_normal((B, Hq, n, d))
    k = g.standard_normal((B, Hkv, n, d))
    v = g.standard_normal((B, Hkv, n, d))
    do = g.standard_normal((B, Hq, n, d))
    s = g.standard_normal((B, Hkv, nb, nb)) * 1.3
    sp = oracle.mask_documents(s, si.doc_first_of(doc_blocks)[None])
    packed = oracle.sas_forward_backward(q, k, v, do, sp, K)
    a = 0
    for dbk in doc_blocks:
        b = a + dbk
        rows = slice(a * BLOCK, b * BLOCK)
        sub = oracle.sas_forward_backward(q[:, :, rows], k[:, :, rows], v[:, :, rows],
                                          do[:, :, rows], s[:, :, a:b, a:b], K)
        for key in ("o", "dq", "dk", "dv"):
            np.testing.assert_allclose(packed[key][:, :, rows], sub[key], rtol=1e-10, atol=1e-12,
                                       err_msg=key)
        np.testing.assert_array_equal(packed["cnt"][:, :, a:b], sub["cnt"])
        shifted = np.where(sub["idx"] >= 0, sub["idx"] + a, -1)
        np.testing.assert_array_equal(packed["idx"][:, :, a:b], shifted)
        np.testing.assert_allclose(packed["ds"][:, :, a:b, a:b], sub["ds"], rtol=1e-10, atol=1e-12)
        # no gradient reaches the blocks of other documents
        assert np.all(packed["ds"][:, :, a:b, :a] == 0.0)
        a = b


def test_masked_row_matches_compacted_row():
    """A row with -inf scores selects exactly what the row without them
    selects, with the indices mapped back, and has the same LSE."""
    g = np.random.default_rng(3)
    i = 40
    row = g.standard_normal(48)
    keep = g.random(i) < 0.6
    masked = row.copy()
    masked[:i][~keep] = NEG_INF
    pos = np.flatnonzero(keep)
    for K in (0, 1, 5, 17, 40):
        ch, lg, lse = oracle.select_row(masked, i, K)
        ch2, lg2, lse2 = oracle.select_row(row[pos], len(pos), K)
        assert ch == [int(pos[c]) for c in ch2]
        assert lse == pytest.approx(lse2, rel=0, abs=1e-12)
        np.testing.assert_allclose(lg, lg2, rtol=0, atol=1e-12)


def test_row_without_candidates():
    """The first block of a document: every history score is -inf, so nothing
    is kept, there is no gate (s_lse = -inf) and the row's ds is zero."""
    s = np.full((1, 1, 4, 4), NEG_INF)
    s[0, 0, 3, :2] = [0.5, -1.0]     # row 3 has two candidates, rows 1 and 2 none
    idx, cnt, lg, s_lse = oracle.select(s, 2)
    assert list(cnt[0, 0]) == [0, 0, 0, 2]
    assert s_lse[0, 0, 1] == NEG_INF and s_lse[0, 0, 2] == NEG_INF
    dlg = np.zeros((1, 1, 4, 2))
    dlg[0, 0, 3] = [0.25, -0.5]
    ds = oracle.gate_jacobian(s, s_lse, idx, cnt, dlg)
    assert np.all(ds[0, 0, :3] == 0.0)
    assert np.all(np.isfinite(ds))
    assert ds[0, 0, 3, 2] == 0.0 and ds[0, 0, 3, 3] == 0.0
    assert ds[0, 0, 3, :2].sum() == pytest.approx(0.0, abs=1e-15)


def test_mask_documents_layout():
    """The mask touches exactly the blocks of earlier documents and clamps
    out-of-range starts."""
    g = np.random.default_rng(5)
    s = g.standard_normal((2, 3, 10, 10))
    first = np.array([si.doc_first_of([3, 4, 3]), [0, 0, -5, 2, 9, 1, 1, 7, 7, 7]])
    out = oracle.mask_documents(s, first)
    for b in range(2):
        for i in range(10):
            f = min(max(int(first[b, i]), 0), i)
            assert np.all(np.isneginf(out[b, :, i, :f]))
            assert np.array_equal(out[b, :, i, f:], s[b, :, i, f:])
    assert np.array_equal(si.doc_first_of([3, 4, 3]), [0, 0, 0, 3, 3, 3, 3, 7, 7, 7])


# ---------------------------------------------------------------- documents of any length
# Each document is cut into 64-token blocks from its own first token; its last
# block holds the rest (1..64 tokens).  The block geometry (first token and
# length of each block) carries that layout; the scores carry the document
# mask as before.

def _run_varlen(doc_lens, K, Hq, Hkv, d, seed, mode, n_extra=0):
    g = np.random.default_rng(seed)
    geom, first = oracle.blocks_of_documents(doc_lens)
    nb = len(geom)
    n = int(sum(doc_lens)) + n_extra
    q = g.standard_normal((1, Hq, n, d))
    k = g.standard_normal((1, Hkv, n, d))
    v = g.standard_normal((1, Hkv, n, d))
    do = g.standard_normal((1, Hq, n, d))
    s = g.standard_normal((1, Hkv, nb, nb)) * 1.3
    sp = oracle.mask_documents(s, first[None])
    packed = oracle.sas_forward_backward(q, k, v, do, sp, K, mode=mode, geom=geom[None])
    return q, k, v, do, s, geom, first, packed


@pytest.mark.parametrize("doc_lens,K,Hq,Hkv,mode", [
    ([100, 37, 230, 64, 1], 2, 2, 1, "gather"),
    ([130, 5, 64], 3, 4, 2, "dense"),
    ([63, 65, 127], 1, 2, 2, "gather"),
    ([300], 4, 2, 1, "dense")])
def test_varlen_documents_match_separate_runs(doc_lens, K, Hq, Hkv, mode):
    """A packed run over documents of any length gives, token for token, what
    a run over each document alone gives (its own blocks, the last one
    partial), and no gradient crosses documents."""
    q, k, v, do, s, geom, first, packed = _run_varlen(doc_lens, K, Hq, Hkv, 16,
                                                      sum(doc_lens) + K, mode)
    a = 0
    for L in doc_lens:
        rows = slice(a, a + L)
        bl = np.flatnonzero((geom[:, 0] >= a) & (geom[:, 0] < a + L))
        b0, b1 = int(bl[0]), int(bl[-1]) + 1
        gdoc, _ = oracle.blocks_of_documents([L])
        assert len(gdoc) == b1 - b0 and np.array_equal(gdoc[:, 0] + a, geom[b0:b1, 0])
        sub = oracle.sas_forward_backward(q[:, :, rows], k[:, :, rows], v[:, :, rows],
                                          do[:, :, rows], s[:, :, b0:b1, b0:b1], K, mode=mode,
                                          geom=gdoc[None])
        for key in ("o", "lse", "dq", "dk", "dv"):
            np.testing.assert_allclose(packed[key][:, :, rows], sub[key], rtol=1e-10, atol=1e-12,
                                       err_msg=key)
        np.testing.assert_array_equal(packed["cnt"][:, :, b0:b1], sub["cnt"])
        shifted = np.where(sub["idx"] >= 0, sub["idx"] + b0, -1)
        np.testing.assert_array_equal(packed["idx"][:, :, b0:b1], shifted)
        np.testing.assert_allclose(packed["ds"][:, :, b0:b1, b0:b1], sub["ds"], rtol=1e-10,
                                   atol=1e-12)
        assert np.all(packed["ds"][:, :, b0:b1, :b0] == 0.0)
        a += L


def test_uniform_geometry_is_the_block_grid():
    """The geometry of 64-token blocks reproduces the computation without a
    geometry exactly (dense and gather)."""
    g = np.random.default_rng(21)
    n, d, K = 5 * BLOCK, 16, 2
    q, k, v, do = (g.standard_normal((1, 2, n, d)) for _ in range(4))
    k, v = k[:, :1], v[:, :1]
    s = g.standard_normal((1, 1, 5, 5))
    geom = np.stack([np.arange(5) * BLOCK, np.full(5, BLOCK)], axis=1)[None]
    for mode in ("dense", "gather"):
        a = oracle.sas_forward_backward(q, k, v, do, s, K, mode=mode)
        b = oracle.sas_forward_backward(q, k, v, do, s, K, mode=mode, geom=geom)
        for key in ("o", "lse", "dq", "dk", "dv", "ds"):
            np.testing.assert_array_equal(a[key], b[key], err_msg=(mode, key))
    np.testing.assert_array_equal(oracle.pool_scores(q, k, 1), oracle.pool_scores(q, k, 1, geom))


def test_varlen_gather_equals_dense_with_tail_tokens():
    """Gather mode equals the dense definition on a packed layout whose
    documents leave tokens at the end of the buffer; those tokens attend to
    nothing (o = 0, lse = -inf) and receive no gradient."""
    lens = [70, 130, 9]
    dense = _run_varlen(lens, 2, 2, 1, 16, 5, "dense", n_extra=23)[-1]
    gath = _run_varlen(lens, 2, 2, 1, 16, 5, "gather", n_extra=23)[-1]
    for key in ("o", "dq", "dk", "dv", "ds"):
        np.testing.assert_allclose(gath[key], dense[key], rtol=1e-10, atol=1e-12, err_msg=key)
    end = sum(lens)
    assert np.all(dense["o"][:, :, end:] == 0.0) and np.all(np.isneginf(dense["lse"][:, :, end:]))
    for key in ("dq", "dk", "dv"):
        assert np.all(dense[key][:, :, end:] == 0.0), key


def test_varlen_finite_differences():
    """Central finite differences in float64 through select + forward on a
    packed layout with partial blocks (selection unchanged at s +- h)."""
    lens = [90, 40]
    K, h = 1, 1e-6
    q, k, v, do, s, geom, first, ref = _run_varlen(lens, K, 2, 1, 8, 77, "dense")
    g = np.random.default_rng(78)

    def loss(q_, k_, v_, s_):
        sp = oracle.mask_documents(s_, first[None])
        idx, cnt, lg, _ = oracle.select(sp, K)
        assert np.array_equal(idx, ref["idx"])
        o, _ = oracle.fwd_dense(q_, k_, v_, idx, cnt, lg, geom=geom[None])
        return float(np.sum(o * do))

    args = [q, k, v, s]
    grads = [ref["dq"], ref["dk"], ref["dv"], ref["ds"]]
    for j in range(4):
        dirn = g.standard_normal(args[j].shape)
        if j == 3:   # only the scores the selection reads (m < i, same document)
            sp = oracle.mask_documents(s, first[None])
            nb = s.shape[-1]
            dirn = np.where(np.isfinite(sp) & (np.arange(nb)[None, :] < np.arange(nb)[:, None]),
                            dirn, 0.0)
        plus = [x.copy() for x in args]
        minus = [x.copy() for x in args]
        plus[j] += h * dirn
        minus[j] -= h * dirn
        fd = (loss(*plus) - loss(*minus)) / (2 * h)
        an = float(np.sum(grads[j] * dirn))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (j, fd, an)


def test_blocks_of_documents_layout():
    geom, first = oracle.blocks_of_documents([100, 64, 1, 130])
    assert geom.tolist() == [[0, 64], [64, 36], [100, 64], [164, 1], [165, 64], [229, 64],
                             [293, 2]]
    assert first.tolist() == [0, 0, 2, 3, 4, 4, 4]
    gb, fb = oracle.packed_geometry([[100, 64], [10]])
    assert gb.shape == (2, 3, 2) and fb.shape == (2, 3)
    assert gb[1].tolist() == [[0, 10], [10, 0], [10, 0]] and fb[1].tolist() == [0, 1, 2]


def test_pool_scores_geometry_brute_force():
    """Mean pooling over each block's own tokens (loops, not the oracle's
    vectorised form); an empty padding block pools to zero."""
    g = np.random.default_rng(9)
    lens = [[70, 20], [33]]
    geom, _ = oracle.packed_geometry(lens)
    n, d, Hq, Hkv = 96, 8, 4, 2
    q = g.standard_normal((2, Hq, n, d))
    k = g.standard_normal((2, Hkv, n, d))
    s = oracle.pool_scores(q, k, Hkv, geom)
    G = Hq // Hkv
    for b in range(2):
        for kv in range(Hkv):
            for i in range(geom.shape[1]):
                for m in range(geom.shape[1]):
                    a_i, L_i = geom[b, i]
                    a_m, L_m = geom[b, m]
                    if L_i == 0 or L_m == 0:
                        assert s[b, kv, i, m] == 0.0
                        continue
                    qb = sum(q[b, kv * G + gg, t] for gg in range(G)
                             for t in range(a_i, a_i + L_i)) / (G * L_i)
                    kb = sum(k[b, kv, t] for t in range(a_m, a_m + L_m)) / L_m
                    assert s[b, kv, i, m] == pytest.approx(float(qb @ kb) / np.sqrt(d), rel=1e-12,
                                                           abs=1e-14)
