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
