"""CPU oracle for SAS gated block-sparse attention (test infrastructure).

THIS IS TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it.  It shares no code with the HIP library and imports nothing
from it.  Everything is plain numpy in float64; inputs are whatever float arrays
the caller passes (bf16 workloads pass the bf16-rounded values as float32).

Sources (the only technical description of the method is the Chinese review
page "论文综述：SAS——通过端到端优化上下文排序实现简单的注意力稀疏化" on
paper.oopus.info, cited below as [Review]; the project README on gitee is
cited as [README]):

* [Review §2.1]  contiguous blocks of b = 64 tokens; the current block is
  always kept.
* [Review §2.2, selector equation]  scores s for every history block; keep the
  Top-K history blocks plus the current block; skip the rest.
* [Review §2.3, equation for o_SAS]  o = softmax(q K_S^T + log g_S) V_S.
* [Review §2.4, equation for log g_m]  log g_m = s_m - LSE(s) over the history
  blocks H; the current block has g_0 = 1 (no bias).
* [Review §2.6]  the fused kernel adds each selected block's log-gate to its
  logits, masks unselected blocks, leaves the current block unbiased; its
  backward sums the logit gradients inside each selected block to get that
  block's gate gradient.
* [README, figure caption (b)]  Top-K stays a discrete choice; gradients
  reach the selector only through the continuous gates.

Readings taken where the pages are silent (each is also listed in the design
notes):

* scale: logits are tau * (q . k) + log g with tau = 1/sqrt(d) by default; the
  gate bias is not scaled.
* selection granularity: one selection per (batch, kv-head, 64-query block),
  shared by the G = Hq/Hkv query heads of the group; query head h uses kv-head
  h // G.
* block numbering is absolute, 0 .. n/64-1; q-block i has history {0..i-1}
  and current block i.
* the LSE runs over all history blocks, selected or not; with fewer than K
  history blocks all of them are selected (still gated).
* a score of -inf marks a history block that is not a candidate: no part of
  the LSE, never kept, ds = 0; a packed batch puts -inf on every block of an
  earlier document (``mask_documents``).
* packed documents of any length: each document is cut into blocks of 64
  tokens from its own first token, its last block holding the remaining 1..64
  tokens; blocks are numbered in token order across the documents.  The
  block geometry ``geom`` [B, NB, 2] gives each block's first token and
  length (a length of 0 marks a padding block at the end of a batch entry,
  which holds no token); without it block i is tokens [64 i, 64 i + 64).  A
  token's current block is the block holding it; causal masking inside it
  runs on token positions.  Tokens outside every block attend to nothing
  (their outputs are 0).
* ties in s go to the lower block index; -0.0 and +0.0 are equal.
* idx lists the selected blocks in ascending order, padded with -1; padded
  log_gate entries are -inf; s_lse of a row with no history is -inf.
* causal rule inside the current block: key j is visible to query t iff j <= t.
* decode: the query is token T = seq_len-1; its current block is T // 64 and
  holds the tokens [64*(T//64), seq_len); its history is the blocks before it.
* pooling stand-in selector: s[i, m] = mean_{G heads, 64 rows}(q) .
  mean_{64 rows}(k_m) / sqrt(d), for every (i, m) pair.
* gate variants of the ablations [Review §2.3, §2.4, §2.5 and the ablation
  table of §4]; the selection is the same Top-K for all of them:
  - "softmax" (the method): log g_m = s_m - LSE(s_H), inside the softmax;
  - "sigmoid": log g_m = log sigmoid(s_m), inside the softmax, each block on
    its own (no normalisation over the history);
  - "hard": the kept blocks enter with g = 1 (no bias) and the backward is
    a straight-through estimator in log space: the gradient a kept block's
    bias receives is passed to the softmax log-gate s_m - LSE(s_H);
  - "external": g_m = exp(s_m - LSE(s_H)) scales the values of block m after
    an unbiased softmax over the kept and current keys (the current block has
    g = 1), o = sum_j P_j g_(block j) v_j.

Every function here is pinned by the CPU tests in ``tests/test_oracle_*.py``
(brute force, closed forms, invariants, library special cases, finite
differences); see each function's docstring for its pins.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 64
NEG_INF = -np.inf


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ============================================================== block geometry
def blocks_of_documents(doc_lens):
    """Blocks of packed documents of the given token lengths: each document is
    cut into 64-token blocks from its own first token (the last one partial).
    Returns (geom [NB, 2] int64: first token and length of each block,
    doc_first [NB] int64: the first block of each block's document)."""
    geom, first = [], []
    tok = 0
    for L in doc_lens:
        L = int(L)
        b0 = len(geom)
        for a in range(0, L, BLOCK):
            geom.append((tok + a, min(BLOCK, L - a)))
            first.append(b0)
        tok += L
    return np.asarray(geom, dtype=np.int64).reshape(-1, 2), np.asarray(first, dtype=np.int64)


def packed_geometry(doc_lens_per_batch):
    """Batch version of ``blocks_of_documents``: geom [B, NB, 2], doc_first
    [B, NB] with NB the largest block count; shorter entries are padded with
    zero-length blocks (first token = end of the entry's documents), each its
    own document."""
    parts = [blocks_of_documents(dl) for dl in doc_lens_per_batch]
    NB = max(len(g) for g, _ in parts)
    B = len(parts)
    geom = np.zeros((B, NB, 2), dtype=np.int64)
    first = np.zeros((B, NB), dtype=np.int64)
    for b, (g, f) in enumerate(parts):
        end = int(sum(int(x) for x in doc_lens_per_batch[b]))
        geom[b, :len(g)] = g
        geom[b, len(g):] = (end, 0)
        first[b, :len(f)] = f
        first[b, len(f):] = np.arange(len(f), NB)
    return geom, first


def _rows(geom_b, i: int):
    """Token rows of block i (geometry row geom_b, or the uniform grid)."""
    if geom_b is None:
        return np.arange(i * BLOCK, (i + 1) * BLOCK)
    a, L = int(geom_b[i][0]), int(geom_b[i][1])
    return np.arange(a, a + L)


def _rsl(geom_b, i: int):
    """The rows of block i as a slice (blocks are contiguous token ranges)."""
    r = _rows(geom_b, i)
    return slice(int(r[0]), int(r[-1]) + 1) if len(r) else slice(0, 0)


def _nblocks(n: int, geom):
    return n // BLOCK if geom is None else np.shape(geom)[1]


# ============================================================== pooling
def pool_scores(q, k, Hkv: int, geom=None):
    """Mean-pooled block scores (the stand-in selector of the 32K workload).

    s[b, kv, i, m] = qbar[b, kv, i] . kbar[b, kv, m] / sqrt(d), where qbar is
    the mean of the 64 rows x G query heads of q-block i in kv-group kv, and
    kbar the mean of the 64 rows of key block m.  Computed for every (i, m).

    Follows [Review §2.2] (a score per history block from q and K_{B_m}) with
    the mean-pool reading of the selector.  Pinned by: constant-block closed
    form and a pure-Python brute force on a tiny case.
    """
    q, k = _f64(q), _f64(k)
    B, Hq, n, d = q.shape
    G = Hq // Hkv
    if geom is None:
        nb = n // BLOCK
        qbar = q.reshape(B, Hkv, G, nb, BLOCK, d).mean(axis=(2, 4))
        kbar = k.reshape(B, Hkv, nb, BLOCK, d).mean(axis=3)
        return np.einsum("bkid,bkmd->bkim", qbar, kbar) / math.sqrt(d)
    # packed geometry: means over each block's own tokens (0 for an empty block)
    nb = np.shape(geom)[1]
    qbar = np.zeros((B, Hkv, nb, d))
    kbar = np.zeros((B, Hkv, nb, d))
    for b in range(B):
        for i in range(nb):
            r = _rows(geom[b], i)
            if len(r) == 0:
                continue
            qbar[b, :, i] = q[b][:, r].reshape(Hkv, G * len(r), d).mean(axis=1)
            kbar[b, :, i] = k[b][:, r].mean(axis=1)
    return np.einsum("bkid,bkmd->bkim", qbar, kbar) / math.sqrt(d)


# ============================================================== selection
def _log_gate(h, s_lse, gate: str):
    """Forward log-gate of a kept block with score h (see the gate variants in
    the module header)."""
    if gate in ("softmax", "external"):
        return float(h) - s_lse
    if gate == "sigmoid":
        return min(float(h), 0.0) - math.log1p(math.exp(-abs(float(h))))
    if gate == "hard":
        return 0.0
    raise ValueError(gate)


def select_row(srow, i: int, topk: int, gate: str = "softmax"):
    """Select for one query block i from its score row (length >= i).

    Returns (chosen ascending list, log_gate list aligned with it, s_lse).
    The log-gates follow ``gate`` (module header); s_lse is the LSE over the
    candidates for every variant.

    [Review §2.2]: keep the Top-K history blocks by score.  [Review §2.4]:
    log g_m = s_m - LSE over all history blocks.  Ranking key (-s_m, m) makes
    ties go to the lower index; adding +0.0 turns -0.0 into +0.0 first.
    A score of -inf marks a block that is not a candidate (in a packed batch,
    a block of an earlier document): it takes no part in the LSE and is never
    kept, so a row keeps min(K, number of finite scores) blocks, and a row
    with no finite score keeps none and has s_lse = -inf.
    Pinned by: a sort-free rank-count brute force, integer and signed-zero tie
    fixtures, shift invariance, permutation covariance, K = 0 and K >= i, and
    packed documents matching separate runs.
    """
    h = _f64(srow[:i]) + 0.0
    cand = [m for m in range(i) if h[m] > NEG_INF]
    if not cand:
        return [], [], NEG_INF
    hc = h[cand]
    mx = float(hc.max())
    s_lse = mx + math.log(float(np.sum(np.exp(hc - mx))))
    order = sorted(cand, key=lambda m: (-h[m], m))
    chosen = sorted(order[:min(topk, len(cand))])
    return chosen, [_log_gate(h[m], s_lse, gate) for m in chosen], s_lse


def mask_documents(s, doc_first):
    """Packed batch: return a copy of s with s[b,kv,i,m] = -inf for every
    m < doc_first[b,i] (the blocks of earlier documents), clamped to
    0 <= doc_first <= i.

    [Review §2.2, §2.4] applied per document: a q-block's candidates and its
    gate normalisation are its own document's earlier blocks.  Pinned by the
    packed-documents test: a packed run through this mask equals, block for
    block, separate runs over each document, with zero ds across documents.
    """
    out = _f64(s).copy()
    B, Hkv, NQB, _ = out.shape
    for b in range(B):
        for i in range(NQB):
            f = min(max(int(doc_first[b][i]), 0), i)
            out[b, :, i, :f] = NEG_INF
    return out


def select(s, topk: int, gate: str = "softmax"):
    """idx [B,Hkv,NQB,K] int32 (ascending, -1 padded), cnt [B,Hkv,NQB] int32,
    log_gate [B,Hkv,NQB,K] float64 (-inf padded), s_lse [B,Hkv,NQB] float64.

    Row i of s is the score row of q-block i; only entries m < i are read.
    """
    s = np.asarray(s)
    B, Hkv, NQB, _ = s.shape
    K = int(topk)
    idx = np.full((B, Hkv, NQB, K), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv, NQB), dtype=np.int32)
    lg = np.full((B, Hkv, NQB, K), NEG_INF)
    lse = np.full((B, Hkv, NQB), NEG_INF)
    for b in range(B):
        for kv in range(Hkv):
            for i in range(NQB):
                ch, g, l = select_row(s[b, kv, i], i, K, gate)
                c = len(ch)
                cnt[b, kv, i] = c
                idx[b, kv, i, :c] = ch
                lg[b, kv, i, :c] = g
                lse[b, kv, i] = l
    return idx, cnt, lg, lse


# ============================================================== forward
def bias_matrix(n: int, idx_row, cnt_row, lg_row, geom_b=None):
    """Dense n x n additive bias of one (batch, kv-head) [Review §2.3, §2.6].

    A[t, j] = 0 if j is in t's own block and j <= t (current block, g_0 = 1);
    A[t, j] = log_gate of block(j) if block(j) is selected by block(t);
    A[t, j] = -inf otherwise (skipped).  Blocks follow ``geom_b`` when given.
    """
    nb = n // BLOCK if geom_b is None else len(geom_b)
    A = np.full((n, n), NEG_INF)
    for i in range(nb):
        r = _rows(geom_b, i)
        if len(r) == 0:
            continue
        for slot in range(int(cnt_row[i])):
            m = int(idx_row[i, slot])
            A[np.ix_(r, _rows(geom_b, m))] = lg_row[i, slot]
        tri = np.tril(np.ones((len(r), len(r)), dtype=bool))
        blk = A[np.ix_(r, r)]
        blk[tri] = 0.0
        A[np.ix_(r, r)] = blk
    return A


def _softmax_rows(Z):
    """Row softmax and row logsumexp; a row with no finite logit (a token
    outside every block) gets weights 0 and logsumexp -inf."""
    M = Z.max(axis=-1, keepdims=True)
    empty = ~np.isfinite(M)
    M = np.where(empty, 0.0, M)
    with np.errstate(divide="ignore"):
        L = M + np.log(np.sum(np.exp(Z - M), axis=-1, keepdims=True))
    P = np.where(empty, 0.0, np.exp(Z - np.where(empty, 0.0, L)))
    return P, np.where(empty, NEG_INF, L)[..., 0]


def _placed(A, gate: str):
    """(logit bias, value weights) of the dense bias A for the gate's place:
    inside the softmax the bias is A and the weights are 1; outside it the
    logits keep only the mask (0 or -inf) and each key's value is scaled by
    g = exp(A) (1 for the current block, 0 where masked)."""
    if gate == "external":
        return np.where(np.isfinite(A), 0.0, NEG_INF), np.exp(A)
    return A, np.ones_like(A)


def fwd_dense(q, k, v, idx, cnt, log_gate, scale=None, gate: str = "softmax", geom=None):
    """Dense definition: for each query head h (kv-head h // G),
    Z = tau Q_h K^T + A, L = rowwise logsumexp(Z), O_h = exp(Z - L) V.
    For the external gate, Z keeps only A's mask and O_h = (exp(Z - L) o W) V
    with W = exp(A) (module header).

    [Review §2.3] equation for o_SAS with the bias A of ``bias_matrix``.
    Returns (o [B,Hq,n,d], lse [B,Hq,n]) in float64.  Pinned by: K = 0 equals
    block-diagonal causal SDPA; constant scores with K >= n/64 equal causal
    SDPA with a -log(i) history bias; q-block 0 equals causal SDPA; output
    permutation and shift invariance; GQA equals MHA with repeated K/V.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    tau = (1.0 / math.sqrt(d)) if not scale else float(scale)
    o = np.zeros_like(q)
    lse = np.zeros((B, Hq, n))
    for b in range(B):
        for kv in range(Hkv):
            A, W = _placed(bias_matrix(n, idx[b, kv], cnt[b, kv], log_gate[b, kv],
                                       None if geom is None else geom[b]), gate)
            for g in range(G):
                h = kv * G + g
                P, L = _softmax_rows(tau * q[b, h] @ k[b, kv].T + A)
                o[b, h] = (P * W) @ v[b, kv]
                lse[b, h] = L
    return o, lse


def _gather_cols(i: int, idx_row, cnt_row, lg_row, geom_b=None):
    """Key columns of q-block i (selected blocks in slot order, then the
    current block) with their per-column log-gate (0 for the current block)
    and block slot (-1 = current)."""
    cols, bias, slot = [], [], []
    for sl in range(int(cnt_row[i])):
        m = int(idx_row[i, sl])
        c = _rows(geom_b, m)
        cols.append(c)
        bias.append(np.full(len(c), float(lg_row[i, sl])))
        slot.append(np.full(len(c), sl))
    c = _rows(geom_b, i)
    cols.append(c)
    bias.append(np.zeros(len(c)))
    slot.append(np.full(len(c), -1))
    return np.concatenate(cols), np.concatenate(bias), np.concatenate(slot)


def _block_logits(qi, kc, bias, slot, tau):
    """Z for the rows of one q-block over its gathered columns, with the
    causal mask (j <= t) on the current block's columns."""
    Z = tau * qi @ kc.T + bias[None, :]
    cur = slot == -1
    nr = qi.shape[0]
    tri = np.tril(np.ones((nr, nr), dtype=bool))
    Zc = Z[:, cur]
    Zc[~tri] = NEG_INF
    Z[:, cur] = Zc
    return Z


def _placed_cols(lgc, gate: str):
    """(logit bias, value weights) of gathered columns with log-gates lgc."""
    if gate == "external":
        return np.zeros_like(lgc), np.exp(lgc)
    return lgc, np.ones_like(lgc)


def fwd_gather_block(q, k, v, idx, cnt, log_gate, b: int, kv: int, i: int, scale=None,
                     gate: str = "softmax", geom=None):
    """Gather-mode forward of one (batch, kv-group, q-block): the formula of
    ``fwd_dense`` evaluated only on columns whose bias is finite, which is
    exact because exp(-inf) = 0.  Returns (o [G,rows,d], lse [G,rows]) for the
    block's rows (64 of them without a geometry)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Hq, d = q.shape[1], q.shape[3]
    Hkv = k.shape[1]
    G = Hq // Hkv
    tau = (1.0 / math.sqrt(d)) if not scale else float(scale)
    gb = None if geom is None else geom[b]
    cols, lgc, slot = _gather_cols(i, idx[b, kv], cnt[b, kv], log_gate[b, kv], gb)
    bias, w = _placed_cols(lgc, gate)
    kc, vc = k[b, kv, cols], v[b, kv, cols] * w[:, None]
    r = _rows(gb, i)
    o = np.zeros((G, len(r), d))
    lse = np.zeros((G, len(r)))
    for g in range(G):
        P, L = _softmax_rows(_block_logits(q[b, kv * G + g, r], kc, bias, slot, tau))
        o[g] = P @ vc
        lse[g] = L
    return o, lse


def fwd_gather(q, k, v, idx, cnt, log_gate, scale=None, blocks=None, gate: str = "softmax",
               geom=None):
    """Gather-mode forward over all q-blocks (or the (b, kv, i) list given).
    Tokens outside every block keep o = 0 and lse = -inf."""
    B, Hq, n, d = np.shape(q)
    Hkv = np.shape(k)[1]
    G = Hq // Hkv
    o = np.zeros((B, Hq, n, d))
    lse = np.full((B, Hq, n), NEG_INF)
    todo = blocks if blocks is not None else [
        (b, kv, i) for b in range(B) for kv in range(Hkv) for i in range(_nblocks(n, geom))]
    for (b, kv, i) in todo:
        ob, lb = fwd_gather_block(q, k, v, idx, cnt, log_gate, b, kv, i, scale, gate, geom)
        r = _rsl(None if geom is None else geom[b], i)
        o[b, kv * G:(kv + 1) * G, r] = ob
        lse[b, kv * G:(kv + 1) * G, r] = lb
    return o, lse


# ============================================================== backward
def gate_jacobian(s, s_lse, idx, cnt, dlg, gate: str = "softmax"):
    """ds from the per-slot gate gradient dlg (chain rule through [Review §2.4]).

    log g_m = s_m - LSE(s_H) for m in H_i, so for every history block m:
    ds[i, m] = [m selected] dlg[i, m] - pi_i[m] * sum_{m' selected} dlg[i, m'],
    pi_i = softmax(s[i, H_i]) = exp(s - s_lse).  Entries m >= i are 0, and so
    are blocks with s = -inf (not candidates, pi = 0) and rows with no
    candidate at all (no gate, s_lse = -inf).
    Pinned by finite differences through select + forward, and by
    sum_m ds[i, m] = 0.

    The "external" gate has the same log-gate, and "hard" passes its bias
    gradient to that log-gate (straight-through), so both use this Jacobian.
    For "sigmoid", d log sigmoid(s)/ds = sigmoid(-s) and blocks do not
    interact: ds[i, m] = [m selected] dlg[i, m] sigmoid(-s[i, m]).
    """
    s = _f64(s)
    B, Hkv, NQB, NKB = s.shape
    ds = np.zeros((B, Hkv, NQB, NKB))
    if gate == "sigmoid":
        for b in range(B):
            for kv in range(Hkv):
                for i in range(NQB):
                    for sl in range(int(cnt[b, kv, i])):
                        m = int(idx[b, kv, i, sl])
                        ds[b, kv, i, m] = dlg[b, kv, i, sl] / (1.0 + math.exp(s[b, kv, i, m]))
        return ds
    for b in range(B):
        for kv in range(Hkv):
            for i in range(1, NQB):
                c = int(cnt[b, kv, i])
                if s_lse[b, kv, i] == NEG_INF:
                    continue
                pi = np.exp(s[b, kv, i, :i] - s_lse[b, kv, i])
                tot = float(np.sum(dlg[b, kv, i, :c]))
                ds[b, kv, i, :i] = -pi * tot
                for sl in range(c):
                    ds[b, kv, i, int(idx[b, kv, i, sl])] += dlg[b, kv, i, sl]
    return ds


def bwd_dense(q, k, v, do, idx, cnt, log_gate, scale=None, gate: str = "softmax", geom=None):
    """Analytic backward of the dense definition (no autograd).

    With P = softmax(Z), O = P V and upstream dO:
      D = rowsum(dO o O), dP = dO V^T, dZ = P o (dP - D),
      dQ_h = tau dZ K, dK = tau sum_h dZ^T Q_h, dV = sum_h P^T dO_h,
      dlg[i, slot] = sum over the group's heads, rows t of block i and columns
      j of the slot's block m of dZ[t, j]  ([Review §2.6] block-sum rule).
    External gate (O = (P o W) V): dP = (dO V^T) o W, dV = sum_h (P o W)^T dO_h,
    and the log-gate gradient of a block is the sum of P o dP over its
    columns (d/dlog g of g * P dP).
    Returns (dq, dk, dv, dlg [B,Hkv,NQB,K]) in float64.  Pinned by central
    finite differences in float64 and by the row identity sum_j dZ[t, j] = 0.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    K = idx.shape[-1]
    tau = (1.0 / math.sqrt(d)) if not scale else float(scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    nb = _nblocks(n, geom)
    dlg = np.zeros((B, Hkv, nb, K))
    for b in range(B):
        gb = None if geom is None else geom[b]
        for kv in range(Hkv):
            A, W = _placed(bias_matrix(n, idx[b, kv], cnt[b, kv], log_gate[b, kv], gb), gate)
            for g in range(G):
                h = kv * G + g
                P, _ = _softmax_rows(tau * q[b, h] @ k[b, kv].T + A)
                O = (P * W) @ v[b, kv]
                D = np.sum(do[b, h] * O, axis=1, keepdims=True)
                dP = (do[b, h] @ v[b, kv].T) * W
                dZ = P * (dP - D)
                dq[b, h] = tau * dZ @ k[b, kv]
                dk[b, kv] += tau * dZ.T @ q[b, h]
                dv[b, kv] += (P * W).T @ do[b, h]
                G_ = P * dP if gate == "external" else dZ
                for i in range(nb):
                    r = _rows(gb, i)
                    for sl in range(int(cnt[b, kv, i])):
                        m = int(idx[b, kv, i, sl])
                        dlg[b, kv, i, sl] += G_[np.ix_(r, _rows(gb, m))].sum()
    return dq, dk, dv, dlg


def bwd_gather_block(q, k, v, do, idx, cnt, log_gate, b: int, kv: int, i: int, scale=None,
                     gate: str = "softmax", geom=None):
    """Backward contributions of one (batch, kv-group, q-block) in gather mode.

    Returns (dq [G,rows,d], cols, dk_cols [len(cols),d], dv_cols, dlg_row [K]):
    dq of the block's rows is complete; dk_cols/dv_cols are this q-block's
    additive contributions to the gathered key rows ``cols``.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    Hq, d = q.shape[1], q.shape[3]
    Hkv = k.shape[1]
    G = Hq // Hkv
    K = idx.shape[-1]
    tau = (1.0 / math.sqrt(d)) if not scale else float(scale)
    gb = None if geom is None else geom[b]
    cols, lgc, slot = _gather_cols(i, idx[b, kv], cnt[b, kv], log_gate[b, kv], gb)
    bias, w = _placed_cols(lgc, gate)
    kc, vc = k[b, kv, cols], v[b, kv, cols] * w[:, None]
    r = _rows(gb, i)
    dq = np.zeros((G, len(r), d))
    dkc = np.zeros((len(cols), d))
    dvc = np.zeros((len(cols), d))
    dlg = np.zeros(K)
    for g in range(G):
        h = kv * G + g
        P, _ = _softmax_rows(_block_logits(q[b, h, r], kc, bias, slot, tau))
        O = P @ vc
        D = np.sum(do[b, h, r] * O, axis=1, keepdims=True)
        dP = do[b, h, r] @ vc.T
        dZ = P * (dP - D)
        dq[g] = tau * dZ @ kc
        dkc += tau * dZ.T @ q[b, h, r]
        dvc += w[:, None] * (P.T @ do[b, h, r])
        colsum = (P * dP if gate == "external" else dZ).sum(axis=0)
        for sl in range(int(cnt[b, kv, i])):
            dlg[sl] += colsum[slot == sl].sum()
    return dq, cols, dkc, dvc, dlg


def bwd_gather(q, k, v, do, idx, cnt, log_gate, scale=None, blocks=None, gate: str = "softmax",
               geom=None):
    """Gather-mode backward over all q-blocks (or the listed (b, kv, i)).

    With ``blocks`` given, dq is exact on those q-blocks' rows only and dk/dv
    hold just their contributions."""
    B, Hq, n, d = np.shape(q)
    Hkv = np.shape(k)[1]
    G = Hq // Hkv
    K = idx.shape[-1]
    dq = np.zeros((B, Hq, n, d))
    dk = np.zeros((B, Hkv, n, d))
    dv = np.zeros((B, Hkv, n, d))
    nb = _nblocks(n, geom)
    dlg = np.zeros((B, Hkv, nb, K))
    todo = blocks if blocks is not None else [
        (b, kv, i) for b in range(B) for kv in range(Hkv) for i in range(nb)]
    for (b, kv, i) in todo:
        dqb, cols, dkc, dvc, dl = bwd_gather_block(q, k, v, do, idx, cnt, log_gate, b, kv, i, scale,
                                                   gate, geom)
        dq[b, kv * G:(kv + 1) * G, _rsl(None if geom is None else geom[b], i)] = dqb
        np.add.at(dk[b, kv], cols, dkc)
        np.add.at(dv[b, kv], cols, dvc)
        dlg[b, kv, i] = dl
    return dq, dk, dv, dlg


def reverse_lists(idx, cnt, b: int, kv: int, m: int):
    """q-blocks whose key set contains block m: those that selected it, plus
    block m itself (its current block)."""
    NQB = idx.shape[2]
    out = [i for i in range(m + 1, NQB)
           if m in set(int(x) for x in idx[b, kv, i, :int(cnt[b, kv, i])])]
    return [m] + out


def bwd_kv_block(q, k, v, do, idx, cnt, log_gate, b: int, kv: int, m: int, scale=None,
                 gate: str = "softmax", geom=None):
    """dk, dv [rows, d] of key block m of (b, kv), summed over every q-block
    that reads it (sampled full-size checks)."""
    d = np.shape(q)[3]
    rows = _rows(None if geom is None else geom[b], m)
    dk = np.zeros((len(rows), d))
    dv = np.zeros((len(rows), d))
    for i in reverse_lists(idx, cnt, b, kv, m):
        _, cols, dkc, dvc, _ = bwd_gather_block(q, k, v, do, idx, cnt, log_gate, b, kv, i, scale,
                                                gate, geom)
        sel = np.isin(cols, rows)
        pos = cols[sel] - (int(rows[0]) if len(rows) else 0)
        np.add.at(dk, pos, dkc[sel])
        np.add.at(dv, pos, dvc[sel])
    return dk, dv


# ============================================================== full pipeline
def sas_forward_backward(q, k, v, do, s, topk: int, scale=None, mode: str = "gather",
                         gate: str = "softmax", geom=None):
    """select -> forward -> backward -> ds, everything float64 (blocks of the
    geometry ``geom`` when given).
    Returns a dict with idx, cnt, log_gate, s_lse, o, lse, dq, dk, dv, dlg, ds."""
    idx, cnt, lg, s_lse = select(s, topk, gate)
    if mode == "dense":
        o, lse = fwd_dense(q, k, v, idx, cnt, lg, scale, gate, geom)
        dq, dk, dv, dlg = bwd_dense(q, k, v, do, idx, cnt, lg, scale, gate, geom)
    else:
        o, lse = fwd_gather(q, k, v, idx, cnt, lg, scale, gate=gate, geom=geom)
        dq, dk, dv, dlg = bwd_gather(q, k, v, do, idx, cnt, lg, scale, gate=gate, geom=geom)
    ds = gate_jacobian(s, s_lse, idx, cnt, dlg, gate)
    return dict(idx=idx, cnt=cnt, log_gate=lg, s_lse=s_lse, o=o, lse=lse,
                dq=dq, dk=dk, dv=dv, dlg=dlg, ds=ds)


# ============================================================== decode
def decode(q, k_cache, v_cache, seq_lens, s, topk: int, scale=None, rows=None,
           gate: str = "softmax"):
    """Single-token decode.  For batch entry b the query is token
    T = seq_len - 1 in block i = T // 64; kv-group kv selects from s[b, kv, :i]
    exactly as ``select_row``; each query head h of the group attends to the
    selected blocks (bias log_gate) and to keys [64 i, seq_len) (bias 0); the
    external gate scales the selected blocks' values instead.

    ``rows`` limits the work to a list of (b, kv); k_cache/v_cache may then be
    dicts {(b, kv): (k [cap,d] or block-indexable array)} - any object with
    [b, kv] indexing that returns the [cap, d] cache of that pair works.
    Returns (o [B,Hq,d] float64, idx [B,Hkv,K] int32); unlisted rows are 0/-1.
    """
    q = _f64(q)
    B, Hq, d = q.shape
    Hkv = s.shape[1]
    G = Hq // Hkv
    K = int(topk)
    tau = (1.0 / math.sqrt(d)) if not scale else float(scale)
    o = np.zeros((B, Hq, d))
    idx = np.full((B, Hkv, K), -1, dtype=np.int32)
    todo = rows if rows is not None else [(b, kv) for b in range(B) for kv in range(Hkv)]
    for (b, kv) in todo:
        L = int(seq_lens[b])
        T = L - 1
        i = T // BLOCK
        chosen, lg, _ = select_row(s[b, kv], i, K, gate)
        idx[b, kv, :len(chosen)] = chosen
        kc_all, vc_all = k_cache[b, kv], v_cache[b, kv]
        cols = [np.arange(m * BLOCK, (m + 1) * BLOCK) for m in chosen]
        lgc = [np.full(BLOCK, g) for g in lg]
        cols.append(np.arange(i * BLOCK, L))
        lgc.append(np.zeros(L - i * BLOCK))
        cols = np.concatenate(cols)
        bias, w = _placed_cols(np.concatenate(lgc), gate)
        kc = _f64(kc_all[cols])
        vc = _f64(vc_all[cols]) * w[:, None]
        for g in range(G):
            h = kv * G + g
            z = tau * kc @ q[b, h] + bias
            z = z - z.max()
            p = np.exp(z)
            o[b, h] = (p / p.sum()) @ vc
    return o, idx


# ============================================================== work counts
def selected_pairs(cnt, geom=None):
    """Valid (query, key) pairs per query head, summed over (b, kv, i):
    64*64 per selected block plus 64*65/2 for the causal current block (with
    a geometry: rows x kept-block length, plus L(L+1)/2 for a current block of
    L tokens; kept blocks are whole blocks of 64)."""
    cnt = np.asarray(cnt, dtype=np.int64)
    if geom is None:
        return int(cnt.sum()) * BLOCK * BLOCK + cnt.size * (BLOCK * (BLOCK + 1) // 2)
    L = np.asarray(geom)[..., 1].astype(np.int64)[:, None, :]      # [B, 1, NB]
    return int(np.sum(cnt * L * BLOCK + L * (L + 1) // 2))
