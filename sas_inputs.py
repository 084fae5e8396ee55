"""Seeded synthetic inputs for the SAS gated block-sparse attention path.

This module is shared by the tests, ``bench.py`` and ``__graft_entry__.smoke``.
It draws random numbers and rounds them to the storage dtype; it contains none
of the method's arithmetic (no pooling, selection, softmax or attention).

Every tensor comes from ``numpy.random.Generator(PCG64(SeedSequence([cfg, tid])))``
with ``tid`` = 0 q, 1 k, 2 v, 3 s, 4 dO, 5 decode lengths; ``cfg`` is the
workload number below (or any integer seed for ad-hoc shapes).  Values are
drawn in float32 and, for bf16 workloads, rounded to bf16 with round-to-nearest-
even; both the GPU path and the oracle read the same rounded values.

Workloads (shapes follow the Qwen3 attention layers named on the pages' model
table; the 32768 training length and the 1024/2048/4096 token budgets are the
ones the review page's setup and results sections state):

1. tiny fp32: B=1, Hq=Hkv=1, d=64, n=512, K=2; q,k,v,s,dO ~ N(0,1).
2. Qwen3-4B layer, bf16: B=1, Hq=32, Hkv=8, d=128, n=8192, K=16;
   q,k,v ~ N(0,1)/sqrt(2); s ~ N(0, variance 2); dO ~ N(0,1).
3. Qwen3-8B layer, bf16: B=1, Hq=32, Hkv=8, d=128, n=32768, K=32;
   q,k,v,dO ~ N(0,1); s is produced on the device by block-score pooling.
4. Qwen3-14B layer, bf16: B=1, Hq=40, Hkv=8, d=128, n=32768, K=64;
   q,k,v,dO ~ N(0,1); s = 3 * Gumbel(0,1) = -3 log(-log U).
5. decode, bf16: B=64, Hq=32, Hkv=8, d=128, cache 32768 (512 blocks), K=32;
   q ~ N(0,1); cache ~ N(0,1); seq_len = 511*64 + L with L ~ U{1..64};
   s ~ N(0,1) of shape [B, Hkv, 512].
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BLOCK = 64

TID_Q, TID_K, TID_V, TID_S, TID_DO, TID_LEN, TID_PAGES, TID_DOCS = 0, 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one training-layer workload (q-block granularity is 64)."""
    cfg: int
    B: int
    Hq: int
    Hkv: int
    n: int
    d: int
    topk: int
    dtype: str          # "f32" or "bf16"
    qkv_std: float = 1.0
    s_kind: str = "normal"   # "normal" | "pool" | "gumbel3"
    s_std: float = 1.0
    packed: bool = False     # each batch entry packs several documents (make_doc_first)
    varlen: bool = False     # packed documents of any token length (doc_token_lens)
    tail: int = 0            # varlen: tokens left after the last document

    @property
    def nqb(self) -> int:
        """Blocks per batch entry: n/64, or for documents of any length the
        most blocks any batch entry needs (each document cut into 64-token
        blocks from its first token)."""
        if not self.varlen:
            return self.n // BLOCK
        return max(sum((L + BLOCK - 1) // BLOCK for L in doc_token_lens(self, b))
                   for b in range(self.B))

    @property
    def name(self) -> str:
        return WORKLOAD_NAMES.get(self.cfg, f"custom{self.cfg}")


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    cfg: int
    B: int
    Hq: int
    Hkv: int
    cap: int
    d: int
    topk: int
    dtype: str = "bf16"
    hist_blocks: int = 511      # history blocks before the partial current block

    @property
    def name(self) -> str:
        return WORKLOAD_NAMES.get(self.cfg, f"custom{self.cfg}")


WORKLOAD_NAMES = {
    1: "tiny-fp32-n512-K2",
    2: "qwen3-4b-layer-n8192-K16",
    3: "qwen3-8b-layer-n32768-K32",
    4: "qwen3-14b-layer-n32768-K64",
    7: "qwen3-8b-layer-n32768-K32-packed",
    10: "qwen3-8b-layer-n32768-K32-packed-aligned",
    8: "qwen3-8b-layer-n32768-full",
    9: "qwen3-4b-layer-n8192-full",
    5: "decode-qwen3-8b-B64-cache32768-K32",
}

WORKLOADS = {
    1: Workload(1, 1, 1, 1, 512, 64, 2, "f32"),
    2: Workload(2, 1, 32, 8, 8192, 128, 16, "bf16", qkv_std=1 / math.sqrt(2),
                s_kind="normal", s_std=math.sqrt(2.0)),
    3: Workload(3, 1, 32, 8, 32768, 128, 32, "bf16", s_kind="pool"),
    4: Workload(4, 1, 40, 8, 32768, 128, 64, "bf16", s_kind="gumbel3"),
    # documents of any token length packed into the 32K sequence
    7: Workload(7, 1, 32, 8, 32768, 128, 32, "bf16", s_kind="normal", varlen=True),
    # documents of whole 64-token blocks (no block table)
    10: Workload(10, 1, 32, 8, 32768, 128, 32, "bf16", s_kind="normal", packed=True),
    # full-range gated attention: K covers every history block
    8: Workload(8, 1, 32, 8, 32768, 128, 512, "bf16", s_kind="pool"),
    9: Workload(9, 1, 32, 8, 8192, 128, 128, "bf16", qkv_std=1 / math.sqrt(2),
                s_kind="normal", s_std=math.sqrt(2.0)),
}

DECODE_WORKLOAD = DecodeWorkload(5, 64, 32, 8, 32768, 128, 32)


@dataclasses.dataclass(frozen=True)
class PagedDecodeWorkload:
    """Long-context paged decode: B sequences of about 64*max_blocks tokens in
    a pool of B*max_blocks one-block pages (every block its own page, the pages
    of a sequence scattered over the pool)."""
    cfg: int
    B: int
    Hq: int
    Hkv: int
    max_blocks: int
    d: int
    topk: int
    dtype: str = "bf16"

    @property
    def name(self) -> str:
        return (f"decode-paged-qwen3-8b-B{self.B}-ctx{self.max_blocks * BLOCK}-K{self.topk}")

    @property
    def num_pages(self) -> int:
        return self.B * self.max_blocks


# Qwen3-8B attention shape, one sequence of a 512K-token context (the batch-1,
# 512K decode setting of the SAS review page, §4)
PAGED_DECODE_WORKLOAD = PagedDecodeWorkload(6, 1, 32, 8, 8192, 128, 32)
# the other decode settings of the review page's §4 speed-up results: batch 1
# at 64K and 256K tokens, batch 8 at 64K
PAGED_DECODE_SWEEP = [PagedDecodeWorkload(11, 1, 32, 8, 1024, 128, 32),
                      PagedDecodeWorkload(12, 1, 32, 8, 4096, 128, 32),
                      PAGED_DECODE_WORKLOAD,
                      PagedDecodeWorkload(13, 8, 32, 8, 1024, 128, 32)]


def rng(cfg: int, tid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(cfg), int(tid)])))


# ---------------------------------------------------------------- bf16 storage
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values that are exactly representable in bf16 (nearest-even)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def _normal(cfg, tid, shape, std=1.0, chunk=1 << 24):
    g = rng(cfg, tid)
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    for o in range(0, flat.size, chunk):
        e = min(flat.size, o + chunk)
        g.standard_normal(e - o, dtype=np.float32, out=flat[o:e])
    if std != 1.0:
        flat *= np.float32(std)
    return out


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return x if dtype == "f32" else round_to_bf16(x)


# ---------------------------------------------------------------- training layer
def make_qkv(w: Workload, with_do: bool = True):
    """q [B,Hq,n,d], k, v [B,Hkv,n,d], dO [B,Hq,n,d] as float32 arrays holding
    values representable in the storage dtype."""
    q = _store(_normal(w.cfg, TID_Q, (w.B, w.Hq, w.n, w.d), w.qkv_std), w.dtype)
    k = _store(_normal(w.cfg, TID_K, (w.B, w.Hkv, w.n, w.d), w.qkv_std), w.dtype)
    v = _store(_normal(w.cfg, TID_V, (w.B, w.Hkv, w.n, w.d), w.qkv_std), w.dtype)
    do = _store(_normal(w.cfg, TID_DO, (w.B, w.Hq, w.n, w.d)), w.dtype) if with_do else None
    return q, k, v, do


def make_scores(w: Workload) -> np.ndarray | None:
    """Selector scores s [B,Hkv,NQB,NKB] fp32, or None when the workload makes
    them on the device (s_kind == "pool")."""
    shape = (w.B, w.Hkv, w.nqb, w.nqb)
    if w.s_kind == "normal":
        return _normal(w.cfg, TID_S, shape, w.s_std)
    if w.s_kind == "gumbel3":
        u = rng(w.cfg, TID_S).random(shape, dtype=np.float64)
        u = np.clip(u, np.finfo(np.float64).tiny, None)
        return (-3.0 * np.log(-np.log(u))).astype(np.float32)
    if w.s_kind == "pool":
        return None
    raise ValueError(w.s_kind)


def custom_workload(seed: int, B: int, Hq: int, Hkv: int, n: int, d: int, topk: int,
                    dtype: str = "bf16", s_kind: str = "normal", qkv_std: float = 1.0,
                    s_std: float = 1.0, packed: bool = False, varlen: bool = False,
                    tail: int = 0) -> Workload:
    """A smaller workload with the same value distributions (parity tests)."""
    return Workload(seed, B, Hq, Hkv, n, d, topk, dtype, qkv_std=qkv_std,
                    s_kind=s_kind, s_std=s_std, packed=packed, varlen=varlen, tail=tail)


# ---------------------------------------------------------------- packed documents
def doc_first_of(doc_blocks) -> np.ndarray:
    """int32 [sum(doc_blocks)]: the first block of the document holding each
    block, for documents of doc_blocks[j] blocks laid end to end."""
    first, start = [], 0
    for nb in doc_blocks:
        first += [start] * int(nb)
        start += int(nb)
    return np.array(first, dtype=np.int32)


def packed_doc_blocks(cfg: int, b: int, nb: int) -> list[int]:
    """Document lengths (in blocks) of batch entry b: log-uniform between one
    block and the whole sequence, drawn until the nb blocks are filled (the
    last document is cut at the end), so long and short documents mix."""
    g = np.random.default_rng([cfg, TID_DOCS, b])
    out, left = [], nb
    while left > 0:
        ln = int(np.exp(g.uniform(0.0, math.log(nb + 1))))
        ln = max(1, min(ln, left))
        out.append(ln)
        left -= ln
    return out


def doc_token_lens(w: Workload, b: int) -> list[int]:
    """Document lengths in tokens of batch entry b of a varlen workload:
    log-uniform between 1 token and the whole sequence, drawn until n - tail
    tokens are filled (the last document is cut there), so documents of every
    length mix and most are not multiples of 64.  Batch entries differ."""
    g = np.random.default_rng([w.cfg, TID_DOCS, b, 1])
    total = w.n - w.tail - (b * 37 if w.B > 1 else 0)    # entries of different lengths
    out, left = [], total
    while left > 0:
        ln = int(np.exp(g.uniform(0.0, math.log(total + 1))))
        ln = max(1, min(ln, left))
        out.append(ln)
        left -= ln
    return out


def cu_seqlens_of(lens) -> list[int]:
    """Document offsets [0, L0, L0+L1, ...] of documents laid end to end."""
    out = [0]
    for L in lens:
        out.append(out[-1] + int(L))
    return out


def make_doc_first(w: Workload) -> np.ndarray | None:
    """doc_first [B, NQB] int32 of a packed workload, None otherwise."""
    if not w.packed:
        return None
    return np.stack([doc_first_of(packed_doc_blocks(w.cfg, b, w.nqb)) for b in range(w.B)])


# ---------------------------------------------------------------- decode
def make_decode_small(w: DecodeWorkload):
    """All decode inputs on the host (small caps only): q [B,Hq,d],
    k_cache, v_cache [B,Hkv,cap,d], seq_lens [B] int32, s [B,Hkv,cap/64]."""
    q = _store(_normal(w.cfg, TID_Q, (w.B, w.Hq, w.d)), w.dtype)
    kc = _store(_normal(w.cfg, TID_K, (w.B, w.Hkv, w.cap, w.d)), w.dtype)
    vc = _store(_normal(w.cfg, TID_V, (w.B, w.Hkv, w.cap, w.d)), w.dtype)
    s = _normal(w.cfg, TID_S, (w.B, w.Hkv, w.cap // BLOCK))
    return q, kc, vc, decode_seq_lens(w), s


def decode_seq_lens(w: DecodeWorkload) -> np.ndarray:
    L = rng(w.cfg, TID_LEN).integers(1, BLOCK + 1, size=w.B)
    return (w.hist_blocks * BLOCK + L).astype(np.int32)


def make_decode_paged(cfg: int, B: int, Hq: int, Hkv: int, max_blocks: int, num_pages: int,
                      d: int, dtype: str = "bf16", seq_lens=None):
    """Inputs of a paged decode, all on the host: q [B,Hq,d]; k_pages, v_pages
    [num_pages,Hkv,64,d]; page_table int32 [B,max_blocks]; seq_lens int32 [B];
    s [B,Hkv,max_blocks].  When the pool holds at least B*max_blocks pages each
    block gets its own page (a random permutation, the rest of the pool
    unused); otherwise blocks draw pages at random and share them, as copies of
    a common prefix would.  seq_lens default to random lengths in
    [1, 64*max_blocks]."""
    q = _store(_normal(cfg, TID_Q, (B, Hq, d)), dtype)
    kp = _store(_normal(cfg, TID_K, (num_pages, Hkv, BLOCK, d)), dtype)
    vp = _store(_normal(cfg, TID_V, (num_pages, Hkv, BLOCK, d)), dtype)
    s = _normal(cfg, TID_S, (B, Hkv, max_blocks))
    g = rng(cfg, TID_PAGES)
    if num_pages >= B * max_blocks:
        table = g.permutation(num_pages)[:B * max_blocks].reshape(B, max_blocks)
    else:
        table = g.integers(0, num_pages, size=(B, max_blocks))
    if seq_lens is None:
        seq_lens = rng(cfg, TID_LEN).integers(1, BLOCK * max_blocks + 1, size=B)
    return (q, kp, vp, table.astype(np.int32), np.asarray(seq_lens, dtype=np.int32), s)


def paged_decode_host(w: PagedDecodeWorkload):
    """q [B,Hq,d], page_table int32 [B,max_blocks] (a random permutation of the
    pool), seq_lens int32 [B] (the last block partly filled) and
    s [B,Hkv,max_blocks]; the pages themselves come from paged_pool_device."""
    q = _store(_normal(w.cfg, TID_Q, (w.B, w.Hq, w.d)), w.dtype)
    s = _normal(w.cfg, TID_S, (w.B, w.Hkv, w.max_blocks))
    table = rng(w.cfg, TID_PAGES).permutation(w.num_pages).reshape(w.B, w.max_blocks)
    L = (w.max_blocks - 1) * BLOCK + rng(w.cfg, TID_LEN).integers(1, BLOCK + 1, size=w.B)
    return q, table.astype(np.int32), L.astype(np.int32), s


def paged_pool_device(w: PagedDecodeWorkload, device):
    """k_pages, v_pages [num_pages,Hkv,64,d] drawn on the device with seeded
    torch generators, filled in slices to bound the float32 temporary."""
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = []
    for tid in (TID_K, TID_V):
        g = torch.Generator(device=device)
        g.manual_seed(1_000_003 * w.cfg + tid)
        t = torch.empty((w.num_pages, w.Hkv, BLOCK, w.d), dtype=dt, device=device)
        step = 4096
        for p0 in range(0, w.num_pages, step):
            p1 = min(w.num_pages, p0 + step)
            t[p0:p1].copy_(torch.randn((p1 - p0, w.Hkv, BLOCK, w.d), generator=g, device=device,
                                       dtype=torch.float32))
        out.append(t)
    return out[0], out[1]


def decode_q_and_scores(w: DecodeWorkload):
    q = _store(_normal(w.cfg, TID_Q, (w.B, w.Hq, w.d)), w.dtype)
    s = _normal(w.cfg, TID_S, (w.B, w.Hkv, w.cap // BLOCK))
    return q, s


def decode_cache_device(w: DecodeWorkload, device, torch_dtype=None):
    """The K/V caches ([B,Hkv,cap,d], several GiB at full size) drawn on the
    device with seeded torch generators (numpy on the host would take minutes).
    Readers that need host values copy back only the blocks they use."""
    import torch
    dt = torch_dtype or (torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    out = []
    for tid in (TID_K, TID_V):
        g = torch.Generator(device=device)
        g.manual_seed(1_000_003 * w.cfg + tid)
        t = torch.empty((w.B, w.Hkv, w.cap, w.d), dtype=dt, device=device)
        # fill per batch entry to bound the float32 temporary
        for b in range(w.B):
            t[b].copy_(torch.randn((w.Hkv, w.cap, w.d), generator=g, device=device,
                                   dtype=torch.float32))
        out.append(t)
    return out[0], out[1]
