"""Python binding of libsas: same names as the C ABI, torch tensors in.

Argument marshalling only: every function checks that tensors are contiguous
device tensors of the expected dtype, builds the shape struct and passes raw
pointers plus the current HIP stream to the library.  All arithmetic happens
in the library's kernels.  Outputs are written into caller-provided tensors;
the ``alloc_*`` helpers only allocate (torch) tensors of the right shapes.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import (BLOCK, GATES, NOALLOC_SCRATCH_BYTES, SAS_BF16, SAS_F32, SasDecodePagedShape, SasDecodeShape, SasError, SasShape, lib,
                   status_string)

_DT = {torch.float32: SAS_F32, torch.bfloat16: SAS_BF16}


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(t, name, dtype=None, numel=None, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _ok(st, where):
    if st != 0:
        raise SasError(st, where)


def _gate(gate) -> int:
    """Gate kind: one of "softmax", "sigmoid", "hard", "external", or its
    SAS_GATE_* code (other integers are passed through for the library to
    reject)."""
    if isinstance(gate, str):
        if gate not in GATES:
            raise ValueError(f"unknown gate {gate!r}; one of {sorted(GATES)}")
        return GATES[gate]
    return int(gate)


def make_shape(B, Hq, Hkv, n, d, topk, dtype=torch.bfloat16, scale=0.0, gate="softmax",
               blocks=None) -> SasShape:
    """Training shape.  blocks: None (blocks of 64 tokens, n % 64 == 0) or a
    device int32 tensor [B, nb, 2] of (first token, length) per block, as
    ``blocks_from_cu_seqlens`` builds for packed documents of any length."""
    if blocks is None:
        return SasShape(B, Hq, Hkv, n, d, topk, float(scale), _DT[dtype], _gate(gate), 0, None)
    _check(blocks, "blocks", torch.int32)
    if blocks.dim() != 3 or blocks.shape[0] != B or blocks.shape[2] != 2:
        raise ValueError("blocks must be [B, nb, 2]")
    sh = SasShape(B, Hq, Hkv, n, d, topk, float(scale), _DT[dtype], _gate(gate),
                  int(blocks.shape[1]), blocks.data_ptr())
    sh._blocks_ref = blocks      # keep the table alive as long as the shape
    return sh


def nblocks(shape: SasShape) -> int:
    """Blocks per batch entry: the table's nb, or n/64 without a table."""
    return int(shape.nb) if shape.blocks else shape.n // BLOCK


def make_decode_shape(B, Hq, Hkv, cap, d, topk, dtype=torch.bfloat16, scale=0.0,
                      gate="softmax") -> SasDecodeShape:
    return SasDecodeShape(B, Hq, Hkv, cap, d, topk, float(scale), _DT[dtype], _gate(gate))


def make_decode_paged_shape(B, Hq, Hkv, max_blocks, num_pages, d, topk, dtype=torch.bfloat16,
                            scale=0.0, gate="softmax") -> SasDecodePagedShape:
    return SasDecodePagedShape(B, Hq, Hkv, max_blocks, num_pages, d, topk, float(scale), _DT[dtype],
                               _gate(gate))


def shape_of(q: torch.Tensor, k: torch.Tensor, topk: int, scale: float = 0.0,
             gate="softmax") -> SasShape:
    B, Hq, n, d = q.shape
    return make_shape(B, Hq, k.shape[1], n, d, topk, q.dtype, scale, gate)


def _dt(shape):
    return torch.float32 if shape.dtype == SAS_F32 else torch.bfloat16


# ------------------------------------------------------------------ entry points
def sas_pool_workspace_bytes(shape: SasShape) -> int:
    return int(lib().sas_pool_workspace_bytes(ctypes.byref(shape)))


def sas_pool_scores(shape: SasShape, q, k, s, ws, stream=None):
    dt = _dt(shape)
    nb = nblocks(shape)
    _check(q, "q", dt, shape.B * shape.Hq * shape.n * shape.d)
    _check(k, "k", dt, shape.B * shape.Hkv * shape.n * shape.d)
    _check(s, "s", torch.float32, shape.B * shape.Hkv * nb * nb)
    _check(ws, "ws", torch.uint8)
    _ok(lib().sas_pool_scores(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(s), _ptr(ws),
                              ws.numel(), _stream(stream)), "sas_pool_scores")


def sas_select(shape: SasShape, s, idx, cnt, log_gate, s_lse, stream=None):
    nb = nblocks(shape)
    rows = shape.B * shape.Hkv * nb
    _check(s, "s", torch.float32, rows * nb)
    _check(idx, "idx", torch.int32, rows * shape.topk)
    _check(cnt, "cnt", torch.int32, rows)
    _check(log_gate, "log_gate", torch.float32, rows * shape.topk)
    _check(s_lse, "s_lse", torch.float32, rows)
    _ok(lib().sas_select(ctypes.byref(shape), _ptr(s), _ptr(idx), _ptr(cnt), _ptr(log_gate),
                         _ptr(s_lse), _stream(stream)), "sas_select")


def sas_mask_documents(shape: SasShape, doc_first, s, stream=None):
    nb = nblocks(shape)
    _check(doc_first, "doc_first", torch.int32, shape.B * nb)
    _check(s, "s", torch.float32, shape.B * shape.Hkv * nb * nb)
    _ok(lib().sas_mask_documents(ctypes.byref(shape), _ptr(doc_first), _ptr(s), _stream(stream)),
        "sas_mask_documents")


def blocks_from_cu_seqlens(cu_seqlens):
    """Block table and doc_first of packed documents of any length (host int32
    tensors [B, nb, 2] and [B, nb]) from per-entry document offsets:
    cu_seqlens[b] is a nondecreasing list starting at 0; document j of entry b
    holds tokens [cu[j], cu[j+1]).  Each document is cut into 64-token blocks
    from its own first token (the library's sas_blocks_from_cu_seqlens);
    entries with fewer blocks are padded with empty blocks."""
    per = []
    for b, offs in enumerate(cu_seqlens):
        cu = (ctypes.c_int32 * len(offs))(*[int(x) for x in offs])
        cap = sum(max(0, (int(y) - int(x) + BLOCK - 1) // BLOCK) for x, y in zip(offs, offs[1:]))
        blk = (ctypes.c_int32 * max(2 * cap, 2))()
        first = (ctypes.c_int32 * max(cap, 1))()
        nb = lib().sas_blocks_from_cu_seqlens(cu, len(offs) - 1, blk, first, cap)
        if nb < 0 or len(offs) < 1:
            raise ValueError(f"cu_seqlens[{b}] must start at 0 and be nondecreasing")
        per.append((list(blk)[:2 * nb], list(first)[:nb], int(offs[-1])))
    NB = max(1, max(len(f) for _, f, _ in per))
    blocks = torch.empty((len(per), NB, 2), dtype=torch.int32)
    doc_first = torch.empty((len(per), NB), dtype=torch.int32)
    for b, (blk, first, end) in enumerate(per):
        nb = len(first)
        blocks[b, :nb] = torch.tensor(blk, dtype=torch.int32).view(nb, 2)
        blocks[b, nb:, 0] = end
        blocks[b, nb:, 1] = 0
        doc_first[b, :nb] = torch.tensor(first, dtype=torch.int32)
        doc_first[b, nb:] = torch.arange(nb, NB, dtype=torch.int32)
    return blocks, doc_first


def doc_first_from_cu_seqlens(cu_seqlens, n: int):
    """doc_first [len(cu_seqlens), n/64] int32 (host) from per-entry document
    token offsets when every document starts on a multiple of 64 (the layout
    without a block table): cu_seqlens[b] is a nondecreasing list starting at 0
    whose entries are multiples of 64 and at most n (the last document runs to
    n).  For documents of any length use ``blocks_from_cu_seqlens``."""
    if n % BLOCK:
        raise ValueError("n must be a multiple of 64")
    nb = n // BLOCK
    out = torch.empty((len(cu_seqlens), nb), dtype=torch.int32)
    for b, offs in enumerate(cu_seqlens):
        offs = [int(x) for x in offs]
        if not offs or offs[0] != 0 or any(x % BLOCK or x > n for x in offs) or \
                any(y < x for x, y in zip(offs, offs[1:])):
            raise ValueError(f"cu_seqlens[{b}] must start at 0, be nondecreasing, "
                             "hold multiples of 64 and stay <= n")
        first = 0
        starts = {x // BLOCK for x in offs}
        for i in range(nb):
            if i in starts:
                first = i
            out[b, i] = first
    return out


def sas_fwd(shape: SasShape, q, k, v, idx, cnt, log_gate, o, lse, stream=None):
    dt = _dt(shape)
    nb = nblocks(shape)
    rows = shape.B * shape.Hkv * nb
    _check(q, "q", dt, shape.B * shape.Hq * shape.n * shape.d)
    _check(k, "k", dt, shape.B * shape.Hkv * shape.n * shape.d)
    _check(v, "v", dt, shape.B * shape.Hkv * shape.n * shape.d)
    _check(idx, "idx", torch.int32, rows * shape.topk)
    _check(cnt, "cnt", torch.int32, rows)
    _check(log_gate, "log_gate", torch.float32, rows * shape.topk)
    _check(o, "o", dt, shape.B * shape.Hq * shape.n * shape.d)
    _check(lse, "lse", torch.float32, shape.B * shape.Hq * shape.n)
    _ok(lib().sas_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(cnt),
                      _ptr(log_gate), _ptr(o), _ptr(lse), _stream(stream)), "sas_fwd")


def sas_bwd_workspace_bytes(shape: SasShape) -> int:
    return int(lib().sas_bwd_workspace_bytes(ctypes.byref(shape)))


def sas_bwd_min_workspace_bytes(shape: SasShape) -> int:
    return int(lib().sas_bwd_min_workspace_bytes(ctypes.byref(shape)))


def sas_bwd(shape: SasShape, q, k, v, o, dO, lse, idx, cnt, log_gate, s, s_lse, dq, dk, dv, ds,
            ws, stream=None):
    dt = _dt(shape)
    nb = nblocks(shape)
    rows = shape.B * shape.Hkv * nb
    nq = shape.B * shape.Hq * shape.n * shape.d
    nk = shape.B * shape.Hkv * shape.n * shape.d
    for t, nm, n_ in ((q, "q", nq), (o, "o", nq), (dO, "dO", nq), (dq, "dq", nq),
                      (k, "k", nk), (v, "v", nk), (dk, "dk", nk), (dv, "dv", nk)):
        _check(t, nm, dt, n_)
    _check(lse, "lse", torch.float32, shape.B * shape.Hq * shape.n)
    _check(idx, "idx", torch.int32, rows * shape.topk)
    _check(cnt, "cnt", torch.int32, rows)
    _check(log_gate, "log_gate", torch.float32, rows * shape.topk)
    _check(s, "s", torch.float32, rows * nb)
    _check(s_lse, "s_lse", torch.float32, rows)
    _check(ds, "ds", torch.float32, rows * nb)
    _check(ws, "ws", torch.uint8)
    _ok(lib().sas_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO),
                      _ptr(lse), _ptr(idx), _ptr(cnt), _ptr(log_gate), _ptr(s), _ptr(s_lse),
                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ds), _ptr(ws), ws.numel(),
                      _stream(stream)), "sas_bwd")


def sas_decode_workspace_bytes(shape: SasDecodeShape) -> int:
    return int(lib().sas_decode_workspace_bytes(ctypes.byref(shape)))


def sas_decode(shape: SasDecodeShape, q, k_cache, v_cache, seq_lens, s, o, idx_out, ws,
               stream=None):
    dt = _dt(shape)
    _check(q, "q", dt, shape.B * shape.Hq * shape.d)
    _check(k_cache, "k_cache", dt, shape.B * shape.Hkv * shape.cap * shape.d)
    _check(v_cache, "v_cache", dt, shape.B * shape.Hkv * shape.cap * shape.d)
    _check(seq_lens, "seq_lens", torch.int32, shape.B)
    _check(s, "s", torch.float32, shape.B * shape.Hkv * (shape.cap // BLOCK))
    _check(o, "o", dt, shape.B * shape.Hq * shape.d)
    _check(idx_out, "idx_out", torch.int32, shape.B * shape.Hkv * shape.topk)
    _check(ws, "ws", torch.uint8)
    _ok(lib().sas_decode(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                         _ptr(seq_lens), _ptr(s), _ptr(o), _ptr(idx_out), _ptr(ws), ws.numel(),
                         _stream(stream)), "sas_decode")


def sas_decode_noalloc(shape: SasDecodeShape, q, k_cache, v_cache, seq_lens, s, o, idx_out,
                       stream=None):
    """sas_decode with its scratch in the library's own per-GPU array (no
    workspace argument, nothing allocated)."""
    dt = _dt(shape)
    _check(q, "q", dt, shape.B * shape.Hq * shape.d)
    _check(k_cache, "k_cache", dt, shape.B * shape.Hkv * shape.cap * shape.d)
    _check(v_cache, "v_cache", dt, shape.B * shape.Hkv * shape.cap * shape.d)
    _check(seq_lens, "seq_lens", torch.int32, shape.B)
    _check(s, "s", torch.float32, shape.B * shape.Hkv * (shape.cap // BLOCK))
    _check(o, "o", dt, shape.B * shape.Hq * shape.d)
    _check(idx_out, "idx_out", torch.int32, shape.B * shape.Hkv * shape.topk)
    _ok(lib().sas_decode_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(seq_lens), _ptr(s), _ptr(o), _ptr(idx_out),
                                 _stream(stream)), "sas_decode_noalloc")


def sas_decode_paged_workspace_bytes(shape: SasDecodePagedShape) -> int:
    return int(lib().sas_decode_paged_workspace_bytes(ctypes.byref(shape)))


def sas_decode_paged(shape: SasDecodePagedShape, q, k_pages, v_pages, page_table, seq_lens, s, o,
                     idx_out, ws, stream=None):
    dt = _dt(shape)
    pool = shape.num_pages * shape.Hkv * BLOCK * shape.d
    _check(q, "q", dt, shape.B * shape.Hq * shape.d)
    _check(k_pages, "k_pages", dt, pool)
    _check(v_pages, "v_pages", dt, pool)
    _check(page_table, "page_table", torch.int32, shape.B * shape.max_blocks)
    _check(seq_lens, "seq_lens", torch.int32, shape.B)
    _check(s, "s", torch.float32, shape.B * shape.Hkv * shape.max_blocks)
    _check(o, "o", dt, shape.B * shape.Hq * shape.d)
    _check(idx_out, "idx_out", torch.int32, shape.B * shape.Hkv * shape.topk)
    _check(ws, "ws", torch.uint8)
    _ok(lib().sas_decode_paged(ctypes.byref(shape), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                               _ptr(page_table), _ptr(seq_lens), _ptr(s), _ptr(o), _ptr(idx_out),
                               _ptr(ws), ws.numel(), _stream(stream)), "sas_decode_paged")


def sas_prof_enable(on: bool):
    _ok(lib().sas_prof_enable(1 if on else 0), "sas_prof_enable")


def sas_prof_collect(max_entries: int = 64):
    """{kernel name: (total ms, launches)} since the last collect."""
    names = (ctypes.c_char_p * max_entries)()
    ms = (ctypes.c_double * max_entries)()
    nl = (ctypes.c_int32 * max_entries)()
    n = lib().sas_prof_collect(names, ms, nl, max_entries)
    return {names[j].decode(): (ms[j], nl[j]) for j in range(min(n, max_entries))}


# ------------------------------------------------------------------ allocation helpers
def alloc_select(shape: SasShape, device="cuda"):
    nb = nblocks(shape)
    lead = (shape.B, shape.Hkv, nb)
    return dict(idx=torch.empty(lead + (shape.topk,), dtype=torch.int32, device=device),
                cnt=torch.empty(lead, dtype=torch.int32, device=device),
                log_gate=torch.empty(lead + (shape.topk,), dtype=torch.float32, device=device),
                s_lse=torch.empty(lead, dtype=torch.float32, device=device))


def alloc_workspace(nbytes: int, device="cuda"):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


__all__ = [
    "make_shape", "make_decode_shape", "make_decode_paged_shape", "shape_of",
    "sas_pool_workspace_bytes", "sas_pool_scores", "sas_select", "sas_mask_documents",
    "doc_first_from_cu_seqlens", "blocks_from_cu_seqlens", "nblocks", "sas_fwd",
    "sas_bwd_workspace_bytes", "sas_bwd_min_workspace_bytes", "sas_bwd", "sas_decode_workspace_bytes", "sas_decode",
    "sas_decode_noalloc", "sas_decode_paged_workspace_bytes", "sas_decode_paged", "sas_prof_enable", "sas_prof_collect",
    "alloc_select", "alloc_workspace", "status_string", "SasError", "SasShape", "SasDecodeShape",
    "SasDecodePagedShape", "NOALLOC_SCRATCH_BYTES",
]
