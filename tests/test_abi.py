"""C-ABI checks that need no GPU: every symbol declared in include/sas.h is
exported by libsas.so, and invalid arguments are rejected on the host before
any launch (these calls touch no device)."""
import ctypes
import os
import re

import pytest
import torch

from gated_block_sparse_select_amd import _lib, api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "sas.h")) as f:
        txt = f.read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(sas_[a-z_0-9]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("sas_pool_scores", "sas_select", "sas_fwd", "sas_bwd", "sas_decode",
                 "sas_bwd_workspace_bytes", "sas_status_string"):
        assert must in names


def test_every_declared_symbol_is_exported():
    L = _lib.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(_lib.EXPORTED) <= set(declared_functions())


def test_abi_version_and_status_strings():
    L = _lib.lib()
    assert L.sas_abi_version() == _lib.ABI_VERSION == 4
    for st in range(6):
        assert _lib.status_string(st).startswith("SAS")
    assert "unknown" in _lib.status_string(99)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def _sel(sh, s=FAKE, idx=FAKE, cnt=FAKE, lg=FAKE, lse=FAKE):
    return _lib.lib().sas_select(ctypes.byref(sh), s, idx, cnt, lg, lse, None)


@pytest.mark.parametrize("B,Hq,Hkv,n,d,K,scale,dt,expect", [
    (1, 4, 2, 500, 128, 2, 0.0, 1, 1),      # n % 64 != 0
    (1, 4, 3, 512, 128, 2, 0.0, 1, 1),      # Hq % Hkv != 0
    (1, 4, 2, 512, 96, 2, 0.0, 1, 1),       # d not in {64,128}
    (1, 4, 2, 512, 128, -1, 0.0, 1, 1),     # K < 0
    (1, 4, 2, 512, 128, 2049, 0.0, 1, 1),   # K beyond the supported block count
    (0, 4, 2, 512, 128, 2, 0.0, 1, 1),      # B < 1
    (1, 34, 2, 512, 128, 2, 0.0, 1, 1),     # G > 16
    (1, 4, 2, 512, 128, 2, -1.0, 1, 1),     # negative scale
    (1, 4, 2, 512, 128, 2, float("nan"), 1, 1),
    (1, 4, 2, 64 * 2049, 128, 2, 0.0, 1, 1),  # more blocks than supported
    (1, 4, 2, 512, 128, 2, 0.0, 7, 2),      # bad dtype
    (1, 4, 2, 0, 128, 2, 0.0, 1, 1),        # empty sequence
])
def test_shape_validation(B, Hq, Hkv, n, d, K, scale, dt, expect):
    sh = _lib.SasShape(B, Hq, Hkv, n, d, K, scale, dt, 0)
    assert _sel(sh) == expect
    L = _lib.lib()
    assert L.sas_fwd(ctypes.byref(sh), *([FAKE] * 8), None) == expect
    assert L.sas_bwd_workspace_bytes(ctypes.byref(sh)) == 0


def test_null_pointers_rejected():
    L = _lib.lib()
    sh = api.make_shape(1, 4, 2, 512, 128, 2)
    assert _sel(sh, s=None) == 1
    assert _sel(sh, idx=None) == 1
    assert L.sas_fwd(ctypes.byref(sh), None, *([FAKE] * 7), None) == 1
    assert L.sas_bwd(ctypes.byref(sh), *([FAKE] * 14), None, FAKE, 1 << 40, None) == 1
    assert L.sas_select(None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.sas_mask_documents(ctypes.byref(sh), None, FAKE, None) == 1
    assert L.sas_mask_documents(ctypes.byref(sh), FAKE, None, None) == 1
    assert L.sas_mask_documents(None, FAKE, FAKE, None) == 1
    bad = api.make_shape(1, 4, 2, 500, 128, 2)     # n not a multiple of 64
    assert L.sas_mask_documents(ctypes.byref(bad), FAKE, FAKE, None) == 1
    # topk == 0 allows NULL idx / log_gate
    sh0 = api.make_shape(1, 4, 2, 512, 128, 0)
    assert L.sas_pool_scores(ctypes.byref(sh0), FAKE, FAKE, FAKE, None, 0, None) == 4


def test_workspace_checks():
    L = _lib.lib()
    sh = api.make_shape(1, 32, 8, 32768, 128, 32)
    need = api.sas_bwd_min_workspace_bytes(sh)
    assert need > 4 * 32 * 32768      # holds at least the row statistics
    args = [FAKE] * 15
    assert L.sas_bwd(ctypes.byref(sh), *args, FAKE, need - 1, None) == 4
    assert L.sas_bwd(ctypes.byref(sh), *args, None, need, None) == 4
    # the dZ-tile path adds one 64 x 64 bf16 tile per (head, q-block, kept or own block)
    dz = 1 * 32 * 512 * 33 * 64 * 64 * 2
    assert api.sas_bwd_workspace_bytes(sh) - need == (dz + 255) // 256 * 256
    # no dZ tiles for the external gate, the float32 path, or tiles beyond 16 GiB
    for other in (api.make_shape(1, 32, 8, 32768, 128, 32, gate="external"),
                  api.make_shape(1, 32, 8, 32768, 128, 32, torch.float32),
                  api.make_shape(1, 32, 8, 32768, 128, 512)):
        assert api.sas_bwd_workspace_bytes(other) == api.sas_bwd_min_workspace_bytes(other) > 0
    pneed = api.sas_pool_workspace_bytes(sh)
    assert L.sas_pool_scores(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, pneed - 1, None) == 4
    dsh = api.make_decode_shape(64, 32, 8, 32768, 128, 32)
    dneed = api.sas_decode_workspace_bytes(dsh)
    assert dneed > 0
    assert L.sas_decode(ctypes.byref(dsh), *([FAKE] * 7), FAKE, dneed - 1, None) == 4
    bad = api.make_decode_shape(64, 32, 8, 1000, 128, 32)
    assert api.sas_decode_workspace_bytes(bad) == 0
    assert L.sas_decode(ctypes.byref(bad), *([FAKE] * 7), FAKE, 1 << 30, None) == 1
    # the allocation-free decode checks its arguments before touching a device
    assert L.sas_decode_noalloc(ctypes.byref(bad), *([FAKE] * 7), None) == 1
    assert L.sas_decode_noalloc(ctypes.byref(dsh), *([None] * 7), None) == 1
    assert L.sas_decode_noalloc(None, *([FAKE] * 7), None) == 1


@pytest.mark.parametrize("B,Hq,Hkv,maxb,pages,d,K,dt,expect", [
    (2, 8, 2, 8192, 100, 128, 32, 1, 0),     # 512K-token rows: accepted
    (2, 8, 2, 8193, 100, 128, 32, 1, 1),     # more blocks than SAS_MAX_DECODE_BLOCKS
    (2, 8, 2, 0, 100, 128, 32, 1, 1),        # no blocks
    (2, 8, 2, 64, 0, 128, 32, 1, 1),         # empty pool
    (2, 8, 2, 64, 100, 96, 32, 1, 1),        # d not in {64,128}
    (2, 8, 3, 64, 100, 128, 32, 1, 1),       # Hq % Hkv != 0
    (2, 8, 2, 64, 100, 128, 2049, 1, 1),     # topk beyond SAS_MAX_BLOCKS
    (2, 8, 2, 64, 100, 128, 32, 5, 2),       # bad dtype
])
def test_paged_decode_shape_validation(B, Hq, Hkv, maxb, pages, d, K, dt, expect):
    L = _lib.lib()
    sh = _lib.SasDecodePagedShape(B, Hq, Hkv, maxb, pages, d, K, 0.0, dt, 0)
    need = L.sas_decode_paged_workspace_bytes(ctypes.byref(sh))
    assert (need > 0) == (expect == 0)
    if expect:   # every pointer non-NULL and the workspace large: only the shape decides
        assert L.sas_decode_paged(ctypes.byref(sh), *([FAKE] * 8), FAKE, 1 << 40, None) == expect


def test_paged_decode_pointer_and_workspace_checks():
    L = _lib.lib()
    sh = api.make_decode_paged_shape(4, 32, 8, 8192, 1 << 16, 128, 32)
    need = api.sas_decode_paged_workspace_bytes(sh)
    assert need > 0
    ptrs = [FAKE] * 8
    for j in range(7):   # q, k_pages, v_pages, page_table, seq_lens, s, o are required
        bad = list(ptrs)
        bad[j] = None
        assert L.sas_decode_paged(ctypes.byref(sh), *bad, FAKE, need, None) == 1
    assert L.sas_decode_paged(ctypes.byref(sh), *ptrs, FAKE, need - 1, None) == 4
    assert L.sas_decode_paged(ctypes.byref(sh), *ptrs, None, need, None) == 4


def test_binding_rejects_host_tensors():
    import torch
    sh = api.make_shape(1, 1, 1, 64, 64, 0, torch.float32)
    t = torch.zeros(64 * 64)
    with pytest.raises(ValueError):
        api.sas_fwd(sh, t, t, t, None, torch.zeros(1, dtype=torch.int32), None, t,
                    torch.zeros(64))


def test_doc_first_from_cu_seqlens():
    df = api.doc_first_from_cu_seqlens([[0, 192, 256], [0], [0, 64, 64, 512]], 512)
    assert df.tolist() == [[0, 0, 0, 3, 4, 4, 4, 4], [0] * 8, [0, 1, 1, 1, 1, 1, 1, 1]]
    for bad in ([[64, 128]], [[0, 100]], [[0, 256, 128]], [[0, 576]]):
        with pytest.raises(ValueError):
            api.doc_first_from_cu_seqlens(bad, 512)


@pytest.mark.parametrize("gate,expect", [(0, 0), (1, 0), (2, 0), (3, 0), (4, 1), (-1, 1)])
def test_gate_kind_validation(gate, expect):
    """Every entry point accepts the four gate kinds and rejects others."""
    L = _lib.lib()
    sh = _lib.SasShape(1, 4, 2, 512, 128, 2, 0.0, 1, gate)
    assert (L.sas_bwd_workspace_bytes(ctypes.byref(sh)) > 0) == (expect == 0)
    if expect:
        assert _sel(sh) == expect
        assert L.sas_fwd(ctypes.byref(sh), *([FAKE] * 8), None) == expect
        dsh = _lib.SasDecodeShape(4, 8, 2, 1024, 128, 2, 0.0, 1, gate)
        assert L.sas_decode_workspace_bytes(ctypes.byref(dsh)) == 0
        psh = _lib.SasDecodePagedShape(4, 8, 2, 64, 100, 128, 2, 0.0, 1, gate)
        assert L.sas_decode_paged_workspace_bytes(ctypes.byref(psh)) == 0
    assert api.make_shape(1, 4, 2, 512, 128, 2, gate="external").gate == 3
    with pytest.raises(ValueError):
        api.make_shape(1, 4, 2, 512, 128, 2, gate="tanh")


def test_blocks_from_cu_seqlens_matches_the_oracle_cut():
    """The library's document cut (sas_blocks_from_cu_seqlens through the
    binding) equals the oracle's, padding included; bad offsets are refused."""
    import numpy as np
    import oracle
    lens = [[100, 64, 1, 130], [5], [64, 64, 63]]
    cus = [[0] + list(np.cumsum(x)) for x in lens]
    blocks, first = api.blocks_from_cu_seqlens(cus)
    geom, ofirst = oracle.packed_geometry(lens)
    assert np.array_equal(blocks.numpy(), geom) and np.array_equal(first.numpy(), ofirst)
    with pytest.raises(ValueError):
        api.blocks_from_cu_seqlens([[1, 5]])
    with pytest.raises(ValueError):
        api.blocks_from_cu_seqlens([[0, 70, 60]])


def test_block_table_shape_validation():
    """A block table frees n from multiples of 64; nb must fit the table rules."""
    L = _lib.lib()
    fake = FAKE
    sh = api.make_shape(1, 8, 2, 512, 128, 4)
    sh.n, sh.nb, sh.blocks = 700, 12, fake.value
    assert api.sas_bwd_workspace_bytes(sh) > 0
    assert api.sas_pool_workspace_bytes(sh) == 2 * 4 * 2 * 12 * 128
    for nb, n in ((0, 700), (2049, 700), (12, 63), (12, 64 * 2048 + 1)):
        sh.nb, sh.n = nb, n
        assert api.sas_bwd_workspace_bytes(sh) == 0, (nb, n)
    sh.blocks, sh.nb, sh.n = None, 3, 512     # without a table nb is 0 or n/64
    assert api.sas_bwd_workspace_bytes(sh) == 0
    sh.nb = 8
    assert api.sas_bwd_workspace_bytes(sh) > 0
    assert L.sas_select(ctypes.byref(sh), None, None, None, None, None, None) == 1
