"""sas_decode_noalloc (scratch in the library's per-GPU array, no workspace
argument) against sas_decode with a caller workspace, through the C ABI: two
calls in a row, the second with a smaller input, both split over several
workgroups per row so that the partial results go through the scratch array.
The kernels are the same, so the outputs must agree bit for bit; the oracle
checks the first call as well."""
import numpy as np
import pytest
import torch

import oracle
import sas_inputs as si
from parity_bars import assert_o
from sas_run import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_block_sparse_select_amd as m
    return m


def _inputs(w):
    q, kc, vc, lens, s = si.make_decode_small(w)
    dt = torch.bfloat16
    return (dev(q, dt), dev(kc, dt), dev(vc, dt), torch.from_numpy(lens).cuda(),
            torch.from_numpy(s).cuda()), (q, kc, vc, lens, s)


def _with_ws(api, sh, x):
    q = x[0]
    o = torch.empty_like(q)
    idx = torch.empty((sh.B, sh.Hkv, sh.topk), dtype=torch.int32, device="cuda")
    ws = api.alloc_workspace(api.sas_decode_workspace_bytes(sh))
    api.sas_decode(sh, *x, o, idx, ws)
    return o, idx


def _noalloc(api, sh, x, stream=None):
    q = x[0]
    o = torch.full_like(q, float("nan"))
    idx = torch.full((sh.B, sh.Hkv, sh.topk), -7, dtype=torch.int32, device="cuda")
    api.sas_decode_noalloc(sh, *x, o, idx, stream=stream)
    return o, idx


def test_noalloc_decode_matches_workspace_decode(api):
    big = si.DecodeWorkload(610, 4, 8, 2, 2048, 128, 8, "bf16", hist_blocks=31)
    small = si.DecodeWorkload(611, 2, 8, 2, 1024, 128, 5, "bf16", hist_blocks=15)
    runs = []
    side = torch.cuda.Stream()
    for w, stream in ((big, None), (small, side)):
        sh = api.make_decode_shape(w.B, w.Hq, w.Hkv, w.cap, w.d, w.topk, torch.bfloat16)
        need = api.sas_decode_workspace_bytes(sh)
        assert need > 4096      # split rows: the partial results use the scratch
        assert need <= api.NOALLOC_SCRATCH_BYTES
        x, xh = _inputs(w)
        with torch.cuda.stream(side if stream is not None else torch.cuda.current_stream()):
            o_na, idx_na = _noalloc(api, sh, x, stream)
        torch.cuda.synchronize()
        o_ws, idx_ws = _with_ws(api, sh, x)
        torch.cuda.synchronize()
        assert torch.equal(idx_na, idx_ws)
        assert torch.equal(o_na, o_ws)
        runs.append((w, xh, o_na, idx_na))
    w, (q, kc, vc, lens, s), o_na, idx_na = runs[0]
    ref_o, ref_idx = oracle.decode(q, kc, vc, lens, s, w.topk)
    assert np.array_equal(host(idx_na), ref_idx)
    assert_o(host(o_na), ref_o, "bf16")
