"""The C-ABI calls under HIP graph capture: the library allocates nothing,
synchronises nothing and records no memset, so a training step (pool,
select, forward, backward) and a decode step can be captured once and
replayed.  Every replay must reproduce the eager results bit for bit (the
kernels use fixed reduction orders), with eager work and synchronisations
between the replays."""
import numpy as np
import pytest
import torch

import sas_inputs as si
from sas_run import dev, host, tdtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_block_sparse_select_amd as m
    return m


def _training_buffers(api, w):
    dt = tdtype(w.dtype)
    q, k, v, do = si.make_qkv(w)
    x = dict(q=dev(q, dt), k=dev(k, dt), v=dev(v, dt), do=dev(do, dt))
    sh = api.make_shape(w.B, w.Hq, w.Hkv, w.n, w.d, w.topk, dt)
    nb = w.nqb
    x["s"] = torch.empty((w.B, w.Hkv, nb, nb), dtype=torch.float32, device="cuda")
    x.update(api.alloc_select(sh))
    x["o"] = torch.empty_like(x["q"])
    x["lse"] = torch.empty((w.B, w.Hq, w.n), dtype=torch.float32, device="cuda")
    for g in ("dq", "dk", "dv"):
        x[g] = torch.empty_like(x[g[1]])
    x["ds"] = torch.empty_like(x["s"])
    x["ws_pool"] = api.alloc_workspace(api.sas_pool_workspace_bytes(sh))
    x["ws_bwd"] = api.alloc_workspace(api.sas_bwd_workspace_bytes(sh))
    return sh, x


def _training_step(api, sh, x):
    api.sas_pool_scores(sh, x["q"], x["k"], x["s"], x["ws_pool"])
    api.sas_select(sh, x["s"], x["idx"], x["cnt"], x["log_gate"], x["s_lse"])
    api.sas_fwd(sh, x["q"], x["k"], x["v"], x["idx"], x["cnt"], x["log_gate"], x["o"], x["lse"])
    api.sas_bwd(sh, x["q"], x["k"], x["v"], x["o"], x["do"], x["lse"], x["idx"], x["cnt"],
                x["log_gate"], x["s"], x["s_lse"], x["dq"], x["dk"], x["dv"], x["ds"], x["ws_bwd"])


OUTS = ("s", "idx", "cnt", "log_gate", "s_lse", "o", "lse", "dq", "dk", "dv", "ds")


def test_training_step_graph_replays(api):
    w = si.custom_workload(140, 1, 8, 2, 2048, 128, 8, "bf16", s_kind="pool")
    sh, x = _training_buffers(api, w)
    _training_step(api, sh, x)
    torch.cuda.synchronize()
    eager = {k: host(x[k]).copy() for k in OUTS}
    for k in OUTS:   # poison the outputs: the replay must rewrite all of them
        x[k].fill_(-7 if x[k].dtype == torch.int32 else float("nan"))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            _training_step(api, sh, x)
    torch.cuda.synchronize()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for k in OUTS:
            assert np.array_equal(host(x[k]), eager[k], equal_nan=True), (rep, k)
        # eager work between the replays: scramble the outputs again
        for k in OUTS:
            x[k].fill_(-7 if x[k].dtype == torch.int32 else 3.0)
        torch.cuda.synchronize()


def test_decode_graph_replays(api):
    w = si.DecodeWorkload(141, 8, 16, 4, 1024, 128, 6, "bf16", hist_blocks=15)
    q, kc, vc, lens, s = si.make_decode_small(w)
    dt = tdtype(w.dtype)
    sh = api.make_decode_shape(w.B, w.Hq, w.Hkv, w.cap, w.d, w.topk, dt)
    qd, kd, vd = dev(q, dt), dev(kc, dt), dev(vc, dt)
    ld, sd = torch.from_numpy(lens).cuda(), torch.from_numpy(s).cuda()
    o = torch.empty_like(qd)
    idx = torch.empty((w.B, w.Hkv, w.topk), dtype=torch.int32, device="cuda")
    ws = api.alloc_workspace(api.sas_decode_workspace_bytes(sh))
    api.sas_decode(sh, qd, kd, vd, ld, sd, o, idx, ws)
    torch.cuda.synchronize()
    eo, ei = host(o).copy(), host(idx).copy()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            api.sas_decode(sh, qd, kd, vd, ld, sd, o, idx, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(float("nan"))
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(o), eo), rep
        assert np.array_equal(host(idx), ei), rep
