"""Helpers for the GPU tests: move seeded inputs to the device, run the C-ABI
path through the binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

from parity_bars import rel_l2  # noqa: F401  (re-exported for the tests)

BLOCK = 64


def dev(x: np.ndarray, dtype) -> torch.Tensor:
    """float32 host array (values representable in dtype) -> device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(dtype)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype != torch.int32 else t.cpu().numpy()


def tdtype(w_dtype: str):
    return torch.float32 if w_dtype == "f32" else torch.bfloat16


def run_layer(api, q, k, v, do, s, topk, dtype, scale=0.0, pool=False, bwd=True, doc_first=None,
              gate="softmax", blocks=None, min_ws=False):
    """Run (pool) -> (mask documents) -> select -> fwd (-> bwd) on device
    tensors; returns a dict of device tensors.  q,k,v,do are device tensors; s
    is a device float32 tensor (masked in place when doc_first, a device int32
    [B, nb] tensor, is given) or None when pool=True.  blocks: None or the
    device block table [B, nb, 2] of packed documents of any length.  min_ws:
    give the backward only sas_bwd_min_workspace_bytes, so that dq recomputes
    the logits instead of reading the stored dZ tiles."""
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    sh = api.make_shape(B, Hq, Hkv, n, d, topk, dtype, scale, gate, blocks=blocks)
    nb = api.nblocks(sh)
    out = {}
    if pool:
        s = torch.empty((B, Hkv, nb, nb), dtype=torch.float32, device="cuda")
        ws = api.alloc_workspace(api.sas_pool_workspace_bytes(sh))
        api.sas_pool_scores(sh, q, k, s, ws)
    if doc_first is not None:
        api.sas_mask_documents(sh, doc_first, s)
    out["s"] = s
    sel = api.alloc_select(sh)
    api.sas_select(sh, s, sel["idx"], sel["cnt"], sel["log_gate"], sel["s_lse"])
    out.update(sel)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, n), dtype=torch.float32, device="cuda")
    api.sas_fwd(sh, q, k, v, sel["idx"], sel["cnt"], sel["log_gate"], o, lse)
    out["o"], out["lse"] = o, lse
    if bwd:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ds = torch.empty_like(s)
        ws = api.alloc_workspace(api.sas_bwd_min_workspace_bytes(sh) if min_ws
                                 else api.sas_bwd_workspace_bytes(sh))
        api.sas_bwd(sh, q, k, v, o, do, lse, sel["idx"], sel["cnt"], sel["log_gate"], s,
                    sel["s_lse"], dq, dk, dv, ds, ws)
        out.update(dq=dq, dk=dk, dv=dv, ds=ds)
    torch.cuda.synchronize()
    return out
