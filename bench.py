"""Benchmark of the SAS gated block-sparse attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--no-decode]

A step is one pass of the training-layer hot path over one synthetic batch:
block-score pooling (when the workload scores by pooling) -> LSE/Top-K select
-> gated block-sparse forward -> backward (dq, dk, dv and ds).  Inputs are
resident in HBM before the timed region; W untimed steps, then K timed steps
between two device synchronisations.  Prints ONE JSON line.

value = effective TFLOP/s: FLOPs counted on valid (query, key) pairs only
(64*64 per kept block plus 64*65/2 for the causal current block, per query
head), 4*d per pair for the forward and 10*d for the backward.

Unless --no-decode is given the line also carries "decode" (batch 64, 32K
contiguous cache: us per call, GB/s, the decode kernel's roofline) and
"decode_paged" (one 512K-token sequence in a paged pool: us per call, GB/s).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores, TFLOP/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", type=int, default=3, choices=[2, 3, 4])
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-full-range", action="store_true", help="skip the full-range (K = n/64) line")
    p.add_argument("--no-gates", action="store_true", help="skip the ablation-gate lines")
    p.add_argument("--no-packed", action="store_true", help="skip the packed-documents line")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    p.add_argument("--no-configs", action="store_true", help="skip the Qwen3-4B / 14B layer lines")
    p.add_argument("--no-recompute", action="store_true",
                   help="skip the headline step on the backward's recompute path")
    p.add_argument("--decode-steps", type=int, default=50)
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run one 1 GiB device copy (reference for HBM byte counters)")
    return p.parse_args()


def pair_count(cnt_np, G, lens=None):
    """Valid (query, key) pairs summed over query heads: 64 rows x 64 keys per
    kept block and the causal 64*65/2 of the current block; with a block table
    (lens [B, nb] tokens per block) L rows x 64 keys per kept block and
    L(L+1)/2 for a current block of L tokens."""
    import numpy as np
    c = cnt_np.astype(np.int64)
    if lens is None:
        return G * (int(c.sum()) * 64 * 64 + c.size * (64 * 65 // 2))
    L = np.asarray(lens, dtype=np.int64)[:, None, :]
    return G * int(np.sum(c * L * 64 + L * (L + 1) // 2))


def timed(torch, step, steps):
    """ms per step of `steps` calls between two synchronisations (no
    per-launch events in the library), and the host wall time."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps, time.perf_counter() - t0


def kernel_pass(api, torch, step, steps):
    """A second pass of the same calls with the library's per-launch HIP
    events (recorded on the launch stream): {kernel: avg ms, launches} and
    that pass's ms per step."""
    torch.cuda.synchronize()
    api.sas_prof_collect()          # drop anything recorded before
    api.sas_prof_enable(True)
    ms, _ = timed(torch, step, steps)
    api.sas_prof_enable(False)
    kern = api.sas_prof_collect()
    per = {name: dict(avg_ms=tot / max(nl, 1), launches=nl) for name, (tot, nl) in kern.items()}
    return per, ms


def run_training(args, api, si, torch, np, w=None, steps=None, warmup=None, gate="softmax",
                 min_ws=False):
    w = si.WORKLOADS[args.workload] if w is None else w
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    dt = torch.bfloat16
    q, k, v, do = si.make_qkv(w)
    dev = lambda x: torch.from_numpy(x).to("cuda").to(dt)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    host = dict(q=q, k=k, v=v, do=do)
    del q, k, v, do
    blocks = lens = None
    if w.varlen:   # packed documents of any length: the block table
        blocks_h, df_h = api.blocks_from_cu_seqlens(
            [si.cu_seqlens_of(si.doc_token_lens(w, b)) for b in range(w.B)])
        blocks, lens = blocks_h.cuda(), blocks_h[..., 1].numpy()
    sh = api.make_shape(w.B, w.Hq, w.Hkv, w.n, w.d, w.topk, dt, gate=gate, blocks=blocks)
    nb = api.nblocks(sh)
    pool = w.s_kind == "pool"
    s = torch.empty((w.B, w.Hkv, nb, nb), dtype=torch.float32, device="cuda")
    if not pool:
        s.copy_(torch.from_numpy(si.make_scores(w)))
    sel = api.alloc_select(sh)
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.n), dtype=torch.float32, device="cuda")
    dq, dk, dv, ds = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd), torch.empty_like(s)
    ws_pool = api.alloc_workspace(api.sas_pool_workspace_bytes(sh))
    # min_ws: only the smallest workspace the backward accepts, so that dq
    # recomputes the logits instead of reading the stored dZ tiles
    ws_bwd = api.alloc_workspace(api.sas_bwd_min_workspace_bytes(sh) if min_ws
                                 else api.sas_bwd_workspace_bytes(sh))
    df = si.make_doc_first(w)
    doc_first = torch.from_numpy(df).cuda() if df is not None else None
    if w.varlen:
        doc_first = df_h.cuda()

    def step():
        if pool:
            api.sas_pool_scores(sh, qd, kd, s, ws_pool)
        if doc_first is not None:   # packed documents: mask the other documents' blocks
            api.sas_mask_documents(sh, doc_first, s)
        api.sas_select(sh, s, sel["idx"], sel["cnt"], sel["log_gate"], sel["s_lse"])
        api.sas_fwd(sh, qd, kd, vd, sel["idx"], sel["cnt"], sel["log_gate"], o, lse)
        api.sas_bwd(sh, qd, kd, vd, o, dod, lse, sel["idx"], sel["cnt"], sel["log_gate"], s,
                    sel["s_lse"], dq, dk, dv, ds, ws_bwd)

    for _ in range(warmup):
        step()
    ms_step, wall = timed(torch, step, steps)
    per_kernel, ms_prof = kernel_pass(api, torch, step, steps)

    cnt = sel["cnt"].cpu().numpy()
    G = w.Hq // w.Hkv
    pairs = pair_count(cnt, G, lens)
    flop_fwd = 4 * w.d * pairs
    flop_bwd = 10 * w.d * pairs
    return dict(w=w, ms_step=ms_step, ms_prof=ms_prof, wall=wall, pairs=pairs, flop_fwd=flop_fwd,
                flop_bwd=flop_bwd, per_kernel=per_kernel, host=host, s=s, sel=sel, steps=steps)


def hbm_kernels(res):
    """HBM rate of the memory-bound kernels of the step: algorithmic bytes
    (each input byte read once, each output byte written once) over the
    kernel's average time.
      pooling:   q and k read (bf16), the block means written and read back
                 (float32), the score matrix written (float32);
      selection: the scores of the history (m < i) read, idx and log_gate
                 (K per row), cnt and s_lse written;
      statistics with the reverse lists (backward, one launch): o and dO read
                 (bf16), lse read, the row statistics [-lse/tau | -D] written
                 (float32, 128 per block); the lists' idx/cnt reads and
                 entries are under 1% of it and not counted;
      dq from the dZ tiles: every dZ tile (8 KB per head, q-block and kept or
                 own block) read, K read, dq written."""
    w = res["w"]
    pk = res["per_kernel"]
    nb = w.nqb
    rows = w.B * w.Hkv * nb
    means = 2 * rows * w.d * 4
    out = {}
    if "sas_pool_means_kernel" in pk and "sas_pool_dot_kernel" in pk:
        qk = (w.B * w.Hq + w.B * w.Hkv) * w.n * w.d * 2
        byt = qk + means + means + rows * nb * 4
        ms = pk["sas_pool_means_kernel"]["avg_ms"] + pk["sas_pool_dot_kernel"]["avg_ms"]
        out["pool"] = dict(bytes=byt, ms=round(ms, 4), GBs=round(byt / (ms * 1e-3) / 1e9, 1),
                           frac=round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    if "sas_select_kernel" in pk:
        hist = w.B * w.Hkv * (nb * (nb - 1) // 2) * 4
        byt = hist + rows * w.topk * 8 + rows * 8
        ms = pk["sas_select_kernel"]["avg_ms"]
        out["select"] = dict(bytes=byt, ms=round(ms, 4), GBs=round(byt / (ms * 1e-3) / 1e9, 1),
                             frac=round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    qsize = w.B * w.Hq * w.n * w.d * 2
    if "sas_revidx_stats_kernel" in pk:
        byt = 2 * qsize + w.B * w.Hq * w.n * 4 + w.B * w.Hq * nb * 128 * 4
        ms = pk["sas_revidx_stats_kernel"]["avg_ms"]
        out["bwd_stats"] = dict(bytes=byt, ms=round(ms, 4), GBs=round(byt / (ms * 1e-3) / 1e9, 1),
                                frac=round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    if "sas_bwd_dqz_kernel" in pk:
        tiles = int((res["sel"]["cnt"].long() + 1).sum().item()) * (w.Hq // w.Hkv)
        byt = tiles * 8192 + w.B * w.Hkv * w.n * w.d * 2 + qsize
        ms = pk["sas_bwd_dqz_kernel"]["avg_ms"]
        out["bwd_dqz"] = dict(bytes=byt, ms=round(ms, 4), GBs=round(byt / (ms * 1e-3) / 1e9, 1),
                              frac=round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    return out


def run_recompute_path(args, api, si, torch, np):
    """The headline step with the backward's minimum workspace (the recompute
    path: dq forms S and dP again, no dZ tiles), timed like the gate lines, so
    the two backward paths are compared on the same box."""
    res = run_training(args, api, si, torch, np, steps=max(1, args.steps // 2), warmup=1,
                       min_ws=True)
    total = res["flop_fwd"] + res["flop_bwd"]
    out = {"ms_per_step": round(res["ms_step"], 4),
           "TFLOPs": round(total / (res["ms_step"] * 1e-3) / 1e12, 1),
           "per_kernel_ms": {k: round(v["avg_ms"], 4) for k, v in res["per_kernel"].items()}}
    res.clear()
    torch.cuda.empty_cache()
    return out


def run_gate_variants(args, api, si, torch, np):
    """The same 32K step with each ablation gate (same selection, same
    effective work): ms per step and per-kernel times."""
    out = {}
    for gate in ("sigmoid", "hard", "external"):
        res = run_training(args, api, si, torch, np, steps=max(1, args.steps // 4), warmup=1,
                           gate=gate)
        total = res["flop_fwd"] + res["flop_bwd"]
        out[gate] = {"ms_per_step": round(res["ms_step"], 3),
                     "TFLOPs": round(total / (res["ms_step"] * 1e-3) / 1e12, 1),
                     "per_kernel_ms": {k: round(v["avg_ms"], 3) for k, v in res["per_kernel"].items()
                                       if k in ("sas_fwd_mfma_kernel", "sas_bwd_dq_kernel",
                                                "sas_bwd_dqz_kernel", "sas_bwd_dkdv_kernel")}}
        res.clear()
        torch.cuda.empty_cache()
    return out


def run_packed(args, api, si, torch, np):
    """The 32K layer holding packed documents of any token length (workload 7):
    each document cut into 64-token blocks from its own first token through the
    block table; document mask + select + fwd + bwd.  Rows near a document's
    start keep fewer blocks, and the effective work counts only the pairs
    kept."""
    w = si.WORKLOADS[7]
    res = run_training(args, api, si, torch, np, w=w, steps=max(1, args.steps // 4), warmup=1)
    total = res["flop_fwd"] + res["flop_bwd"]
    tf = total / (res["ms_step"] * 1e-3) / 1e12
    lens = [si.doc_token_lens(w, b) for b in range(w.B)]
    docs = [len(x) for x in lens]
    out = {"workload": w.name, "documents": docs, "document_tokens": lens,
           "blocks": w.nqb, "steps": res["steps"],
           "ms_per_step": round(res["ms_step"], 3), "TFLOPs": round(tf, 1),
           "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4), "pairs": res["pairs"],
           "per_kernel_ms": {k: round(v["avg_ms"], 3) for k, v in res["per_kernel"].items()}}
    res.clear()
    return out


def run_configs(args, api, si, torch, np):
    """The other training-layer workloads (Qwen3-4B at 8K with
    K = 16, Qwen3-14B at 32K with K = 64 and Gumbel scores): select + fwd +
    bwd, ms per step, effective TFLOP/s and per-kernel times."""
    out = {}
    for cfg in (2, 4):
        if cfg == args.workload:
            continue
        w = si.WORKLOADS[cfg]
        res = run_training(args, api, si, torch, np, w=w, steps=max(2, args.steps // 2), warmup=2)
        total = res["flop_fwd"] + res["flop_bwd"]
        tf = total / (res["ms_step"] * 1e-3) / 1e12
        out[w.name] = {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.d, "n": w.n,
                       "topk": w.topk, "scores": w.s_kind, "steps": res["steps"],
                       "ms_per_step": round(res["ms_step"], 4), "TFLOPs": round(tf, 1),
                       "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                       "effective_flop": total, "roofline": roofline_for(res),
                       "per_kernel_ms": {k: round(v["avg_ms"], 4)
                                         for k, v in res["per_kernel"].items()}}
        res.clear()
        torch.cuda.empty_cache()
    return out


def run_full_range(args, api, si, torch, np):
    """Full-range gated attention (every history block kept with its gate) on
    the 32K layer: the same kernels with K = n/64."""
    w = si.WORKLOADS[8]
    res = run_training(args, api, si, torch, np, w=w, steps=max(1, args.steps // 4), warmup=1)
    total = res["flop_fwd"] + res["flop_bwd"]
    tf = total / (res["ms_step"] * 1e-3) / 1e12
    out = {"workload": w.name, "topk": w.topk, "steps": res["steps"],
           "ms_per_step": round(res["ms_step"], 3), "TFLOPs": round(tf, 1),
           "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
           "per_kernel_ms": {k: round(v["avg_ms"], 3) for k, v in res["per_kernel"].items()}}
    res.clear()
    return out


# Translation units of the kernels whose HBM traffic the committed counter
# summary records; the summary is used only while these sources hash to the
# value recorded with the counters.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_qwen3-8b-n32768-K32_and_decode.md")
KERNEL_SOURCES = {
    "sas_bwd_dkdv_kernel": ["mfma_bwd.hip", "mfma_common.h", "common.h", "launch.h"],
    "sas_bwd_dq_kernel": ["mfma_bwd.hip", "mfma_common.h", "common.h", "launch.h"],
    "sas_bwd_dqz_kernel": ["mfma_bwd.hip", "mfma_common.h", "common.h", "launch.h"],
    "sas_revidx_stats_kernel": ["revidx.hip", "bwd_stats.h", "common.h", "launch.h"],
    "sas_fwd_mfma_kernel": ["mfma_fwd.hip", "mfma_common.h", "common.h", "launch.h"],
    "sas_decode_kernel": ["decode.hip", "decode_kernel.h", "select_row.h", "common.h", "launch.h"],
    "sas_decode_paged_kernel": ["decode_paged.hip", "decode_kernel.h", "select_row.h", "common.h",
                                "launch.h"],
    "sas_pool_means_kernel": ["pool.hip", "common.h", "launch.h"],
    "sas_select_kernel": ["select.hip", "select_row.h", "common.h", "launch.h"],
}


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` (rocprofv3 FETCH_SIZE / WRITE_SIZE,
    scaled by a copy of known size) from the committed summary, or None when
    there is none or the kernel's sources changed since it was taken."""
    import hashlib
    import re
    if kernel not in KERNEL_SOURCES or not os.path.exists(TRAFFIC_FILE):
        return None
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_block_sparse_select_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            m = re.match(r"traffic (\S+) bytes_per_launch=(\d+) source_sha256=(\w+)", line.strip())
            if m and m.group(1) == kernel:
                return int(m.group(2)) if m.group(3) == h.hexdigest() else None
    return None


def roofline_for(res):
    """Dominant kernel by time; its algorithmic FLOPs per launch are the
    contractions it performs on valid pairs: forward 2 (4d per pair), dq pass
    recomputing the logits 3 (S, dP, dQ: 6d), dq from the stored dZ tiles 1
    (dQ: 2d), dk/dv pass 4 (S, dP, dV, dK: 8d)."""
    w = res["w"]
    per = {"sas_fwd_mfma_kernel": 4, "sas_bwd_dq_kernel": 6, "sas_bwd_dqz_kernel": 2,
           "sas_bwd_dkdv_kernel": 8}
    pk = res["per_kernel"]
    name = max(pk, key=lambda n: pk[n]["avg_ms"] * pk[n]["launches"])
    if name in per:
        flops = per[name] * w.d * res["pairs"]
        ach = flops / (pk[name]["avg_ms"] * 1e-3) / 1e12
        traffic = measured_traffic(name) if w.name == "qwen3-8b-layer-n32768-K32" else None
        return dict(bound="mfma", achieved=round(ach, 2), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / BF16_PEAK_TFLOPS, 4), traffic=traffic, kernel=name,
                    avg_ms=round(pk[name]["avg_ms"], 4), flop_per_launch=flops,
                    traffic_unit="bytes per launch (HBM, rocprofv3 counters)")
    return dict(bound="hbm", achieved=None, peak=HBM_PEAK_GBS, unit="GB/s", frac=None,
                traffic=None, kernel=name)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(res, np, budget_s=15.0):
    """The oracle as it stands (numpy, float64 gather mode: it is the
    correctness reference, so it computes in float64 throughout) on a bounded
    sample of the same workload: whole q-blocks, forward + backward, until
    ~budget_s of CPU time."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    w = res["w"]
    h = res["host"]
    s = res["s"].cpu().numpy()
    idx, cnt, lg, _ = oracle.select(s[:, :1], w.topk)          # kv-head 0 rows
    G = w.Hq // w.Hkv
    k0, v0 = h["k"][:, :1], h["v"][:, :1]
    q0, do0 = h["q"][:, :G], h["do"][:, :G]
    rng = np.random.default_rng(0)
    order = rng.permutation(w.nqb)
    t0 = time.perf_counter()
    done, pairs = 0, 0
    for i in order:
        oracle.fwd_gather_block(q0, k0, v0, idx, cnt, lg, 0, 0, int(i))
        oracle.bwd_gather_block(q0, k0, v0, do0, idx, cnt, lg, 0, 0, int(i))
        done += 1
        pairs += G * (int(cnt[0, 0, i]) * 4096 + 2080)
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    flops = 14 * w.d * pairs
    return dict(value=round(flops / el / 1e12, 6), unit="TFLOP/s", cores=int(threads), kind="oracle",
                cpu_model=cpu_model(), dtype="f64",
                sample=f"{done} of {w.nqb * w.Hkv * w.B} (batch, kv-head, q-block) units of the "
                       f"{w.name} workload, kv-head 0, forward+backward in float64 gather mode, "
                       f"{el:.1f} s")


def run_decode(args, api, si, torch, np):
    w = si.DECODE_WORKLOAD
    dt = torch.bfloat16
    qh, sh_ = si.decode_q_and_scores(w)
    lens = si.decode_seq_lens(w)
    kc, vc = si.decode_cache_device(w, "cuda")
    q = torch.from_numpy(qh).cuda().to(dt)
    s = torch.from_numpy(sh_).cuda()
    L = torch.from_numpy(lens).cuda()
    shp = api.make_decode_shape(w.B, w.Hq, w.Hkv, w.cap, w.d, w.topk, dt)
    o = torch.empty_like(q)
    idx = torch.empty((w.B, w.Hkv, w.topk), dtype=torch.int32, device="cuda")
    ws = api.alloc_workspace(api.sas_decode_workspace_bytes(shp))
    # warm-up: the first passes over a freshly allocated 8.6 GB cache run slow
    for _ in range(20):
        api.sas_decode(shp, q, kc, vc, L, s, o, idx, ws)
    torch.cuda.synchronize()
    # timed calls without the per-launch profiling events (each pair of event
    # records adds a few microseconds of idle time per call)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.decode_steps):
        api.sas_decode(shp, q, kc, vc, L, s, o, idx, ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.decode_steps
    # kernel durations from a second pass of the same calls with the events
    api.sas_prof_collect()
    api.sas_prof_enable(True)
    for _ in range(args.decode_steps):
        api.sas_decode(shp, q, kc, vc, L, s, o, idx, ws)
    torch.cuda.synchronize()
    api.sas_prof_enable(False)
    kern = api.sas_prof_collect()
    G = w.Hq // w.Hkv
    kv_bytes = sum(w.Hkv * (w.topk * 64 + (int(x) - 511 * 64)) * w.d * 2 * 2 for x in lens)
    other = q.numel() * 2 * 2 + s.numel() * 4 + idx.numel() * 4 + w.B * 4
    alg = kv_bytes + other
    per_kernel = {n: dict(avg_us=round(t * 1e3 / max(c, 1), 2), launches=c) for n, (t, c) in kern.items()}
    split = per_kernel.get("sas_decode_kernel", {}).get("avg_us")
    out = dict(workload=w.name, us_per_call=round(us, 2), algorithmic_bytes=alg,
               GBs=round(alg / (us * 1e-6) / 1e9, 1),
               frac_hbm=round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), per_kernel=per_kernel)
    if split:
        gbs = kv_bytes / (split * 1e-6) / 1e9
        out["roofline"] = dict(bound="hbm", kernel="sas_decode_kernel", achieved=round(gbs, 1),
                               peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4),
                               traffic=measured_traffic("sas_decode_kernel"),
                               algorithmic_bytes=kv_bytes, avg_us=split)
    del kc, vc
    torch.cuda.empty_cache()
    return out


def run_decode_paged(args, api, si, torch, np, w=None):
    """Long-context paged decode (selection of every history block, then the
    kept tiles): us per call, and GB/s of the bytes a call must read (kept K/V
    rows, score rows, page-table entries, q) over that time."""
    w = si.PAGED_DECODE_WORKLOAD if w is None else w
    dt = torch.bfloat16
    qh, table, lens, sh_ = si.paged_decode_host(w)
    kp, vp = si.paged_pool_device(w, "cuda")
    q = torch.from_numpy(qh).cuda().to(dt)
    pt = torch.from_numpy(table).cuda()
    L = torch.from_numpy(lens).cuda()
    s = torch.from_numpy(sh_).cuda()
    shp = api.make_decode_paged_shape(w.B, w.Hq, w.Hkv, w.max_blocks, w.num_pages, w.d, w.topk, dt)
    o = torch.empty_like(q)
    idx = torch.empty((w.B, w.Hkv, w.topk), dtype=torch.int32, device="cuda")
    ws = api.alloc_workspace(api.sas_decode_paged_workspace_bytes(shp))

    def call():
        api.sas_decode_paged(shp, q, kp, vp, pt, L, s, o, idx, ws)

    for _ in range(20):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.decode_steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.decode_steps
    api.sas_prof_collect()
    api.sas_prof_enable(True)
    for _ in range(args.decode_steps):
        call()
    torch.cuda.synchronize()
    api.sas_prof_enable(False)
    kern = api.sas_prof_collect()
    kept = 0
    for x in lens:
        icur = (int(x) - 1) // 64
        kept += w.Hkv * (min(w.topk, icur) * 64 + (int(x) - 64 * icur))
    icur0 = (int(lens[0]) - 1) // 64
    kv_bytes = kept * w.d * 2 * 2
    score_bytes = sum(w.Hkv * ((int(x) - 1) // 64) * 4 for x in lens)
    other = q.numel() * 2 * 2 + w.B * w.Hkv * (w.topk + 1) * 4 * 2 + w.B * 4
    alg = kv_bytes + score_bytes + other
    per_kernel = {n: dict(avg_us=round(t * 1e3 / max(c, 1), 2), launches=c) for n, (t, c) in kern.items()}
    out = dict(workload=w.name, us_per_call=round(us, 2), algorithmic_bytes=alg,
               GBs=round(alg / (us * 1e-6) / 1e9, 1),
               frac_hbm=round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), per_kernel=per_kernel,
               history_blocks_per_row=icur0, kept_blocks_per_row=min(w.topk, icur0) + 1,
               pool_pages=w.num_pages)
    del kp, vp
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py runs on one GPU only; run with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch
    import gated_block_sparse_select_amd as api
    import sas_inputs as si

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        # a plain copy of known size: 1 GiB read + 1 GiB written
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    res = run_training(args, api, si, torch, np)
    w = res["w"]
    total = res["flop_fwd"] + res["flop_bwd"]
    tflops = total / (res["ms_step"] * 1e-3) / 1e12
    line = {
        "metric": "SAS fwd+bwd effective TFLOP/s @32K (Qwen3-8B shape) + % bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.d,
                   "n": w.n, "block": 64, "topk": w.topk,
                   "scores": "device mean-pool" if w.s_kind == "pool" else w.s_kind,
                   "step": "pool+select+fwd+bwd(dq,dk,dv,ds)" if w.s_kind == "pool"
                   else "select+fwd+bwd(dq,dk,dv,ds)",
                   "backward": "dZ tiles" if "sas_bwd_dqz_kernel" in res["per_kernel"]
                   else "recompute"},
        "frac_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
        "roofline": roofline_for(res),
        "effective_flop": {"fwd": res["flop_fwd"], "bwd": res["flop_bwd"], "pairs": res["pairs"]},
        "per_kernel_ms": {k: round(v["avg_ms"], 4) for k, v in res["per_kernel"].items()},
        "per_kernel_pass_ms_per_step": round(res["ms_prof"], 4),
        "hbm_kernels": hbm_kernels(res),
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(res, np)
    res.clear()
    torch.cuda.empty_cache()
    if not args.no_recompute:
        line["recompute_path"] = run_recompute_path(args, api, si, torch, np)
    if not args.no_configs:
        line["configs"] = run_configs(args, api, si, torch, np)
    if not args.no_full_range:
        line["full_range"] = run_full_range(args, api, si, torch, np)
        torch.cuda.empty_cache()
    if not args.no_gates:
        line["gate_variants"] = run_gate_variants(args, api, si, torch, np)
    if not args.no_packed:
        line["packed"] = run_packed(args, api, si, torch, np)
        torch.cuda.empty_cache()
    if not args.no_decode:
        torch.cuda.empty_cache()
        line["decode"] = run_decode(args, api, si, torch, np)
        line["decode_paged"] = run_decode_paged(args, api, si, torch, np)
        line["decode_paged_sweep"] = [
            {k: r[k] for k in ("workload", "us_per_call", "GBs", "per_kernel")}
            for r in (line["decode_paged"] if w is si.PAGED_DECODE_WORKLOAD
                      else run_decode_paged(args, api, si, torch, np, w)
                      for w in si.PAGED_DECODE_SWEEP)]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
