"""The C-ABI used from plain C (tests/c_caller/sas_c_caller.c, built with gcc
as C11 against include/sas.h): host-side checks on the CPU, and a whole
select -> fwd -> bwd layer on the GPU compared with the oracle."""
import os
import subprocess
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "c_caller"))
import build as c_build  # noqa: E402

import oracle  # noqa: E402
from parity_bars import assert_o, assert_rel  # noqa: E402
import sas_inputs as si  # noqa: E402


def _run(args, timeout):
    exe = c_build.ensure_built()
    return subprocess.run([exe, *args], capture_output=True, text=True, timeout=timeout)


def test_c_caller_host_checks():
    r = _run(["abi"], 60)
    assert r.returncode == 0, r.stderr
    assert "abi checks ok" in r.stdout


def _bf16_bits(x):
    return si.f32_to_bf16_bits(np.ascontiguousarray(x, np.float32))


def _from_bf16(path, shape):
    return si.bf16_bits_to_f32(np.fromfile(path, dtype=np.uint16)).reshape(shape)


@pytest.mark.gpu
@pytest.mark.parametrize("gate", [0, 3])
def test_c_caller_layer_parity(tmp_path, gate):
    """bf16 layer (GQA 4, d = 128, 12 blocks, K = 3) run by the C program; its
    outputs, read back from files, against the oracle at the bf16 bars."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = si.custom_workload(150 + gate, 1, 8, 2, 768, 128, 3, "bf16")
    q, k, v, do = si.make_qkv(w)
    s = si.make_scores(w)
    for name, x in (("q", q), ("k", k), ("v", v), ("do", do)):
        _bf16_bits(x).tofile(tmp_path / f"{name}.bin")
    np.ascontiguousarray(s, np.float32).tofile(tmp_path / "s.bin")
    r = _run(["layer", str(tmp_path), str(w.B), str(w.Hq), str(w.Hkv), str(w.n), str(w.d),
              str(w.topk), str(gate)], 120)
    assert r.returncode == 0, r.stderr
    gname = {0: "softmax", 3: "external"}[gate]
    ref = oracle.sas_forward_backward(q, k, v, do, s, w.topk, gate=gname)
    nb = w.nqb
    idx = np.fromfile(tmp_path / "idx.bin", dtype=np.int32).reshape(w.B, w.Hkv, nb, w.topk)
    cnt = np.fromfile(tmp_path / "cnt.bin", dtype=np.int32).reshape(w.B, w.Hkv, nb)
    assert np.array_equal(idx, ref["idx"]) and np.array_equal(cnt, ref["cnt"])
    o = _from_bf16(tmp_path / "o.bin", q.shape)
    assert_o(o, ref["o"], "bf16")
    for name, shape in (("dq", q.shape), ("dk", k.shape), ("dv", v.shape)):
        x = _from_bf16(tmp_path / f"{name}.bin", shape)
        assert_rel(x, ref[name], 2e-2, name)
    ds = np.fromfile(tmp_path / "ds.bin", dtype=np.float32).reshape(s.shape)
    assert_rel(ds, ref["ds"], 2e-2, "ds")
