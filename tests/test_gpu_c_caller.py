"""The decode path driven from a plain host program (tests/c/decode_step.cpp: HIP runtime
calls for memory, the library's C entry points for the work, no Python in the process),
checked against the fp64 oracle like the Python-driven tests."""
import os
import subprocess

import numpy as np
import pytest
import torch

import workloads as W
from oracle import oracle as O
from parity_util import LSE_TOL, check_index_row, check_outputs

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "decode_step")


def test_c_program_runs_the_decode_path(tmp_path):
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    assert os.path.exists(EXE), "tests/c/decode_step is built with the library (__graft_entry__.build)"
    # n = 1024, 750, 150 (every block a candidate), 4 visible latents
    wl = W.make_decode(B=4, n_raw=[2048, 1500, 300, 9], ratio=2, key_dtype="bf16", with_compress=False,
                       name="c-caller", seed=61)
    T, B = wl.T, wl.B
    with open(tmp_path / "meta.txt", "w") as f:
        f.write(f"{B} {wl.nc_cap} {wl.wcap} {T} {int(wl.visible().max())} {wl.ratio}\n")
    for name, arr, dt in (("seq", wl.seq, np.int32), ("pos", wl.pos, np.int32), ("q", wl.q, np.uint16),
                          ("qi", wl.qI, np.uint16), ("w", wl.w, np.float32), ("lat", wl.C, np.uint16),
                          ("win", wl.R, np.uint16), ("keys", wl.KI, np.uint16)):
        np.ascontiguousarray(arr, dtype=dt).tofile(tmp_path / f"{name}.bin")
    print(f"[case] {wl.name} via {EXE}", flush=True)
    # SPARSE_ATTN_LOG=1: one line per accepted call on stderr, naming the path taken
    r = subprocess.run([EXE, str(tmp_path)], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, SPARSE_ATTN_LOG="1"))
    assert r.returncode == 0, r.stderr
    log = [ln for ln in r.stderr.splitlines() if ln.startswith("[sparse_attn] ")]
    assert any(ln.startswith("[sparse_attn] indexer_score: T=4 ") and "per-query kernel" in ln for ln in log), log
    assert any(ln.startswith("[sparse_attn] select_topk: T=4 ") for ln in log), log
    assert any(ln.startswith("[sparse_attn] sparse_attn_fwd: T=4 ") for ln in log), log
    topk = np.fromfile(tmp_path / "topk.bin", dtype=np.int32).reshape(T, 512)
    out = np.fromfile(tmp_path / "out.bin", dtype=np.uint16).reshape(T, 64, 512)
    lse = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(T, 64)
    res = O.run(wl)
    res2 = O.run(wl, idx_override=[topk[t][topk[t] >= 0] for t in range(T)])
    o = O.bf16_to_f64(out)
    for t in range(T):
        check_index_row(topk[t], res.idx[t], res.scores[t], 512, f"t={t} topk")
        check_outputs(o[t], res2.o[t], f"t={t} out")
        assert np.abs(lse[t] - res2.lse[t]).max() <= LSE_TOL, t
