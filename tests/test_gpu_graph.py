"""A whole step captured in a HIP graph must reproduce the eager step exactly on every
replay (the kernels are deterministic and the library only enqueues launches)."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def _snapshot(d):
    return {k: getattr(d, k).clone() for k in ("scores", "block_max", "cand", "topk", "out", "lse", "C")}


@pytest.mark.parametrize("name", ["decode-b4-ctx2k", "prefill-small"])
def test_graph_replays_match_eager(name):
    from sparse_attention_score_amd.step import DeviceBatch
    if name == "prefill-small":
        wl = W.make_prefill(T=48, offset=5000, ratio=1, key_dtype="bf16", name=name, seed=31)
    else:
        wl = W.make(name)
    print(f"[case] graph {name} T={wl.T}", flush=True)
    d = DeviceBatch(wl)
    d.run()
    torch.cuda.synchronize()
    ref = _snapshot(d)
    g = d.capture()
    for r in range(4):
        # the program's own eager work between replays: clobber the outputs, run eagerly
        for k in ("scores", "out", "topk"):
            getattr(d, k).fill_(0)
        d.run()
        torch.cuda.synchronize()
        for k in ("scores", "block_max", "out", "lse", "topk"):
            getattr(d, k).fill_(0)
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(d)
        for k, v in ref.items():
            assert torch.equal(v, got[k]), f"replay {r}: {k} differs from the eager step"
