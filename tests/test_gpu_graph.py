"""A whole step captured in a HIP graph must reproduce the eager step exactly on every
replay (the kernels are deterministic and the library only enqueues launches)."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def _snapshot(d):
    # the defined parts: score rows up to E (max_visible rounded to 8) and their block maxima;
    # the rows' padding past them is never written
    snap = {k: getattr(d, k).clone() for k in ("cand", "topk", "out", "lse", "C")}
    snap["scores"] = d.scores[:, :d.E].clone()
    snap["block_max"] = d.block_max[:, :d.E // 8].clone()
    return snap


@pytest.mark.parametrize("name", ["decode-b4-ctx2k", "prefill-small", "ragged-small", "mq-small",
                                  "mxfp4-small", "fp4kv-small"])
def test_graph_replays_match_eager(name):
    # ragged-small issues several indexer launches from one call (chunk, group, per-query)
    from sparse_attention_score_amd.step import DeviceBatch
    if name == "prefill-small":
        wl = W.make_prefill(T=48, offset=5000, ratio=1, key_dtype="bf16", name=name, seed=31)
    elif name == "ragged-small":
        wl = W.make_ragged([9000, 3001, 4000, 5000, 700], [20, 1, 6, 6, 1], ratio=2, key_dtype="fp8",
                           name=name, seed=32)
    elif name == "mq-small":
        wl = W.make_decode_mq(B=5, n_raw=[3001, 9000, 700, 20000, 64], G=6, ratio=2, key_dtype="fp8",
                              name=name, seed=33)
    elif name == "mxfp4-small":
        wl = W.make_decode(B=6, n_raw=[3001, 9000, 700, 40006, 64, 2], ratio=2, key_dtype="mxfp4",
                           name=name, seed=34, with_compress=False)
    elif name == "fp4kv-small":
        # MXFP4 latents and e4m3 window rows (key splits: 6 queries)
        wl = W.make_decode(B=6, n_raw=[3001, 9000, 700, 40006, 64, 2], ratio=2, key_dtype="fp8",
                           kv_dtype="mxfp4", name=name, seed=35)
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
