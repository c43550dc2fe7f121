"""The measured workloads at full size, in the launch configuration bench.py times: the five
layer configurations and the further batches bench.py reports (MXFP4 keys, e4m3 and MXFP4
latent rows, the ragged serving batch; the multi-token batch has its own test).

All queries are checked for properties that hold at any size (selection well-formed,
block maxima consistent with the scores); a sample of queries per workload is checked
against the fp64 oracle one query at a time (index sets within the tie band, outputs
within tolerance on the GPU's selection)."""
import gc
import time

import numpy as np
import pytest
import torch

import workloads as W
from oracle import oracle as O
from parity_util import (LSE_TOL, SCORE_REL, bf16_dev_to_f64, check_index_row, check_outputs,
                         kth_score)

pytestmark = pytest.mark.gpu

SAMPLES = {
    "decode-b4-ctx2k": [0, 1, 2, 3],
    "decode-b64-ctx32k": [0, 17, 42, 63],
    "decode-b128-ctx128k-fp8": [0, 77, 127],
    "prefill-4096-at-61440": [0, 1, 127, 2048, 4094, 4095],
    "decode-b8-ctx1m-fp8": [0, 7],
}


# sampled queries of the further batches (ragged: first and last query of each prefill chunk,
# single decode queries, the first and last query of a draft step)
MORE_SAMPLES = {
    "decode-b128-ctx128k-mxfp4": [0, 127],
    "decode-b128-ctx128k-fp8kv": [0, 127],
    "decode-b128-ctx128k-fp4kv": [0, 64, 127],
    "ragged-2x1024+64+16x6-ctx128k-fp8": [0, 1023, 1024, 2047, 2048, 2111, 2112, 2117, 2207],
}


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_full_size(name):
    _full_size(name, SAMPLES[name])


@pytest.mark.parametrize("name", list(MORE_SAMPLES))
def test_more_workloads_full_size(name):
    _full_size(name, MORE_SAMPLES[name])


def _full_size(name, samples):
    assert torch.cuda.is_available()
    from sparse_attention_score_amd.step import DeviceBatch
    t0 = time.time()
    print(f"[workload] {name}: generating", flush=True)
    wl = W.make(name)
    print(f"[workload] {name}: generated in {time.time() - t0:.1f}s; uploading", flush=True)
    d = DeviceBatch(wl)
    d.run()
    torch.cuda.synchronize()
    print(f"[workload] {name}: GPU pass done at {time.time() - t0:.1f}s", flush=True)
    n = wl.visible()
    topk = d.topk.cpu().numpy()
    cand = d.cand.cpu().numpy()
    # well-formed selection for every query
    for t in range(wl.T):
        k = min(512, int(n[t]))
        row = topk[t]
        assert np.all(row[:k] >= 0) and np.all(row[k:] == -1), t
        assert np.all(np.diff(row[:k]) > 0) and row[:k].max(initial=-1) < n[t], t
        nb = -(-int(n[t]) // 8)
        kc = min(2048, nb)
        assert np.all(cand[t, :kc] >= 0) and np.all(cand[t, kc:] == -1), t
        assert np.all(np.diff(cand[t, :kc]) > 0), t
        # every selected position lies in a kept block
        assert np.all(np.isin(row[:k] // 8, cand[t, :kc])), t
    keys_cache = {}
    C_new = O.step_compress(wl)
    for t in samples:
        b = int(wl.seq[t])
        if b not in keys_cache:
            nn = int(n[wl.seq == b].max())
            keys_cache = {b: O.index_keys_f64(wl.KI[b, :nn], None if wl.KS is None else wl.KS[b, :nn])}
        I, c_ref, i_ref, _, _ = O.run_query(wl, t, keys_cache[b], C_new)
        got = d.scores[t, :n[t]].cpu().numpy().astype(np.float64)
        Ik = kth_score(I, 512)
        assert np.all(np.abs(got - I) <= SCORE_REL * np.maximum(np.abs(I), abs(Ik))), t
        bm = d.block_max[t].cpu().numpy()
        nb = -(-int(n[t]) // 8)
        g32 = d.scores[t, :nb * 8].cpu().numpy()
        g32 = np.where(np.arange(nb * 8) < n[t], g32, -np.inf).reshape(nb, 8).max(1)
        assert np.array_equal(bm[:nb], g32), t
        check_index_row(topk[t], i_ref, I, 512, f"{name} t={t} topk")
        check_index_row(cand[t], c_ref, O.block_scores(I), 2048, f"{name} t={t} cand")
        sel = topk[t][topk[t] >= 0]
        _, _, _, o_ref, lse_ref = O.run_query(wl, t, keys_cache[b], C_new, idx_override=sel)
        o = bf16_dev_to_f64(d.out[t])
        mx, mn = check_outputs(o, o_ref, f"{name} t={t}")
        assert np.abs(d.lse[t].cpu().numpy() - lse_ref).max() <= LSE_TOL, t
        print(f"[workload] {name} t={t}: ok (max {mx:.2e} mean {mn:.2e}) at {time.time() - t0:.1f}s",
              flush=True)
    del d, wl, keys_cache
    gc.collect()
    torch.cuda.empty_cache()
