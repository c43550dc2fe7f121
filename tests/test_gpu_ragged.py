"""Ragged batches: runs of consecutive queries of one sequence each (prefill chunks, decode
steps with drafted tokens, single decode queries) in one call. indexer_score launches the
chunk, group and per-query kernels over the matching query ranges; checked end to end
against the fp64 oracle, and the scores of every run against the per-query path."""
import numpy as np
import pytest
import torch

import sparse_attention_score_amd as S
import workloads as W
from oracle import oracle as O
from parity_util import LSE_TOL, SCORE_REL, bf16_dev_to_f64, check_index_row, check_outputs, kth_score

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"


@pytest.mark.parametrize("kd", ["bf16", "fp8", "mxfp4"])
def test_ragged_batch_end_to_end(kd):
    # a 100-query chunk, decode singles, two 6-query draft steps (one group launch), a
    # 20-query chunk, a 3-query step, a 9-query run (chunk kernel); contexts up to 20k
    lengths = [100, 1, 6, 6, 1, 20, 3, 9]
    n_raw = [12000, 3001, 40006, 5000, 2, 9000, 700, 2048]
    wl = W.make_ragged(n_raw, lengths, ratio=2, key_dtype=kd, name=f"ragged-{kd}", seed=61)
    from sparse_attention_score_amd.step import DeviceBatch
    print(f"[case] {wl.name} T={wl.T} runs={wl.runs}", flush=True)
    d = DeviceBatch(wl)
    d.index()
    d.select()
    d.attend()
    torch.cuda.synchronize()
    res = O.run(wl)
    scores = d.scores.cpu().numpy()
    topk = d.topk.cpu().numpy()
    o = bf16_dev_to_f64(d.out)
    lse = d.lse.cpu().numpy()
    res2 = O.run(wl, idx_override=[topk[t][topk[t] >= 0] for t in range(wl.T)])
    n = wl.visible()
    for t in range(wl.T):
        I = res.scores[t]
        if n[t]:
            tol = SCORE_REL * np.maximum(np.abs(I), abs(kth_score(I, 512)))
            assert np.all(np.abs(scores[t, :n[t]] - I) <= tol + 1e-30), f"t={t} scores"
        assert np.all(np.isneginf(scores[t, n[t]:d.E])), f"t={t} masked"
        check_index_row(topk[t], res.idx[t], I, 512, f"t={t} topk")
        check_outputs(o[t], res2.o[t], f"t={t} out")
        assert np.abs(lse[t] - res2.lse[t]).max() <= LSE_TOL, f"t={t} lse"
    # the same batch without runs (one key stream per query): the same selections up to the
    # tie band, scores within rounding
    q = S.Queries(d.seq, d.pos, d.max_visible)
    sc = torch.empty_like(d.scores)
    bm = torch.empty_like(d.block_max)
    S.indexer_score(d.plan, q, d.cache, d.qI, d.w, sc, bm)
    torch.cuda.synchronize()
    sc = sc.cpu().numpy()
    for t in range(wl.T):
        if n[t]:
            Ik = kth_score(res.scores[t], 512)
            ref = sc[t, :n[t]].astype(np.float64)
            assert np.all(np.abs(scores[t, :n[t]] - ref) <= 2 * SCORE_REL * np.maximum(np.abs(ref), abs(Ik)) + 1e-30), t
