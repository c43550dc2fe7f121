"""Multi-token decode: groups of consecutive queries that read one sequence (a verified
token and the drafted tokens after it) share one key stream in the indexer. Checked
end to end against the fp64 oracle, and bit for bit against the per-query decode
indexer (the grouped kernel does each query's arithmetic in the same order)."""
import numpy as np
import pytest
import torch

import sparse_attention_score_amd as S
import workloads as W
from oracle import oracle as O
from parity_util import LSE_TOL, bf16_dev_to_f64, check_index_row, check_outputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"


def _batch(wl):
    from sparse_attention_score_amd.step import DeviceBatch
    print(f"[case] {wl.name} T={wl.T} group={wl.group} keys={wl.key_dtype} "
          f"n={wl.visible().min()}..{wl.visible().max()}", flush=True)
    return DeviceBatch(wl)


def _scores(d, group, T=None):
    """Indexer scores and block maxima of the first T queries with the given grouping."""
    T = d.T if T is None else T
    q = S.Queries(d.seq[:T], d.pos[:T], d.max_visible, group)
    sc = torch.full((T, d.scores.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
    bm = torch.full((T, d.block_max.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
    S.indexer_score(d.plan, q, d.cache, d.qI[:T], d.w[:T], sc, bm)
    torch.cuda.synchronize()
    return sc.cpu().numpy(), bm.cpu().numpy()


def _same_bits(a, b, E, what):
    assert np.array_equal(a[:, :E].view(np.uint32), b[:, :E].view(np.uint32)), what


@pytest.mark.parametrize("kd", ["bf16", "fp8", "mxfp4"])
def test_multiquery_decode_end_to_end(kd):
    # 3 sequences x 6 queries (positions n_raw-6 .. n_raw-1), ragged contexts; the
    # longest prunes blocks in the candidate stage
    wl = W.make_decode_mq(B=3, n_raw=[3001, 1030, 40006], G=6, ratio=2, key_dtype=kd,
                          name=f"mq6-{kd}", seed=31)
    d = _batch(wl)
    d.index()
    d.select()
    d.attend()
    torch.cuda.synchronize()
    res = O.run(wl)
    topk = d.topk.cpu().numpy()
    o_gpu = bf16_dev_to_f64(d.out)
    lse_gpu = d.lse.cpu().numpy()
    res2 = O.run(wl, idx_override=[topk[t][topk[t] >= 0] for t in range(wl.T)])
    for t in range(wl.T):
        check_index_row(topk[t], res.idx[t], res.scores[t], 512, f"{wl.name} t={t} topk")
        check_outputs(o_gpu[t], res2.o[t], f"{wl.name} t={t} out")
        assert np.abs(lse_gpu[t] - res2.lse[t]).max() <= LSE_TOL, f"t={t} lse"
    # the grouped scores are the per-query kernel's, bit for bit
    g_sc, g_bm = d.scores.cpu().numpy(), d.block_max.cpu().numpy()
    u_sc, u_bm = _scores(d, 0)
    _same_bits(g_sc, u_sc, d.E, "scores")
    _same_bits(g_bm, u_bm, d.E // 8, "block maxima")


@pytest.mark.parametrize("kd", ["fp8", "mxfp4"])
@pytest.mark.parametrize("G", [2, 3, 5, 6, 7, 8])
def test_multiquery_group_sizes_bitwise(G, kd):
    # group sizes that run in the next even kernel size (masked extra queries) and the
    # largest; short contexts so every group has keys past some queries' n. MXFP4 keys:
    # the grouped MXFP4 kernel against the per-query MXFP4 kernel.
    wl = W.make_decode_mq(B=3, n_raw=[70, 2500, 9001], G=G, ratio=2, key_dtype=kd,
                          name=f"mq{G}-{kd}", seed=32 + G)
    d = _batch(wl)
    g_sc, g_bm = _scores(d, G)
    u_sc, u_bm = _scores(d, 0)
    _same_bits(g_sc, u_sc, d.E, f"G={G} scores")
    _same_bits(g_bm, u_bm, d.E // 8, f"G={G} block maxima")
    n = wl.visible()
    for t in range(wl.T):
        assert np.all(np.isneginf(g_sc[t, n[t]:d.E])), t


def test_multiquery_partial_last_group_and_foreign_query():
    # 4 sequences x 4 queries, called on the first 14 queries in groups of 4: the last
    # group holds 2 queries. Then groups of 5 straddle sequences: a query whose sequence
    # differs from its group's first query gets -inf scores by contract.
    wl = W.make_decode_mq(B=4, n_raw=[500, 4000, 1200, 17], G=4, ratio=2, key_dtype="bf16",
                          name="mq-partial", seed=40)
    d = _batch(wl)
    g_sc, g_bm = _scores(d, 4, T=14)
    u_sc, u_bm = _scores(d, 0, T=14)
    _same_bits(g_sc, u_sc, d.E, "partial group scores")
    _same_bits(g_bm, u_bm, d.E // 8, "partial group block maxima")
    f_sc, _ = _scores(d, 5)
    u_all, _ = _scores(d, 0)
    seq = wl.seq
    for t in range(wl.T):
        first = (t // 5) * 5
        if seq[t] == seq[first]:
            assert np.array_equal(f_sc[t, :d.E].view(np.uint32), u_all[t, :d.E].view(np.uint32)), t
        else:
            assert np.all(np.isneginf(f_sc[t, :d.E])), t


def test_multiquery_full_size_sampled():
    # the multi-token decode batch at full size: 128 sequences x 6 queries at 128K context,
    # e4m3 keys; grouped scores bitwise against the per-query kernel on a few sequences,
    # sampled queries end to end against the oracle
    wl = W.make("decode-mq6-b128-ctx128k-fp8")
    d = _batch(wl)
    d.run()
    torch.cuda.synchronize()
    topk = d.topk.cpu().numpy()
    o_gpu = bf16_dev_to_f64(d.out)
    C_new = O.step_compress(wl)
    keys = {}
    for t in (0, 5, 383, 767):
        b = int(wl.seq[t])
        if b not in keys:
            nn = int(wl.visible()[wl.seq == b].max())
            keys = {b: O.index_keys_f64(wl.KI[b, :nn], wl.KS[b, :nn])}
        I, cand, idx, _, _ = O.run_query(wl, t, keys[b], C_new)
        check_index_row(topk[t], idx, I, 512, f"full t={t}")
        _, _, _, o, lse = O.run_query(wl, t, keys[b], C_new, idx_override=topk[t][topk[t] >= 0])
        check_outputs(o_gpu[t], o, f"full t={t} out")
    u_sc, _ = _scores(d, 0, T=12)   # sequences 0 and 1
    _same_bits(d.scores[:12].cpu().numpy(), u_sc, d.E, "full-size scores")
