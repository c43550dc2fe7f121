"""Paged compressed stores: the latents, index keys and e4m3 scales scattered over shuffled
pages of a pool and addressed through a block table. The paged path must give the same
bits as the contiguous one (same rows through the same arithmetic), for the indexer scores,
the selection and the attention output; one case also goes through the oracle."""
import numpy as np
import pytest
import torch

import sparse_attention_score_amd as S
import workloads as W
from oracle import oracle as O
from parity_util import bf16_dev_to_f64, check_index_row, check_outputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"


def _batch(wl):
    from sparse_attention_score_amd.step import DeviceBatch
    print(f"[case] {wl.name} T={wl.T} keys={wl.key_dtype} n={wl.visible().min()}..{wl.visible().max()}",
          flush=True)
    return DeviceBatch(wl)


def _paged_cache(d, P, seed, spare=3):
    """Copy the batch's stores into pools of P-row pages in a random order."""
    B, cap = d.C.shape[0], d.C.shape[1]
    per = -(-cap // P)
    npages = B * per + spare
    rng = np.random.default_rng(seed)
    ids = rng.permutation(npages)[:B * per].reshape(B, per).astype(np.int32)
    table = torch.from_numpy(ids).cuda()

    def pool_of(x, row_shape):
        pool = torch.zeros((npages * P,) + row_shape, dtype=x.dtype, device="cuda")
        for b in range(B):
            for i in range(per):
                r0, r1 = i * P, min(cap, (i + 1) * P)
                pg = int(ids[b, i])
                pool[pg * P:pg * P + (r1 - r0)] = x[b, r0:r1]
        return pool

    lat = pool_of(d.C, tuple(d.C.shape[2:]))
    keys = pool_of(d.KI, tuple(d.KI.shape[2:]))      # 128 bf16 / e4m3, or 64 MXFP4 bytes
    scales = pool_of(d.KS, tuple(d.KS.shape[2:])) if d.KS is not None else None   # fp32, or 4 E8M0 bytes
    lscales = pool_of(d.CS, tuple(d.CS.shape[2:])) if d.CS is not None else None
    cache = S.Cache(latents=lat, window=d.R, idx_keys=keys, idx_scales=scales, num_seqs=B,
                    compressed_cap=cap, block_table=table, page_size=P, latent_scales=lscales,
                    window_scales=d.RS)
    return cache


def _run(d, cache):
    sc = torch.full_like(d.scores, float("nan"))
    bm = torch.full_like(d.block_max, float("nan"))
    topk = torch.empty_like(d.topk)
    cand = torch.empty_like(d.cand)
    out = torch.empty_like(d.out)
    lse = torch.empty_like(d.lse)
    S.indexer_score(d.plan, d.queries, cache, d.qI, d.w, sc, bm)
    S.select_topk(d.plan, d.queries, sc, bm, topk, cand=cand, workspace=d.workspace)
    S.sparse_attn_fwd(d.plan, d.queries, cache, d.q, topk, out, lse, workspace=d.workspace)
    torch.cuda.synchronize()
    return sc, bm, topk, out, lse


def _same(d, res_p, res_c):
    E = d.E
    sp, bp, tp, op, lp = res_p
    sc, bc, tc, oc, lc = res_c
    assert torch.equal(sp[:, :E].view(torch.int32), sc[:, :E].view(torch.int32)), "scores"
    assert torch.equal(bp[:, :E // 8].view(torch.int32), bc[:, :E // 8].view(torch.int32)), "block maxima"
    assert torch.equal(tp, tc), "selection"
    assert torch.equal(op.view(torch.int16), oc.view(torch.int16)), "attention output"
    assert torch.equal(lp.view(torch.int32), lc.view(torch.int32)), "lse"


@pytest.mark.parametrize("kd,P", [("fp8", 16), ("fp8", 256), ("bf16", 64), ("mxfp4", 16), ("mxfp4", 128)])
def test_paged_decode_matches_contiguous(kd, P):
    # n = 20003 (pruning, ragged last block), 1500, 0 (window only), 17
    wl = W.make_decode(B=4, n_raw=[40006, 3000, 1, 35], ratio=2, key_dtype=kd,
                       name=f"paged-{kd}-{P}", with_compress=False, seed=51)
    d = _batch(wl)
    res_c = _run(d, d.cache)
    res_p = _run(d, _paged_cache(d, P, seed=P))
    _same(d, res_p, res_c)


def test_paged_prefill_chunk_runs_per_query_and_matches_oracle():
    # one sequence, 40 queries on 32-row pages: below the chunk kernel's 64-row stage, so
    # the indexer runs one key stream per query
    wl = W.make_prefill(T=40, offset=5000, ratio=1, key_dtype="bf16", name="paged-prefill", seed=52)
    d = _batch(wl)
    sc, bm, topk, out, lse = _run(d, _paged_cache(d, 32, seed=7))
    res = O.run(wl)
    topk = topk.cpu().numpy()
    res2 = O.run(wl, idx_override=[topk[t][topk[t] >= 0] for t in range(wl.T)])
    o = bf16_dev_to_f64(out)
    for t in range(wl.T):
        check_index_row(topk[t], res.idx[t], res.scores[t], 512, f"t={t}")
        check_outputs(o[t], res2.o[t], f"t={t} out")


@pytest.mark.parametrize("kd,P", [("bf16", 64), ("fp8", 256), ("mxfp4", 64)])
def test_paged_prefill_chunk_kernel_matches_contiguous(kd, P):
    # pages of at least 64 rows: the chunk kernel reads each 64-key stage from its page;
    # 300 queries over 20000+ keys (several chunks and stages, a ragged end)
    wl = W.make_prefill(T=300, offset=20000, ratio=1, key_dtype=kd, name=f"paged-chunk-{kd}", seed=54)
    d = _batch(wl)
    res_c = _run(d, d.cache)
    res_p = _run(d, _paged_cache(d, P, seed=3))
    _same(d, res_p, res_c)


@pytest.mark.parametrize("kind", ["mq", "ragged", "mq-mxfp4", "ragged-mxfp4"])
def test_paged_group_and_ragged_match_contiguous(kind):
    # the group kernel (6-query draft steps) and a ragged batch (chunk, group and per-query
    # launches from one call) on 64-row pages, with e4m3 / bf16 and with MXFP4 keys
    mx = kind.endswith("mxfp4")
    if kind.startswith("mq"):
        wl = W.make_decode_mq(B=3, n_raw=[3001, 40006, 700], G=6, ratio=2, key_dtype="mxfp4" if mx else "fp8",
                              name=f"paged-{kind}", seed=55)
    else:
        wl = W.make_ragged([9000, 3001, 4000, 5000, 700], [20, 1, 6, 6, 1], ratio=2,
                           key_dtype="mxfp4" if mx else "bf16", name=f"paged-{kind}", seed=56)
    d = _batch(wl)
    res_c = _run(d, d.cache)
    res_p = _run(d, _paged_cache(d, 64, seed=5))
    _same(d, res_p, res_c)


@pytest.mark.parametrize("kv", ["fp8", "mxfp4"])
def test_paged_code_latents_match_contiguous(kv):
    wl = W.make_decode(B=4, n_raw=[40006, 3000, 1, 35], ratio=2, key_dtype="fp8", kv_dtype=kv,
                       name=f"paged-{kv}kv", seed=57)
    d = _batch(wl)
    res_c = _run(d, d.cache)
    res_p = _run(d, _paged_cache(d, 64, seed=9))
    _same(d, res_p, res_c)


def test_paged_rejects():
    wl = W.make_decode(B=2, n_raw=300, ratio=2, key_dtype="fp8", name="paged-args",
                       with_compress=False, seed=53)
    d = _batch(wl)
    cache = _paged_cache(d, 16, seed=1)
    cache.c.page_size = 24                      # not a power of two
    with pytest.raises(S.SparseAttnError):
        S.indexer_score(d.plan, d.queries, cache, d.qI, d.w, d.scores, d.block_max)
    cache = _paged_cache(d, 16, seed=1)
    cand = torch.full((2, 2048), -1, dtype=torch.int32, device="cuda")
    sc = torch.empty((2, 16384), dtype=torch.float32, device="cuda")
    bm = torch.empty((2, 2048), dtype=torch.float32, device="cuda")
    with pytest.raises(S.SparseAttnError) as ei:
        S.indexer_score_cand(d.plan, d.queries, cache, d.qI, d.w, cand, sc, bm)
    assert ei.value.status == S.SA_EUNSUPPORTED
