"""S0 and S1 in one launch (indexer_score_compress): the compressor's work-groups ride in the
indexer's grid. The compressed rows (bf16, or e4m3 / MXFP4 codes with their scales) and the
indexer's scores and block maxima must be the same bits as the two separate calls
(sparse_attn_compress or sparse_attn_compress_codes, then indexer_score), for every indexer
kernel (per-query, grouped, chunk, ragged runs, paged stores) and every key and latent
format; also the job's fallbacks: a job whose rows would not fit the grid, and a batch with
no visible keys. Whole steps through the fused path are checked against the oracle by the
workload parity tests, which run DeviceBatch.run."""
import numpy as np
import pytest
import torch

import sparse_attention_score_amd as S
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"


def _job_inputs(G, ratio, kv, seed):
    """Random raw rows, gate logits and slot biases for G groups, and zeroed outputs."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    raw = torch.randn((G, ratio, 512), generator=g).to(torch.bfloat16).cuda()
    gate = torch.randn((G, ratio, 512), generator=g).to(torch.bfloat16).cuda()
    bias = torch.randn((ratio, 512), generator=g).float().cuda()
    if kv == "bf16":
        out, sc = torch.zeros((G, 512), dtype=torch.bfloat16, device="cuda"), None
    elif kv == "fp8":
        out, sc = torch.zeros((G, 512), dtype=torch.uint8, device="cuda"), torch.zeros((G,), device="cuda")
    else:
        out = torch.zeros((G, 256), dtype=torch.uint8, device="cuda")
        sc = torch.zeros((G, 16), dtype=torch.uint8, device="cuda")
    return raw, gate, bias, out, sc


def _compress_separately(plan, kv, raw, gate, bias, out, sc, G):
    ratio = raw.shape[1]
    if kv == "bf16":
        S.sparse_attn_compress(plan, raw, ratio * 512, gate, ratio * 512, bias, out, 512, G)
    else:
        S.sparse_attn_compress_codes(plan, raw, ratio * 512, gate, ratio * 512, bias, out, out.stride(0),
                                     sc, sc.stride(0) * sc.element_size(), G)


def _job(kv, raw, gate, bias, out, sc, G):
    ratio = raw.shape[1]
    if kv == "bf16":
        return S.CompressJob(raw, ratio * 512, gate, ratio * 512, bias, out, 512, G)
    return S.CompressJob(raw, ratio * 512, gate, ratio * 512, bias, out, out.stride(0), G, sc,
                         sc.stride(0) * sc.element_size())


def _check(d, G, seed, cache=None):
    """Separate calls, then the fused call, on fresh outputs; every output bitwise equal."""
    kvn, ratio = d.plan.kv_dtype, d.ratio
    cache = cache or d.cache
    raw, gate, bias, out_a, sc_a = _job_inputs(G, ratio, kvn, seed)
    out_b = torch.zeros_like(out_a)
    sc_b = None if sc_a is None else torch.zeros_like(sc_a)
    sc1, bm1 = torch.full_like(d.scores, float("nan")), torch.full_like(d.block_max, float("nan"))
    sc2, bm2 = torch.full_like(sc1, float("nan")), torch.full_like(bm1, float("nan"))
    if G:
        _compress_separately(d.plan, kvn, raw, gate, bias, out_a, sc_a, G)
    S.indexer_score(d.plan, d.queries, cache, d.qI, d.w, sc1, bm1)
    S.indexer_score_compress(d.plan, d.queries, cache, d.qI, d.w, sc2, bm2,
                             _job(kvn, raw, gate, bias, out_b, sc_b, G))
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b), "compressed rows differ"
    if sc_a is not None:
        assert torch.equal(sc_a, sc_b), "compressed row scales differ"
    if G:
        assert out_a.abs().sum() > 0 if out_a.dtype == torch.bfloat16 else bool((out_a != 0).any())
    E = d.E
    assert torch.equal(sc1[:, :E].view(torch.int32), sc2[:, :E].view(torch.int32)), "scores differ"
    assert torch.equal(bm1[:, :E // 8].view(torch.int32), bm2[:, :E // 8].view(torch.int32)), "block maxima differ"


def _batch(wl):
    from sparse_attention_score_amd.step import DeviceBatch
    print(f"[case] {wl.name} T={wl.T} keys={wl.key_dtype} kv={getattr(wl, 'kv_dtype', 'bf16')}", flush=True)
    return DeviceBatch(wl)


@pytest.mark.parametrize("kd,kv,G", [("bf16", "bf16", 6), ("fp8", "bf16", 300), ("mxfp4", "bf16", 7),
                                     ("fp8", "fp8", 6), ("fp8", "mxfp4", 129), ("bf16", "fp8", 1)])
def test_per_query_kernel(kd, kv, G):
    wl = W.make_decode(B=6, n_raw=[3001, 9000, 700, 40006, 64, 2], ratio=2, key_dtype=kd, kv_dtype=kv,
                       with_compress=False, name=f"fused-decode-{kd}-{kv}", seed=41)
    _check(_batch(wl), G, seed=1)


@pytest.mark.parametrize("kd", ["fp8", "mxfp4", "bf16"])
def test_group_kernel(kd):
    wl = W.make_decode_mq(B=3, n_raw=[3001, 1030, 40006], G=6, ratio=2, key_dtype=kd, name=f"fused-mq-{kd}", seed=42)
    _check(_batch(wl), 40, seed=2)


@pytest.mark.parametrize("kd,G", [("bf16", 48), ("fp8", 5000)])
def test_chunk_kernel_ratio1(kd, G):
    # a prefill chunk: ratio-1 layers copy raw rows; 5000 groups need many job rows
    wl = W.make_prefill(T=48, offset=5000, ratio=1, key_dtype=kd, name=f"fused-prefill-{kd}", seed=43)
    _check(_batch(wl), G, seed=3)


def test_ragged_runs():
    # the job rides in the first of the batch's launches
    wl = W.make_ragged([9000, 3001, 4000, 5000, 700], [20, 1, 6, 6, 1], ratio=2, key_dtype="fp8",
                       name="fused-ragged", seed=44)
    _check(_batch(wl), 17, seed=4)


def test_paged_stores():
    from test_gpu_paged import _paged_cache
    wl = W.make_decode(B=4, n_raw=[40006, 3000, 1, 35], ratio=2, key_dtype="fp8", with_compress=False,
                       name="fused-paged", seed=45)
    d = _batch(wl)
    _check(d, 9, seed=5, cache=_paged_cache(d, 64, seed=6))


def test_job_past_the_grid_limit():
    # 270,000 groups of e4m3 code rows want more work-groups (one wave per group) than the
    # grid's rows allow beside the queries': the job runs in a launch of its own, first,
    # with the same results
    wl = W.make_decode(B=2, n_raw=[3001, 900], ratio=1, key_dtype="bf16", kv_dtype="fp8", with_compress=False,
                       name="fused-big-job", seed=46)
    _check(_batch(wl), 270000, seed=7)


def test_no_visible_keys():
    # every query at raw position 0 of a ratio-2 layer sees no compressed position: the job
    # alone runs (and the indexer writes nothing)
    wl = W.make_decode(B=3, n_raw=[1, 1, 1], ratio=2, key_dtype="bf16", with_compress=False,
                       name="fused-empty", seed=47)
    d = _batch(wl)
    assert d.E == 0
    raw, gate, bias, out_a, _ = _job_inputs(5, 2, "bf16", 8)
    out_b = torch.zeros_like(out_a)
    S.sparse_attn_compress(d.plan, raw, 1024, gate, 1024, bias, out_a, 512, 5)
    S.indexer_score_compress(d.plan, d.queries, d.cache, d.qI, d.w, d.scores, d.block_max,
                             _job("bf16", raw, gate, bias, out_b, None, 5))
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and out_a.abs().sum() > 0


def test_step_fused_matches_unfused():
    # a whole step of a uniform decode batch (with its compressor inputs) both ways; the
    # compressed row the step writes is cleared before the fused pass
    wl = W.make_decode(B=5, n_raw=4002, ratio=2, key_dtype="fp8", name="fused-step", seed=48)
    d = _batch(wl)
    n = 4002 // 2
    d.run(fused=False)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (d.C, d.scores, d.block_max, d.topk, d.out, d.lse)]
    d.C[:, n - 1].zero_()
    for t in (d.scores, d.block_max, d.lse):
        t.fill_(float("nan"))
    d.topk.fill_(-7)
    d.out.zero_()
    d.run(fused=True)
    torch.cuda.synchronize()
    E = d.E   # entries past E (scores) and E / 8 (block maxima) are not written
    ref[1], ref[2] = ref[1][:, :E], ref[2][:, :E // 8]
    for a, b, name in zip(ref, (d.C, d.scores[:, :E], d.block_max[:, :E // 8], d.topk, d.out, d.lse),
                          ("latents", "scores", "block max", "topk", "out", "lse")):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), name
