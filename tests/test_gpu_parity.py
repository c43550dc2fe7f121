"""Parity of the HIP path (through the C ABI) with the fp64 oracle on small and ragged
batches that span several tiles, per stage and end to end, plus edge cases."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import oracle as O
from parity_util import (LSE_TOL, SCORE_REL, bf16_dev_to_f64, bf16_ulp, check_index_row,
                         check_outputs, compress_tol, kth_score)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import sparse_attention_score_amd  # noqa: F401  (raises if the library is not built)


def _run(wl, stages=("compress", "index", "select", "attend")):
    from sparse_attention_score_amd.step import DeviceBatch
    print(f"[case] {wl.name} T={wl.T} B={wl.B} ratio={wl.ratio} keys={wl.key_dtype} "
          f"n={wl.visible().min()}..{wl.visible().max()}", flush=True)
    d = DeviceBatch(wl)
    for s in stages:
        getattr(d, s)()
    torch.cuda.synchronize()
    return d


def _scores_check(d, res, wl, t):
    n = int(wl.visible()[t])
    got = d.scores[t].cpu().numpy()
    I = res.scores[t]
    if n:
        Ik = kth_score(I, 512)
        tol = SCORE_REL * np.maximum(np.abs(I), abs(Ik))
        err = np.abs(got[:n].astype(np.float64) - I)
        assert np.all(err <= tol + 1e-30), f"t={t}: score err {err.max():.3g} > tol at j={err.argmax()}"
    assert np.all(np.isneginf(got[n:d.E])), f"t={t}: masked scores not -inf"
    # block maxima equal the max of the GPU's own scores, bit for bit
    bm = d.block_max[t].cpu().numpy()
    nb = -(-n // 8)
    for b in range(nb):
        assert bm[b] == got[8 * b:min(n, 8 * b + 8)].max(), f"t={t} block {b}"
    assert np.all(np.isneginf(bm[nb:d.E // 8]))


def _e2e(wl, check_scores=True, lse_tol=LSE_TOL):
    d = _run(wl)
    res = O.run(wl)
    topk = d.topk.cpu().numpy()
    cand = d.cand.cpu().numpy()
    o_gpu = bf16_dev_to_f64(d.out)
    lse_gpu = d.lse.cpu().numpy()
    idx_gpu = [topk[t][topk[t] >= 0] for t in range(wl.T)]
    res2 = O.run(wl, idx_override=idx_gpu)   # oracle attention on the GPU's selection
    for t in range(wl.T):
        if check_scores:
            _scores_check(d, res, wl, t)
        check_index_row(topk[t], res.idx[t], res.scores[t], 512, f"{wl.name} t={t} topk")
        n = int(wl.visible()[t])
        if n:
            M = O.block_scores(res.scores[t])
            check_index_row(cand[t], res.cand[t], M, 2048, f"{wl.name} t={t} cand")
        check_outputs(o_gpu[t], res2.o[t], f"{wl.name} t={t} out")
        assert np.abs(lse_gpu[t] - res2.lse[t]).max() <= lse_tol, f"t={t} lse"
    return d, res


# ------------------------------------------------------------------ end to end, small

def test_decode_small_bf16():
    _e2e(W.make("decode-b4-ctx2k"))


def test_decode_ragged_fp8_mixed_positions():
    wl = W.make_decode(B=3, n_raw=[3001, 1022, 20001], ratio=2, key_dtype="fp8",
                       name="ragged-fp8", with_compress=False, seed=3)
    _e2e(wl)


@pytest.mark.parametrize("kd", ["bf16", "fp8"])
def test_decode_candidate_stage_prunes(kd):
    # n = 20003 -> 2501 blocks, 2048 kept; the last block holds 3 positions
    wl = W.make_decode(B=2, n_raw=40006, ratio=2, key_dtype=kd, name=f"prune-{kd}", seed=5)
    d, res = _e2e(wl)
    cand = d.cand.cpu().numpy()
    assert np.all(cand >= 0)  # exactly 2048 kept


@pytest.mark.parametrize("n_raw", [[40006, 3001], [1, 2, 17, 130, 1031]])
def test_decode_mxfp4_keys(n_raw):
    # MXFP4 index keys (E2M1 elements, E8M0 block scales): pruning and a ragged last
    # block, then n = 0, 1, 8, 65, 515
    wl = W.make_decode(B=len(n_raw), n_raw=n_raw, ratio=2, key_dtype="mxfp4",
                       name=f"mxfp4-{len(n_raw)}", with_compress=False, seed=17)
    _e2e(wl)


def test_mxfp4_keys_in_a_prefill_chunk_and_a_group():
    # chunks of one sequence (the chunk kernel widens E2M1 x scale while staging; several
    # chunks and stages, a ragged end) and a multi-token decode batch (per-query kernel)
    _e2e(W.make_prefill(T=40, offset=20000, ratio=1, key_dtype="mxfp4", name="prefill-mxfp4", seed=18))
    _e2e(W.make_prefill(T=150, offset=9001, ratio=2, key_dtype="mxfp4", name="prefill-mxfp4-r2", seed=20))
    _e2e(W.make_decode_mq(B=2, n_raw=[3001, 9000], G=6, ratio=2, key_dtype="mxfp4",
                          name="mq-mxfp4", seed=19), check_scores=True)


@pytest.mark.parametrize("B,n_raw", [(6, [40006, 3001, 2, 130, 1031, 9000]), (40, 5000), (20, 3000)])
def test_fp8_latents_and_window(B, n_raw):
    # e4m3 latent and window rows with fp32 row scales: 6 queries (key splits, two head
    # sets), 20 queries (key splits, one head set), 40 queries (two head sets), pruning and
    # tiny contexts
    wl = W.make_decode(B=B, n_raw=n_raw, ratio=2, key_dtype="fp8", kv_dtype="fp8",
                       name=f"fp8kv-{B}", seed=41)
    _e2e(wl)


@pytest.mark.parametrize("B,n_raw", [(6, [40006, 3001, 2, 130, 1031, 9000]), (40, 5000)])
def test_mxfp4_latents_fp8_window(B, n_raw):
    # MXFP4 latent rows (E8M0 scale per 32 elements) with e4m3 window rows: key splits, two
    # head sets, pruning and tiny contexts
    wl = W.make_decode(B=B, n_raw=n_raw, ratio=2, key_dtype="fp8", kv_dtype="mxfp4",
                       name=f"fp4kv-{B}", seed=43)
    _e2e(wl)


def test_mxfp4_latents_prefill_chunk():
    wl = W.make_prefill(T=150, offset=3000, ratio=1, key_dtype="bf16", name="fp4kv-prefill", seed=44)
    import workloads as Wm
    C, CS = Wm.normal_mxfp4_rows(44, "C", 0, wl.nc_cap, 512)
    R, RS = Wm.normal_e4m3_rows(44, "R", 0, wl.wcap, 512)
    wl.C, wl.R, wl.CS, wl.RS, wl.kv_dtype = C[None], R[None], CS[None], RS[None], "mxfp4"
    _e2e(wl)


def test_fp8_latents_prefill_chunk():
    # one work-group per query (150 queries), ratio 1
    wl = W.make_prefill(T=150, offset=3000, ratio=1, key_dtype="bf16", name="fp8kv-prefill", seed=42)
    import workloads as Wm
    C, CS = Wm.normal_e4m3_rows(42, "C", 0, wl.nc_cap, 512)
    R, RS = Wm.normal_e4m3_rows(42, "R", 0, wl.wcap, 512)
    wl.C, wl.R, wl.CS, wl.RS, wl.kv_dtype = C[None], R[None], CS[None], RS[None], "fp8"
    _e2e(wl)


def test_decode_tiny_contexts():
    # n = 0 (window only), 1, 1, 8, 65 visible compressed latents
    wl = W.make_decode(B=5, n_raw=[1, 2, 3, 17, 130], ratio=2, key_dtype="bf16", name="tiny",
                       with_compress=False, seed=7)
    d, res = _e2e(wl)
    assert np.all(d.topk[0].cpu().numpy() == -1)


def test_decode_uniform_with_compressor_ratio2_small():
    wl = W.make_decode(B=6, n_raw=1234, ratio=2, key_dtype="fp8", name="compress-step", seed=9)
    d, res = _e2e(wl)
    # the compressed row written this step matches the oracle within one bf16 ulp
    n = 617
    got = d.C[:, n - 1].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    for b in range(6):
        ref = res.C_new[b][0]
        g = O.bf16_to_f64(got[b])
        x = O.bf16_to_f64(wl.Xp[b])
        assert np.all(np.abs(g - ref) <= compress_tol(ref, x[0], x[1])), b


def test_attention_late_dominant_keys():
    """For two heads, window rows (the last keys of the list) score ~100 log2 units above the
    selected latents of the first step: past the range a single pass accepts, so the kernel
    must redo the query against the true maximum. Those heads' outputs are then a softmax
    mixture of the window rows only (all entries near 0.5)."""
    wl = W.make_decode(B=2, n_raw=[4000, 3000], ratio=2, key_dtype="bf16", name="late-dominant",
                       with_compress=False, seed=15)
    rng = np.random.default_rng(15)
    wl.R[...] = O.f64_to_bf16(0.5 + 0.25 * rng.standard_normal(wl.R.shape))
    # only heads 5 and 37 are dominated by the window: the redo decision must look at every
    # head, not one per lane group or wave
    wl.q[:, [5, 37], :] = O.f64_to_bf16(np.full((wl.T, 2, wl.q.shape[2]), 8.0))
    # logits near 100 (natural units): fp32 accumulation of 512 products of size ~4 moves
    # them by ~1e-4, so lse is held to a tolerance relative to that magnitude
    d, res = _e2e(wl, lse_tol=LSE_TOL * 10)
    o = bf16_dev_to_f64(d.out)[:, [5, 37], :]
    assert np.all(o > -0.5) and np.all(o < 1.5), "output must be the window rows' mixture"
    # the same with one work-group per query (a small batch otherwise splits the key list,
    # and the window rows then sit at the start of the last split)
    topk = d.topk.cpu().numpy()
    res2 = O.run(wl, idx_override=[topk[t][topk[t] >= 0] for t in range(wl.T)])
    d.attend(split=False)
    torch.cuda.synchronize()
    o1, lse1 = bf16_dev_to_f64(d.out), d.lse.cpu().numpy()
    for t in range(wl.T):
        check_outputs(o1[t], res2.o[t], f"one group t={t}")
        assert np.abs(lse1[t] - res2.lse[t]).max() <= LSE_TOL * 10


def test_attention_large_batch_redo_and_invalid():
    """A batch of 600 short-context queries (one work-group per query, window rows first in
    the key list; key lists of 1 to 20 steps): every 7th has two heads dominated by its window
    rows (the redo pass), and every 50th is invalid (raw position -1: zero output, lse =
    -inf, between valid ones)."""
    rng = np.random.default_rng(83)
    B = 600
    n_raw = [int(x) for x in rng.integers(3, 1500, size=B)]
    wl = W.make_decode(B=B, n_raw=n_raw, ratio=2, key_dtype="bf16", name="large-batch",
                       with_compress=False, seed=83)
    dom = np.arange(0, B, 7)
    wl.R[dom] = O.f64_to_bf16(0.5 + 0.25 * rng.standard_normal(wl.R[dom].shape))
    for h in (5, 37):
        wl.q[dom, h, :] = O.f64_to_bf16(np.full((len(dom), wl.q.shape[2]), 8.0))
    bad = np.arange(3, B, 50)
    wl.pos[bad] = -1
    d = _run(wl)
    good = [t for t in range(B) if t not in set(bad.tolist())]
    topk = d.topk.cpu().numpy()
    res = O.run(wl, queries=good, idx_override={t: topk[t][topk[t] >= 0] for t in good})
    o = bf16_dev_to_f64(d.out)
    lse = d.lse.cpu().numpy()
    for t in good:
        check_outputs(o[t], res.o[t], f"large batch t={t}")
        assert np.abs(lse[t] - res.lse[t]).max() <= LSE_TOL * 10, f"t={t} lse"
    for t in bad:
        assert np.all(o[t] == 0) and np.all(np.isneginf(lse[t])), f"invalid query {t}"
    dd = o[dom][:, [5, 37], :]
    assert np.all(dd > -0.5) and np.all(dd < 1.5), "dominated heads must be the window rows' mixture"


def test_attention_key_splits_match_one_group_per_query():
    """A small batch spreads each query's key list over several work-groups and the last
    to finish combines their partial softmax results: the same output as one work-group per
    query up to fp32 summation order. Includes queries with fewer steps than splits (empty
    splits). The per-query counters reset themselves: a second call with other queries
    must be combined as well (a stale count would leave the first call's output)."""
    from sparse_attention_score_amd.step import DeviceBatch
    wl = W.make_decode(B=8, n_raw=[6000, 100, 1400, 40000, 3, 3000, 18000, 128], ratio=2,
                       key_dtype="bf16", name="splits", with_compress=False, seed=71)
    print(f"[case] {wl.name} T={wl.T}", flush=True)
    d = DeviceBatch(wl)
    d.index()
    d.select()
    topk = d.topk.cpu().numpy()
    sel = [topk[t][topk[t] >= 0] for t in range(wl.T)]
    for it, scale in enumerate((1.0, -0.75)):
        if it:
            d.q.mul_(scale)
            wl.q = d.q.cpu().contiguous().view(torch.int16).numpy().view(np.uint16).reshape(wl.q.shape)
        d.attend()
        torch.cuda.synchronize()
        o_s, l_s = bf16_dev_to_f64(d.out), d.lse.cpu().numpy()
        d.attend(split=False)
        torch.cuda.synchronize()
        o_1, l_1 = bf16_dev_to_f64(d.out), d.lse.cpu().numpy()
        # the probabilities enter the value products as bf16 relative to each group's own
        # reference, so the two paths differ by that rounding (well inside the oracle bar)
        mx, mn = check_outputs(o_s, o_1, f"call {it}: split vs one group")
        print(f"split vs one group: max {mx:.3g} mean {mn:.3g}", flush=True)
        assert np.abs(l_s - l_1).max() <= 1e-5, f"call {it}: lse"
        res = O.run(wl, idx_override=sel)
        for t in range(wl.T):
            check_outputs(o_s[t], res.o[t], f"split t={t} call {it}")
            assert np.abs(l_s[t] - res.lse[t]).max() <= LSE_TOL


@pytest.mark.parametrize("B", [17, 32])
def test_attention_key_splits_one_head_set(B):
    """17 to 32 queries: each key list is spread over four work-groups that hold all 64
    heads (one head set); the last to finish combines the four partials of every head."""
    rng = np.random.default_rng(85 + B)
    n_raw = [int(x) for x in rng.integers(3, 6000, size=B)]
    n_raw[0] = 2   # a one-key list beside longer ones
    wl = W.make_decode(B=B, n_raw=n_raw, ratio=2, key_dtype="bf16", name=f"splits-{B}",
                       with_compress=False, seed=85 + B)
    _e2e(wl)


def test_attention_head_sets():
    """33 to 128 queries: each query's heads are split over two work-groups (32 heads each).
    Ragged contexts, both key dtypes' paths share this kernel; bf16 keys here."""
    rng = np.random.default_rng(81)
    n_raw = [int(x) for x in rng.integers(3, 4000, size=36)]
    wl = W.make_decode(B=36, n_raw=n_raw, ratio=2, key_dtype="bf16", name="head-sets",
                       with_compress=False, seed=81)
    _e2e(wl)


def test_prefill_small_ratio1():
    wl = W.make_prefill(T=200, offset=900, ratio=1, key_dtype="bf16", name="prefill-small", seed=11)
    _e2e(wl)


def test_prefill_from_position_zero():
    # more than 128 queries (one work-group per query, window first in the key list) from
    # raw position 0: short windows (fewer than one step of rows for the first 31 queries),
    # key lists of one step, every visible latent selected, then the full window
    _e2e(W.make_prefill(T=300, offset=0, ratio=1, key_dtype="bf16", name="prefill-from-zero", seed=19))
    _e2e(W.make_prefill(T=160, offset=5, ratio=2, key_dtype="bf16", name="prefill-from-five-r2", seed=21))


def test_prefill_prunes_ratio1():
    wl = W.make_prefill(T=40, offset=20000, ratio=1, key_dtype="bf16", name="prefill-prune", seed=12)
    _e2e(wl)


def test_prefill_fp8_ratio2():
    wl = W.make_prefill(T=70, offset=3001, ratio=2, key_dtype="fp8", name="prefill-fp8-r2", seed=13)
    _e2e(wl)


# ------------------------------------------------------------------ stage isolated

def test_select_exact_on_given_scores_with_ties():
    """Selection fed fixed fp32 scores (many exact ties) must equal the oracle's selection on
    the same fp32 values exactly: this is integer work."""
    from sparse_attention_score_amd.step import DeviceBatch
    rng = np.random.default_rng(21)
    wl = W.make_decode(B=4, n_raw=[2 * 20003, 2 * 9000, 2 * 700, 2 * 60000], ratio=2,
                       name="select-ties", with_compress=False, seed=21)
    d = DeviceBatch(wl)
    n = wl.visible()
    S = np.full((wl.T, d.scores.shape[1]), -np.inf, np.float32)
    for t in range(wl.T):
        S[t, :n[t]] = rng.integers(0, 50, n[t]).astype(np.float32) * np.float32(0.25)
    d.scores.copy_(torch.from_numpy(S))
    for use_bm in (False, True):
        if use_bm:
            bm = np.full(d.block_max.shape, -np.inf, np.float32)
            for t in range(wl.T):
                bm[t, :-(-n[t] // 8)] = O.block_scores(S[t, :n[t]].astype(np.float64))
            d.block_max.copy_(torch.from_numpy(bm))
        d.select(use_block_max=use_bm)
        torch.cuda.synchronize()
        topk, cand = d.topk.cpu().numpy(), d.cand.cpu().numpy()
        for t in range(wl.T):
            c_ref, i_ref = O.select(S[t, :n[t]].astype(np.float64))
            assert np.array_equal(topk[t][topk[t] >= 0], i_ref), t
            assert np.array_equal(cand[t][cand[t] >= 0], c_ref), t


@pytest.mark.parametrize("T,n_lo,n_hi", [(1040, 16500, 24000), (300, 16500, 60000), (6, 66000, 140000),
                                         (520, 66000, 70000)])
def test_select_many_queries_and_long_rows(T, n_lo, n_hi):
    """Selection alone on given fp32 scores with ties: 1040 queries (the small-work-group
    kernels used for large batches), 300 queries (one large work-group per query doing both
    stages), and rows past 65536 positions (the two-level candidate stage, with few and with
    many queries), against the oracle's selection on the same values; exact integer
    results."""
    rng = np.random.default_rng(23 + T)
    n = rng.integers(n_lo, n_hi, T)
    n[0] = n_hi   # one row at the maximum
    _select_given_scores(n, rng, levels=200)


@pytest.mark.parametrize("rows,levels", [
    # parts of 8192 blocks: a last part of 13 blocks (100 positions, all kept), of 300 blocks
    # (2400 positions, every block a core block), of 500 blocks, and a long row
    ([65636, 67936, 135072, 300000], 200),
    # parts of 16384 blocks (rows past 65536 blocks): a last part of 2 blocks, the longest rows
    ([524304, 700000, 1 << 20], 200),
    # every score equal: the lowest positions and blocks win in every part and overall
    ([70000, 200000], 1),
])
def test_select_two_level_edges(rows, levels):
    """The two-level selection's part boundaries: parts whose visible positions are at most
    512, parts of at most 512 blocks, 16384-block parts, and all-equal scores; exact against
    the oracle's selection on the same fp32 values."""
    rng = np.random.default_rng(len(rows) + levels)
    _select_given_scores(np.array(rows, np.int64), rng, levels=levels, every=True)


def _select_given_scores(n, rng, levels, every=False):
    from sparse_attention_score_amd import Plan, Queries, select_topk
    T = len(n)
    E = int(-(-n.max() // 8) * 8)
    plan = Plan(ratio=1, max_queries=T, max_compressed=int(n.max()))
    seq = torch.zeros(T, dtype=torch.int32, device="cuda")
    pos = torch.from_numpy((n - 1).astype(np.int32)).cuda()
    qs = Queries(seq, pos, int(n.max()))
    S = np.full((T, E), -np.inf, np.float32)
    for t in range(T):
        S[t, :n[t]] = rng.integers(0, levels, n[t]).astype(np.float32) * np.float32(0.5)
    scores = torch.from_numpy(S).cuda()
    bm_np = np.full((T, (E // 8 + 3) // 4 * 4), -np.inf, np.float32)
    for t in range(T):
        nb = -(-int(n[t]) // 8)
        pad = np.full(nb * 8, -np.inf, np.float32)
        pad[:n[t]] = S[t, :n[t]]
        bm_np[t, :nb] = pad.reshape(nb, 8).max(axis=1)
    block_max = torch.from_numpy(bm_np).cuda()
    topk = torch.empty((T, 512), dtype=torch.int32, device="cuda")
    cand = torch.empty((T, 2048), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(16, plan.workspace_bytes), dtype=torch.uint8, device="cuda")
    print(f"[case] select T={T} n={n.min()}..{n.max()} workspace={plan.workspace_bytes}", flush=True)
    for use_bm in (True, False):
        select_topk(plan, qs, scores, block_max if use_bm else None, topk, cand=cand, workspace=ws)
        torch.cuda.synchronize()
        tk, cd = topk.cpu().numpy(), cand.cpu().numpy()
        for t in range(0, T, 1 if every else max(1, T // 40)):
            c_ref, i_ref = O.select(S[t, :n[t]].astype(np.float64))
            assert np.array_equal(tk[t][tk[t] >= 0], i_ref), (use_bm, t)
            assert np.array_equal(cd[t][cd[t] >= 0], c_ref), (use_bm, t)


def test_select_all_ties_takes_lowest():
    from sparse_attention_score_amd.step import DeviceBatch
    wl = W.make_decode(B=2, n_raw=[2 * 30000, 2 * 300], ratio=2, name="zero-w", with_compress=False, seed=2)
    wl.w[:] = 0.0
    d = DeviceBatch(wl)
    d.index()
    d.select()
    torch.cuda.synchronize()
    assert np.all(d.scores[0, :30000].cpu().numpy() == 0.0)
    assert d.topk[0].cpu().numpy().tolist() == list(range(512))
    assert d.cand[0].cpu().numpy().tolist() == list(range(2048))
    assert d.topk[1].cpu().numpy().tolist() == list(range(300)) + [-1] * 212


def test_attention_stage_isolated_and_permutation():
    """K4 fed the oracle's selection, then the same selection reversed (order must not matter)."""
    wl = W.make_decode(B=3, n_raw=[2 * 5000, 2 * 40, 2 * 3000 + 1], ratio=2, key_dtype="bf16",
                       name="attn-iso", with_compress=False, seed=31)
    res = O.run(wl)
    from sparse_attention_score_amd.step import DeviceBatch
    d = DeviceBatch(wl)
    tk = np.full((wl.T, 512), -1, np.int32)
    for t in range(wl.T):
        tk[t, :len(res.idx[t])] = res.idx[t]
    for order in ("asc", "rev"):
        tt = tk.copy()
        if order == "rev":
            for t in range(wl.T):
                m = int((tt[t] >= 0).sum())
                tt[t, :m] = tt[t, :m][::-1]
        d.attend(topk=torch.from_numpy(tt).cuda())
        torch.cuda.synchronize()
        o = bf16_dev_to_f64(d.out)
        lse = d.lse.cpu().numpy()
        for t in range(wl.T):
            check_outputs(o[t], res.o[t], f"iso t={t} {order}")
            assert np.abs(lse[t] - res.lse[t]).max() <= LSE_TOL


def test_attention_window_edges_and_dominant_key():
    """Make one window row dominate every head (+~30 logit); it must be attended when it
    is at p-127 and not when it is at p-128 (window_cap 256 so the rows do not alias)."""
    from sparse_attention_score_amd.step import DeviceBatch
    B = 2
    wl = W.make_decode(B=B, n_raw=1000, ratio=2, key_dtype="bf16", name="edges",
                       with_compress=False, wcap=256, seed=41)
    p = 999
    rng = np.random.default_rng(41)
    for b, u in enumerate((p - 127, p - 128)):
        v = np.zeros(512)
        v[:8] = 4.0
        wl.R[b, u % 256] = O.f64_to_bf16(v)
        qv = np.zeros((64, 512))
        qv[:, :8] = 30.0 / (O.SCALE * 4.0 * 8)
        wl.q[b] = O.f64_to_bf16(qv)
    res = O.run(wl)
    d = _run(wl)
    o = bf16_dev_to_f64(d.out)
    for b in range(B):
        check_outputs(o[b], res.o[b], f"edge b={b}")
    assert np.allclose(o[0][:, :8], 4.0, atol=1e-2)        # dominated by the p-127 row
    assert not np.allclose(o[1][:, :8], 4.0, atol=0.5)     # p-128 row is outside the window


def test_compress_standalone_one_ulp():
    from sparse_attention_score_amd import Plan, sparse_attn_compress
    from sparse_attention_score_amd.step import to_device_bf16
    X, Z, beta = W.make_compress_input(B=3, n_raw=2 * 777, seed=51)
    big = O.f64_to_bf16(np.full(512, 60.0))
    Z[0, 0], Z[0, 1] = big, big ^ 0x8000       # gate gap of +120: slot 0 only
    Z[0, 2], Z[0, 3] = big ^ 0x8000, big       # gap of -120: slot 1 only
    plan = Plan(ratio=2, max_queries=1, max_compressed=1)
    Xd, Zd = to_device_bf16(X), to_device_bf16(Z)
    bd = torch.from_numpy(beta).cuda()
    out = torch.empty((3, 777, 512), dtype=torch.bfloat16, device="cuda")
    sparse_attn_compress(plan, Xd, 1024, Zd, 1024, bd, out, 512, 3 * 777)
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(out).reshape(-1, 512)
    ref = O.compress(O.bf16_to_f64(X).reshape(-1, 2, 512), O.bf16_to_f64(Z).reshape(-1, 2, 512), beta)
    err = np.abs(got - ref)
    xs = O.bf16_to_f64(X).reshape(-1, 2, 512)
    tol = compress_tol(ref, xs[:, 0], xs[:, 1])
    assert np.all(err <= tol), f"max err/tol {np.max(err / tol):.3f}"
    # away from cancellation the result is within one bf16 ulp
    far = np.abs(ref) > 0.25 * (np.abs(xs[:, 0]) + np.abs(xs[:, 1]))
    assert np.all(err[far] <= bf16_ulp(ref[far]))
    # ratio 1 is the identity copy
    plan1 = Plan(ratio=1, max_queries=1, max_compressed=1)
    out1 = torch.empty((3 * 777, 512), dtype=torch.bfloat16, device="cuda")
    sparse_attn_compress(plan1, Xd, 512, None, 0, None, out1, 512, 3 * 777)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16).cpu(), Xd.reshape(-1, 512)[:3 * 777].view(torch.int16).cpu())


def _grid_step(ref, table):
    """Spacing of the code grid (ascending non-negative values `table`) at |ref|."""
    i = np.clip(np.searchsorted(table, np.abs(ref), side="right"), 1, len(table) - 1)
    return table[i] - table[i - 1]


@pytest.mark.parametrize("kv", ["fp8", "mxfp4"])
def test_compress_codes_against_oracle(kv):
    # the compressor writing e4m3 (row scale) or MXFP4 (block scales) code rows: 2331 groups,
    # one all-zero, one with a zero block, one with a huge dynamic range
    from sparse_attention_score_amd import Plan, sparse_attn_compress_codes
    from sparse_attention_score_amd.step import to_device_bf16
    X, Z, beta = W.make_compress_input(B=3, n_raw=2 * 777, seed=52)
    X = X.reshape(-1, 2, 512)
    Z = Z.reshape(-1, 2, 512)
    X[0] = 0
    X[1, :, 64:96] = 0
    X[2, :, :256] = O.f64_to_bf16(O.bf16_to_f64(X[2, :, :256]) * 2.0 ** -40)
    G = X.shape[0]
    fp4 = kv == "mxfp4"
    plan = Plan(ratio=2, max_queries=1, max_compressed=1, kv_dtype=kv)
    Xd, Zd = to_device_bf16(X), to_device_bf16(Z)
    bd = torch.from_numpy(beta).cuda()
    rb = 256 if fp4 else 512
    out = torch.full((G, rb), 0xAB, dtype=torch.uint8, device="cuda")
    sc = (torch.full((G, 16), 0xAB, dtype=torch.uint8, device="cuda") if fp4
          else torch.full((G,), float("nan"), dtype=torch.float32, device="cuda"))
    sparse_attn_compress_codes(plan, Xd, 1024, Zd, 1024, bd, out, rb, sc, 16 if fp4 else 4, G)
    torch.cuda.synchronize()
    codes, scales = out.cpu().numpy(), sc.cpu().numpy()
    ref = O.compress(O.bf16_to_f64(X), O.bf16_to_f64(Z), beta)
    xs = O.bf16_to_f64(X)
    slack = 1e-5 * (np.abs(xs[:, 0]) + np.abs(xs[:, 1])) + 1e-30   # fp32 arithmetic vs fp64
    if fp4:
        rc, rs = O.quantize_mxfp4_rows(ref)
        dec = O.mxfp4_to_f64(codes, scales)
        step = _grid_step(ref / np.repeat(2.0 ** (rs.astype(np.int64) - 127), 32, axis=1), O.E2M1_TABLE[:8])
        unit = np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=1)
        # block exponents agree unless the block's amax sits at a power of two
        amax = np.abs(ref).reshape(G, 16, 32).max(axis=2)
        frac = amax / 2.0 ** np.floor(np.log2(np.maximum(amax, 1e-300)))
        edge = (frac - 1 < 1e-5) | (2 - frac < 2e-5)
        assert np.all((scales == rs) | edge), "block exponents"
        assert scales[0].tolist() == [0] * 16 and scales[1, 2] == 0 and not np.any(codes[0])
        keep = np.repeat(~edge | (amax == 0), 32, axis=1)
        # values past 6 x 2^X saturate to 6 x 2^X (the MX scale rule leaves |x| 2^-X < 8)
        y = np.abs(ref) / np.repeat(2.0 ** (rs.astype(np.int64) - 127), 32, axis=1)
        sat = np.maximum(y - 6, 0)
    else:
        rc, rs = O.quantize_e4m3_rows(ref)
        dec = O.kv_rows_f64(codes, scales)
        assert np.all(np.abs(scales - rs) <= 1e-6 * rs), "row scales"
        assert scales[0] == 1.0 and not np.any(codes[0])
        step = _grid_step(ref / rs[:, None].astype(np.float64), O.E4M3_TABLE[:0x7F])
        unit = scales[:, None].astype(np.float64)
        keep = np.ones_like(ref, dtype=bool)
        sat = np.zeros_like(ref)
    # every element within half a grid step (plus the fp32 slack) of the exact value; codes
    # equal the oracle's but for the few values on a rounding boundary
    err = np.abs(dec - ref)
    bound = np.maximum(0.5 * step, sat) * unit * (1 + 1e-5) + slack
    assert np.all((err <= bound)[keep]), f"max {np.max((err / bound)[keep]):.3f}"
    same = np.mean(codes == rc)
    print(f"[compress-codes {kv}] code bytes equal to the oracle's: {same:.6f}", flush=True)
    assert same > 0.999
    # ratio 1 quantises the raw rows themselves (exact bf16 values): bit for bit the oracle's
    plan1 = Plan(ratio=1, max_queries=1, max_compressed=1, kv_dtype=kv)
    out1 = torch.empty((2 * G, rb), dtype=torch.uint8, device="cuda")
    sc1 = (torch.empty((2 * G, 16), dtype=torch.uint8, device="cuda") if fp4
           else torch.empty((2 * G,), dtype=torch.float32, device="cuda"))
    sparse_attn_compress_codes(plan1, Xd, 512, None, 0, None, out1, rb, sc1, 16 if fp4 else 4, 2 * G)
    torch.cuda.synchronize()
    raw = O.bf16_to_f64(X).reshape(2 * G, 512)
    rc1, rs1 = O.quantize_mxfp4_rows(raw) if fp4 else O.quantize_e4m3_rows(raw)
    assert np.array_equal(out1.cpu().numpy(), rc1) and np.array_equal(sc1.cpu().numpy(), rs1)


@pytest.mark.parametrize("kv", ["fp8", "mxfp4"])
def test_decode_step_with_code_row_compressor(kv):
    # the whole step on code-row stores: the compressor writes each sequence's new latent as
    # codes and scales, then indexer, selection and attention run (40 queries at raw position
    # 9001, each completing a group)
    wl = W.make_decode(B=40, n_raw=9002, ratio=2, key_dtype="fp8", kv_dtype=kv, compress_codes=True,
                       name=f"compress-{kv}", seed=53)
    d, res = _e2e(wl)
    n = 4501
    for b in range(40):
        v, (rc, rs) = res.C_new[b]
        got_c = d.C[b, n - 1].cpu().numpy()
        got_s = d.CS[b, n - 1].cpu().numpy()
        dec = O.kv_rows_f64(got_c[None], got_s[None])[0]
        ref = O.kv_rows_f64(rc[None], rs[None])[0]
        assert np.mean(got_c == rc) > 0.99, b
        assert np.abs(dec - v).max() <= np.abs(ref - v).max() * 1.5 + 1e-6 * np.abs(v).max(), b


def test_deterministic_bitwise():
    wl = W.make_decode(B=3, n_raw=2 * 20003, ratio=2, key_dtype="fp8", name="determinism", seed=61)
    d = _run(wl)
    a = (d.scores.clone(), d.topk.clone(), d.out.clone(), d.lse.clone())
    d.run()
    torch.cuda.synchronize()
    assert torch.equal(a[0], d.scores) and torch.equal(a[1], d.topk)
    assert torch.equal(a[2].view(torch.int16), d.out.view(torch.int16)) and torch.equal(a[3], d.lse)
