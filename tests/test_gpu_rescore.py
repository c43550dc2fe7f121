"""Candidate-bounded re-scoring (indexer_score_cand + select_topk_cand) against the fp64
oracle's rescore_select, and against the two-stage path when the carried set is the
query's own candidate set. For decode batches (one query per sequence) the two-stage path
scores with the same per-query kernel, so the scores and the selection must then be
identical, bit for bit: the same keys go through the same arithmetic, and the candidate
blocks hold the 512 best positions."""
import numpy as np
import pytest
import torch

import sparse_attention_score_amd as S
import workloads as W
from oracle import oracle as O
from parity_util import SCORE_REL, TIE_BAND, kth_score

pytestmark = pytest.mark.gpu

CAND = 2048
SLOT_E = CAND * 8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"


def _batch(wl):
    from sparse_attention_score_amd.step import DeviceBatch
    print(f"[case] {wl.name} T={wl.T} keys={wl.key_dtype} "
          f"n={wl.visible().min()}..{wl.visible().max()}", flush=True)
    return DeviceBatch(wl)


def _rescore(d, cand):
    """Run both candidate-mode calls on carried sets `cand` (device int32 [T][2048])."""
    T = d.T
    scores = torch.empty((T, SLOT_E + 4), dtype=torch.float32, device="cuda")
    bm = torch.empty((T, CAND + 4), dtype=torch.float32, device="cuda")
    topk = torch.empty((T, 512), dtype=torch.int32, device="cuda")
    S.indexer_score_cand(d.plan, d.queries, d.cache, d.qI, d.w, cand, scores, bm)
    S.select_topk_cand(d.plan, d.queries, cand, scores, bm, topk)
    torch.cuda.synchronize()
    return scores.cpu().numpy()[:, :SLOT_E], bm.cpu().numpy()[:, :CAND], topk.cpu().numpy()


def _slot_positions(row, n):
    """Position of every slot entry (8i + r -> 8 row[i] + r), -1 where the slot is empty
    or the position is not visible."""
    ids = row.astype(np.int64)
    p = ids[:, None] * 8 + np.arange(8)[None, :]
    ok = (ids[:, None] >= 0) & (ids[:, None] < (n + 7) // 8) & (p < n)
    return np.where(ok, p, -1).reshape(-1)


def _check_query(wl, t, cand_row, sc, bm, tk, keys):
    n = int(wl.visible()[t])
    pos, I, ref = O.rescore_select(O.bf16_to_f64(wl.qI[t]), wl.w[t], keys, cand_row, n)
    sp = _slot_positions(cand_row, n)
    # scores: visible entries of valid slots within SCORE_REL of the oracle, the rest -inf
    live = sp >= 0
    assert np.all(np.isneginf(sc[~live])), f"t={t}: empty entries not -inf"
    if pos.size:
        Ik = kth_score(I, 512)
        ref_at = np.full(n, np.nan)
        ref_at[pos] = I
        want = ref_at[sp[live]]
        err = np.abs(sc[live].astype(np.float64) - want)
        tol = SCORE_REL * np.maximum(np.abs(want), abs(Ik))
        assert np.all(err <= tol + 1e-30), f"t={t}: score err {err.max():.3g}"
    # slot maxima equal the max of the slot's own entries, bit for bit
    assert np.array_equal(bm, sc.reshape(CAND, 8).max(axis=1)), f"t={t}: block_max"
    # selection: the oracle's top-min(512, m) of the candidate positions, within the tie band
    k = min(512, pos.size)
    assert np.all(tk[k:] == -1), f"t={t}: padding"
    sel = tk[:k].astype(np.int64)
    assert np.all(np.diff(sel) > 0), f"t={t}: not ascending"
    assert np.all(np.isin(sel, pos)), f"t={t}: a selected position is not a candidate"
    diff = np.setxor1d(sel, ref)
    if diff.size:
        ref_at = np.full(n, np.nan)
        ref_at[pos] = I
        Ik = kth_score(I, 512)
        bad = diff[np.abs(ref_at[diff] - Ik) > TIE_BAND * abs(Ik)]
        assert bad.size == 0, f"t={t}: {bad.size} positions outside the tie band"


def _keys(wl, b, n):
    return O.index_keys_f64(wl.KI[b, :n], None if wl.KS is None else wl.KS[b, :n])


def _random_sets(rng, n_per_query, sizes):
    """Ascending random block-id sets, -1 padded; a size of -1 means every block id up to
    two past the last visible one (a set reaching past the visible blocks)."""
    rows = np.full((len(n_per_query), CAND), -1, np.int32)
    for t, (n, m) in enumerate(zip(n_per_query, sizes)):
        nb = (int(n) + 7) // 8 + 2
        m = nb if m < 0 else min(m, nb)
        m = min(m, CAND)
        ids = np.sort(rng.choice(nb, size=m, replace=False)) if m else np.zeros(0, np.int64)
        rows[t, :m] = ids
    return rows


@pytest.mark.parametrize("kd", ["bf16", "fp8", "mxfp4"])
def test_rescore_own_candidates_match_two_stage(kd):
    # n = 20003 (2501 blocks, 2048 carried), 1500, 65000 (8125 blocks), 9
    wl = W.make_decode(B=4, n_raw=[40006, 3000, 130001, 18], ratio=2, key_dtype=kd,
                       name=f"rescore-own-{kd}", with_compress=False, seed=21)
    d = _batch(wl)
    d.index()
    d.select()
    torch.cuda.synchronize()
    sc, bm, tk = _rescore(d, d.cand)
    full = d.scores.cpu().numpy()
    cand = d.cand.cpu().numpy()
    topk = d.topk.cpu().numpy()
    for t in range(wl.T):
        n = int(wl.visible()[t])
        sp = _slot_positions(cand[t], n)
        live = sp >= 0
        assert np.array_equal(sc[t][live].view(np.uint32), full[t][sp[live]].view(np.uint32)), t
        assert np.all(np.isneginf(sc[t][~live])), t
        assert np.array_equal(tk[t], topk[t]), f"t={t}: selection differs from the two-stage path"
    # and one query against the oracle
    t = 0
    _check_query(wl, t, cand[t], sc[t], bm[t], tk[t], _keys(wl, int(wl.seq[t]), int(wl.visible()[t])))


@pytest.mark.parametrize("kd", ["bf16", "fp8", "mxfp4"])
def test_rescore_carried_sets_vs_oracle(kd):
    # carried sets from another layer: random block subsets of every size class, including
    # blocks past the visible ones and more than 512 slots (the slot pre-selection runs)
    n_raw = [40006, 40006, 40006, 9000, 5000, 801, 130]
    sizes = [2048, 700, 513, -1, 64, -1, 3]
    wl = W.make_decode(B=len(n_raw), n_raw=n_raw, ratio=2, key_dtype=kd,
                       name=f"rescore-carried-{kd}", with_compress=False, seed=22)
    d = _batch(wl)
    rng = np.random.default_rng(23)
    rows = _random_sets(rng, wl.visible(), sizes)
    sc, bm, tk = _rescore(d, torch.from_numpy(rows).cuda())
    for t in range(wl.T):
        n = int(wl.visible()[t])
        _check_query(wl, t, rows[t], sc[t], bm[t], tk[t], _keys(wl, int(wl.seq[t]), n))


@pytest.mark.parametrize("kd", ["fp8", "mxfp4"])
def test_rescore_edge_cases(kd):
    # n = 0 (no keys), 1, 8, 9, 17; sets: empty, ids past the visible blocks only,
    # a single partly visible block, every block, a full row of ids past the end
    wl = W.make_decode(B=6, n_raw=[1, 2, 16, 18, 34, 34], ratio=2, key_dtype=kd,
                       name=f"rescore-edges-{kd}", with_compress=False, seed=24)
    n = wl.visible()
    rows = np.full((wl.T, CAND), -1, np.int32)
    rows[0, :3] = [0, 1, 2]                 # n = 0: every slot empty
    rows[1, :2] = [0, 5]                    # n = 1: one position, then a block past the end
    rows[2, :1] = [0]                       # n = 8: one full block
    rows[3, :2] = [0, 1]                    # n = 9: the second block holds one position
    rows[4, :1] = [2]                       # n = 17: only the partly visible last block
    rows[5, :] = np.arange(10, 10 + CAND)   # n = 17: every id past the end
    d = _batch(wl)
    sc, bm, tk = _rescore(d, torch.from_numpy(rows).cuda())
    for t in range(wl.T):
        _check_query(wl, t, rows[t], sc[t], bm[t], tk[t], _keys(wl, int(wl.seq[t]), int(n[t])))
    assert np.all(tk[0] == -1) and np.all(tk[5] == -1)
    assert tk[1, 0] == 0 and np.all(tk[1, 1:] == -1)
    assert list(tk[3, :9]) == list(range(9)) and list(tk[4, :1]) == [16]


def test_rescore_many_queries_prefill():
    # a prefill chunk: 300 queries of one sequence at consecutive positions, carried sets
    # from the chunk's own candidate stage. The two-stage path scored them with the chunk
    # kernel (another summation order), so scores agree within rounding and selections
    # within the tie band of the k-th score; sampled queries are checked against the oracle.
    wl = W.make_prefill(T=300, offset=20000, ratio=1, key_dtype="bf16", name="rescore-prefill",
                        seed=25)
    d = _batch(wl)
    d.index()
    d.select()
    torch.cuda.synchronize()
    sc, bm, tk = _rescore(d, d.cand)
    full = d.scores.cpu().numpy().astype(np.float64)
    cand = d.cand.cpu().numpy()
    topk = d.topk.cpu().numpy()
    same = 0
    for t in range(wl.T):
        n = int(wl.visible()[t])
        sp = _slot_positions(cand[t], n)
        live = sp >= 0
        Ik = kth_score(full[t][:n], 512)
        ref = full[t][sp[live]]
        err = np.abs(sc[t][live] - ref)
        assert np.all(err <= 2 * SCORE_REL * np.maximum(np.abs(ref), abs(Ik))), t
        diff = np.setxor1d(tk[t][tk[t] >= 0], topk[t][topk[t] >= 0])
        assert int((tk[t] >= 0).sum()) == int((topk[t] >= 0).sum()) == min(512, n), t
        assert np.all(np.abs(full[t][diff] - Ik) <= TIE_BAND * abs(Ik)), t
        same += diff.size == 0
    print(f"[rescore-prefill] {same} of {wl.T} selections identical to the two-stage path")
    for t in (0, 151, 299):
        n = int(wl.visible()[t])
        _check_query(wl, t, cand[t], sc[t], bm[t], tk[t], _keys(wl, 0, n))


def test_rescore_rejects_bad_strides():
    wl = W.make_decode(B=2, n_raw=200, ratio=2, key_dtype="bf16", name="rescore-args",
                       with_compress=False, seed=26)
    d = _batch(wl)
    cand = torch.full((2, CAND), -1, dtype=torch.int32, device="cuda")
    small = torch.empty((2, 8 * CAND - 4), dtype=torch.float32, device="cuda")
    bm = torch.empty((2, CAND), dtype=torch.float32, device="cuda")
    with pytest.raises(S.SparseAttnError):
        S.indexer_score_cand(d.plan, d.queries, d.cache, d.qI, d.w, cand, small, bm)
    topk = torch.empty((2, 512), dtype=torch.int32, device="cuda")
    with pytest.raises(S.SparseAttnError):
        S.select_topk_cand(d.plan, d.queries, cand, small, bm, topk)
