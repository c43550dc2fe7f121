"""Pins of the fp64 oracle to things other than itself.

Each test ties one oracle function to a hand-derived worked example
(tests/golden), a library routine on a special case, a closed form, an
invariant, or the independent pure-Python brute force on tiny inputs. The set
is chosen so that a dropped term, wrong sign, wrong index or transposed
operand in any stage fails at least one test.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- formats

def test_e4m3_anchors_from_spec():
    g = _gold("e4m3_anchors.json")
    for code, val in g["anchors"]:
        v = O.e4m3_value(int(code, 16))
        assert v == val and math.copysign(1, v) == math.copysign(1, val), code
    for code in g["nan_codes"]:
        assert math.isnan(O.e4m3_value(int(code, 16)))


def test_e4m3_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])


def test_e4m3_structure():
    t = O.E4M3_TABLE
    pos = t[0x00:0x7F]
    assert np.all(np.diff(pos) > 0)                          # strictly increasing
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])       # sign symmetry
    finite = t[~np.isnan(t)]
    assert np.array_equal(finite.astype(np.float32).astype(np.float64), finite)
    assert len(np.unique(finite)) == 253                     # +-0 coincide, 2 NaNs


def test_e2m1_and_e8m0_anchors_from_spec():
    g = _gold("mxfp4_anchors.json")
    for code, val in g["e2m1"]:
        v = O.e2m1_value(code)
        assert v == val and math.copysign(1, v) == math.copysign(1, val), code
    for code, val in g["e8m0"]:
        assert O.e8m0_value(code) == val, code
    for code in g["e8m0_nan"]:
        assert math.isnan(O.e8m0_value(code))


def test_e8m0_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 1 and np.isnan(O.E8M0_TABLE[255])
    assert np.array_equal(ref[~nan], O.E8M0_TABLE[~nan])


def test_e2m1_values_are_e4m3_values():
    # every E2M1 value times a power of two in [2^-3, 2^3] is an E4M3 value (torch's
    # float8_e4m3fn table): E2M1 has one mantissa bit, E4M3 three, and a wider range
    e4 = set(torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
             .to(torch.float64).numpy().tolist())
    for k in range(-3, 4):
        for v in O.E2M1_TABLE:
            assert v * 2.0 ** k in e4, (v, k)
    t = O.E2M1_TABLE
    assert np.all(np.diff(t[:8]) > 0) and np.array_equal(t[8:], -t[:8])


def test_mxfp4_worked_row():
    g = _gold("mxfp4_anchors.json")["worked_row"]
    codes = np.zeros(64, np.uint8)
    for i, b in g["bytes"].items():
        codes[int(i)] = b
    v = O.mxfp4_to_f64(codes, np.array(g["scales"], np.uint8))
    want = np.zeros(128)
    for i, x in g["values"].items():
        want[int(i)] = x
    assert np.array_equal(v, want)


def test_mxfp4_decode_against_scalar_loops():
    # the vectorised decode (nibble split, interleave, block repeat) against one element
    # at a time from the scalar definitions
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (3, 64), dtype=np.uint8)
    scales = rng.integers(100, 150, (3, 4), dtype=np.uint8)
    v = O.mxfp4_to_f64(codes, scales)
    for r in range(3):
        for d in range(128):
            byte = int(codes[r, d // 2])
            nib = byte & 0xF if d % 2 == 0 else byte >> 4
            assert v[r, d] == O.e2m1_value(nib) * O.e8m0_value(int(scales[r, d // 32])), (r, d)


def test_mxfp4_scores_equal_bf16_scores():
    # MXFP4 keys are exact bf16 values (at most 2 significant bits times a power of two):
    # scoring the decoded keys equals scoring the same keys stored as bf16
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 256, (40, 64), dtype=np.uint8)
    scales = rng.integers(120, 132, (40, 4), dtype=np.uint8)
    k = O.mxfp4_to_f64(codes, scales)
    kb = torch.from_numpy(k).to(torch.bfloat16)
    assert np.array_equal(kb.to(torch.float64).numpy(), k)
    bits = kb.view(torch.int16).numpy().view(np.uint16)
    qI = rng.standard_normal((16, 128))
    w = rng.uniform(0, 1, 16)
    a = O.index_scores(qI, w, O.index_keys_f64(codes, scales))
    b = O.index_scores(qI, w, O.index_keys_f64(bits, None))
    assert np.array_equal(a, b)


def test_fp8_kv_rows_with_power_of_two_scales_equal_bf16_rows():
    # e4m3 latent and window rows with power-of-two row scales are exact bf16 values: the
    # attention over them equals the attention over the same rows stored as bf16
    import workloads as W
    wl8 = W.make_decode(B=2, n_raw=[1100, 90], ratio=2, key_dtype="bf16", kv_dtype="fp8", seed=3)
    wl8.CS[:] = 2.0 ** np.round(np.log2(wl8.CS))
    wl8.RS[:] = 2.0 ** np.round(np.log2(wl8.RS))
    wlb = W.make_decode(B=2, n_raw=[1100, 90], ratio=2, key_dtype="bf16", seed=3, with_compress=False)
    for b in range(2):
        cv = O.kv_rows_f64(wl8.C[b], wl8.CS[b])
        rv = O.kv_rows_f64(wl8.R[b], wl8.RS[b])
        wlb.C[b] = torch.from_numpy(cv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        wlb.R[b] = torch.from_numpy(rv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(O.bf16_to_f64(wlb.C[b]), cv) and np.array_equal(O.bf16_to_f64(wlb.R[b]), rv)
    r8, rb = O.run(wl8), O.run(wlb)
    for t in range(2):
        assert np.array_equal(r8.idx[t], rb.idx[t])
        assert np.array_equal(r8.o[t], rb.o[t]) and np.array_equal(r8.lse[t], rb.lse[t])


def test_mxfp4_latent_rows_equal_bf16_rows():
    # MXFP4 latent rows (256 bytes, 16 block scales) are exact bf16 values: the attention over
    # them (e4m3 window with power-of-two row scales) equals the attention over the same rows
    # stored as bf16. The bf16 rows are built from a per-element decode written here (E2M1
    # sign, exponent, mantissa fields; one scale per 32 elements), rounded by torch.
    import workloads as W
    wl4 = W.make_decode(B=2, n_raw=[1100, 90], ratio=2, key_dtype="bf16", kv_dtype="mxfp4", seed=4)
    wl4.RS[:] = 2.0 ** np.round(np.log2(wl4.RS))
    wlb = W.make_decode(B=2, n_raw=[1100, 90], ratio=2, key_dtype="bf16", seed=4, with_compress=False)

    def e2m1(code):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        v = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        return -v if s else v

    for b in range(2):
        codes, sc = wl4.C[b], wl4.CS[b]
        assert codes.shape == (wl4.nc_cap, 256) and sc.shape == (wl4.nc_cap, 16)
        x = np.empty((wl4.nc_cap, 512))
        for r in range(wl4.nc_cap):
            for k in range(512):
                byte = int(codes[r, k // 2])
                x[r, k] = e2m1(byte >> 4 if k % 2 else byte & 15) * 2.0 ** (int(sc[r, k // 32]) - 127)
        assert np.array_equal(O.kv_rows_f64(codes, sc), x)
        wlb.C[b] = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        rv = O.kv_rows_f64(wl4.R[b], wl4.RS[b])
        wlb.R[b] = torch.from_numpy(rv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(O.bf16_to_f64(wlb.C[b]), x) and np.array_equal(O.bf16_to_f64(wlb.R[b]), rv)
    r4, rb = O.run(wl4), O.run(wlb)
    for t in range(2):
        assert np.array_equal(r4.idx[t], rb.idx[t])
        assert np.array_equal(r4.o[t], rb.o[t]) and np.array_equal(r4.lse[t], rb.lse[t])


def test_bf16_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10 ** rng.uniform(-30, 30, 20000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 1e-40, -1e-41], np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = O.f64_to_bf16(x.astype(np.float64))
    assert np.array_equal(ref, ours)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, O.bf16_to_f64(ref))


def test_bf16_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0)
    assert O.f64_to_bf16(np.array([1.0 + 2 ** -8]))[0] == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even)
    assert O.f64_to_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 0x3F82


# ---------------------------------------------------------------- visibility, window

def test_visibility_and_window_counts():
    g = _gold("layer_shapes.json")
    for c in g["derived"]["cases"]:
        p = c["N"] - 1
        n = O.visible_count(p, c["r"])
        assert n == c["n"], c
        assert -(-n // g["block"]) == c["blocks"], c
        assert len(O.window_positions(p, g["window"])) == c["window_rows"], c
    assert (O.HEADS, O.DIM, O.WINDOW, O.TOPK, O.CAND_BLOCKS, O.BLOCK) == (
        g["heads"], g["latent_dim"], g["window"], g["topk"], g["cand_blocks"], g["block"])


def test_window_edges():
    w = O.window_positions(1000)
    assert w[0] == 1000 - 127 and w[-1] == 1000 and 1000 - 128 not in w


def test_ratio2_group_visibility():
    # group j covers raw positions 2j, 2j+1; visible only once both are <= p
    assert O.visible_count(0, 2) == 0
    assert O.visible_count(1, 2) == 1
    assert O.visible_count(2, 2) == 1
    assert O.visible_count(3, 2) == 2
    # ratio 1 includes the diagonal
    assert O.visible_count(0, 1) == 1


# ---------------------------------------------------------------- indexer

def _worked_keys(g):
    n = len(g["a"])
    keys = np.zeros((n, 128))
    keys[:, 0] = g["a"]
    keys[:, 1] = g["b"]
    qI = np.zeros((16, 128))
    qI[0, 0] = 1.0
    qI[1, 1] = -1.0
    w = np.zeros(16)
    w[:2] = g["w01"]
    return qI, w, keys


def test_worked_indexer_and_selection():
    g = _gold("worked_tiny.json")["indexer_select"]
    qI, w, keys = _worked_keys(g)
    I = O.index_scores(qI, w, keys)
    assert np.array_equal(I, np.array(g["scores"], float))
    assert np.array_equal(O.block_scores(I), np.array(g["block_max"], float))
    cand, idx = O.select(I, k=g["k"], cb=2)
    assert cand.tolist() == g["cb2"]["cand"] and idx.tolist() == g["cb2"]["idx"]
    cand, idx = O.select(I, k=g["k"], cb=3)
    assert cand.tolist() == g["cb3"]["cand"] and idx.tolist() == g["cb3"]["idx"]
    cand, idx = O.select(I)
    assert idx.tolist() == list(range(20))


def test_indexer_brute_force_tiny():
    rng = np.random.default_rng(7)
    for n in (1, 7, 8, 9, 23, 40):
        qI = rng.standard_normal((16, 128))
        w = rng.uniform(0, 1, 16)
        keys = rng.standard_normal((n, 128))
        ref = brute.scores(qI.tolist(), w.tolist(), keys.tolist())
        got = O.index_scores(qI, w, keys)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_indexer_one_hot_and_relu():
    qI = np.zeros((16, 128))
    w = np.zeros(16)
    qI[5, 17] = 2.0
    w[5] = 0.25
    keys = np.zeros((3, 128))
    keys[0, 17] = 3.0     # positive dot: 0.25 * 6
    keys[1, 17] = -3.0    # negative dot clipped to 0
    keys[2, 18] = 9.0     # orthogonal
    assert O.index_scores(qI, w, keys).tolist() == [1.5, 0.0, 0.0]


def test_indexer_head_weights_not_transposed():
    # head h uses weight w[h] and query row h: distinct values catch a swap
    qI = np.zeros((16, 128))
    for h in range(16):
        qI[h, h] = h + 1.0
    w = np.arange(16) / 16.0
    keys = np.eye(128)[:16]
    I = O.index_scores(qI, w, keys)
    assert np.allclose(I, (np.arange(16) + 1.0) * np.arange(16) / 16.0, rtol=0, atol=0)


def test_indexer_scale_homogeneity_and_zero_weights():
    rng = np.random.default_rng(3)
    qI = rng.standard_normal((16, 128))
    w = rng.uniform(0, 1, 16)
    codes = rng.integers(0, 0x7E, (50, 128)).astype(np.uint8)
    s = np.float32(0.0078125)        # a power of two keeps the product exact
    k1 = O.index_keys_f64(codes, np.full(50, s, np.float32))
    k0 = O.index_keys_f64(codes, np.ones(50, np.float32))
    assert np.array_equal(O.index_scores(qI, w, k1), float(s) * O.index_scores(qI, w, k0))
    assert np.all(O.index_scores(qI, np.zeros(16), k1) == 0.0)


# ---------------------------------------------------------------- selection

def _lemma_case(I, k, cb, blk):
    cand, idx = O.select(I, k=k, cb=cb, blk=blk)
    direct = O.topk_of(I, np.arange(I.shape[0]), k)
    assert np.array_equal(idx, direct)
    return cand, idx


def test_two_stage_equals_global_topk_random_and_ties():
    rng = np.random.default_rng(11)
    for trial in range(30):
        n = int(rng.integers(1, 3000))
        blk = int(rng.choice([1, 2, 4, 8]))
        k = int(rng.integers(1, 200))
        cb = int(rng.integers(k, k + 50))       # cb >= k: lossless
        if trial % 2:
            I = rng.integers(0, 6, n).astype(float)     # many ties
        else:
            I = rng.standard_normal(n)
        _lemma_case(I, k, cb, blk)


def test_two_stage_production_sizes():
    rng = np.random.default_rng(12)
    n = 40000                                  # 5000 blocks > 2048: the stage prunes
    I = rng.standard_normal(n)
    cand, idx = _lemma_case(I, O.TOPK, O.CAND_BLOCKS, O.BLOCK)
    assert cand.shape[0] == O.CAND_BLOCKS and idx.shape[0] == O.TOPK
    assert np.all(np.diff(idx) > 0) and np.all(np.diff(cand) > 0)


def test_selection_brute_force_tiny():
    rng = np.random.default_rng(5)
    for n in (1, 5, 8, 17, 40):
        I = rng.integers(0, 4, n).astype(float)
        for k, cb in ((3, 1), (3, 2), (5, 8), (40, 40)):
            kept_b, idx_b = brute.select(I.tolist(), k=k, cb=cb, blk=8)
            cand, idx = O.select(I, k=k, cb=cb, blk=8)
            assert cand.tolist() == kept_b and idx.tolist() == idx_b


def test_selection_all_ties_takes_lowest_positions():
    for n in (100, 511, 512, 513, 20000):
        cand, idx = O.select(np.zeros(n))
        assert idx.tolist() == list(range(min(512, n)))


def test_selection_monotone_takes_last_positions_with_partial_block():
    n = 20003                                   # last block holds 3 positions
    cand, idx = O.select(np.arange(n, dtype=float))
    assert idx.tolist() == list(range(n - 512, n))
    nb = -(-n // 8)
    assert cand.tolist() == list(range(nb - 2048, nb))


def test_selection_small_takes_everything():
    rng = np.random.default_rng(2)
    for n in (0, 1, 300, 512):
        cand, idx = O.select(rng.standard_normal(n))
        assert idx.tolist() == list(range(n))


# ---------------------------------------------------------------- candidate-bounded re-scoring

def test_rescore_own_candidates_equals_two_stage_path():
    """Re-scoring inside the query's own candidate blocks gives the two-stage path's top-512
    (the candidate-stage lemma): a wrong block-to-position map or a dropped partial block
    fails it."""
    rng = np.random.default_rng(91)
    for n in (20003, 40000):
        qI = rng.standard_normal((16, 128))
        w = rng.uniform(0, 1, 16)
        keys = rng.standard_normal((n, 128))
        I = O.index_scores(qI, w, keys)
        cand, idx = O.select(I)
        pos, Ic, sel = O.rescore_select(qI, w, keys, cand, n)
        assert np.array_equal(sel, idx)
        assert pos.shape[0] == sum(min(8, n - 8 * int(b)) for b in cand)
        assert np.array_equal(Ic, I[pos])


def test_rescore_brute_force_tiny():
    rng = np.random.default_rng(92)
    for n in (1, 7, 8, 9, 30, 61):
        nb = -(-n // 8)
        qI = rng.integers(-2, 3, (16, 128)).astype(float)
        w = rng.integers(0, 3, 16).astype(float)
        keys = rng.integers(-1, 2, (n, 128)).astype(float)   # many ties
        for trial in range(4):
            m = int(rng.integers(1, nb + 1))
            cand = np.sort(rng.choice(nb, m, replace=False))
            cand = np.concatenate([cand, -np.ones(3, np.int64)])   # -1 padding is ignored
            for k in (1, 3, 16, 512):
                _, _, sel = O.rescore_select(qI, w, keys, cand, n, k=k)
                want = brute.rescore(qI.tolist(), w.tolist(), keys.tolist(), cand.tolist(), n, k=k)
                assert sel.tolist() == want, (n, k, cand)


def test_rescore_small_set_takes_everything_and_ignores_invisible():
    rng = np.random.default_rng(93)
    n = 1000
    qI, w, keys = rng.standard_normal((16, 128)), rng.uniform(0, 1, 16), rng.standard_normal((n, 128))
    cand = np.array([3, 40, 124, 125, -1])      # block 124 holds 992..999, block 125 nothing visible
    pos, _, sel = O.rescore_select(qI, w, keys, cand, n)
    want = list(range(24, 32)) + list(range(320, 328)) + list(range(992, 1000))
    assert pos.tolist() == want and sel.tolist() == want


# ---------------------------------------------------------------- attention

def test_worked_attention():
    g = _gold("worked_tiny.json")["attention"]
    q = np.zeros((1, 512))
    q[0, 0] = math.log(2.0) / O.SCALE
    X = np.zeros((3, 512))
    X[:, 0] = [0, 1, 2]
    X[:, 1] = [0, 10, 40]
    o, lse = O.attend(q, X)
    assert abs(o[0, 0] - g["o0"]) < 1e-12 and abs(o[0, 1] - g["o1"]) < 1e-12
    assert abs(lse[0] - g["lse"]) < 1e-12


def test_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((64, 512))
    X = rng.standard_normal((300, 512))
    o, lse = O.attend(q, X)
    qt = torch.from_numpy(q)[None, :, None, :]            # [1, H, 1, D]
    kt = torch.from_numpy(X)[None, None].expand(1, 64, 300, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=O.SCALE)
    assert np.allclose(o, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)
    s = O.SCALE * (torch.from_numpy(q) @ torch.from_numpy(X).T)
    assert np.allclose(lse, torch.logsumexp(s, dim=1).numpy(), rtol=1e-13, atol=1e-13)


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((3, 16))
    X = rng.standard_normal((7, 16))
    ob, lb = brute.attend(q.tolist(), X.tolist(), 0.3)
    o, lse = O.attend(q, X, 0.3)
    assert np.allclose(o, ob, rtol=1e-12, atol=1e-13) and np.allclose(lse, lb, rtol=1e-13)


def test_attention_invariants():
    rng = np.random.default_rng(8)
    X = rng.standard_normal((640, 512))
    q = rng.standard_normal((64, 512)) * 3
    o, lse = O.attend(q, X)
    assert np.all(o <= X.max(0) + 1e-12) and np.all(o >= X.min(0) - 1e-12)   # convex hull
    perm = rng.permutation(640)
    o2, lse2 = O.attend(q, X[perm])
    assert np.allclose(o, o2, atol=1e-12) and np.allclose(lse, lse2, atol=1e-12)
    o0, l0 = O.attend(np.zeros((64, 512)), X)
    assert np.allclose(o0, X.mean(0)[None], atol=1e-12) and np.allclose(l0, math.log(640))
    o1, l1 = O.attend(q, X[:1])
    assert np.allclose(o1, X[:1], atol=0) and np.allclose(l1, O.SCALE * (q @ X[0]))
    # one key 30 nats above the rest dominates
    Y = X[:5].copy()
    Y[:, 0] = [0.0, 1.0, 0.0, 0.0, 0.0]
    qs = np.zeros((1, 512))
    qs[0, 0] = 30.0 / O.SCALE
    oo, ll = O.attend(qs, Y)
    assert np.allclose(oo[0], Y[1], atol=1e-11) and abs(ll[0] - 30.0) < 1e-11


# ---------------------------------------------------------------- compressor

def test_worked_compress():
    g = _gold("worked_tiny.json")["compress"]
    x = np.array([[[g["x"][0]], [g["x"][1]]]])
    out = O.compress(x, np.array([[[math.log(3.0)], [0.0]]]), np.zeros((2, 1)))
    assert abs(out[0, 0] - g["gap_ln3"]) < 1e-12
    out = O.compress(x, np.array([[[1.7], [1.7]]]), np.zeros((2, 1)))
    assert abs(out[0, 0] - g["equal"]) < 1e-12


def test_compress_matches_torch_softmax_and_brute():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 2, 512))
    z = rng.standard_normal((5, 2, 512)) * 4
    beta = rng.standard_normal((2, 512))
    out = O.compress(x, z, beta)
    pi = torch.softmax(torch.from_numpy(z + beta[None]), dim=1).numpy()
    assert np.allclose(out, (pi * x).sum(1), rtol=1e-13, atol=1e-13)
    for g in range(5):
        ref = brute.compress_pair(x[g, 0].tolist(), x[g, 1].tolist(), z[g, 0].tolist(),
                                  z[g, 1].tolist(), beta[0].tolist(), beta[1].tolist())
        assert np.allclose(out[g], ref, rtol=1e-13, atol=1e-13)


def test_compress_invariants():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((9, 2, 64))
    z = rng.standard_normal((9, 2, 64))
    beta = rng.standard_normal((2, 64))
    out = O.compress(x, z, beta)
    assert np.all(out <= x.max(1) + 1e-12) and np.all(out >= x.min(1) - 1e-12)
    assert np.allclose(O.compress(x, z + 5.0, beta), out, atol=1e-12)     # shift invariance
    zz = np.zeros_like(z)
    zz[:, 0] = 40.0
    assert np.allclose(O.compress(x, zz, np.zeros((2, 64))), x[:, 0], atol=1e-15)
    # slot bias is per slot: a bias on slot 1 only favours slot 1
    b1 = np.zeros((2, 64))
    b1[1] = 40.0
    assert np.allclose(O.compress(x, np.zeros_like(z), b1), x[:, 1], atol=1e-15)


# ---------------------------------------------------------------- whole path

class _TinyWL:
    """A tiny hand-built workload (no generator) for whole-path checks."""

    def __init__(self, rng, B, n_raw, ratio, fp8=False, wcap=128):
        self.ratio, self.B, self.T, self.wcap = ratio, B, B, wcap
        self.seq = np.arange(B, dtype=np.int32)
        self.pos = (np.asarray(n_raw) - 1).astype(np.int32)
        nc = max(1, int(((self.pos + 1) // ratio).max()))
        self.nc_cap = nc

        def bf(shape):
            return O.f64_to_bf16(rng.standard_normal(shape).astype(np.float32).astype(np.float64))
        self.q = bf((B, 64, 512))
        self.qI = bf((B, 16, 128))
        self.w = rng.uniform(0, 1, (B, 16)).astype(np.float32)
        self.C = bf((B, nc, 512))
        self.R = bf((B, wcap, 512))
        if fp8:
            self.KI = rng.integers(0, 0x7F, (B, nc, 128)).astype(np.uint8) | (
                rng.integers(0, 2, (B, nc, 128)).astype(np.uint8) << 7)
            self.KI[self.KI == 0xFF] = 0xFE
            self.KS = rng.uniform(0.001, 0.01, (B, nc)).astype(np.float32)
        else:
            self.KI, self.KS = bf((B, nc, 128)), None
        self.Xp = bf((B, 2, 512)) if ratio == 2 else None
        self.Zp = bf((B, 2, 512)) if ratio == 2 else None
        self.beta = rng.standard_normal((2, 512)).astype(np.float32) if ratio == 2 else None

    def compress_groups(self):
        if self.ratio != 2:
            return np.zeros(0, np.int64)
        return self.seq[((self.pos.astype(np.int64) + 1) % 2) == 0].astype(np.int64)


def test_whole_path_small_context_is_dense_attention():
    """n <= 512: everything is selected, so the output is dense attention over all
    compressed rows plus the window rows (library SDPA in fp64)."""
    rng = np.random.default_rng(20)
    wl = _TinyWL(rng, B=2, n_raw=[600, 901], ratio=2)
    res = O.run(wl)
    for t in range(2):
        b, p = int(wl.seq[t]), int(wl.pos[t])
        n = (p + 1) // 2
        assert res.idx[t].tolist() == list(range(n))
        C = O.bf16_to_f64(wl.C[b, :n])
        if (p + 1) % 2 == 0:                      # this query completes group n-1
            C[n - 1] = O.bf16_to_f64(res.C_new[b][1])
        else:
            assert b not in res.C_new
        X = np.concatenate([C, O.bf16_to_f64(wl.R[b, np.arange(p - 127, p + 1) % 128])])
        qt = torch.from_numpy(O.bf16_to_f64(wl.q[t]))[None, :, None, :]
        kt = torch.from_numpy(X)[None, None].expand(1, 64, X.shape[0], 512)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=O.SCALE)
        assert np.allclose(res.o[t], ref[0, :, 0].numpy(), atol=1e-12)


def test_whole_path_fp8_keys_equal_decoded_bf16_path():
    """An e4m3 key with a power-of-two scale is exactly a bf16 key; both stores must
    give identical scores and selections."""
    rng = np.random.default_rng(21)
    wl = _TinyWL(rng, B=1, n_raw=[3000], ratio=2, fp8=True)
    wl.KS[:] = 0.0078125
    k = O.index_keys_f64(wl.KI, wl.KS)
    wl2 = _TinyWL(np.random.default_rng(21), B=1, n_raw=[3000], ratio=2)
    wl2.qI, wl2.w = wl.qI, wl.w
    wl2.KI, wl2.KS = O.f64_to_bf16(k), None
    r1, r2 = O.run(wl), O.run(wl2)
    assert np.array_equal(r1.scores[0], r2.scores[0])
    assert np.array_equal(r1.idx[0], r2.idx[0])


def test_compressor_row_feeds_attention():
    """The compressed latent written this step is the one attention reads at n-1."""
    rng = np.random.default_rng(22)
    wl = _TinyWL(rng, B=1, n_raw=[64], ratio=2)
    res = O.run(wl)
    n = 32
    expect = O.compress(O.bf16_to_f64(wl.Xp[0])[None], O.bf16_to_f64(wl.Zp[0])[None], wl.beta)[0]
    assert np.array_equal(res.C_new[0][1], O.f64_to_bf16(expect))
    q = O.bf16_to_f64(wl.q[0])
    C = O.bf16_to_f64(wl.C[0, :n])
    C[n - 1] = O.bf16_to_f64(res.C_new[0][1])
    X = np.concatenate([C, O.bf16_to_f64(wl.R[0, np.arange(0, 64) % 128])])
    o, lse = O.attend(q, X)
    assert np.allclose(res.o[0], o, atol=0) and np.allclose(res.lse[0], lse, atol=0)


# ------------------------------------------------- quantising the compressor's output rows

def test_e4m3_row_quantiser_matches_torch_cast():
    # rows whose amax is 448 have scale 1, so the codes are the plain fp32 -> e4m3 cast, which
    # torch implements independently (nearest, ties to even); include every code's value and
    # every midpoint between neighbouring codes (ties), negative values and subnormals
    finite = O.E4M3_TABLE[:0x7F]
    mids = (finite[:-1] + finite[1:]) / 2
    rng = np.random.default_rng(5)
    vals = np.concatenate([finite, mids, rng.uniform(0, 448, 4000), 2.0 ** rng.uniform(-12, 8, 4000)])
    vals = np.concatenate([vals, -vals])
    vals = vals[: len(vals) // 511 * 511].reshape(-1, 511)
    x = np.concatenate([vals, np.full((vals.shape[0], 1), 448.0)], axis=1).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), np.asarray(x, np.float64))   # exact in fp32
    codes, s = O.quantize_e4m3_rows(x)
    assert np.all(s == 1.0)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_code_row_quantisers_match_the_input_quantisers():
    # the inputs module quantises with its own C code (same rules): rows of N(0,1) values at
    # several magnitudes, plus zero rows and blocks
    import workloads as W
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((64, 512)) * 10.0 ** rng.uniform(-20, 20, (64, 1))).astype(np.float32)
    x[3] = 0.0
    x[5, 64:96] = 0.0
    c8, s8 = O.quantize_e4m3_rows(x)
    w8, ws8 = W.quant_e4m3_rows(x)
    assert np.array_equal(c8, w8) and np.array_equal(s8, ws8)
    c4, s4 = O.quantize_mxfp4_rows(x)
    w4, ws4 = W.quant_mxfp4_rows(x)
    assert np.array_equal(c4, w4) and np.array_equal(s4, ws4)
    assert s4[3].tolist() == [0] * 16 and s4[5, 2] == 0


def test_mxfp4_row_quantiser_round_trip_and_ties():
    # every E2M1 value times a block scale encodes to itself; midpoints take the even code
    mags = O.E2M1_TABLE[:8]
    for X in (-3, 0, 5):
        blk = np.zeros(32)
        blk[:8] = mags * 2.0 ** X
        blk[8:16] = -mags * 2.0 ** X
        blk[31] = 6 * 2.0 ** X          # amax 6 * 2^X: floor(log2) - 2 = X
        c, s = O.quantize_mxfp4_rows(np.tile(blk, 16)[None])
        assert np.all(s == X + 127)
        assert np.array_equal(O.mxfp4_to_f64(c, s)[0, :32], blk)
        mid = np.zeros(32)
        mid[:7] = (mags[:-1] + mags[1:]) / 2 * 2.0 ** X
        mid[31] = 6 * 2.0 ** X
        c, s = O.quantize_mxfp4_rows(np.tile(mid, 16)[None])
        got = O.mxfp4_to_f64(c, s)[0, :7] / 2.0 ** X
        assert got.tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]   # ties to codes 0, 2, 2, 4, 4, 6, 6
