"""C-ABI checks that need no GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any HIP call.

No call here passes validation: every device pointer below is either NULL or paired
with an argument the host check refuses, so no kernel is ever launched."""
import ctypes
import os
import re

import pytest

import sparse_attention_score_amd as S

HDR = os.path.join(os.path.dirname(__file__), "..", "include", "sparse_attn.h")


def _declared():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    assert _declared() == sorted(S.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(S.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_library_exports_only_declared_symbols():
    import shutil
    import subprocess
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--defined-only", S.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    funcs = {ln.split()[-1] for ln in out.splitlines() if len(ln.split()) == 3 and ln.split()[1] == "T"}
    funcs = {f for f in funcs if not f.startswith("_")}
    assert funcs == set(_declared()), funcs ^ set(_declared())


def _plan(**kw):
    args = dict(ratio=2, key_dtype="bf16", max_queries=8, max_compressed=4096)
    args.update(kw)
    return S.Plan(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(ratio=3), S.SA_EUNSUPPORTED),
    (dict(ratio=0), S.SA_EUNSUPPORTED),
    (dict(num_heads=32), S.SA_EUNSUPPORTED),
    (dict(topk=256), S.SA_EUNSUPPORTED),
    (dict(cand_blocks=1024), S.SA_EUNSUPPORTED),
    (dict(max_queries=0), S.SA_EINVAL),
    (dict(max_compressed=-1), S.SA_EINVAL),
    (dict(max_compressed=(1 << 20) + 1), S.SA_EUNSUPPORTED),
    (dict(softmax_scale=float("nan")), S.SA_EINVAL),
    (dict(softmax_scale=0.0), S.SA_EINVAL),
])
def test_plan_rejects(kw, status):
    with pytest.raises(S.SparseAttnError) as ei:
        _plan(**kw)
    assert ei.value.status == status
    assert S.lib.sparse_attn_last_error()


def _splits(T):
    # key splits of the attention for T queries: 4 work-groups per head set for T <= 32
    return 4 if T <= 32 else 1


def _expected_workspace(max_queries):
    a256 = lambda b: (b + 255) // 256 * 256
    select = max_queries * 2048 * 4                       # candidate blocks
    units = max([T * _splits(T) for T in range(1, max_queries + 1) if _splits(T) > 1] or [0])
    if units == 0:
        return select
    counters = a256(select)
    ml = counters + a256(8 * max_queries)        # one counter per (query, head set)
    o = ml + a256(units * 64 * 2 * 4)
    return o + units * 64 * 512 * 4


@pytest.mark.parametrize("mq", [1, 7, 100, 128, 255, 256, 4096])
def test_plan_workspace_and_last_error_reset(mq):
    p = _plan(max_queries=mq)
    assert p.workspace_bytes == _expected_workspace(mq)
    assert S.lib.sparse_attn_last_error() == b""


@pytest.mark.parametrize("maxc,parts", [(65536, 1), (65544, 2), (524288, 8), (524296, 5),
                                         (1 << 20, 8)])
def test_plan_accepts_long_rows(maxc, parts):
    # ratio-1 layers at the pages' 1,048,576-token context: rows up to 2^20 positions. Rows
    # past 8192 blocks run the candidate stage over parts (8192 blocks, or 16384 past 65536
    # blocks), whose 2048-id lists live in the select area of the workspace.
    mq = 3
    p = _plan(ratio=1, key_dtype="fp8", max_queries=mq, max_compressed=maxc)
    nb = (maxc + 7) // 8
    size = 8192 if nb <= 8 * 8192 else 16384
    expect = 1 if nb <= 8192 else -(-nb // size)
    assert expect == parts
    extra = mq * parts * 2048 * 8 if parts > 1 else 0   # ids and keys
    a256 = lambda b: (b + 255) // 256 * 256
    select = mq * 2048 * 4 + extra
    counters = a256(select)
    ml = counters + a256(8 * mq)
    o = ml + a256(4 * mq * 64 * 2 * 4)
    assert p.workspace_bytes == o + 4 * mq * 64 * 512 * 4


def test_select_refuses_grid_overflow():
    # parts in grid x, queries in grid y: rows longer than 65536 positions take at most 65535
    # queries per call (refused on the host, nothing enqueued)
    p = _plan(ratio=1, max_queries=70000, max_compressed=1 << 20)
    q = _q(T=65536, max_visible=65544)
    st = S.lib.select_topk(p.handle, ctypes.byref(q), 0x60000, 65544, None, 0, 0x80000, 0xA0000,
                           0x90000, 1 << 40, None)
    assert st == S.SA_EUNSUPPORTED and b"65535" in S.lib.sparse_attn_last_error()


def test_indexer_refuses_chunk_grid_overflow():
    # the chunk kernel holds ceil(T / 16) query tiles in grid y
    T = 65535 * 16 + 1
    p = _plan(ratio=1, max_queries=T, max_compressed=4096)
    q = _q(T=T, max_visible=100)
    c = _c(num_seqs=1)
    assert _indexer(p, q, c) == S.SA_EUNSUPPORTED
    arr = (ctypes.c_int32 * 1)(T)
    q.runs = ctypes.cast(arr, ctypes.c_void_p)
    q.num_runs = 1
    assert _indexer(p, q, c) == S.SA_EUNSUPPORTED
    assert b"per run" in S.lib.sparse_attn_last_error()


@pytest.mark.parametrize("case,wcap", [("group6", 132), ("runs3-7", 133), ("one_seq_T4", 130)])
def test_attn_refuses_aliasing_window_ring(case, wcap):
    # window rows live at u % window_cap: queries of one sequence spanning s positions need
    # window_cap >= 127 + s, or later positions overwrite rows earlier queries read
    p = _plan(max_queries=16)
    q, c = _q(T=10 if case != "one_seq_T4" else 4), _c(window_cap=wcap, window_seq_stride=wcap * 512)
    if case == "group6":
        q.group = 6
    if case == "runs3-7":
        arr = (ctypes.c_int32 * 2)(3, 7)
        q.runs = ctypes.cast(arr, ctypes.c_void_p)
        q.num_runs = 2
    if case == "one_seq_T4":
        c.num_seqs = 1
    st = S.lib.sparse_attn_fwd(p.handle, ctypes.byref(q), ctypes.byref(c), 0x40000, 0x50000,
                               0x60000, None, None, 0, None)
    assert st == S.SA_EINVAL and b"window_cap" in S.lib.sparse_attn_last_error()


def test_workspace_init_checks():
    p = _plan(max_queries=8)
    assert S.lib.sparse_attn_workspace_init(None, 0x1000, 1 << 30, None) != 0
    assert S.lib.sparse_attn_workspace_init(p.handle, None, 1 << 30, None) == 3        # SA_EWORKSPACE
    assert S.lib.sparse_attn_workspace_init(p.handle, 0x1008, 1 << 30, None) == 3      # misaligned
    assert S.lib.sparse_attn_workspace_init(p.handle, 0x1000, p.workspace_bytes - 1, None) == 3
    assert b"workspace" in S.lib.sparse_attn_last_error()


def _q(T=4, max_visible=100, seq=0x1000, pos=0x2000):
    return S.sa_queries(T=T, seq_id=seq, pos=pos, max_visible=max_visible)


def _c(**kw):
    c = S.sa_cache(num_seqs=4, compressed_cap=1000, latents=0x10000, latents_seq_stride=1000 * 512,
                   window=0x20000, window_seq_stride=128 * 512, window_cap=128,
                   idx_keys=0x30000, idx_keys_seq_stride=1000 * 128, idx_scales=None,
                   idx_scales_seq_stride=0)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _indexer(p, q, c, qi=0x40000, w=0x50000, scores=0x60000, ld=104, bm=None, ldb=0):
    return S.lib.indexer_score(p.handle, ctypes.byref(q), ctypes.byref(c), qi, w, scores, ld, bm, ldb, None)


@pytest.mark.parametrize("case", [
    "T0", "Tbig", "seq_null", "maxvis_big", "cap_small", "keys_null", "keys_misaligned",
    "qidx_null", "scores_null", "ld_small", "ldb_small", "fp8_no_scales", "stride_small",
])
def test_indexer_rejects(case):
    p = _plan()
    q, c = _q(), _c()
    kw = {}
    if case == "T0": q.T = 0
    if case == "Tbig": q.T = 9
    if case == "seq_null": q.seq_id = None
    if case == "maxvis_big": q.max_visible = 5000
    if case == "cap_small": c.compressed_cap = 50
    if case == "keys_null": c.idx_keys = None
    if case == "keys_misaligned": c.idx_keys = 0x30008
    if case == "qidx_null": kw["qi"] = None
    if case == "scores_null": kw["scores"] = None
    if case == "ld_small": kw["ld"] = 100   # max_visible 100 -> rows of 104
    if case == "ldb_small": kw.update(bm=0x70000, ldb=12)
    if case == "stride_small": c.idx_keys_seq_stride = 999 * 128
    if case == "fp8_no_scales":
        p = _plan(key_dtype="fp8")
    st = _indexer(p, q, c, **kw)
    assert st == S.SA_EINVAL, (case, st, S.lib.sparse_attn_last_error())
    assert S.lib.sparse_attn_last_error()


@pytest.mark.parametrize("group", [-1, 9])
def test_indexer_rejects_group(group):
    p = _plan()
    q, c = _q(), _c()
    q.group = group
    assert _indexer(p, q, c) == S.SA_EUNSUPPORTED
    assert b"group" in S.lib.sparse_attn_last_error()


@pytest.mark.parametrize("case", ["no_scales", "scale_stride", "key_stride", "cand"])
def test_mxfp4_rejects(case):
    p = _plan(key_dtype="mxfp4")
    q = _q()
    c = _c(idx_keys_seq_stride=1000 * 64, idx_scales=0x70000, idx_scales_seq_stride=4000)
    if case == "no_scales": c.idx_scales = None
    if case == "scale_stride": c.idx_scales_seq_stride = 3999
    if case == "key_stride": c.idx_keys_seq_stride = 999 * 64
    if case == "cand":
        # re-scoring takes MXFP4 keys, but only from contiguous stores: refused on pages
        c.block_table, c.block_table_stride, c.page_size, c.num_pages = 0xA0000, 63, 16, 300
        st = S.lib.indexer_score_cand(p.handle, ctypes.byref(q), ctypes.byref(c), 0x40000, 0x50000,
                                      0x80000, 0x60000, 16384, 0x90000, 2048, None)
        assert st == S.SA_EUNSUPPORTED and b"contiguous" in S.lib.sparse_attn_last_error()
        return
    assert _indexer(p, q, c) == S.SA_EINVAL, S.lib.sparse_attn_last_error()


@pytest.mark.parametrize("runs", [[1, 2], [4, 0], [5]])
def test_indexer_rejects_bad_runs(runs):
    # T = 4: runs must be >= 1 each and sum to T
    p = _plan()
    q, c = _q(), _c()
    arr = (ctypes.c_int32 * len(runs))(*runs)
    q.runs = ctypes.cast(arr, ctypes.c_void_p)
    q.num_runs = len(runs)
    assert _indexer(p, q, c) == S.SA_EINVAL
    assert b"runs" in S.lib.sparse_attn_last_error()


def test_select_rejects():
    p = _plan()
    q = _q()
    lib = S.lib
    # topk NULL
    assert lib.select_topk(p.handle, ctypes.byref(q), 0x60000, 104, None, 0, 0x80000, None,
                           0x90000, 1 << 20, None) == S.SA_EINVAL
    # no cand and no workspace
    assert lib.select_topk(p.handle, ctypes.byref(q), 0x60000, 104, None, 0, None, 0xA0000,
                           None, 0, None) == S.SA_EWORKSPACE
    # workspace too small for T queries
    assert lib.select_topk(p.handle, ctypes.byref(q), 0x60000, 104, None, 0, None, 0xA0000,
                           0x90000, 4 * 2048 * 4 - 1, None) == S.SA_EWORKSPACE
    # ld_scores below max_visible
    assert lib.select_topk(p.handle, ctypes.byref(q), 0x60000, 96, None, 0, 0x80000, 0xA0000,
                           0x90000, 1 << 20, None) == S.SA_EINVAL


def test_attn_rejects():
    p = _plan()
    q = _q()
    lib = S.lib
    for c in (_c(window_cap=127), _c(latents=None), _c(window=None), _c(latents_seq_stride=512 * 999)):
        assert lib.sparse_attn_fwd(p.handle, ctypes.byref(q), ctypes.byref(c), 0x40000, 0x50000,
                                   0x60000, None, None, 0, None) == S.SA_EINVAL
    c = _c()
    assert lib.sparse_attn_fwd(p.handle, ctypes.byref(q), ctypes.byref(c), None, 0x50000, 0x60000,
                               None, None, 0, None) == S.SA_EINVAL
    assert lib.sparse_attn_fwd(p.handle, ctypes.byref(q), ctypes.byref(c), 0x40000, 0x50000, 0x60000,
                               0x70004, None, 0, None) == S.SA_EINVAL


def test_attn_noalloc_rejects():
    # the same host checks as sparse_attn_fwd, before any HIP call (no scratch lookup)
    p = _plan()
    q = _q()
    lib = S.lib
    for c in (_c(window_cap=127), _c(latents=None), _c(window=None)):
        assert lib.sparse_attn_fwd_noalloc(p.handle, ctypes.byref(q), ctypes.byref(c), 0x40000, 0x50000,
                                           0x60000, None, None) == S.SA_EINVAL
    c = _c()
    assert lib.sparse_attn_fwd_noalloc(None, ctypes.byref(q), ctypes.byref(c), 0x40000, 0x50000, 0x60000,
                                       None, None) == S.SA_EINVAL
    assert lib.sparse_attn_fwd_noalloc(p.handle, ctypes.byref(q), ctypes.byref(c), None, 0x50000, 0x60000,
                                       None, None) == S.SA_EINVAL
    assert lib.sparse_attn_fwd_noalloc(p.handle, ctypes.byref(q), ctypes.byref(c), 0x40000, 0x50000, 0x60000,
                                       0x70004, None) == S.SA_EINVAL
    assert S.lib.sparse_attn_last_error()


def test_compress_rejects():
    p = _plan()
    lib = S.lib
    assert lib.sparse_attn_compress(p.handle, None, 1024, 0x1000, 1024, 0x2000, 0x3000, 512, 4, None) == S.SA_EINVAL
    assert lib.sparse_attn_compress(p.handle, 0x1000, 1000, 0x1000, 1024, 0x2000, 0x3000, 512, 4, None) == S.SA_EINVAL
    assert lib.sparse_attn_compress(p.handle, 0x1000, 1024, None, 1024, 0x2000, 0x3000, 512, 4, None) == S.SA_EINVAL
    assert lib.sparse_attn_compress(p.handle, 0x1000, 1024, 0x1000, 1024, 0x2000, 0x3000, 512, -1, None) == S.SA_EINVAL
    assert lib.sparse_attn_compress(None, 0x1000, 1024, 0x1000, 1024, 0x2000, 0x3000, 512, 4, None) == S.SA_EINVAL


@pytest.mark.parametrize("case", ["no_latent_scales", "no_window_scales", "lat_stride_small",
                                  "lat_stride_odd", "scale_stride_small", "scale_stride_odd",
                                  "scales_misaligned"])
def test_mxfp4_latent_rejects(case):
    # MXFP4 latent rows: 256 code bytes and 16 E8M0 bytes per row, strides in bytes
    p = _plan(kv_dtype="mxfp4")
    q = _q()
    good = dict(latents_seq_stride=1000 * 256, window_seq_stride=128 * 512,
                latent_scales=0x70000, latent_scales_seq_stride=1000 * 16,
                window_scales=0x80000, window_scales_seq_stride=128)
    bad = {"no_latent_scales": dict(latent_scales=None), "no_window_scales": dict(window_scales=None),
           "lat_stride_small": dict(latents_seq_stride=999 * 256),
           "lat_stride_odd": dict(latents_seq_stride=1000 * 256 + 8),
           "scale_stride_small": dict(latent_scales_seq_stride=999 * 16),
           "scale_stride_odd": dict(latent_scales_seq_stride=1000 * 16 + 4),
           "scales_misaligned": dict(latent_scales=0x70004)}[case]
    c = _c(**{**good, **bad})
    assert S.lib.sparse_attn_fwd(p.handle, ctypes.byref(q), ctypes.byref(c), 0x40000, 0x50000,
                                 0x60000, None, None, 0, None) == S.SA_EINVAL
    assert b"latent" in S.lib.sparse_attn_last_error() or b"window" in S.lib.sparse_attn_last_error()
    assert S.lib.sparse_attn_compress(p.handle, 0x1000, 1024, 0x1000, 1024, 0x2000, 0x3000, 512, 4,
                                      None) == S.SA_EUNSUPPORTED


def test_compress_codes_rejects():
    lib = S.lib
    args = lambda **k: dict(dict(raw=0x1000, rs=1024, gate=0x1000, gs=1024, bias=0x3000, out=0x4000,
                                 os=512, sc=0x5000, ss=4, G=4), **k)
    call = lambda p, a: lib.sparse_attn_compress_codes(p.handle, a["raw"], a["rs"], a["gate"], a["gs"], a["bias"],
                                                       a["out"], a["os"], a["sc"], a["ss"], a["G"], None)
    assert call(_plan(), args()) == S.SA_EUNSUPPORTED              # bf16 latents: not a code store
    p8, p4 = _plan(kv_dtype="fp8"), _plan(kv_dtype="mxfp4")
    for bad in (dict(raw=None), dict(out=0x4008), dict(os=500), dict(os=496), dict(sc=None), dict(sc=0x5002),
                dict(ss=2), dict(ss=6), dict(G=-1), dict(gate=None), dict(gs=1000), dict(rs=1000)):
        assert call(p8, args(**bad)) == S.SA_EINVAL, bad
    assert call(p4, args(os=240)) == S.SA_EINVAL                   # MXFP4 rows are 256 bytes
    assert call(p4, args(os=256, ss=12)) == S.SA_EINVAL            # and 16 scale bytes
    assert call(p8, args(G=0)) == S.SA_OK and call(p4, args(os=256, ss=16, G=0)) == S.SA_OK


def _job(**k):
    a = dict(raw=0x1000, raw_group_stride=1024, gate=0x1000, gate_group_stride=1024, slot_bias=0x3000,
             out=0x4000, out_group_stride=512, out_scales=None, scales_group_stride=0, G=4)
    a.update(k)
    return S.sa_compress_job(**a)


def _index_compress(p, q, c, job, ld=104):
    return S.lib.indexer_score_compress(p.handle, ctypes.byref(q), ctypes.byref(c), 0x40000, 0x50000, 0x60000, ld,
                                        None, 0, None if job is None else ctypes.byref(job), None)


@pytest.mark.parametrize("bad", [dict(raw=None), dict(raw_group_stride=1000), dict(gate=None),
                                 dict(gate_group_stride=1000), dict(slot_bias=None), dict(out=0x4008),
                                 dict(out_group_stride=500), dict(G=-1)])
def test_indexer_compress_rejects_bad_job(bad):
    # the job's checks are the compressor's; a refused call enqueues nothing
    assert _index_compress(_plan(), _q(), _c(), _job(**bad)) == S.SA_EINVAL, S.lib.sparse_attn_last_error()


def test_indexer_compress_code_rows_job():
    # code-row plans check the scales of the job like sparse_attn_compress_codes
    p8 = _plan(kv_dtype="fp8")
    c8 = _c(latent_scales=0x70000, latent_scales_seq_stride=1000, window_scales=0x80000,
            window_scales_seq_stride=128)
    assert _index_compress(p8, _q(), c8, _job(out_scales=None)) == S.SA_EINVAL
    assert _index_compress(p8, _q(), c8, _job(out_scales=0x5002, scales_group_stride=4)) == S.SA_EINVAL
    assert _index_compress(p8, _q(), c8, _job(out_scales=0x5000, scales_group_stride=2)) == S.SA_EINVAL


def test_indexer_compress_checks_the_indexer_too():
    # a good job does not lift the indexer's own checks; no job or G = 0 is indexer_score
    q = _q()
    q.seq_id = None
    assert _index_compress(_plan(), q, _c(), _job()) == S.SA_EINVAL
    assert _index_compress(_plan(), _q(), _c(), _job(), ld=100) == S.SA_EINVAL
    assert _index_compress(_plan(), _q(), _c(idx_keys=None), None) == S.SA_EINVAL
    assert _index_compress(_plan(), _q(), _c(idx_keys=None), _job(G=0)) == S.SA_EINVAL
    assert b"idx_keys" in S.lib.sparse_attn_last_error() or S.lib.sparse_attn_last_error()


def test_plain_c_caller(tmp_path):
    # the library from C alone: tests/c/abi_host_check.c built with gcc against the header and
    # the built .so, run on the host (plan creation and argument errors need no GPU)
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.join(root, "sparse_attention_score_amd")
    exe = str(tmp_path / "abi_host_check")
    subprocess.run([gcc, "-std=c11", "-Wall", "-Werror", os.path.join(root, "tests", "c", "abi_host_check.c"),
                    "-I", os.path.join(root, "include"), "-L", libdir, "-lsparse_attn",
                    f"-Wl,-rpath,{libdir}", "-lm", "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "abi host checks ok" in r.stdout
