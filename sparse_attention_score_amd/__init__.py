"""Python binding of libsparse_attn.so: the two-tier sparse-attention hot path on MI355X.

Argument marshalling only. Every stage runs in the library's HIP kernels; torch is used
for device memory and the current stream. The entry points have the names of the C ABI
(include/sparse_attn.h): sparse_attn_plan, indexer_score, indexer_score_compress,
indexer_score_cand, select_topk, select_topk_cand, sparse_attn_fwd, sparse_attn_fwd_noalloc,
sparse_attn_compress, sparse_attn_compress_codes. If the built library is missing, importing
this package raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SPARSE_ATTN_LIB selects another build of the library (same ABI); default: the in-tree one
LIB_PATH = os.environ.get("SPARSE_ATTN_LIB") or os.path.join(_PKG, "libsparse_attn.so")

SA_OK, SA_EINVAL, SA_EUNSUPPORTED, SA_EWORKSPACE, SA_EHIP = 0, 1, 2, 3, 4
SA_KEY_BF16, SA_KEY_FP8_E4M3, SA_KEY_MXFP4 = 0, 1, 2
KEY_DTYPES = {"bf16": SA_KEY_BF16, "fp8": SA_KEY_FP8_E4M3, "mxfp4": SA_KEY_MXFP4}
SA_KV_BF16, SA_KV_FP8_E4M3, SA_KV_MXFP4 = 0, 1, 2
KV_DTYPES = {"bf16": SA_KV_BF16, "fp8": SA_KV_FP8_E4M3, "mxfp4": SA_KV_MXFP4}
STATUS_NAMES = {0: "SA_OK", 1: "SA_EINVAL", 2: "SA_EUNSUPPORTED", 3: "SA_EWORKSPACE", 4: "SA_EHIP"}

EXPORTS = ("sparse_attn_plan", "sparse_attn_plan_destroy", "sparse_attn_last_error",
           "sparse_attn_workspace_init", "indexer_score", "select_topk", "indexer_score_cand",
           "select_topk_cand", "sparse_attn_fwd", "sparse_attn_fwd_noalloc", "sparse_attn_compress",
           "sparse_attn_compress_codes", "indexer_score_compress")


class sa_params(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("latent_dim", ctypes.c_int32),
                ("window", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
                ("block", ctypes.c_int32), ("cand_blocks", ctypes.c_int32),
                ("ratio", ctypes.c_int32), ("idx_key_dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("max_queries", ctypes.c_int64),
                ("max_compressed", ctypes.c_int64), ("kv_dtype", ctypes.c_int32)]


class sa_queries(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("seq_id", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("max_visible", ctypes.c_int64), ("group", ctypes.c_int32),
                ("runs", ctypes.c_void_p), ("num_runs", ctypes.c_int32)]


class sa_cache(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int64), ("compressed_cap", ctypes.c_int64),
                ("latents", ctypes.c_void_p), ("latents_seq_stride", ctypes.c_int64),
                ("window", ctypes.c_void_p), ("window_seq_stride", ctypes.c_int64),
                ("window_cap", ctypes.c_int32),
                ("idx_keys", ctypes.c_void_p), ("idx_keys_seq_stride", ctypes.c_int64),
                ("idx_scales", ctypes.c_void_p), ("idx_scales_seq_stride", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("block_table_stride", ctypes.c_int64),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int64),
                ("latent_scales", ctypes.c_void_p), ("latent_scales_seq_stride", ctypes.c_int64),
                ("window_scales", ctypes.c_void_p), ("window_scales_seq_stride", ctypes.c_int64)]


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class sa_compress_job(ctypes.Structure):
    _fields_ = [("raw", ctypes.c_void_p), ("raw_group_stride", ctypes.c_int64),
                ("gate", ctypes.c_void_p), ("gate_group_stride", ctypes.c_int64),
                ("slot_bias", ctypes.c_void_p), ("out", ctypes.c_void_p), ("out_group_stride", ctypes.c_int64),
                ("out_scales", ctypes.c_void_p), ("scales_group_stride", ctypes.c_int64), ("G", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          f"python sparse_attention_score_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    lib.sparse_attn_plan.argtypes = [ctypes.POINTER(sa_params), ctypes.POINTER(vp), ctypes.POINTER(sz)]
    lib.sparse_attn_plan.restype = ctypes.c_int
    lib.sparse_attn_plan_destroy.argtypes = [vp]
    lib.sparse_attn_plan_destroy.restype = None
    lib.sparse_attn_last_error.argtypes = []
    lib.sparse_attn_last_error.restype = ctypes.c_char_p
    lib.sparse_attn_workspace_init.argtypes = [vp, vp, sz, vp]
    lib.sparse_attn_workspace_init.restype = ctypes.c_int
    lib.indexer_score.argtypes = [vp, ctypes.POINTER(sa_queries), ctypes.POINTER(sa_cache), vp, vp,
                                  vp, i64, vp, i64, vp]
    lib.indexer_score.restype = ctypes.c_int
    lib.select_topk.argtypes = [vp, ctypes.POINTER(sa_queries), vp, i64, vp, i64, vp, vp, vp, sz, vp]
    lib.select_topk.restype = ctypes.c_int
    lib.indexer_score_cand.argtypes = [vp, ctypes.POINTER(sa_queries), ctypes.POINTER(sa_cache), vp, vp,
                                       vp, vp, i64, vp, i64, vp]
    lib.indexer_score_cand.restype = ctypes.c_int
    lib.select_topk_cand.argtypes = [vp, ctypes.POINTER(sa_queries), vp, vp, i64, vp, i64, vp, vp]
    lib.select_topk_cand.restype = ctypes.c_int
    lib.sparse_attn_fwd.argtypes = [vp, ctypes.POINTER(sa_queries), ctypes.POINTER(sa_cache), vp, vp,
                                    vp, vp, vp, sz, vp]
    lib.sparse_attn_fwd.restype = ctypes.c_int
    lib.sparse_attn_fwd_noalloc.argtypes = [vp, ctypes.POINTER(sa_queries), ctypes.POINTER(sa_cache), vp, vp,
                                            vp, vp, vp]
    lib.sparse_attn_fwd_noalloc.restype = ctypes.c_int
    lib.sparse_attn_compress.argtypes = [vp, vp, i64, vp, i64, vp, vp, i64, i64, vp]
    lib.sparse_attn_compress.restype = ctypes.c_int
    lib.sparse_attn_compress_codes.argtypes = [vp, vp, i64, vp, i64, vp, vp, i64, vp, i64, i64, vp]
    lib.sparse_attn_compress_codes.restype = ctypes.c_int
    lib.indexer_score_compress.argtypes = [vp, ctypes.POINTER(sa_queries), ctypes.POINTER(sa_cache), vp, vp,
                                           vp, i64, vp, i64, ctypes.POINTER(sa_compress_job), vp]
    lib.indexer_score_compress.restype = ctypes.c_int
    return lib


lib = _load()


def _check(status: int):
    if status != SA_OK:
        msg = lib.sparse_attn_last_error()
        raise SparseAttnError(status, msg.decode() if msg else "")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _need(t: torch.Tensor, name: str, dtype, cuda: bool = True):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if cuda and not t.is_cuda:
        raise TypeError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


class Plan:
    """sparse_attn_plan: fixed layer shape, ratio, key dtype and maximum sizes."""

    def __init__(self, ratio: int, key_dtype: str = "bf16", max_queries: int = 1,
                 max_compressed: int = 0, softmax_scale: float = 1.0 / math.sqrt(512.0),
                 kv_dtype: str = "bf16", **dims):
        p = sa_params(num_heads=dims.get("num_heads", 64), latent_dim=dims.get("latent_dim", 512),
                      window=dims.get("window", 128), topk=dims.get("topk", 512),
                      idx_heads=dims.get("idx_heads", 16), idx_dim=dims.get("idx_dim", 128),
                      block=dims.get("block", 8), cand_blocks=dims.get("cand_blocks", 2048),
                      ratio=ratio,
                      idx_key_dtype=KEY_DTYPES[key_dtype],
                      softmax_scale=softmax_scale, max_queries=max_queries,
                      max_compressed=max_compressed, kv_dtype=KV_DTYPES[kv_dtype])
        h = ctypes.c_void_p()
        ws = ctypes.c_size_t()
        _check(lib.sparse_attn_plan(ctypes.byref(p), ctypes.byref(h), ctypes.byref(ws)))
        self.handle = h
        self.params = p
        self.workspace_bytes = ws.value
        self.key_dtype = key_dtype
        self.kv_dtype = kv_dtype
        self.ratio = ratio

    def __del__(self, _destroy=lib.sparse_attn_plan_destroy):
        # the default argument keeps the function reachable at interpreter exit, when the
        # module's globals may already be cleared
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            _destroy(h)
            self.handle = None


def sparse_attn_plan(**kw) -> Plan:
    return Plan(**kw)


class Queries:
    """sa_queries from device int32 tensors seq_id[T], pos[T], a host max_visible and the
    number of consecutive queries that share a sequence (group; 0 = none)."""

    def __init__(self, seq_id: torch.Tensor, pos: torch.Tensor, max_visible: int, group: int = 0,
                 runs=None):
        _need(seq_id, "seq_id", torch.int32)
        _need(pos, "pos", torch.int32)
        self.c = sa_queries(T=seq_id.shape[0], seq_id=seq_id.data_ptr(), pos=pos.data_ptr(),
                            max_visible=int(max_visible), group=int(group))
        host_runs = None
        if runs is not None:   # host run lengths of a ragged batch
            host_runs = (ctypes.c_int32 * len(runs))(*[int(r) for r in runs])
            self.c.runs = ctypes.cast(host_runs, ctypes.c_void_p)
            self.c.num_runs = len(runs)
        self._keep = (seq_id, pos, host_runs)

    @property
    def T(self) -> int:
        return self.c.T


def _seq_stride(t: torch.Tensor) -> int:
    """Stride of dim 0 in elements; a single-sequence tensor may carry any stride there (a
    size-1 dimension), so its row block size is used instead."""
    if t.shape[0] > 1:
        return t.stride(0)
    n = 1
    for d in t.shape[1:]:
        n *= d
    return n


class Cache:
    """sa_cache from device tensors: latents [S,cap,512] bf16 or uint8 (e4m3 codes) or uint8
    [S,cap,256] (MXFP4 codes), window [S,wcap,512] bf16 or uint8 (e4m3 codes), latent_scales
    [S,cap] fp32 (e4m3) or uint8 [S,cap,16] (MXFP4 E8M0 scales), window_scales [S,wcap] fp32,
    idx_keys [S,cap,128] bf16 or uint8 (e4m3 codes), or uint8 [S,cap,64] (MXFP4 codes);
    idx_scales [S,cap] fp32 (e4m3), uint8 [S,cap,4] (MXFP4 E8M0 scales) or None.
    Any of them may be None when the call at hand does not read it."""

    def __init__(self, latents=None, window=None, idx_keys=None, idx_scales=None,
                 num_seqs: Optional[int] = None, compressed_cap: Optional[int] = None,
                 block_table: Optional[torch.Tensor] = None, page_size: int = 0,
                 latent_scales: Optional[torch.Tensor] = None,
                 window_scales: Optional[torch.Tensor] = None):
        ref = latents if latents is not None else idx_keys
        if num_seqs is None:
            num_seqs = ref.shape[0]
        if compressed_cap is None:
            compressed_cap = ref.shape[1]
        c = sa_cache(num_seqs=num_seqs, compressed_cap=compressed_cap)
        # latents / window: bf16 rows, or uint8 e4m3 codes with fp32 row scales (strides in
        # elements of the tensor: bf16 or bytes, as the C ABI counts them)
        if latents is not None:
            if latents.dtype not in (torch.bfloat16, torch.uint8):
                raise TypeError("latents must be bfloat16 or uint8 (e4m3 codes)")
            _need(latents, "latents", latents.dtype)
            c.latents, c.latents_seq_stride = latents.data_ptr(), _seq_stride(latents)
        if window is not None:
            if window.dtype not in (torch.bfloat16, torch.uint8):
                raise TypeError("window must be bfloat16 or uint8 (e4m3 codes)")
            _need(window, "window", window.dtype)
            c.window, c.window_seq_stride, c.window_cap = window.data_ptr(), _seq_stride(window), window.shape[1]
        if latent_scales is not None:
            if latent_scales.dtype not in (torch.float32, torch.uint8):
                raise TypeError("latent_scales must be float32 (e4m3) or uint8 (MXFP4 E8M0)")
            _need(latent_scales, "latent_scales", latent_scales.dtype)
            c.latent_scales, c.latent_scales_seq_stride = latent_scales.data_ptr(), _seq_stride(latent_scales)
        if window_scales is not None:
            _need(window_scales, "window_scales", torch.float32)
            c.window_scales, c.window_scales_seq_stride = window_scales.data_ptr(), _seq_stride(window_scales)
        if idx_keys is not None:
            if idx_keys.dtype not in (torch.bfloat16, torch.uint8):
                raise TypeError("idx_keys must be bfloat16 or uint8 (e4m3 or MXFP4 codes)")
            _need(idx_keys, "idx_keys", idx_keys.dtype)
            c.idx_keys, c.idx_keys_seq_stride = idx_keys.data_ptr(), _seq_stride(idx_keys)
        if idx_scales is not None:
            if idx_scales.dtype not in (torch.float32, torch.uint8):
                raise TypeError("idx_scales must be float32 (e4m3) or uint8 (MXFP4 E8M0)")
            _need(idx_scales, "idx_scales", idx_scales.dtype)
            c.idx_scales, c.idx_scales_seq_stride = idx_scales.data_ptr(), _seq_stride(idx_scales)
        if block_table is not None:
            # paged stores: latents [pages*page_size, 512], idx_keys [pages*page_size, 128],
            # idx_scales [pages*page_size] are pools; block_table [num_seqs, pages per seq]
            _need(block_table, "block_table", torch.int32)
            pool = latents if latents is not None else idx_keys
            c.block_table, c.block_table_stride = block_table.data_ptr(), _seq_stride(block_table)
            c.page_size = int(page_size)
            c.num_pages = pool.shape[0] // int(page_size)
        self._keep = (latents, window, idx_keys, idx_scales, block_table, latent_scales, window_scales)
        self.c = c


def indexer_score(plan: Plan, queries: Queries, cache: Cache, q_idx: torch.Tensor, w: torch.Tensor,
                  scores: torch.Tensor, block_max: Optional[torch.Tensor] = None, stream=None):
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(w, "w", torch.float32)
    _need(scores, "scores", torch.float32)
    if block_max is not None:
        _need(block_max, "block_max", torch.float32)
    _check(lib.indexer_score(plan.handle, ctypes.byref(queries.c), ctypes.byref(cache.c),
                             _ptr(q_idx), _ptr(w), _ptr(scores), scores.stride(0),
                             _ptr(block_max), 0 if block_max is None else block_max.stride(0),
                             _stream(stream)))


class CompressJob:
    """A compressor job for indexer_score_compress: the arguments of sparse_attn_compress (bf16
    plans; strides in bf16 elements) or sparse_attn_compress_codes (code-row plans: out and
    out_scales strides in bytes). Tensors are passed as base pointers and kept alive here."""

    def __init__(self, raw: torch.Tensor, raw_group_stride: int, gate: Optional[torch.Tensor],
                 gate_group_stride: int, slot_bias: Optional[torch.Tensor], out: torch.Tensor,
                 out_group_stride: int, G: int, out_scales: Optional[torch.Tensor] = None,
                 scales_group_stride: int = 0):
        for t, name in ((raw, "raw"), (gate, "gate")):
            if t is not None and (t.dtype != torch.bfloat16 or not t.is_cuda):
                raise TypeError(f"{name}: expected a bfloat16 device tensor")
        if not out.is_cuda or out.dtype not in (torch.bfloat16, torch.uint8):
            raise TypeError("out: expected a bfloat16 (bf16 rows) or uint8 (code rows) device tensor")
        if slot_bias is not None:
            _need(slot_bias, "slot_bias", torch.float32)
        if out_scales is not None and (out_scales.dtype not in (torch.float32, torch.uint8) or not out_scales.is_cuda):
            raise TypeError("out_scales: expected a float32 (e4m3) or uint8 (MXFP4) device tensor")
        j = sa_compress_job()
        j.raw, j.raw_group_stride = _ptr(raw), raw_group_stride
        j.gate, j.gate_group_stride = _ptr(gate), gate_group_stride
        j.slot_bias = _ptr(slot_bias)
        j.out, j.out_group_stride = _ptr(out), out_group_stride
        j.out_scales, j.scales_group_stride = _ptr(out_scales), scales_group_stride
        j.G = G
        self._keep = (raw, gate, slot_bias, out, out_scales)
        self.c = j


def indexer_score_compress(plan: Plan, queries: Queries, cache: Cache, q_idx: torch.Tensor, w: torch.Tensor,
                           scores: torch.Tensor, block_max: Optional[torch.Tensor], job: Optional[CompressJob],
                           stream=None):
    """indexer_score with a compressor job in the same launch (job None: indexer_score)."""
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(w, "w", torch.float32)
    _need(scores, "scores", torch.float32)
    if block_max is not None:
        _need(block_max, "block_max", torch.float32)
    _check(lib.indexer_score_compress(plan.handle, ctypes.byref(queries.c), ctypes.byref(cache.c),
                                      _ptr(q_idx), _ptr(w), _ptr(scores), scores.stride(0),
                                      _ptr(block_max), 0 if block_max is None else block_max.stride(0),
                                      None if job is None else ctypes.byref(job.c), _stream(stream)))


def indexer_score_cand(plan: Plan, queries: Queries, cache: Cache, q_idx: torch.Tensor,
                       w: torch.Tensor, cand: torch.Tensor, scores: torch.Tensor,
                       block_max: torch.Tensor, stream=None):
    """Candidate-bounded re-scoring: scores in slot order of the carried blocks `cand`."""
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(w, "w", torch.float32)
    _need(cand, "cand", torch.int32)
    _need(scores, "scores", torch.float32)
    _need(block_max, "block_max", torch.float32)
    _check(lib.indexer_score_cand(plan.handle, ctypes.byref(queries.c), ctypes.byref(cache.c),
                                  _ptr(q_idx), _ptr(w), _ptr(cand), _ptr(scores), scores.stride(0),
                                  _ptr(block_max), block_max.stride(0), _stream(stream)))


def select_topk_cand(plan: Plan, queries: Queries, cand: torch.Tensor, scores: torch.Tensor,
                     block_max: torch.Tensor, topk: torch.Tensor, stream=None):
    """Top-512 positions inside the carried candidate blocks (after indexer_score_cand)."""
    _need(cand, "cand", torch.int32)
    _need(scores, "scores", torch.float32)
    _need(block_max, "block_max", torch.float32)
    _need(topk, "topk", torch.int32)
    _check(lib.select_topk_cand(plan.handle, ctypes.byref(queries.c), _ptr(cand), _ptr(scores),
                                scores.stride(0), _ptr(block_max), block_max.stride(0), _ptr(topk),
                                _stream(stream)))


def select_topk(plan: Plan, queries: Queries, scores: torch.Tensor,
                block_max: Optional[torch.Tensor], topk: torch.Tensor,
                cand: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream=None):
    _need(scores, "scores", torch.float32)
    _need(topk, "topk", torch.int32)
    if block_max is not None:
        _need(block_max, "block_max", torch.float32)
    if cand is not None:
        _need(cand, "cand", torch.int32)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.select_topk(plan.handle, ctypes.byref(queries.c), _ptr(scores), scores.stride(0),
                           _ptr(block_max), 0 if block_max is None else block_max.stride(0),
                           _ptr(cand), _ptr(topk), _ptr(workspace), ws_bytes, _stream(stream)))


def sparse_attn_workspace_init(plan: Plan, workspace: torch.Tensor, stream=None):
    """Zero the attention counters of a fresh workspace (once per allocation)."""
    _need(workspace, "workspace", torch.uint8)
    _check(lib.sparse_attn_workspace_init(plan.handle, _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream(stream)))


def workspace_for(plan: Plan, device="cuda") -> torch.Tensor:
    """A workspace of the plan's size, ready for use by select_topk and sparse_attn_fwd."""
    ws = torch.empty((max(16, plan.workspace_bytes),), dtype=torch.uint8, device=device)
    sparse_attn_workspace_init(plan, ws)
    return ws


def sparse_attn_fwd(plan: Plan, queries: Queries, cache: Cache, q: torch.Tensor, topk: torch.Tensor,
                    out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None):
    _need(q, "q", torch.bfloat16)
    _need(topk, "topk", torch.int32)
    _need(out, "out", torch.bfloat16)
    if lse is not None:
        _need(lse, "lse", torch.float32)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.sparse_attn_fwd(plan.handle, ctypes.byref(queries.c), ctypes.byref(cache.c), _ptr(q),
                               _ptr(topk), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                               _stream(stream)))


def sparse_attn_fwd_noalloc(plan: Plan, queries: Queries, cache: Cache, q: torch.Tensor, topk: torch.Tensor,
                            out: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None):
    """sparse_attn_fwd without a workspace: key-split state in the library's fixed per-GPU array."""
    _need(q, "q", torch.bfloat16)
    _need(topk, "topk", torch.int32)
    _need(out, "out", torch.bfloat16)
    if lse is not None:
        _need(lse, "lse", torch.float32)
    _check(lib.sparse_attn_fwd_noalloc(plan.handle, ctypes.byref(queries.c), ctypes.byref(cache.c), _ptr(q),
                                       _ptr(topk), _ptr(out), _ptr(lse), _stream(stream)))


def sparse_attn_compress(plan: Plan, raw: torch.Tensor, raw_group_stride: int, gate: Optional[torch.Tensor],
                         gate_group_stride: int, slot_bias: Optional[torch.Tensor], out: torch.Tensor,
                         out_group_stride: int, G: int, stream=None):
    """Tensors are passed as base pointers; groups are addressed by the given element strides."""
    for t, name in ((raw, "raw"), (out, "out")):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError(f"{name}: expected a bfloat16 device tensor")
    if gate is not None and (gate.dtype != torch.bfloat16 or not gate.is_cuda):
        raise TypeError("gate: expected a bfloat16 device tensor")
    if slot_bias is not None:
        _need(slot_bias, "slot_bias", torch.float32)
    _check(lib.sparse_attn_compress(plan.handle, _ptr(raw), raw_group_stride, _ptr(gate),
                                    gate_group_stride, _ptr(slot_bias), _ptr(out), out_group_stride,
                                    G, _stream(stream)))


def sparse_attn_compress_codes(plan: Plan, raw: torch.Tensor, raw_group_stride: int,
                               gate: Optional[torch.Tensor], gate_group_stride: int,
                               slot_bias: Optional[torch.Tensor], out: torch.Tensor, out_group_stride: int,
                               out_scales: torch.Tensor, scales_group_stride: int, G: int, stream=None):
    """The compressor into e4m3 or MXFP4 code rows (the plan's kv_dtype). raw / gate strides in
    bf16 elements; out (uint8) and out_scales (fp32 for e4m3, uint8 for MXFP4) strides in bytes."""
    for t, name in ((raw, "raw"), (gate, "gate")):
        if t is not None and (t.dtype != torch.bfloat16 or not t.is_cuda):
            raise TypeError(f"{name}: expected a bfloat16 device tensor")
    if out.dtype != torch.uint8 or not out.is_cuda:
        raise TypeError("out: expected a uint8 device tensor (code bytes)")
    if out_scales.dtype not in (torch.float32, torch.uint8) or not out_scales.is_cuda:
        raise TypeError("out_scales: expected a float32 (e4m3) or uint8 (MXFP4) device tensor")
    if slot_bias is not None:
        _need(slot_bias, "slot_bias", torch.float32)
    _check(lib.sparse_attn_compress_codes(plan.handle, _ptr(raw), raw_group_stride, _ptr(gate),
                                          gate_group_stride, _ptr(slot_bias), _ptr(out), out_group_stride,
                                          _ptr(out_scales), scales_group_stride, G, _stream(stream)))
