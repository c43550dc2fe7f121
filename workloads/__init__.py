"""Seeded synthetic workloads for the two-tier sparse-attention hot path.

This module only draws input tensors (as raw bf16 / e4m3 bit patterns and fp32
arrays). It holds none of the method's arithmetic. The fp64 oracle and the
HIP library both consume what it produces; neither is imported here.

Shapes follow the pages: one 512-wide latent per position shared by 64 query
heads ("DeepSeek-V4.1 Flash", section 1 Model Introduction), a 128-position
sliding window, compression ratios 1 and 2, top-512 after 2048 candidate
blocks of 8 ("deepseek-ai/DeepSeek-V4.1-Flash" recipe, Overview, two-tier
sparse attention bullet), up to 1,048,576 tokens of context (same recipe,
Context length). The indexer is 16 heads x 128 dims with one 128-d key per
compressed position.

Value recipe (the pages give none): every tensor is i.i.d. N(0,1) drawn in
fp32 and rounded to bf16 (RNE), except the indexer head weights w ~ U[0,1) in
fp32, the compressor slot bias beta ~ N(0,1) in fp32, and fp8 index keys,
which are N(0,1) fp32 rows quantised to OCP e4m3 with one fp32 scale per row.
Each (tensor, sequence) pair is its own Philox stream, so the result does not
depend on thread count and any sequence can be regenerated alone.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

# Stream tags: stream id = (tag << 32) | sequence.
TAG = {"q": 1, "qI": 2, "w": 3, "C": 4, "KI": 5, "R": 6, "Xp": 7, "Zp": 8, "beta": 9, "Xraw": 10, "Zraw": 11,
       "q-mq": 12, "qI-mq": 13, "w-mq": 14}

# Layer shapes the pages fix.
HEADS = 64          # query heads sharing one latent
DIM = 512           # latent width (key = value)
WINDOW = 128        # sliding-window positions
TOPK = 512          # selected compressed latents per query
IDX_HEADS = 16      # indexer heads (stated choice)
IDX_DIM = 128       # indexer key / query width (stated choice)
BLOCK = 8           # positions per candidate block
CAND_BLOCKS = 2048  # candidate blocks kept


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        lib.synth_normal_f32.argtypes = [u64, u64, vp, i64]
        lib.synth_normal_bf16.argtypes = [u64, u64, vp, i64]
        lib.synth_uniform_f32.argtypes = [u64, u64, vp, i64]
        lib.synth_quant_e4m3_rows.argtypes = [vp, i64, i64, vp, vp]
        lib.synth_normal_e4m3_rows.argtypes = [u64, u64, i64, i64, vp, vp]
        lib.synth_quant_mxfp4_rows.argtypes = [vp, i64, i64, vp, vp]
        lib.synth_normal_mxfp4_rows.argtypes = [u64, u64, i64, i64, vp, vp]
        for f in (lib.synth_normal_f32, lib.synth_normal_bf16, lib.synth_uniform_f32,
                  lib.synth_quant_e4m3_rows, lib.synth_normal_e4m3_rows,
                  lib.synth_quant_mxfp4_rows, lib.synth_normal_mxfp4_rows):
            f.restype = None
        _lib = lib
    return _lib


def _stream(tag: str, seq: int) -> int:
    return (TAG[tag] << 32) | int(seq)


def normal_bf16(seed: int, tag: str, seq: int, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    _L().synth_normal_bf16(seed, _stream(tag, seq), out.ctypes.data, out.size)
    return out


def normal_f32(seed: int, tag: str, seq: int, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _L().synth_normal_f32(seed, _stream(tag, seq), out.ctypes.data, out.size)
    return out


def uniform_f32(seed: int, tag: str, seq: int, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _L().synth_uniform_f32(seed, _stream(tag, seq), out.ctypes.data, out.size)
    return out


def quant_e4m3_rows(x: np.ndarray):
    """Row-wise OCP e4m3 quantisation of an fp32 array [..., cols] -> (codes u8, scale f32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    cols = x.shape[-1]
    rows = x.size // cols
    codes = np.empty(x.shape, dtype=np.uint8)
    scale = np.empty(x.shape[:-1], dtype=np.float32)
    _L().synth_quant_e4m3_rows(x.ctypes.data, rows, cols, codes.ctypes.data, scale.ctypes.data)
    return codes, scale


def quant_mxfp4_rows(x: np.ndarray):
    """Row-wise OCP MXFP4 quantisation of fp32 [..., cols] -> (codes u8 [..., cols/2],
    E8M0 block scales u8 [..., cols/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    cols = x.shape[-1]
    assert cols % 32 == 0
    rows = x.size // cols
    codes = np.empty(x.shape[:-1] + (cols // 2,), dtype=np.uint8)
    scales = np.empty(x.shape[:-1] + (cols // 32,), dtype=np.uint8)
    _L().synth_quant_mxfp4_rows(x.ctypes.data, rows, cols, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def normal_mxfp4_rows(seed: int, tag: str, seq: int, rows: int, cols: int):
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    scales = np.empty((rows, cols // 32), dtype=np.uint8)
    _L().synth_normal_mxfp4_rows(seed, _stream(tag, seq), rows, cols, codes.ctypes.data,
                                 scales.ctypes.data)
    return codes, scales


def normal_e4m3_rows(seed: int, tag: str, seq: int, rows: int, cols: int):
    codes = np.empty((rows, cols), dtype=np.uint8)
    scale = np.empty((rows,), dtype=np.float32)
    _L().synth_normal_e4m3_rows(seed, _stream(tag, seq), rows, cols, codes.ctypes.data,
                                scale.ctypes.data)
    return codes, scale


@dataclass
class Workload:
    """One batch of queries against per-sequence stores (host arrays).

    Bit-pattern arrays: q [T,64,512], qI [T,16,128], C [B,nc_cap,512], R [B,wcap,512],
    Xp/Zp [B,2,512] are uint16 bf16 bits; KI is uint16 (bf16) or uint8 (e4m3) [B,nc_cap,128].
    w [T,16], KS [B,nc_cap] (e4m3 row scales, or None), beta [2,512] are fp32.
    Window row for raw position u of sequence b is R[b, u % wcap].
    """
    name: str
    kind: str            # "decode" | "prefill"
    ratio: int
    key_dtype: str       # "bf16" | "fp8" | "mxfp4"
    B: int
    T: int
    nc_cap: int
    wcap: int
    seq: np.ndarray
    pos: np.ndarray
    q: np.ndarray
    qI: np.ndarray
    w: np.ndarray
    C: np.ndarray
    KI: np.ndarray
    KS: Optional[np.ndarray]
    R: np.ndarray
    Xp: Optional[np.ndarray] = None   # raw latent pair completed by each sequence's query
    Zp: Optional[np.ndarray] = None   # gate logits of that pair
    beta: Optional[np.ndarray] = None
    seed: int = 0
    meta: dict = field(default_factory=dict)
    group: int = 0       # consecutive queries that share a sequence (multi-token decode)
    runs: Optional[list] = None   # ragged batch: lengths of the runs of one sequence each
    kv_dtype: str = "bf16"        # latents and window: "bf16", "fp8" (e4m3 codes + row scales),
                                  # or "mxfp4" (MXFP4 latents + E8M0 block scales, e4m3 window)
    CS: Optional[np.ndarray] = None   # fp8 latents: fp32 row scales [B, nc_cap]
    RS: Optional[np.ndarray] = None   # fp8 window: fp32 row scales [B, wcap]

    def visible(self) -> np.ndarray:
        return (self.pos.astype(np.int64) + 1) // self.ratio

    def compress_groups(self) -> np.ndarray:
        """Sequences whose query completes a group of `ratio` raw positions (ratio 2 only)."""
        if self.ratio != 2 or self.Xp is None:
            return np.zeros((0,), dtype=np.int64)
        done = ((self.pos.astype(np.int64) + 1) % 2) == 0
        return np.unique(self.seq[done].astype(np.int64))


def _keys(seed, key_dtype, B, nc_cap):
    if key_dtype == "bf16":
        KI = np.empty((B, nc_cap, IDX_DIM), dtype=np.uint16)
        for b in range(B):
            KI[b] = normal_bf16(seed, "KI", b, (nc_cap, IDX_DIM))
        return KI, None
    if key_dtype == "fp8":
        KI = np.empty((B, nc_cap, IDX_DIM), dtype=np.uint8)
        KS = np.empty((B, nc_cap), dtype=np.float32)
        for b in range(B):
            KI[b], KS[b] = normal_e4m3_rows(seed, "KI", b, nc_cap, IDX_DIM)
        return KI, KS
    if key_dtype == "mxfp4":
        KI = np.empty((B, nc_cap, IDX_DIM // 2), dtype=np.uint8)
        KS = np.empty((B, nc_cap, IDX_DIM // 32), dtype=np.uint8)
        for b in range(B):
            KI[b], KS[b] = normal_mxfp4_rows(seed, "KI", b, nc_cap, IDX_DIM)
        return KI, KS
    raise ValueError(key_dtype)


def make_decode(B: int, n_raw, ratio: int = 2, key_dtype: str = "bf16", seed: int = 0,
                wcap: int = WINDOW, name: str = "decode", nc_cap: Optional[int] = None,
                with_compress: bool = True, kv_dtype: str = "bf16",
                compress_codes: bool = False) -> Workload:
    """B sequences, one decode query each at raw position n_raw-1 (per-sequence if an array).
    kv_dtype "fp8": latents and window rows are N(0,1) rows quantised to e4m3 with one fp32
    scale per row (no compressor inputs then: the compressor writes bf16 rows). kv_dtype
    "mxfp4": N(0,1) latent rows quantised to MXFP4 (E8M0 scale per 32 elements) and e4m3
    window rows as for "fp8". compress_codes: compressor inputs for code-row stores too (the
    compressor then writes its group's row as codes and scales)."""
    n_raw = np.broadcast_to(np.asarray(n_raw, dtype=np.int64), (B,)).copy()
    pos = (n_raw - 1).astype(np.int32)
    vis = (pos.astype(np.int64) + 1) // ratio
    if nc_cap is None:
        nc_cap = int(max(1, vis.max()))
    T = B
    seq = np.arange(B, dtype=np.int32)
    q = np.empty((T, HEADS, DIM), np.uint16)
    qI = np.empty((T, IDX_HEADS, IDX_DIM), np.uint16)
    w = np.empty((T, IDX_HEADS), np.float32)
    C = np.empty((B, nc_cap, DIM), np.uint16) if kv_dtype == "bf16" else None
    R = np.empty((B, wcap, DIM), np.uint16) if kv_dtype == "bf16" else None
    for b in range(B):
        q[b] = normal_bf16(seed, "q", b, (HEADS, DIM))
        qI[b] = normal_bf16(seed, "qI", b, (IDX_HEADS, IDX_DIM))
        w[b] = uniform_f32(seed, "w", b, (IDX_HEADS,))
        if kv_dtype == "bf16":
            C[b] = normal_bf16(seed, "C", b, (nc_cap, DIM))
            R[b] = normal_bf16(seed, "R", b, (wcap, DIM))
    KI, KS = _keys(seed, key_dtype, B, nc_cap)
    CS = RS = None
    if kv_dtype in ("fp8", "mxfp4"):
        fp4 = kv_dtype == "mxfp4"
        C = np.empty((B, nc_cap, DIM // 2 if fp4 else DIM), np.uint8)
        R = np.empty((B, wcap, DIM), np.uint8)
        CS = np.empty((B, nc_cap, DIM // 32), np.uint8) if fp4 else np.empty((B, nc_cap), np.float32)
        RS = np.empty((B, wcap), np.float32)
        for b in range(B):
            if fp4:
                C[b], CS[b] = normal_mxfp4_rows(seed, "C", b, nc_cap, DIM)
            else:
                C[b], CS[b] = normal_e4m3_rows(seed, "C", b, nc_cap, DIM)
            R[b], RS[b] = normal_e4m3_rows(seed, "R", b, wcap, DIM)
        with_compress = compress_codes
    Xp = Zp = beta = None
    if ratio == 2 and with_compress:
        Xp = np.empty((B, 2, DIM), np.uint16)
        Zp = np.empty((B, 2, DIM), np.uint16)
        for b in range(B):
            Xp[b] = normal_bf16(seed, "Xp", b, (2, DIM))
            Zp[b] = normal_bf16(seed, "Zp", b, (2, DIM))
        beta = normal_f32(seed, "beta", 0, (2, DIM))
    return Workload(name=name, kind="decode", ratio=ratio, key_dtype=key_dtype, B=B, T=T,
                    nc_cap=nc_cap, wcap=wcap, seq=seq, pos=pos, q=q, qI=qI, w=w, C=C, KI=KI,
                    KS=KS, R=R, Xp=Xp, Zp=Zp, beta=beta, seed=seed, kv_dtype=kv_dtype, CS=CS, RS=RS)


def make_decode_mq(B: int, n_raw, G: int = 6, ratio: int = 2, key_dtype: str = "bf16",
                   seed: int = 0, name: str = "decode-mq", nc_cap: Optional[int] = None) -> Workload:
    """B sequences, G decode queries each at raw positions n_raw-G .. n_raw-1 (a verified
    token and the G-1 drafted tokens after it). Queries g*G .. g*G+G-1 read sequence g; the
    block's own latents, index keys and window rows are already in the stores. The window
    store holds 128 + G rows, so no query's window wraps onto another's rows."""
    n_raw = np.broadcast_to(np.asarray(n_raw, dtype=np.int64), (B,)).copy()
    assert np.all(n_raw >= G)
    T = B * G
    seq = np.repeat(np.arange(B, dtype=np.int32), G)
    pos = (np.repeat(n_raw, G) - G + np.tile(np.arange(G), B)).astype(np.int32)
    vis = (pos.astype(np.int64) + 1) // ratio
    if nc_cap is None:
        nc_cap = int(max(1, vis.max()))
    wcap = WINDOW + G
    q = np.empty((T, HEADS, DIM), np.uint16)
    qI = np.empty((T, IDX_HEADS, IDX_DIM), np.uint16)
    w = np.empty((T, IDX_HEADS), np.float32)
    C = np.empty((B, nc_cap, DIM), np.uint16)
    R = np.empty((B, wcap, DIM), np.uint16)
    for b in range(B):
        q[b * G:(b + 1) * G] = normal_bf16(seed, "q-mq", b, (G, HEADS, DIM))
        qI[b * G:(b + 1) * G] = normal_bf16(seed, "qI-mq", b, (G, IDX_HEADS, IDX_DIM))
        w[b * G:(b + 1) * G] = uniform_f32(seed, "w-mq", b, (G, IDX_HEADS))
        C[b] = normal_bf16(seed, "C", b, (nc_cap, DIM))
        R[b] = normal_bf16(seed, "R", b, (wcap, DIM))
    KI, KS = _keys(seed, key_dtype, B, nc_cap)
    return Workload(name=name, kind="decode", ratio=ratio, key_dtype=key_dtype, B=B, T=T,
                    nc_cap=nc_cap, wcap=wcap, seq=seq, pos=pos, q=q, qI=qI, w=w, C=C, KI=KI,
                    KS=KS, R=R, seed=seed, group=G)


def make_ragged(n_raw, lengths, ratio: int = 2, key_dtype: str = "bf16", seed: int = 0,
                name: str = "ragged") -> Workload:
    """A ragged batch: sequence b contributes lengths[b] consecutive queries at raw positions
    n_raw[b] - lengths[b] .. n_raw[b] - 1 (a prefill chunk, a decode step with drafted tokens,
    or one decode query), in sequence order. Their latents, keys and window rows are already
    in the stores; the window store holds 128 + max(lengths) rows."""
    n_raw = np.asarray(n_raw, dtype=np.int64)
    lengths = np.asarray(lengths, dtype=np.int64)
    B = len(n_raw)
    assert len(lengths) == B and np.all(lengths >= 1) and np.all(n_raw >= lengths)
    T = int(lengths.sum())
    seq = np.repeat(np.arange(B, dtype=np.int32), lengths)
    pos = np.concatenate([n_raw[b] - lengths[b] + np.arange(lengths[b]) for b in range(B)]).astype(np.int32)
    nc_cap = int(max(1, ((pos.astype(np.int64) + 1) // ratio).max()))
    wcap = WINDOW + int(lengths.max())
    q = np.empty((T, HEADS, DIM), np.uint16)
    qI = np.empty((T, IDX_HEADS, IDX_DIM), np.uint16)
    w = np.empty((T, IDX_HEADS), np.float32)
    C = np.empty((B, nc_cap, DIM), np.uint16)
    R = np.empty((B, wcap, DIM), np.uint16)
    t0 = 0
    for b in range(B):
        L = int(lengths[b])
        q[t0:t0 + L] = normal_bf16(seed, "q-mq", b, (L, HEADS, DIM))
        qI[t0:t0 + L] = normal_bf16(seed, "qI-mq", b, (L, IDX_HEADS, IDX_DIM))
        w[t0:t0 + L] = uniform_f32(seed, "w-mq", b, (L, IDX_HEADS))
        C[b] = normal_bf16(seed, "C", b, (nc_cap, DIM))
        R[b] = normal_bf16(seed, "R", b, (wcap, DIM))
        t0 += L
    KI, KS = _keys(seed, key_dtype, B, nc_cap)
    return Workload(name=name, kind="decode", ratio=ratio, key_dtype=key_dtype, B=B, T=T,
                    nc_cap=nc_cap, wcap=wcap, seq=seq, pos=pos, q=q, qI=qI, w=w, C=C, KI=KI,
                    KS=KS, R=R, seed=seed, runs=[int(x) for x in lengths])


def make_prefill(T: int, offset: int, ratio: int = 1, key_dtype: str = "bf16", seed: int = 0,
                 name: str = "prefill", wcap: Optional[int] = None) -> Workload:
    """One sequence; a chunk of T causal queries at raw positions offset .. offset+T-1.

    The chunk's own latents, index keys and window rows are already in the stores.
    """
    pos = (offset + np.arange(T, dtype=np.int64)).astype(np.int32)
    nc_cap = (offset + T) // ratio
    if wcap is None:
        wcap = T + WINDOW
    B = 1
    q = normal_bf16(seed, "q", 0, (T, HEADS, DIM))
    qI = normal_bf16(seed, "qI", 0, (T, IDX_HEADS, IDX_DIM))
    w = uniform_f32(seed, "w", 0, (T, IDX_HEADS))
    C = normal_bf16(seed, "C", 0, (1, nc_cap, DIM))
    R = normal_bf16(seed, "R", 0, (1, wcap, DIM))
    KI, KS = _keys(seed, key_dtype, 1, nc_cap)
    return Workload(name=name, kind="prefill", ratio=ratio, key_dtype=key_dtype, B=B, T=T,
                    nc_cap=nc_cap, wcap=wcap, seq=np.zeros(T, np.int32), pos=pos, q=q, qI=qI,
                    w=w, C=C, KI=KI, KS=KS, R=R, seed=seed)


def make_compress_input(B: int, n_raw: int, seed: int = 0):
    """Raw latents X, gate logits Z [B, n_raw, 512] bf16 bits and slot bias beta [2,512] fp32."""
    X = np.empty((B, n_raw, DIM), np.uint16)
    Z = np.empty((B, n_raw, DIM), np.uint16)
    for b in range(B):
        X[b] = normal_bf16(seed, "Xraw", b, (n_raw, DIM))
        Z[b] = normal_bf16(seed, "Zraw", b, (n_raw, DIM))
    beta = normal_f32(seed, "beta", 1, (2, DIM))
    return X, Z, beta


# The five measured workloads, named by what they are.
WORKLOADS = {
    "decode-b4-ctx2k": dict(kind="decode", B=4, n_raw=2048, ratio=2, key_dtype="bf16"),
    "decode-b64-ctx32k": dict(kind="decode", B=64, n_raw=32768, ratio=2, key_dtype="bf16"),
    "decode-b128-ctx128k-fp8": dict(kind="decode", B=128, n_raw=131072, ratio=2, key_dtype="fp8"),
    "prefill-4096-at-61440": dict(kind="prefill", T=4096, offset=61440, ratio=1, key_dtype="bf16"),
    "decode-b8-ctx1m-fp8": dict(kind="decode", B=8, n_raw=1048576, ratio=2, key_dtype="fp8"),
}


# Further workloads of the same layer: a multi-token decode step (the verified token and
# 5 drafted tokens per sequence: 128 x (1 + 5) = 768 queries, the decode capture size the
# MI355X recipe names for its 5-token draft).
MORE_WORKLOADS = {
    "decode-mq6-b128-ctx128k-fp8": dict(kind="decode_mq", B=128, n_raw=131072, G=6, ratio=2,
                                        key_dtype="fp8"),
    # the multi-token step with the 4-bit indexer cache: each sequence's MXFP4 keys streamed
    # once for its 6 queries
    "decode-mq6-b128-ctx128k-mxfp4": dict(kind="decode_mq", B=128, n_raw=131072, G=6, ratio=2,
                                          key_dtype="mxfp4"),
    # the headline decode batch with the 4-bit indexer cache (MXFP4 keys)
    "decode-b128-ctx128k-mxfp4": dict(kind="decode", B=128, n_raw=131072, ratio=2, key_dtype="mxfp4"),
    # the headline decode batch with e4m3 latent and window rows (fp32 row scales)
    "decode-b128-ctx128k-fp8kv": dict(kind="decode", B=128, n_raw=131072, ratio=2, key_dtype="fp8",
                                      kv_dtype="fp8", compress_codes=True),
    # ... and with MXFP4 latent rows (the 4-bit compressed state) and e4m3 window rows
    "decode-b128-ctx128k-fp4kv": dict(kind="decode", B=128, n_raw=131072, ratio=2, key_dtype="fp8",
                                      kv_dtype="mxfp4", compress_codes=True),
    # a 1-to-1 layer (the ratio of the pages' layers from 20 on) at the 1,048,576-token context:
    # every position is a compressed latent, 131072 blocks of 8
    "decode-b2-ctx1m-r1-fp8": dict(kind="decode", B=2, n_raw=1048576, ratio=1, key_dtype="fp8"),
    # a ragged serving batch at 128K context: two 1024-query prefill chunks, 64 single decode
    # queries and 16 decode steps with 5 drafted tokens (2208 queries, 82 sequences)
    "ragged-2x1024+64+16x6-ctx128k-fp8": dict(kind="ragged", n_raw=[131072] * 82,
                                              lengths=[1024, 1024] + [1] * 64 + [6] * 16,
                                              ratio=2, key_dtype="fp8"),
}


def make(name: str, seed: int = 0) -> Workload:
    cfg = dict(WORKLOADS[name] if name in WORKLOADS else MORE_WORKLOADS[name])
    kind = cfg.pop("kind")
    if kind == "decode":
        return make_decode(name=name, seed=seed, **cfg)
    if kind == "decode_mq":
        return make_decode_mq(name=name, seed=seed, **cfg)
    if kind == "ragged":
        return make_ragged(name=name, seed=seed, **cfg)
    return make_prefill(name=name, seed=seed, **cfg)
