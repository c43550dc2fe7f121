"""Comparison rules between the HIP path and the fp64 oracle.

Index sets: the GPU set must hold only visible positions, no duplicates, the same count
as the oracle's, ascending then -1 padded; every position in the symmetric difference
must have an oracle score within 1e-5 relative of the oracle's k-th score (the only
place where fp32 and fp64 rounding may legitimately reorder).
Outputs: max |diff| <= 2e-2 and mean |diff| <= 2e-3 for bf16 data with fp32 accumulation.
"""
import numpy as np

from oracle import oracle as O

TIE_BAND = 1e-5
OUT_MAX = 2e-2
OUT_MEAN = 2e-3
LSE_TOL = 1e-4
SCORE_REL = 2e-6


def kth_score(I: np.ndarray, k: int) -> float:
    n = I.shape[0]
    if n == 0:
        return 0.0
    kk = min(k, n)
    return float(np.sort(I)[::-1][kk - 1])


def check_index_row(gpu_row: np.ndarray, ref_idx: np.ndarray, I_ref: np.ndarray, k: int, what=""):
    """gpu_row: int32 [k] ascending, -1 padded. ref_idx: oracle selection (ascending)."""
    n = I_ref.shape[0]
    cnt = int((gpu_row >= 0).sum())
    assert cnt == ref_idx.shape[0] == min(k, n), f"{what}: count {cnt} vs {ref_idx.shape[0]} (n={n})"
    sel = gpu_row[:cnt]
    assert np.all(gpu_row[cnt:] == -1), f"{what}: padding not -1"
    assert np.all(np.diff(sel) > 0), f"{what}: not strictly ascending"
    assert sel.min(initial=0) >= 0 and (cnt == 0 or sel.max() < n), f"{what}: position out of range"
    diff = np.setxor1d(sel.astype(np.int64), ref_idx.astype(np.int64))
    if diff.size:
        Ik = kth_score(I_ref, k)
        bad = diff[np.abs(I_ref[diff] - Ik) > TIE_BAND * abs(Ik)]
        assert bad.size == 0, (f"{what}: {diff.size} positions differ, {bad.size} outside the tie band; "
                               f"e.g. j={bad[:5]} I={I_ref[bad[:5]]} kth={Ik}")
    return diff.size


def check_outputs(o_gpu: np.ndarray, o_ref: np.ndarray, what="", max_tol=OUT_MAX, mean_tol=OUT_MEAN):
    d = np.abs(o_gpu.astype(np.float64) - o_ref)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite output"
    mx, mn = float(d.max()), float(d.mean())
    assert mx <= max_tol and mn <= mean_tol, f"{what}: max {mx:.3g} mean {mn:.3g}"
    return mx, mn


def bf16_dev_to_f64(t) -> np.ndarray:
    """bfloat16 torch tensor (any device) -> float64 numpy, through the oracle's own decoder."""
    import torch
    bits = t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
    return O.bf16_to_f64(bits)


def bf16_ulp(ref: np.ndarray) -> np.ndarray:
    """One bf16 ulp at each value of ref (8 significant bits)."""
    return 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)


def compress_tol(ref: np.ndarray, x0: np.ndarray, x1: np.ndarray) -> np.ndarray:
    """Error bound of the fp32 compressor after rounding to bf16: one bf16 ulp of the result
    plus 16 fp32 unit roundoffs of the slot magnitudes (the gate exp, reciprocal and blend
    are evaluated in fp32, so near cancellation the absolute error scales with |x|)."""
    return bf16_ulp(ref) + 2.0 ** -20 * (np.abs(x0) + np.abs(x1))
