"""sparse_attn_fwd_noalloc (key-split state in the library's fixed per-GPU array, no
workspace) against sparse_attn_fwd with a workspace, through the C ABI: two calls in a row,
the second on a smaller batch (the array keeps the first call's contents), a batch whose
heads are split over two work-groups, then a batch large enough to use no scratch at all. Outputs must meet the parity bar against the
existing entry point (max |diff| <= 2e-2, mean <= 2e-3, lse within 1e-4); the two run the
same kernels with the same splits, so they are also expected to agree bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W
from parity_util import LSE_TOL, OUT_MAX, OUT_MEAN, bf16_dev_to_f64

pytestmark = pytest.mark.gpu


def _batch(B, n_raw, seed, key_dtype="fp8"):
    from sparse_attention_score_amd.step import DeviceBatch
    wl = W.make_decode(B=B, n_raw=n_raw, ratio=2, key_dtype=key_dtype, name=f"noalloc-{B}", seed=seed,
                       with_compress=False)
    d = DeviceBatch(wl)
    d.index()
    d.select()
    torch.cuda.synchronize()
    return d


def _compare(d, what):
    import sparse_attention_score_amd as S
    out_ws = torch.empty_like(d.out)
    lse_ws = torch.empty_like(d.lse)
    S.sparse_attn_fwd(d.plan, d.queries, d.cache, d.q, d.topk, out_ws, lse_ws, workspace=d.workspace)
    out_na = torch.full_like(d.out, float("nan"))
    lse_na = torch.full_like(d.lse, float("nan"))
    S.sparse_attn_fwd_noalloc(d.plan, d.queries, d.cache, d.q, d.topk, out_na, lse_na)
    torch.cuda.synchronize()
    a, b = bf16_dev_to_f64(out_na), bf16_dev_to_f64(out_ws)
    assert np.isfinite(a).all(), what
    diff = np.abs(a - b)
    assert diff.max() <= OUT_MAX and diff.mean() <= OUT_MEAN, (what, diff.max(), diff.mean())
    dl = (lse_na - lse_ws).abs().max().item()
    assert dl <= LSE_TOL, (what, dl)
    assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16)), what
    assert torch.equal(lse_na, lse_ws), what
    print(f"[noalloc] {what}: T={d.T} bit-equal to sparse_attn_fwd with a workspace", flush=True)


def test_noalloc_matches_workspace_entry_point():
    assert torch.cuda.is_available()
    print("[noalloc] T=20 then T=5 (key splits in the fixed array; T=5 also splits its heads), T=40 and "
          "T=100 (no splits)", flush=True)
    d1 = _batch(20, [131072] * 10 + [9001] * 5 + [700, 64, 2, 1, 300], seed=91)
    _compare(d1, "first call")
    d2 = _batch(5, [40000, 1030, 3, 65536, 2048], seed=92, key_dtype="bf16")
    _compare(d2, "second call, smaller batch")
    _compare(d1, "third call, the first batch again")
    d3 = _batch(40, 6000, seed=93)
    _compare(d3, "head sets without key splits")
    d4 = _batch(100, 3000, seed=94)
    _compare(d4, "batch above the split size")
