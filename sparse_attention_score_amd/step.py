"""One pass of the hot path over a batch: compressor (if a group completes) and indexer in
one launch, candidate + top-512 selection, gather attention. Allocation and call order only;
every stage runs in the library's kernels through the C ABI."""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import (Cache, CompressJob, Plan, Queries, indexer_score, indexer_score_compress, select_topk,
               sparse_attn_compress, sparse_attn_compress_codes, sparse_attn_fwd, workspace_for)


def to_device_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> a bfloat16 device tensor (a bit copy, no rounding)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


class DeviceBatch:
    """Device copies of a batch's inputs and buffers for every stage's outputs.

    `wl` needs the attributes of workloads.Workload (host arrays as bit patterns)."""

    def __init__(self, wl, device="cuda", max_queries: Optional[int] = None):
        self.wl = wl
        self.T = wl.T
        self.ratio = wl.ratio
        dev = torch.device(device)
        kv = getattr(wl, "kv_dtype", "bf16")
        self.plan = Plan(ratio=wl.ratio, key_dtype=wl.key_dtype, kv_dtype=kv,
                         max_queries=max_queries or wl.T, max_compressed=wl.nc_cap)
        self.seq = torch.from_numpy(wl.seq.astype(np.int32)).to(dev)
        self.pos = torch.from_numpy(wl.pos.astype(np.int32)).to(dev)
        self.max_visible = int(((wl.pos.astype(np.int64) + 1) // wl.ratio).max())
        self.queries = Queries(self.seq, self.pos, self.max_visible, getattr(wl, "group", 0),
                               getattr(wl, "runs", None))
        self.q = to_device_bf16(wl.q, dev)
        self.qI = to_device_bf16(wl.qI, dev)
        self.w = torch.from_numpy(wl.w).to(dev)
        self.CS = self.RS = None
        if kv in ("fp8", "mxfp4"):   # code rows with their scales (e4m3 window either way)
            self.C = torch.from_numpy(np.ascontiguousarray(wl.C)).to(dev)
            self.R = torch.from_numpy(np.ascontiguousarray(wl.R)).to(dev)
            self.CS = torch.from_numpy(np.ascontiguousarray(wl.CS)).to(dev)
            self.RS = torch.from_numpy(np.ascontiguousarray(wl.RS)).to(dev)
        else:
            self.C = to_device_bf16(wl.C, dev)
            self.R = to_device_bf16(wl.R, dev)
        if wl.key_dtype in ("fp8", "mxfp4"):
            self.KI = torch.from_numpy(wl.KI).to(dev)
            self.KS = torch.from_numpy(wl.KS).to(dev)
        else:
            self.KI = to_device_bf16(wl.KI, dev)
            self.KS = None
        self.cache = Cache(latents=self.C, window=self.R, idx_keys=self.KI, idx_scales=self.KS,
                           latent_scales=self.CS, window_scales=self.RS)
        # compressor inputs for the group each query completes (ratio 2, uniform position)
        self.groups = wl.compress_groups() if hasattr(wl, "compress_groups") else np.zeros(0)
        self.Xp = self.Zp = self.beta = None
        if len(self.groups):
            self.Xp = to_device_bf16(wl.Xp, dev)
            self.Zp = to_device_bf16(wl.Zp, dev)
            self.beta = torch.from_numpy(wl.beta).to(dev)
        E = (self.max_visible + 7) // 8 * 8
        self.E = E
        ld = max(4, (E + 3) // 4 * 4)
        self.scores = torch.empty((wl.T, ld), dtype=torch.float32, device=dev)
        self.block_max = torch.empty((wl.T, max(4, (E // 8 + 3) // 4 * 4)), dtype=torch.float32, device=dev)
        self.cand = torch.empty((wl.T, 2048), dtype=torch.int32, device=dev)
        self.topk = torch.empty((wl.T, 512), dtype=torch.int32, device=dev)
        self.out = torch.empty((wl.T, 64, 512), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((wl.T, 64), dtype=torch.float32, device=dev)
        self.workspace = workspace_for(self.plan, dev)

    # -- stages -------------------------------------------------------------------------
    def compress(self, stream=None):
        """Compress the group completed by every sequence's query into its compressed row
        n-1 (all queries at one position)."""
        if not len(self.groups):
            return
        wl = self.wl
        n = (int(wl.pos[0]) + 1) // 2
        assert np.all((wl.pos.astype(np.int64) + 1) // 2 == n), "uniform positions required"
        assert len(self.groups) == wl.B and np.array_equal(self.groups, np.arange(wl.B))
        out_view = self.C[:, n - 1]
        if self.CS is not None:   # code rows: codes into C, scales into CS (strides in bytes)
            sc_view = self.CS[:, n - 1]
            sparse_attn_compress_codes(self.plan, self.Xp, 1024, self.Zp, 1024, self.beta, out_view,
                                       self.C.stride(0), sc_view, self.CS.stride(0) * self.CS.element_size(),
                                       wl.B, stream=stream)
            return
        sparse_attn_compress(self.plan, self.Xp, 1024, self.Zp, 1024, self.beta, out_view,
                             self.C.stride(0), wl.B, stream=stream)

    def compress_job(self) -> Optional[CompressJob]:
        """The compress() call's arguments as a job for indexer_score_compress (None without
        compressor inputs)."""
        if not len(self.groups):
            return None
        if getattr(self, "_job", None) is None:
            wl = self.wl
            n = (int(wl.pos[0]) + 1) // 2
            assert np.all((wl.pos.astype(np.int64) + 1) // 2 == n), "uniform positions required"
            assert len(self.groups) == wl.B and np.array_equal(self.groups, np.arange(wl.B))
            out_view = self.C[:, n - 1]
            if self.CS is not None:
                self._job = CompressJob(self.Xp, 1024, self.Zp, 1024, self.beta, out_view, self.C.stride(0), wl.B,
                                        self.CS[:, n - 1], self.CS.stride(0) * self.CS.element_size())
            else:
                self._job = CompressJob(self.Xp, 1024, self.Zp, 1024, self.beta, out_view, self.C.stride(0), wl.B)
        return self._job

    def index(self, stream=None):
        indexer_score(self.plan, self.queries, self.cache, self.qI, self.w, self.scores,
                      self.block_max, stream=stream)

    def index_compress(self, stream=None):
        """compress() and index() in one launch (the compressor's work-groups ride in the
        indexer's grid)."""
        indexer_score_compress(self.plan, self.queries, self.cache, self.qI, self.w, self.scores,
                               self.block_max, self.compress_job(), stream=stream)

    def step_fns(self, fused: bool = True):
        """The launches of one step: the compressor in the indexer's launch (fused) or as a
        launch of its own."""
        if fused:
            return [self.index_compress, self.select, self.attend]
        return [self.compress, self.index, self.select, self.attend]

    def select(self, stream=None, use_block_max=True):
        select_topk(self.plan, self.queries, self.scores, self.block_max if use_block_max else None,
                    self.topk, cand=self.cand, workspace=self.workspace, stream=stream)

    def attend(self, stream=None, topk: Optional[torch.Tensor] = None, split: bool = True):
        # split=False passes no workspace: one work-group per query, whatever T is
        sparse_attn_fwd(self.plan, self.queries, self.cache, self.q,
                        self.topk if topk is None else topk, self.out, self.lse,
                        workspace=self.workspace if split else None, stream=stream)

    def run(self, stream=None, fused: bool = True):
        for f in self.step_fns(fused):
            f(stream)

    def capture(self):
        """One whole step (its three launches) captured in a HIP graph. The library
        enqueues kernels only (no allocation, copy, memset or synchronisation), so every
        launch is recorded; replaying the graph re-runs the step on the same buffers."""
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()          # first launches outside capture (lazy initialisation)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        torch.cuda.synchronize()
        return g
