"""Helpers of the GPU parity tests: move a seeded workload to the device, run
the HIP path through the C-ABI binding, and compare with the oracle.

Tolerance for fp16/bf16 outputs: |gpu - oracle| <= 1e-2 * (1 + |oracle|), on
every compared element; the same bound is applied to the fp32 v.  Metadata and
integer-valued cases are compared bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import lora_serving_build_amd as lsb
import workloads as W

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}
TOL = 1e-2
# A NaN payload that no kernel produces: rows of tokens without an adapter
# must keep it bit for bit.
V_SENTINEL = np.uint32(0x7FC0DEAD)


def dev_bits(bits: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")
    return t.view(TORCH_DT[dtype])


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    return W.bits_to_f32(bits, dtype).astype(np.float64)


def tol_ratio(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / (TOL * (1 + |ref|)); <= 1 passes.  NaN counts as a failure."""
    if gpu.size == 0:
        return 0.0
    err = np.abs(gpu - ref) / (TOL * (1.0 + np.abs(ref)))
    if np.isnan(err).any():
        return float("inf")
    return float(err.max())


def sentinel_v(T: int, r: int, ldv: int | None = None) -> torch.Tensor:
    ldv = ldv or r
    v = torch.from_numpy(np.full((T, ldv), V_SENTINEL, np.uint32).view(np.float32)).cuda()
    return v


class DeviceWorkload:
    """A workload's inputs on the GPU (y buffers start as copies of y0)."""

    def __init__(self, w: W.Workload, ldv: int | None = None):
        self.w = w
        self.ids = torch.from_numpy(w.ids.astype(np.int32)).cuda()
        self.x = dev_bits(w.x, w.dtype)
        self.A = dev_bits(w.A, w.dtype)
        self.Bs = [[dev_bits(s.B, w.dtype) for s in o.slices] for o in w.outputs]
        self.ys = [dev_bits(o.y0, w.dtype).clone() for o in w.outputs]
        self.v = sentinel_v(w.T, w.r, ldv)

    def run(self, add: bool | None = None, lora_rank: np.ndarray | None = None):
        """build -> shrink -> expand of every output; lora_rank (optional):
        the per-adapter live ranks handed to the segment kernels."""
        w = self.w
        add = w.add if add is None else add
        rk = torch.from_numpy(np.ascontiguousarray(lora_rank, np.int32)).cuda() if lora_rank is not None else None
        seg = lsb.lora_build_segments(self.ids, w.L, lora_rank=rk)
        lsb.lora_shrink(self.x, self.A, seg, self.v)
        for o, Bs, y in zip(w.outputs, self.Bs, self.ys):
            if len(o.slices) == 1 and o.slices[0].col_off == 0:
                lsb.lora_expand(self.v, Bs[0], seg, y, add)
            else:
                lsb.lora_expand_slice(self.v, Bs, [s.col_off for s in o.slices], seg, y, add)
        torch.cuda.synchronize()
        self.seg = seg
        return seg


def seg_host(seg: lsb.Segments):
    T = seg.num_tokens
    return (seg.sorted_token[:T].cpu().numpy(), seg.seg_lora.cpu().numpy(),
            seg.seg_start.cpu().numpy(), seg.counts.cpu().numpy())


def check_neg_rows(dw: DeviceWorkload):
    """Rows of tokens without an adapter: v keeps its sentinel, y keeps y0."""
    w = dw.w
    inactive = np.nonzero(~w.active)[0]
    if inactive.size == 0:
        return
    vb = dw.v.cpu().numpy().view(np.uint32)
    assert np.all(vb[inactive] == V_SENTINEL)
    idx = torch.from_numpy(inactive).cuda()
    for o, y in zip(w.outputs, dw.ys):
        got = host_bits(y.index_select(0, idx))
        assert np.array_equal(got, o.y0[inactive])


def check_outside_slices(dw: DeviceWorkload):
    """Columns that no slice covers keep y0 in every row."""
    w = dw.w
    for o, y in zip(w.outputs, dw.ys):
        covered = np.zeros(o.ldy, bool)
        for s in o.slices:
            covered[s.col_off:s.col_off + s.n] = True
        if covered.all():
            continue
        cols = torch.from_numpy(np.nonzero(~covered)[0]).cuda()
        got = host_bits(y.index_select(1, cols))
        assert np.array_equal(got, o.y0[:, ~covered])
