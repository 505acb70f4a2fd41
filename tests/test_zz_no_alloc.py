"""lora_shrink_noalloc (the shrink whose H-split partial rows go to the
library's static device scratch, for callers that cannot allocate) against
lora_shrink with a workspace, on calls in a row, the later ones smaller:
identical bits where the workspace holds no more chunks of the H split than
the scratch does (both calls then take the same split), else the same
within the tolerance, and both within the oracle's tolerance."""
import numpy as np
import pytest
import torch

import lora_serving_build_amd as lsb
import oracle
import workloads as W
from parity_util import dev_bits, sentinel_v, tol_ratio, V_SENTINEL

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, T, H, r, L, seq_len: tile path with an H split (scratch in use),
    # the second call smaller than the first
    ("bf16", 4096, 8192, 64, 16, (1, 200)),
    ("f16", 700, 4096, 32, 7, (1, 40)),
    # a few sequences of a large adapter pool: the kernel raises the split
    ("bf16", 600, 4096, 16, 900, (100, 300)),
]


def test_noalloc_shrink_matches_workspace_shrink():
    outs = []
    for dtype, T, H, r, L, sl in CASES:
        print(f"\n[case] noalloc shrink {dtype} T={T} H={H} r={r} L={L}", flush=True)
        need = lsb.lora_shrink_workspace_bytes(T, L, H, r)
        assert need > 0   # the noalloc call fits its split into the scratch
        w = W.make("noalloc", dtype, T, H, r, L, [[64]], seed=T + r, seq_len=sl, neg_frac=0.1)
        ids = torch.from_numpy(w.ids).cuda()
        seg = lsb.lora_build_segments(ids, w.L)
        x = dev_bits(w.x, dtype)
        A = dev_bits(w.A, dtype)
        v_ws = sentinel_v(T, r)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        lsb.lora_shrink(x, A, seg, v_ws, workspace=ws)
        v_na = sentinel_v(T, r)
        lsb.lora_shrink_noalloc(x, A, seg, v_na)
        torch.cuda.synchronize()
        a = v_ws.cpu().numpy().view(np.uint32)
        b = v_na.cpu().numpy().view(np.uint32)
        act = w.active
        if need <= lsb.LORA_NOALLOC_SCRATCH_BYTES:
            # the same bound on the split: the same split, the same bits
            assert np.array_equal(a, b)
        else:
            # the scratch holds fewer chunks than the workspace, so the kernel
            # may take another split: the sums differ by rounding only
            assert np.array_equal(a[~act], b[~act])
            assert tol_ratio(v_na.cpu().numpy()[act].astype(np.float64),
                             v_ws.cpu().numpy()[act].astype(np.float64)) <= 1
        assert np.all(b[~act] == V_SENTINEL)
        v_or = oracle.shrink(dtype, w.x, w.A, w.ids)
        assert tol_ratio(v_na.cpu().numpy()[act].astype(np.float64), v_or[act]) <= 1
        outs.append(b)
    assert len(outs) == len(CASES)
