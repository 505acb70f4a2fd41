"""The seeded input generator: shapes, structure and determinism (CPU only)."""
import numpy as np
import pytest

import workloads as W


def test_bf16_rounding_is_rne():
    import torch
    a = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 100
    a[:4] = [0.0, -0.0, np.inf, -np.inf]
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_bits(a, "bf16"), ref)
    assert np.array_equal(W.bits_to_f32(W.f32_to_bits(a, "bf16"), "bf16"),
                          torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_deterministic():
    a = W.config(2)
    b = W.config(2)
    assert np.array_equal(a.ids, b.ids) and np.array_equal(a.x, b.x)
    assert np.array_equal(a.outputs[0].slices[0].B, b.outputs[0].slices[0].B)


@pytest.mark.parametrize("k", [1, 2, 3])
def test_small_configs_shapes(k):
    w = W.config(k)
    T, H, r = {1: (16, 1024, 16), 2: (256, 4096, 16), 3: (2048, 4096, 16)}[k]
    assert (w.T, w.H, w.r, w.L) == (T, H, r, 4)
    assert w.x.shape == (T, H) and w.A.shape == (4, r, H)
    assert w.outputs[0].slices[0].B.shape == (4, H if k > 1 else 1024, r)
    assert w.ids.min() >= 0 and w.ids.max() < 4
    if k == 3:
        assert np.all(np.diff(w.ids) >= 0)          # sorted by adapter id
        assert all(n == 8 for n in w.seq_lens)


def test_mixed_rank_padding_structure():
    w = W.make("t", "bf16", 512, 256, 128, 16, [[64, 32], [48]], seed=4, seq_len=(1, 64),
               neg_frac=0.1, ranks_from=[8, 16, 32, 64, 128])
    for l in range(16):
        rl = w.ranks[l]
        assert np.all(w.A[l, rl:] == 0)
        for o in w.outputs:
            for s in o.slices:
                assert np.all(s.B[l, :, rl:] == 0)
                assert np.any(s.B[l, :, :rl] != 0)
    assert sum(w.seq_lens) == 512 and max(w.seq_lens) <= 64
    # -1 is drawn per sequence: every sequence is all -1 or all active
    pos = 0
    for n in w.seq_lens:
        seg = w.ids[pos:pos + n]
        assert np.all(seg == seg[0])
        pos += n


def test_zipf_popularity():
    w = W.make("t", "bf16", 60000, 8, 8, 64, [[8]], seed=3, seq_len=(1, 4), id_dist="zipf",
               zipf_s=1.1)
    seq_ids = np.array([w.ids[sum(w.seq_lens[:i])] for i in range(0, len(w.seq_lens), 1)][:20000])
    freq = np.bincount(seq_ids, minlength=64) / seq_ids.size
    p = W.zipf_probs(64, 1.1)
    assert abs(freq[0] - p[0]) < 0.02 and freq[0] > freq[1] > freq[4] > freq[40]


def test_mixed_batch_structure():
    """make_mixed: prefill sequences on the first adapters, one-token decode
    requests each on an adapter of its own, shuffled; x and weights are
    make()'s."""
    w = W.make_mixed("m", "bf16", 500, 4, 100, 200, 64, 8, [[32]], seed=3, neg_frac=0.0)
    assert w.T == 600 and w.ids.shape == (600,)
    ids = w.ids
    pre = ids[ids < 4]
    dec = ids[ids >= 4]
    assert pre.size == 500 and dec.size == 100
    assert np.unique(dec).size == 100                      # each decode adapter used once
    assert sum(w.seq_lens) == 600
    ref = W.make("m", "bf16", 600, 64, 8, 200, [[32]], seed=3)
    assert np.array_equal(ref.x, w.x) and np.array_equal(ref.A, w.A)
    first_dec = int(np.argmax(ids >= 4))
    assert 0 < first_dec < 600 or ids[0] >= 4               # decode tokens are not all at the end
