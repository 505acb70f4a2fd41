"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: a library
routine on a special case that reduces to it, exact integer arithmetic, exact
rational arithmetic on tiny inputs, an independent dense re-association, a
brute-force sort, or an invariant the pages state.  Shapes use distinct H, r
and n so that a transposed operand or a swapped index cannot pass.
"""
from fractions import Fraction
import itertools
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _decode(bits, dtype):
    # Independent widening through numpy / bit patterns (not the oracle's).
    return W.bits_to_f32(bits, dtype).astype(np.float64)


# ------------------------------------------------------------------ decoding
def test_decode_f16_exhaustive(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros and infinities keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_bf16_exhaustive(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.decode(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ------------------------------------------------------------------ metadata
def _brute_segments(ids, L):
    T = len(ids)
    act = [0 <= i < L for i in ids]
    order = sorted(range(T), key=lambda t: (not act[t], ids[t] if act[t] else 0, t))
    t_a = sum(act)
    seg_lora, seg_start = [], []
    pos = 0
    for key, grp in itertools.groupby(order[:t_a], key=lambda t: ids[t]):
        n = len(list(grp))
        seg_lora.append(key)
        seg_start.append(pos)
        pos += n
    S = len(seg_lora)
    lens = [seg_start[i + 1] - seg_start[i] for i in range(S - 1)] + ([t_a - seg_start[-1]] if S else [])
    bad = sum(1 for i in ids if not (0 <= i < L) and i != -1)
    return (np.array(order, np.int32),
            np.array(seg_lora + [-1] * (L - S), np.int32),
            np.array(seg_start + [t_a] * (L + 1 - S), np.int32),
            np.array([S, t_a, max(lens) if lens else 0, bad], np.int32))


@pytest.mark.parametrize("T,L,kind", [
    (0, 1, "uniform"), (1, 1, "uniform"), (1, 4, "neg"), (7, 3, "uniform"),
    (64, 4, "uniform"), (257, 4, "neg"), (1000, 64, "bad"), (513, 1, "uniform"),
    (300, 16, "allneg"), (129, 5, "one"), (2048, 200, "bad"),
])
def test_metadata_vs_brute_sort(oracle_mod, T, L, kind):
    rng = np.random.default_rng(T * 31 + L)
    ids = rng.integers(0, L, size=T).astype(np.int32)
    if kind == "neg":
        ids[rng.random(T) < 0.3] = -1
    elif kind == "bad":
        m = rng.random(T)
        ids[m < 0.1] = -1
        ids[(m >= 0.1) & (m < 0.15)] = L + 3
        ids[(m >= 0.15) & (m < 0.2)] = -7
    elif kind == "allneg":
        ids[:] = -1
    elif kind == "one":
        ids[:] = L - 1
    got = oracle_mod.build_segments(ids, L)
    ref = _brute_segments(ids.tolist(), L)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)


# ------------------------------------------------------------------ helpers
def _tiny(seed, dtype, T=6, H=40, r=6, n=24, L=3, neg=True, integer=False):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, L, size=T).astype(np.int32)
    if neg:
        ids[rng.random(T) < 0.3] = -1
    if integer:
        x = W.int_bits(rng, (T, H), -2, 2, dtype)
        A = W.int_bits(rng, (L, r, H), -2, 2, dtype)
        B = W.int_bits(rng, (L, n, r), -2, 2, dtype)
        y0 = W.int_bits(rng, (T, n), -4, 4, dtype)
    else:
        x = W.normal_bits(rng, (T, H), 1.0, dtype)
        A = W.normal_bits(rng, (L, r, H), 1 / np.sqrt(H), dtype)
        B = W.normal_bits(rng, (L, n, r), 1 / np.sqrt(r), dtype)
        y0 = W.normal_bits(rng, (T, n), 1.0, dtype)
    return ids, x, A, B, y0


# ------------------------------------------------------------------ exact rational
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_exact_rational_tiny(oracle_mod, dtype):
    """Pure-Python exact arithmetic (Fractions) on a tiny case: the oracle's
    fp64 result must sit within the fp64 summation error bound of the exact
    value."""
    ids, x, A, B, y0 = _tiny(5, dtype, T=4, H=7, r=3, n=5, L=2)
    ids[0] = 1
    ids[1] = -1
    xd, Ad, Bd, yd = (_decode(a, dtype) for a in (x, A, B, y0))
    v = oracle_mod.shrink(dtype, x, A, ids)
    y = oracle_mod.expand(dtype, v, B, ids, y0, 0, True)
    eps = 2.0 ** -52
    for t in range(4):
        l = ids[t]
        if l < 0:
            assert np.all(np.isnan(v[t]))
            assert np.array_equal(y[t], yd[t])
            continue
        for j in range(3):
            terms = [Fraction(xd[t, h]) * Fraction(Ad[l, j, h]) for h in range(7)]
            exact = sum(terms)
            bound = 7 * eps * float(sum(abs(q) for q in terms))
            assert abs(Fraction(v[t, j]) - exact) <= Fraction(bound)
        for c in range(5):
            exact_v = [sum(Fraction(xd[t, h]) * Fraction(Ad[l, j, h]) for h in range(7)) for j in range(3)]
            terms = [ev * Fraction(Bd[l, c, j]) for j, ev in enumerate(exact_v)]
            exact = Fraction(yd[t, c]) + sum(terms)
            mag = float(abs(Fraction(yd[t, c]))) + float(sum(abs(q) for q in terms))
            assert abs(Fraction(y[t, c]) - exact) <= Fraction(20 * eps * (mag + 1e-300))


# ------------------------------------------------------------------ dense re-association
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("add", [True, False])
def test_dense_reassociation(oracle_mod, dtype, add):
    """y = (add ? y0 : 0) + x . (A_l B_l), with the per-adapter dense H x n
    matrix W_l = A_l B_l formed first by numpy: a different association of the
    same product."""
    ids, x, A, B, y0 = _tiny(11, dtype, T=8, H=48, r=5, n=20, L=3)
    xd, Ad, Bd, yd = (_decode(a, dtype) for a in (x, A, B, y0))
    v = oracle_mod.shrink(dtype, x, A, ids)
    y = oracle_mod.expand(dtype, v, B, ids, y0, 0, add)
    for t in range(8):
        l = ids[t]
        if l < 0:
            assert np.array_equal(y[t], yd[t])
            continue
        Wl = Ad[l].T @ Bd[l].T            # (H x r)(r x n) = H x n
        ref = (yd[t] if add else 0.0) + xd[t] @ Wl
        np.testing.assert_allclose(y[t], ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(v[t], Ad[l] @ xd[t], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_single_adapter_is_plain_matmul(oracle_mod, dtype):
    """With one adapter and no token without one, shrink is x . A_0 and expand
    adds (x . A_0) . B_0: the micro-benchmark PR uses one plain matmul as the
    single-LoRA roofline of exactly this case."""
    T, H, r, n = 33, 96, 12, 40
    rng = np.random.default_rng(3)
    ids = np.zeros(T, np.int32)
    x = W.normal_bits(rng, (T, H), 1.0, dtype)
    A = W.normal_bits(rng, (1, r, H), 1 / np.sqrt(H), dtype)
    B = W.normal_bits(rng, (1, n, r), 1 / np.sqrt(r), dtype)
    y0 = W.normal_bits(rng, (T, n), 1.0, dtype)
    xd, Ad, Bd, yd = (_decode(a, dtype) for a in (x, A, B, y0))
    v = oracle_mod.shrink(dtype, x, A, ids)
    np.testing.assert_allclose(v, xd @ Ad[0].T, rtol=1e-12, atol=1e-12)
    y = oracle_mod.expand(dtype, v, B, ids, y0, 0, True)
    np.testing.assert_allclose(y, yd + (xd @ Ad[0].T) @ Bd[0].T, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ integer exact
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_integer_inputs_exact(oracle_mod, dtype):
    """Integer-valued inputs: every product and partial sum is an integer far
    below 2^53, so the oracle must equal int64 arithmetic exactly."""
    ids, x, A, B, y0 = _tiny(17, dtype, T=30, H=72, r=9, n=28, L=4, integer=True)
    xi, Ai, Bi, yi = (_decode(a, dtype).astype(np.int64) for a in (x, A, B, y0))
    v = oracle_mod.shrink(dtype, x, A, ids)
    y = oracle_mod.expand(dtype, v, B, ids, y0, 0, True)
    for t in range(30):
        l = ids[t]
        if l < 0:
            assert np.all(np.isnan(v[t])) and np.array_equal(y[t], yi[t])
            continue
        vi = Ai[l] @ xi[t]
        assert np.array_equal(v[t], vi.astype(np.float64))
        assert np.array_equal(y[t], (yi[t] + Bi[l] @ vi).astype(np.float64))


# ------------------------------------------------------------------ invariants
def test_neg_and_bad_ids_untouched(oracle_mod):
    dtype = "bf16"
    ids, x, A, B, y0 = _tiny(23, dtype, T=12, H=32, r=4, n=16, L=3)
    ids[2], ids[5], ids[7] = -1, 3, -9          # none, and two out-of-range ids
    sentinel = np.full((12, 4), 12345.5)
    v = oracle_mod.shrink(dtype, x, A, ids, out=sentinel.copy())
    for t in (2, 5, 7):
        assert np.array_equal(v[t], sentinel[t])
    for add in (True, False):
        y = oracle_mod.expand(dtype, v, B, ids, y0, 0, add)
        for t in (2, 5, 7):
            assert np.array_equal(y[t], _decode(y0[t], dtype))


def test_expand_slice_equals_separate_expands(oracle_mod):
    """expand_slice is the same as one expand per slice into that slice's
    columns (micro-benchmark PR: slices emulated by back-to-back calls)."""
    dtype = "bf16"
    rng = np.random.default_rng(9)
    T, r, L = 20, 8, 3
    widths = [24, 8, 16]
    offs = [0, 24, 32]
    ids = rng.integers(-1, L, size=T).astype(np.int32)
    Bs = [W.normal_bits(rng, (L, n, r), 0.3, dtype) for n in widths]
    y0 = W.normal_bits(rng, (T, 48), 1.0, dtype)
    v = rng.standard_normal((T, 3 * r))           # per-slice v via the stride
    for stride in (0, r):
        got = oracle_mod.expand_slice(dtype, v, Bs, offs, ids, y0, True, v_slice_stride=stride)
        parts = [oracle_mod.expand(dtype, v[:, s * stride:s * stride + r], Bs[s], ids, y0,
                                   offs[s], True) for s in range(3)]
        assert np.array_equal(got, np.concatenate(parts, axis=1))


def _rank_bins():
    rows = []
    with open(os.path.join(GOLDEN, "rank_bins.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                a, b = line.split()
                rows.append((int(a), int(b)))
    return rows


def test_rank_bins_match_printed_examples(oracle_mod):
    for r, b in _rank_bins():
        assert oracle_mod.rank_bin(r) == b


@pytest.mark.parametrize("r_true,r_pad", [(r, b) for r, b in _rank_bins()] + [(8, 128), (45, 128)])
def test_rank_padding_invariance(oracle_mod, r_true, r_pad):
    """Zero-padding the rank up to a bin leaves results unchanged (punica
    issue's mitigation); exact in fp64 since only exact zeros are added."""
    dtype = "bf16"
    rng = np.random.default_rng(r_true * 7 + r_pad)
    T, H, n, L = 10, 64, 24, 2
    ids = rng.integers(-1, L, size=T).astype(np.int32)
    x = W.normal_bits(rng, (T, H), 1.0, dtype)
    A = W.normal_bits(rng, (L, r_true, H), 1 / np.sqrt(H), dtype)
    B = W.normal_bits(rng, (L, n, r_true), 1 / np.sqrt(r_true), dtype)
    y0 = W.normal_bits(rng, (T, n), 1.0, dtype)
    Ap = np.zeros((L, r_pad, H), np.uint16)
    Ap[:, :r_true] = A
    Bp = np.zeros((L, n, r_pad), np.uint16)
    Bp[:, :, :r_true] = B
    v = oracle_mod.shrink(dtype, x, A, ids)
    vp = oracle_mod.shrink(dtype, x, Ap, ids)
    act = ids >= 0
    assert np.array_equal(vp[act, :r_true], v[act])
    assert np.all(vp[act, r_true:] == 0)
    y = oracle_mod.expand(dtype, np.nan_to_num(v), B, ids, y0, 0, True)
    yp = oracle_mod.expand(dtype, np.nan_to_num(vp), Bp, ids, y0, 0, True)
    assert np.array_equal(y, yp)


def test_permutation_equivariance(oracle_mod):
    dtype = "f16"
    ids, x, A, B, y0 = _tiny(31, dtype, T=16, H=40, r=6, n=24, L=3)
    perm = np.random.default_rng(1).permutation(16)
    v = oracle_mod.shrink(dtype, x, A, ids)
    vp = oracle_mod.shrink(dtype, x[perm], A, ids[perm])
    assert np.array_equal(np.nan_to_num(vp, nan=7.0), np.nan_to_num(v[perm], nan=7.0))
    y = oracle_mod.expand(dtype, np.nan_to_num(v), B, ids, y0, 0, True)
    yp = oracle_mod.expand(dtype, np.nan_to_num(vp), B, ids[perm], y0[perm], 0, True)
    assert np.array_equal(yp, y[perm])


def test_add_inputs_false_equals_zero_y0(oracle_mod):
    dtype = "bf16"
    ids, x, A, B, y0 = _tiny(41, dtype, T=12, H=40, r=6, n=24, L=3, neg=False)
    v = oracle_mod.shrink(dtype, x, A, ids)
    y_noadd = oracle_mod.expand(dtype, v, B, ids, y0, 0, False)
    y_zero = oracle_mod.expand(dtype, v, B, ids, np.zeros_like(y0), 0, True)
    assert np.array_equal(y_noadd, y_zero)


def test_rows_subset_matches_full(oracle_mod):
    """Evaluating a sample of rows gives the same values as the full pass."""
    dtype = "bf16"
    ids, x, A, B, y0 = _tiny(43, dtype, T=40, H=64, r=8, n=32, L=4)
    rows = np.array([39, 0, 17, 5, 17], np.int32)
    v = oracle_mod.shrink(dtype, x, A, ids)
    vr = oracle_mod.shrink(dtype, x, A, ids, rows=rows)
    assert np.array_equal(np.nan_to_num(vr, nan=3.0), np.nan_to_num(v[rows], nan=3.0))
    y = oracle_mod.expand(dtype, np.nan_to_num(v), B, ids, y0, 0, True)
    yr = oracle_mod.expand(dtype, np.nan_to_num(v), B, ids, y0, 0, True, rows=rows)
    assert np.array_equal(yr, y[rows])


def test_thread_count_does_not_change_results(oracle_mod, tmp_path):
    """Each row's sum order is fixed, so results are bit-identical for any
    OpenMP thread count (checked in a subprocess with one thread)."""
    import subprocess, sys, json
    code = (
        "import sys, json, numpy as np; sys.path.insert(0, %r);"
        "import oracle, workloads as W;"
        "w = W.make('t', 'bf16', 64, 256, 16, 4, [[128]], seed=5, neg_frac=0.2, seq_len=(1, 8));"
        "v = oracle.shrink('bf16', w.x, w.A, w.ids);"
        "print(json.dumps([oracle.num_threads(), float(np.nansum(v * np.arange(v.size).reshape(v.shape)))]))"
    ) % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for th in ("1", "4"):
        env = dict(os.environ, OMP_NUM_THREADS=th)
        outs.append(json.loads(subprocess.check_output([sys.executable, "-c", code], env=env)))
    assert outs[0][0] == 1 and outs[1][0] == 4
    assert outs[0][1] == outs[1][1]


@pytest.mark.parametrize("stride", [0, 8])
def test_expand_slice_against_dense(oracle_mod, stride):
    """Each slice s lands in columns [off_s, off_s + n_s) of y and uses
    v_s = v shifted by s * stride, checked against numpy on decoded values."""
    dtype = "f16"
    rng = np.random.default_rng(101 + stride)
    T, r, L = 14, 8, 3
    widths, offs = [16, 8, 24], [8, 40, 56]        # gaps between slices
    ldy = 88
    ids = rng.integers(-1, L, size=T).astype(np.int32)
    Bs = [W.normal_bits(rng, (L, n, r), 0.3, dtype) for n in widths]
    y0 = W.normal_bits(rng, (T, ldy), 1.0, dtype)
    v = rng.standard_normal((T, 3 * r))
    got = oracle_mod.expand_slice(dtype, v, Bs, offs, ids, y0, True, v_slice_stride=stride)
    yd = _decode(y0, dtype)
    col = 0
    for s, (n, off) in enumerate(zip(widths, offs)):
        Bd = _decode(Bs[s], dtype)
        for t in range(T):
            l = ids[t]
            ref = yd[t, off:off + n].copy()
            if l >= 0:
                ref = ref + Bd[l] @ v[t, s * stride:s * stride + r]
            np.testing.assert_allclose(got[t, col:col + n], ref, rtol=1e-12, atol=1e-12)
        col += n
