"""GPU parity: the HIP path (through the C-ABI) against the fp64 oracle.

Every test builds seeded inputs with ``workloads``, runs
lora_build_segments -> lora_shrink -> lora_expand[_slice] on the GPU and
compares with the oracle run on the same bits:
  * metadata bit for bit,
  * v and y within |gpu - oracle| <= 1e-2 (1 + |oracle|) ("chained": the
    oracle's own fp64 v feeds its expand; "isolated": the GPU's fp32 v does),
  * integer-valued inputs bit for bit against the oracle rounded once,
  * rows of tokens without an adapter and columns outside the slices
    untouched, bit for bit.
The five named workloads run at full size, each compared on every row
(the largest streamed through the oracle in row blocks).
"""
import math
import os

import numpy as np
import pytest
import torch

import lora_serving_build_amd as lsb
import oracle
import workloads as W
from parity_util import (DeviceWorkload, check_neg_rows, check_outside_slices, decode, dev_bits,
                         host_bits, seg_host, sentinel_v, tol_ratio, V_SENTINEL)

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _slice_cols(o):
    return np.concatenate([np.arange(s.col_off, s.col_off + s.n) for s in o.slices])


def compare_all_rows(dw: DeviceWorkload, isolated=True, max_block_elems=16 << 20):
    """compare_with_oracle over every active row, streamed through the oracle
    in row blocks (no fp64 copy of a whole wide output is ever held)."""
    w = dw.w
    act = np.nonzero(w.active)[0].astype(np.int32)
    widest = max(o.ldy for o in w.outputs)
    block = max(1, max_block_elems // widest)
    worst = (0.0, 0.0, 0.0)
    for b in range(0, act.size, block):
        r = compare_with_oracle(dw, rows=act[b:b + block], isolated=isolated)
        worst = tuple(max(a, c) for a, c in zip(worst, r))
    return worst


def compare_with_oracle(dw: DeviceWorkload, rows=None, isolated=True):
    """Returns the worst tolerance ratios (v, y chained, y isolated)."""
    w = dw.w
    act_rows = np.nonzero(w.active)[0].astype(np.int32)
    rows = act_rows if rows is None else np.asarray(rows, np.int32)
    v_gpu = dw.v.cpu().numpy().astype(np.float64)
    v_or = oracle.shrink(w.dtype, w.x, w.A, w.ids, rows=rows)
    rv = tol_ratio(v_gpu[rows, :w.r], v_or)
    v_full = np.zeros((w.T, w.r))
    v_full[rows] = v_or
    ry = ryi = 0.0
    for o, y in zip(w.outputs, dw.ys):
        Bs = [s.B for s in o.slices]
        offs = [s.col_off for s in o.slices]
        cols = _slice_cols(o)
        got = decode(host_bits(y.index_select(0, torch.from_numpy(rows).long().cuda())), w.dtype)[:, cols]
        ref = oracle.expand_slice(w.dtype, v_full, Bs, offs, w.ids, o.y0, w.add, rows=rows)
        ry = max(ry, tol_ratio(got, ref))
        if isolated:
            ref_i = oracle.expand_slice(w.dtype, np.ascontiguousarray(v_gpu[:, :w.r]), Bs, offs, w.ids,
                                        o.y0, w.add, rows=rows)
            ryi = max(ryi, tol_ratio(got, ref_i))
    return rv, ry, ryi


# ---------------------------------------------------------------- metadata
META_CASES = [(0, 1, "uniform"), (1, 1, "uniform"), (1, 4, "neg"), (7, 3, "uniform"),
              (64, 4, "uniform"), (257, 4, "neg"), (1000, 64, "bad"), (513, 1, "uniform"),
              (300, 16, "allneg"), (129, 5, "one"), (2048, 200, "bad"), (5000, 2048, "neg"),
              (20000, 7, "uniform"), (3000, 3, "sorted"), (8192, 64, "bad"), (8193, 64, "bad"),
              (40000, 300, "bad"), (9000, 1500, "bad"),
              # key widths at powers of two, every lane of a chunk on its own key,
              # the register-reload threshold of the 16-wave form, the largest L
              (256, 63, "uniform"), (256, 64, "cyclic"), (640, 64, "cyclic"), (4096, 1023, "neg"),
              (4096, 1024, "bad"), (32768, 64, "bad"), (32769, 1024, "neg"), (65536, 2048, "bad"),
              (1, 2048, "neg"), (100, 2048, "one"), (2049, 2048, "cyclic")]


@pytest.mark.parametrize("T,L,kind", META_CASES)
def test_segments_bit_exact(T, L, kind):
    _announce(f"segments T={T} L={L} {kind}")
    rng = np.random.default_rng(T * 17 + L)
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
    elif kind == "sorted":
        ids.sort()
    elif kind == "cyclic":
        ids = (np.arange(T) % L).astype(np.int32)
    seg = lsb.lora_build_segments(torch.from_numpy(ids).cuda(), L)
    torch.cuda.synchronize()
    got = seg_host(seg)
    ref = oracle.build_segments(ids, L)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_segments_of_named_workloads(k, named):
    w = named(k)
    _announce(f"segments of {w.name}")
    seg = lsb.lora_build_segments(torch.from_numpy(w.ids).cuda(), w.L)
    torch.cuda.synchronize()
    for g, r in zip(seg_host(seg), oracle.build_segments(w.ids, w.L)):
        assert np.array_equal(g, r)


# ---------------------------------------------------------------- named workloads
@pytest.fixture(scope="module")
def named():
    cache = {}

    def get(k):
        if k not in cache:
            cache.clear()
            cache[k] = W.config(k)
        return cache[k]
    return get


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_named_workload_parity(k, named):
    w = named(k)
    _announce(f"parity {w.name}")
    dw = DeviceWorkload(w)
    seg = dw.run()
    for g, r in zip(seg_host(seg), oracle.build_segments(w.ids, w.L)):
        assert np.array_equal(g, r)
    rv, ry, ryi = compare_with_oracle(dw)
    print(f"  tolerance ratios: v {rv:.3g}  y {ry:.3g}  y(isolated) {ryi:.3g}")
    assert rv <= 1 and ry <= 1 and ryi <= 1
    check_neg_rows(dw)
    check_outside_slices(dw)


@pytest.mark.timeout(900)
def test_largest_workload_every_row(named):
    """The 8192-token, H = 8192, r = 64, 64-adapter layer in the launch
    configuration the benchmark times: metadata bit for bit, v and both
    outputs on every active row and column (streamed through the oracle in
    row blocks), and every untouched row in full."""
    w = named(5)
    _announce(f"parity (every row) {w.name}")
    dw = DeviceWorkload(w)
    seg = dw.run()
    for g, r in zip(seg_host(seg), oracle.build_segments(w.ids, w.L)):
        assert np.array_equal(g, r)
    rv, ry, ryi = compare_all_rows(dw)
    print(f"  rows {w.T_a}; tolerance ratios: v {rv:.3g}  y {ry:.3g}  y(isolated) {ryi:.3g}")
    assert rv <= 1 and ry <= 1 and ryi <= 1
    check_neg_rows(dw)


# ---------------------------------------------------------------- exactness
INT_CASES = [
    ("f16", 200, 256, 16, 4, [[256]], 1),
    ("bf16", 333, 512, 20, 5, [[64, 48, 100]], (1, 40)),
    ("bf16", 97, 1024, 128, 3, [[128]], 1),
    ("f16", 1000, 128, 8, 64, [[72, 8]], (1, 8)),
    ("bf16", 64, 2049, 2, 2, [[33]], 4),
]


@pytest.mark.parametrize("dtype,T,H,r,L,slices,sl", INT_CASES)
def test_integer_inputs_bit_exact(dtype, T, H, r, L, slices, sl):
    """Integer inputs keep every fp32 partial sum exact, so the GPU must equal
    the oracle's exact value rounded once to the output type."""
    _announce(f"integer exact {dtype} T={T} H={H} r={r} L={L} slices={slices}")
    w = W.make("int", dtype, T, H, r, L, slices, seed=T + H + r, seq_len=sl, neg_frac=0.15,
               integer=True)
    dw = DeviceWorkload(w)
    dw.run()
    act = np.nonzero(w.active)[0]
    v_or = oracle.shrink(w.dtype, w.x, w.A, w.ids)
    v_gpu = dw.v.cpu().numpy()
    assert np.array_equal(v_gpu[act].astype(np.float64), v_or[act])
    for o, y in zip(w.outputs, dw.ys):
        ref = oracle.expand_slice(w.dtype, np.nan_to_num(v_or), [s.B for s in o.slices],
                                  [s.col_off for s in o.slices], w.ids, o.y0, w.add)
        ref_bits = W.f32_to_bits(ref.astype(np.float32), dtype) if dtype == "bf16" else \
            ref.astype(np.float16).view(np.uint16)
        got = host_bits(y)[:, _slice_cols(o)]
        assert np.array_equal(got[act], ref_bits[act])
    check_neg_rows(dw)
    check_outside_slices(dw)


# ---------------------------------------------------------------- shapes and edges
EDGE_CASES = [
    # dtype, T, H, r, L, slices, seq_len, neg_frac, id_dist
    ("f16", 1, 64, 16, 1, [[64]], 1, 0.0, "uniform"),
    ("bf16", 77, 2049, 20, 3, [[2049]], (1, 9), 0.2, "uniform"),   # odd H, r: scalar path
    ("f16", 130, 1024, 2, 4, [[100]], 1, 0.1, "uniform"),           # ragged n
    ("bf16", 515, 4096, 128, 8, [[1024, 512]], (1, 100), 0.1, "uniform"),
    ("bf16", 300, 512, 64, 1, [[512]], (1, 300), 0.0, "uniform"),   # one adapter
    ("f16", 4099, 256, 32, 300, [[256]], (1, 3), 0.05, "zipf"),     # many short segments
    ("bf16", 2000, 16384, 16, 4, [[1024]], 8, 0.0, "uniform"),      # widest H of the sweep
    ("f16", 260, 1024, 48, 6, [[40, 24, 8, 128]], (1, 50), 0.3, "uniform"),
    ("f16", 33, 1, 1, 2, [[1]], 1, 0.1, "uniform"),                  # H = r = n = 1
    ("bf16", 17, 8, 1, 3, [[8, 1]], (1, 5), 0.0, "uniform"),         # rank 1, a one-column slice
    ("f16", 1, 4096, 64, 2048, [[4096]], 1, 0.0, "uniform"),        # one token, the most adapters
]


@pytest.mark.parametrize("dtype,T,H,r,L,slices,sl,neg,dist", EDGE_CASES)
def test_edge_shapes(dtype, T, H, r, L, slices, sl, neg, dist):
    _announce(f"edge {dtype} T={T} H={H} r={r} L={L} slices={slices} seq={sl} neg={neg} {dist}")
    w = W.make("edge", dtype, T, H, r, L, slices, seed=T * 3 + r, seq_len=sl, neg_frac=neg,
               id_dist=dist)
    dw = DeviceWorkload(w)
    dw.run()
    rv, ry, ryi = compare_with_oracle(dw)
    print(f"  tolerance ratios: v {rv:.3g}  y {ry:.3g}  y(isolated) {ryi:.3g}")
    assert rv <= 1 and ry <= 1 and ryi <= 1
    check_neg_rows(dw)
    check_outside_slices(dw)


def _random_cases(n=24, seed=2024):
    """Seeded random shapes: odd and aligned H, r and slice widths, one to
    four slices, mixed segment lengths, -1 tokens, every path choice."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ("f16", "bf16")[i % 2]
        T = int(np.exp(rng.uniform(0, np.log(1200)))) if i % 3 == 0 else int(rng.integers(64, 1201))
        H = int(rng.integers(1, 3000))
        if rng.random() < 0.6:
            H = max(8, H // 8 * 8)
        r = int(rng.choice([8, 16, 32, 64, 128])) if rng.random() < 0.5 else int(rng.integers(1, 129))
        L = int(rng.integers(1, 41))
        widths = []
        for _ in range(int(rng.integers(1, 5))):
            wd = int(rng.integers(1, 1500))
            widths.append(max(8, wd // 8 * 8) if rng.random() < 0.6 else wd)
        while T * max(H, sum(widths)) > 3_000_000:
            T = max(1, T // 2)
        sl = (1, int(rng.integers(1, 200)))
        neg = float(rng.choice([0.0, 0.1, 0.3]))
        dist = ("uniform", "zipf")[int(rng.integers(0, 2))]
        path = ("auto", "bgmv", "sgmv")[int(rng.integers(0, 3))]
        if path == "bgmv" and r > 64 and not (r == 128 and H % 8 == 0):
            path = "sgmv"
        cases.append((i, dtype, T, H, r, L, widths, sl, neg, dist, path))
    return cases


@pytest.mark.parametrize("i,dtype,T,H,r,L,widths,sl,neg,dist,path", _random_cases())
def test_random_shapes(force_path, i, dtype, T, H, r, L, widths, sl, neg, dist, path):
    _announce(f"random {i}: {dtype} T={T} H={H} r={r} L={L} slices={widths} seq={sl} neg={neg} "
              f"{dist} path={path}")
    force_path({"auto": lsb.PATH_AUTO, "bgmv": lsb.PATH_BGMV, "sgmv": lsb.PATH_SGMV}[path])
    w = W.make("rand", dtype, T, H, r, L, [widths], seed=1000 + i, seq_len=sl, neg_frac=neg,
               id_dist=dist)
    dw = DeviceWorkload(w)
    dw.run()
    rv, ry, ryi = compare_with_oracle(dw)
    print(f"  tolerance ratios: v {rv:.3g}  y {ry:.3g}  y(isolated) {ryi:.3g}")
    assert rv <= 1 and ry <= 1 and ryi <= 1
    check_neg_rows(dw)
    check_outside_slices(dw)


LARGE_RANDOM = [
    # dtype, T, H, r, L, slices, seq_len, neg_frac, id_dist: multi-round shrink splits and
    # multi-item expands at sizes the oracle checks on sampled rows
    ("bf16", 6000, 8192, 64, 48, [[4096, 1024, 1024]], (1, 400), 0.05, "zipf"),
    ("f16", 8192, 4096, 128, 4, [[5000]], (1, 64), 0.0, "uniform"),
    ("bf16", 3000, 5000, 100, 20, [[2048, 1000]], (1, 300), 0.1, "uniform"),
    ("f16", 4096, 4096, 16, 64, [[4096], [3000, 1000]], (1, 16), 0.2, "zipf"),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype,T,H,r,L,slices,sl,neg,dist", LARGE_RANDOM)
def test_large_shapes_every_row(dtype, T, H, r, L, slices, sl, neg, dist):
    _announce(f"large {dtype} T={T} H={H} r={r} L={L} slices={slices} seq={sl} neg={neg} {dist}")
    w = W.make("large", dtype, T, H, r, L, slices, seed=T + H + r, seq_len=sl, neg_frac=neg,
               id_dist=dist)
    dw = DeviceWorkload(w)
    dw.run()
    rv, ry, ryi = compare_all_rows(dw)
    print(f"  rows {w.T_a}; tolerance ratios: v {rv:.3g}  y {ry:.3g}  y(isolated) {ryi:.3g}")
    assert rv <= 1 and ry <= 1 and ryi <= 1
    check_neg_rows(dw)
    check_outside_slices(dw)


def test_empty_and_all_negative_batches():
    _announce("empty and all -1 batches")
    for T, neg in ((0, 0.0), (50, 1.0)):
        w = W.make("e", "bf16", T, 256, 16, 3, [[64]], seed=9, neg_frac=neg) if T else None
        if T == 0:
            ids = torch.empty(0, dtype=torch.int32, device="cuda")
            seg = lsb.lora_build_segments(ids, 3)
            x = torch.empty(0, 256, dtype=torch.bfloat16, device="cuda")
            A = torch.zeros(3, 16, 256, dtype=torch.bfloat16, device="cuda")
            v = torch.empty(0, 16, device="cuda")
            lsb.lora_shrink(x, A, seg, v)
            B = torch.zeros(3, 64, 16, dtype=torch.bfloat16, device="cuda")
            y = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
            lsb.lora_expand(v, B, seg, y)
            torch.cuda.synchronize()
            assert seg.counts.cpu().tolist() == [0, 0, 0, 0]
            assert seg.seg_lora.cpu().tolist() == [-1, -1, -1]
            assert seg.seg_start.cpu().tolist() == [0, 0, 0, 0]
        else:
            assert not w.active.any()
            dw = DeviceWorkload(w)
            dw.run()
            check_neg_rows(dw)


def test_strided_rows():
    """x with ldx > H, v with ldv > r and y with ldy wider than the slices."""
    _announce("strided rows")
    w = W.make("s", "bf16", 150, 512, 16, 4, [[256]], seed=12, seq_len=(1, 20), neg_frac=0.1)
    x_wide = np.zeros((w.T, 520), np.uint16)
    x_wide[:, :512] = w.x
    xd = dev_bits(x_wide, w.dtype)[:, :512]
    A = dev_bits(w.A, w.dtype)
    ids = torch.from_numpy(w.ids).cuda()
    seg = lsb.lora_build_segments(ids, w.L)
    v = sentinel_v(w.T, 16, ldv=24)[:, :16]
    lsb.lora_shrink(xd, A, seg, v)
    y0_wide = W.normal_bits(np.random.default_rng(1), (w.T, 272), 1.0, w.dtype)
    y = dev_bits(y0_wide, w.dtype)
    B = dev_bits(w.outputs[0].slices[0].B, w.dtype)
    lsb.lora_expand_slice(v, [B], [8], seg, y, True)
    torch.cuda.synchronize()
    act = np.nonzero(w.active)[0]
    v_or = oracle.shrink(w.dtype, w.x, w.A, w.ids)
    vg = v.cpu().numpy().astype(np.float64)
    assert tol_ratio(vg[act], v_or[act]) <= 1
    ref = oracle.expand(w.dtype, np.nan_to_num(v_or), w.outputs[0].slices[0].B, w.ids, y0_wide, 8, True)
    got = decode(host_bits(y), w.dtype)
    assert tol_ratio(got[act][:, 8:264], ref[act]) <= 1
    outside = np.r_[0:8, 264:272]
    assert np.array_equal(host_bits(y)[:, outside], y0_wide[:, outside])
    inact = np.nonzero(~w.active)[0]
    assert np.array_equal(host_bits(y)[inact], y0_wide[inact])


def test_expand_slice_equals_separate_expands():
    """expand_slice gives the same bits as one lora_expand per slice into a
    column view (the micro-benchmark PR emulates slices that way)."""
    _announce("expand_slice vs separate expands")
    w = W.make("q", "bf16", 700, 1024, 32, 6, [[256, 64, 64]], seed=21, seq_len=(1, 30), neg_frac=0.1)
    dw = DeviceWorkload(w)
    dw.run()
    y2 = dev_bits(w.outputs[0].y0, w.dtype)
    for s, B in zip(w.outputs[0].slices, dw.Bs[0]):
        lsb.lora_expand(dw.v, B, dw.seg, y2[:, s.col_off:s.col_off + s.n], True)
    torch.cuda.synchronize()
    assert torch.equal(dw.ys[0].view(torch.int16), y2.view(torch.int16))


def test_v_slice_stride():
    """Per-slice v through v_slice_stride against the oracle."""
    _announce("v_slice_stride")
    w = W.make("vs", "f16", 200, 256, 16, 3, [[128, 64]], seed=31, seq_len=(1, 10), neg_frac=0.1)
    ids = torch.from_numpy(w.ids).cuda()
    seg = lsb.lora_build_segments(ids, w.L)
    vh = np.random.default_rng(2).standard_normal((w.T, 32)).astype(np.float32)
    v = torch.from_numpy(vh).cuda()
    y = dev_bits(w.outputs[0].y0, w.dtype)
    Bs = [dev_bits(s.B, w.dtype) for s in w.outputs[0].slices]
    lsb.lora_expand_slice(v, Bs, [0, 128], seg, y, True, v_slice_stride=16)
    torch.cuda.synchronize()
    ref = oracle.expand_slice(w.dtype, vh.astype(np.float64), [s.B for s in w.outputs[0].slices],
                              [0, 128], w.ids, w.outputs[0].y0, True, v_slice_stride=16)
    act = w.active
    assert tol_ratio(decode(host_bits(y), w.dtype)[act], ref[act]) <= 1


def test_add_inputs_false():
    _announce("add_inputs = False")
    w = W.make("na", "bf16", 400, 1024, 16, 4, [[512]], seed=41, seq_len=(1, 16), neg_frac=0.2,
               add=False)
    dw = DeviceWorkload(w)
    dw.run()
    rv, ry, ryi = compare_with_oracle(dw)
    assert rv <= 1 and ry <= 1 and ryi <= 1
    check_neg_rows(dw)


def _rank_pairs():
    pairs = []
    with open(os.path.join(os.path.dirname(__file__), "golden", "rank_bins.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                a, b = line.split()
                pairs.append((int(a), int(b)))
    return pairs + [(8, 128), (45, 128)]


@pytest.mark.parametrize("r_true,r_pad", _rank_pairs())
def test_rank_padding(r_true, r_pad, force_path):
    """Zero-padding the rank (punica issue's mitigation): the padded run gives
    the oracle's true-rank result within tolerance, its padded v columns are
    exactly zero, and expand fed the same v gives the same bits for the true and
    the padded rank (the extra products are exact zeros).  Shrink may split the
    H-sum differently for different ranks, so chained results are compared
    within tolerance only."""
    _announce(f"rank padding {r_true} -> {r_pad}")
    w = W.make("rp", "bf16", 300, 1024, r_true, 5, [[512]], seed=r_true, seq_len=(1, 20), neg_frac=0.1)
    Ap = np.zeros((w.L, r_pad, w.H), np.uint16)
    Ap[:, :r_true] = w.A
    B = w.outputs[0].slices[0].B
    Bp = np.zeros((w.L, B.shape[1], r_pad), np.uint16)
    Bp[:, :, :r_true] = B
    ids = torch.from_numpy(w.ids).cuda()
    seg = lsb.lora_build_segments(ids, w.L)
    x = dev_bits(w.x, w.dtype)
    act = w.active
    v_or = oracle.shrink(w.dtype, w.x, w.A, w.ids)
    ref = oracle.expand(w.dtype, np.nan_to_num(v_or), B, w.ids, w.outputs[0].y0, 0, True)
    vs = []
    for A_, B_, rr in ((w.A, B, r_true), (Ap, Bp, r_pad)):
        v = sentinel_v(w.T, rr)
        lsb.lora_shrink(x, dev_bits(A_, w.dtype), seg, v)
        y = dev_bits(w.outputs[0].y0, w.dtype)
        lsb.lora_expand(v, dev_bits(B_, w.dtype), seg, y, True)
        torch.cuda.synchronize()
        vg = v.cpu().numpy()
        assert tol_ratio(vg[act, :r_true].astype(np.float64), v_or[act]) <= 1
        assert tol_ratio(decode(host_bits(y), w.dtype)[act], ref[act]) <= 1
        vs.append(v)
    assert np.all(vs[1].cpu().numpy()[act, r_true:] == 0)
    # Same v into both expands, on one kernel family at a time: identical bits.
    v_pad = torch.zeros(w.T, r_pad, device="cuda")
    v_pad[:, :r_true] = vs[0]
    modes = [lsb.PATH_SGMV] + ([lsb.PATH_BGMV] if (r_pad <= 64 or r_pad == 128) else [])
    for mode in modes:
        force_path(mode)
        ys = []
        for vv, B_ in ((vs[0], B), (v_pad, Bp)):
            y = dev_bits(w.outputs[0].y0, w.dtype)
            lsb.lora_expand(vv, dev_bits(B_, w.dtype), seg, y, True)
            ys.append(y)
        torch.cuda.synchronize()
        assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16)), f"path {mode}"


def test_shrink_repeatable_and_workspace_reuse(force_path):
    """The segment-tile shrink with its H split (partial rows in the
    workspace, then the reduce kernel) overwrites v: repeated calls give
    identical bits, also with a workspace that starts full of garbage and
    after a call on a different batch has used it."""
    _announce("shrink repeatability")
    force_path(lsb.PATH_SGMV)
    big = W.make("rep", "f16", 256, 4096, 16, 4, [[64]], seed=51)
    small = W.make("rep2", "f16", 40, 4096, 16, 4, [[64]], seed=52, neg_frac=0.2, seq_len=(1, 5))
    need = max(lsb.lora_shrink_workspace_bytes(w.T, w.L, w.H, w.r) for w in (big, small))
    assert lsb.lora_shrink_workspace_bytes(256, 4, 4096, 16) > 0
    ws = torch.from_numpy(np.random.default_rng(3).integers(0, 256, need, dtype=np.uint8)).cuda()
    res = []
    for w in (big, small, big):
        ids = torch.from_numpy(w.ids).cuda()
        seg = lsb.lora_build_segments(ids, w.L)
        v = sentinel_v(w.T, 16)
        lsb.lora_shrink(dev_bits(w.x, w.dtype), dev_bits(w.A, w.dtype), seg, v, workspace=ws)
        lsb.lora_shrink(dev_bits(w.x, w.dtype), dev_bits(w.A, w.dtype), seg, v, workspace=ws)
        torch.cuda.synchronize()
        res.append(v.cpu().numpy().view(np.uint32).copy())
        act = w.active
        v_or = oracle.shrink(w.dtype, w.x, w.A, w.ids)
        assert tol_ratio(v.cpu().numpy()[act].astype(np.float64), v_or[act]) <= 1
        assert np.all(res[-1][~act] == V_SENTINEL)
    assert np.array_equal(res[0], res[2])


@pytest.mark.parametrize("dtype,T,H,r,L,sl", [
    ("bf16", 4096, 8192, 64, 16, (1, 200)),   # the host's split equals what the workspace holds
    ("f16", 5000, 4096, 48, 5, (1, 600)),
    ("bf16", 6000, 2048, 64, 40, (1, 300)),
    ("f16", 4096, 2048, 40, 7, (1, 100)),     # the smallest batch and H that take 128-token tiles
    ("bf16", 4500, 4096, 64, 600, (1, 60)),   # a pool of 600 adapters: lazy tile table
])
def test_shrink_128_token_tiles_every_row(dtype, T, H, r, L, sl):
    """The shrink at r = 33..64 from 4096 tokens (128-token tiles, the H split
    chosen in the kernel from the true tile count): every active row against
    the oracle, with a workspace that starts full of garbage, so a reduce that
    summed chunks the kernel did not write would show."""
    _announce(f"shrink, 128-token tiles: {dtype} T={T} H={H} r={r} L={L}")
    w = W.make("tb2", dtype, T, H, r, L, [[64]], seed=T + H + r, seq_len=sl, neg_frac=0.1)
    ids = torch.from_numpy(w.ids).cuda()
    seg = lsb.lora_build_segments(ids, w.L)
    need = lsb.lora_shrink_workspace_bytes(T, L, H, r)
    ws = torch.from_numpy(np.random.default_rng(T).integers(0, 256, need, dtype=np.uint8)).cuda()
    v = sentinel_v(T, r)
    lsb.lora_shrink(dev_bits(w.x, dtype), dev_bits(w.A, dtype), seg, v, workspace=ws)
    torch.cuda.synchronize()
    act = w.active
    v_or = oracle.shrink(dtype, w.x, w.A, w.ids)
    assert tol_ratio(v.cpu().numpy()[act].astype(np.float64), v_or[act]) <= 1
    assert np.all(v.cpu().numpy().view(np.uint32)[~act] == V_SENTINEL)


@pytest.mark.parametrize("dtype,T,H,r,L,sl", [
    ("f16", 2048, 1024, 16, 4, 8),        # 2048 tokens in 8-token sequences, sorted by the builder
    ("bf16", 1024, 2048, 16, 4, 1),       # one token per sequence
    ("bf16", 3000, 1024, 32, 9, (1, 40)),  # ragged segments, two rank tiles, 10 % without adapter
])
def test_shrink_groups_chosen_at_size(force_path, dtype, T, H, r, L, sl):
    """Mid-size batches at small H, where the launcher itself takes the
    16-token groups (no workspace): every active row against the oracle, and
    the rows without an adapter left as they were."""
    _announce(f"shrink, 16-token groups by the launcher: {dtype} T={T} H={H} r={r} L={L}")
    force_path(lsb.PATH_SGMV)
    assert lsb.lora_shrink_workspace_bytes(T, L, H, r) == 0
    w = W.make("grp", dtype, T, H, r, L, [[64]], seed=T + H + r, seq_len=sl,
               neg_frac=0.1 if isinstance(sl, tuple) else 0.0)
    seg = lsb.lora_build_segments(torch.from_numpy(w.ids).cuda(), w.L)
    v = sentinel_v(T, r)
    lsb.lora_shrink(dev_bits(w.x, dtype), dev_bits(w.A, dtype), seg, v)
    torch.cuda.synchronize()
    act = w.active
    v_or = oracle.shrink(dtype, w.x, w.A, w.ids)
    assert tol_ratio(v.cpu().numpy()[act].astype(np.float64), v_or[act]) <= 1
    assert np.all(v.cpu().numpy().view(np.uint32)[~act] == V_SENTINEL)


@pytest.mark.parametrize("dtype,T,H,r", [("bf16", 700, 4096, 16), ("f16", 301, 2001, 32)])
def test_single_adapter_shrink_groups(force_path, monkeypatch, tuning_from_env, dtype, T, H, r):
    """lora_shrink_single in the 16-token-group form (forced): bit for bit
    the segment entry point on the same batch with every id 0 (the same
    groups and block order), and the oracle's result."""
    _announce(f"single-adapter shrink, 16-token groups: {dtype} T={T} H={H} r={r}")
    monkeypatch.setenv("LORA_SHRINK_GROUP", "1")
    tuning_from_env()
    force_path(lsb.PATH_SGMV)
    w = W.make("grp_single", dtype, T, H, r, 1, [[64]], seed=T + H + r)
    x = dev_bits(w.x, dtype)
    A = dev_bits(w.A, dtype)
    v = sentinel_v(T, r)
    lsb.lora_shrink_single(x, A[0], v)
    seg = lsb.lora_build_segments(torch.zeros(T, dtype=torch.int32, device="cuda"), 1)
    v_seg = sentinel_v(T, r)
    lsb.lora_shrink(x, A, seg, v_seg)
    torch.cuda.synchronize()
    assert np.array_equal(v.cpu().numpy().view(np.uint32), v_seg.cpu().numpy().view(np.uint32))
    v_or = oracle.shrink(dtype, w.x, w.A, np.zeros(T, np.int32))
    assert tol_ratio(v.cpu().numpy().astype(np.float64), v_or) <= 1


def test_single_adapter_shrink_128_token_tiles():
    """lora_shrink_single (no metadata) at r = 64, 8192 tokens: the dense form
    of the 128-token-tile kernel, every row against the oracle."""
    _announce("single-adapter shrink, 128-token tiles: f16 T=8192 H=2048 r=64")
    T, H, r = 8192, 2048, 64
    w = W.make("single_tb2", "f16", T, H, r, 1, [[64]], seed=77)
    x = dev_bits(w.x, "f16")
    A = dev_bits(w.A, "f16")[0]
    v = sentinel_v(T, r)
    lsb.lora_shrink_single(x, A, v)
    torch.cuda.synchronize()
    v_or = oracle.shrink("f16", w.x, w.A, np.zeros(T, np.int32))
    assert tol_ratio(v.cpu().numpy().astype(np.float64), v_or) <= 1


WIDE_V_CASES = [
    # dtype, r, n, path: each expand kernel form (per-token aligned r = 16 / 64,
    # per-token general, tiles at r <= 16, 64, 128, tiles on the scalar path)
    ("f16", 16, 1024, "bgmv"),
    ("f16", 64, 512, "bgmv"),
    ("f16", 24, 300, "bgmv"),
    ("f16", 16, 1024, "sgmv"),
    ("f16", 64, 512, "sgmv"),
    ("f16", 128, 256, "sgmv"),
    ("f16", 20, 100, "sgmv"),
    ("bf16", 16, 1024, "bgmv"),
    ("bf16", 64, 512, "sgmv"),
]
# Per-adapter magnitude of v (powers of ten) and of its weights: together
# they keep each token's output well inside the binary16 range.
WIDE_V_EXP = [-6, -4, -2, 0, 2, 4, 5, 6]


@pytest.mark.parametrize("dtype,r,n,path", WIDE_V_CASES)
def test_expand_wide_range_v(force_path, dtype, r, n, path):
    """expand takes any finite fp32 v (the micro-benchmark PR's f32 x f16 =>
    f16 expand): token rows of v from about 1e-6 to 1e6, beyond the binary16
    range (|v| >= 65520) and below its normal range, on both kernel families.
    The weights of adapter l scale as 10^-clip(u_l, -3, 3), so the output
    y = v . B (add_inputs = 0) has a known order s_t per token; the bound is the
    stated tolerance in units of s_t: |gpu - oracle| <= 1e-2 (s_t + |oracle|)."""
    _announce(f"wide-range v {dtype} r={r} n={n} path={path}")
    force_path(lsb.PATH_BGMV if path == "bgmv" else lsb.PATH_SGMV)
    rng = np.random.default_rng(r * 1000 + n)
    L, T = len(WIDE_V_EXP), 200
    ids = rng.integers(0, L, T).astype(np.int32)
    ids[rng.random(T) < 0.1] = -1
    u = np.array(WIDE_V_EXP, np.float64)
    bexp = -np.clip(u, -3, 3)
    B = np.stack([W.normal_bits(rng, (n, r), 10.0 ** bexp[l] / np.sqrt(r), dtype) for l in range(L)])
    v = (rng.standard_normal((T, r)) * 10.0 ** u[np.maximum(ids, 0)][:, None]).astype(np.float32)
    y0 = W.normal_bits(rng, (T, n), 1.0, dtype)
    act = ids >= 0
    if dtype == "f16":
        assert np.abs(v[act]).max() >= 65520 and np.abs(v[act]).min() < 6.1e-5
    seg = lsb.lora_build_segments(torch.from_numpy(ids).cuda(), L)
    y = dev_bits(y0, dtype)
    lsb.lora_expand(torch.from_numpy(v).cuda(), dev_bits(B, dtype), seg, y, False)
    torch.cuda.synchronize()
    ref = oracle.expand(dtype, v.astype(np.float64), B, ids, y0, 0, False)
    got = decode(host_bits(y), dtype)
    scale = (10.0 ** (u + bexp))[np.maximum(ids, 0)][:, None]
    ratio = np.abs(got - ref) / (1e-2 * (scale + np.abs(ref)))
    assert np.isfinite(got[act]).all()
    assert not np.isnan(ratio[act]).any() and ratio[act].max() <= 1, ratio[act].max()
    assert np.array_equal(host_bits(y)[~act], y0[~act])


# ---------------------------------------------------------------- BGMV and SGMV paths
@pytest.fixture
def tuning_from_env(monkeypatch):
    """Reloads the library's launch-plan overrides after a test has set them
    in the environment (through monkeypatch), and again afterwards, once the
    environment is restored: this teardown runs before monkeypatch's own, so
    it undoes the environment first."""
    yield lsb.lora_reload_tuning
    monkeypatch.undo()
    lsb.lora_reload_tuning()


@pytest.fixture
def force_path():
    def setter(mode):
        lsb.lora_set_path(mode)
    yield setter
    lsb.lora_set_path(lsb.PATH_AUTO)


PATH_CASES = [
    # dtype, T, H, r, L, slices, seq_len, neg_frac
    ("bf16", 40, 2048, 128, 5, [[1024, 512]], (1, 4), 0.1),   # rank 128 (per-token: 16 lanes a column)
    ("f16", 16, 1000, 128, 3, [[256]], 1, 0.0),               # rank 128, shrink on the element-wise path
    ("f16", 16, 1024, 16, 4, [[1024]], 1, 0.0),
    ("f16", 256, 4096, 16, 4, [[4096]], 1, 0.0),
    ("bf16", 300, 2048, 32, 7, [[512, 256, 256]], (1, 20), 0.1),
    ("bf16", 130, 1536, 64, 3, [[1000]], (1, 9), 0.2),
    ("f16", 77, 2049, 20, 3, [[300]], (1, 9), 0.2),      # scalar path
    ("bf16", 1100, 1024, 8, 40, [[256, 64]], (1, 4), 0.05),
]


@pytest.mark.parametrize("mode", [lsb.PATH_BGMV, lsb.PATH_SGMV])
@pytest.mark.parametrize("dtype,T,H,r,L,slices,sl,neg", PATH_CASES)
def test_each_path_matches_oracle(force_path, mode, dtype, T, H, r, L, slices, sl, neg):
    """Both kernel families, forced, against the oracle (BGMV semantics are a
    strict subset of SGMV, so either must give the oracle's result)."""
    _announce(f"path {mode} {dtype} T={T} H={H} r={r} L={L} slices={slices}")
    force_path(mode)
    w = W.make("path", dtype, T, H, r, L, slices, seed=T + 17 * r, seq_len=sl, neg_frac=neg)
    dw = DeviceWorkload(w)
    dw.run()
    rv, ry, ryi = compare_with_oracle(dw)
    print(f"  tolerance ratios: v {rv:.3g}  y {ry:.3g}  y(isolated) {ryi:.3g}")
    assert rv <= 1 and ry <= 1 and ryi <= 1
    check_neg_rows(dw)
    check_outside_slices(dw)


@pytest.mark.parametrize("mode", [lsb.PATH_BGMV, lsb.PATH_SGMV])
@pytest.mark.parametrize("dtype,T,H,r,L,slices,sl", [
    ("f16", 200, 256, 16, 4, [[256]], 1),
    ("bf16", 333, 512, 24, 5, [[64, 48, 100]], (1, 40)),
    ("bf16", 90, 2048, 64, 3, [[136]], (1, 5)),
])
def test_each_path_integer_exact(force_path, mode, dtype, T, H, r, L, slices, sl):
    _announce(f"integer exact, path {mode} {dtype} T={T} H={H} r={r}")
    force_path(mode)
    w = W.make("int", dtype, T, H, r, L, slices, seed=T + H, seq_len=sl, neg_frac=0.15, integer=True)
    dw = DeviceWorkload(w)
    dw.run()
    act = np.nonzero(w.active)[0]
    v_or = oracle.shrink(w.dtype, w.x, w.A, w.ids)
    assert np.array_equal(dw.v.cpu().numpy()[act].astype(np.float64), v_or[act])
    for o, y in zip(w.outputs, dw.ys):
        ref = oracle.expand_slice(w.dtype, np.nan_to_num(v_or), [s.B for s in o.slices],
                                  [s.col_off for s in o.slices], w.ids, o.y0, w.add)
        ref_bits = W.f32_to_bits(ref.astype(np.float32), dtype) if dtype == "bf16" else \
            ref.astype(np.float16).view(np.uint16)
        assert np.array_equal(host_bits(y)[:, _slice_cols(o)][act], ref_bits[act])
    check_neg_rows(dw)


PLAN_VARIANTS = [
    # (environment overrides of the launch plan, kernel path, dtype, T, H, r, L, slices)
    ({"LORA_SHRINK_KSPLIT": "1"}, "sgmv", "bf16", 300, 2048, 32, 7, [[512, 256, 256]]),
    ({"LORA_SHRINK_KSPLIT": "2"}, "sgmv", "f16", 300, 2048, 32, 7, [[512, 256, 256]]),
    ({"LORA_SHRINK_KSPLIT": "5"}, "sgmv", "bf16", 500, 4096, 64, 9, [[1024]]),
    # the rotated block walk with even and odd chunk counts, ragged chunk ends
    ({"LORA_SHRINK_KSPLIT": "4"}, "sgmv", "bf16", 500, 4096, 64, 9, [[1024]]),
    ({"LORA_SHRINK_KSPLIT": "1"}, "sgmv", "f16", 300, 1408, 16, 5, [[256]]),
    ({"LORA_SHRINK_KSPLIT": "3"}, "sgmv", "bf16", 300, 2000, 40, 5, [[256]]),
    ({"LORA_SHRINK_KSPLIT": "2"}, "sgmv", "bf16", 260, 1152, 128, 4, [[128]]),
    # 128-token shrink tiles at r = 33..64 (two 16-token blocks per wave):
    # ragged tiles, split and unsplit H, the element-wise path
    ({"LORA_SHRINK_TB": "2"}, "sgmv", "bf16", 700, 2048, 64, 5, [[512]]),
    ({"LORA_SHRINK_TB": "2", "LORA_SHRINK_KSPLIT": "1"}, "sgmv", "f16", 300, 1024, 48, 4, [[256]]),
    ({"LORA_SHRINK_TB": "2", "LORA_SHRINK_KSPLIT": "3"}, "sgmv", "bf16", 500, 4096, 64, 9, [[1024]]),
    ({"LORA_SHRINK_TB": "2"}, "sgmv", "f16", 200, 2001, 40, 3, [[256]]),
    # 16-token groups with the H split inside the workgroup (r <= 32): H in
    # whole 256-element blocks, a ragged last block, the element-wise path,
    # waves with no block (H = 1024), eight blocks per wave (the pipelined
    # loop), one and two rank tiles, and a pool past the eagerly copied table
    ({"LORA_SHRINK_GROUP": "1"}, "sgmv", "bf16", 300, 4096, 16, 7, [[512]]),
    ({"LORA_SHRINK_GROUP": "1"}, "sgmv", "f16", 500, 2000, 32, 9, [[256]]),
    ({"LORA_SHRINK_GROUP": "1"}, "sgmv", "bf16", 200, 2001, 20, 3, [[256]]),
    ({"LORA_SHRINK_GROUP": "1"}, "sgmv", "f16", 77, 1024, 8, 4, [[128]]),
    ({"LORA_SHRINK_GROUP": "1"}, "sgmv", "bf16", 260, 16384, 32, 5, [[256]]),
    ({"LORA_SHRINK_GROUP": "1"}, "sgmv", "f16", 600, 1024, 16, 300, [[256]]),
    ({"LORA_EXPAND_TB": "2"}, "sgmv", "bf16", 700, 1024, 64, 5, [[2048, 512]]),
    ({"LORA_EXPAND_TB": "2"}, "sgmv", "f16", 300, 1024, 16, 3, [[1000]]),
    ({"LORA_EXPAND_TB": "2"}, "sgmv", "bf16", 300, 512, 128, 3, [[384]]),
    ({"LORA_EXPAND_CPR": "1"}, "sgmv", "bf16", 400, 1024, 32, 6, [[1536, 256]]),
    ({"LORA_EXPAND_CPR": "3"}, "sgmv", "f16", 400, 1024, 32, 6, [[1536, 256]]),
    ({"LORA_EXPAND_CPR": "40"}, "sgmv", "bf16", 400, 1024, 32, 6, [[1536, 256]]),
    # the tile expand's two schedules, forced: balanced ranges of (run, tile,
    # chunk) units (128-token tiles) cut runs anywhere (ragged slice ends,
    # 3-chunk runs, the element-wise path); the forms that always walk
    # round-robin (64-token tiles, rank 128) ignore the override; and
    # round-robin items
    ({"LORA_EXPAND_BALANCE": "2", "LORA_EXPAND_TB": "2"}, "sgmv", "bf16", 700, 1024, 64, 5, [[2048, 520, 136]]),
    ({"LORA_EXPAND_BALANCE": "2", "LORA_EXPAND_TB": "2", "LORA_EXPAND_CPR": "3"}, "sgmv", "f16", 400, 1024, 32, 6,
     [[1536, 256]]),
    ({"LORA_EXPAND_BALANCE": "2", "LORA_EXPAND_TB": "2"}, "sgmv", "f16", 900, 1024, 16, 6, [[1000]]),
    ({"LORA_EXPAND_BALANCE": "2", "LORA_EXPAND_TB": "2"}, "sgmv", "f16", 77, 2049, 20, 3, [[300]]),
    ({"LORA_EXPAND_BALANCE": "2"}, "sgmv", "bf16", 300, 512, 128, 3, [[384]]),
    ({"LORA_EXPAND_BALANCE": "2", "LORA_EXPAND_TB": "1"}, "sgmv", "bf16", 400, 1024, 32, 6, [[1536, 256]]),
    ({"LORA_EXPAND_BALANCE": "1"}, "sgmv", "bf16", 700, 1024, 64, 5, [[2048, 520, 136]]),
    # per-token expand: rounds of 512 columns per wave and column blocks per token
    ({"LORA_BGMV_RPI": "2"}, "bgmv", "f16", 20, 1024, 16, 3, [[4096, 1024]]),
    ({"LORA_BGMV_RPI": "2"}, "bgmv", "bf16", 9, 512, 8, 3, [[2048, 4096]]),
    ({"LORA_BGMV_RPI": "1", "LORA_BGMV_CB": "1"}, "bgmv", "bf16", 37, 1024, 16, 4, [[3072, 1024, 1024]]),
    ({"LORA_BGMV_CB": "2"}, "bgmv", "bf16", 5, 1024, 32, 3, [[8192]]),
    ({}, "bgmv", "f16", 3, 1024, 64, 2, [[16384, 512]]),
    ({"LORA_BGMV_RPI": "2"}, "bgmv", "bf16", 600, 1024, 16, 5, [[14336, 14336]]),
    # per-token shrink: ranks per workgroup
    ({"LORA_BGMV_SHRINK_RT": "4"}, "bgmv", "f16", 40, 2048, 16, 3, [[1024]]),
    ({"LORA_BGMV_SHRINK_RT": "8"}, "bgmv", "bf16", 300, 1024, 40, 5, [[512]]),
    ({"LORA_BGMV_SHRINK_RT": "16"}, "bgmv", "f16", 7, 4096, 64, 3, [[512]]),
    ({}, "bgmv", "bf16", 11, 1000, 24, 3, [[1000]]),
    # per-token shrink over long rows (several trips per rank block), ragged ends
    ({"LORA_BGMV_SHRINK_RT": "16"}, "bgmv", "bf16", 40, 20000, 16, 3, [[512]]),
    ({"LORA_BGMV_SHRINK_RT": "8"}, "bgmv", "f16", 30, 17000, 16, 3, [[512]]),
    ({"LORA_BGMV_SHRINK_RT": "4"}, "bgmv", "bf16", 20, 40000, 16, 2, [[256]]),
    ({}, "bgmv", "f16", 300, 12288, 16, 4, [[1024]]),
]


@pytest.mark.parametrize("env,path,dtype,T,H,r,L,slices", PLAN_VARIANTS)
@pytest.mark.parametrize("integer", [False, True])
def test_plan_variants(force_path, monkeypatch, tuning_from_env, env, path, dtype, T, H, r, L, slices, integer):
    """Launch plans the defaults never pick (other H splits, 128-token expand
    tiles, other column runs, other per-token column blocks), selected through
    the library's tuning overrides, still give the oracle's result; with
    integer inputs, its exact bits."""
    _announce(f"plan {env} {path} {dtype} T={T} H={H} r={r} L={L} slices={slices} integer={integer}")
    for k, val in env.items():
        monkeypatch.setenv(k, val)
    tuning_from_env()
    force_path(lsb.PATH_SGMV if path == "sgmv" else lsb.PATH_BGMV)
    w = W.make("plan", dtype, T, H, r, L, slices, seed=T + r + (7 if integer else 0), seq_len=(1, 40),
               neg_frac=0.1, integer=integer)
    dw = DeviceWorkload(w)
    dw.run()
    if integer:
        act = np.nonzero(w.active)[0]
        v_or = oracle.shrink(w.dtype, w.x, w.A, w.ids)
        assert np.array_equal(dw.v.cpu().numpy()[act].astype(np.float64), v_or[act])
        for o, y in zip(w.outputs, dw.ys):
            ref = oracle.expand_slice(w.dtype, np.nan_to_num(v_or), [s.B for s in o.slices],
                                      [s.col_off for s in o.slices], w.ids, o.y0, w.add)
            ref_bits = W.f32_to_bits(ref.astype(np.float32), dtype) if dtype == "bf16" else \
                ref.astype(np.float16).view(np.uint16)
            assert np.array_equal(host_bits(y)[:, _slice_cols(o)][act], ref_bits[act])
    else:
        rv, ry, ryi = compare_with_oracle(dw)
        assert rv <= 1 and ry <= 1 and ryi <= 1
    check_neg_rows(dw)
    check_outside_slices(dw)


LINE_CASES = [
    # (dtype, T, r, slice widths, LORA_EXPAND_TB, LORA_EXPAND_BALANCE): whole-line
    # y loads and stores on round-robin walks at r = 64, loads only on balanced
    # ranges at r = 64 and at r = 128, both at r <= 32; ragged slice ends
    ("bf16", 1500, 64, [2048, 520], "2", "1"),
    ("bf16", 1500, 64, [2048, 520], "2", "2"),
    ("f16", 900, 16, [1000], "2", "2"),
    ("f16", 700, 32, [1536, 256], "1", "0"),
    ("bf16", 500, 128, [384, 136], "0", "0"),
]


@pytest.mark.parametrize("dtype,T,r,widths,tb,balance", LINE_CASES)
def test_expand_whole_line_y_bit_identical(force_path, monkeypatch, tuning_from_env, dtype, T, r, widths, tb, balance):
    """The tile expand's whole-line y paths (loads and stores, loads only)
    leave y bit for bit as the op-layout loads and stores do: the same sums,
    only the memory access shape differs."""
    _announce(f"whole-line y: {dtype} T={T} r={r} slices={widths} tb={tb} balance={balance}")
    force_path(lsb.PATH_SGMV)
    monkeypatch.setenv("LORA_EXPAND_TB", tb)
    monkeypatch.setenv("LORA_EXPAND_BALANCE", balance)
    w = W.make("line", dtype, T, 64, r, 6, [widths], seed=T + r, seq_len=(1, 40), neg_frac=0.1)
    o = w.outputs[0]
    seg = lsb.lora_build_segments(torch.from_numpy(w.ids).cuda(), w.L)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(T)
    v = torch.randn(T, r, generator=gen, device="cuda")
    Bs = [dev_bits(q.B, dtype) for q in o.slices]
    got = []
    for mode in ("2", "1", "0"):
        monkeypatch.setenv("LORA_EXPAND_LINE_Y", mode)
        tuning_from_env()
        y = dev_bits(o.y0, dtype).clone()
        lsb.lora_expand_slice(v, Bs, [q.col_off for q in o.slices], seg, y, True)
        torch.cuda.synchronize()
        got.append(host_bits(y))
    assert np.array_equal(got[0], got[1]) and np.array_equal(got[0], got[2])
    assert np.array_equal(got[2][~w.active], host_bits(dev_bits(o.y0, dtype))[~w.active])


RANK_CASES = [
    # (dtype, T, H, r, L, slices, ranks_from, integer, seq_len)
    ("bf16", 500, 1024, 128, 16, [[1024, 256, 256], [2048]], [8, 16, 32, 64, 128], False, (1, 40)),
    ("f16", 300, 2048, 64, 7, [[1536]], [8, 24, 40, 64], False, (1, 40)),   # ranks off the 16 / 32 grid
    ("bf16", 200, 512, 32, 5, [[512, 128]], [8, 16, 32], True, (1, 40)),
    ("f16", 130, 1001, 16, 3, [[1001]], [8, 16], False, (1, 40)),           # unaligned: element-wise loads
    # pools of more than 256 adapters: the tile tables copy only the segments
    # in use and look each segment's rank up from its adapter -- a few
    # segments, and more than 256 of them
    ("bf16", 600, 1024, 64, 600, [[1024]], [8, 16, 40, 64], False, (1, 40)),
    ("f16", 1500, 512, 32, 700, [[512, 256]], [8, 16, 24, 32], True, (1, 4)),
]


@pytest.mark.parametrize("path", ["sgmv", "bgmv"])
@pytest.mark.parametrize("dtype,T,H,r,L,slices,ranks_from,integer,seq_len", RANK_CASES)
def test_live_ranks(force_path, path, dtype, T, H, r, L, slices, ranks_from, integer, seq_len):
    """Per-adapter live ranks (zero-padded adapters, the issue's mixed-rank
    batch): the segment kernels skip the padding, the per-token kernels read
    the zero padding as it is; both give the same values as without the
    ranks, within the tolerance of the oracle; ranks above r are clamped to r."""
    if path == "bgmv" and r > 64 and r != 128:
        pytest.skip("the per-token kernels take r <= 64 or 128")
    _announce(f"live ranks {path} {dtype} T={T} H={H} r={r} L={L} slices={slices} ranks={ranks_from}")
    force_path(lsb.PATH_SGMV if path == "sgmv" else lsb.PATH_BGMV)
    w = W.make("ranks", dtype, T, H, r, L, slices, seed=T + r, seq_len=seq_len, neg_frac=0.1,
               ranks_from=ranks_from, integer=integer)
    if L > 256:
        S = len(np.unique(w.ids[w.ids >= 0]))
        print(f"  segments in use: {S}")
    plain = DeviceWorkload(w)
    plain.run()
    ranked = DeviceWorkload(w)
    ranked.run(lora_rank=w.ranks)
    rv, ry, ryi = compare_with_oracle(ranked)
    assert rv <= 1 and ry <= 1 and ryi <= 1
    check_neg_rows(ranked)
    check_outside_slices(ranked)
    act = np.nonzero(w.active)[0]
    # Skipped steps only drop additions of exact zeros: values agree exactly
    # (a zero may differ in sign).
    assert np.array_equal(ranked.v.cpu().numpy()[act], plain.v.cpu().numpy()[act])
    for y_r, y_p in zip(ranked.ys, plain.ys):
        assert np.array_equal(decode(host_bits(y_r), w.dtype), decode(host_bits(y_p), w.dtype))
    big = DeviceWorkload(w)
    big.run(lora_rank=np.full(L, 10 * r, np.int32))
    assert np.array_equal(big.v.cpu().numpy()[act], plain.v.cpu().numpy()[act])


GRAPH_CASES = [
    # dtype, T, H, r, L, slices, seq_len, ranks_from: the per-token decode path;
    # the tile path with the H split (workspace and reduce kernel); live ranks
    ("f16", 256, 4096, 16, 4, [[4096]], 1, None),
    ("bf16", 700, 2048, 32, 7, [[512, 256, 256]], (1, 40), None),
    ("bf16", 500, 1024, 128, 16, [[1024, 256, 256], [2048]], (1, 40), [8, 16, 32, 64, 128]),
]


@pytest.mark.parametrize("dtype,T,H,r,L,slices,seq_len,ranks_from", GRAPH_CASES)
def test_graph_replays_match_eager(dtype, T, H, r, L, slices, seq_len, ranks_from):
    """One step (build, shrink, every expand) captured in a HIP graph and
    replayed three times, with eager work between the replays (y reset to y0,
    v and the metadata buffers overwritten): every replay gives the eager
    step's bits."""
    _announce(f"graph replays {dtype} T={T} H={H} r={r} L={L} slices={slices}")
    w = W.make("graph", dtype, T, H, r, L, slices, seed=T + 3 * r, seq_len=seq_len, neg_frac=0.1,
               ranks_from=ranks_from)
    rk = None if w.ranks is None else torch.from_numpy(np.ascontiguousarray(w.ranks, np.int32)).cuda()
    eager = DeviceWorkload(w)
    seg_e = eager.run(lora_rank=None if rk is None else w.ranks)
    meta_e = seg_host(seg_e)
    act = np.nonzero(w.active)[0]
    v_e = eager.v.cpu().numpy()

    g_w = DeviceWorkload(w)
    y0 = [y.clone() for y in g_w.ys]
    v0 = g_w.v.clone()
    seg = lsb.Segments(g_w.ids, w.L, rk)
    need = lsb.lora_shrink_workspace_bytes(w.T, w.L, w.H, w.r)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")

    def step():
        lsb.lora_build_segments(g_w.ids, w.L, seg=seg)
        lsb.lora_shrink(g_w.x, g_w.A, seg, g_w.v, workspace=ws)
        for o, Bs, y in zip(w.outputs, g_w.Bs, g_w.ys):
            if len(o.slices) == 1 and o.slices[0].col_off == 0:
                lsb.lora_expand(g_w.v, Bs[0], seg, y, w.add)
            else:
                lsb.lora_expand_slice(g_w.v, Bs, [q.col_off for q in o.slices], seg, y, w.add)

    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        for y, y_init in zip(g_w.ys, y0):
            y.copy_(y_init)
        g_w.v.copy_(v0)
        seg.sorted_token.fill_(-5)
        seg.seg_lora.fill_(-5)
        seg.seg_start.fill_(-5)
        seg.counts.fill_(-5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a_, b_ in zip(seg_host(seg), meta_e):
            assert np.array_equal(a_, b_)
        assert np.array_equal(g_w.v.cpu().numpy()[act].view(np.uint32), v_e[act].view(np.uint32))
        for y_g, y_e in zip(g_w.ys, eager.ys):
            assert np.array_equal(host_bits(y_g), host_bits(y_e))


@pytest.mark.parametrize("path", ["auto", "bgmv"])
def test_logits_vocabulary_expand(force_path, path):
    """LoRA on the logits layer (TPU PR): expand r -> a 128256-column
    vocabulary, on both kernel families."""
    _announce(f"logits expand path={path}")
    if path == "bgmv":
        force_path(lsb.PATH_BGMV)
    w = W.make("logits", "bf16", 48, 512, 16, 4, [[128256]], seed=128, seq_len=(1, 4), neg_frac=0.1)
    dw = DeviceWorkload(w)
    dw.run()
    rv, ry, ryi = compare_with_oracle(dw)
    assert rv <= 1 and ry <= 1 and ryi <= 1
    check_neg_rows(dw)


def test_single_adapter_batch(force_path):
    """One adapter for every token (the unmasked single-adapter case): one
    segment covering the batch, on both kernel families."""
    _announce("single adapter")
    w = W.make("single", "f16", 700, 2048, 32, 1, [[3072]], seed=11, seq_len=(1, 30))
    for mode in (lsb.PATH_BGMV, lsb.PATH_SGMV):
        force_path(mode)
        dw = DeviceWorkload(w)
        dw.run()
        rv, ry, ryi = compare_with_oracle(dw)
        assert rv <= 1 and ry <= 1 and ryi <= 1


MAX_CASES = [
    # (dtype, T, H, r, L, slices, seq_len, path): the limits of the boundary
    ("bf16", 3000, 256, 128, 2048, [[256]], (1, 3), "sgmv"),            # max adapters at max rank
    ("f16", 2500, 512, 64, 2048, [[512]], (1, 3), "bgmv"),              # max adapters, per-token path
    ("bf16", 600, 512, 32, 9, [[64, 32, 96, 8, 40, 16, 24, 200]], (1, 20), "auto"),  # 8 slices
]


@pytest.mark.parametrize("dtype,T,H,r,L,slices,seq_len,path", MAX_CASES)
def test_boundary_limits(force_path, dtype, T, H, r, L, slices, seq_len, path):
    """The largest adapter count (its tile table fills most of the LDS left
    beside the weights), the largest rank and the most slices the header
    allows."""
    _announce(f"limits {dtype} T={T} H={H} r={r} L={L} slices={len(slices[0])} path={path}")
    if path != "auto":
        force_path(lsb.PATH_SGMV if path == "sgmv" else lsb.PATH_BGMV)
    w = W.make("limits", dtype, T, H, r, L, slices, seed=L + r, seq_len=seq_len, neg_frac=0.05)
    dw = DeviceWorkload(w)
    dw.run()
    rv, ry, ryi = compare_with_oracle(dw)
    assert rv <= 1 and ry <= 1 and ryi <= 1
    check_neg_rows(dw)
    check_outside_slices(dw)


THRESHOLD_CASES = [
    # (dtype, T, H, r, slices): shapes on both sides of the automatic path
    # choice (at most 512 tokens for the per-token kernels; the expand's
    # T n <= 4M at r <= 16 and <= 1M at r <= 32; the shrink's fitted costs)
    ("f16", 512, 1024, 16, [[8192]]),
    ("f16", 513, 1024, 16, [[8192]]),
    ("bf16", 256, 2048, 16, [[16384]]),
    ("bf16", 256, 2048, 16, [[16392]]),
    ("f16", 128, 4096, 32, [[8192]]),
    ("f16", 128, 4096, 32, [[8200]]),
    ("bf16", 64, 16384, 64, [[1024]]),
    ("bf16", 300, 8192, 64, [[1024]]),
]


@pytest.mark.parametrize("dtype,T,H,r,slices", THRESHOLD_CASES)
def test_automatic_path_thresholds(dtype, T, H, r, slices):
    """The automatic choice between the kernel families gives the oracle's
    result on both sides of each of its thresholds."""
    _announce(f"auto path {dtype} T={T} H={H} r={r} n={slices}")
    w = W.make("auto", dtype, T, H, r, 4, slices, seed=T + H + r, seq_len=1, neg_frac=0.05)
    dw = DeviceWorkload(w)
    dw.run()
    rv, ry, ryi = compare_with_oracle(dw)
    assert rv <= 1 and ry <= 1 and ryi <= 1
    check_neg_rows(dw)


def test_bgmv_and_sgmv_agree(force_path):
    """The per-token and the segment kernels on the same batch agree with each
    other within the tolerance (punica issue: BGMV is a subset of SGMV)."""
    _announce("bgmv vs sgmv on one batch")
    w = W.make("agree", "bf16", 400, 4096, 16, 4, [[4096, 1024]], seed=77, seq_len=(1, 8),
               neg_frac=0.1)
    outs = []
    for mode in (lsb.PATH_BGMV, lsb.PATH_SGMV):
        force_path(mode)
        dw = DeviceWorkload(w)
        dw.run()
        outs.append((dw.v.cpu().numpy().astype(np.float64), decode(host_bits(dw.ys[0]), w.dtype)))
    act = w.active
    assert tol_ratio(outs[0][0][act], outs[1][0][act]) <= 1
    assert tol_ratio(outs[0][1][act], outs[1][1][act]) <= 1


def test_forced_bgmv_rejects_unsupported_expand_rank(force_path):
    """The per-token expand takes r <= 64, or 128 on aligned data: r = 100
    forced onto it is refused (the per-token shrink takes it)."""
    force_path(lsb.PATH_BGMV)
    w = W.make("big", "bf16", 32, 256, 100, 2, [[64]], seed=3)
    dw = DeviceWorkload(w)
    with pytest.raises(lsb.LoraError) as e:
        dw.run()
    assert e.value.code == lsb.LORA_ERR_UNSUPPORTED
    assert "lora_expand" in str(e.value)


# ---------------------------------------------------------------- one adapter, no metadata
SINGLE_CASES = [
    # dtype, T, H, r, slices, path, integer
    ("f16", 1, 64, 16, [64], "auto", False),
    ("bf16", 63, 2049, 20, [300], "auto", False),            # element-wise path
    ("f16", 700, 4096, 32, [4096, 1024], "sgmv", False),
    ("bf16", 700, 4096, 32, [4096, 1024], "bgmv", False),
    ("bf16", 300, 4096, 16, [4096], "auto", False),           # per-token kernels by the automatic choice
    ("bf16", 4099, 1024, 64, [2048], "auto", False),          # ragged last tile, 128-token expand tiles
    ("f16", 8192, 4096, 128, [1024, 512], "auto", False),     # rank 128, split H
    ("bf16", 1500, 2048, 24, [512, 64, 104], "sgmv", True),   # integer inputs: exact
]


@pytest.mark.parametrize("dtype,T,H,r,widths,path,integer", SINGLE_CASES)
def test_single_adapter_forms(force_path, dtype, T, H, r, widths, path, integer):
    """The single-adapter entry points (no metadata, token index = row)
    against the oracle, and bit for bit against the segment entry points run
    on the same batch with every id 0 (same kernels, same tiles)."""
    _announce(f"single-adapter forms {dtype} T={T} H={H} r={r} slices={widths} path={path}")
    force_path({"auto": lsb.PATH_AUTO, "bgmv": lsb.PATH_BGMV, "sgmv": lsb.PATH_SGMV}[path])
    w = W.make("single", dtype, T, H, r, 1, [widths], seed=T + H + r, seq_len=(1, 40), integer=integer)
    assert (w.ids == 0).all()
    seg_w = DeviceWorkload(w)
    seg_w.run()
    x = dev_bits(w.x, dtype)
    A = dev_bits(w.A, dtype)
    o = w.outputs[0]
    Bs = [dev_bits(q.B, dtype) for q in o.slices]
    v = sentinel_v(T, r)
    lsb.lora_shrink_single(x, A, v)
    y = dev_bits(o.y0, dtype)
    if len(widths) == 1:
        lsb.lora_expand_single(v, Bs[0], y, True)
    else:
        lsb.lora_expand_slice_single(v, Bs, [q.col_off for q in o.slices], y, True)
    torch.cuda.synchronize()
    assert np.array_equal(v.cpu().numpy().view(np.uint32), seg_w.v.cpu().numpy().view(np.uint32))
    assert np.array_equal(host_bits(y), host_bits(seg_w.ys[0]))
    v_or = oracle.shrink(dtype, w.x, w.A, w.ids)
    cols = _slice_cols(o)
    if integer:
        assert np.array_equal(v.cpu().numpy().astype(np.float64), v_or)
        ref = oracle.expand_slice(dtype, v_or, [q.B for q in o.slices], [q.col_off for q in o.slices],
                                  w.ids, o.y0, True)
        assert np.array_equal(host_bits(y)[:, cols], W.f32_to_bits(ref.astype(np.float32), dtype))
    else:
        assert tol_ratio(v.cpu().numpy().astype(np.float64), v_or) <= 1
        ref = oracle.expand_slice(dtype, v_or, [q.B for q in o.slices], [q.col_off for q in o.slices],
                                  w.ids, o.y0, True)
        assert tol_ratio(decode(host_bits(y), dtype)[:, cols], ref) <= 1


def test_single_adapter_empty_batch():
    """T = 0 launches nothing and touches nothing."""
    _announce("single-adapter forms, T = 0")
    x = torch.empty(0, 256, dtype=torch.float16, device="cuda")
    A = torch.zeros(16, 256, dtype=torch.float16, device="cuda")
    v = torch.empty(0, 16, device="cuda")
    lsb.lora_shrink_single(x, A, v)
    y = torch.empty(0, 64, dtype=torch.float16, device="cuda")
    lsb.lora_expand_single(v, torch.zeros(64, 16, dtype=torch.float16, device="cuda"), y)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- decode + prefill mixes
MIXED_CASES = [
    # dtype, n_prefill, prefill_loras, n_decode, L, H, r, slices, integer: batches
    # of >= 256 adapters, where the shrink and the expand (up to r = 64) send
    # one-token segments to the per-token kernel and the rest to the tile kernel
    ("bf16", 2000, 16, 700, 1024, 1024, 16, [[1024]], False),
    ("f16", 1500, 8, 600, 700, 2048, 64, [[512, 256]], False),
    ("bf16", 1200, 12, 400, 512, 512, 24, [[300]], False),        # per-token general kernel
    ("bf16", 900, 4, 300, 400, 1024, 32, [[512], [256, 256]], True),
    ("f16", 0, 1, 800, 1024, 512, 16, [[1024]], False),          # decode only, above 512 tokens
    # the tile shrink splits H (a reduce kernel writes every active row) and the
    # per-token pass then writes the one-token segments' rows
    ("f16", 400, 4, 200, 256, 2048, 16, [[512]], False),
    ("bf16", 450, 4, 150, 256, 2048, 32, [[256, 256]], True),
    ("bf16", 3000, 16, 300, 320, 1024, 128, [[512]], False),      # rank 128: the expand keeps tiles throughout
    ("f16", 1200, 8, 500, 600, 1024, 8, [[1024, 512]], True),     # rank 8: one-token items with one lane a column
    # prefill only, a few segments of a large pool: the tile bound (one partial
    # tile per adapter) is loose, and the kernels raise the H split and
    # shorten the column runs from the true tile count
    ("bf16", 3000, 8, 0, 1024, 4096, 16, [[4096]], False),
    ("f16", 2500, 6, 0, 2000, 2048, 64, [[1024, 512]], True),
    ("bf16", 1800, 3, 0, 1500, 4096, 128, [[2048], [512]], False),
]


@pytest.mark.parametrize("dtype,n_pre,pre_l,n_dec,L,H,r,slices,integer", MIXED_CASES)
def test_decode_prefill_mix(dtype, n_pre, pre_l, n_dec, L, H, r, slices, integer):
    """Mixed batches through the automatic path: every row against the
    oracle (integer inputs: bit for bit), untouched rows and columns kept."""
    _announce(f"decode+prefill mix {dtype} prefill={n_pre}/{pre_l} decode={n_dec} L={L} H={H} r={r} "
              f"slices={slices} integer={integer}")
    w = W.make_mixed("mix", dtype, n_pre, pre_l, n_dec, L, H, r, slices, seed=n_pre + n_dec + r,
                     neg_frac=0.05, integer=integer)
    dw = DeviceWorkload(w)
    seg = dw.run()
    for g, ref in zip(seg_host(seg), oracle.build_segments(w.ids, w.L)):
        assert np.array_equal(g, ref)
    if integer:
        act = np.nonzero(w.active)[0]
        v_or = oracle.shrink(w.dtype, w.x, w.A, w.ids)
        assert np.array_equal(dw.v.cpu().numpy()[act].astype(np.float64), v_or[act])
        for o, y in zip(w.outputs, dw.ys):
            ref = oracle.expand_slice(w.dtype, np.nan_to_num(v_or), [s.B for s in o.slices],
                                      [s.col_off for s in o.slices], w.ids, o.y0, w.add)
            ref_bits = W.f32_to_bits(ref.astype(np.float32), dtype) if dtype == "bf16" else \
                ref.astype(np.float16).view(np.uint16)
            assert np.array_equal(host_bits(y)[:, _slice_cols(o)][act], ref_bits[act])
    else:
        rv, ry, ryi = compare_all_rows(dw)
        print(f"  tolerance ratios: v {rv:.3g}  y {ry:.3g}  y(isolated) {ryi:.3g}")
        assert rv <= 1 and ry <= 1 and ryi <= 1
    check_neg_rows(dw)
    check_outside_slices(dw)


@pytest.mark.parametrize("case", [MIXED_CASES[i] for i in (1, 3, 6, 8, 10)])
@pytest.mark.parametrize("balance", ["1", "2"])
def test_decode_prefill_mix_schedules(monkeypatch, tuning_from_env, case, balance):
    """Mixed batches with the tile expand's schedule forced (round-robin
    items, balanced ranges), its per-token items walked after the tile work:
    bit for bit against the automatic choice's result, and against the
    oracle as in the automatic case."""
    dtype, n_pre, pre_l, n_dec, L, H, r, slices, integer = case
    _announce(f"decode+prefill mix, expand schedule {balance}: {dtype} prefill={n_pre}/{pre_l} "
              f"decode={n_dec} L={L} r={r} slices={slices} integer={integer}")
    w = W.make_mixed("mix", dtype, n_pre, pre_l, n_dec, L, H, r, slices, seed=n_pre + n_dec + r,
                     neg_frac=0.05, integer=integer)
    auto = DeviceWorkload(w)
    auto.run()
    monkeypatch.setenv("LORA_EXPAND_BALANCE", balance)
    tuning_from_env()
    forced = DeviceWorkload(w)
    forced.run()
    for ya, yf in zip(auto.ys, forced.ys):
        assert np.array_equal(host_bits(ya), host_bits(yf))
    if integer:
        act = np.nonzero(w.active)[0]
        v_or = oracle.shrink(w.dtype, w.x, w.A, w.ids)
        for o, y in zip(w.outputs, forced.ys):
            ref = oracle.expand_slice(w.dtype, np.nan_to_num(v_or), [s.B for s in o.slices],
                                      [s.col_off for s in o.slices], w.ids, o.y0, w.add)
            ref_bits = W.f32_to_bits(ref.astype(np.float32), dtype) if dtype == "bf16" else \
                ref.astype(np.float16).view(np.uint16)
            assert np.array_equal(host_bits(y)[:, _slice_cols(o)][act], ref_bits[act])
    else:
        rv, ry, ryi = compare_all_rows(forced)
        assert rv <= 1 and ry <= 1 and ryi <= 1
    check_neg_rows(forced)
    check_outside_slices(forced)


@pytest.mark.parametrize("dtype,widths,r", [("f16", [4096], 64), ("bf16", [16384], 16),
                                           ("bf16", [16384, 4096], 64)])
def test_expand_balanced_choice_at_size(monkeypatch, tuning_from_env, dtype, widths, r):
    """8192 tokens over four sorted segments of 1952-2288 tokens (66 token
    tiles of 128 against 64 for aligned ones): the tile expand takes balanced
    ranges by itself here, also over two slices, whose runs the ranges cross.
    Its result is bit for bit the forced round-robin one, and sampled rows
    (first and last of every segment, and random ones) match the oracle in
    every slice."""
    _announce(f"expand, balanced ranges chosen at 8192 tokens: {dtype} slices={widths} r={r}")
    T, L = 8192, 4
    ids_np = W.sweep_point("sgmv", T, 8, 8, L=L).ids
    counts = np.bincount(ids_np, minlength=L)
    assert sum(-(-int(c) // 128) for c in counts) == 66
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    n = sum(widths)
    offs = [int(o) for o in np.cumsum([0] + widths[:-1])]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(n + r)
    v = torch.randn(T, r, generator=gen, device="cuda")
    Bs = [(torch.randn(L, wd, r, generator=gen, device="cuda") / math.sqrt(r)).to(tdt) for wd in widths]
    y0 = torch.randn(T, n, generator=gen, device="cuda").to(tdt)
    seg = lsb.lora_build_segments(torch.from_numpy(ids_np).cuda(), L)
    y_auto = y0.clone()
    lsb.lora_expand_slice(v, Bs, offs, seg, y_auto, True)
    monkeypatch.setenv("LORA_EXPAND_BALANCE", "1")
    tuning_from_env()
    y_rr = y0.clone()
    lsb.lora_expand_slice(v, Bs, offs, seg, y_rr, True)
    torch.cuda.synchronize()
    assert torch.equal(y_auto.view(torch.int16), y_rr.view(torch.int16))
    starts = np.concatenate([[0], np.cumsum(counts)])
    rows = np.unique(np.concatenate([starts[:-1], starts[1:] - 1,
                                     np.random.default_rng(r).choice(T, 128, replace=False)])).astype(np.int64)
    ridx = torch.from_numpy(rows).cuda()
    v_rows = v.index_select(0, ridx).cpu().numpy().astype(np.float64)
    y0_rows = host_bits(y0.index_select(0, ridx))
    got = decode(host_bits(y_auto.index_select(0, ridx)), dtype)
    for B, off, wd in zip(Bs, offs, widths):
        ref = oracle.expand(dtype, v_rows, host_bits(B), ids_np[rows], y0_rows, off, True)
        assert tol_ratio(got[:, off:off + wd], ref) <= 1


def test_decode_prefill_mix_graph_replays():
    """The split expand (tile launch + per-token launch) captured in a HIP
    graph: three replays with the metadata and outputs overwritten between
    them give the eager step's bits."""
    _announce("decode+prefill mix, graph replays")
    w = W.make_mixed("mixg", "bf16", 1500, 8, 500, 600, 1024, 16, [[1024, 512]], seed=77, neg_frac=0.05)
    eager = DeviceWorkload(w)
    eager.run()
    g_w = DeviceWorkload(w)
    y0 = [y.clone() for y in g_w.ys]
    v0 = g_w.v.clone()
    seg = lsb.Segments(g_w.ids, w.L)
    ws = torch.zeros(max(lsb.lora_shrink_workspace_bytes(w.T, w.L, w.H, w.r), 256), dtype=torch.uint8,
                     device="cuda")

    def step():
        lsb.lora_build_segments(g_w.ids, w.L, seg=seg)
        lsb.lora_shrink(g_w.x, g_w.A, seg, g_w.v, workspace=ws)
        o = w.outputs[0]
        lsb.lora_expand_slice(g_w.v, g_w.Bs[0], [q.col_off for q in o.slices], seg, g_w.ys[0], w.add)

    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    act = np.nonzero(w.active)[0]
    for _ in range(3):
        g_w.ys[0].copy_(y0[0])
        g_w.v.copy_(v0)
        for b in (seg.sorted_token, seg.seg_lora, seg.seg_start, seg.counts):
            b.fill_(-5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(g_w.v.cpu().numpy()[act].view(np.uint32),
                              eager.v.cpu().numpy()[act].view(np.uint32))
        assert np.array_equal(host_bits(g_w.ys[0]), host_bits(eager.ys[0]))


# ---------------------------------------------------------------- fused decode call
FUSED_CASES = [
    # dtype, T, H, r, L, slices, add, integer
    ("f16", 16, 1024, 16, 4, [1024], True, False),         # the 16-token decode shape
    ("f16", 256, 4096, 16, 4, [4096], True, False),        # the 256-token decode shape
    ("bf16", 100, 2048, 8, 7, [512, 256, 256], False, False),
    ("bf16", 300, 1024, 32, 5, [1536, 512], True, True),
    ("f16", 37, 4096, 64, 3, [4096, 1024, 1024], True, False),
    ("bf16", 1, 8192, 64, 2, [2048], True, True),
    ("f16", 700, 512, 16, 600, [2560], True, True),        # a large pool, wider than 2048 columns
    ("bf16", 64, 3000, 32, 9, [520, 8], True, False),      # H and slices off the 2048 / 512 grids
]


@pytest.mark.parametrize("dtype,T,H,r,L,widths,add,integer", FUSED_CASES)
def test_fused_decode(dtype, T, H, r, L, widths, add, integer):
    """lora_shrink_expand (one launch) against the oracle's shrink then
    expand_slice: v and every slice of y (integer inputs: bit for bit); rows
    of tokens without an adapter and columns outside the slices keep their
    values."""
    _announce(f"fused decode {dtype} T={T} H={H} r={r} L={L} slices={widths} add={add} integer={integer}")
    w = W.make("fused", dtype, T, H, r, L, [widths], seed=T + H + r, seq_len=1, neg_frac=0.1, add=add,
               integer=integer)
    dw = DeviceWorkload(w)
    seg = lsb.lora_build_segments(dw.ids, w.L)
    o = w.outputs[0]
    offs = [q.col_off for q in o.slices]
    lsb.lora_shrink_expand(dw.x, dw.A, dw.Bs[0], offs, seg, dw.v, dw.ys[0], add)
    torch.cuda.synchronize()
    act = np.nonzero(w.active)[0]
    cols = _slice_cols(o)
    v_gpu = dw.v.cpu().numpy()
    v_or = oracle.shrink(dtype, w.x, w.A, w.ids)
    Bh = [q.B for q in o.slices]
    ref = oracle.expand_slice(dtype, v_or, Bh, offs, w.ids, o.y0, add)
    if integer:
        assert np.array_equal(v_gpu[act].astype(np.float64), v_or[act])
        ref_bits = W.f32_to_bits(ref[:, cols].astype(np.float32), dtype) if dtype == "bf16" else \
            ref[:, cols].astype(np.float16).view(np.uint16)
        assert np.array_equal(host_bits(dw.ys[0])[:, cols][act], ref_bits[act])
    else:
        assert tol_ratio(v_gpu[act].astype(np.float64), v_or[act]) <= 1
        got = decode(host_bits(dw.ys[0]), dtype)[:, cols]
        assert tol_ratio(got[act], ref[:, cols][act]) <= 1
        # the expand alone, from the GPU's own v
        ref_i = oracle.expand_slice(dtype, np.ascontiguousarray(v_gpu[:, :r].astype(np.float64)), Bh, offs,
                                    w.ids, o.y0, add)
        assert tol_ratio(got[act], ref_i[:, cols][act]) <= 1
    check_neg_rows(dw)
    check_outside_slices(dw)


def test_fused_decode_graph_replays():
    """lora_shrink_expand captured in a HIP graph: three replays, with v and
    y overwritten between them, give the eager call's bits."""
    _announce("fused decode, graph replays")
    w = W.make("fusedg", "bf16", 200, 4096, 16, 4, [[4096, 1024]], seed=9, seq_len=1, neg_frac=0.1)
    o = w.outputs[0]
    offs = [q.col_off for q in o.slices]
    eager = DeviceWorkload(w)
    seg_e = lsb.lora_build_segments(eager.ids, w.L)
    lsb.lora_shrink_expand(eager.x, eager.A, eager.Bs[0], offs, seg_e, eager.v, eager.ys[0], True)
    torch.cuda.synchronize()
    g_w = DeviceWorkload(w)
    seg = lsb.lora_build_segments(g_w.ids, w.L)
    y0 = g_w.ys[0].clone()
    v0 = g_w.v.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lsb.lora_shrink_expand(g_w.x, g_w.A, g_w.Bs[0], offs, seg, g_w.v, g_w.ys[0], True)
    for _ in range(3):
        g_w.ys[0].copy_(y0)
        g_w.v.copy_(v0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(g_w.v.cpu().numpy().view(np.uint32), eager.v.cpu().numpy().view(np.uint32))
        assert np.array_equal(host_bits(g_w.ys[0]), host_bits(eager.ys[0]))


# ---------------------------------------------------------------- metadata that breaks its invariants
@pytest.mark.parametrize("L", [5, 300])
@pytest.mark.parametrize("path", ["auto", "bgmv", "sgmv"])
def test_invalid_metadata_stays_in_bounds(force_path, L, path):
    """The caller may fill lora_segments itself.  Metadata that breaks its
    invariants (random values, S past L, descending starts, counts out of
    range) gives unspecified rows but no error and no access outside the
    buffers, through every kernel family, the lazy tile tables of pools over
    256 adapters and the short-segment pass; a valid step afterwards still
    matches the oracle."""
    _announce(f"invalid metadata L={L} path={path}")
    force_path({"auto": lsb.PATH_AUTO, "bgmv": lsb.PATH_BGMV, "sgmv": lsb.PATH_SGMV}[path])
    T, H, r = 700, 1024, 16
    w = W.make("badmeta", "bf16", T, H, r, L, [[512, 256]], seed=L + 3, seq_len=(1, 8), neg_frac=0.1)
    dw = DeviceWorkload(w)
    o = w.outputs[0]
    offs = [q.col_off for q in o.slices]
    seg = lsb.Segments(dw.ids, L)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(L)
    fills = [
        lambda t: t.copy_(torch.randint(-2 * T, 2 * T, t.shape, generator=gen, dtype=torch.int32)),
        lambda t: t.fill_(L + 5),
        lambda t: t.copy_(torch.arange(t.numel(), 0, -1, dtype=torch.int32).reshape(t.shape) * 3),
        lambda t: t.fill_(-7),
    ]
    for fill in fills:
        for b in (seg.sorted_token, seg.seg_lora, seg.seg_start, seg.counts):
            host = torch.empty(b.shape, dtype=torch.int32)
            fill(host)
            b.copy_(host)
        lsb.lora_shrink(dw.x, dw.A, seg, dw.v)
        lsb.lora_expand_slice(dw.v, dw.Bs[0], offs, seg, dw.ys[0], True)
        lsb.lora_shrink_expand(dw.x, dw.A, dw.Bs[0], offs, seg, dw.v, dw.ys[0], True)
        torch.cuda.synchronize()
    fresh = DeviceWorkload(w)
    fresh.run()
    rv, ry, ryi = compare_with_oracle(fresh)
    assert rv <= 1 and ry <= 1 and ryi <= 1


# ---------------------------------------------------------------- the micro-benchmark PR's shapes
def _golden_shapes():
    out = []
    with open(os.path.join(os.path.dirname(__file__), "golden", "microbench_shapes.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                src, bs, sl, m, k, n, L, srt, ns = line.split()
                out.append((src, int(bs), int(sl), int(m), int(k), int(n), int(L), bool(int(srt)), int(ns)))
    return out


@pytest.mark.parametrize("src,bs,sl,m,rank,n,L,sort,ns", _golden_shapes())
def test_microbench_shapes(src, bs, sl, m, rank, n, L, sort, ns):
    """The problem shapes the micro-benchmark PR prints (tests/golden/
    microbench_shapes.txt): bs sequences of sl tokens (m = bs sl tokens),
    rank k, n columns, sorted by adapter, shrink n -> k then expand k -> n.
    The console table's shape is compared in full; the review thread's
    65536-token example (2 GiB of x) is drawn on the GPU and compared on 256
    sampled rows, each row's inputs copied to the host for the oracle."""
    _announce(f"micro-benchmark shape {src}: {bs} x {sl} tokens, rank {rank}, {n} columns, {L} adapters")
    assert bs * sl == m and ns == 1
    if m <= 4096:
        w = W.make(f"golden_{src}", "f16", m, n, rank, L, [[n]], seed=m + n, seq_len=sl, sort_by_id=sort)
        dw = DeviceWorkload(w)
        dw.run()
        rv, ry, ryi = compare_all_rows(dw)
        assert rv <= 1 and ry <= 1 and ryi <= 1
        return
    ids_np = W.make(f"golden_{src}", "f16", m, 8, 8, L, [[8]], seed=m + n, seq_len=sl, sort_by_id=sort).ids
    gen = torch.Generator(device="cuda")
    gen.manual_seed(m + n)
    x = torch.randn(m, n, generator=gen, device="cuda").half()
    A = (torch.randn(L, rank, n, generator=gen, device="cuda") / math.sqrt(n)).half()
    B = (torch.randn(L, n, rank, generator=gen, device="cuda") / math.sqrt(rank)).half()
    y = torch.randn(m, n, generator=gen, device="cuda").half()
    rows = np.sort(np.random.default_rng(m).choice(m, 256, replace=False)).astype(np.int64)
    ridx = torch.from_numpy(rows).cuda()
    y0_rows = host_bits(y.index_select(0, ridx))
    x_rows = host_bits(x.index_select(0, ridx))
    ids = torch.from_numpy(ids_np).cuda()
    seg = lsb.lora_build_segments(ids, L)
    v = sentinel_v(m, rank)
    lsb.lora_shrink(x, A, seg, v)
    lsb.lora_expand(v, B, seg, y, True)
    torch.cuda.synchronize()
    sub_ids = ids_np[rows]
    A_h, B_h = host_bits(A), host_bits(B)
    v_or = oracle.shrink("f16", x_rows, A_h, sub_ids)
    v_gpu = v.index_select(0, ridx).cpu().numpy().astype(np.float64)
    assert tol_ratio(v_gpu, v_or) <= 1
    y_or = oracle.expand("f16", v_or, B_h, sub_ids, y0_rows, 0, True)
    got = decode(host_bits(y.index_select(0, ridx)), "f16")
    assert tol_ratio(got, y_or) <= 1
