"""The C-ABI library: it loads, exports every symbol that include/lora.h
declares, and rejects host-checkable errors before launching anything.  CPU
only: every call here returns from argument validation, no kernel runs."""
import ctypes
import os
import re

import pytest

import lora_serving_build_amd as lsb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]

FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: validation fails first


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(lora_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


# The boundary's calls: the four operations, the metadata workspace query and
# the error message, plus this library's shrink workspace query, path switch
# and tuning reload.
BOUNDARY = ("lora_segments_workspace_bytes", "lora_build_segments", "lora_shrink", "lora_expand",
            "lora_expand_slice", "lora_last_error", "lora_shrink_workspace_bytes", "lora_set_path",
            "lora_reload_tuning")


def test_header_declares_the_entry_points():
    names = declared_functions()
    for f in BOUNDARY:
        assert f in names


def test_binding_carries_the_boundary_names():
    for f in BOUNDARY:
        assert callable(getattr(lsb, f)), f


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports_symbol(name):
    lib = lsb.lib()
    assert hasattr(lib, name)


def _seg(T=16, L=4, token=True):
    return lsb._CSegments(T, L, FAKE.value if token else None, FAKE.value, FAKE.value, FAKE.value,
                          FAKE.value)


def _expect(rc, code, text):
    assert rc == code, (rc, lsb.lora_last_error())
    assert text in lsb.lora_last_error()


def test_build_segments_validation():
    lib = lsb.lib()
    s = _seg()
    sp = ctypes.byref(s)
    _expect(lib.lora_build_segments(FAKE, 16, 4, None, None, 0, None), lsb.LORA_ERR_INVALID_ARG,
            "seg is NULL")
    _expect(lib.lora_build_segments(FAKE, -1, 4, sp, None, 0, None), lsb.LORA_ERR_INVALID_ARG,
            "num_tokens")
    for L in (0, lsb.LORA_MAX_LORAS + 1):
        _expect(lib.lora_build_segments(FAKE, 16, L, sp, None, 0, None), lsb.LORA_ERR_UNSUPPORTED,
                "num_loras")
    _expect(lib.lora_build_segments(None, 16, 4, sp, None, 0, None), lsb.LORA_ERR_INVALID_ARG,
            "token buffers")
    s2 = lsb._CSegments(0, 0, None, None, FAKE.value, FAKE.value, FAKE.value)
    _expect(lib.lora_build_segments(FAKE, 16, 4, ctypes.byref(s2), None, 0, None),
            lsb.LORA_ERR_INVALID_ARG, "token buffers")


def test_build_segments_fills_the_struct():
    """The call records T, L and the id pointer in the struct before it
    checks the output buffers (a missing one here, so nothing is launched)."""
    lib = lsb.lib()
    s = lsb._CSegments(99, 99, None, FAKE.value, None, FAKE.value, FAKE.value)
    _expect(lib.lora_build_segments(FAKE, 5, 7, ctypes.byref(s), None, 0, None),
            lsb.LORA_ERR_INVALID_ARG, "segment buffers")
    assert (s.num_tokens, s.num_loras, s.token_lora) == (5, 7, FAKE.value)


@pytest.mark.parametrize("T,L", [(0, 1), (16, 4), (8192, 64), (65536, 2048)])
def test_segments_workspace_bytes(T, L):
    # The one-workgroup builder keeps its scratch in LDS.
    assert lsb.lora_segments_workspace_bytes(T, L) == 0


def test_shrink_validation():
    lib = lsb.lib()
    s = _seg()
    sp = ctypes.byref(s)
    call = lambda **k: lib.lora_shrink(k.get("x", FAKE), k.get("ldx", 64), k.get("A", FAKE), k.get("H", 64),
                                       k.get("r", 16), k.get("seg", sp), k.get("v", FAKE), k.get("ldv", 16),
                                       k.get("ws", FAKE), k.get("wsb", 1 << 30), k.get("dt", 0), None)
    _expect(call(dt=2), lsb.LORA_ERR_INVALID_ARG, "dtype")
    _expect(call(r=0), lsb.LORA_ERR_UNSUPPORTED, "rank")
    _expect(call(r=129), lsb.LORA_ERR_UNSUPPORTED, "rank")
    _expect(call(H=0), lsb.LORA_ERR_INVALID_ARG, "H 0")
    _expect(call(ldx=63), lsb.LORA_ERR_INVALID_ARG, "ldx")
    _expect(call(ldv=15), lsb.LORA_ERR_INVALID_ARG, "ldv")
    _expect(call(x=None), lsb.LORA_ERR_INVALID_ARG, "must not be NULL")
    need = lsb.lora_shrink_workspace_bytes(16, 4, 4096, 16)
    assert need > 0
    prev = lib.lora_set_path(2)          # the segment path is the one that needs a workspace
    try:
        _expect(call(H=4096, ldx=4096, wsb=need - 1), lsb.LORA_ERR_WORKSPACE, "workspace")
        _expect(call(H=4096, ldx=4096, ws=None), lsb.LORA_ERR_WORKSPACE, "workspace")
    finally:
        lib.lora_set_path(prev)
    _expect(call(seg=None), lsb.LORA_ERR_INVALID_ARG, "seg is NULL")
    # T = 0 is valid and launches nothing.
    s0 = _seg(T=0)
    assert call(seg=ctypes.byref(s0)) == lsb.LORA_OK


def test_workspace_size_is_zero_when_not_split():
    # Large batches need no split of H across workgroups, hence no workspace.
    assert lsb.lora_shrink_workspace_bytes(0, 4, 4096, 16) == 0
    assert lsb.lora_shrink_workspace_bytes(65536, 4, 4096, 16) == 0
    assert lsb.lora_shrink_workspace_bytes(256, 4, 4096, 16) > 0
    # 16-token groups (r <= 32, one round of groups, small H): the H split
    # stays inside the workgroup, so no partial rows either.
    assert lsb.lora_shrink_workspace_bytes(2048, 4, 1024, 16) == 0
    assert lsb.lora_shrink_workspace_bytes(1024, 4, 2048, 32) > 0


@pytest.mark.parametrize("T,L,H,r,ks_cap,rp", [
    (8192, 64, 8192, 64, 12, 64),   # r = 64 from 4096 tokens: 128-token tiles, 64 at the fewest,
                                    # 3 workgroups per CU: up to 12 chunks
    (2048, 4, 8192, 64, 16, 64),    # r = 64 below 4096 tokens: 64-token tiles, 32 at the fewest,
                                    # capped at 16 chunks (512-wide)
    (16384, 4, 4096, 16, 4, 16),    # 256 tiles: 4 chunks
    (32768, 4, 4096, 16, 2, 16),    # 512 tiles: 2 chunks
    (8192, 4, 4096, 128, 4, 128),   # rank 128 holds 512 workgroups: 128 tiles take 4 chunks
    (2048, 4, 4096, 16, 8, 16),     # 32 tiles: capped at four 128-wide blocks per chunk
    (1024, 16, 4096, 128, 8, 128),  # the same cap at rank 128
    (4096, 1040, 4096, 16, 8, 16),  # a large adapter pool: the bound (1104 tiles) takes no split
])
def test_shrink_split_fills_one_round(T, L, H, r, ks_cap, rp):
    """The workspace holds a 256-byte header and ks_cap chunks of fp32
    partial rows (rp = r padded to a rank tile): the most chunks the kernel
    may choose.  With 64-token tiles that is the split the fewest tiles of T
    tokens would take to fill one round of resident workgroups; with
    128-token tiles (r = 33..64 from 4096 tokens), the most chunks that keep
    the fewest tiles' items within the resident workgroups."""
    assert lsb.lora_shrink_workspace_bytes(T, L, H, r) == 256 + ks_cap * T * rp * 4


def _slice_call(lib, sp, Bs, ns, offs, ldy=64, r=16, stride=0, dt=0, nsl=None, ldv=16):
    k = len(ns) if nsl is None else nsl
    B = (ctypes.c_void_p * max(len(Bs), 1))(*Bs)
    n = (ctypes.c_int32 * max(len(ns), 1))(*ns)
    o = (ctypes.c_int64 * max(len(offs), 1))(*offs)
    return lib.lora_expand_slice(FAKE, ldv, stride, B, n, o, k, r, sp, FAKE, ldy, 1, dt, None)


def test_expand_slice_validation():
    lib = lsb.lib()
    s = _seg()
    sp = ctypes.byref(s)
    F = FAKE.value
    _expect(_slice_call(lib, sp, [F], [32], [0], nsl=0), lsb.LORA_ERR_UNSUPPORTED, "num_slices")
    _expect(_slice_call(lib, sp, [F] * 9, [4] * 9, list(range(0, 36, 4)), nsl=9),
            lsb.LORA_ERR_UNSUPPORTED, "num_slices")
    _expect(_slice_call(lib, sp, [F, F], [32, 32], [0, 16]), lsb.LORA_ERR_INVALID_ARG, "overlap")
    _expect(_slice_call(lib, sp, [F, F], [32, 32], [32, 0], ldy=63), lsb.LORA_ERR_INVALID_ARG, "outside")
    _expect(_slice_call(lib, sp, [F], [0], [0]), lsb.LORA_ERR_INVALID_ARG, "n_s[0]")
    _expect(_slice_call(lib, sp, [F], [8], [-8]), lsb.LORA_ERR_INVALID_ARG, "outside")
    _expect(_slice_call(lib, sp, [None], [8], [0]), lsb.LORA_ERR_INVALID_ARG, "B[0] is NULL")
    _expect(_slice_call(lib, sp, [F], [8], [0], r=200, ldv=200), lsb.LORA_ERR_UNSUPPORTED, "rank")
    _expect(_slice_call(lib, sp, [F], [8], [0], stride=-1), lsb.LORA_ERR_INVALID_ARG, "v_slice_stride")
    _expect(_slice_call(lib, sp, [F], [8], [0], dt=5), lsb.LORA_ERR_INVALID_ARG, "dtype")
    # Slices given out of column order but disjoint are fine (T = 0: no launch).
    s0 = _seg(T=0)
    assert _slice_call(lib, ctypes.byref(s0), [F, F], [16, 16], [16, 0], ldy=32) == lsb.LORA_OK


def test_expand_reports_under_its_name():
    lib = lsb.lib()
    s = _seg()
    rc = lib.lora_expand(FAKE, 16, FAKE, 16, 0, ctypes.byref(s), FAKE, 64, 1, 0, None)
    assert rc == lsb.LORA_ERR_INVALID_ARG
    assert lsb.lora_last_error().startswith("lora_expand:")


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(lsb, "_lib", None)
    monkeypatch.setattr(lsb, "library_path", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        lsb.lib()


def test_set_path_validation():
    lib = lsb.lib()
    prev = lib.lora_set_path(0)
    assert prev in (0, 1, 2)
    _expect(lib.lora_set_path(3), lsb.LORA_ERR_INVALID_ARG, "mode 3")
    _expect(lib.lora_set_path(-1), lsb.LORA_ERR_INVALID_ARG, "mode -1")
    assert lib.lora_set_path(2) == 0
    assert lib.lora_set_path(1) == 2
    assert lib.lora_set_path(prev) == 1


def test_forced_bgmv_rejects_large_rank_before_launch():
    """Forced onto the per-token kernels, an expand rank they do not take
    (above 64 and not an aligned 128) is refused before any launch; a rank
    above 128 is refused by every entry point."""
    lib = lsb.lib()
    s = _seg()
    prev = lib.lora_set_path(1)
    try:
        rc = lib.lora_shrink(FAKE, 4096, FAKE, 4096, 129, ctypes.byref(s), FAKE, 129, FAKE, 1 << 30, 0,
                             None)
        _expect(rc, lsb.LORA_ERR_UNSUPPORTED, "rank")
        rc = _slice_call(lib, ctypes.byref(s), [FAKE.value], [8], [0], r=100, ldy=64, ldv=100)
        _expect(rc, lsb.LORA_ERR_UNSUPPORTED, "per-token path")
        rc = _slice_call(lib, ctypes.byref(s), [FAKE.value], [12], [0], r=128, ldy=64, ldv=128)
        _expect(rc, lsb.LORA_ERR_UNSUPPORTED, "per-token path")     # n % 8 != 0: not aligned
    finally:
        lib.lora_set_path(prev)


def test_noalloc_shrink_rejects_splits_beyond_its_scratch():
    """lora_shrink_noalloc refuses, before anything is launched or looked up
    on a device, a shrink whose H split needs more than the static scratch."""
    lib = lsb.lib()
    # rank 128 (64-token tiles): 65 tiles at the bound take 8 chunks of
    # 4096 x 128 fp32 partial rows, 256 bytes past 16 MiB with the header
    T, L, H, r = 4096, 1, 8192, 128
    assert lsb.lora_shrink_workspace_bytes(T, L, H, r) > lsb.LORA_NOALLOC_SCRATCH_BYTES
    s = _seg(T=T, L=L)
    prev = lib.lora_set_path(2)
    try:
        rc = lib.lora_shrink_noalloc(FAKE, H, FAKE, H, r, ctypes.byref(s), FAKE, r, 0, None)
        _expect(rc, lsb.LORA_ERR_UNSUPPORTED, "static scratch")
        _expect(lib.lora_shrink_noalloc(FAKE, H, FAKE, H, r, ctypes.byref(s), FAKE, r, 7, None),
                lsb.LORA_ERR_INVALID_ARG, "dtype")
        _expect(lib.lora_shrink_noalloc(FAKE, H - 8, FAKE, H, r, ctypes.byref(s), FAKE, r, 0, None),
                lsb.LORA_ERR_INVALID_ARG, "ldx")
    finally:
        lib.lora_set_path(prev)
    assert lsb.lora_last_error().startswith("lora_shrink_noalloc:")


def test_shrink_expand_validation():
    """The fused decode call refuses, before anything is launched, ranks
    other than 8, 16, 32 and 64, unaligned data and the usual argument
    errors; T = 0 launches nothing."""
    lib = lsb.lib()
    s = _seg()
    sp = ctypes.byref(s)
    B = (ctypes.c_void_p * 1)(FAKE.value)
    ns = (ctypes.c_int32 * 1)(64)
    off = (ctypes.c_int64 * 1)(0)

    def call(**k):
        return lib.lora_shrink_expand(k.get("x", FAKE), k.get("ldx", 64), k.get("A", FAKE), k.get("H", 64),
                                      k.get("r", 16), k.get("B", B), k.get("ns", ns), k.get("off", off),
                                      k.get("nsl", 1), k.get("seg", sp), k.get("v", FAKE), k.get("ldv", 16),
                                      k.get("y", FAKE), k.get("ldy", 64), 1, k.get("dt", 0), None)

    _expect(call(dt=3), lsb.LORA_ERR_INVALID_ARG, "dtype")
    _expect(call(r=24), lsb.LORA_ERR_UNSUPPORTED, "8, 16, 32 or 64")
    _expect(call(r=128, ldv=128), lsb.LORA_ERR_UNSUPPORTED, "8, 16, 32 or 64")
    _expect(call(r=0), lsb.LORA_ERR_UNSUPPORTED, "rank")
    _expect(call(H=0), lsb.LORA_ERR_INVALID_ARG, "H 0")
    _expect(call(ldx=60), lsb.LORA_ERR_INVALID_ARG, "ldx")
    _expect(call(ldv=8), lsb.LORA_ERR_INVALID_ARG, "ldv")
    _expect(call(nsl=0), lsb.LORA_ERR_UNSUPPORTED, "num_slices")
    _expect(call(ldy=32), lsb.LORA_ERR_INVALID_ARG, "outside [0, ldy")
    _expect(call(x=None), lsb.LORA_ERR_INVALID_ARG, "must not be NULL")
    _expect(call(seg=None), lsb.LORA_ERR_INVALID_ARG, "seg is NULL")
    _expect(call(H=60, ldx=64), lsb.LORA_ERR_UNSUPPORTED, "aligned")
    _expect(call(x=ctypes.c_void_p(FAKE.value + 2)), lsb.LORA_ERR_UNSUPPORTED, "aligned")
    _expect(call(ns=(ctypes.c_int32 * 1)(60)), lsb.LORA_ERR_UNSUPPORTED, "aligned")
    s0 = _seg(T=0)
    assert call(seg=ctypes.byref(s0)) == lsb.LORA_OK


def test_single_adapter_validation():
    """The single-adapter entry points: T < 0 and the usual argument errors
    are refused before anything is launched."""
    lib = lsb.lib()
    _expect(lib.lora_shrink_single(FAKE, 64, FAKE, 64, 16, -1, FAKE, 16, None, 0, 0, None),
            lsb.LORA_ERR_INVALID_ARG, "T -1")
    _expect(lib.lora_shrink_single(FAKE, 63, FAKE, 64, 16, 8, FAKE, 16, None, 0, 0, None),
            lsb.LORA_ERR_INVALID_ARG, "ldx")
    _expect(lib.lora_shrink_single(FAKE, 64, FAKE, 64, 200, 8, FAKE, 200, None, 0, 0, None),
            lsb.LORA_ERR_UNSUPPORTED, "rank")
    need = lsb.lora_shrink_single_workspace_bytes(256, 4096, 16)
    assert need == lsb.lora_shrink_workspace_bytes(256, 1, 4096, 16)
    prev = lib.lora_set_path(2)
    try:
        _expect(lib.lora_shrink_single(FAKE, 4096, FAKE, 4096, 16, 256, FAKE, 16, FAKE, need - 1, 0, None),
                lsb.LORA_ERR_WORKSPACE, "workspace")
    finally:
        lib.lora_set_path(prev)
    assert lib.lora_shrink_single(FAKE, 64, FAKE, 64, 16, 0, FAKE, 16, None, 0, 0, None) == lsb.LORA_OK
    _expect(lib.lora_expand_single(FAKE, 16, FAKE, 16, 64, -2, FAKE, 64, 1, 0, None),
            lsb.LORA_ERR_INVALID_ARG, "T -2")
    assert lsb.lora_last_error().startswith("lora_expand_single:")
    B = (ctypes.c_void_p * 2)(FAKE.value, FAKE.value)
    n = (ctypes.c_int32 * 2)(32, 32)
    o = (ctypes.c_int64 * 2)(0, 16)
    _expect(lib.lora_expand_slice_single(FAKE, 16, 0, B, n, o, 2, 16, 8, FAKE, 64, 1, 0, None),
            lsb.LORA_ERR_INVALID_ARG, "overlap")
