"""fp64 CPU oracle for the multi-LoRA shrink / expand / expand_slice path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``lora_serving_build_amd``) never imports it, and it imports nothing from the
product path: the two share no code.  Inputs reach both sides through the
seeded generators in ``workloads`` (which hold none of the method's arithmetic).

The arithmetic lives in ``lora_oracle.c`` (plain C, fp64, OpenMP over tokens);
this module only builds it with gcc and marshals numpy arrays into it.  Each
function below restates the passage it follows; see the C file for the
definitions written out as loops.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lora_oracle.c")
_LIB = os.path.join(_HERE, "liblora_oracle.so")
# A deliberately broken copy of the oracle can be loaded instead, so that the
# test-suite can show its pins catch planted mistakes (tests/test_oracle_mutants.py).
_LIB = os.environ.get("LORA_ORACLE_MUTANT_LIB", _LIB)

F16, BF16 = 0, 1
_DTYPES = {"f16": F16, "bf16": BF16, F16: F16, BF16: BF16}

_lib = None
_tables: dict = {}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
             "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        stale = (_LIB.endswith("liblora_oracle.so") and os.path.exists(_LIB)
                 and os.path.getmtime(_LIB) < os.path.getmtime(_SRC))
        if not os.path.exists(_LIB) or stale:
            build(force=True)
        L = ctypes.CDLL(_LIB)
        i32, i64, p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        L.oracle_decode_f16.restype = ctypes.c_double
        L.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_decode_bf16.restype = ctypes.c_double
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = ctypes.c_int
        L.oracle_build_segments.argtypes = [p, i32, i32, p, p, p, p]
        L.oracle_shrink.argtypes = [ctypes.c_int, p, i64, p, i32, i32, p, i32,
                                    i32, p, i32, p]
        L.oracle_expand.argtypes = [ctypes.c_int, p, i64, p, i32, i32, p, i32,
                                    i32, p, i64, i64, ctypes.c_int, p, i32, p]
        L.oracle_expand_slice.argtypes = [ctypes.c_int, p, i64, i64, p, p, p,
                                          i32, i32, p, i32, i32, p, i64,
                                          ctypes.c_int, p, i32, p]
        L.oracle_rank_bin.argtypes = [i32]
        L.oracle_rank_bin.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> int:
    """Sets the oracle's OpenMP thread count; returns the previous one.
    Results do not depend on it (every row's sum order is fixed)."""
    return int(lib().oracle_set_num_threads(int(n)))


def decode(bits: np.ndarray, dtype) -> np.ndarray:
    """Exact fp64 value of every 16-bit pattern in ``bits`` (IEEE binary16 or
    bfloat16), by the oracle's own decoder."""
    code = _DTYPES[dtype]
    if code not in _tables:
        f = lib().oracle_decode_f16 if code == F16 else lib().oracle_decode_bf16
        _tables[code] = np.array([f(b) for b in range(65536)], dtype=np.float64)
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return _tables[code][flat].reshape(np.shape(bits))


def build_segments(ids: np.ndarray, L: int):
    """Segment metadata: stable sort of tokens by adapter id, one segment per
    adapter present, tokens without an adapter after the active ones (punica
    issue, SGMV segments).  Returns (sorted_token, seg_lora, seg_start, counts)."""
    ids = _c(ids, np.int32)
    T = ids.shape[0]
    st = np.empty(T, np.int32)
    sl = np.empty(L, np.int32)
    ss = np.empty(L + 1, np.int32)
    cn = np.empty(4, np.int32)
    rc = lib().oracle_build_segments(_ptr(ids), T, L, _ptr(st), _ptr(sl), _ptr(ss), _ptr(cn))
    if rc:
        raise ValueError("oracle_build_segments: bad arguments")
    return st, sl, ss, cn


def shrink(dtype, x: np.ndarray, A: np.ndarray, ids: np.ndarray, rows=None,
           out: np.ndarray | None = None) -> np.ndarray:
    """v[t, j] = sum_h x[t, h] * A[id(t)][j][h] in fp64 (micro-benchmark PR:
    the per-token LoRA-id product).  x is uint16 bits [T][ldx] (first H columns
    used), A is uint16 bits [L][r][H].  Returns [nrows][r]; rows of tokens with
    no adapter hold whatever ``out`` held (NaN by default)."""
    x = np.asarray(x, np.uint16)
    A = _c(A, np.uint16)
    ids = _c(ids, np.int32)
    L, r, H = A.shape
    T, ldx = x.shape
    if x.strides[1] != 2:
        raise ValueError("x rows must be contiguous")
    ldx_e = x.strides[0] // 2
    rows_a = None if rows is None else _c(rows, np.int32)
    nrows = T if rows_a is None else rows_a.shape[0]
    if out is None:
        out = np.full((nrows, r), np.nan, np.float64)
    rc = lib().oracle_shrink(_DTYPES[dtype], _ptr(x), ldx_e, _ptr(A), H, r, _ptr(ids), T, L,
                             _ptr(rows_a), nrows, _ptr(out))
    if rc:
        raise ValueError("oracle_shrink: bad arguments")
    return out


def expand(dtype, v: np.ndarray, B: np.ndarray, ids: np.ndarray, y0: np.ndarray,
           col_off: int, add: bool, rows=None) -> np.ndarray:
    """y[t, col_off + c] = (add ? y0 : 0) + sum_j v[t, j] * B[id(t)][c][j] in
    fp64 (micro-benchmark PR: expand, add_inputs).  v is fp64 [T][ldv], B is
    uint16 bits [L][n][r], y0 uint16 bits [T][ldy].  Returns [nrows][n]; rows of
    tokens with no adapter are y0 unchanged."""
    v = np.asarray(v, np.float64)
    B = _c(B, np.uint16)
    ids = _c(ids, np.int32)
    y0 = np.asarray(y0, np.uint16)
    if v.strides[1] != 8 or y0.strides[1] != 2:
        raise ValueError("rows must be contiguous")
    L, n, r = B.shape
    T = ids.shape[0]
    rows_a = None if rows is None else _c(rows, np.int32)
    nrows = T if rows_a is None else rows_a.shape[0]
    out = np.empty((nrows, n), np.float64)
    rc = lib().oracle_expand(_DTYPES[dtype], _ptr(v), v.strides[0] // 8, _ptr(B), r, n,
                             _ptr(ids), T, L, _ptr(y0), y0.strides[0] // 2, int(col_off),
                             int(bool(add)), _ptr(rows_a), nrows, _ptr(out))
    if rc:
        raise ValueError("oracle_expand: bad arguments")
    return out


def expand_slice(dtype, v: np.ndarray, Bs, col_offs, ids, y0, add: bool,
                 v_slice_stride: int = 0, rows=None) -> np.ndarray:
    """expand_slice: one expand per output slice, back to back (micro-benchmark
    PR).  Bs is a list of uint16 [L][n_s][r]; col_offs the slices' first
    columns; v_slice_stride (elements) moves v between slices (0 = shared v).
    Returns [nrows][sum n_s] with the slices side by side in order."""
    v = np.asarray(v, np.float64)
    Bs = [_c(b, np.uint16) for b in Bs]
    ids = _c(ids, np.int32)
    y0 = np.asarray(y0, np.uint16)
    r = Bs[0].shape[2]
    L = Bs[0].shape[0]
    n_s = np.array([b.shape[1] for b in Bs], np.int32)
    offs = np.array(col_offs, np.int64)
    T = ids.shape[0]
    rows_a = None if rows is None else _c(rows, np.int32)
    nrows = T if rows_a is None else rows_a.shape[0]
    out = np.empty((nrows, int(n_s.sum())), np.float64)
    ptrs = (ctypes.c_void_p * len(Bs))(*[b.ctypes.data for b in Bs])
    rc = lib().oracle_expand_slice(_DTYPES[dtype], _ptr(v), v.strides[0] // 8,
                                   int(v_slice_stride), ptrs, _ptr(n_s), _ptr(offs),
                                   len(Bs), r, _ptr(ids), T, L, _ptr(y0),
                                   y0.strides[0] // 2, int(bool(add)), _ptr(rows_a),
                                   nrows, _ptr(out))
    if rc:
        raise ValueError("oracle_expand_slice: bad arguments")
    return out


def rank_bin(r: int) -> int:
    """Rank rounded up to the nearest supported bin (punica issue: 16 or a
    multiple of 32)."""
    return int(lib().oracle_rank_bin(int(r)))
