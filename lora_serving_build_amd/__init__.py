"""Python binding of liblora_mi355x (multi-LoRA shrink / expand on MI355X).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  The entry
points carry the C-ABI names of ``include/lora.h``:

    lora_segments_workspace_bytes, lora_build_segments, lora_shrink,
    lora_expand, lora_expand_slice, lora_shrink_workspace_bytes,
    lora_set_path, lora_reload_tuning, lora_last_error, lora_shrink_noalloc,
    and the single-adapter forms lora_shrink_single, lora_expand_single,
    lora_expand_slice_single, lora_shrink_single_workspace_bytes

If the shared library has not been built (``python -m
lora_serving_build_amd.build``), every entry point raises: there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "LoraError", "Segments", "lib", "lora_build_segments", "lora_shrink", "lora_expand",
    "lora_expand_slice", "lora_shrink_workspace_bytes", "lora_segments_workspace_bytes",
    "lora_last_error", "lora_set_path", "lora_reload_tuning", "lora_shrink_noalloc",
    "LORA_NOALLOC_SCRATCH_BYTES", "lora_shrink_single", "lora_shrink_single_workspace_bytes",
    "lora_expand_single", "lora_expand_slice_single",
    "PATH_AUTO", "PATH_BGMV", "PATH_SGMV", "LORA_F16", "LORA_BF16", "LORA_MAX_RANK", "LORA_MAX_LORAS",
    "LORA_MAX_SLICES", "library_path",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "liblora_mi355x.so")

LORA_OK, LORA_ERR_INVALID_ARG, LORA_ERR_UNSUPPORTED, LORA_ERR_WORKSPACE, LORA_ERR_HIP = 0, -1, -2, -3, -4
LORA_F16, LORA_BF16 = 0, 1
LORA_MAX_RANK, LORA_MAX_LORAS, LORA_MAX_SLICES = 128, 2048, 8
LORA_NOALLOC_SCRATCH_BYTES = 16 << 20


class LoraError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


class _CSegments(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("num_loras", ctypes.c_int32),
        ("token_lora", ctypes.c_void_p),
        ("sorted_token", ctypes.c_void_p),
        ("seg_lora", ctypes.c_void_p),
        ("seg_start", ctypes.c_void_p),
        ("counts", ctypes.c_void_p),
        ("lora_rank", ctypes.c_void_p),
    ]


_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """Loads liblora_mi355x.so; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(library_path):
                raise ImportError(
                    f"{library_path} is missing: build it with "
                    "`python -m lora_serving_build_amd.build` (hipcc, gfx950)")
            L = ctypes.CDLL(library_path)
            p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
            seg_p = ctypes.POINTER(_CSegments)
            L.lora_segments_workspace_bytes.argtypes = [i32, i32]
            L.lora_segments_workspace_bytes.restype = sz
            L.lora_build_segments.argtypes = [p, i32, i32, seg_p, p, sz, p]
            L.lora_reload_tuning.argtypes = []
            L.lora_reload_tuning.restype = None
            L.lora_shrink_workspace_bytes.argtypes = [i32, i32, i32, i32]
            L.lora_shrink_workspace_bytes.restype = sz
            L.lora_shrink.argtypes = [p, i64, p, i32, i32, seg_p, p, i64, p, sz, ctypes.c_int, p]
            L.lora_shrink_noalloc.argtypes = [p, i64, p, i32, i32, seg_p, p, i64, ctypes.c_int, p]
            L.lora_shrink_single_workspace_bytes.argtypes = [i32, i32, i32]
            L.lora_shrink_single_workspace_bytes.restype = sz
            L.lora_shrink_single.argtypes = [p, i64, p, i32, i32, i32, p, i64, p, sz, ctypes.c_int, p]
            L.lora_expand_single.argtypes = [p, i64, p, i32, i32, i32, p, i64, ctypes.c_int, ctypes.c_int, p]
            L.lora_expand_slice_single.argtypes = [p, i64, i64, p, p, p, i32, i32, i32, p, i64,
                                                   ctypes.c_int, ctypes.c_int, p]
            L.lora_expand.argtypes = [p, i64, p, i32, i32, seg_p, p, i64, ctypes.c_int, ctypes.c_int, p]
            L.lora_expand_slice.argtypes = [p, i64, i64, p, p, p, i32, i32, seg_p, p, i64,
                                            ctypes.c_int, ctypes.c_int, p]
            L.lora_shrink_expand.argtypes = [p, i64, p, i32, i32, p, p, p, i32, seg_p, p, i64, p, i64,
                                             ctypes.c_int, ctypes.c_int, p]
            L.lora_last_error.restype = ctypes.c_char_p
            L.lora_set_path.argtypes = [ctypes.c_int]
            L.lora_set_path.restype = ctypes.c_int
            for f in ("lora_build_segments", "lora_shrink", "lora_shrink_noalloc", "lora_expand",
                      "lora_expand_slice", "lora_shrink_single", "lora_expand_single",
                      "lora_expand_slice_single", "lora_shrink_expand"):
                getattr(L, f).restype = ctypes.c_int
            _lib = L
    return _lib


PATH_AUTO, PATH_BGMV, PATH_SGMV = 0, 1, 2


def lora_set_path(mode: int) -> int:
    """Selects the kernel path (0 auto, 1 per-token BGMV, 2 segment SGMV);
    returns the previous mode."""
    rc = lib().lora_set_path(int(mode))
    if rc < 0:
        raise LoraError(rc, lora_last_error())
    return rc


def lora_reload_tuning() -> None:
    """Re-reads the launch-plan override variables from the environment
    (tests and measurement only)."""
    lib().lora_reload_tuning()


def lora_last_error() -> str:
    return lib().lora_last_error().decode()


def _check(rc: int):
    if rc != LORA_OK:
        raise LoraError(rc, lora_last_error())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float16:
        return LORA_F16
    if t == torch.bfloat16:
        return LORA_BF16
    raise TypeError(f"unsupported dtype {t}: x, A, B and y must be float16 or bfloat16")


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _row_major(t: torch.Tensor, name: str):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with contiguous rows")
    return t.stride(0)


class Segments:
    """Segment metadata buffers of one batch (device tensors) and the C
    struct that points at them."""

    def __init__(self, token_lora: torch.Tensor, num_loras: int, lora_rank: torch.Tensor | None = None,
                 buffers=None):
        """buffers (optional): the four int32 device tensors (sorted_token [>= T],
        seg_lora [L], seg_start [L + 1], counts [4]) to use instead of new ones."""
        if token_lora.dtype != torch.int32 or token_lora.dim() != 1 or not token_lora.is_cuda:
            raise ValueError("token_lora must be a 1-D int32 CUDA tensor")
        if lora_rank is not None and (lora_rank.dtype != torch.int32 or lora_rank.shape != (int(num_loras),)
                                      or not lora_rank.is_cuda or not lora_rank.is_contiguous()):
            raise ValueError("lora_rank must be a contiguous int32 CUDA tensor of num_loras entries")
        token_lora = token_lora.contiguous()
        dev = token_lora.device
        T = token_lora.shape[0]
        self.token_lora = token_lora
        self.num_loras = int(num_loras)
        if buffers is None:
            self.sorted_token = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
            self.seg_lora = torch.empty(self.num_loras, dtype=torch.int32, device=dev)
            self.seg_start = torch.empty(self.num_loras + 1, dtype=torch.int32, device=dev)
            self.counts = torch.empty(4, dtype=torch.int32, device=dev)
        else:
            st, sl, ss, cn = buffers
            for t, n in ((st, max(T, 1)), (sl, self.num_loras), (ss, self.num_loras + 1), (cn, 4)):
                if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() < n or t.device != dev:
                    raise ValueError("metadata buffers must be contiguous int32 tensors on the ids' device, "
                                     "of at least T, L, L + 1 and 4 elements")
            self.sorted_token, self.seg_lora, self.seg_start, self.counts = st, sl, ss, cn
        self.lora_rank = lora_rank
        self.c = _CSegments(T, self.num_loras, token_lora.data_ptr(), self.sorted_token.data_ptr(),
                            self.seg_lora.data_ptr(), self.seg_start.data_ptr(),
                            self.counts.data_ptr(), lora_rank.data_ptr() if lora_rank is not None else None)

    @property
    def num_tokens(self) -> int:
        return int(self.c.num_tokens)

    @property
    def device(self) -> torch.device:
        return self.token_lora.device

    def ref(self):
        return ctypes.byref(self.c)


def lora_segments_workspace_bytes(T: int, L: int) -> int:
    return int(lib().lora_segments_workspace_bytes(int(T), int(L)))


def lora_build_segments(token_lora: torch.Tensor, num_loras: int,
                        seg: Segments | None = None, lora_rank: torch.Tensor | None = None) -> Segments:
    """Groups the batch's tokens by adapter id (see include/lora.h).  lora_rank
    (optional, [L] int32): live rank of each adapter, for the segment kernels.
    With seg given, its buffers are reused (seg must have been made for this
    token_lora tensor and num_loras)."""
    if seg is None:
        seg = Segments(token_lora, num_loras, lora_rank)
    elif seg.token_lora.data_ptr() != token_lora.data_ptr() or seg.num_loras != int(num_loras):
        raise ValueError("seg was made for another token_lora tensor or adapter count")
    T = seg.num_tokens
    need = lora_segments_workspace_bytes(T, seg.num_loras)
    ws = _workspace(seg.device, need)
    ws_ptr = ctypes.c_void_p(ws.data_ptr()) if ws is not None else None
    ws_bytes = ws.numel() if ws is not None else 0
    _check(lib().lora_build_segments(ctypes.c_void_p(seg.token_lora.data_ptr()), T, seg.num_loras,
                                     seg.ref(), ws_ptr, ws_bytes, _stream(seg.device)))
    return seg


def lora_shrink_workspace_bytes(T: int, L: int, H: int, r: int) -> int:
    return int(lib().lora_shrink_workspace_bytes(T, L, H, r))


_ws_cache: dict = {}


def _workspace(device: torch.device, nbytes: int) -> torch.Tensor | None:
    """A workspace per (device, stream), grown on demand.  Calls on one stream
    run in order, so they can share it."""
    if nbytes == 0:
        return None
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty((nbytes + 255) // 256 * 256, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def lora_shrink(x: torch.Tensor, A: torch.Tensor, seg: Segments, v: torch.Tensor,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """v[t, :r] = x[t, :H] . A_l for active tokens (A is [L][r][H]); v is fp32."""
    if A.dim() != 3 or not A.is_contiguous():
        raise ValueError("A must be a contiguous [L][r][H] tensor")
    L, r, H = A.shape
    if L != seg.num_loras:
        raise ValueError(f"A holds {L} adapters, segments were built for {seg.num_loras}")
    if v.dtype != torch.float32:
        raise TypeError("v must be float32")
    if x.dtype != A.dtype:
        raise TypeError("x and A must share a dtype")
    ldx = _row_major(x, "x")
    ldv = _row_major(v, "v")
    need = lora_shrink_workspace_bytes(seg.num_tokens, L, H, r)
    if workspace is None:
        workspace = _workspace(x.device, need)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().lora_shrink(ctypes.c_void_p(x.data_ptr()), ldx, ctypes.c_void_p(A.data_ptr()), H, r,
                             seg.ref(), ctypes.c_void_p(v.data_ptr()), ldv, ws_ptr, ws_bytes,
                             _dtype_code(x.dtype), _stream(x.device)))
    return v


def lora_shrink_noalloc(x: torch.Tensor, A: torch.Tensor, seg: Segments, v: torch.Tensor) -> torch.Tensor:
    """lora_shrink whose H-split partial rows go to the library's static
    device scratch: no workspace, no allocation (see include/lora.h)."""
    if A.dim() != 3 or not A.is_contiguous():
        raise ValueError("A must be a contiguous [L][r][H] tensor")
    L, r, H = A.shape
    if L != seg.num_loras:
        raise ValueError(f"A holds {L} adapters, segments were built for {seg.num_loras}")
    if v.dtype != torch.float32:
        raise TypeError("v must be float32")
    if x.dtype != A.dtype:
        raise TypeError("x and A must share a dtype")
    ldx = _row_major(x, "x")
    ldv = _row_major(v, "v")
    _check(lib().lora_shrink_noalloc(ctypes.c_void_p(x.data_ptr()), ldx, ctypes.c_void_p(A.data_ptr()), H, r,
                                     seg.ref(), ctypes.c_void_p(v.data_ptr()), ldv, _dtype_code(x.dtype),
                                     _stream(x.device)))
    return v


def lora_expand(v: torch.Tensor, B: torch.Tensor, seg: Segments, y: torch.Tensor,
                add_inputs: bool = True) -> torch.Tensor:
    """y[t, :n] (+)= v[t, :r] . B_l for active tokens (B is [L][n][r])."""
    if B.dim() != 3 or not B.is_contiguous():
        raise ValueError("B must be a contiguous [L][n][r] tensor")
    L, n, r = B.shape
    if L != seg.num_loras:
        raise ValueError(f"B holds {L} adapters, segments were built for {seg.num_loras}")
    if v.dtype != torch.float32 or y.dtype != B.dtype:
        raise TypeError("v must be float32 and y must share B's dtype")
    ldv = _row_major(v, "v")
    ldy = _row_major(y, "y")
    _check(lib().lora_expand(ctypes.c_void_p(v.data_ptr()), ldv, ctypes.c_void_p(B.data_ptr()), r, n,
                             seg.ref(), ctypes.c_void_p(y.data_ptr()), ldy, int(bool(add_inputs)),
                             _dtype_code(y.dtype), _stream(y.device)))
    return y


def lora_expand_slice(v: torch.Tensor, Bs, col_offs, seg: Segments, y: torch.Tensor,
                      add_inputs: bool = True, v_slice_stride: int = 0) -> torch.Tensor:
    """For each slice s: y[t, off_s : off_s + n_s] (+)= v_s[t, :r] . B_s,l with
    v_s = v shifted by s * v_slice_stride elements."""
    Bs = list(Bs)
    ns = len(Bs)
    if ns != len(col_offs):
        raise ValueError("one column offset per slice")
    r = None
    for b in Bs:
        if b.dim() != 3 or not b.is_contiguous():
            raise ValueError("every B must be a contiguous [L][n_s][r] tensor")
        if b.shape[0] != seg.num_loras or b.dtype != y.dtype:
            raise ValueError("every B must hold num_loras adapters in y's dtype")
        if r is not None and b.shape[2] != r:
            raise ValueError("all slices must share the rank")
        r = b.shape[2]
    if v.dtype != torch.float32:
        raise TypeError("v must be float32")
    ldv = _row_major(v, "v")
    ldy = _row_major(y, "y")
    ptrs = (ctypes.c_void_p * ns)(*[b.data_ptr() for b in Bs])
    n_s = (ctypes.c_int32 * ns)(*[b.shape[1] for b in Bs])
    offs = (ctypes.c_int64 * ns)(*[int(o) for o in col_offs])
    _check(lib().lora_expand_slice(ctypes.c_void_p(v.data_ptr()), ldv, int(v_slice_stride), ptrs, n_s,
                                   offs, ns, r, seg.ref(), ctypes.c_void_p(y.data_ptr()), ldy,
                                   int(bool(add_inputs)), _dtype_code(y.dtype), _stream(y.device)))
    return y


def lora_shrink_expand(x: torch.Tensor, A: torch.Tensor, Bs, col_offs, seg: Segments, v: torch.Tensor,
                       y: torch.Tensor, add_inputs: bool = True) -> torch.Tensor:
    """Shrink then expand_slice in one launch (decode batches): v = x . A_l
    (written) and y[t, off_s : off_s + n_s] (+)= v[t] . B_s,l for every slice.
    r must be 8, 16, 32 or 64 and every row and size 16-byte aligned."""
    if A.dim() != 3 or not A.is_contiguous():
        raise ValueError("A must be a contiguous [L][r][H] tensor")
    L, r, H = A.shape
    if L != seg.num_loras:
        raise ValueError(f"A holds {L} adapters, segments were built for {seg.num_loras}")
    if x.dtype != A.dtype or y.dtype != A.dtype:
        raise TypeError("x, A and y must share a dtype")
    if v.dtype != torch.float32:
        raise TypeError("v must be float32")
    Bs = list(Bs)
    ns = len(Bs)
    if ns != len(col_offs):
        raise ValueError("one column offset per slice")
    for b in Bs:
        if b.dim() != 3 or not b.is_contiguous() or b.shape[0] != L or b.shape[2] != r or b.dtype != y.dtype:
            raise ValueError("every B must be a contiguous [L][n_s][r] tensor in y's dtype")
    ldx = _row_major(x, "x")
    ldv = _row_major(v, "v")
    ldy = _row_major(y, "y")
    ptrs = (ctypes.c_void_p * ns)(*[b.data_ptr() for b in Bs])
    n_s = (ctypes.c_int32 * ns)(*[b.shape[1] for b in Bs])
    offs = (ctypes.c_int64 * ns)(*[int(o) for o in col_offs])
    _check(lib().lora_shrink_expand(ctypes.c_void_p(x.data_ptr()), ldx, ctypes.c_void_p(A.data_ptr()), H, r,
                                    ptrs, n_s, offs, ns, seg.ref(), ctypes.c_void_p(v.data_ptr()), ldv,
                                    ctypes.c_void_p(y.data_ptr()), ldy, int(bool(add_inputs)),
                                    _dtype_code(y.dtype), _stream(y.device)))
    return y


# ---------------------------------------------------------------- one adapter
def _weight2d(W: torch.Tensor, name: str):
    if W.dim() == 3 and W.shape[0] == 1:
        W = W[0]
    if W.dim() != 2 or not W.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D tensor (or [1][..][..])")
    return W


def lora_shrink_single_workspace_bytes(T: int, H: int, r: int) -> int:
    return int(lib().lora_shrink_single_workspace_bytes(T, H, r))


def lora_shrink_single(x: torch.Tensor, A: torch.Tensor, v: torch.Tensor,
                       workspace: torch.Tensor | None = None) -> torch.Tensor:
    """v[t, :r] = x[t, :H] . A for every row t of x, one adapter, no metadata
    (A is [r][H])."""
    A = _weight2d(A, "A")
    r, H = A.shape
    T = x.shape[0]
    if v.dtype != torch.float32 or v.shape[0] < T:
        raise TypeError("v must be float32 with at least as many rows as x")
    if x.dtype != A.dtype:
        raise TypeError("x and A must share a dtype")
    ldx = _row_major(x, "x")
    ldv = _row_major(v, "v")
    need = lora_shrink_single_workspace_bytes(T, H, r)
    if workspace is None:
        workspace = _workspace(x.device, need)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().lora_shrink_single(ctypes.c_void_p(x.data_ptr()), ldx, ctypes.c_void_p(A.data_ptr()), H, r,
                                    T, ctypes.c_void_p(v.data_ptr()), ldv, ws_ptr, ws_bytes,
                                    _dtype_code(x.dtype), _stream(x.device)))
    return v


def lora_expand_single(v: torch.Tensor, B: torch.Tensor, y: torch.Tensor,
                       add_inputs: bool = True) -> torch.Tensor:
    """y[t, :n] (+)= v[t, :r] . B for every row t of y, one adapter, no
    metadata (B is [n][r])."""
    B = _weight2d(B, "B")
    n, r = B.shape
    T = y.shape[0]
    if v.dtype != torch.float32 or y.dtype != B.dtype or v.shape[0] < T:
        raise TypeError("v must be float32 with at least as many rows as y, and y must share B's dtype")
    ldv = _row_major(v, "v")
    ldy = _row_major(y, "y")
    _check(lib().lora_expand_single(ctypes.c_void_p(v.data_ptr()), ldv, ctypes.c_void_p(B.data_ptr()), r, n,
                                    T, ctypes.c_void_p(y.data_ptr()), ldy, int(bool(add_inputs)),
                                    _dtype_code(y.dtype), _stream(y.device)))
    return y


def lora_expand_slice_single(v: torch.Tensor, Bs, col_offs, y: torch.Tensor, add_inputs: bool = True,
                             v_slice_stride: int = 0) -> torch.Tensor:
    """expand_slice for one adapter and no metadata (each B is [n_s][r])."""
    Bs = [_weight2d(b, "B") for b in Bs]
    ns = len(Bs)
    if ns != len(col_offs):
        raise ValueError("one column offset per slice")
    r = Bs[0].shape[1]
    if any(b.shape[1] != r or b.dtype != y.dtype for b in Bs):
        raise ValueError("all slices must share the rank and y's dtype")
    T = y.shape[0]
    if v.dtype != torch.float32 or v.shape[0] < T:
        raise TypeError("v must be float32 with at least as many rows as y")
    ldv = _row_major(v, "v")
    ldy = _row_major(y, "y")
    ptrs = (ctypes.c_void_p * ns)(*[b.data_ptr() for b in Bs])
    n_s = (ctypes.c_int32 * ns)(*[b.shape[0] for b in Bs])
    offs = (ctypes.c_int64 * ns)(*[int(o) for o in col_offs])
    _check(lib().lora_expand_slice_single(ctypes.c_void_p(v.data_ptr()), ldv, int(v_slice_stride), ptrs, n_s,
                                          offs, ns, r, T, ctypes.c_void_p(y.data_ptr()), ldy,
                                          int(bool(add_inputs)), _dtype_code(y.dtype), _stream(y.device)))
    return y
