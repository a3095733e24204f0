"""ctypes binding of libattn.so (include/attn.h).

Argument marshalling only: torch provides device memory (outputs and
workspace) and the current HIP stream; every step of the computation runs
in the library's HIP kernels.  There is no fallback: if the library is
missing or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_F32, ATTN_BF16 = 0, 1
MASK_MODES = {"none": 0, "causal": 1, "bitmask": 2}
STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_STRIDE",
    4: "ATTN_ERR_DTYPE", 5: "ATTN_ERR_MASK", 6: "ATTN_ERR_UNSUPPORTED",
    7: "ATTN_ERR_WORKSPACE", 8: "ATTN_ERR_ALIAS", 9: "ATTN_ERR_HIP",
}
EXPORTS = ["attn_workspace_size", "attn_fwd", "attn_bwd", "attn_bwd_noalloc", "attn_debug_tile_map",
           "attn_debug_dropout_mask",
           "attn_debug_count_tiles", "attn_timing_enable", "attn_timing_read", "attn_timing_reset",
           "attn_status_str", "attn_last_error", "attn_version"]
KERNELS = ["tile_map", "fwd", "bwd_pre", "bwd", "bwd_post", "bwd_dq", "fwd_merge", "bwd_dq_merge"]


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class AttnProblem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("n", ctypes.c_int64),
        ("d", ctypes.c_int64), ("v", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("mask_mode", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("mask", ctypes.c_void_p),
        ("mask_sb", ctypes.c_int64), ("mask_sh", ctypes.c_int64), ("mask_si", ctypes.c_int64),
        ("sq", ctypes.c_int64 * 3), ("sk", ctypes.c_int64 * 3),
        ("sv", ctypes.c_int64 * 3), ("so", ctypes.c_int64 * 3),
        ("deterministic", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("nk", ctypes.c_int64), ("causal_offset", ctypes.c_int64),
        ("dropout_p", ctypes.c_double), ("dropout_seed", ctypes.c_uint64),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libattn.so once; raise if it is absent (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} not found: build it with `python -m exact_tiled_attention_attn_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(AttnProblem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.attn_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(sz)]
    lib.attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.attn_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.attn_debug_tile_map.argtypes = [P, ctypes.c_int, vp, sz, i32p, i32p, i32p, i32p, vp, sz, vp]
    lib.attn_debug_dropout_mask.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int32, ctypes.c_int32, vp, sz, vp]
    lib.attn_debug_count_tiles.argtypes = [vp]
    for f in ("attn_workspace_size", "attn_fwd", "attn_bwd", "attn_bwd_noalloc", "attn_debug_tile_map",
              "attn_debug_dropout_mask", "attn_debug_count_tiles"):
        getattr(lib, f).restype = ctypes.c_int
    lib.attn_status_str.argtypes = [ctypes.c_int]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_version.restype = ctypes.c_int32
    lib.attn_timing_enable.argtypes = [ctypes.c_int]
    lib.attn_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    for f in ("attn_timing_enable", "attn_timing_read", "attn_timing_reset"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(st: int):
    if st != 0:
        raise AttnError(st, load_library().attn_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _on_gpu(name, t, device=None, dtype=None, shape=None):
    """Checks a tensor argument before its address reaches the library, which
    sees only pointers: device memory, on the inputs' device, of the expected
    dtype and shape."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be in GPU memory, got a tensor on {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _like(t):
    """An output with t's shape and strides (also for views with gaps, which
    torch.empty_like would make contiguous)."""
    return torch.empty_strided(t.size(), t.stride(), dtype=t.dtype, device=t.device)


def make_problem(q, k, v, o_like, scale, mask_mode="none", mask=None, deterministic=False,
                 causal_offset=0, dropout_p=0.0, dropout_seed=0) -> AttnProblem:
    """Fill the ABI problem struct (strides in elements).

    q [B, H, n, d]; k [B, H, nk, d]; v [B, H, nk, v]; o_like [B, H, n, v].
    causal_offset (causal mask only): key j is allowed for query i iff
    j <= i + causal_offset.  dropout_p / dropout_seed: dropout on the
    weights, replayed by the backward with the same values (include/attn.h).
    """
    _on_gpu("q", q)
    _on_gpu("k", k, q.device, q.dtype)
    _on_gpu("v", v, q.device, q.dtype)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("tensors must be [B, H, rows, dim]")
    B, H, n, d = q.shape
    nk = k.shape[2]
    if tuple(k.shape) != (B, H, nk, d) or tuple(v.shape[:3]) != (B, H, nk):
        raise ValueError(f"shapes do not match: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if o_like.device.type != "meta":
        _on_gpu("O", o_like, q.device, q.dtype, (B, H, n, v.shape[-1]))
    p = AttnProblem()
    p.B, p.H, p.n, p.d, p.v = B, H, n, d, v.shape[-1]
    p.nk = nk
    p.causal_offset = int(causal_offset)
    p.dropout_p = float(dropout_p)
    p.dropout_seed = int(dropout_seed) & 0xFFFFFFFFFFFFFFFF
    p.dtype = _dtype_code(q)
    p.mask_mode = MASK_MODES[mask_mode] if isinstance(mask_mode, str) else int(mask_mode)
    p.scale = float(scale)
    for name, t in (("sq", q), ("sk", k), ("sv", v), ("so", o_like)):
        if t.stride(-1) != 1:
            raise ValueError("last dimension must be contiguous")
        arr = getattr(p, name)
        for i in range(3):
            arr[i] = t.stride(i)
    if mask is not None:
        m = _on_gpu("mask", mask, q.device)
        if m.dtype not in (torch.int32, torch.uint32):
            raise TypeError("mask must be int32/uint32 words")
        words = (nk + 31) // 32
        if m.dim() == 3:  # [H, n, words]: shared across the batch
            lead = (H, n)
            p.mask_sb, p.mask_sh, p.mask_si = 0, m.stride(0), m.stride(1)
        elif m.dim() == 4:  # [B, H, n, words]
            lead = (B, H, n)
            p.mask_sb, p.mask_sh, p.mask_si = m.stride(0), m.stride(1), m.stride(2)
        else:
            raise ValueError("mask must be [H, n, words] or [B, H, n, words]")
        # The library reads H (or B H) masks of n rows of ceil(nk / 32) words.
        if tuple(m.shape[:-1]) != lead or m.shape[-1] < words or m.stride(-1) != 1:
            raise ValueError(f"mask of shape {tuple(m.shape)} does not cover {lead} rows of {words} words")
        p.mask = m.data_ptr()
    p.deterministic = int(bool(deterministic))
    return p


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace_size(p: AttnProblem, is_bwd: bool) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    _check(lib.attn_workspace_size(ctypes.byref(p), int(is_bwd), ctypes.byref(out)))
    return out.value


def _workspace(nbytes: int, device, given=None) -> torch.Tensor | None:
    if given is not None:
        _on_gpu("workspace", given, device)
        if not given.is_contiguous():
            raise ValueError("workspace must be contiguous")
        return given
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def fwd(q, k, v, scale, mask_mode="none", mask=None, *, out=None, lse=None, workspace=None,
        causal_offset=0, dropout_p=0.0, dropout_seed=0):
    """O [B,H,n,v] (dtype of q) and L [B,H,n] (fp32 natural-log logsumexp).

    q has n rows, k and v nk rows (any nk >= 1); causal_offset shifts the
    causal mask (key j allowed for query i iff j <= i + causal_offset).
    """
    lib = load_library()
    _on_gpu("q", q)
    B, H, n, _ = q.shape
    o = out if out is not None else torch.empty((B, H, n, v.shape[-1]), dtype=q.dtype, device=q.device)
    L = lse if lse is not None else torch.empty((B, H, n), dtype=torch.float32, device=q.device)
    _on_gpu("lse", L, q.device, torch.float32, (B, H, n))
    if not L.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [B, H, n]")
    p = make_problem(q, k, v, o, scale, mask_mode, mask, causal_offset=causal_offset, dropout_p=dropout_p,
                     dropout_seed=dropout_seed)
    need = workspace_size(p, False)
    ws = _workspace(need, q.device, workspace)
    with torch.cuda.device(q.device):
        _check(lib.attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L),
                            _ptr(ws), ctypes.c_size_t(_nbytes(ws)), _stream()))
    return o, L


def bwd(q, k, v, o, do, lse, scale, mask_mode="none", mask=None, *, dq=None, dk=None, dv=None,
        workspace=None, deterministic=True, causal_offset=0, dropout_p=0.0, dropout_seed=0):
    """dQ, dK, dV (dtype of q) from the forward's O and L and the upstream dO.

    ``deterministic`` (the default) selects the query-tile-outer dQ kernel
    (bitwise reproducible, and the faster path: fp32 atomic adds run at
    about 1.3 TB/s on MI355X, which doubles the backward); False selects
    fp32 atomics in the key-tile-outer kernel.
    """
    lib = load_library()
    _on_gpu("q", q)
    _on_gpu("O", o, q.device, q.dtype)
    _on_gpu("dO", do, q.device, q.dtype, o.shape)
    if do.stride() != o.stride():
        if not o.is_contiguous():
            raise ValueError("dO must have the strides of O")
        do = do.contiguous()
    dq = dq if dq is not None else _like(q)
    dk = dk if dk is not None else _like(k)
    dv = dv if dv is not None else _like(v)
    for name, t, ref in (("dQ", dq, q), ("dK", dk, k), ("dV", dv, v)):
        _on_gpu(name, t, q.device, q.dtype, ref.shape)
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != v.stride():
        raise ValueError("dQ, dK, dV must have the strides of Q, K, V")
    _on_gpu("lse", lse, q.device, torch.float32, q.shape[:3])
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [B, H, n]")
    p = make_problem(q, k, v, o, scale, mask_mode, mask, deterministic, causal_offset, dropout_p, dropout_seed)
    need = workspace_size(p, True)
    ws = _workspace(need, q.device, workspace)
    with torch.cuda.device(q.device):
        _check(lib.attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ctypes.c_size_t(_nbytes(ws)), _stream()))
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, do, lse, scale, mask_mode="none", mask=None, *, dq=None, dk=None, dv=None,
                deterministic=True, causal_offset=0, dropout_p=0.0, dropout_seed=0):
    """attn_bwd_noalloc: bwd() with the library's static scratch as the
    workspace.  The library allocates nothing; dQ, dK, dV are the caller's
    (allocated here only when not given)."""
    lib = load_library()
    _on_gpu("q", q)
    _on_gpu("O", o, q.device, q.dtype)
    _on_gpu("dO", do, q.device, q.dtype, o.shape)
    if do.stride() != o.stride():
        raise ValueError("dO must have the strides of O")
    dq = dq if dq is not None else _like(q)
    dk = dk if dk is not None else _like(k)
    dv = dv if dv is not None else _like(v)
    for name, t, ref in (("dQ", dq, q), ("dK", dk, k), ("dV", dv, v)):
        _on_gpu(name, t, q.device, q.dtype, ref.shape)
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != v.stride():
        raise ValueError("dQ, dK, dV must have the strides of Q, K, V")
    _on_gpu("lse", lse, q.device, torch.float32, q.shape[:3])
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [B, H, n]")
    p = make_problem(q, k, v, o, scale, mask_mode, mask, deterministic, causal_offset, dropout_p, dropout_seed)
    with torch.cuda.device(q.device):
        _check(lib.attn_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                    _ptr(dq), _ptr(dk), _ptr(dv), _stream()))
    return dq, dk, dv


def debug_tile_map(q, k, v, scale, mask_mode="none", mask=None, is_bwd=0, causal_offset=0, deterministic=True):
    """The kernels' (query tile x key tile) classification as uint8 [units, tq, tk].

    is_bwd: 0 forward, 1 key-tile-outer backward, 2 query-tile-outer dQ; the
    key-tile-outer tiling depends on the dQ path (``deterministic``, as in bwd).
    """
    lib = load_library()
    o_like = torch.empty((*q.shape[:3], v.shape[-1]), device="meta")  # strides of a contiguous O
    p = make_problem(q, k, v, o_like, scale, mask_mode, mask, deterministic, causal_offset)
    bq, bk, tq, tk = (ctypes.c_int32() for _ in range(4))
    _check(lib.attn_debug_tile_map(ctypes.byref(p), int(is_bwd), None, 0, ctypes.byref(bq),
                                   ctypes.byref(bk), ctypes.byref(tq), ctypes.byref(tk), None, 0,
                                   _stream()))
    units = 1 if p.mask_mode != 2 else (p.H if p.mask_sb == 0 else p.B * p.H)
    out = torch.empty((units, tq.value, tk.value), dtype=torch.uint8, device=q.device)
    _check(lib.attn_debug_tile_map(ctypes.byref(p), int(is_bwd), _ptr(out), out.numel(),
                                   ctypes.byref(bq), ctypes.byref(bk), ctypes.byref(tq),
                                   ctypes.byref(tk), None, 0, _stream()))
    return out, bq.value, bk.value


def dropout_mask(q, k, v, dropout_p, dropout_seed, b, h, i0, j0, rows, cols):
    """The kernels' dropout keep decisions (uint8 [rows, cols], 1 = kept) of
    unit (b, h), query rows i0.. and keys j0.. (multiples of 4)."""
    lib = load_library()
    o_like = torch.empty((*q.shape[:3], v.shape[-1]), device="meta")
    p = make_problem(q, k, v, o_like, 1.0, dropout_p=dropout_p, dropout_seed=dropout_seed)
    out = torch.empty((rows, cols), dtype=torch.uint8, device=q.device)
    _check(lib.attn_debug_dropout_mask(ctypes.byref(p), b, h, i0, j0, rows, cols, _ptr(out), out.numel(),
                                       _stream()))
    return out


def count_tiles(counters):
    """Set (an int64 device tensor of 3 zeros) or clear (None) the executed-tile
    counters: forward, key-tile-outer backward, query-tile-outer dQ."""
    if counters is not None:
        _on_gpu("counters", counters, dtype=torch.int64, shape=(3,))
        if not counters.is_contiguous():
            raise ValueError("counters must be contiguous")
    _check(load_library().attn_debug_count_tiles(_ptr(counters)))


def timing_enable(on: bool = True):
    """Bracket every library kernel launch with HIP events on its stream."""
    _check(load_library().attn_timing_enable(int(on)))


def timing_read() -> dict:
    """{kernel: (total ms, launches)} accumulated since the last read; waits for the events."""
    n = len(KERNELS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(load_library().attn_timing_read(ms, cnt))
    return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNELS)}
