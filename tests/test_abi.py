"""The C-ABI library on the CPU: it loads, exports what include/attn.h
declares, and rejects every invalid argument before anything is launched
(no call here reaches a HIP API)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import exact_tiled_attention_attn_amd as E
from exact_tiled_attention_attn_amd._binding import AttnProblem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(attn_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = E.load_library()
    names = declared_functions()
    assert set(names) == set(E.EXPORTS)
    for name in names:
        assert getattr(lib, name) is not None
    assert lib.attn_version() == 600


def problem(B=1, H=2, n=100, d=64, v=64, dtype=1, mask_mode=0, contiguous=True):
    p = AttnProblem()
    p.B, p.H, p.n, p.d, p.v = B, H, n, d, v
    p.dtype, p.mask_mode, p.scale = dtype, mask_mode, 0.125
    for name, w in (("sq", d), ("sk", d), ("sv", v), ("so", v)):
        arr = getattr(p, name)
        arr[0], arr[1], arr[2] = H * n * w, n * w, w
    return p


def call_fwd(p, Q=FAKE, K=FAKE + (1 << 30), V=FAKE + (2 << 30), O=FAKE + (3 << 30),
             L=FAKE + (4 << 30), ws=None, ws_bytes=0):
    lib = E.load_library()
    vp = ctypes.c_void_p
    return lib.attn_fwd(ctypes.byref(p), vp(Q), vp(K), vp(V), vp(O), vp(L), vp(ws),
                        ctypes.c_size_t(ws_bytes), None)


def call_bwd(p, ptrs=None, ws=None, ws_bytes=0):
    lib = E.load_library()
    base = [FAKE + (i << 30) for i in range(9)]
    if ptrs:
        base = [ptrs.get(i, x) for i, x in enumerate(base)]
    vp = ctypes.c_void_p
    return lib.attn_bwd(ctypes.byref(p), *[vp(x) for x in base], vp(ws), ctypes.c_size_t(ws_bytes), None)


def err():
    return E.load_library().attn_last_error().decode()


def wsize(p, is_bwd):
    out = ctypes.c_size_t()
    st = E.load_library().attn_workspace_size(ctypes.byref(p), is_bwd, ctypes.byref(out))
    return st, out.value


def test_workspace_formula():
    for dtype in (0, 1):
        for (B, H, n, d, v) in ((1, 1, 1, 64, 64), (2, 3, 1000, 80, 80), (1, 32, 16384, 128, 128)):
            p = problem(B, H, n, d, v, dtype)
            st, fw = wsize(p, 0)
            assert st == 0 and fw == 0
            st, bw = wsize(p, 1)
            al = lambda x: (x + 255) // 256 * 256  # noqa: E731
            npad = (n + 127) // 128 * 128  # D and L log2(e) rows, padded per head
            assert st == 0 and bw == 2 * al(4 * B * H * npad) + al(4 * B * H * n * d)
            p.deterministic = 1  # no dQ accumulator; bf16 with a two-wave dK/dV kernel: -L/c rows too
            st, bw = wsize(p, 1)
            rows = 3 if dtype == 1 and (d, v) in ((64, 64), (64, 128), (128, 128)) else 2
            assert st == 0 and bw == rows * al(4 * B * H * npad)
    # bitmask: + tile map (units x tq x tk bytes); forward tiles 128 x 64, backward 64 x 128 (bf16)
    p = problem(2, 8, 8192, 64, 128, 1, 2)
    p.mask = FAKE
    p.mask_sb, p.mask_sh, p.mask_si = 0, 8192 * 256, 256
    st, fw = wsize(p, 0)
    assert st == 0 and fw == (8 * 64 * 128 + 255) // 256 * 256
    st, bw = wsize(p, 1)
    assert bw == 2 * 4 * 16 * 8192 + 4 * 16 * 8192 * 64 + 8 * 128 * 64
    p.deterministic = 1  # D, L2 + key-tile-outer map (64 x 128 tiles) + dQ map (256 x 64 tiles)
    st, bw = wsize(p, 1)
    assert bw == 2 * 4 * 16 * 8192 + 8 * 128 * 64 + 8 * 32 * 128
    p.dtype = 0  # fp32: key-tile-outer map at 32 x 128 tiles, dQ map at 128 x 32 tiles
    st, bw = wsize(p, 1)
    assert bw == 2 * 4 * 16 * 8192 + 8 * 256 * 64 + 8 * 64 * 256


@pytest.mark.parametrize("mut,status", [
    (lambda p: setattr(p, "n", 0), 2),
    (lambda p: setattr(p, "B", 0), 2),
    (lambda p: setattr(p, "d", 96), 6),
    (lambda p: (setattr(p, "d", 128), setattr(p, "v", 64)), 6),
    (lambda p: setattr(p, "dtype", 7), 4),
    (lambda p: setattr(p, "mask_mode", 3), 5),
    (lambda p: setattr(p, "mask_mode", 2), 5),  # bitmask without mask
    (lambda p: setattr(p, "deterministic", 2), 6),
    (lambda p: setattr(p, "reserved", 1), 6),
    (lambda p: setattr(p, "scale", float("inf")), 2),
    (lambda p: setattr(p, "scale", float("nan")), 2),
    (lambda p: p.sq.__setitem__(2, 63), 3),   # row stride not 16-byte multiple / overlapping
    (lambda p: p.sq.__setitem__(2, 32), 3),   # rows overlap
    (lambda p: p.sk.__setitem__(1, -6400), 3),
    (lambda p: p.so.__setitem__(1, 64 * 99), 3),  # heads overlap
    (lambda p: (setattr(p, "n", 1), p.sq.__setitem__(2, 1 << 31)), 6),  # row stride past 32-bit offsets
    (lambda p: (setattr(p, "n", 1), p.sq.__setitem__(2, 1 << 24)), 6),  # 256 padded rows span > 4 GiB
    (lambda p: (setattr(p, "nk", 3), p.sv.__setitem__(2, 3 << 22)), 6),  # the same for V at nk rows
    (lambda p: setattr(p, "nk", -1), 2),
    (lambda p: setattr(p, "causal_offset", 3), 5),  # offset without the causal mask
    (lambda p: (setattr(p, "mask_mode", 1), setattr(p, "causal_offset", (1 << 30) + 1)), 2),
    (lambda p: (setattr(p, "mask_mode", 1), setattr(p, "causal_offset", -(1 << 30) - 1)), 2),
    (lambda p: (setattr(p, "nk", 1 << 20), p.sk.__setitem__(1, 64 * 99)), 3),  # K heads overlap at nk rows
    (lambda p: setattr(p, "dropout_p", 1.0), 2),
    (lambda p: setattr(p, "dropout_p", -0.25), 2),
    (lambda p: setattr(p, "dropout_p", float("nan")), 2),
])
def test_invalid_problem_rejected(mut, status):
    p = problem()
    mut(p)
    assert call_fwd(p) == status, err()
    assert call_bwd(p) == status, err()
    assert wsize(p, 0)[0] == status
    assert err() != ""


def test_rectangular_problems():
    """nk key rows (0 = n) and a causal offset: validation, tiling, workspace."""
    p = problem(n=100)
    p.nk, p.mask_mode, p.causal_offset = 0, 1, -40
    assert wsize(p, 0) == (0, 0)
    p.nk = 300  # K and V views [B, H, 300, .] inside their strides
    for name, w in (("sk", 64), ("sv", 64)):
        arr = getattr(p, name)
        arr[0], arr[1], arr[2] = 2 * 300 * w, 300 * w, w
    assert wsize(p, 0) == (0, 0) and wsize(p, 1)[0] == 0, err()
    bq, bk, tq, tk = (ctypes.c_int32() for _ in range(4))
    lib = E.load_library()
    assert lib.attn_debug_tile_map(ctypes.byref(p), 0, None, 0, ctypes.byref(bq), ctypes.byref(bk),
                                   ctypes.byref(tq), ctypes.byref(tk), None, 0, None) == 0
    assert (tq.value, tk.value) == (-(-100 // bq.value), -(-300 // bk.value))
    # Bitmask: a row holds ceil(nk / 32) words; the maps follow nk.
    p.mask_mode, p.causal_offset = 2, 0
    p.mask = FAKE + (6 << 30)
    p.mask_sb, p.mask_sh, p.mask_si = 0, 100 * 10, 10  # ceil(300 / 32) = 10 words
    st, bw = wsize(p, 1)
    assert st == 0
    rows = 2 * 128  # B H n_pad
    map_kv = 2 * 2 * 3   # heads x (100 / 64 -> 2 query tiles) x (300 / 128 -> 3 key tiles)
    assert bw == 4 * rows + 4 * rows + 4 * 1 * 2 * 100 * 64 + 256 * (-(-map_kv // 256))
    p.mask_si = 9
    assert wsize(p, 1)[0] == 5, err()


def test_dropout_mask_entry_validation():
    lib = E.load_library()
    p = problem()
    out = FAKE
    call = lambda pp, b=0, h=0, i0=0, j0=0, rows=4, cols=4, nbytes=16: lib.attn_debug_dropout_mask(  # noqa: E731
        ctypes.byref(pp), b, h, i0, j0, rows, cols, ctypes.c_void_p(out), nbytes, None)
    assert call(p) == 6, err()  # dropout not enabled
    p.dropout_p = 0.001  # rounds to p8 = 0: still disabled
    assert call(p) == 6, err()
    p.dropout_p = 0.1
    assert call(p, i0=2) == 2 and call(p, j0=6) == 2 and call(p, rows=0) == 2, err()
    assert call(p, b=1) == 2 and call(p, h=2) == 2, err()
    assert call(p, nbytes=15) == 7, err()
    assert lib.attn_debug_dropout_mask(ctypes.byref(p), 0, 0, 0, 0, 4, 4, None, 16, None) == 1


def test_forward_split_workspace():
    """Few query tiles against many key tiles (bf16, d, v in {64, 128}): the
    forward's workspace holds S <= 16 key-range splits of fp32 O and L."""
    p = problem(B=1, H=2, n=100, d=128, v=128)
    p.nk = 8192
    for name, w in (("sk", 128), ("sv", 128)):
        arr = getattr(p, name)
        arr[0], arr[1], arr[2] = 2 * 8192 * w, 8192 * w, w
    S = 16  # 2 query tiles' worth of work is far below one workgroup per CU
    rows = S * 2 * 100
    align = lambda x: -(-x // 256) * 256  # noqa: E731
    assert wsize(p, 0) == (0, align(rows * 128 * 4) + align(rows * 4))
    p.dropout_p = 0.2  # dropout splits the same way (each split replays its keys' decisions)
    assert wsize(p, 0) == (0, align(rows * 128 * 4) + align(rows * 4))
    p.dropout_p, p.nk = 0.0, 1000  # 16 key tiles: four per split at most
    for name, w in (("sk", 128), ("sv", 128)):
        arr = getattr(p, name)
        arr[0], arr[1], arr[2] = 2 * 1000 * w, 1000 * w, w
    rows = 4 * 2 * 100
    assert wsize(p, 0) == (0, align(rows * 128 * 4) + align(rows * 4))
    p.dtype = 0  # fp32: no splits
    assert wsize(p, 0) == (0, 0)


def test_dq_split_workspace_with_and_without_dropout():
    """Deterministic backward, few query tiles against many key tiles (bf16,
    (d, v) = (128, 128)): the workspace holds D, L log2(e) (and, without
    dropout, the -L/c rows of the two-wave dK/dV kernel) and the dQ kernel's
    S key-range partials, with dropout too (the pipelined dQ kernel replays
    the mask)."""
    p = problem(B=1, H=2, n=100, d=128, v=128)
    p.nk, p.deterministic = 8192, 1
    for name, w in (("sk", 128), ("sv", 128)):
        arr = getattr(p, name)
        arr[0], arr[1], arr[2] = 2 * 8192 * w, 8192 * w, w
    align = lambda x: -(-x // 256) * 256  # noqa: E731
    S = 16  # 2 workgroups of 256 queries: min(16, ceil(512 / 2), 128 key tiles / 4)
    expected = 2 * align(4 * 2 * 128) + align(S * 2 * 100 * 128 * 4)
    assert wsize(p, 1) == (0, expected + align(4 * 2 * 128))
    p.dropout_p = 0.2
    assert wsize(p, 1) == (0, expected)
    p.deterministic = 0  # atomic path: the fp32 dQ accumulator, no splits
    assert wsize(p, 1) == (0, 2 * align(4 * 2 * 128) + align(4 * 2 * 100 * 128))


def test_null_and_misaligned_pointers():
    p = problem()
    assert call_fwd(p, Q=0) == 1 and "Q" in err()
    assert call_fwd(p, L=0) == 1
    assert call_fwd(p, V=FAKE + 8) == 3 and "aligned" in err()
    assert call_bwd(p, {4: 0}) == 1 and "dO" in err()
    lib = E.load_library()
    assert lib.attn_fwd(None, None, None, None, None, None, None, 0, None) == 1


def test_aliasing_outputs_rejected():
    p = problem()
    assert call_fwd(p, O=FAKE) == 8  # O on top of Q
    assert call_fwd(p, L=FAKE + (2 << 30) + 64) == 8  # L inside V
    assert call_bwd(p, {6: FAKE + (7 << 30)}) == 8  # dQ on dK
    assert call_bwd(p, {8: FAKE + (3 << 30)}) == 8  # dV on O


def test_workspace_checks():
    p = problem()
    st, need = wsize(p, 1)
    assert need > 0
    assert call_bwd(p) == 7 and "workspace" in err()
    assert call_bwd(p, ws=FAKE + (20 << 30), ws_bytes=need - 1) == 7
    assert call_bwd(p, ws=FAKE + (20 << 30) + 16, ws_bytes=need) == 7  # not 256-byte aligned
    assert call_bwd(p, ws=FAKE, ws_bytes=need) == 8  # workspace overlaps Q


def test_noalloc_backward_validation():
    """attn_bwd_noalloc validates like attn_bwd and refuses problems whose
    workspace exceeds its static 64 MiB buffer, before any device call."""
    lib = E.load_library()
    vp = ctypes.c_void_p
    ptrs = [vp(FAKE + (i << 30)) for i in range(9)]
    p = problem(B=2, H=32, n=4096, d=128, v=128)  # atomic path: 4 B H n d = 128 MiB of accumulator
    assert lib.attn_bwd_noalloc(ctypes.byref(p), *ptrs, None) == 7
    assert "static" in err() and "attn_workspace_size" in err()
    p = problem()
    assert lib.attn_bwd_noalloc(ctypes.byref(p), *([vp(0)] + ptrs[1:]), None) == 1 and "Q" in err()
    p.d = 96
    assert lib.attn_bwd_noalloc(ctypes.byref(p), *ptrs, None) == 6


def test_tile_counter_setting():
    """attn_debug_count_tiles only records the pointer (no device access):
    misaligned pointers are refused, NULL switches counting off."""
    lib = E.load_library()
    assert lib.attn_debug_count_tiles(ctypes.c_void_p(FAKE + 4)) == 3 and "aligned" in err()
    assert lib.attn_debug_count_tiles(ctypes.c_void_p(FAKE)) == 0
    assert lib.attn_debug_count_tiles(None) == 0


def test_status_strings():
    lib = E.load_library()
    for s in range(10):
        assert lib.attn_status_str(s)
    assert lib.attn_status_str(99) == b"unknown status"


def test_missing_library_fails_loudly(tmp_path):
    from exact_tiled_attention_attn_amd import _binding
    with pytest.raises(RuntimeError, match="not found"):
        _binding._lib, saved = None, _binding._lib
        try:
            _binding.load_library(str(tmp_path / "libattn.so"))
        finally:
            _binding._lib = saved


def test_size_limits_of_32_bit_slice_addressing():
    # The largest accepted head: rows 0..n-1 end just below 2^31 bytes.  With a
    # padded row stride, n times the stride passes 2^31 (the kernels' buffer
    # sizes are formed in 64 bits and clamped, so this stays valid).
    es, w = 2, 128
    stride = (1 << 20) + 8  # elements, 16-byte multiple
    p = problem(B=1, H=1, n=1024, d=w, v=w)
    for name in ("sq", "sk", "sv", "so"):
        arr = getattr(p, name)
        arr[0] = arr[1] = 1024 * stride
        arr[2] = stride
    assert 1024 * stride * es > (1 << 31) and 1023 * stride * es + w * es < (1 << 31)
    assert wsize(p, 0)[0] == 0 and wsize(p, 1)[0] == 0, err()
    p.n = 1025  # row 1024 would end past 2^31 - 1
    assert wsize(p, 0)[0] == 6 and "2 GiB" in err()
    # Atomic dQ path: one head's fp32 accumulator must stay within 2^31 - 1 bytes.
    p = problem(B=1, H=1, n=1 << 22, d=128, v=128)
    assert wsize(p, 0)[0] == 0
    assert wsize(p, 1)[0] == 6 and "accumulator" in err()
    assert call_bwd(p) == 6
    p.deterministic = 1
    st, need = wsize(p, 1)
    assert st == 0 and need > 0
    assert call_bwd(p) == 7  # validation passes; stops at the missing workspace, before any launch


def test_binding_refuses_host_tensors():
    import torch

    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU memory"):
        E.fwd(q, q, q, 0.125)
    with pytest.raises(ValueError, match="GPU memory"):
        E.bwd(q, q, q, q, q, torch.zeros((1, 1, 8)), 0.125)
