"""numpy front-end of the C oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The product path never imports it.

bf16 arrays are carried as ``uint16`` bit patterns, e4m3 arrays as ``uint8``.
Every function here only marshals arguments; the arithmetic is in ``oracle.c``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def lib():
    """Load liboracle.so, building it first if it does not exist yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = load(_build.LIB)
    return _lib


def load(path):
    """Open an oracle library at ``path`` and declare its signatures."""
    L = ctypes.CDLL(path)
    L.oracle_bf16_to_f32.restype = ctypes.c_float
    L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_f32_to_bf16.restype = ctypes.c_uint16
    L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    L.oracle_e4m3_to_f32.restype = ctypes.c_float
    L.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    L.oracle_f32_to_e4m3.restype = ctypes.c_uint8
    L.oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
    L.oracle_bf16_to_f32_n.argtypes = [_u16p, _f32p, _i64]
    L.oracle_f32_to_bf16_n.argtypes = [_f32p, _u16p, _i64]
    L.oracle_e4m3_to_f32_n.argtypes = [_u8p, _f32p, _i64]
    L.oracle_f32_to_e4m3_n.argtypes = [_f32p, _u8p, _i64]
    L.oracle_capacity.restype = _i64
    L.oracle_capacity.argtypes = [_i32, _i32, _i32, _i32]
    L.oracle_layout.restype = ctypes.c_int
    L.oracle_layout.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32p,
                                _i32p, _i32p, _u8p, _i32p, _i32p, _i32p]
    L.oracle_recv_meta.argtypes = [_i32, _i32, _i64, _i32p, _f32p, _i32p, _f32p]
    L.oracle_dispatch_quantized.argtypes = [_i32, _i32, _i32, _u8p, _f32p, _i32p, _u8p, _f32p]
    L.oracle_zero_padding.argtypes = [_i32, _i32, _i32, _i32p, _i32p, _u8p, _vp]
    L.oracle_accumulate_stats.argtypes = [_i32, _i32p, np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")]
    L.oracle_ll_layout.restype = ctypes.c_int
    L.oracle_ll_layout.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32p, _i32p, _i32p, _i32p]
    L.oracle_dispatch_bf16.argtypes = [_i32, _i32, _i32, _u16p, _i32p, _u16p]
    L.oracle_quantize_row.argtypes = [_i32, _u16p, _u8p, _f32p]
    L.oracle_dispatch_fp8.argtypes = [_i32, _i32, _i32, _u16p, _i32p, _u8p, _f32p]
    L.oracle_combine.argtypes = [_i32, _i32, _i32, _vp, _i32, _i32p, _f32p,
                                 _vp, _vp, _vp, _i32]
    L.oracle_dispatch_bf16_mt.restype = ctypes.c_int
    L.oracle_dispatch_bf16_mt.argtypes = [_i32, _i32, _i32, _u16p, _i32p, _u16p, ctypes.c_int]
    L.oracle_dispatch_fp8_mt.restype = ctypes.c_int
    L.oracle_dispatch_fp8_mt.argtypes = [_i32, _i32, _i32, _u16p, _i32p, _u8p, _f32p,
                                         ctypes.c_int]
    L.oracle_combine_mt.restype = ctypes.c_int
    L.oracle_combine_mt.argtypes = [_i32, _i32, _i32, _vp, _i32, _i32p, _f32p, _vp, _vp,
                                    ctypes.c_int]
    return L


class swapped:
    """Context manager: route every call of this module to another build of
    the oracle (used by the test that plants mistakes in copies of oracle.c)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = load(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---------------------------------------------------------------- formats
def bf16_to_f32(bits):
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float32)
    lib().oracle_bf16_to_f32_n(bits.reshape(-1), out.reshape(-1), bits.size)
    return out


def f32_to_bf16(vals):
    vals = _c(vals, np.float32)
    out = np.empty(vals.shape, np.uint16)
    lib().oracle_f32_to_bf16_n(vals.reshape(-1), out.reshape(-1), vals.size)
    return out


def e4m3_to_f32(codes):
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float32)
    lib().oracle_e4m3_to_f32_n(codes.reshape(-1), out.reshape(-1), codes.size)
    return out


def f32_to_e4m3(vals):
    vals = _c(vals, np.float32)
    out = np.empty(vals.shape, np.uint8)
    lib().oracle_f32_to_e4m3_n(vals.reshape(-1), out.reshape(-1), vals.size)
    return out


# ---------------------------------------------------------------- layout
def capacity(N, K, E, A):
    return int(lib().oracle_capacity(N, K, E, A))


def layout(topk_idx, num_experts, num_ranks, expert_alignment=1):
    """Return a dict with the six layout outputs and the error flags."""
    topk_idx = _c(topk_idx, np.int32)
    N, K = topk_idx.shape
    E, R, A = int(num_experts), int(num_ranks), int(expert_alignment)
    out = dict(
        num_tokens_per_rank=np.zeros((R, R), np.int32),
        num_tokens_per_expert=np.zeros((R, E), np.int32),
        is_token_in_rank=np.zeros((N, R), np.uint8),
        expert_slot_offset=np.zeros(E + 1, np.int32),
        num_recv_per_expert=np.zeros(E, np.int32),
        slot_of=np.zeros((N, K), np.int32),
    )
    rc = lib().oracle_layout(N, K, E, R, A, topk_idx.reshape(-1) if N else np.zeros(1, np.int32),
                             out["num_tokens_per_rank"].reshape(-1),
                             out["num_tokens_per_expert"].reshape(-1),
                             out["is_token_in_rank"].reshape(-1) if N else np.zeros(1, np.uint8),
                             out["expert_slot_offset"],
                             out["num_recv_per_expert"],
                             out["slot_of"].reshape(-1) if N else np.zeros(1, np.int32))
    if rc < 0:
        raise ValueError("oracle_layout: invalid sizes")
    out["error_flags"] = rc
    return out


def ll_layout(topk_idx, num_experts, num_ranks, max_tokens_per_rank):
    """Low-latency layout: dict(recv_count [E, R], slot_of [N, K], flags [R])."""
    topk_idx = _c(topk_idx, np.int32)
    N, K = topk_idx.shape
    E, R, M = int(num_experts), int(num_ranks), int(max_tokens_per_rank)
    out = dict(recv_count=np.zeros((E, R), np.int32), slot_of=np.zeros((N, K), np.int32),
               flags=np.zeros(R, np.int32))
    rc = lib().oracle_ll_layout(N, K, E, R, M, topk_idx.reshape(-1) if N else np.zeros(1, np.int32),
                                out["recv_count"].reshape(-1),
                                out["slot_of"].reshape(-1) if N else np.zeros(1, np.int32),
                                out["flags"])
    if rc < 0:
        raise ValueError("oracle_ll_layout: invalid sizes")
    out["error_flags"] = rc
    return out


def recv_meta(slot_of, topk_weights, cap):
    slot_of = _c(slot_of, np.int32)
    w = _c(topk_weights, np.float32)
    N, K = slot_of.shape
    src = np.empty(cap, np.int32)
    rw = np.empty(cap, np.float32)
    if cap == 0:
        return src, rw
    lib().oracle_recv_meta(N, K, cap, slot_of.reshape(-1) if N else np.zeros(1, np.int32),
                           w.reshape(-1) if N else np.zeros(1, np.float32), src, rw)
    return src, rw


# ---------------------------------------------------------------- dispatch
def dispatch_bf16(x_bits, slot_of, cap, fill=0, threads=1):
    """recv_x[cap, H] (uint16 bits); rows no pair maps to keep ``fill``.
    ``threads`` > 1 runs the threaded driver (token ranges in parallel)."""
    x_bits = _c(x_bits, np.uint16)
    slot_of = _c(slot_of, np.int32)
    N, H = x_bits.shape
    K = slot_of.shape[1]
    recv = np.full((cap, H), fill, np.uint16)
    if N and cap:
        if threads > 1:
            if lib().oracle_dispatch_bf16_mt(N, K, H, x_bits.reshape(-1), slot_of.reshape(-1),
                                             recv.reshape(-1), int(threads)) != 0:
                raise RuntimeError("oracle_dispatch_bf16_mt: could not start threads")
        else:
            lib().oracle_dispatch_bf16(N, K, H, x_bits.reshape(-1), slot_of.reshape(-1),
                                       recv.reshape(-1))
    return recv


def quantize_rows(x_bits):
    """Per-token FP8 quantisation: (codes [N, H] uint8, scales [N, H/128] f32)."""
    x_bits = _c(x_bits, np.uint16)
    N, H = x_bits.shape
    q = np.zeros((N, H), np.uint8)
    sc = np.zeros((N, H // 128), np.float32)
    for t in range(N):
        lib().oracle_quantize_row(H, x_bits[t], q[t], sc[t])
    return q, sc


def dispatch_fp8(x_bits, slot_of, cap, threads=1):
    """(codes [cap, H] uint8, scales [cap, H/128] f32); rows no pair maps to
    stay zero.  ``threads`` > 1 runs the threaded driver."""
    x_bits = _c(x_bits, np.uint16)
    slot_of = _c(slot_of, np.int32)
    N, H = x_bits.shape
    K = slot_of.shape[1]
    q = np.zeros((cap, H), np.uint8)
    sc = np.zeros((cap, H // 128), np.float32)
    if N and cap:
        if threads > 1:
            if lib().oracle_dispatch_fp8_mt(N, K, H, x_bits.reshape(-1), slot_of.reshape(-1),
                                            q.reshape(-1), sc.reshape(-1), int(threads)) != 0:
                raise RuntimeError("oracle_dispatch_fp8_mt: could not start threads")
        else:
            lib().oracle_dispatch_fp8(N, K, H, x_bits.reshape(-1), slot_of.reshape(-1),
                                      q.reshape(-1), sc.reshape(-1))
    return q, sc


def dispatch_quantized(codes, scales, slot_of, cap):
    """Copy given e4m3 codes [N, H] and scales [N, H/128] to every slot."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    slot_of = _c(slot_of, np.int32)
    N, H = codes.shape
    K = slot_of.shape[1]
    q = np.zeros((cap, H), np.uint8)
    sc = np.zeros((cap, H // 128), np.float32)
    if N and cap:
        lib().oracle_dispatch_quantized(N, K, H, codes.reshape(-1), scales.reshape(-1),
                                        slot_of.reshape(-1), q.reshape(-1), sc.reshape(-1))
    return q, sc


def zero_padding(recv_x, recv_scales, expert_slot_offset, num_recv_per_expert):
    """In place: zero the padding rows (and scale rows) of every expert region."""
    assert recv_x.flags["C_CONTIGUOUS"]
    E = int(num_recv_per_expert.size)
    row_bytes = recv_x.shape[1] * recv_x.itemsize
    raw = recv_x.reshape(-1).view(np.uint8)
    G = 0 if recv_scales is None else recv_scales.shape[1]
    lib().oracle_zero_padding(E, row_bytes, G, _c(expert_slot_offset, np.int32),
                              _c(num_recv_per_expert, np.int32), raw,
                              None if recv_scales is None else recv_scales.ctypes.data)


def accumulate_stats(count, stats):
    """In place: stats[e] += count[e] (stats int64)."""
    lib().oracle_accumulate_stats(int(count.size), _c(count, np.int32), stats)


# ---------------------------------------------------------------- combine
def combine(expert_out, slot_of, topk_weights, tokens=None, threads=1):
    """Return (y bf16 bits, acc float32) for all tokens or for ``tokens``.

    ``expert_out`` is either uint16 (bf16 bits) or float32, shape [cap, H].
    ``threads`` > 1 (all tokens only) runs the threaded driver.
    """
    slot_of = _c(slot_of, np.int32)
    w = _c(topk_weights, np.float32)
    N, K = slot_of.shape
    if expert_out.dtype == np.float32:
        eo, is_f32 = _c(expert_out, np.float32), 1
    else:
        eo, is_f32 = _c(expert_out, np.uint16), 0
    H = eo.shape[1]
    if tokens is None:
        tok_arr, rows = None, N
    else:
        tok_arr = _c(tokens, np.int32)
        rows = tok_arr.size
    y = np.zeros((rows, H), np.uint16)
    acc = np.zeros((rows, H), np.float32)
    if rows and H:
        if threads > 1 and tok_arr is None:
            if lib().oracle_combine_mt(N, K, H, eo.ctypes.data, is_f32, slot_of.reshape(-1),
                                       w.reshape(-1), y.ctypes.data, acc.ctypes.data,
                                       int(threads)) != 0:
                raise RuntimeError("oracle_combine_mt: could not start threads")
        else:
            lib().oracle_combine(N, K, H, eo.ctypes.data, is_f32, slot_of.reshape(-1),
                                 w.reshape(-1), y.ctypes.data, acc.ctypes.data,
                                 None if tok_arr is None else tok_arr.ctypes.data, rows)
    return y, acc
