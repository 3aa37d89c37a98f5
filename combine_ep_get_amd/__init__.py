"""Python binding of ``libepget.so`` (MoE expert-parallel layout / dispatch /
combine on one MI355X, virtual EP ranks).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels.  Tensors are torch CUDA (HIP) tensors; calls are enqueued on
``torch.cuda.current_stream()``.  When the library is missing, every call
raises -- there is no fallback of any kind.

    lay = get_layout(topk_idx, num_experts, num_ranks, expert_alignment)
    recv_x, recv_scales, recv_src_idx, recv_w = dispatch(x, topk_weights, lay, use_fp8)
    y = combine(expert_out, lay, topk_weights)

Options (same kernels): ``topk_idx`` int32 or int64; ``dispatch(...,
x_scales=sf)`` for pre-quantised e4m3 input, ``zero_padding=True``,
``cumulative_stats=t``; ``cu_budget=n`` on dispatch and combine;
``ll_dispatch`` for decode batches (routing and payload in one launch).

The names follow DeepEP's (DeepEP book ch.1 "positioning and version
boundaries", sec. 1.1 and 1.4): num_tokens_per_rank, num_tokens_per_expert,
is_token_in_rank, expert_alignment, num_experts.
"""
import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_lib", "libepget.so")

EP_OK = 0
EP_LAYOUT_ERR_INDEX = 1

_lib = None


class Problem(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_topk", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("num_ranks", ctypes.c_int32), ("expert_alignment", ctypes.c_int32),
                ("use_fp8", ctypes.c_int32), ("topk_idx_bytes", ctypes.c_int32),
                ("cu_budget", ctypes.c_int32)]


EP_DISPATCH_ZERO_PADDING = 1


class DispatchArgs(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("x_scales", ctypes.c_void_p),
                ("topk_weights", ctypes.c_void_p), ("slot_of", ctypes.c_void_p),
                ("expert_slot_offset", ctypes.c_void_p), ("num_recv_per_expert", ctypes.c_void_p),
                ("recv_x", ctypes.c_void_p), ("recv_scales", ctypes.c_void_p),
                ("recv_src_idx", ctypes.c_void_p), ("recv_topk_weights", ctypes.c_void_p),
                ("recv_capacity", ctypes.c_int64), ("cumulative_recv_stats", ctypes.c_void_p),
                ("flags", ctypes.c_uint32)]


class EPError(RuntimeError):
    def __init__(self, fn, code):
        msg = lib().ep_status_str(code).decode()
        super().__init__(f"{fn}: {msg} (status {code})")
        self.code = code


class LLArgs(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("x_scales", ctypes.c_void_p), ("topk_weights", ctypes.c_void_p),
                ("recv_count", ctypes.c_void_p), ("slot_of", ctypes.c_void_p),
                ("flags", ctypes.c_void_p), ("recv_x", ctypes.c_void_p),
                ("recv_scales", ctypes.c_void_p), ("recv_src_idx", ctypes.c_void_p),
                ("recv_topk_weights", ctypes.c_void_p), ("cumulative_recv_stats", ctypes.c_void_p)]


EXPORTS = ("ep_recv_capacity", "ep_workspace_bytes", "ep_get_layout", "ep_dispatch",
           "ep_dispatch_ex", "ep_combine", "ep_layout_error", "ep_status_str", "ep_ll_capacity",
           "ep_ll_dispatch", "ep_ll_dispatch_ex", "ep_get_layout_noalloc")
EP_ERR_SCRATCH = 5
NOALLOC_SCRATCH_BYTES = 2 << 20
EP_LAYOUT_ERR_OVERFLOW = 2


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        _lib = load(LIB_PATH)
    return _lib


def use_library(path):
    """Route every later call to the build of the library at ``path`` (a
    build of the same sources with other compile-time launch parameters)."""
    global _lib
    _lib = load(path)
    return _lib


def load(path):
    """Open a build of libepget.so and declare its C signatures."""
    L = ctypes.CDLL(path)
    vp, i64, P = ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(Problem)
    L.ep_recv_capacity.restype = i64
    L.ep_recv_capacity.argtypes = [P]
    L.ep_workspace_bytes.restype = i64
    L.ep_workspace_bytes.argtypes = [P]
    L.ep_get_layout.restype = ctypes.c_int
    L.ep_get_layout.argtypes = [P] + [vp] * 9
    L.ep_get_layout_noalloc.restype = ctypes.c_int
    L.ep_get_layout_noalloc.argtypes = [P] + [vp] * 9
    L.ep_dispatch.restype = ctypes.c_int
    L.ep_dispatch.argtypes = [P] + [vp] * 9 + [i64, vp]
    L.ep_dispatch_ex.restype = ctypes.c_int
    L.ep_dispatch_ex.argtypes = [P, ctypes.POINTER(DispatchArgs), vp]
    L.ep_combine.restype = ctypes.c_int
    L.ep_combine.argtypes = [P, vp, vp, vp, vp, i64, vp]
    L.ep_layout_error.restype = ctypes.c_int
    L.ep_layout_error.argtypes = [vp, ctypes.POINTER(ctypes.c_int32), vp]
    L.ep_status_str.restype = ctypes.c_char_p
    L.ep_status_str.argtypes = [ctypes.c_int]
    L.ep_ll_capacity.restype = i64
    L.ep_ll_capacity.argtypes = [P, ctypes.c_int32]
    L.ep_ll_dispatch.restype = ctypes.c_int
    L.ep_ll_dispatch.argtypes = [P, ctypes.c_int32] + [vp] * 10 + [vp]
    L.ep_ll_dispatch_ex.restype = ctypes.c_int
    L.ep_ll_dispatch_ex.argtypes = [P, ctypes.c_int32, ctypes.POINTER(LLArgs), vp]
    return L


def problem(num_tokens, hidden, num_topk, num_experts, num_ranks, expert_alignment=1,
            use_fp8=False, topk_idx_bytes=4, cu_budget=0):
    return Problem(int(num_tokens), int(hidden), int(num_topk), int(num_experts),
                   int(num_ranks), int(expert_alignment), int(bool(use_fp8)),
                   int(topk_idx_bytes), int(cu_budget))


def _idx_bytes(topk_idx):
    import torch
    if topk_idx.dtype == torch.int32:
        return 4
    if topk_idx.dtype == torch.int64:
        return 8
    raise ValueError(f"topk_idx: need int32 or int64, got {topk_idx.dtype}")


def recv_capacity(num_tokens, num_topk, num_experts, num_ranks, expert_alignment=1):
    p = problem(num_tokens, 8, num_topk, num_experts, num_ranks, expert_alignment)
    v = lib().ep_recv_capacity(ctypes.byref(p))
    if v < 0:
        raise ValueError("invalid problem sizes")
    return int(v)


def workspace_bytes(num_tokens, num_topk, num_experts, num_ranks, expert_alignment=1):
    p = problem(num_tokens, 8, num_topk, num_experts, num_ranks, expert_alignment)
    v = lib().ep_workspace_bytes(ctypes.byref(p))
    if v < 0:
        raise ValueError("invalid problem sizes")
    return int(v)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, rc):
    if rc != EP_OK:
        raise EPError(fn, rc)


def _need(t, dtype, shape, name):
    import torch
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() \
            or t.device.type != "cuda":
        raise ValueError(f"{name}: need contiguous {dtype} {tuple(shape)} on the GPU, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    return t


@dataclass
class Layout:
    """Output of get_layout; ``slot_of`` (with the caller's topk_weights) is the
    handle that dispatch and combine consume."""
    num_tokens: int
    num_topk: int
    num_experts: int
    num_ranks: int
    expert_alignment: int
    capacity: int
    num_tokens_per_rank: object    # [R, R] int32
    num_tokens_per_expert: object  # [R, E] int32
    is_token_in_rank: object       # [N, R] uint8
    num_recv_per_expert: object    # [E] int32
    expert_slot_offset: object     # [E + 1] int32
    slot_of: object                # [N, K] int32
    workspace: object              # uint8, ep_workspace_bytes

    def problem(self, hidden=8, use_fp8=False):
        return problem(self.num_tokens, hidden, self.num_topk, self.num_experts,
                       self.num_ranks, self.expert_alignment, use_fp8)


def alloc_layout(num_tokens, num_topk, num_experts, num_ranks, expert_alignment=1,
                 device="cuda"):
    """Allocate (but do not compute) the layout outputs and workspace."""
    import torch
    N, K, E, R, A = num_tokens, num_topk, num_experts, num_ranks, expert_alignment
    cap = recv_capacity(N, K, E, R, A)
    ws = workspace_bytes(N, K, E, R, A)
    i32, u8 = torch.int32, torch.uint8
    return Layout(N, K, E, R, A, cap,
                  torch.empty((R, R), dtype=i32, device=device),
                  torch.empty((R, E), dtype=i32, device=device),
                  torch.empty((N, R), dtype=u8, device=device),
                  torch.empty((E,), dtype=i32, device=device),
                  torch.empty((E + 1,), dtype=i32, device=device),
                  torch.empty((N, K), dtype=i32, device=device),
                  torch.empty((max(ws, 256),), dtype=u8, device=device))


def get_layout(topk_idx, num_experts, num_ranks, expert_alignment=1, out=None):
    """Routing layout of ``topk_idx`` [N, K] int32 or int64 (see ep_get_layout)."""
    import torch
    N, K = topk_idx.shape
    if out is None:
        out = alloc_layout(N, K, num_experts, num_ranks, expert_alignment, topk_idx.device)
    if (out.num_experts, out.num_ranks, out.expert_alignment) != \
            (num_experts, num_ranks, expert_alignment):
        raise ValueError("get_layout: `out` was allocated for another problem")
    nb = _idx_bytes(topk_idx)
    _need(topk_idx, topk_idx.dtype, (out.num_tokens, out.num_topk), "topk_idx")
    p = out.problem()
    p.topk_idx_bytes = nb
    rc = lib().ep_get_layout(ctypes.byref(p), _ptr(topk_idx), _ptr(out.num_tokens_per_rank),
                             _ptr(out.num_tokens_per_expert), _ptr(out.is_token_in_rank),
                             _ptr(out.num_recv_per_expert), _ptr(out.expert_slot_offset),
                             _ptr(out.slot_of), _ptr(out.workspace), _stream())
    _check("ep_get_layout", rc)
    return out


def get_layout_noalloc(topk_idx, out, error_word=None):
    """ep_get_layout_noalloc: the layout of ``topk_idx`` into the preallocated
    ``out`` (from alloc_layout; its workspace is not used) with the library's
    static scratch as workspace; ``error_word`` ([1] int32 on the GPU) receives
    the error bits when given.  Nothing is allocated."""
    nb = _idx_bytes(topk_idx)
    _need(topk_idx, topk_idx.dtype, (out.num_tokens, out.num_topk), "topk_idx")
    p = out.problem()
    p.topk_idx_bytes = nb
    rc = lib().ep_get_layout_noalloc(ctypes.byref(p), _ptr(topk_idx),
                                     _ptr(out.num_tokens_per_rank),
                                     _ptr(out.num_tokens_per_expert), _ptr(out.is_token_in_rank),
                                     _ptr(out.num_recv_per_expert), _ptr(out.expert_slot_offset),
                                     _ptr(out.slot_of), _ptr(error_word), _stream())
    _check("ep_get_layout_noalloc", rc)
    return out


def alloc_recv(layout, hidden, use_fp8=False, device="cuda", capacity=None):
    import torch
    cap = layout.capacity if capacity is None else capacity
    if use_fp8:
        recv_x = torch.empty((cap, hidden), dtype=torch.float8_e4m3fn, device=device)
        scales = torch.empty((cap, hidden // 128), dtype=torch.float32, device=device)
    else:
        recv_x = torch.empty((cap, hidden), dtype=torch.bfloat16, device=device)
        scales = None
    return (recv_x, scales, torch.empty((cap,), dtype=torch.int32, device=device),
            torch.empty((cap,), dtype=torch.float32, device=device))


def dispatch(x, topk_weights, layout, use_fp8=False, out=None, with_meta=True,
             x_scales=None, zero_padding=False, cumulative_stats=None, cu_budget=0):
    """Scatter ``x`` [N, H] into expert-contiguous receive slots.

    Returns (recv_x, recv_scales, recv_src_idx, recv_topk_weights); recv_x is
    bf16 or float8_e4m3fn [cap, H]; recv_scales is [cap, H/128] fp32 or None.
    ``x`` is bf16, or, with ``x_scales`` [N, H/128] fp32 given, pre-quantised
    float8_e4m3fn codes that are copied unchanged (needs use_fp8).
    With ``with_meta=False`` the per-slot source/weight tags are skipped;
    ``zero_padding`` zeroes the padding rows of every expert region;
    ``cumulative_stats`` ([E] int64) gets the per-expert receive counts added.
    ``cu_budget`` > 0 keeps the kernel on at most that many CUs.
    """
    import torch
    N, H = x.shape
    if x_scales is not None:
        if not use_fp8:
            raise ValueError("dispatch: pre-quantised x needs use_fp8=True")
        _need(x, torch.float8_e4m3fn, (layout.num_tokens, H), "x")
        _need(x_scales, torch.float32, (layout.num_tokens, H // 128), "x_scales")
    else:
        _need(x, torch.bfloat16, (layout.num_tokens, H), "x")
    if cumulative_stats is not None:
        _need(cumulative_stats, torch.int64, (layout.num_experts,), "cumulative_stats")
    if out is None:
        out = alloc_recv(layout, H, use_fp8, x.device)
    recv_x, scales, src, rw = out
    cap = recv_x.shape[0]
    _need(recv_x, torch.float8_e4m3fn if use_fp8 else torch.bfloat16, (cap, H), "recv_x")
    if use_fp8:
        _need(scales, torch.float32, (cap, H // 128), "recv_scales")
    if with_meta:
        _need(src, torch.int32, (cap,), "recv_src_idx")
        _need(rw, torch.float32, (cap,), "recv_topk_weights")
        _need(topk_weights, torch.float32, (layout.num_tokens, layout.num_topk), "topk_weights")
    p = layout.problem(H, use_fp8)
    p.cu_budget = int(cu_budget)
    a = DispatchArgs()
    a.x = x.data_ptr()
    a.x_scales = None if x_scales is None else x_scales.data_ptr()
    a.topk_weights = topk_weights.data_ptr() if with_meta else None
    a.slot_of = layout.slot_of.data_ptr()
    a.expert_slot_offset = layout.expert_slot_offset.data_ptr()
    a.num_recv_per_expert = layout.num_recv_per_expert.data_ptr()
    a.recv_x = recv_x.data_ptr()
    a.recv_scales = scales.data_ptr() if use_fp8 else None
    a.recv_src_idx = src.data_ptr() if with_meta else None
    a.recv_topk_weights = rw.data_ptr() if with_meta else None
    a.recv_capacity = cap
    a.cumulative_recv_stats = None if cumulative_stats is None else cumulative_stats.data_ptr()
    a.flags = EP_DISPATCH_ZERO_PADDING if zero_padding else 0
    if x_scales is None and not zero_padding and cumulative_stats is None:
        rc = lib().ep_dispatch(ctypes.byref(p), _ptr(x), _ptr(topk_weights if with_meta else None),
                               _ptr(layout.slot_of), _ptr(layout.expert_slot_offset),
                               _ptr(layout.num_recv_per_expert), _ptr(recv_x),
                               _ptr(scales if use_fp8 else None),
                               _ptr(src if with_meta else None), _ptr(rw if with_meta else None),
                               cap, _stream())
        _check("ep_dispatch", rc)
    else:
        _check("ep_dispatch_ex", lib().ep_dispatch_ex(ctypes.byref(p), ctypes.byref(a),
                                                      _stream()))
    return recv_x, (scales if use_fp8 else None), src, rw


def combine(expert_out, layout, topk_weights, out=None, cu_budget=0):
    """Weighted top-k reduction of ``expert_out`` [cap, H] bf16 into token order;
    ``cu_budget`` > 0 keeps the kernel on at most that many CUs."""
    import torch
    cap, H = expert_out.shape
    _need(expert_out, torch.bfloat16, (cap, H), "expert_out")
    _need(topk_weights, torch.float32, (layout.num_tokens, layout.num_topk), "topk_weights")
    if out is None:
        out = torch.empty((layout.num_tokens, H), dtype=torch.bfloat16, device=expert_out.device)
    _need(out, torch.bfloat16, (layout.num_tokens, H), "y")
    p = layout.problem(H)
    p.cu_budget = int(cu_budget)
    rc = lib().ep_combine(ctypes.byref(p), _ptr(expert_out), _ptr(layout.slot_of),
                          _ptr(topk_weights), _ptr(out), cap, _stream())
    _check("ep_combine", rc)
    return out


def layout_error(layout):
    """Synchronous: error flags of the last get_layout into ``layout``."""
    v = ctypes.c_int32(0)
    _check("ep_layout_error", lib().ep_layout_error(_ptr(layout.workspace), ctypes.byref(v),
                                                    _stream()))
    return int(v.value)


# ------------------------------------------------------------ low latency
@dataclass
class LLLayout:
    """Output of ll_dispatch's routing half: recv_count [E, R] (rows used per
    (expert, source) sub-block of M rows), slot_of [N, K] (the handle for
    combine), flags [R] (per-source EP_LAYOUT_ERR_* bits)."""
    num_tokens: int
    num_topk: int
    num_experts: int
    num_ranks: int
    max_tokens_per_rank: int
    capacity: int
    recv_count: object
    slot_of: object
    flags: object
    expert_alignment: int = 1

    def problem(self, hidden=8, use_fp8=False):
        return problem(self.num_tokens, hidden, self.num_topk, self.num_experts,
                       self.num_ranks, 1, use_fp8)


def ll_capacity(num_tokens, num_topk, num_experts, num_ranks, max_tokens_per_rank):
    p = problem(num_tokens, 8, num_topk, num_experts, num_ranks, 1)
    v = lib().ep_ll_capacity(ctypes.byref(p), int(max_tokens_per_rank))
    if v < 0:
        raise ValueError("invalid problem sizes")
    return int(v)


def alloc_ll(num_tokens, num_topk, num_experts, num_ranks, max_tokens_per_rank, hidden,
             use_fp8=False, device="cuda"):
    """Allocate the low-latency layout and receive buffers."""
    import torch
    N, K, E, R, M = num_tokens, num_topk, num_experts, num_ranks, max_tokens_per_rank
    cap = ll_capacity(N, K, E, R, M)
    lay = LLLayout(N, K, E, R, M, cap,
                   torch.empty((E, R), dtype=torch.int32, device=device),
                   torch.empty((N, K), dtype=torch.int32, device=device),
                   torch.empty((R,), dtype=torch.int32, device=device))
    return lay, alloc_recv(lay, hidden, use_fp8, device)


def ll_dispatch(x, topk_idx, topk_weights, num_experts, num_ranks, max_tokens_per_rank,
                use_fp8=False, out=None, with_meta=True, x_scales=None, cumulative_stats=None):
    """Routing and payload in one launch (see ep_ll_dispatch / ep_ll_dispatch_ex).

    Returns (layout, (recv_x, recv_scales, recv_src_idx, recv_topk_weights)).
    ``out`` is a pair from alloc_ll for allocation-free calls.  ``x_scales``
    [N, H/128] fp32 makes ``x`` pre-quantised float8_e4m3fn codes (needs
    use_fp8); ``cumulative_stats`` ([E] int64) gets the rows each expert
    received added."""
    import torch
    N, H = x.shape
    K = topk_idx.shape[1]
    if out is None:
        out = alloc_ll(N, K, num_experts, num_ranks, max_tokens_per_rank, H, use_fp8, x.device)
    lay, recv = out
    if (lay.num_tokens, lay.num_topk, lay.num_experts, lay.num_ranks,
            lay.max_tokens_per_rank) != (N, K, num_experts, num_ranks, max_tokens_per_rank):
        raise ValueError("ll_dispatch: `out` was allocated for another problem")
    if x_scales is not None:
        if not use_fp8:
            raise ValueError("ll_dispatch: pre-quantised x needs use_fp8=True")
        _need(x, torch.float8_e4m3fn, (N, H), "x")
        _need(x_scales, torch.float32, (N, H // 128), "x_scales")
    else:
        _need(x, torch.bfloat16, (N, H), "x")
    if cumulative_stats is not None:
        _need(cumulative_stats, torch.int64, (num_experts,), "cumulative_stats")
    nb = _idx_bytes(topk_idx)
    _need(topk_idx, topk_idx.dtype, (N, K), "topk_idx")
    recv_x, scales, src, rw = recv
    _need(recv_x, torch.float8_e4m3fn if use_fp8 else torch.bfloat16, (lay.capacity, H), "recv_x")
    if use_fp8:
        _need(scales, torch.float32, (lay.capacity, H // 128), "recv_scales")
    if with_meta:
        _need(src, torch.int32, (lay.capacity,), "recv_src_idx")
        _need(rw, torch.float32, (lay.capacity,), "recv_topk_weights")
        _need(topk_weights, torch.float32, (N, K), "topk_weights")
    p = problem(N, H, K, num_experts, num_ranks, 1, use_fp8, nb)
    if x_scales is None and cumulative_stats is None:
        rc = lib().ep_ll_dispatch(ctypes.byref(p), int(max_tokens_per_rank), _ptr(topk_idx),
                                  _ptr(x), _ptr(topk_weights if with_meta else None),
                                  _ptr(lay.recv_count), _ptr(lay.slot_of), _ptr(lay.flags),
                                  _ptr(recv_x), _ptr(scales if use_fp8 else None),
                                  _ptr(src if with_meta else None),
                                  _ptr(rw if with_meta else None), _stream())
        _check("ep_ll_dispatch", rc)
    else:
        a = LLArgs()
        a.topk_idx = topk_idx.data_ptr()
        a.x = x.data_ptr()
        a.x_scales = None if x_scales is None else x_scales.data_ptr()
        a.topk_weights = topk_weights.data_ptr() if with_meta else None
        a.recv_count = lay.recv_count.data_ptr()
        a.slot_of = lay.slot_of.data_ptr()
        a.flags = lay.flags.data_ptr()
        a.recv_x = recv_x.data_ptr()
        a.recv_scales = scales.data_ptr() if use_fp8 else None
        a.recv_src_idx = src.data_ptr() if with_meta else None
        a.recv_topk_weights = rw.data_ptr() if with_meta else None
        a.cumulative_recv_stats = (None if cumulative_stats is None
                                   else cumulative_stats.data_ptr())
        _check("ep_ll_dispatch_ex", lib().ep_ll_dispatch_ex(ctypes.byref(p),
                                                            int(max_tokens_per_rank),
                                                            ctypes.byref(a), _stream()))
    return lay, (recv_x, scales if use_fp8 else None, src, rw)


def ep_dispatch_ex(p, args, stream=None):
    """The C call itself: ``p`` a Problem, ``args`` a DispatchArgs whose fields
    are device addresses (ints) and sizes, exactly as include/ep_get.h states;
    enqueued on ``stream`` (a raw hipStream_t as int, default: torch's current
    stream).  Raises EPError on a non-OK status."""
    st = _stream() if stream is None else ctypes.c_void_p(stream)
    _check("ep_dispatch_ex", lib().ep_dispatch_ex(ctypes.byref(p), ctypes.byref(args), st))


def ep_ll_dispatch_ex(p, max_tokens_per_rank, args, stream=None):
    """The C call itself: ``p`` a Problem, ``args`` an LLArgs of device
    addresses, as include/ep_get.h states; see ep_dispatch_ex."""
    st = _stream() if stream is None else ctypes.c_void_p(stream)
    _check("ep_ll_dispatch_ex", lib().ep_ll_dispatch_ex(ctypes.byref(p), int(max_tokens_per_rank),
                                                        ctypes.byref(args), st))


# The other C entry points under their own names, for callers who read
# include/ep_get.h: each is the function above that marshals that entry
# point's arguments from tensors.
ep_recv_capacity = recv_capacity
ep_workspace_bytes = workspace_bytes
ep_get_layout = get_layout
ep_get_layout_noalloc = get_layout_noalloc
ep_dispatch = dispatch
ep_combine = combine
ep_layout_error = layout_error
ep_ll_capacity = ll_capacity
ep_ll_dispatch = ll_dispatch
