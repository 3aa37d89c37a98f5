"""C-ABI checks that need no GPU: the library loads, exports every function
include/ep_get.h declares, and its host-only entry points (capacity,
workspace sizing, status strings, argument validation) behave as documented.
No call here reaches a kernel launch: each one is rejected by host validation
first or is host-only by contract.
"""
import ctypes
import os
import re

import pytest

import combine_ep_get_amd as ep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep_get.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ("ep_get_layout", "ep_dispatch", "ep_combine", "ep_recv_capacity",
               "ep_workspace_bytes", "ep_layout_error", "ep_status_str"):
        assert fn in names
    assert set(names) == set(ep.EXPORTS)


def test_library_exports_every_declared_symbol():
    assert os.path.exists(ep.LIB_PATH), "build the library first (__graft_entry__.build())"
    L = ctypes.CDLL(ep.LIB_PATH)
    for fn in declared_functions():
        assert hasattr(L, fn), fn
    out = os.popen(f"nm -D --defined-only {ep.LIB_PATH}").read()
    exported = set(re.findall(r"\bT (ep_[a-z_]+)\b", out))
    assert set(declared_functions()) <= exported


def test_capacity_and_workspace():
    # N*K + E*(A-1)
    assert ep.recv_capacity(4096, 8, 256, 8, 128) == 4096 * 8 + 256 * 127
    assert ep.recv_capacity(128, 2, 16, 4, 1) == 256
    assert ep.recv_capacity(0, 8, 256, 8, 128) == 256 * 127
    ws = ep.workspace_bytes(4096, 8, 256, 8, 128)
    assert ws > 0 and ws % 256 == 0
    assert ep.workspace_bytes(0, 8, 256, 8, 1) >= 256
    with pytest.raises(ValueError):
        ep.recv_capacity(10, 8, 256, 8, 1)        # N % R != 0
    with pytest.raises(ValueError):
        ep.recv_capacity(16, 8, 250, 8, 1)        # E % R != 0
    with pytest.raises(ValueError):
        ep.recv_capacity(16, 33, 256, 8, 1)       # K too large
    with pytest.raises(ValueError):
        ep.recv_capacity(16, 8, 2048, 8, 1)       # E too large
    with pytest.raises(ValueError):
        ep.recv_capacity(2 ** 28, 16, 256, 8, 1)  # bound beyond int32


def test_status_strings():
    L = ep.lib()
    for code in range(6):
        assert L.ep_status_str(code)
    assert b"unknown" in L.ep_status_str(99)
    assert b"scratch" in L.ep_status_str(ep.EP_ERR_SCRATCH)


def _p(**kw):
    base = dict(num_tokens=16, hidden=256, num_topk=2, num_experts=16, num_ranks=4,
                expert_alignment=1, use_fp8=False)
    base.update(kw)
    return ep.problem(**base)


BAD = [dict(num_tokens=-1), dict(num_topk=0), dict(num_topk=33), dict(num_experts=0),
       dict(num_experts=1025), dict(num_ranks=0), dict(num_ranks=32, num_experts=16),
       dict(num_experts=18), dict(num_tokens=18), dict(expert_alignment=0)]


@pytest.mark.parametrize("kw", BAD, ids=[str(b) for b in BAD])
def test_layout_rejects_bad_descriptors(kw):
    L = ep.lib()
    p = _p(**kw)
    fake = ctypes.c_void_p(256)   # never dereferenced: validation runs first
    rc = L.ep_get_layout(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, None)
    assert rc == 1


@pytest.mark.parametrize("kw", BAD, ids=[str(b) for b in BAD])
def test_noalloc_layout_rejects_bad_descriptors(kw):
    L = ep.lib()
    p = _p(**kw)
    fake = ctypes.c_void_p(256)   # never dereferenced: validation runs first
    rc = L.ep_get_layout_noalloc(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake,
                                 None)
    assert rc == 1


def test_noalloc_layout_missing_outputs_and_scratch_bound():
    L = ep.lib()
    fake = ctypes.c_void_p(256)
    p = _p()
    # outputs that must exist
    assert L.ep_get_layout_noalloc(ctypes.byref(p), fake, None, fake, fake, fake, fake, fake,
                                   None, None) == 1
    assert L.ep_get_layout_noalloc(ctypes.byref(p), None, fake, fake, fake, fake, fake, fake,
                                   None, None) == 1
    # the static scratch covers the largest workspace any valid descriptor needs
    worst = max(ep.workspace_bytes(n, k, 1024, r, 1)
                for r in (1, 8, 64, 256) for k in (1, 8, 32)
                for n in (r, 64 * r, 1024 * r, 65536 * r // 8) if n * k < 2 ** 31 - 1)
    assert 0 < worst <= ep.NOALLOC_SCRATCH_BYTES


def test_payload_rejects_bad_descriptors():
    L = ep.lib()
    fake = ctypes.c_void_p(256)
    for kw in (dict(hidden=0), dict(hidden=12), dict(hidden=200, use_fp8=True),
               dict(hidden=(1 << 24) + 8), dict(hidden=(1 << 24) + 128, use_fp8=True)):
        p = _p(**kw)
        assert L.ep_dispatch(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake,
                             fake, 10 ** 6, None) == 1
        assert L.ep_combine(ctypes.byref(p), fake, fake, fake, fake, 10 ** 6, None) == 1
    p = _p()
    # capacity below N*K + E*(A-1)
    assert L.ep_dispatch(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                         16 * 2 - 1, None) == 2
    # missing pointers
    assert L.ep_dispatch(ctypes.byref(p), None, fake, fake, fake, fake, fake, None, fake, fake,
                         10 ** 6, None) == 1
    assert L.ep_combine(ctypes.byref(p), fake, None, fake, fake, 10 ** 6, None) == 1
    # tokens but a zero-row expert_out: rejected (pairs without a slot read row 0)
    assert L.ep_combine(ctypes.byref(p), fake, fake, fake, fake, 0, None) == 1
    # fp8 needs a scale buffer
    p8 = _p(use_fp8=True)
    assert L.ep_dispatch(ctypes.byref(p8), fake, fake, fake, fake, fake, fake, None, fake, fake,
                         10 ** 6, None) == 1
    # workspace must be 256-byte aligned
    assert L.ep_get_layout(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake,
                           ctypes.c_void_p(260), None) == 1
    assert L.ep_layout_error(None, None, None) == 1


def test_ll_capacity_and_validation():
    L = ep.lib()
    assert ep.ll_capacity(1024, 8, 256, 8, 128) == 256 * 8 * 128
    with pytest.raises(ValueError):
        ep.ll_capacity(1024, 8, 256, 8, 0)                # M >= 1
    with pytest.raises(ValueError):
        ep.ll_capacity(1024, 8, 1024, 256, 1 << 20)       # E*R*M beyond int32
    fake = ctypes.c_void_p(256)
    args = [fake] * 10 + [None]
    # (N/R)*K above 4096 pairs per source
    p = _p(num_tokens=8 * 1024, num_topk=8, num_experts=16, num_ranks=8)
    assert L.ep_ll_dispatch(ctypes.byref(p), 1024, *args) == 1
    # fp8 needs hidden % 128 and a scale buffer
    p = _p(hidden=136, use_fp8=True)
    assert L.ep_ll_dispatch(ctypes.byref(p), 8, *args) == 1
    p = _p(use_fp8=True)
    a = list(args)
    a[7] = None
    assert L.ep_ll_dispatch(ctypes.byref(p), 8, *a) == 1


def test_index_width_validation():
    for nb, ok in ((0, True), (4, True), (8, True), (2, False), (16, False)):
        p = _p(topk_idx_bytes=nb)
        assert (ep.lib().ep_recv_capacity(ctypes.byref(p)) >= 0) == ok


def test_dispatch_ex_validation():
    L = ep.lib()
    fake = ctypes.c_void_p(256).value

    def args(**kw):
        a = ep.DispatchArgs()
        for f in ("x", "topk_weights", "slot_of", "expert_slot_offset", "num_recv_per_expert",
                  "recv_x", "recv_src_idx", "recv_topk_weights"):
            setattr(a, f, fake)
        a.recv_capacity = 10 ** 6
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    p = _p()
    p8 = _p(use_fp8=True)
    assert L.ep_dispatch_ex(ctypes.byref(p), None, None) == 1
    # unknown flag bits
    assert L.ep_dispatch_ex(ctypes.byref(p), ctypes.byref(args(flags=2)), None) == 1
    # capacity below the bound
    assert L.ep_dispatch_ex(ctypes.byref(p), ctypes.byref(args(recv_capacity=31)), None) == 2
    # pre-quantised input needs use_fp8
    assert L.ep_dispatch_ex(ctypes.byref(p), ctypes.byref(args(x_scales=fake)), None) == 1
    # fp8 needs a scale buffer, also for zero padding
    assert L.ep_dispatch_ex(ctypes.byref(p8), ctypes.byref(args(x_scales=fake)), None) == 1
    # statistics and zero padding need the counts and offsets
    assert L.ep_dispatch_ex(ctypes.byref(p), ctypes.byref(
        args(recv_src_idx=None, recv_topk_weights=None, cumulative_recv_stats=fake,
             num_recv_per_expert=None)), None) == 1
    pa = _p(expert_alignment=4)
    assert L.ep_dispatch_ex(ctypes.byref(pa), ctypes.byref(
        args(recv_src_idx=None, recv_topk_weights=None, flags=1,
             expert_slot_offset=None)), None) == 1


def test_cu_budget_validation():
    L = ep.lib()
    p = _p(cu_budget=-1)
    assert ep.lib().ep_recv_capacity(ctypes.byref(p)) == -1
    assert L.ep_combine(ctypes.byref(p), None, None, None, None, 0, None) == 1
    p = _p(cu_budget=4)
    assert ep.lib().ep_recv_capacity(ctypes.byref(p)) == 32


def test_ll_dispatch_ex_validation():
    L = ep.lib()
    fake = ctypes.c_void_p(256).value
    p = _p()
    assert L.ep_ll_dispatch_ex(ctypes.byref(p), 8, None, None) == 1
    a = ep.LLArgs()
    for f in ("topk_idx", "x", "topk_weights", "recv_count", "slot_of", "flags", "recv_x",
              "recv_src_idx", "recv_topk_weights"):
        setattr(a, f, fake)
    a.x_scales = fake                  # pre-quantised input without use_fp8
    assert L.ep_ll_dispatch_ex(ctypes.byref(p), 8, ctypes.byref(a), None) == 1
    p8 = _p(use_fp8=True)              # fp8 without a scale buffer
    assert L.ep_ll_dispatch_ex(ctypes.byref(p8), 8, ctypes.byref(a), None) == 1
    a.x_scales = None
    a.recv_count = None                # the mask is required
    assert L.ep_ll_dispatch_ex(ctypes.byref(p), 8, ctypes.byref(a), None) == 1


def test_binding_offers_every_entry_point_by_its_c_name():
    for fn in declared_functions():
        if fn == "ep_status_str":
            continue   # raised as the message of EPError
        assert callable(getattr(ep, fn, None)), fn


def test_c_shaped_wrappers_pass_the_structs_through():
    """ep_dispatch_ex / ep_ll_dispatch_ex in Python are the C calls with their
    own argument structs; host validation errors come back as EPError."""
    p = _p()
    a = ep.DispatchArgs()
    a.recv_capacity = 10 ** 6          # no payload pointers: rejected before any launch
    with pytest.raises(ep.EPError) as ex:
        ep.ep_dispatch_ex(p, a, stream=0)
    assert ex.value.code == 1
    a.recv_capacity = 1                # below N*K + E*(A-1)
    with pytest.raises(ep.EPError) as ex:
        ep.ep_dispatch_ex(p, a, stream=0)
    assert ex.value.code == 2
    with pytest.raises(ep.EPError) as ex:
        ep.ep_ll_dispatch_ex(p, 8, ep.LLArgs(), stream=0)
    assert ex.value.code == 1
