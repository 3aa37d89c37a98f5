"""GPU parity of the dispatch variants (DeepEP book ch.1 sec. 1.1: int64
routing indices, x as a pair of FP8 codes and scales,
cumulative_local_expert_recv_stats, do_zero_padding, a reused handle) against
the CPU oracle, through the C ABI.  Integer and byte outputs are bit-exact;
combine is held to the same bar as the main parity tests.
"""
import numpy as np
import pytest
import torch

import combine_ep_get_amd as ep
import oracle
from combine_ep_get_amd import workloads as wl

from .gpu_util import check_combine, check_layout, dev_bf16, host_u16, host_u8, say

pytestmark = pytest.mark.gpu

SMALL = [wl.custom(N=60, H=384, E=12, K=3, R=3, A=16, name="ragged"),
         wl.custom(N=256, H=1024, E=32, K=4, R=4, A=32, name="aligned32")]


def _dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ------------------------------------------------------------ int64 indices
@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_int64_layout_parity(cid):
    w = wl.CONFIGS[cid]
    inp = wl.make_inputs(w, 0)
    say(f"int64 layout parity {w.desc}")
    idx = torch.from_numpy(inp["topk_idx"].astype(np.int64)).cuda()
    lay = ep.get_layout(idx, w.E, w.R, w.A)
    check_layout(lay, oracle.layout(inp["topk_idx"], w.E, w.R, w.A))


@pytest.mark.parametrize("N", [64, 4096])
def test_int64_out_of_int32_range_is_flagged(N):
    """Values that only a wrong truncation would map into [0, E) must be
    skipped and flagged; the expected layout is the oracle's on the same
    entries replaced by E (out of range in int32)."""
    w = wl.custom(N=N, H=128, E=32, K=4, R=4, A=8, name="int64edge")
    inp = wl.make_inputs(w, 1)
    say(f"int64 range edge N={N}")
    idx64 = inp["topk_idx"].astype(np.int64)
    idx32 = inp["topk_idx"].copy()
    rng = np.random.default_rng(5)
    pos = rng.choice(idx64.size, size=max(4, idx64.size // 50), replace=False)
    bad = np.array([2 ** 32 + 3, -(2 ** 40), 2 ** 31, -(2 ** 31) - 1], np.int64)
    idx64.reshape(-1)[pos] = bad[np.arange(pos.size) % bad.size]
    idx32.reshape(-1)[pos] = w.E
    lay = ep.get_layout(torch.from_numpy(idx64).cuda(), w.E, w.R, w.A)
    ref = oracle.layout(idx32, w.E, w.R, w.A)
    assert ref["error_flags"] == ep.EP_LAYOUT_ERR_INDEX
    check_layout(lay, ref)


def test_int64_low_latency_parity():
    w = wl.CONFIGS[2]
    inp = wl.make_inputs(w, 0)
    M = 128
    say(f"int64 low-latency parity {w.desc} M={M}")
    x = dev_bf16(inp["x"])
    wts = torch.from_numpy(inp["topk_weights"]).cuda()
    idx = torch.from_numpy(inp["topk_idx"].astype(np.int64)).cuda()
    lay, (recv_x, _, src, _) = ep.ll_dispatch(x, idx, wts, w.E, w.R, M)
    torch.cuda.synchronize()
    ref = oracle.ll_layout(inp["topk_idx"], w.E, w.R, M)
    np.testing.assert_array_equal(lay.slot_of.cpu().numpy(), ref["slot_of"])
    np.testing.assert_array_equal(lay.recv_count.cpu().numpy(), ref["recv_count"])
    np.testing.assert_array_equal(lay.flags.cpu().numpy(), ref["flags"])
    t, k = np.nonzero(ref["slot_of"] >= 0)
    s = torch.from_numpy(ref["slot_of"][t, k].astype(np.int64)).cuda()
    np.testing.assert_array_equal(host_u16(recv_x.index_select(0, s)), inp["x"][t])


# ------------------------------------------------------------ pre-quantised x
def _prequant_case(w, seed):
    rng = np.random.default_rng(300 + seed)
    inp = wl.make_inputs(w, seed)
    codes = rng.integers(0, 256, size=(w.N, w.H), dtype=np.uint8)   # NaN codes included
    scales = rng.standard_normal((w.N, w.H // 128)).astype(np.float32)
    return inp, codes, scales


@pytest.mark.parametrize("w", SMALL + [wl.CONFIGS[4]], ids=lambda w: w.name)
def test_prequantized_dispatch_parity(w):
    inp, codes, scales = _prequant_case(w, 0)
    say(f"pre-quantised dispatch {w.desc}")
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    lay = ep.get_layout(idx, w.E, w.R, w.A)
    ref = oracle.layout(inp["topk_idx"], w.E, w.R, w.A)
    cap = lay.capacity
    xq = _dev_u8(codes).view(torch.float8_e4m3fn)
    xs = torch.from_numpy(scales).cuda()
    wts = torch.from_numpy(inp["topk_weights"]).cuda()
    out = ep.alloc_recv(lay, w.H, True)
    out[0].view(torch.uint8).fill_(0x5A)
    out[1].fill_(-3.0)
    recv_x, sc, src, rw = ep.dispatch(xq, wts, lay, True, out=out, x_scales=xs)
    torch.cuda.synchronize()
    ref_src, ref_w = oracle.recv_meta(ref["slot_of"], inp["topk_weights"], cap)
    np.testing.assert_array_equal(src.cpu().numpy(), ref_src)
    np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), ref_w.view(np.uint32))
    # every valid slot against the oracle's pass-through of the same codes
    t, k = np.nonzero(ref["slot_of"] >= 0)
    slots = ref["slot_of"][t, k]
    st = torch.from_numpy(slots.astype(np.int64)).cuda()
    got_q = host_u8(recv_x.view(torch.uint8).index_select(0, st))
    got_s = sc.index_select(0, st).cpu().numpy()
    np.testing.assert_array_equal(got_q, codes[t])
    np.testing.assert_array_equal(got_s.view(np.uint32), scales[t].view(np.uint32))
    if cap * w.H <= 64 << 20:
        q_ref, s_ref = oracle.dispatch_quantized(codes, scales, ref["slot_of"], cap)
        invalid = ref_src < 0
        q_ref[invalid] = 0x5A
        s_ref[invalid] = -3.0
        np.testing.assert_array_equal(host_u8(recv_x.view(torch.uint8)), q_ref)
        np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    else:
        pad = torch.from_numpy(np.nonzero(ref_src < 0)[0]).cuda()
        assert bool((recv_x.view(torch.uint8).index_select(0, pad) == 0x5A).all())
    say(f"  {slots.size} valid slots compared")


def test_prequantized_equals_fused_on_gpu():
    """Quantising with the fused path and passing the oracle's quantisation
    through give the same bytes."""
    w = wl.custom(N=128, H=2048, E=16, K=4, R=4, A=4, fp8=True, name="fp8eq")
    inp = wl.make_inputs(w, 2)
    say("pre-quantised vs fused e4m3")
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    lay = ep.get_layout(idx, w.E, w.R, w.A)
    wts = torch.from_numpy(inp["topk_weights"]).cuda()
    a = ep.dispatch(dev_bf16(inp["x"]), wts, lay, True)
    codes, scales = oracle.quantize_rows(inp["x"])
    b = ep.dispatch(_dev_u8(codes).view(torch.float8_e4m3fn), wts, lay, True,
                    x_scales=torch.from_numpy(scales).cuda())
    torch.cuda.synchronize()
    valid = a[2] >= 0
    assert torch.equal(a[0].view(torch.uint8)[valid], b[0].view(torch.uint8)[valid])
    assert torch.equal(a[1][valid].view(torch.int32), b[1][valid].view(torch.int32))


# ------------------------------------------------------------ zero padding
def _padding_mask(ref, cap):
    off = ref["expert_slot_offset"].astype(np.int64)
    cnt = ref["num_recv_per_expert"].astype(np.int64)
    m = np.zeros(cap, bool)
    for e in range(cnt.size):
        m[off[e] + cnt[e]:off[e + 1]] = True
    return m


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("w", SMALL + [wl.CONFIGS[3]], ids=lambda w: w.name)
def test_zero_padding_parity(w, fp8):
    inp = wl.make_inputs(w, 0)
    say(f"zero padding {w.name} fp8={fp8}")
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    lay = ep.get_layout(idx, w.E, w.R, w.A)
    ref = oracle.layout(inp["topk_idx"], w.E, w.R, w.A)
    cap = lay.capacity
    wts = torch.from_numpy(inp["topk_weights"]).cuda()
    out = ep.alloc_recv(lay, w.H, fp8)
    out[0].view(torch.uint8).fill_(0x7E)
    if fp8:
        out[1].fill_(2.5)
    recv_x, sc, src, _ = ep.dispatch(dev_bf16(inp["x"]), wts, lay, fp8, out=out,
                                     zero_padding=True)
    torch.cuda.synchronize()
    pad = _padding_mask(ref, cap)
    used = int(ref["expert_slot_offset"][-1])
    ref_src, _ = oracle.recv_meta(ref["slot_of"], inp["topk_weights"], cap)
    np.testing.assert_array_equal(src.cpu().numpy(), ref_src)
    raw = recv_x.view(torch.uint8)
    pad_t = torch.from_numpy(np.nonzero(pad)[0]).cuda()
    tail_t = torch.arange(used, cap, device="cuda")
    assert int(pad.sum()) == used - int((ref["slot_of"] >= 0).sum())
    assert not bool(raw.index_select(0, pad_t).any())
    assert bool((raw.index_select(0, tail_t) == 0x7E).all())
    if fp8:
        assert not bool(sc.index_select(0, pad_t).any())
        assert bool((sc.index_select(0, tail_t) == 2.5).all())
    # valid rows: the ordinary dispatch result (sampled at the full size)
    t, k = np.nonzero(ref["slot_of"] >= 0)
    if t.size > 8192:
        pick = np.random.default_rng(1).choice(t.size, 8192, replace=False)
        t, k = t[pick], k[pick]
    st = torch.from_numpy(ref["slot_of"][t, k].astype(np.int64)).cuda()
    if fp8:
        q, s = oracle.quantize_rows(inp["x"][np.unique(t)])
        row = {tt: i for i, tt in enumerate(np.unique(t))}
        ti = np.array([row[tt] for tt in t])
        np.testing.assert_array_equal(host_u8(raw.index_select(0, st)), q[ti])
        np.testing.assert_array_equal(sc.index_select(0, st).cpu().numpy().view(np.uint32),
                                      s[ti].view(np.uint32))
    else:
        np.testing.assert_array_equal(host_u16(recv_x.index_select(0, st)), inp["x"][t])
    say(f"  {int(pad.sum())} padding rows zeroed, {cap - used} tail rows untouched")


# ------------------------------------------------------------ running statistics
@pytest.mark.parametrize("cid", [1, 3])
def test_cumulative_stats(cid):
    w = wl.CONFIGS[cid]
    inp = wl.make_inputs(w, 0)
    say(f"cumulative stats {w.desc}")
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    lay = ep.get_layout(idx, w.E, w.R, w.A)
    ref = oracle.layout(inp["topk_idx"], w.E, w.R, w.A)
    start = torch.arange(w.E, dtype=torch.int64, device="cuda") * (1 << 33) - 7
    stats = start.clone()
    x = dev_bf16(inp["x"])
    wts = torch.from_numpy(inp["topk_weights"]).cuda()
    ep.dispatch(x, wts, lay, w.fp8, cumulative_stats=stats)
    ep.dispatch(x, wts, lay, w.fp8, with_meta=False, cumulative_stats=stats)
    torch.cuda.synchronize()
    want = start.cpu().numpy().copy()
    oracle.accumulate_stats(ref["num_recv_per_expert"], want)
    oracle.accumulate_stats(ref["num_recv_per_expert"], want)
    np.testing.assert_array_equal(stats.cpu().numpy(), want)


# ------------------------------------------------------------ handle reuse
@pytest.mark.parametrize("cid", [2, 3])
def test_handle_reuse(cid):
    """One layout, then two rounds of dispatch -> identity experts -> combine
    with new token rows; the handle is unchanged and both rounds match."""
    w = wl.CONFIGS[cid]
    inp = wl.make_inputs(w, 0)
    say(f"handle reuse {w.desc}")
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    lay = ep.get_layout(idx, w.E, w.R, w.A)
    ref = oracle.layout(inp["topk_idx"], w.E, w.R, w.A)
    handle = [t.clone() for t in (lay.slot_of, lay.expert_slot_offset, lay.num_recv_per_expert)]
    wts = torch.from_numpy(inp["topk_weights"]).cuda()
    recv = ep.alloc_recv(lay, w.H)
    y = torch.empty((w.N, w.H), dtype=torch.bfloat16, device="cuda")
    for seed in (5, 6):
        x_bits = wl.make_inputs(w, seed)["x"]
        recv_x, _, _, _ = ep.dispatch(dev_bf16(x_bits), wts, lay, out=recv)
        ep.combine(recv_x, lay, wts, out=y)
        torch.cuda.synchronize()
        tok = np.arange(w.N) if w.N <= 1024 else np.random.default_rng(seed).choice(w.N, 512,
                                                                                   replace=False)
        recv_ref = np.zeros((lay.capacity, w.H), np.uint16)
        t, k = np.nonzero(ref["slot_of"][tok] >= 0)
        recv_ref[ref["slot_of"][tok][t, k]] = x_bits[tok[t]]
        ref_y, ref_acc = oracle.combine(recv_ref, ref["slot_of"], inp["topk_weights"],
                                        tokens=tok)
        got = host_u16(y)[tok]
        assert check_combine(got, ref_y, ref_acc) == 0
    for a, b in zip(handle, (lay.slot_of, lay.expert_slot_offset, lay.num_recv_per_expert)):
        assert torch.equal(a, b)
