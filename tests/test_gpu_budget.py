"""GPU parity of the CU-budget launches (ep_problem_t.cu_budget > 0: persistent
grids, one workgroup per CU).  Every budget must give the bytes of the
ordinary launch, which the main parity tests hold to the oracle; the ragged
case and the prefill workload (ordinary launch and one budget) are also
compared with the oracle directly.
"""
import numpy as np
import pytest
import torch

import combine_ep_get_amd as ep
import oracle
from combine_ep_get_amd import workloads as wl

from .gpu_util import check_combine, dev_bf16, host_u16, oracle_threads, say

pytestmark = pytest.mark.gpu

RAGGED = wl.custom(N=60, H=384, E=12, K=3, R=3, A=16, name="ragged")


def _run(w, inp, mode, budget, lay, eo):
    """dispatch (with tags, zero padding, statistics) + combine at one budget."""
    fp8 = mode != "bf16"
    wts = torch.from_numpy(inp["topk_weights"]).cuda()
    out = ep.alloc_recv(lay, w.H, fp8)
    out[0].view(torch.uint8).fill_(0x3C)
    if fp8:
        out[1].fill_(7.0)
    out[2].fill_(-9)
    out[3].fill_(9.0)
    stats = torch.full((w.E,), 11, dtype=torch.int64, device="cuda")
    kw = dict(out=out, zero_padding=True, cumulative_stats=stats, cu_budget=budget)
    if mode == "prequant":
        codes, scales = oracle.quantize_rows(inp["x"])
        xq = torch.from_numpy(codes).cuda().view(torch.float8_e4m3fn)
        ep.dispatch(xq, wts, lay, True, x_scales=torch.from_numpy(scales).cuda(), **kw)
    else:
        ep.dispatch(dev_bf16(inp["x"]), wts, lay, fp8, **kw)
    y = ep.combine(eo, lay, wts, cu_budget=budget)
    torch.cuda.synchronize()
    res = [out[0].view(torch.uint8).cpu(), out[2].cpu(), out[3].cpu(), stats.cpu(),
           y.view(torch.int16).cpu()]
    if fp8:
        res.append(out[1].cpu())
    return res


def _check_oracle(w, inp, mode, res, cap, eo_bits):
    """One launch's outputs (from _run) against the oracle: payload with zeroed
    padding rows and the pre-fill elsewhere, scales, tags, running statistics
    and combine."""
    r = oracle.layout(inp["topk_idx"], w.E, w.R, w.A)
    th = oracle_threads()
    off, cnt = r["expert_slot_offset"], r["num_recv_per_expert"]
    src, rw = oracle.recv_meta(r["slot_of"], inp["topk_weights"], cap)
    np.testing.assert_array_equal(res[1].numpy(), src)
    np.testing.assert_array_equal(res[2].numpy().view(np.uint32), rw.view(np.uint32))
    want = np.full(w.E, 11, np.int64)
    oracle.accumulate_stats(cnt, want)
    np.testing.assert_array_equal(res[3].numpy(), want)
    if mode == "bf16":
        rx = oracle.dispatch_bf16(inp["x"], r["slot_of"], cap, fill=0x3C3C, threads=th)
        oracle.zero_padding(rx, None, off, cnt)
        np.testing.assert_array_equal(res[0].numpy().view(np.uint16), rx)
    else:
        if mode == "fp8":
            q, sc = oracle.dispatch_fp8(inp["x"], r["slot_of"], cap, threads=th)
        else:
            codes, scales = oracle.quantize_rows(inp["x"])
            q, sc = oracle.dispatch_quantized(codes, scales, r["slot_of"], cap)
        valid = src >= 0
        q_want = np.full((cap, w.H), 0x3C, np.uint8)
        sc_want = np.full((cap, w.H // 128), 7.0, np.float32)
        q_want[valid] = q[valid]
        sc_want[valid] = sc[valid]
        oracle.zero_padding(q_want, sc_want, off, cnt)
        np.testing.assert_array_equal(res[0].numpy().reshape(cap, w.H), q_want)
        np.testing.assert_array_equal(res[5].numpy().view(np.uint32), sc_want.view(np.uint32))
    ref_y, ref_acc = oracle.combine(eo_bits, r["slot_of"], inp["topk_weights"], threads=th)
    assert check_combine(res[4].numpy().view(np.uint16), ref_y, ref_acc) == 0


@pytest.mark.parametrize("mode", ["bf16", "fp8", "prequant"])
@pytest.mark.parametrize("cid", [0, 3])
def test_budget_matches_ordinary_launch(cid, mode):
    """Every budget gives the ordinary launch's bytes; the ordinary launch and
    one budgeted launch are also held to the oracle directly."""
    w = RAGGED if cid == 0 else wl.CONFIGS[cid]
    inp = wl.make_inputs(w, 0)
    say(f"CU budget parity {w.desc} mode={mode}")
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    lay = ep.get_layout(idx, w.E, w.R, w.A)
    eo = wl.make_expert_out_device(w, lay.capacity, 0)
    eo_bits = host_u16(eo)
    ref = _run(w, inp, mode, 0, lay, eo)
    budgets = [1, 3, 256] if cid == 0 else [5, 64, 255, 4096]
    got = None
    for b in budgets:
        got = _run(w, inp, mode, b, lay, eo)
        for i, (a, c) in enumerate(zip(ref, got)):
            assert torch.equal(a, c), f"budget {b}: output {i} differs from the ordinary launch"
        say(f"  budget {b}: identical")
    _check_oracle(w, inp, mode, ref, lay.capacity, eo_bits)
    _check_oracle(w, inp, mode, got, lay.capacity, eo_bits)
    say(f"  ordinary launch and budget {budgets[-1]} equal the oracle")


EDGE = [(wl.custom(N=48, H=136, E=16, K=12, R=4, A=3, name="k12_h136"), "bf16"),
        (wl.custom(N=32, H=16392, E=8, K=2, R=2, A=1, name="h16392"), "bf16"),
        (wl.custom(N=64, H=16384, E=8, K=3, R=4, A=4, name="fp8_h16384"), "fp8"),
        (wl.custom(N=256, H=256, E=1024, K=32, R=256, A=2, name="e1024_k32"), "bf16"),
        (wl.custom(N=40, H=1152, E=10, K=5, R=5, A=7, name="prequant_ragged"), "prequant")]


@pytest.mark.parametrize("w,mode", EDGE, ids=[e[0].name for e in EDGE])
def test_budget_edge_shapes(w, mode):
    inp = wl.make_inputs(w, 1)
    say(f"CU budget edge {w.desc} mode={mode}")
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    lay = ep.get_layout(idx, w.E, w.R, w.A)
    eo_bits = wl.make_expert_out(w, lay.capacity, 1)
    eo = dev_bf16(eo_bits)
    ref = _run(w, inp, mode, 0, lay, eo)
    for b in (1, 2, 37):
        got = _run(w, inp, mode, b, lay, eo)
        for i, (a, c) in enumerate(zip(ref, got)):
            assert torch.equal(a, c), f"budget {b}: output {i} differs from the ordinary launch"
    r = oracle.layout(inp["topk_idx"], w.E, w.R, w.A)
    ref_y, ref_acc = oracle.combine(eo_bits, r["slot_of"], inp["topk_weights"])
    assert check_combine(ref[4].numpy().view(np.uint16), ref_y, ref_acc) == 0
