"""Seeded random shapes through every entry point, compared in full with the
oracle: layout outputs, every receive row and tag, combine outputs, the
low-latency layout and rows, and a CU budget.  Routing indices are raw draws
that include -1 entries and repeated experts inside a token, which the
workload generators never produce.
"""
import numpy as np
import pytest
import torch

import combine_ep_get_amd as ep
import oracle

from .gpu_util import check_combine, check_layout, dev_bf16, host_u16, host_u8, say

pytestmark = pytest.mark.gpu


def _case(seed, wide=False):
    """wide: rows of up to 3,192 bf16 channels or 24 e4m3 groups (several
    dispatch pieces with a ragged last one), for seeds of their own."""
    rng = np.random.default_rng(7000 + seed)
    R = int(rng.choice([1, 2, 3, 4, 8]))
    E = R * int(rng.integers(1, 9))
    K = int(rng.integers(1, min(E, 12) + 1)) if rng.random() < 0.8 else int(rng.integers(1, 33))
    N = R * int(rng.integers(0, 40))
    A = int(rng.choice([1, 1, 2, 3, 8, 16]))
    fp8 = bool(rng.random() < 0.4)
    if wide:
        H = 128 * int(rng.integers(1, 25)) if fp8 else 8 * int(rng.integers(1, 400))
    else:
        H = 128 * int(rng.integers(1, 5)) if fp8 else 8 * int(rng.integers(1, 80))
    idx = rng.integers(-1, E, size=(N, K)).astype(np.int32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    x = (rng.standard_normal((N, H)).astype(np.float32) * rng.uniform(0.01, 100))
    x_bits = oracle.f32_to_bf16(x)
    return dict(R=R, E=E, K=K, N=N, A=A, H=H, fp8=fp8, idx=idx, w=w, x=x_bits,
                budget=int(rng.choice([0, 1, 3, 17])), M=int(rng.integers(1, 6)),
                rng=rng)


@pytest.mark.parametrize("seed", range(40))
def test_random_shape_parity(seed):
    _run(seed, _case(seed))


@pytest.mark.parametrize("seed", range(100, 112))
def test_random_shape_parity_wide_rows(seed):
    c = _case(seed, wide=True)
    c["budget"] = 0      # the ordinary launches: rows in several pieces
    _run(seed, c)


def _run(seed, c):
    N, H, K, E, R, A, fp8 = c["N"], c["H"], c["K"], c["E"], c["R"], c["A"], c["fp8"]
    say(f"random seed={seed}: N={N} H={H} K={K} E={E} R={R} A={A} fp8={fp8} "
        f"budget={c['budget']}")
    idx_t = torch.from_numpy(c["idx"] if seed % 2 else c["idx"].astype(np.int64)).cuda()
    lay = ep.get_layout(idx_t, E, R, A)
    ref = oracle.layout(c["idx"], E, R, A)
    check_layout(lay, ref)
    cap = lay.capacity
    wts = torch.from_numpy(c["w"]).cuda()
    out = ep.alloc_recv(lay, H, fp8)
    out[0].view(torch.uint8).fill_(0xA5)
    if fp8:
        out[1].fill_(-1.0)
    stats = torch.zeros(E, dtype=torch.int64, device="cuda")
    zero = bool(seed % 3 == 0)
    ep.dispatch(dev_bf16(c["x"]), wts, lay, fp8, out=out, zero_padding=zero,
                cumulative_stats=stats, cu_budget=c["budget"])
    torch.cuda.synchronize()
    src, rw = oracle.recv_meta(ref["slot_of"], c["w"], cap)
    np.testing.assert_array_equal(out[2].cpu().numpy(), src)
    np.testing.assert_array_equal(out[3].cpu().numpy().view(np.uint32), rw.view(np.uint32))
    if fp8:
        q, sc = oracle.dispatch_fp8(c["x"], ref["slot_of"], cap)
        q[src < 0] = 0xA5
        sc[src < 0] = -1.0
        if zero:
            oracle.zero_padding(q, sc, ref["expert_slot_offset"], ref["num_recv_per_expert"])
        np.testing.assert_array_equal(host_u8(out[0].view(torch.uint8)), q)
        np.testing.assert_array_equal(out[1].cpu().numpy().view(np.uint32), sc.view(np.uint32))
    else:
        rx = oracle.dispatch_bf16(c["x"], ref["slot_of"], cap, fill=0xA5A5)
        if zero:
            oracle.zero_padding(rx, None, ref["expert_slot_offset"], ref["num_recv_per_expert"])
        np.testing.assert_array_equal(host_u16(out[0]), rx)
    want = np.zeros(E, np.int64)
    oracle.accumulate_stats(ref["num_recv_per_expert"], want)
    np.testing.assert_array_equal(stats.cpu().numpy(), want)
    # combine of random expert outputs
    eo_bits = oracle.f32_to_bf16(c["rng"].standard_normal((cap, H)).astype(np.float32))
    y = ep.combine(dev_bf16(eo_bits), lay, wts, cu_budget=c["budget"])
    torch.cuda.synchronize()
    ref_y, ref_acc = oracle.combine(eo_bits, ref["slot_of"], c["w"])
    assert check_combine(host_u16(y), ref_y, ref_acc) == 0
    # low-latency path on the same routing when a source's pairs fit
    if N and (N // R) * K <= 4096:
        M = c["M"]
        ll_lay, (lx, lsc, lsrc, _) = ep.ll_dispatch(dev_bf16(c["x"]), idx_t, wts, E, R, M, fp8)
        torch.cuda.synchronize()
        lref = oracle.ll_layout(c["idx"], E, R, M)
        np.testing.assert_array_equal(ll_lay.slot_of.cpu().numpy(), lref["slot_of"])
        np.testing.assert_array_equal(ll_lay.recv_count.cpu().numpy(), lref["recv_count"])
        np.testing.assert_array_equal(ll_lay.flags.cpu().numpy(), lref["flags"])
        t, k = np.nonzero(lref["slot_of"] >= 0)
        if t.size:
            sl = torch.from_numpy(lref["slot_of"][t, k].astype(np.int64)).cuda()
            if fp8:
                qq, ss = oracle.quantize_rows(c["x"])
                np.testing.assert_array_equal(host_u8(lx.view(torch.uint8).index_select(0, sl)),
                                              qq[t])
                np.testing.assert_array_equal(lsc.index_select(0, sl).cpu().numpy()
                                              .view(np.uint32), ss[t].view(np.uint32))
            else:
                np.testing.assert_array_equal(host_u16(lx.index_select(0, sl)), c["x"][t])
            np.testing.assert_array_equal(lsrc.index_select(0, sl).cpu().numpy(), t)
