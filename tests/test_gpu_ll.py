"""GPU parity of the single-launch low-latency dispatch against the oracle:
routing (recv_count, slot_of, per-source flags) bit-exact, payload rows (bf16
or e4m3 codes + scales) and slot tags bit-exact, and combine through the
low-latency handle within the contract (bit-exact expected)."""
import numpy as np
import pytest
import torch

import combine_ep_get_amd as ep
import oracle
from combine_ep_get_amd import workloads as wl

from .gpu_util import check_combine, dev_bf16, host_u16, host_u8, say

pytestmark = pytest.mark.gpu


def run_ll(idx, x_bits, wts, E, R, M, fp8):
    idx = np.ascontiguousarray(idx, np.int32)
    N, K = idx.shape
    H = x_bits.shape[1]
    say(f"ll N={N} H={H} E={E} K={K} R={R} M={M} fp8={fp8}")
    lay, recv = ep.alloc_ll(N, K, E, R, M, H, fp8)
    recv[0].view(torch.uint8).fill_(0x55)
    recv[2].fill_(-7)
    recv[3].fill_(-7.0)
    lay, recv = ep.ll_dispatch(dev_bf16(x_bits), torch.from_numpy(idx).cuda(),
                               torch.from_numpy(wts).cuda(), E, R, M, fp8, out=(lay, recv))
    torch.cuda.synchronize()
    ref = oracle.ll_layout(idx, E, R, M)
    np.testing.assert_array_equal(lay.recv_count.cpu().numpy(), ref["recv_count"])
    np.testing.assert_array_equal(lay.slot_of.cpu().numpy(), ref["slot_of"])
    np.testing.assert_array_equal(lay.flags.cpu().numpy(), ref["flags"])
    cap = lay.capacity
    src = recv[2].cpu().numpy()
    rw = recv[3].cpu().numpy()
    t_of, k_of = np.nonzero(ref["slot_of"] >= 0)
    slots = ref["slot_of"][t_of, k_of]
    np.testing.assert_array_equal(src[slots], t_of)
    np.testing.assert_array_equal(rw[slots].view(np.uint32), wts[t_of, k_of].view(np.uint32))
    untouched = np.ones(cap, bool)
    untouched[slots] = False
    assert np.all(src[untouched] == -7)
    st = torch.from_numpy(slots.astype(np.int64)).cuda()
    if fp8:
        q, sc = oracle.quantize_rows(x_bits)
        got = host_u8(recv[0].view(torch.uint8).index_select(0, st))
        np.testing.assert_array_equal(got, q[t_of])
        gsc = recv[1].index_select(0, st).cpu().numpy()
        np.testing.assert_array_equal(gsc.view(np.uint32), sc[t_of].view(np.uint32))
    else:
        got = host_u16(recv[0].view(torch.int16).index_select(0, st))
        np.testing.assert_array_equal(got, x_bits[t_of])
    # combine through the low-latency handle
    rng = np.random.default_rng(5)
    eo_rows = torch.from_numpy(rng.standard_normal((slots.size, H), dtype=np.float32)) \
        .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    eo_bits = np.zeros((cap, H), np.uint16)
    eo_bits[slots] = eo_rows
    y = ep.combine(dev_bf16(eo_bits), lay, torch.from_numpy(wts).cuda())
    torch.cuda.synchronize()
    ref_y, ref_acc = oracle.combine(eo_bits, ref["slot_of"], wts)
    assert check_combine(host_u16(y), ref_y, ref_acc) == 0
    return lay


@pytest.mark.parametrize("fp8", [False, True])
def test_ll_decode_workload(fp8):
    w = wl.CONFIGS[2]
    inp = wl.make_inputs(w, 0)
    run_ll(inp["topk_idx"], inp["x"], inp["topk_weights"], w.E, w.R, w.N // w.R, fp8)


def test_ll_overflow_and_bad_indices():
    rng = np.random.default_rng(9)
    N, K, E, R, H = 64, 4, 16, 4, 256
    idx = rng.integers(0, 4, size=(N, K)).astype(np.int32)      # hot experts, duplicates
    idx[5, 2] = -1
    idx[9, 0] = 99
    x = torch.from_numpy(rng.standard_normal((N, H), dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)
    wts = rng.random((N, K), dtype=np.float32)
    lay = run_ll(idx, x, wts, E, R, 3, False)                    # M=3 overflows
    assert (lay.flags.cpu().numpy() & ep.EP_LAYOUT_ERR_OVERFLOW).any()


def test_ll_small_and_empty():
    rng = np.random.default_rng(10)
    for N, K, E, R, H, M, fp8 in ((16, 2, 8, 4, 128, 4, True), (128, 2, 16, 4, 256, 40, False),
                                  (0, 2, 16, 4, 64, 4, False)):
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(N)]) if N else \
            np.zeros((0, K), np.int32)
        x = torch.from_numpy(rng.standard_normal((N, H), dtype=np.float32)).to(torch.bfloat16) \
            .view(torch.int16).numpy().view(np.uint16)
        run_ll(idx, x, rng.random((N, K), dtype=np.float32), E, R, M, fp8)


@pytest.mark.parametrize("M", [64, 3])
def test_ll_prequantized_and_stats(M):
    """Pre-quantised e4m3 input copied unchanged into the sub-blocks, and the
    running per-expert counts growing by the placed rows once per call (M = 3
    overflows many sub-blocks, so placed rows < routed pairs)."""
    w = wl.CONFIGS[2]
    inp = wl.make_inputs(w, 1)
    rng = np.random.default_rng(17)
    N, H, K, E, R = w.N, w.H, w.K, w.E, w.R
    codes = rng.integers(0, 256, size=(N, H), dtype=np.uint8)
    scales = rng.standard_normal((N, H // 128)).astype(np.float32)
    say(f"ll pre-quantised + stats {w.desc} M={M}")
    stats = torch.full((E,), 5, dtype=torch.int64, device="cuda")
    xq = torch.from_numpy(codes).cuda().view(torch.float8_e4m3fn)
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    wts = torch.from_numpy(inp["topk_weights"]).cuda()
    for _ in range(2):
        lay, (rx, rs, src, _) = ep.ll_dispatch(xq, idx, wts, E, R, M, True,
                                               x_scales=torch.from_numpy(scales).cuda(),
                                               cumulative_stats=stats)
    torch.cuda.synchronize()
    ref = oracle.ll_layout(inp["topk_idx"], E, R, M)
    np.testing.assert_array_equal(lay.slot_of.cpu().numpy(), ref["slot_of"])
    np.testing.assert_array_equal(lay.recv_count.cpu().numpy(), ref["recv_count"])
    t, k = np.nonzero(ref["slot_of"] >= 0)
    sl = torch.from_numpy(ref["slot_of"][t, k].astype(np.int64)).cuda()
    np.testing.assert_array_equal(host_u8(rx.view(torch.uint8).index_select(0, sl)), codes[t])
    np.testing.assert_array_equal(rs.index_select(0, sl).cpu().numpy().view(np.uint32),
                                  scales[t].view(np.uint32))
    np.testing.assert_array_equal(src.index_select(0, sl).cpu().numpy(), t)
    want = np.full(E, 5, np.int64)
    per_expert = ref["recv_count"].sum(axis=1).astype(np.int32)
    oracle.accumulate_stats(per_expert, want)
    oracle.accumulate_stats(per_expert, want)
    np.testing.assert_array_equal(stats.cpu().numpy(), want)
