"""Pins for the oracle's dispatch variants (DeepEP book ch.1 sec. 1.1: x as a
pair of FP8 data and scales, cumulative_local_expert_recv_stats,
do_zero_padding).

- pre-quantised pass-through: brute force per pair (every slot holds its
  token's codes and scales, every other row stays zero), and quantising first
  then passing through equals the fused FP8 dispatch;
- zero padding: the zeroed rows are exactly the slots of an expert region past
  its pairs, found here by walking the regions in Python; every other byte is
  unchanged; their number is off[E] minus the valid pairs (closed form);
- running statistics: the increments equal a histogram of the routing indices
  (np.bincount), and repeated calls add up.
"""
import numpy as np
import pytest

from combine_ep_get_amd import workloads as wl

CASES = [wl.custom(N=24, H=256, E=8, K=3, R=2, A=4, fp8=True, name="small"),
         wl.custom(N=60, H=384, E=12, K=3, R=3, A=16, fp8=True, name="ragged"),
         wl.custom(N=0, H=128, E=4, K=2, R=2, A=8, fp8=True, name="empty")]


def _codes(rng, N, H):
    # any byte is a valid payload for a copy, NaN codes included
    return rng.integers(0, 256, size=(N, H), dtype=np.uint8)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_prequantized_passthrough_bruteforce(orc, w):
    rng = np.random.default_rng(7)
    inp = wl.make_inputs(w, seed=3)
    lay = orc.layout(inp["topk_idx"], w.E, w.R, w.A)
    cap = orc.capacity(w.N, w.K, w.E, w.A)
    codes = _codes(rng, w.N, w.H)
    scales = rng.standard_normal((w.N, w.H // 128)).astype(np.float32)
    q, sc = orc.dispatch_quantized(codes, scales, lay["slot_of"], cap)
    written = np.zeros(cap, bool)
    for t in range(w.N):
        for k in range(w.K):
            s = lay["slot_of"][t, k]
            if s < 0:
                continue
            written[s] = True
            assert np.array_equal(q[s], codes[t])
            assert np.array_equal(sc[s].view(np.uint32), scales[t].view(np.uint32))
    assert not q[~written].any() and not sc[~written].any()


@pytest.mark.parametrize("w", CASES[:2], ids=lambda w: w.name)
def test_quantize_then_passthrough_equals_fused(orc, w):
    inp = wl.make_inputs(w, seed=4)
    lay = orc.layout(inp["topk_idx"], w.E, w.R, w.A)
    cap = orc.capacity(w.N, w.K, w.E, w.A)
    codes, scales = orc.quantize_rows(inp["x"])
    q1, s1 = orc.dispatch_quantized(codes, scales, lay["slot_of"], cap)
    q2, s2 = orc.dispatch_fp8(inp["x"], lay["slot_of"], cap)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1.view(np.uint32), s2.view(np.uint32))


def _padding_rows(off, cnt):
    rows = set()
    for e in range(len(cnt)):
        start = int(off[e]) + int(cnt[e])
        for s in range(start, int(off[e + 1])):
            rows.add(s)
    return rows


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("fp8", [False, True])
def test_zero_padding_bruteforce(orc, w, fp8):
    rng = np.random.default_rng(11)
    inp = wl.make_inputs(w, seed=5)
    lay = orc.layout(inp["topk_idx"], w.E, w.R, w.A)
    cap = orc.capacity(w.N, w.K, w.E, w.A)
    if fp8:
        before = rng.integers(1, 256, size=(cap, w.H), dtype=np.uint8)
        sbefore = rng.uniform(1, 2, size=(cap, w.H // 128)).astype(np.float32)
    else:
        before = rng.integers(1, 65536, size=(cap, w.H), dtype=np.uint16)
        sbefore = None
    x = before.copy()
    sc = None if sbefore is None else sbefore.copy()
    off, cnt = lay["expert_slot_offset"], lay["num_recv_per_expert"]
    orc.zero_padding(x, sc, off, cnt)
    pad = _padding_rows(off, cnt)
    valid = int((lay["slot_of"] >= 0).sum())
    assert len(pad) == int(off[-1]) - valid
    for s in range(cap):
        if s in pad:
            assert not x[s].any()
            if sc is not None:
                assert not sc[s].any()
        else:
            assert np.array_equal(x[s], before[s])
            if sc is not None:
                assert np.array_equal(sc[s], sbefore[s])


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_cumulative_stats_are_a_histogram(orc, w):
    inp = wl.make_inputs(w, seed=6)
    lay = orc.layout(inp["topk_idx"], w.E, w.R, w.A)
    idx = inp["topk_idx"].reshape(-1)
    hist = np.bincount(idx[(idx >= 0) & (idx < w.E)], minlength=w.E).astype(np.int64)
    start = np.arange(w.E, dtype=np.int64) * (1 << 33) - 5
    stats = start.copy()
    orc.accumulate_stats(lay["num_recv_per_expert"], stats)
    np.testing.assert_array_equal(stats, start + hist)
    orc.accumulate_stats(lay["num_recv_per_expert"], stats)
    np.testing.assert_array_equal(stats, start + 2 * hist)
