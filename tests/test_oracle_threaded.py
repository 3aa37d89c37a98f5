"""The oracle's threaded driver (token ranges split over threads, each piece
run by the single-threaded function) gives the same bytes as one
single-threaded call: bf16 and e4m3 dispatch, combine (bf16 and its fp32
accumulator), on uneven splits, more threads than tokens, and tokens
with -1 entries and duplicate experts."""
import numpy as np
import pytest

from combine_ep_get_amd import workloads as wl

CASES = [
    wl.custom(N=1024, H=1024, E=64, K=8, R=8, A=16, name="mid"),
    wl.custom(N=21, H=256, E=12, K=3, R=3, A=5, name="ragged"),
    wl.custom(N=4, H=128, E=4, K=2, R=2, A=1, name="tiny"),
]


@pytest.mark.parametrize("threads", [2, 3, 7, 64])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_threaded_driver_is_byte_identical(orc, w, threads):
    inp = wl.make_inputs(w, seed=threads)
    idx = inp["topk_idx"].copy()
    idx[1, 0] = -1                                   # a pair without an expert
    idx[2, -1] = idx[2, 0]                           # a repeated expert
    lay = orc.layout(idx, w.E, w.R, w.A)
    cap = orc.capacity(w.N, w.K, w.E, w.A)
    a = orc.dispatch_bf16(inp["x"], lay["slot_of"], cap, fill=0x1234)
    b = orc.dispatch_bf16(inp["x"], lay["slot_of"], cap, fill=0x1234, threads=threads)
    np.testing.assert_array_equal(a, b)
    qa, sa = orc.dispatch_fp8(inp["x"], lay["slot_of"], cap)
    qb, sb = orc.dispatch_fp8(inp["x"], lay["slot_of"], cap, threads=threads)
    np.testing.assert_array_equal(qa, qb)
    np.testing.assert_array_equal(sa.view(np.uint32), sb.view(np.uint32))
    eo = wl.make_expert_out(w, cap, seed=threads)
    ya, acca = orc.combine(eo, lay["slot_of"], inp["topk_weights"])
    yb, accb = orc.combine(eo, lay["slot_of"], inp["topk_weights"], threads=threads)
    np.testing.assert_array_equal(ya, yb)
    np.testing.assert_array_equal(acca.view(np.uint32), accb.view(np.uint32))
