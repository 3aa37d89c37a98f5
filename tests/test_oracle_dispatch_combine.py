"""Pins for the oracle's dispatch and combine.

- bf16 dispatch is a bit copy: every valid slot holds its source row, other
  rows are untouched (closed form).
- combine after dispatch with identity experts equals sum_k w_k * x_t computed
  directly per token in float64 (the round-trip the DeepEP walkthrough asks for
  in its correctness-check section), within the float32 error bound, and the
  bf16 result is within one ulp of the correctly rounded float64 value.
- combine with random expert outputs per slot (so slot swaps inside a token are
  visible) agrees with a float64 sum within K * 2^-23 * sum |w * eo|.
- FP8 dispatch copies one quantisation of the token to every slot, and the
  identity round-trip stays within the E4M3 error bound of sum_k w_k * x_t.
"""
import numpy as np
import pytest

from combine_ep_get_amd import workloads as wl

CASES = [wl.CONFIGS[1],
         wl.custom(N=60, H=136, E=12, K=3, R=3, A=4, name="ragged"),
         wl.custom(N=64, H=1024, E=32, K=4, R=4, A=16, fp8=True, name="fp8small")]


def _ulp_dist_bf16(a, b):
    """Distance in bf16 ulps between two arrays of bf16 bit patterns (finite)."""
    def key(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + u)
    return np.abs(key(a) - key(b))


def _f64_to_bf16_bits(a64):
    import torch
    return torch.from_numpy(a64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_dispatch_bf16_is_row_copy(orc, w):
    inp = wl.make_inputs(w, seed=1)
    lay = orc.layout(inp["topk_idx"], w.E, w.R, w.A)
    cap = orc.capacity(w.N, w.K, w.E, w.A)
    recv = orc.dispatch_bf16(inp["x"], lay["slot_of"], cap, fill=0xDEAD)
    src, rw = orc.recv_meta(lay["slot_of"], inp["topk_weights"], cap)
    valid = src >= 0
    np.testing.assert_array_equal(recv[valid], inp["x"][src[valid]])
    assert np.all(recv[~valid] == 0xDEAD)
    t, k = np.nonzero(lay["slot_of"] >= 0)
    np.testing.assert_array_equal(rw[lay["slot_of"][t, k]], inp["topk_weights"][t, k])
    assert np.all(rw[~valid] == 0)


@pytest.mark.parametrize("w", CASES[:2], ids=lambda w: w.name)
def test_identity_round_trip_bf16(orc, w):
    inp = wl.make_inputs(w, seed=2)
    lay = orc.layout(inp["topk_idx"], w.E, w.R, w.A)
    cap = orc.capacity(w.N, w.K, w.E, w.A)
    recv = orc.dispatch_bf16(inp["x"], lay["slot_of"], cap)
    y, acc = orc.combine(recv, lay["slot_of"], inp["topk_weights"])
    # direct formula, per token, float64
    x64 = orc.bf16_to_f32(inp["x"]).astype(np.float64)
    w64 = inp["topk_weights"].astype(np.float64)
    a64 = w64.sum(axis=1, keepdims=True) * x64
    bound = w.K * 2.0 ** -23 * np.abs(w64).sum(axis=1, keepdims=True) * np.abs(x64)
    assert np.all(np.abs(acc - a64) <= bound + 1e-45)
    assert np.all(_ulp_dist_bf16(y, _f64_to_bf16_bits(a64)) <= 1)
    # weights are normalised, so the round trip returns x up to ~1 bf16 ulp
    assert np.all(_ulp_dist_bf16(y, inp["x"]) <= 2)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_combine_random_expert_outputs(orc, w):
    inp = wl.make_inputs(w, seed=3)
    lay = orc.layout(inp["topk_idx"], w.E, w.R, w.A)
    cap = orc.capacity(w.N, w.K, w.E, w.A)
    eo = wl.make_expert_out(w, cap, seed=3)
    y, acc = orc.combine(eo, lay["slot_of"], inp["topk_weights"])
    e64 = orc.bf16_to_f32(eo).astype(np.float64)
    w64 = inp["topk_weights"].astype(np.float64)
    terms = w64[:, :, None] * e64[lay["slot_of"]]            # [N, K, H]
    a64 = terms.sum(axis=1)
    bound = w.K * 2.0 ** -23 * np.abs(terms).sum(axis=1)
    assert np.all(np.abs(acc - a64) <= bound + 1e-45)
    # bf16 store: correctly rounded from the float32 accumulator
    assert np.all(_ulp_dist_bf16(y, _f64_to_bf16_bits(acc.astype(np.float64))) == 0)
    # a subset of tokens gives the same rows
    toks = np.array([w.N - 1, 0, w.N // 2], np.int32)
    y2, acc2 = orc.combine(eo, lay["slot_of"], inp["topk_weights"], tokens=toks)
    np.testing.assert_array_equal(y2, y[toks])
    np.testing.assert_array_equal(acc2, acc[toks])


def test_fp8_dispatch_and_identity_round_trip(orc):
    w = CASES[2]
    inp = wl.make_inputs(w, seed=4)
    lay = orc.layout(inp["topk_idx"], w.E, w.R, w.A)
    cap = orc.capacity(w.N, w.K, w.E, w.A)
    q, sc = orc.dispatch_fp8(inp["x"], lay["slot_of"], cap)
    qt, sct = orc.quantize_rows(inp["x"])
    src, _ = orc.recv_meta(lay["slot_of"], inp["topk_weights"], cap)
    valid = src >= 0
    np.testing.assert_array_equal(q[valid], qt[src[valid]])
    np.testing.assert_array_equal(sc[valid].view(np.uint32), sct[src[valid]].view(np.uint32))
    # identity experts read the dequantised row back as bf16
    G = w.H // 128
    deq = orc.e4m3_to_f32(q).reshape(cap, G, 128) * sc[:, :, None]
    eo = orc.f32_to_bf16(deq.reshape(cap, w.H))
    y, acc = orc.combine(eo, lay["slot_of"], inp["topk_weights"])
    x64 = orc.bf16_to_f32(inp["x"]).astype(np.float64)
    w64 = inp["topk_weights"].astype(np.float64)
    a64 = w64.sum(axis=1, keepdims=True) * x64
    amax = np.abs(x64.reshape(w.N, G, 128)).max(axis=2).repeat(128, axis=1)
    # E4M3 half-ulp (2^-4 rel, or 2^-10 * amax/448 abs) plus the bf16 rounding of eo
    bound = (2.0 ** -4 + 2.0 ** -8) * np.abs(a64) + 2.0 ** -10 * amax / 448 + 1e-6
    assert np.all(np.abs(acc - a64) <= bound)
