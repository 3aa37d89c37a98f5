"""Pins for the oracle's number formats (bf16 RNE, OCP E4M3FN encode/decode,
per-128-channel quantisation).

The encoder is checked exhaustively over all 65,536 bf16 inputs times a set of
scale factors against a brute-force nearest-even search over the 256-code
table, and against torch's float8_e4m3fn cast where that cast is defined
(in range).  The decoder is checked against torch's float8_e4m3fn -> float32.
bf16 rounding is checked against torch's float32 -> bfloat16 cast.
"""
import numpy as np
import pytest
import torch


def _torch_e4m3_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def test_e4m3_decode_all_codes(orc):
    ours = orc.e4m3_to_f32(np.arange(256, dtype=np.uint8))
    ref = _torch_e4m3_table()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert ours[0x7E] == 448.0 and ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9


def brute_force_e4m3(y):
    """Nearest finite code by exhaustive search; ties to the even code; beyond
    the largest finite value saturate; NaN -> 0x7F with the sign bit."""
    table = _torch_e4m3_table()[:0x7F].astype(np.float64)   # codes 0x00..0x7E, ascending
    y = y.astype(np.float32)
    a = np.abs(y.astype(np.float64))
    sign = np.where(np.signbit(y), 0x80, 0x00)
    dist = np.abs(a[:, None] - table[None, :])
    best = dist.min(axis=1)
    cand = dist == best[:, None]
    # among equally near codes pick the even one (there are at most two)
    even = cand & (np.arange(0x7F)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    pick = np.where(a >= 448.0, 0x7E, pick)
    out = (pick | sign).astype(np.uint8)
    out = np.where(np.isnan(y), (0x7F | sign).astype(np.uint8), out)
    return out


ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


@pytest.mark.parametrize("inv", [1.0, 448.0 / 3.0, 448.0 / 0.7109375, 2.0 ** 7, 2.0 ** -7,
                                 448.0 / 4.25, 1.7320508])
def test_e4m3_encode_exhaustive_bf16_times_inv(orc, inv):
    v = orc.bf16_to_f32(ALL_BF16)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (v * np.float32(inv)).astype(np.float32)
    fin = np.isfinite(y)
    ours = orc.f32_to_e4m3(y)
    # brute force in chunks (the search matrix is 127 wide)
    ref = np.concatenate([brute_force_e4m3(y[i:i + 8192]) for i in range(0, y.size, 8192)])
    np.testing.assert_array_equal(ours[fin], ref[fin])
    # NaN inputs stay NaN codes
    assert np.all((ours[np.isnan(y)] & 0x7F) == 0x7F)
    # infinities saturate
    inf = np.isinf(y)
    np.testing.assert_array_equal(ours[inf], np.where(y[inf] > 0, 0x7E, 0xFE).astype(np.uint8))


def test_e4m3_encode_matches_torch_in_range(orc):
    rng = np.random.default_rng(7)
    y = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 100,
        rng.uniform(-448, 448, 200_000).astype(np.float32),
        (rng.standard_normal(100_000) * 2.0 ** -7).astype(np.float32),   # subnormal region
        _torch_e4m3_table()[:0x7F],                                     # exact codes
        ((_torch_e4m3_table()[:0x7E] + _torch_e4m3_table()[1:0x7F]) / 2).astype(np.float32),  # ties
    ])
    y = y[np.abs(y) <= 448]
    ours = orc.f32_to_e4m3(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_bf16_decode_exhaustive(orc):
    ours = orc.bf16_to_f32(ALL_BF16)
    ref = torch.from_numpy(ALL_BF16.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_round_matches_torch(orc):
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    # add exact ties and near-ties around every 64th bf16 value, and the overflow edge
    hi = (np.arange(0, 65536, 64, dtype=np.uint32) << 16)
    bits = np.concatenate([bits, hi | 0x8000, hi | 0x7FFF, hi | 0x8001,
                           np.array([0x7F7FFFFF, 0x7F7F8000, 0xFF7F8000], np.uint32)])
    f = bits.view(np.float32)
    ours = orc.f32_to_bf16(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x7F) != 0)


def test_quantize_amax_maps_to_448_and_error_bound(orc):
    """Closed forms: the amax element encodes to +-448 (0x7E/0xFE), because
    fl(amax * fl(448/amax)) lies within 448 (1 +- 2^-23); and the dequantised
    value q * scale stays within half an E4M3 ulp of v (relative 2^-4 for
    normals, 2^-10 * scale absolute in the subnormal range), with slack for
    the rounding of scale and of the scaled value."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 1024)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, size=(64, 8)).repeat(128, axis=1)).astype(np.float32)
    x[0, :128] = 0.0                       # an all-zero group
    x[0, 128:256] = -0.0
    x[1, :128] *= 1e-30                    # tiny but normal group
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q, sc = orc.quantize_rows(bits)
    v = orc.bf16_to_f32(bits).reshape(64, 8, 128).astype(np.float64)
    qv = orc.e4m3_to_f32(q).reshape(64, 8, 128).astype(np.float64)
    scale = sc.astype(np.float64)[:, :, None]
    amax = np.abs(v).max(axis=2)
    nz = amax > 0
    # zero groups: scale 1, signed zero codes
    assert sc[0, 0] == 1.0 and sc[0, 1] == 1.0
    assert np.all(q[0, :128] == 0x00) and np.all(q[0, 128:256] == 0x80)
    # the scale is amax/448 rounded once
    np.testing.assert_allclose(sc[nz], (amax / 448.0)[nz], rtol=2.0 ** -23)
    # the amax element encodes to the largest code
    am = np.abs(v).argmax(axis=2)
    qa = np.take_along_axis(q.reshape(64, 8, 128), am[:, :, None], axis=2)[:, :, 0]
    assert np.all((qa[nz] & 0x7F) == 0x7E)
    # dequantisation error
    err = np.abs(qv * scale - v)
    bound = np.maximum(2.0 ** -4 * np.abs(v), 2.0 ** -10 * scale) * (1 + 2.0 ** -20) + 1e-45
    assert np.all(err[nz] <= bound[nz])
