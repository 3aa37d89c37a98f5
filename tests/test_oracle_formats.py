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


# Group maxima (bf16 bit patterns) where the float32 inverse 448/amax is
# infinite or only just finite: the smallest bf16 subnormal (2^-133), a
# mid-range subnormal, the smallest normal (2^-126), 1e-37, and the two bf16
# values around 448/FLT_MAX (0x03E0: the inverse overflows; 0x03E1: finite).
TINY_MAXIMA = (0x0001, 0x0015, 0x0080, 0x0208, 0x03E0, 0x03E1, 0x0400, 0x0C00)


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def tiny_groups(rng, n_per=6):
    """[n, 128] bf16 groups whose maximum |v| is one of TINY_MAXIMA, with
    the maximum itself (either sign), mixed-sign values below it (bf16
    subnormals included), and +0 / -0 elements."""
    rows = []
    for mb in TINY_MAXIMA:
        m = np.float32((np.uint32(mb) << 16).view(np.float32))
        for j in range(n_per):
            g = (rng.uniform(-1.0, 1.0, 128) * m).astype(np.float32)
            g[rng.integers(0, 128, 8)] = 0.0
            g[rng.integers(0, 128, 8)] = -0.0
            g[rng.integers(0, 128)] = m if j % 2 == 0 else -m
            bits = _bf16(g)
            # values of the draw may round up past m; keep the group maximum at m
            over = np.abs((bits.astype(np.uint32) << 16).view(np.float32)) > m
            bits[over] = 0x8000
            rows.append(bits)
    return np.stack(rows)


def _check_quantised_groups(orc, bits):
    """The closed forms for [rows, H] bf16 groups: the amax element encodes to
    +-448 (0x7E/0xFE); the scale is amax/448 rounded once to float32; the
    dequantised value decode(q) * scale lies within half an E4M3 ulp of v
    (relative 2^-4 for normals, 2^-10 * amax/448 absolute in the subnormal
    range), plus the rounding of the float32 inverse and product (2^-22 |v|)
    and of the stored scale (448 |scale - amax/448|); zero groups have scale 1
    and keep each zero's sign."""
    n, H = bits.shape
    G = H // 128
    q, sc = orc.quantize_rows(bits)
    v = orc.bf16_to_f32(bits).reshape(n, G, 128).astype(np.float64)
    qv = orc.e4m3_to_f32(q).reshape(n, G, 128).astype(np.float64)
    scale = sc.astype(np.float64)[:, :, None]
    amax = np.abs(v).max(axis=2)
    nz = amax > 0
    # zero groups: scale 1, signed zero codes
    assert np.all(sc[~nz] == 1.0)
    qz = q.reshape(n, G, 128)[~nz]
    sz = np.signbit(v[~nz])
    assert np.all(qz == np.where(sz, 0x80, 0x00))
    # the scale is amax/448 rounded once (float32 subnormals included)
    np.testing.assert_array_equal(sc[nz], (amax / 448.0).astype(np.float32)[nz])
    # the amax element encodes to the largest code
    am = np.abs(v).argmax(axis=2)
    qa = np.take_along_axis(q.reshape(n, G, 128), am[:, :, None], axis=2)[:, :, 0]
    assert np.all((qa[nz] & 0x7F) == 0x7E)
    # every zero element of a non-zero group stays a zero of its sign
    zero_el = (v == 0) & nz[:, :, None]
    qg = q.reshape(n, G, 128)
    assert np.all(qg[zero_el] == np.where(np.signbit(v[zero_el]), 0x80, 0x00))
    # dequantisation error
    s_star = (amax / 448.0)[:, :, None]
    err = np.abs(qv * scale - v)
    bound = (np.maximum(2.0 ** -4 * np.abs(v), 2.0 ** -10 * s_star) * (1 + 2.0 ** -22)
             + 2.0 ** -22 * np.abs(v) + 448.0 * np.abs(scale - s_star)) * (1 + 2.0 ** -40)
    ok = err <= bound
    assert np.all(ok[nz]), f"{int((~ok[nz]).sum())} elements beyond the dequantisation bound"
    return q, sc


def test_quantize_amax_maps_to_448_and_error_bound(orc):
    """Closed forms (see _check_quantised_groups) over groups spanning 40
    binades, all-zero and signed-zero groups, and groups whose maximum sits
    where the float32 inverse 448/amax overflows or nearly does (bf16
    subnormal maxima included)."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 1024)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, size=(64, 8)).repeat(128, axis=1)).astype(np.float32)
    x[0, :128] = 0.0                       # an all-zero group
    x[0, 128:256] = -0.0
    x[1, :128] *= 1e-30                    # tiny but normal group
    bits = _bf16(x)
    _check_quantised_groups(orc, bits)
    _check_quantised_groups(orc, tiny_groups(rng))


def test_quantize_codes_invariant_under_power_of_two_scaling(orc):
    """What the codes approximate, v * 448 / amax, does not change when a
    group is multiplied by 2^j, and float32 rounding commutes with exact
    power-of-two scaling in the normal range.  So a group whose maximum lies
    where 448/amax overflows (or is a bf16 subnormal) must get exactly the
    codes of the same group scaled up into the range of ordinary magnitudes,
    which the encoder and closed-form pins above hold to the OCP definition;
    and its scale must be the float32 quotient of its own maximum by 448."""
    rng = np.random.default_rng(12)
    tiny = tiny_groups(rng, n_per=10)
    v = (tiny.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    amax = np.abs(v).max(axis=1)
    for target in (1.0, 2.0 ** 40, 2.0 ** -30):
        j = np.round(np.log2(target / amax)).astype(int)
        big = v * np.exp2(j)[:, None]                 # exact: bf16 values scaled up
        big_bits = _bf16(big.astype(np.float32))
        assert np.array_equal(((big_bits.astype(np.uint32) << 16).view(np.float32)), big), \
            "scaled group not exact in bf16"
        q_t, s_t = orc.quantize_rows(tiny)
        q_b, s_b = orc.quantize_rows(big_bits)
        np.testing.assert_array_equal(q_t, q_b)
        np.testing.assert_array_equal(s_t[:, 0], (amax / 448.0).astype(np.float32))
        np.testing.assert_array_equal(s_b[:, 0], (np.abs(big).max(axis=1) / 448.0)
                                      .astype(np.float32))
