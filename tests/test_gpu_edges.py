"""GPU edge cases against the oracle, each compared in full: empty and ragged
inputs, minimum / multi-pass hidden sizes, K=1 and K=32, one expert per rank,
everything routed to one expert, alignment above N, -1 entries, duplicate
experts in a row, out-of-range indices (error flag), many ranks, the largest
expert count, chunking with ragged tails; and an exhaustive on-device check of
the fused E4M3 quantiser over every finite bf16 value."""
import numpy as np
import pytest
import torch

import combine_ep_get_amd as ep
import oracle

from .gpu_util import check_combine, check_layout, dev_bf16, host_u16, host_u8, say

pytestmark = pytest.mark.gpu


def run_case(idx, H, E, R, A, fp8=False, seed=0, x_bits=None):
    idx = np.ascontiguousarray(idx, np.int32)
    N, K = idx.shape
    rng = np.random.default_rng(seed)
    if x_bits is None:
        x_bits = torch.from_numpy(rng.standard_normal((N, H), dtype=np.float32)) \
            .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    wts = rng.random((N, K), dtype=np.float32)
    say(f"case N={N} H={H} E={E} K={K} R={R} A={A} fp8={fp8}")
    lay = ep.get_layout(torch.from_numpy(idx).cuda(), E, R, A)
    ref = oracle.layout(idx, E, R, A)
    check_layout(lay, ref)
    cap = lay.capacity
    out = ep.alloc_recv(lay, H, fp8)
    out[0].view(torch.uint8).fill_(0x55)
    out[2].fill_(-7)
    out[3].fill_(-7.0)
    if fp8:
        out[1].fill_(-7.0)
    x = dev_bf16(x_bits)
    w_dev = torch.from_numpy(wts).cuda()
    recv_x, sc, src, rw = ep.dispatch(x, w_dev, lay, fp8, out=out)
    torch.cuda.synchronize()
    ref_src, ref_w = oracle.recv_meta(ref["slot_of"], wts, cap)
    np.testing.assert_array_equal(src.cpu().numpy(), ref_src)
    np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), ref_w.view(np.uint32))
    valid = ref_src >= 0
    if fp8:
        q_ref, sc_ref = oracle.dispatch_fp8(x_bits, ref["slot_of"], cap)
        got = host_u8(recv_x)
        np.testing.assert_array_equal(got[valid], q_ref[valid])
        assert np.all(got[~valid] == 0x55)
        gsc = sc.cpu().numpy()
        np.testing.assert_array_equal(gsc[valid].view(np.uint32), sc_ref[valid].view(np.uint32))
        assert np.all(gsc[~valid] == -7.0)
    else:
        r_ref = oracle.dispatch_bf16(x_bits, ref["slot_of"], cap)
        got = host_u16(recv_x)
        np.testing.assert_array_equal(got[valid], r_ref[valid])
        assert np.all(got[~valid] == 0x5555)
    eo_bits = torch.from_numpy(rng.standard_normal((cap, H), dtype=np.float32)) \
        .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    y = ep.combine(dev_bf16(eo_bits), lay, w_dev)
    torch.cuda.synchronize()
    ref_y, ref_acc = oracle.combine(eo_bits, ref["slot_of"], wts)
    assert check_combine(host_u16(y), ref_y, ref_acc) == 0
    return lay


def distinct(rng, N, K, E):
    return np.stack([rng.choice(E, K, replace=False) for _ in range(N)]) if N else \
        np.zeros((0, K), np.int32)


def test_empty():
    lay = run_case(np.zeros((0, 2), np.int32), H=64, E=16, R=4, A=8)
    assert int(lay.expert_slot_offset[-1]) == 0


def test_one_token_per_rank():
    run_case(distinct(np.random.default_rng(1), 8, 4, 64), H=256, E=64, R=8, A=4)


def test_k1_and_all_to_one_expert():
    N = 256
    run_case(np.full((N, 1), 5, np.int32), H=128, E=32, R=4, A=16)
    rng = np.random.default_rng(2)
    idx = distinct(rng, N, 4, 32)
    idx[~(idx == 0).any(axis=1), 0] = 0        # expert 0 in every row, still distinct
    run_case(idx, H=128, E=32, R=4, A=16)


def test_one_expert_per_rank_and_alignment_above_n():
    rng = np.random.default_rng(3)
    run_case(distinct(rng, 64, 3, 8), H=64, E=8, R=8, A=1)
    run_case(distinct(rng, 16, 2, 8), H=64, E=8, R=4, A=64)


@pytest.mark.parametrize("H", [8, 136, 7176, 16392])
def test_ragged_and_multipass_hidden_bf16(H):
    run_case(distinct(np.random.default_rng(H), 96, 4, 32), H=H, E=32, R=4, A=8)


@pytest.mark.parametrize("K", [1, 3, 6, 9, 13])
def test_topk_not_a_multiple_of_the_piece_wavefronts(K):
    # bf16 rows move as 2 KiB pieces whose slots are shared round robin by the
    # wavefronts of a workgroup: K above, below and not a multiple of their
    # number, with a ragged last piece (H = 2088: pieces of 128, 128, 5 chunks)
    run_case(distinct(np.random.default_rng(K), 80, K, 64), H=2088, E=64, R=4, A=4)


@pytest.mark.parametrize("H", [128, 1152, 16384])
def test_hidden_sizes_fp8(H):
    run_case(distinct(np.random.default_rng(H), 64, 4, 32), H=H, E=32, R=4, A=8, fp8=True)


def test_minus_one_and_duplicates():
    rng = np.random.default_rng(4)
    idx = rng.integers(-1, 12, size=(120, 6)).astype(np.int32)   # duplicates and -1 allowed
    run_case(idx, H=72, E=12, R=3, A=5)
    run_case(idx, H=256, E=12, R=3, A=5, fp8=True)


def test_out_of_range_indices_set_the_error_word():
    rng = np.random.default_rng(5)
    idx = distinct(rng, 64, 4, 16).astype(np.int32)
    idx[3, 1] = 16
    idx[40, 0] = -5
    lay = run_case(idx, H=64, E=16, R=4, A=1)
    assert ep.layout_error(lay) == ep.EP_LAYOUT_ERR_INDEX
    # the next clean layout into the same workspace clears the word
    ep.get_layout(torch.from_numpy(distinct(rng, 64, 4, 16).astype(np.int32)).cuda(), 16, 4, 1,
                  out=lay)
    assert ep.layout_error(lay) == 0


def test_k32_many_ranks_and_max_experts():
    rng = np.random.default_rng(6)
    run_case(distinct(rng, 256, 32, 256), H=64, E=256, R=256, A=2)
    run_case(distinct(rng, 512, 8, 1024), H=64, E=1024, R=8, A=32)


@pytest.mark.parametrize("N", [4096, 4104])
def test_layout_paths_at_the_single_launch_threshold(N):
    # 32768 pairs take the single-launch layout, 32832 the two-launch one
    rng = np.random.default_rng(N)
    run_case(rng.integers(-1, 256, size=(N, 8)).astype(np.int32), H=8, E=256, R=8, A=128)


def test_ragged_chunks_and_large_n():
    rng = np.random.default_rng(7)
    # T = 100 tokens per source: chunks of 64 + 36
    run_case(distinct(rng, 400, 8, 64), H=64, E=64, R=4, A=16)
    # N above 512 * 64: chunk grows past 512 / K tokens
    idx = rng.integers(0, 256, size=(65536, 8)).astype(np.int32)
    run_case(idx, H=8, E=256, R=8, A=128)


# bf16 group maxima: ordinary scale factors (exactly 1 among them), and the
# ones where the float32 inverse 448/amax overflows or only just does not --
# the smallest bf16 subnormal (2^-133), a mid-range subnormal, the smallest
# normal (2^-126), about 1e-37 and the two bf16 values around 448/FLT_MAX.
QUANT_MAXIMA_F32 = (448.0, 1.0, 3.0, 0.7109375, 1e-3, 65504.0, 3.0e38, 1e-30)
QUANT_MAXIMA_BITS = (0x0001, 0x0015, 0x0080, 0x0208, 0x03E0, 0x03E1)


def test_fp8_quantiser_exhaustive_on_device():
    """Every finite bf16 value is quantised by the fused dispatch kernel for
    several group maxima (so several scale factors, including exactly 1 and
    the tiny maxima whose inverse overflows float32; every group also holds
    +0 and -0) and the codes and scales are compared with the oracle bit for
    bit."""
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(allv)
    finite = allv[np.isfinite(f)]
    rows = []
    maxima = [torch.tensor([m], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy()
              .view(np.uint16)[0] for m in QUANT_MAXIMA_F32] + \
        [np.uint16(b) for b in QUANT_MAXIMA_BITS]
    for mbits in maxima:
        mval = oracle.bf16_to_f32(np.array([mbits]))[0]
        vals = finite[np.abs(oracle.bf16_to_f32(finite)) <= mval]
        n = -(-vals.size // 127)
        pad = np.concatenate([vals, np.zeros(n * 127 - vals.size, np.uint16)]).reshape(n, 127)
        rows.append(np.concatenate([np.full((n, 1), mbits, np.uint16), pad], axis=1))
    # all-zero and signed-zero groups
    rows.append(np.zeros((1, 128), np.uint16))
    rows.append(np.full((1, 128), 0x8000, np.uint16))
    g = np.concatenate(rows)                                   # [groups, 128]
    ng = g.shape[0]
    G = 8                                                      # 8 groups per token (H = 1024)
    ntok = -(-ng // G)
    ntok = -(-ntok // 4) * 4
    xb = np.zeros((ntok * G, 128), np.uint16)
    xb[:ng] = g
    x_bits = xb.reshape(ntok, G * 128)
    idx = np.arange(ntok, dtype=np.int32).reshape(ntok, 1) % 16
    say(f"quantiser exhaustive: {ng} groups in {ntok} tokens")
    run_case(idx, H=G * 128, E=16, R=4, A=1, fp8=True, x_bits=x_bits)


def test_combine_bf16_rounding_at_ties_on_device():
    """The bf16 store of combine rounds to nearest even: for every normal bf16
    value a (exponent field 9..246, both signs) the second pair adds b = half
    an ulp of a (an exact tie), a little more, or a little less, with either
    sign; a + b is exact in fp32, so the stored bf16 is decided by the
    rounding rule alone.  Compared bit for bit with the oracle."""
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ex = (allv >> 7) & 0xFF
    a = allv[(ex >= 9) & (ex <= 246)]
    ea = ((a >> 7) & 0xFF).astype(np.int64)
    sign = (a & 0x8000).astype(np.uint16)

    def bf16_pow2(e):                      # bf16 bits of 2^(e - 127)
        return (e << 7).astype(np.uint16)

    half = bf16_pow2(ea - 8)                               # exact tie
    above = (bf16_pow2(ea - 8) | 0x01).astype(np.uint16)   # 2^(e-8) (1 + 2^-7)
    below = (bf16_pow2(ea - 9) | 0x7F).astype(np.uint16)   # 2^(e-8) - 2^(e-16)
    pairs_a, pairs_b = [], []
    for bb in (half, above, below):
        for same in (True, False):
            pairs_a.append(a)
            pairs_b.append(bb | (sign if same else (sign ^ 0x8000)))
    va = np.concatenate(pairs_a)
    vb = np.concatenate(pairs_b)
    H, R, E = 1024, 4, 8
    n = -(-va.size // H)
    n = -(-n // R) * R
    A_rows = np.zeros(n * H, np.uint16)
    B_rows = np.zeros(n * H, np.uint16)
    A_rows[:va.size] = va
    B_rows[:vb.size] = vb
    idx = np.stack([np.arange(n) % E, (np.arange(n) + 1) % E], axis=1).astype(np.int32)
    ref = oracle.layout(idx, E, R, 1)
    cap = ep.recv_capacity(n, 2, E, R, 1)
    eo = np.zeros((cap, H), np.uint16)
    eo[ref["slot_of"][:, 0]] = A_rows.reshape(n, H)
    eo[ref["slot_of"][:, 1]] = B_rows.reshape(n, H)
    wts = np.ones((n, 2), np.float32)
    say(f"bf16 rounding: {va.size} tie / near-tie sums in {n} tokens")
    lay = ep.get_layout(torch.from_numpy(idx).cuda(), E, R, 1)
    y = ep.combine(dev_bf16(eo), lay, torch.from_numpy(wts).cuda())
    torch.cuda.synchronize()
    ref_y, _ = oracle.combine(eo, ref["slot_of"], wts)
    got = host_u16(y)
    np.testing.assert_array_equal(got, ref_y)
