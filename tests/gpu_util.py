"""Shared helpers for the GPU tests: move seeded inputs to the device, run the
three entry points through the C ABI, and compare with the oracle."""
import os
import sys

import numpy as np
import torch

import combine_ep_get_amd as ep


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def ulp_dist_bf16(a, b):
    def key(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + u)
    return np.abs(key(a) - key(b))


def check_layout(lay, ref):
    torch.cuda.synchronize()
    pairs = [("num_tokens_per_rank", lay.num_tokens_per_rank),
             ("num_tokens_per_expert", lay.num_tokens_per_expert),
             ("is_token_in_rank", lay.is_token_in_rank),
             ("num_recv_per_expert", lay.num_recv_per_expert),
             ("expert_slot_offset", lay.expert_slot_offset),
             ("slot_of", lay.slot_of)]
    for name, t in pairs:
        got = t.cpu().numpy()
        np.testing.assert_array_equal(got, ref[name], err_msg=name)
    assert ep.layout_error(lay) == ref["error_flags"]


def check_combine(y_bits, ref_y, ref_acc):
    """Bit-exact expected; the contract's tolerance is asserted regardless:
    |y - acc| <= 2^-8 |acc| or <= 1e-3, and at most 1 bf16 ulp from the oracle."""
    y = torch.from_numpy(y_bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    err = np.abs(y.astype(np.float64) - ref_acc.astype(np.float64))
    ok = (err <= 2.0 ** -8 * np.abs(ref_acc)) | (err <= 1e-3)
    assert ok.all(), f"{(~ok).sum()} elements outside tolerance"
    d = ulp_dist_bf16(y_bits, ref_y)
    assert d.size == 0 or d.max() <= 1
    return int((d != 0).sum())


def oracle_threads():
    """Threads for the oracle's threaded driver: the CPUs this process may use,
    at most 16 (a GPU machine's CPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))
