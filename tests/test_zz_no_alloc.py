"""ep_get_layout_noalloc (the layout with the library's static scratch as its
workspace, for callers that cannot allocate) against ep_get_layout, through
the C ABI: two calls in a row on the same outputs, the second with a smaller
input, both large enough for the two-launch layout that uses the scratch's
per-block histograms; then a decode-sized call (single-launch layout).  Every
output must be bit-identical to ep_get_layout's on the same input, and the
error word must match ep_layout_error's."""
import numpy as np
import pytest
import torch

import combine_ep_get_amd as ep

from .gpu_util import say

pytestmark = pytest.mark.gpu

FIELDS = ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
          "num_recv_per_expert", "expert_slot_offset", "slot_of")


def _routing(rng, N, K, E, bad=False):
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(N)]).astype(np.int32)
    if bad:
        idx[N // 3, 1] = E + 5          # out of range: skipped, error bit set
        idx[N // 2, 0] = -1             # no expert
    return idx


def test_noalloc_layout_matches_layout():
    rng = np.random.default_rng(2024)
    E, R, A, K = 256, 8, 128, 8
    err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    for N, bad in ((16384, False), (8192, True), (1024, True)):
        say(f"noalloc layout N={N} K={K} E={E} R={R} A={A} bad={bad}")
        idx = torch.from_numpy(_routing(rng, N, K, E, bad)).cuda()
        want = ep.get_layout(idx, E, R, A)
        got = ep.alloc_layout(N, K, E, R, A)
        for f in FIELDS:
            getattr(got, f).fill_(-3)
        ep.get_layout_noalloc(idx, got, error_word=err)
        torch.cuda.synchronize()
        for f in FIELDS:
            assert torch.equal(getattr(got, f), getattr(want, f)), f"N={N}: {f} differs"
        assert int(err.item()) == ep.layout_error(want) == (1 if bad else 0)
        # again on the same outputs, without the error word
        ep.get_layout_noalloc(idx, got)
        torch.cuda.synchronize()
        for f in FIELDS:
            assert torch.equal(getattr(got, f), getattr(want, f)), f"N={N} (repeat): {f} differs"
