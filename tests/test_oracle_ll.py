"""Pins for the oracle's low-latency layout (fixed (expert, source)
sub-blocks of M rows): hand-derived cases, a sort-based brute force, and the
relation to the compact layout, which is pinned on its own."""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ll_worked_example.json")


def test_ll_golden(orc):
    for case in json.load(open(GOLDEN))["cases"]:
        out = orc.ll_layout(np.array(case["topk_idx"], np.int32), case["num_experts"],
                            case["num_ranks"], case["max_tokens_per_rank"])
        np.testing.assert_array_equal(out["slot_of"], np.array(case["slot_of"]))
        np.testing.assert_array_equal(out["recv_count"], np.array(case["recv_count"]))
        np.testing.assert_array_equal(out["flags"], np.array(case["flags"]))


def brute_ll(idx, E, R, M):
    N, K = idx.shape
    T = N // R
    pairs = sorted((int(idx[t, k]), t // T, t, k) for t in range(N) for k in range(K)
                   if 0 <= idx[t, k] < E)
    slot = -np.ones((N, K), np.int64)
    count = np.zeros((E, R), np.int64)
    flags = np.zeros(R, np.int64)
    for t in range(N):
        for k in range(K):
            if not (-1 <= idx[t, k] < E):
                flags[t // T] |= 1
    j = {}
    for e, s, t, k in pairs:
        n = j.get((e, s), 0)
        j[(e, s)] = n + 1
        if n < M:
            slot[t, k] = (e * R + s) * M + n
            count[e, s] += 1
        else:
            flags[s] |= 2
    return slot, count, flags


@pytest.mark.parametrize("trial", range(30))
def test_ll_bruteforce(orc, trial):
    rng = np.random.default_rng(100 + trial)
    R = int(rng.choice([1, 2, 4]))
    T = int(rng.integers(0, 6))
    E = R * int(rng.integers(1, 4))
    K = int(rng.integers(1, 5))
    M = int(rng.integers(1, 5))
    idx = rng.integers(-2, E + 1, size=(R * T, K)).astype(np.int32)
    out = orc.ll_layout(idx, E, R, M)
    slot, count, flags = brute_ll(idx, E, R, M)
    np.testing.assert_array_equal(out["slot_of"], slot)
    np.testing.assert_array_equal(out["recv_count"], count)
    np.testing.assert_array_equal(out["flags"], flags)


@pytest.mark.parametrize("trial", range(10))
def test_ll_agrees_with_compact_layout(orc, trial):
    """Within expert e, source s's rows of the compact layout start at
    off[e] + sum_{s' < s} count[e][s'] and follow the same order."""
    rng = np.random.default_rng(200 + trial)
    R, E, K, T = 4, 16, 3, 12
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(R * T)]).astype(np.int32)
    M = T
    ll = orc.ll_layout(idx, E, R, M)
    cp = orc.layout(idx, E, R, 1)
    assert ll["error_flags"] == 0
    off = cp["expert_slot_offset"]
    before = np.concatenate([np.zeros((E, 1), np.int64),
                             np.cumsum(ll["recv_count"], axis=1)[:, :-1]], axis=1)
    for t in range(R * T):
        for k in range(K):
            e, s = idx[t, k], t // T
            j = ll["slot_of"][t, k] - (e * R + s) * M
            assert 0 <= j < M
            assert cp["slot_of"][t, k] - off[e] == before[e, s] + j
    np.testing.assert_array_equal(ll["recv_count"].sum(axis=1), cp["num_recv_per_expert"])
    np.testing.assert_array_equal(ll["recv_count"].T, cp["num_tokens_per_expert"])
