"""Pins for the oracle's layout (counts, mask, padded offsets, slot order).

Each test checks the oracle against something other than itself: a worked
example derived by hand (golden file), the lesson-14 simulator's own end-to-end
assertion, a brute-force sort in pure Python, numpy's stable argsort, and the
invariants the method fixes (counts sum to N*K, order, bijection, alignment).
"""
import json
import os

import numpy as np
import pytest

from combine_ep_get_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lesson14_worked_example.json")


# --------------------------------------------------------------------------
def test_worked_example_golden(orc):
    g = json.load(open(GOLDEN))
    idx = np.array(g["topk_idx"], np.int32)
    for case in g["cases"]:
        out = orc.layout(idx, g["num_experts"], case["num_ranks"], case["expert_alignment"])
        assert out["error_flags"] == 0
        for key in ("num_recv_per_expert", "expert_slot_offset", "slot_of",
                    "num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank"):
            np.testing.assert_array_equal(out[key], np.array(case[key]), err_msg=key)
        cap = int(out["expert_slot_offset"][-1])
        src, _ = orc.recv_meta(out["slot_of"], np.ones(idx.shape, np.float32), cap)
        np.testing.assert_array_equal(src, np.array(case["recv_src_idx"]))


def test_lesson14_simulator_end_to_end(orc):
    """The practice task's own test, run through the oracle.

    Same seed, same draws, same routing as the page; experts are H x H matrices;
    the page's assertion is that combine equals the dense per-token reference
    sum_k w * (x @ W_e) within atol 1e-5, and that N*K rows were dispatched.
    """
    rs = np.random.RandomState(42)
    N, H, K, E = 4, 4, 2, 4
    tokens = rs.randn(N, H).astype(np.float32)
    topk_idx = np.array([[0, 2], [1, 3], [0, 3], [1, 2]], np.int32)
    raw = rs.uniform(0.1, 1.0, size=(N, K))
    topk_weights = (raw / raw.sum(axis=1, keepdims=True)).astype(np.float32)
    expert_w = {e: rs.randn(H, H).astype(np.float32) for e in range(E)}

    lay = orc.layout(topk_idx, E, 1, 1)
    assert int(lay["num_recv_per_expert"].sum()) == N * K
    cap = int(lay["expert_slot_offset"][-1])
    # dispatch is a bit copy of whole rows: move the float32 rows as pairs of 16-bit words
    recv = orc.dispatch_bf16(tokens.view(np.uint16), lay["slot_of"], cap).view(np.float32)
    off = lay["expert_slot_offset"]
    eo = np.zeros((cap, H), np.float32)
    for e in range(E):
        for s in range(off[e], off[e] + lay["num_recv_per_expert"][e]):
            eo[s] = np.matmul(recv[s], expert_w[e])
    _, acc = orc.combine(eo, lay["slot_of"], topk_weights)

    ref = np.zeros((N, H), np.float32)
    for i in range(N):
        for k in range(K):
            ref[i] += topk_weights[i, k] * np.matmul(tokens[i], expert_w[topk_idx[i, k]])
    assert np.allclose(acc, ref, atol=1e-5)


# --------------------------------------------------------------------------
def brute_force_layout(idx, E, R, A):
    """Pure-Python reference: sort (expert, source, token, k) tuples."""
    N, K = idx.shape
    T, L = N // R, E // R
    pairs = sorted((int(idx[t, k]), t // T, t, k) for t in range(N) for k in range(K)
                   if 0 <= idx[t, k] < E)
    slot_of = -np.ones((N, K), np.int64)
    counts = [0] * E
    for e, _, _, _ in pairs:
        counts[e] += 1
    off = [0]
    for e in range(E):
        off.append(off[-1] + -(-counts[e] // A) * A)
    pos = list(off[:-1])
    for e, _, t, k in pairs:
        slot_of[t, k] = pos[e]
        pos[e] += 1
    in_rank = np.zeros((N, R), np.int64)
    for t in range(N):
        for k in range(K):
            if 0 <= idx[t, k] < E:
                in_rank[t, idx[t, k] // L] = 1
    ntpr = np.zeros((R, R), np.int64)
    ntpe = np.zeros((R, E), np.int64)
    for t in range(N):
        ntpr[t // T] += in_rank[t]
        for k in range(K):
            if 0 <= idx[t, k] < E:
                ntpe[t // T, idx[t, k]] += 1
    return dict(slot_of=slot_of, num_recv_per_expert=np.array(counts),
                expert_slot_offset=np.array(off), is_token_in_rank=in_rank,
                num_tokens_per_rank=ntpr, num_tokens_per_expert=ntpe)


@pytest.mark.parametrize("trial", range(40))
def test_bruteforce_tiny(orc, trial):
    rng = np.random.default_rng(trial)
    R = int(rng.choice([1, 2, 4]))
    T = int(rng.integers(0, 5))
    N = R * T
    L = int(rng.integers(1, 4))
    E = R * L
    K = int(rng.integers(1, 6))
    A = int(rng.choice([1, 2, 3, 4, 8]))
    # duplicates allowed, and -1 entries ("no expert")
    idx = rng.integers(-1, E, size=(N, K)).astype(np.int32)
    out = orc.layout(idx, E, R, A)
    ref = brute_force_layout(idx, E, R, A)
    assert out["error_flags"] == 0
    for key, val in ref.items():
        np.testing.assert_array_equal(out[key], val, err_msg=f"{key} trial={trial}")


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_argsort_matches_slots(orc, cid):
    """With A=1, slot_of is the inverse of numpy's stable argsort of topk_idx."""
    w = wl.CONFIGS[cid]
    inp = wl.make_inputs(w, seed=0)
    idx = inp["topk_idx"]
    out = orc.layout(idx, w.E, w.R, 1)
    order = np.argsort(idx.reshape(-1), kind="stable")
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    np.testing.assert_array_equal(out["slot_of"].reshape(-1), inv)


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
@pytest.mark.parametrize("seed", [0, 1])
def test_invariants(orc, cid, seed):
    w = wl.CONFIGS[cid]
    inp = wl.make_inputs(w, seed=seed)
    idx = inp["topk_idx"]
    N, K, E, R, A = w.N, w.K, w.E, w.R, w.A
    T, L = N // R, E // R
    out = orc.layout(idx, E, R, A)
    assert out["error_flags"] == 0
    cnt = out["num_recv_per_expert"]
    off = out["expert_slot_offset"].astype(np.int64)
    slot = out["slot_of"]
    # counts: sum to N*K and agree with the per-source matrix
    assert cnt.sum() == N * K
    np.testing.assert_array_equal(out["num_tokens_per_expert"].sum(axis=0), cnt)
    np.testing.assert_array_equal(np.bincount(idx.reshape(-1), minlength=E), cnt)
    # alignment
    assert off[0] == 0 and np.all(off % A == 0)
    np.testing.assert_array_equal(np.diff(off), -(-cnt // A) * A)
    assert off[-1] <= orc.capacity(N, K, E, A)
    # bijection onto the valid slots and consistency with recv_src_idx
    cap = int(off[-1])
    src, _ = orc.recv_meta(slot, inp["topk_weights"], cap)
    flat = slot.reshape(-1)
    assert np.unique(flat).size == flat.size
    np.testing.assert_array_equal(src[flat], np.repeat(np.arange(N), K))
    # order: inside each region, valid prefix strictly increasing in token, then padding
    for e in range(E):
        reg = src[off[e]:off[e + 1]]
        valid = reg[:cnt[e]]
        assert np.all(np.diff(valid) > 0)
        assert np.all(np.diff(valid // T) >= 0)
        assert np.all(reg[cnt[e]:] == -1)
        assert (idx[valid] == e).any(axis=1).all()
    # mask
    ranks = idx // L
    m = np.zeros((N, R), np.uint8)
    np.put_along_axis(m, ranks, 1, axis=1)
    np.testing.assert_array_equal(out["is_token_in_rank"], m)
    per_tok = m.sum(axis=1)
    assert per_tok.min() >= 1 and per_tok.max() <= min(K, R)
    if w.routing == "group_limited":
        assert per_tok.max() <= w.topk_groups   # group == rank, 4 groups per token
    np.testing.assert_array_equal(out["num_tokens_per_rank"],
                                  m.reshape(R, T, R).sum(axis=1))


def test_out_of_range_index_sets_flag(orc):
    idx = np.array([[0, 5], [1, -3], [2, -1], [3, 0]], np.int32)
    out = orc.layout(idx, 4, 2, 1)
    assert out["error_flags"] == 1
    # bad entries and -1 get no slot and count nowhere
    assert out["slot_of"][0, 1] == -1 and out["slot_of"][1, 1] == -1 and out["slot_of"][2, 1] == -1
    assert out["num_recv_per_expert"].sum() == 5


def test_empty_and_invalid_sizes(orc):
    out = orc.layout(np.zeros((0, 8), np.int32), 16, 4, 8)
    assert np.all(out["expert_slot_offset"] == 0) and out["num_recv_per_expert"].sum() == 0
    with pytest.raises(ValueError):
        orc.layout(np.zeros((6, 2), np.int32), 16, 4, 1)   # N % R != 0
    with pytest.raises(ValueError):
        orc.layout(np.zeros((8, 2), np.int32), 6, 4, 1)    # E % R != 0
