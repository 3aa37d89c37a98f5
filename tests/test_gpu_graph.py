"""The three entry points only enqueue kernels, so one step can be captured
into a HIP graph and replayed.  The captured graph is replayed several times
with different routing and token rows copied into its input buffers between
replays (ordinary eager work and synchronisations in between), and every
replay must equal the eager result for those inputs bit for bit."""
import numpy as np
import pytest
import torch

import combine_ep_get_amd as ep
from combine_ep_get_amd import workloads as wl

from .gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu


def _snapshot(lay, recv, y):
    torch.cuda.synchronize()
    out = [lay.slot_of.clone(), lay.expert_slot_offset.clone(), lay.num_recv_per_expert.clone(),
           lay.is_token_in_rank.clone(), lay.num_tokens_per_rank.clone(),
           lay.num_tokens_per_expert.clone(), recv[2].clone(), recv[3].clone(),
           y.view(torch.int16).clone()]
    # payload rows (and scale rows) that hold a pair; padding rows keep
    # whatever earlier calls left there, by contract
    valid = (recv[2] >= 0).nonzero().flatten()
    out.append(recv[0].view(torch.uint8).index_select(0, valid))
    if recv[1] is not None:
        out.append(recv[1].index_select(0, valid))
    return out


@pytest.mark.parametrize("cid", [2, 4])
def test_graph_replay_matches_eager(cid):
    w = wl.CONFIGS[cid]
    say(f"graph replay {w.desc}")
    sets = [wl.make_inputs(w, seed) for seed in (0, 1)]
    dev = torch.device("cuda")
    idx = torch.from_numpy(sets[0]["topk_idx"]).to(dev)
    wts = torch.from_numpy(sets[0]["topk_weights"]).to(dev)
    x = dev_bf16(sets[0]["x"])
    cap = ep.recv_capacity(w.N, w.K, w.E, w.R, w.A)
    eo = dev_bf16(wl.make_expert_out(w, cap, seed=0))
    lay = ep.alloc_layout(w.N, w.K, w.E, w.R, w.A, dev)
    recv = ep.alloc_recv(lay, w.H, w.fp8, dev)
    y = torch.empty((w.N, w.H), dtype=torch.bfloat16, device=dev)

    def load(i):
        idx.copy_(torch.from_numpy(sets[i]["topk_idx"]))
        wts.copy_(torch.from_numpy(sets[i]["topk_weights"]))
        x.copy_(dev_bf16(sets[i]["x"]))
        recv[0].view(torch.uint8).fill_(0)
        recv[2].fill_(-7)
        torch.cuda.synchronize()

    def step():
        ep.get_layout(idx, w.E, w.R, w.A, out=lay)
        ep.dispatch(x, wts, lay, w.fp8, out=recv)
        ep.combine(eo, lay, wts, out=y)

    expected = []
    for i in (0, 1):
        load(i)
        step()
        expected.append(_snapshot(lay, recv, y))

    load(0)
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            step()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()

    for i in (1, 0, 1, 0, 1):
        load(i)
        g.replay()
        got = _snapshot(lay, recv, y)
        for a, b in zip(got, expected[i]):
            assert torch.equal(a, b)


@pytest.mark.parametrize("budget", [0, 48])
def test_graph_replay_with_options(budget):
    """int64 routing, zero padding, running statistics and a CU budget inside
    a captured step: every replay equals the eager step, and the statistics
    grow by the per-expert counts once per replay."""
    w = wl.CONFIGS[3]
    say(f"graph replay with options {w.desc} budget={budget}")
    sets = [wl.make_inputs(w, seed) for seed in (0, 1)]
    dev = torch.device("cuda")
    idx = torch.from_numpy(sets[0]["topk_idx"].astype(np.int64)).to(dev)
    wts = torch.from_numpy(sets[0]["topk_weights"]).to(dev)
    x = dev_bf16(sets[0]["x"])
    cap = ep.recv_capacity(w.N, w.K, w.E, w.R, w.A)
    eo = dev_bf16(wl.make_expert_out(w, cap, seed=0))
    lay = ep.alloc_layout(w.N, w.K, w.E, w.R, w.A, dev)
    recv = ep.alloc_recv(lay, w.H, False, dev)
    y = torch.empty((w.N, w.H), dtype=torch.bfloat16, device=dev)
    stats = torch.zeros(w.E, dtype=torch.int64, device=dev)

    def load(i):
        idx.copy_(torch.from_numpy(sets[i]["topk_idx"].astype(np.int64)))
        wts.copy_(torch.from_numpy(sets[i]["topk_weights"]))
        x.copy_(dev_bf16(sets[i]["x"]))
        recv[0].view(torch.uint8).fill_(0x77)
        recv[2].fill_(-7)
        torch.cuda.synchronize()

    def step():
        ep.get_layout(idx, w.E, w.R, w.A, out=lay)
        ep.dispatch(x, wts, lay, False, out=recv, zero_padding=True, cumulative_stats=stats,
                    cu_budget=budget)
        ep.combine(eo, lay, wts, out=y, cu_budget=budget)

    def snap():
        torch.cuda.synchronize()
        return [lay.slot_of.clone(), lay.expert_slot_offset.clone(), recv[2].clone(),
                recv[3].clone(), y.view(torch.int16).clone(),
                recv[0].view(torch.uint8)[: int(lay.expert_slot_offset[-1])].clone()]

    expected, counts = [], []
    for i in (0, 1):
        load(i)
        step()
        expected.append(snap())
        counts.append(lay.num_recv_per_expert.to(torch.int64).clone())

    load(0)
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            step()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()

    stats.zero_()
    want = torch.zeros_like(stats)
    for i in (1, 0, 1, 1, 0):
        load(i)
        g.replay()
        got = snap()
        for a, b in zip(got, expected[i]):
            assert torch.equal(a, b)
        want += counts[i]
        assert torch.equal(stats, want)
