"""Seeded synthetic workloads for MoE dispatch/combine.

This module only draws inputs: routing (topk_idx), gate weights, token rows and
stand-in expert outputs.  It holds none of the layout / dispatch / combine
arithmetic, so both the HIP path and the CPU oracle can take their inputs from
it.  bf16 values are produced by torch's float32 -> bfloat16 cast (round to
nearest even) and handed out as uint16 bit patterns.

Shapes follow the DeepSeek-V3 setting that the DeepEP analysis page
("DeepEP expert-parallel all-to-all communication", hotdry blog, section on the
core theoretical challenge of MoE communication) gives: 4096 tokens per batch,
hidden 7168, top-4 groups and top-8 experts; 256 routed experts per token
choice (Lesson 14 "DeepSeek DeepEP core architecture", section 1).

Draw order per workload: routing, then weight logits (if separate), then x.
Generator: numpy ``default_rng(1000 * config_id + seed)``.
"""
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    cid: int                 # configuration id (1..5)
    name: str
    N: int                   # tokens over all virtual source ranks
    H: int                   # hidden size
    E: int                   # routed experts
    K: int                   # top-k
    R: int                   # virtual EP ranks
    A: int                   # expert_alignment
    fp8: bool                # FP8 (e4m3) dispatch payload
    routing: str             # "uniform" | "group_limited" | "zipf"
    weights: str             # "softmax" | "sigmoid"
    groups: int = 8          # expert groups (group-limited routing)
    topk_groups: int = 4     # groups kept per token (group-limited routing)
    zipf_s: float = 1.2      # Zipf exponent (skewed routing)

    @property
    def desc(self):
        return (f"{self.name}: N={self.N} H={self.H} E={self.E} K={self.K} R={self.R} "
                f"A={self.A} {'e4m3' if self.fp8 else 'bf16'} routing={self.routing}")


CONFIGS = {
    1: Workload(1, "tiny", 128, 256, 16, 2, 4, 1, False, "uniform", "softmax"),
    2: Workload(2, "decode", 1024, 7168, 256, 8, 8, 1, False, "uniform", "softmax"),
    3: Workload(3, "prefill", 4096, 7168, 256, 8, 8, 128, False, "group_limited", "sigmoid"),
    4: Workload(4, "prefill_fp8", 4096, 7168, 256, 8, 8, 128, True, "group_limited", "sigmoid"),
    5: Workload(5, "skewed", 16384, 7168, 256, 8, 32, 128, False, "zipf", "softmax"),
}


def custom(N, H, E, K, R, A=1, fp8=False, routing="uniform", weights="softmax", cid=0,
           name="custom"):
    """A workload of arbitrary shape (tests: ragged tails, edge cases)."""
    return Workload(cid, name, N, H, E, K, R, A, fp8, routing, weights)


def _input_seed(w: Workload, seed: int) -> int:
    # config 4 draws exactly the inputs of config 3 (same routing, same x)
    cid = 3 if w.cid == 4 else w.cid
    return 1000 * cid + seed


def _softmax(z):
    z = z - z.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=1, keepdims=True)


def _bf16_bits(f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _routing(w: Workload, rng):
    N, E, K = w.N, w.E, w.K
    if w.routing == "uniform":
        idx = np.empty((N, K), np.int64)
        for t in range(N):
            idx[t] = rng.choice(E, K, replace=False)
        return idx, None
    if w.routing == "group_limited":
        G, TG = w.groups, w.topk_groups
        s = rng.standard_normal((N, E))
        gscore = s.reshape(N, G, E // G).max(axis=2)
        keep_g = np.argsort(-gscore, axis=1, kind="stable")[:, :TG]
        mask = np.zeros((N, G), bool)
        np.put_along_axis(mask, keep_g, True, axis=1)
        masked = np.where(np.repeat(mask, E // G, axis=1), s, -np.inf)
        idx = np.argsort(-masked, axis=1, kind="stable")[:, :K]
        return idx, np.take_along_axis(s, idx, axis=1)
    if w.routing == "zipf":
        perm = rng.permutation(E)
        p = np.arange(1, E + 1, dtype=np.float64) ** (-w.zipf_s)
        p /= p.sum()
        idx = np.empty((N, K), np.int64)
        for t in range(N):
            idx[t] = perm[rng.choice(E, K, replace=False, p=p)]
        return idx, None
    raise ValueError(w.routing)


def make_inputs(w: Workload, seed: int = 0):
    """Return dict(topk_idx int32 [N,K], topk_weights f32 [N,K], x uint16 [N,H])."""
    rng = np.random.default_rng(_input_seed(w, seed))
    idx, scores = _routing(w, rng)
    if w.weights == "softmax":
        logits = rng.standard_normal((w.N, w.K))
        wts = _softmax(logits)
    elif w.weights == "sigmoid":
        if scores is None:
            scores = rng.standard_normal((w.N, w.K))
        sig = 1.0 / (1.0 + np.exp(-scores))
        wts = sig / sig.sum(axis=1, keepdims=True)
    else:
        raise ValueError(w.weights)
    x = _bf16_bits(rng.standard_normal((w.N, w.H), dtype=np.float32))
    return dict(topk_idx=idx.astype(np.int32), topk_weights=wts.astype(np.float32), x=x)


def make_expert_out(w: Workload, rows: int, seed: int = 0, chunk_rows: int = 4096):
    """Stand-in expert outputs: bf16 bits of N(0,1), shape [rows, H].

    Drawn from its own stream so that the routing/x draws are unaffected.
    """
    rng = np.random.default_rng(_input_seed(w, seed) + 500_000)
    out = np.empty((rows, w.H), np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = _bf16_bits(rng.standard_normal((r1 - r0, w.H), dtype=np.float32))
    return out


def make_expert_out_device(w: Workload, rows: int, seed: int = 0, device="cuda"):
    """Stand-in expert outputs drawn on the GPU: bf16 N(0,1) [rows, H] from
    torch's seeded generator on ``device`` (a counter-based stream, so the
    same seed gives the same tensor on the same software stack).  Used where a
    host draw of hundreds of millions of values would take tens of seconds;
    callers that check against the oracle copy the tensor to the host."""
    g = torch.Generator(device=device)
    g.manual_seed(_input_seed(w, seed) + 700_000)
    out = torch.empty((rows, w.H), dtype=torch.bfloat16, device=device)
    step = 8192
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = torch.randn((r1 - r0, w.H), generator=g, device=device,
                                 dtype=torch.float32).to(torch.bfloat16)
    return out


def with_routing(w: Workload, **kw) -> Workload:
    return replace(w, **kw)
