"""The library called from plain C (tests/c/abi_gpu_example.c, built by
__graft_entry__.build()): hipMalloc'd buffers, no Python or torch in the call
path.  Its outputs are compared with the oracle: layout, receive rows and tags
bit-exact, combine bit-exact."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from combine_ep_get_amd import workloads as wl

from .gpu_util import check_combine, say

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "_build", "abi_gpu_example")

CASES = [wl.CONFIGS[1],
         wl.custom(N=96, H=1024, E=24, K=5, R=3, A=8, fp8=True, name="c_fp8"),
         wl.custom(N=60, H=136, E=12, K=3, R=3, A=16, name="c_ragged")]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_plain_c_caller(tmp_path, w):
    assert os.path.exists(EXE), "build the C caller first (__graft_entry__.build())"
    say(f"plain C caller {w.desc}")
    inp = wl.make_inputs(w, 3)
    cap = oracle.capacity(w.N, w.K, w.E, w.A)
    eo = wl.make_expert_out(w, cap, 3)
    d = str(tmp_path)
    open(os.path.join(d, "problem.txt"), "w").write(
        f"{w.N} {w.H} {w.K} {w.E} {w.R} {w.A} {int(w.fp8)}\n")
    inp["topk_idx"].astype(np.int32).tofile(os.path.join(d, "topk_idx.bin"))
    inp["topk_weights"].astype(np.float32).tofile(os.path.join(d, "topk_weights.bin"))
    inp["x"].tofile(os.path.join(d, "x.bin"))
    eo.tofile(os.path.join(d, "expert_out.bin"))
    r = subprocess.run([EXE, d], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    say("  " + r.stdout.strip())

    def load(name, dt, shape):
        return np.fromfile(os.path.join(d, name), dtype=dt).reshape(shape)

    ref = oracle.layout(inp["topk_idx"], w.E, w.R, w.A)
    np.testing.assert_array_equal(load("slot_of.bin", np.int32, (w.N, w.K)), ref["slot_of"])
    np.testing.assert_array_equal(load("offsets.bin", np.int32, (w.E + 1,)),
                                  ref["expert_slot_offset"])
    np.testing.assert_array_equal(load("counts.bin", np.int32, (w.E,)),
                                  ref["num_recv_per_expert"])
    src, _ = oracle.recv_meta(ref["slot_of"], inp["topk_weights"], cap)
    np.testing.assert_array_equal(load("recv_src_idx.bin", np.int32, (cap,)), src)
    valid = src >= 0
    if w.fp8:
        q, sc = oracle.dispatch_fp8(inp["x"], ref["slot_of"], cap)
        np.testing.assert_array_equal(load("recv_x.bin", np.uint8, (cap, w.H))[valid], q[valid])
        got_sc = load("recv_scales.bin", np.float32, (cap, w.H // 128))
        np.testing.assert_array_equal(got_sc[valid].view(np.uint32), sc[valid].view(np.uint32))
    else:
        rx = oracle.dispatch_bf16(inp["x"], ref["slot_of"], cap)
        np.testing.assert_array_equal(load("recv_x.bin", np.uint16, (cap, w.H))[valid], rx[valid])
    ref_y, ref_acc = oracle.combine(eo, ref["slot_of"], inp["topk_weights"])
    assert check_combine(load("y.bin", np.uint16, (w.N, w.H)), ref_y, ref_acc) == 0
