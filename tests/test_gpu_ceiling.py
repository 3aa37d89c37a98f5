"""The HBM ceiling kernels that the benchmark times beside the EP kernels move
the bytes they claim to: every scatter form writes each token row to exactly
the rows its map names, and the gather writes the XOR of the K mapped rows.
A ceiling kernel that skipped part of its traffic would report a rate no
kernel can reach."""
import ctypes
import os

import numpy as np
import pytest
import torch

from .gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    lib = ctypes.CDLL(os.path.join(ROOT, "combine_ep_get_amd", "_lib", "libepceil.so"))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    for name in ("epc_scatter", "epc_scatter_items", "epc_scatter_pieces", "epc_gather"):
        getattr(lib, name).argtypes = [vp, vp, vp, i32, i32, i64, vp]
    return lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("H", [64, 2088, 7168])
def test_scatter_forms_write_the_mapped_rows(H):
    rng = np.random.default_rng(H)
    N, K, rows = 96, 6, 700
    perm = rng.permutation(rows)[:N * K].reshape(N, K).astype(np.int32)
    perm[rng.random((N, K)) < 0.1] = -1
    lib = _lib()
    x = torch.from_numpy(rng.integers(0, 1 << 15, size=(N, H), dtype=np.int16)).cuda()
    want = np.full((rows, H), -1, np.int16)
    xs = x.cpu().numpy()
    for t in range(N):
        for k in range(K):
            if perm[t, k] >= 0:
                want[perm[t, k]] = xs[t]
    m = torch.from_numpy(perm).cuda()
    for name in ("epc_scatter", "epc_scatter_items", "epc_scatter_pieces"):
        say(f"ceiling {name} H={H}")
        dst = torch.full((rows, H), -1, dtype=torch.int16, device="cuda")
        rc = getattr(lib, name)(x.data_ptr(), dst.data_ptr(), m.data_ptr(), N, K, 2 * H, _stream())
        assert rc == 0
        torch.cuda.synchronize()
        np.testing.assert_array_equal(dst.cpu().numpy(), want, err_msg=name)


def test_gather_writes_the_xor_of_the_mapped_rows():
    rng = np.random.default_rng(5)
    N, K, rows, H = 64, 8, 300, 7168
    m = rng.integers(-1, rows, size=(N, K)).astype(np.int32)
    src = rng.integers(0, 1 << 15, size=(rows, H), dtype=np.int16)
    want = np.zeros((N, H), np.int16)
    for t in range(N):
        for k in range(K):
            want[t] ^= src[max(m[t, k], 0)]     # -1 is read as row 0
    out = torch.zeros((N, H), dtype=torch.int16, device="cuda")
    s = torch.from_numpy(src).cuda()
    md = torch.from_numpy(m).cuda()
    say("ceiling epc_gather")
    assert _lib().epc_gather(s.data_ptr(), out.data_ptr(), md.data_ptr(), N, K, 2 * H, _stream()) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), want)
