"""The float32 -> OCP E4M3 conversion instruction that the fused-quantisation
dispatch kernels use for every scaled value (v_cvt_pk_fp8_f32 on gfx950)
against the oracle's encoder, on every float32 whose magnitude is below 464:
both signs, zeros and subnormals included, 2,278,555,648 inputs compared code
by code.  The kernels only feed it values of magnitude at most
448 (1 + 2^-23), so this covers every input they can produce.
"""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle

from .gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tests", "c", "_build", "libcvtsweep.so")
LIMIT = 0x43E80000          # float32 bit pattern of 464.0
CHUNK = 1 << 26             # inputs per launch
PIECE = 1 << 22             # inputs per oracle call (spread over threads)


def _oracle_codes(first, n):
    bits = np.arange(first, first + n, dtype=np.uint64).astype(np.uint32)
    return oracle.f32_to_e4m3(bits.view(np.float32))


def test_cvt_e4m3_equals_oracle_encoder_below_464():
    L = ctypes.CDLL(LIB)
    L.cvt_e4m3_sweep.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_void_p]
    L.cvt_e4m3_sweep.restype = ctypes.c_int
    oracle.lib()
    out = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    workers = max(1, min(16, os.cpu_count() or 1))
    total = 0
    with ThreadPoolExecutor(workers) as pool:
        for sign in (0x00000000, 0x80000000):
            for first in range(0, LIMIT, CHUNK):
                n = min(CHUNK, LIMIT - first)
                base = sign | first
                assert L.cvt_e4m3_sweep(base, n, out.data_ptr(), st) == 0
                futs = [pool.submit(_oracle_codes, base + a, min(PIECE, n - a))
                        for a in range(0, n, PIECE)]
                got = out[:n].cpu().numpy()
                ref = np.concatenate([f.result() for f in futs])
                bad = np.nonzero(got != ref)[0]
                assert bad.size == 0, (f"{bad.size} codes differ from the oracle; first at "
                                       f"float32 bits {base + int(bad[0]):#010x}: "
                                       f"gpu {got[bad[0]]:#04x} oracle {ref[bad[0]]:#04x}")
                total += n
            say(f"  sign {sign >> 31}: every input below 464 matches")
    assert total == 2 * LIMIT
