"""The MFMA ceiling loops (libllceiling.so) do the work the bench credits them with.

The bench prices each launch at blocks x 4 waves x 4 iters MFMAs of 32x32x16.  The sum
of every output element of one such MFMA is sum_k (sum_m A[m,k]) (sum_n B[k,n]); the lanes
with the same lane // 32 hold the same k range of A and of B, in the same order, so the
total over all lanes of the kernel's outputs is fixed by the operands alone and by how
many MFMAs ran on which pair.  A wrong iteration count, a dropped accumulator or a
different pair order moves it.
"""

import ctypes

import numpy as np
import pytest

import bench
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _lib():
    L = ctypes.CDLL(bench.CEILING_LIB)
    L.llc_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.llc_mfma_loop_data.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return L


def _pair_total(A, B):
    """Sum of all outputs of one 32x32x16 MFMA per wave, summed over the 4 waves.
    A, B: [256 lanes][8] float64 fragments."""
    tot = 0.0
    for w in range(4):
        for h in range(2):
            lanes = slice(64 * w + 32 * h, 64 * w + 32 * h + 32)
            tot += float(np.dot(A[lanes].sum(axis=0), B[lanes].sum(axis=0)))
    return tot


def test_low_bit_loop_total(torch_gpu):
    torch = torch_gpu
    blocks, iters = 3, 8
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    assert _lib().llc_mfma_loop(out.data_ptr(), blocks, iters, None) == 0
    torch.cuda.synchronize()
    t = np.arange(256)[:, None]
    i = np.arange(8)[None, :]
    a = ((t + i) & 7) * 0.125
    b = ((t * 3 + i) & 7) * 0.0625
    want = blocks * iters * (_pair_total(a, b) + _pair_total(b, a) + _pair_total(a, a) + _pair_total(b, b))
    got = float(out.double().sum().item())
    print(f"low-bit loop: total {got} against {want}", flush=True)
    assert got == want          # multiples of 2^-7 far below 2^24 ulps: exact in fp32


def test_data_operand_loop_total(torch_gpu):
    """The operand-buffer form on random small integers (exact in bf16, and every partial
    sum exact in fp32), so the total must match to the last bit."""
    torch = torch_gpu
    blocks, iters = 2, 8
    vals = np.random.default_rng(978).integers(-8, 9, size=256 * 64).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)          # exact: small integers
    data = synth.to_device(bits)
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    assert _lib().llc_mfma_loop_data(out.data_ptr(), data.data_ptr(), blocks, iters, None) == 0
    torch.cuda.synchronize()
    f = vals.astype(np.float64).reshape(256, 8, 8)                   # [lane][fragment][8]
    pairs = [(0, 4), (1, 5), (2, 6), (3, 7), (1, 6), (2, 7), (3, 4), (0, 5),
             (2, 5), (3, 6), (0, 7), (1, 4), (3, 7), (0, 4), (1, 5), (2, 6)]
    per_pair = [_pair_total(f[:, x], f[:, y]) for x, y in pairs]
    want = blocks * (iters // 4) * sum(per_pair)
    got = float(out.double().sum().item())
    print(f"operand-buffer loop: total {got} against {want}; pair totals {per_pair}", flush=True)
    assert got == want
