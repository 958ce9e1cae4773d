"""ctypes binding of the seeded input generator's device twin (synth/libsynthfill.so).

Input preparation only.  The 65536-entry quantile table is built on the host
(synth.philox.normal_table) and copied to each device once.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynthfill.so")
_lib = None
_tables = {}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m streaming_kv_cache_block_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.synth_fill_normal_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint32,
                                             ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p]
        L.synth_fill_normal_bf16.restype = ctypes.c_int
        _lib = L
    return _lib


def _table(device):
    import torch
    from . import philox
    dev = torch.device(device)
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    if dev not in _tables:
        _tables[dev] = torch.from_numpy(philox.normal_table().copy()).to(dev)
    return _tables[dev]


def fill_normal_bf16(shape, sigma, key64, device="cuda"):
    """torch.bfloat16 tensor of the generator's N(0, sigma^2) draws for key64, made on the
    device on torch's current stream."""
    import torch
    t = torch.empty(shape, dtype=torch.bfloat16, device=device)
    table = _table(device)
    err = lib().synth_fill_normal_bf16(t.data_ptr(), t.numel(), key64 & 0xFFFFFFFF, key64 >> 32, table.data_ptr(),
                                       float(sigma), torch.cuda.current_stream(t.device).cuda_stream)
    if err != 0:
        raise RuntimeError(f"synth_fill_normal_bf16 failed with HIP error {err}")
    return t
