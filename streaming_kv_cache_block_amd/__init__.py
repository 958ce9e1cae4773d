"""Python binding of the gfx950 streaming sink+window KV-cache library (libllcache.so).

Argument marshalling only: every step runs in the library's HIP kernels.  PyTorch
provides device memory and streams.  The functions mirror the C ABI declared in
``include/ll_cache.h``:

    Cache(layers, heads, head_dim, tokens_per_frame, sink, window, kv_dtype)
    Cache.append(layer, K, V)                      -> ll_cache_append
    Cache.attn(layer, Q, K_chunk, V_chunk, out)    -> ll_attn_sink_window
    Cache.recache(layer, K_all, V_all)             -> ll_cache_recache
    Cache.recache_window(layer, K_win, V_win)      -> ll_cache_recache_window
    kv_project(h, W_K, W_V, K_all, V_all)          -> ll_kv_project

If the library has not been built, importing works but the first call raises
RuntimeError; there is no fallback implementation.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libllcache.so")

LL_OK, LL_ERR_INVALID, LL_ERR_OOM, LL_ERR_STATE, LL_ERR_HIP = range(5)
LL_KV_BF16, LL_KV_INT8, LL_KV_FP8 = 0, 1, 2
_KV_NAMES = {"bf16": LL_KV_BF16, "int8": LL_KV_INT8, "fp8": LL_KV_FP8}
MAX_SLOTS = 128

EXPORTS = [
    "ll_cache_create", "ll_cache_destroy", "ll_cache_append", "ll_attn_sink_window",
    "ll_cache_recache", "ll_cache_recache_window", "ll_kv_project", "ll_cache_recache_from_hidden",
    "ll_cache_create_shots", "ll_cache_begin_shot", "ll_cache_shot_start", "ll_cache_frames_seen",
    "ll_cache_slot_frames", "ll_cache_slot_view", "ll_last_error",
]

_lib = None


class LLError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"status {status}: {message}")
        self.status = status
        self.message = message


def lib():
    """Load libllcache.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m streaming_kv_cache_block_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64p = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int64)
    sig = {
        "ll_cache_create": [i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(vp)],
        "ll_cache_create_shots": [i32, i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(vp)],
        "ll_cache_begin_shot": [vp, i32],
        "ll_cache_shot_start": [vp, i32, i64p],
        "ll_cache_destroy": [vp],
        "ll_cache_append": [vp, i32, vp, vp, i32, vp],
        "ll_attn_sink_window": [vp, i32, vp, vp, vp, i32, vp, vp],
        "ll_cache_recache": [vp, i32, vp, vp, i32, vp],
        "ll_cache_recache_window": [vp, i32, vp, vp, i32, vp],
        "ll_kv_project": [vp, vp, vp, i32, i32, i32, vp, vp, vp],
        "ll_cache_recache_from_hidden": [vp, i32, vp, vp, vp, i32, i32, vp],
        "ll_cache_frames_seen": [vp, i32, i64p],
        "ll_cache_slot_frames": [vp, i32, i64p],
        "ll_cache_slot_view": [vp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                               ctypes.POINTER(vp)],
        "ll_last_error": [],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = None if name == "ll_cache_destroy" else (ctypes.c_char_p if name == "ll_last_error" else i32)
    _lib = L
    return L


def _check(status):
    if status != LL_OK:
        raise LLError(status, lib().ll_last_error().decode())


def _ptr(x):
    """Device pointer of a torch tensor (must be contiguous bf16 on a GPU), or an int."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    import torch
    if not x.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not x.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if x.dtype != torch.bfloat16:
        raise ValueError(f"tensor must be bfloat16, got {x.dtype}")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Cache:
    """Per-layer sink + window KV cache living in device memory."""

    def __init__(self, layers, heads, head_dim, tokens_per_frame, sink, window, kv_dtype="bf16", shot_sink=0):
        self.layers, self.heads, self.head_dim = layers, heads, head_dim
        self.T, self.S, self.W, self.Ss = tokens_per_frame, sink, window, shot_sink
        self.kv_dtype = kv_dtype
        if kv_dtype not in _KV_NAMES and kv_dtype not in _KV_NAMES.values():
            raise ValueError(f"kv_dtype must be 'bf16', 'int8' or 'fp8', got {kv_dtype!r}")
        dt = _KV_NAMES.get(kv_dtype, kv_dtype)
        self.kv_code = dt
        h = ctypes.c_void_p()
        _check(lib().ll_cache_create_shots(layers, heads, head_dim, tokens_per_frame, sink, shot_sink, window, dt,
                                           ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            lib().ll_cache_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _frames(self, t, n_frames):
        if n_frames is not None:
            return n_frames
        rows = t.shape[0]
        if rows % self.T:
            raise ValueError("tensor rows are not a whole number of frames")
        return rows // self.T

    def append(self, layer, K, V, n_frames=None, stream=None):
        _check(lib().ll_cache_append(self._h, layer, _ptr(K), _ptr(V), self._frames(K, n_frames),
                                     _stream(stream)))

    def attn(self, layer, Q, K_chunk, V_chunk, out=None, n_frames=None, stream=None):
        if out is None:
            import torch
            out = torch.empty_like(Q)
        _check(lib().ll_attn_sink_window(self._h, layer, _ptr(Q), _ptr(K_chunk), _ptr(V_chunk),
                                         self._frames(Q, n_frames), _ptr(out), _stream(stream)))
        return out

    def recache(self, layer, K_all, V_all, n_frames=None, stream=None):
        _check(lib().ll_cache_recache(self._h, layer, _ptr(K_all), _ptr(V_all),
                                      self._frames(K_all, n_frames), _stream(stream)))

    def recache_window(self, layer, K_win, V_win, n_frames=None, stream=None):
        _check(lib().ll_cache_recache_window(self._h, layer, _ptr(K_win), _ptr(V_win),
                                             self._frames(K_win, n_frames), _stream(stream)))

    def recache_from_hidden(self, layer, h, W_K, W_V, n_frames=None, stream=None):
        """Recache from hidden states h [n_frames*T][d_in]: K/V = h W^T written into the slots."""
        _check(lib().ll_cache_recache_from_hidden(self._h, layer, _ptr(h), _ptr(W_K), _ptr(W_V),
                                                  self._frames(h, n_frames), h.shape[1], _stream(stream)))

    def begin_shot(self, layer):
        _check(lib().ll_cache_begin_shot(self._h, layer))

    def shot_start(self, layer):
        v = ctypes.c_int64()
        _check(lib().ll_cache_shot_start(self._h, layer, ctypes.byref(v)))
        return v.value

    def frames_seen(self, layer):
        v = ctypes.c_int64()
        _check(lib().ll_cache_frames_seen(self._h, layer, ctypes.byref(v)))
        return v.value

    def slot_frames(self, layer):
        arr = (ctypes.c_int64 * (self.S + self.Ss + self.W))()
        _check(lib().ll_cache_slot_frames(self._h, layer, arr))
        return list(arr)

    def slot_view(self, layer):
        """(K, V, K_scale, V_scale) device pointers of the layer's slot arrays."""
        ptrs = [ctypes.c_void_p() for _ in range(4)]
        _check(lib().ll_cache_slot_view(self._h, layer, *[ctypes.byref(p) for p in ptrs]))
        return tuple(p.value for p in ptrs)

    def slot_bytes(self, layer):
        """Copy the layer's slot arrays to the host (synchronising the device first).

        Returns a dict with 'K', 'V' as uint8 byte arrays shaped [S+W][T][H][D*elt]
        and, for int8 / fp8 caches, 'K_scale', 'V_scale' as float32 [S+W][T][H].
        """
        import numpy as np
        import torch
        torch.cuda.synchronize()
        kp, vp, ksp, vsp = self.slot_view(layer)
        slots = self.S + self.Ss + self.W
        elt = 1 if self.kv_code != LL_KV_BF16 else 2
        nbytes = slots * self.T * self.heads * self.head_dim * elt
        out = {"K": _d2h(kp, nbytes).reshape(slots, self.T, self.heads, self.head_dim * elt),
               "V": _d2h(vp, nbytes).reshape(slots, self.T, self.heads, self.head_dim * elt)}
        if ksp:
            sb = slots * self.T * self.heads * 4
            out["K_scale"] = _d2h(ksp, sb).view(np.float32).reshape(slots, self.T, self.heads)
            out["V_scale"] = _d2h(vsp, sb).view(np.float32).reshape(slots, self.T, self.heads)
        return out


_hip = None


def _d2h(ptr, nbytes):
    """Synchronous device -> host copy of raw library memory (introspection only)."""
    import numpy as np
    global _hip
    if _hip is None:
        # the HIP runtime the library is linked against (the one already in the process)
        _hip = lib()
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    buf = np.empty(nbytes, dtype=np.uint8)
    err = _hip.hipMemcpy(buf.ctypes.data, ptr, nbytes, 2)   # hipMemcpyDeviceToHost
    if err != 0:
        raise RuntimeError(f"hipMemcpy failed with {err}")
    return buf


def kv_project(h, W_K, W_V, K_all=None, V_all=None, stream=None):
    """K_all = h W_K^T, V_all = h W_V^T (bf16).  h [n][d_in], W [d_out][d_in]."""
    import torch
    n, d_in = h.shape
    d_out = W_K.shape[0]
    if K_all is None:
        K_all = torch.empty((n, d_out), dtype=torch.bfloat16, device=h.device)
    if V_all is None:
        V_all = torch.empty((n, d_out), dtype=torch.bfloat16, device=h.device)
    _check(lib().ll_kv_project(_ptr(h), _ptr(W_K), _ptr(W_V), n, d_in, d_out, _ptr(K_all), _ptr(V_all),
                               _stream(stream)))
    return K_all, V_all
