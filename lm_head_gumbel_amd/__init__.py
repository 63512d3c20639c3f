"""Python binding of libfs (fused LM-head Gumbel sampling on MI355X).

Argument marshalling only: every function below forwards to the extern "C"
entry point of the same name in libfs.so (declared in include/fs.h) and
returns its status code.  Device buffers are passed as torch tensors (their
data pointers are used) or as raw integer addresses; `stream` defaults to
torch's current HIP stream.  Every step of the sampling path runs in the HIP
kernels of libfs.so; there is no fallback.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfs.so")

FS_OK, FS_ERR_INVALID_ARG, FS_ERR_UNSUPPORTED, FS_ERR_WORKSPACE, FS_ERR_HIP = range(5)
FS_NO_NOISE = 1
(FS_VARIANT_FLAT, FS_VARIANT_GROUPED, FS_VARIANT_TOPK, FS_VARIANT_MULTINOMIAL,
 FS_VARIANT_LOGITS) = range(5)


class fs_params(ctypes.Structure):
    """Mirror of the C struct fs_params (include/fs.h)."""
    _fields_ = [("B", ctypes.c_int32), ("d", ctypes.c_int32), ("V", ctypes.c_int32),
                ("n_valid", ctypes.c_int32), ("v_offset", ctypes.c_int32),
                ("tile_v", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("step", ctypes.c_uint32), ("flags", ctypes.c_uint32),
                ("seeds", ctypes.c_void_p), ("step_ptr", ctypes.c_void_p)]


def params(B, d, V, n_valid=None, v_offset=0, tile_v=0, seed=0, step=0, flags=0, seeds=None,
           step_ptr=None):
    """Build an fs_params; n_valid defaults to v_offset + V (nothing masked).
    seeds / step_ptr: optional device uint64 [B] per-row keys and device uint32
    step (tensors or raw addresses)."""
    if n_valid is None:
        n_valid = v_offset + V
    return fs_params(B, d, V, n_valid, v_offset, tile_v, seed & 0xFFFFFFFFFFFFFFFF,
                     step & 0xFFFFFFFF, flags, _ptr(seeds), _ptr(step_ptr))


class FsError(RuntimeError):
    def __init__(self, status, where=""):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None
_P = ctypes.c_void_p
_SIGS = {
    "fs_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fs_version": (ctypes.c_char_p, []),
    "fs_num_tiles": (ctypes.c_int32, [ctypes.POINTER(fs_params)]),
    "fs_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(fs_params), ctypes.c_int,
                                             ctypes.c_int32]),
    "fs_sample": (ctypes.c_int, [ctypes.POINTER(fs_params), _P, _P, _P, _P, _P, _P, _P,
                                 ctypes.c_size_t, _P]),
    "fs_sample_noalloc": (ctypes.c_int, [ctypes.POINTER(fs_params), _P, _P, _P, _P, _P, _P,
                                         _P]),
    "fs_sample_stage1": (ctypes.c_int, [ctypes.POINTER(fs_params), _P, _P, _P, _P, _P,
                                        ctypes.c_size_t, _P]),
    "fs_sample_grouped": (ctypes.c_int, [ctypes.POINTER(fs_params), _P, _P, _P, _P, _P, _P, _P,
                                         _P, _P, ctypes.c_size_t, _P]),
    "fs_sample_topk": (ctypes.c_int, [ctypes.POINTER(fs_params), _P, _P, _P, _P, ctypes.c_int32,
                                      _P, _P, ctypes.c_size_t, _P]),
    "fs_sample_topk_topp": (ctypes.c_int, [ctypes.POINTER(fs_params), _P, _P, _P, _P,
                                           ctypes.c_int32, ctypes.c_float, _P, _P,
                                           ctypes.c_size_t, _P]),
    "fs_merge_online": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                                       ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, _P, _P,
                                       _P]),
    "fs_merge_online_dev": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                                           ctypes.c_uint64, _P, ctypes.c_uint32, _P,
                                           ctypes.c_uint32, _P, _P, _P]),
    "fs_logits": (ctypes.c_int, [ctypes.POINTER(fs_params), _P, _P, _P, _P, ctypes.c_size_t,
                                 _P]),
    "fs_multinomial": (ctypes.c_int, [ctypes.POINTER(fs_params), _P, _P, _P, _P, _P,
                                      ctypes.c_size_t, _P]),
    "fs_debug_noise": (ctypes.c_int, [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                      ctypes.c_int32, _P, _P, _P]),
    "fs_debug_read_probe": (ctypes.c_int, [_P, ctypes.c_size_t, _P, ctypes.c_int32, _P]),
    "fs_debug_read_probe_nt": (ctypes.c_int, [_P, ctypes.c_size_t, _P, ctypes.c_int32, _P]),
    "fs_debug_copy": (ctypes.c_int, [_P, _P, ctypes.c_size_t, ctypes.c_int32, _P]),
    "fs_debug_shared_read_probe": (ctypes.c_int, [_P, ctypes.c_size_t, ctypes.c_int32, _P,
                                                  ctypes.c_int32, _P]),
}


def lib():
    """The loaded libfs.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libfs.so not found at {LIB_PATH}: build it with "
                               "`python -m lm_head_gumbel_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _lib = handle
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return None          # no device: the call fails validation or reports it
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ws(ws, ws_bytes):
    if ws is None:
        return None, 0
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    return _ptr(ws), ws_bytes


def status_string(status):
    return lib().fs_status_string(int(status)).decode()


def fs_status_string(status):
    return status_string(status)


def fs_version():
    return lib().fs_version().decode()


def fs_num_tiles(p):
    return lib().fs_num_tiles(ctypes.byref(p))


def fs_workspace_bytes(p, variant, k=0):
    return lib().fs_workspace_bytes(ctypes.byref(p), variant, k)


def fs_sample(p, H, W, temp, allow, out_idx, out_score=None, ws=None, ws_bytes=None,
              stream=None):
    w, n = _ws(ws, ws_bytes)
    return lib().fs_sample(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(temp), _ptr(allow),
                           _ptr(out_idx), _ptr(out_score), w, n, _stream(stream))


def fs_sample_noalloc(p, H, W, temp, allow, out_idx, out_score=None, stream=None):
    return lib().fs_sample_noalloc(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(temp), _ptr(allow),
                                   _ptr(out_idx), _ptr(out_score), _stream(stream))


FS_NOALLOC_SCRATCH_BYTES = 8 << 20


def fs_sample_stage1(p, H, W, temp, allow, ws=None, ws_bytes=None, stream=None):
    w, n = _ws(ws, ws_bytes)
    return lib().fs_sample_stage1(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(temp), _ptr(allow),
                                  w, n, _stream(stream))


def fs_sample_grouped(p, H, W, temp, allow, tile_max, tile_idx, tile_logmass, out_idx=None,
                      ws=None, ws_bytes=None, stream=None):
    w, n = _ws(ws, ws_bytes)
    return lib().fs_sample_grouped(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(temp), _ptr(allow),
                                   _ptr(tile_max), _ptr(tile_idx), _ptr(tile_logmass),
                                   _ptr(out_idx), w, n, _stream(stream))


def fs_sample_topk(p, H, W, temp, allow, k, out_idx, ws=None, ws_bytes=None, stream=None):
    w, n = _ws(ws, ws_bytes)
    return lib().fs_sample_topk(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(temp), _ptr(allow), k,
                                _ptr(out_idx), w, n, _stream(stream))


def fs_sample_topk_topp(p, H, W, temp, allow, k, top_p, out_idx, ws=None, ws_bytes=None,
                        stream=None):
    w, n = _ws(ws, ws_bytes)
    return lib().fs_sample_topk_topp(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(temp), _ptr(allow),
                                     k, float(top_p), _ptr(out_idx), w, n, _stream(stream))


def fs_merge_online(B, C, z, L, temp, seed, step, flags, out_idx, out_L=None, stream=None):
    return lib().fs_merge_online(B, C, _ptr(z), _ptr(L), _ptr(temp),
                                 seed & 0xFFFFFFFFFFFFFFFF, step & 0xFFFFFFFF, flags,
                                 _ptr(out_idx), _ptr(out_L), _stream(stream))


def fs_merge_online_dev(B, C, z, L, temp, seed, seeds, step, step_ptr, flags, out_idx, out_L=None,
                        stream=None):
    return lib().fs_merge_online_dev(B, C, _ptr(z), _ptr(L), _ptr(temp),
                                     seed & 0xFFFFFFFFFFFFFFFF, _ptr(seeds), step & 0xFFFFFFFF,
                                     _ptr(step_ptr), flags, _ptr(out_idx), _ptr(out_L),
                                     _stream(stream))


def fs_logits(p, H, W, logits, ws=None, ws_bytes=None, stream=None):
    w, n = _ws(ws, ws_bytes)
    return lib().fs_logits(ctypes.byref(p), _ptr(H), _ptr(W), _ptr(logits), w, n,
                           _stream(stream))


def fs_multinomial(p, logits, temp, allow, out_idx, ws=None, ws_bytes=None, stream=None):
    w, n = _ws(ws, ws_bytes)
    return lib().fs_multinomial(ctypes.byref(p), _ptr(logits), _ptr(temp), _ptr(allow),
                                _ptr(out_idx), w, n, _stream(stream))


def fs_debug_noise(seed, step, stream_id, b0, nb, i0, ni, words=None, gumbel=None, stream=None):
    return lib().fs_debug_noise(seed & 0xFFFFFFFFFFFFFFFF, step & 0xFFFFFFFF, stream_id, b0, nb,
                                i0, ni, _ptr(words), _ptr(gumbel), _stream(stream))


def fs_debug_read_probe(src, nbytes, sink, grid, stream=None):
    return lib().fs_debug_read_probe(_ptr(src), nbytes, _ptr(sink), grid, _stream(stream))


def fs_debug_read_probe_nt(src, nbytes, sink, grid, stream=None):
    return lib().fs_debug_read_probe_nt(_ptr(src), nbytes, _ptr(sink), grid, _stream(stream))


def fs_debug_shared_read_probe(src, nbytes, reps, sink, grid, stream=None):
    return lib().fs_debug_shared_read_probe(_ptr(src), nbytes, reps, _ptr(sink), grid,
                                            _stream(stream))


def fs_debug_copy(dst, src, nbytes, grid, stream=None):
    return lib().fs_debug_copy(_ptr(dst), _ptr(src), nbytes, grid, _stream(stream))


def check(status, where=""):
    """Raise FsError unless status is FS_OK."""
    if status != FS_OK:
        raise FsError(status, where)
