"""ctypes loader for libfp8mlp.so (built in-tree by fp8_relu_mlp_amd.build).

There is no fallback: if the library is missing or does not load, every call
raises.  The product path never computes anything in Python.
"""
import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8mlp.so")

_lib = None
_lock = threading.Lock()

c_i64 = ctypes.c_int64
c_size = ctypes.c_size_t
c_int = ctypes.c_int
c_float = ctypes.c_float
vp = ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/fp8mlp.h
SIGNATURES = {
    "fp8mlp_abi_version": (c_int, []),
    "fp8mlp_status_str": (ctypes.c_char_p, [c_int]),
    "fp8mlp_last_hip_error": (c_int, []),
    "fp8mlp_last_failed_kernel": (ctypes.c_char_p, []),
    "mlp_relu2_fwd_workspace": (c_size, [c_i64, c_i64, c_i64]),
    "mlp_relu2_fwd": (c_int, [c_int, vp, vp, vp, vp, vp, vp, c_float, vp, vp, vp, vp, vp,
                              c_i64, c_i64, c_i64, vp, c_size, vp]),
    "mlp_relu2_fwd_noalloc_max_bytes": (c_size, []),
    "mlp_relu2_fwd_noalloc": (c_int, [c_int, vp, vp, vp, vp, vp, vp, c_float, vp, vp, vp, vp, vp,
                                      c_i64, c_i64, c_i64, vp]),
    "mlp_relu2_fwd_fp8up_workspace": (c_size, [c_i64, c_i64, c_i64]),
    "mlp_relu2_fwd_fp8up": (c_int, [vp, vp, vp, vp, vp, vp, vp, c_float, vp, vp, vp, vp, vp, vp,
                                    c_i64, c_i64, c_i64, vp, c_size, vp]),
    "mlp_relu2_bwd_workspace": (c_size, [c_i64, c_i64, c_i64]),
    "mlp_relu2_bwd": (c_int, [vp, vp, vp, vp, vp, vp, vp, vp, c_int, c_i64, c_i64, c_i64, vp, c_size, vp]),
    "mlp_relu2_bwd_fp8post": (c_int, [vp, vp, vp, vp, vp, vp, vp, vp, vp, c_int, c_i64, c_i64, c_i64, vp, c_size,
                                      vp]),
    "fp8_cast_transpose_workspace": (c_size, [c_i64, c_i64]),
    "fp8_cast_transpose": (c_int, [vp, c_i64, c_i64, vp, vp, vp, vp, vp, vp, c_size, vp]),
    "fp8_cast_transpose_w2": (c_int, [vp, c_i64, c_i64, vp, vp, vp, vp, vp, c_size, vp]),
    "amax_reduce_workspace": (c_size, [c_i64]),
    "amax_reduce": (c_int, [c_int, vp, c_i64, vp, vp, c_size, vp]),
    "fp8_scale_from_amax": (c_int, [vp, c_float, vp, vp, vp]),
    "fp8_saturation_count_workspace": (c_size, [c_i64]),
    "fp8_saturation_count": (c_int, [vp, c_i64, vp, vp, c_size, vp]),
    "fp8_linear_workspace": (c_size, [c_i64, c_i64]),
    "fp8_linear": (c_int, [vp, vp, vp, vp, vp, vp, c_i64, c_i64, c_i64, vp, c_size, vp]),
    "softcap_ce_workspace": (c_size, [c_i64, c_i64, c_i64, c_int]),
    "softcap_ce_fwd_bwd": (c_int, [vp, vp, vp, c_int, vp, c_float, vp, vp, vp, vp, vp, c_int, c_i64, c_i64, c_i64,
                                   vp, c_size, vp]),
    "softcap_ce_fp8_workspace": (c_size, [c_i64, c_i64, c_i64, c_int]),
    "softcap_ce_fwd_bwd_fp8": (c_int, [vp, vp, vp, vp, vp, vp, c_int, vp, c_float, vp, vp, vp, vp, vp, c_int, c_i64,
                                       c_i64, c_i64, vp, c_size, vp]),
    "rmsnorm_fwd": (c_int, [vp, vp, vp, c_i64, c_i64, c_float, vp]),
    "rmsnorm_bwd": (c_int, [vp, vp, vp, vp, vp, c_i64, c_i64, vp]),
    "add_bf16": (c_int, [vp, vp, vp, c_i64, vp]),
    "sgd_update_bf16": (c_int, [vp, vp, c_i64, c_float, vp]),
    "fp8mlp_mfma_probe": (c_int, [c_int, vp, c_i64, vp, c_i64, c_i64, vp, vp]),
    "fp8mlp_timing_start": (c_int, [c_int]),
    "fp8mlp_timing_stop": (c_int, []),
    "fp8mlp_timing_get": (c_int, [c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(c_float)]),
    "fp8mlp_timing_dropped": (c_int, []),
}


class Fp8MlpError(RuntimeError):
    def __init__(self, name, status, msg):
        super().__init__(f"{name} failed with status {status}: {msg}")
        self.status = status


def lib():
    """The loaded library (loaded once, on first use)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise ImportError(
                        f"{LIB_PATH} is not built; run `python -m fp8_relu_mlp_amd.build` "
                        "(or __graft_entry__.build()) first")
                L = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    f = getattr(L, name)
                    f.restype = res
                    f.argtypes = args
                _lib = L
    return _lib


def check(name, status):
    if status != 0:
        msg = lib().fp8mlp_status_str(status).decode()
        if status == -6:
            msg += f" (hipError_t {lib().fp8mlp_last_hip_error()})"
            failed = lib().fp8mlp_last_failed_kernel()
            if failed:
                msg += f" in kernel {failed.decode()}"
        raise Fp8MlpError(name, status, msg)
