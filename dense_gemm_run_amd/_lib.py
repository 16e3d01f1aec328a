"""ctypes binding of ``libdense_gemm_run_amd.so`` (include/dense_gemm.h).

Argument marshalling only: every step of the product runs in the library's
HIP kernels.  If the library is missing this module raises; there is no
fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdense_gemm_run_amd.so")

GEMM_F32, GEMM_F16, GEMM_BF16, GEMM_FP8_E4M3, GEMM_FP8_E5M2 = 0, 1, 2, 3, 4

STATUS = {
    0: "GEMM_OK",
    1: "GEMM_ERR_INVALID_VALUE",
    2: "GEMM_ERR_UNSUPPORTED_DTYPE",
    3: "GEMM_ERR_UNSUPPORTED_DEVICE",
    4: "GEMM_ERR_TOO_LARGE",
    5: "GEMM_ERR_ALIASING",
    6: "GEMM_ERR_HIP",
    7: "GEMM_ERR_CONFIG_MISMATCH",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}

# Every function the header declares, with its ctypes signature.
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_VP = ctypes.c_void_p


class ConfigInfo(ctypes.Structure):
    _fields_ = [("id", _I32), ("bm", _I32), ("bn", _I32), ("bk", _I32),
                ("group_m", _I32), ("threads", _I32), ("dtype_mask", _I32),
                ("needs_vec_align", _I32), ("xcd_remap", _I32),
                ("name", ctypes.c_char * 40)]


SIGNATURES = {
    "gemm_create": (_I32, [ctypes.POINTER(_VP)]),
    "gemm_run": (_I32, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _I32, _VP]),
    "gemm_destroy": (_I32, [_VP]),
    "gemm_status_string": (ctypes.c_char_p, [_I32]),
    "gemm_check_args": (_I32, [_VP, _VP, _VP, _I64, _I64, _I64, _I32]),
    "gemm_config_count": (_I32, []),
    "gemm_config_info": (_I32, [_I32, ctypes.POINTER(ConfigInfo)]),
    "gemm_select_config": (_I32, [_VP, _VP, _VP, _I64, _I64, _I64, _I32]),
    "gemm_tile_of_block": (_I32, [_I32, _I64, _I64, _I64, ctypes.POINTER(_I64),
                                  ctypes.POINTER(_I64)]),
    "gemm_run_config": (_I32, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _I32, _I32, _VP]),
    "gemm_run_batched": (_I32, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                _I32, _VP]),
    "gemm_check_args_batched": (_I32, [_VP, _VP, _VP, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                       _I32]),
    "gemm_select_config_batched": (_I32, [_VP, _VP, _VP, _I64, _I64, _I64, _I64, _I64, _I64,
                                          _I64, _I32]),
    "gemm_tile_of_block_batched": (_I32, [_I32, _I64, _I64, _I64, _I64, ctypes.POINTER(_I64),
                                          ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "gemm_run_batched_config": (_I32, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _I64, _I64,
                                       _I64, _I32, _I32, _VP]),
    "gemm_workspace_size": (_I64, [_I64, _I64, _I64, _I32]),
    "gemm_run_ws": (_I32, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _I32, _VP, _I64, _VP]),
    "gemm_run_ws_config": (_I32, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _I32, _I32, _I32, _VP, _I64,
                                  _VP]),
    "gemm_select_config_ws": (_I32, [_VP, _VP, _VP, _I64, _I64, _I64, _I32, _I64,
                                     ctypes.POINTER(_I32)]),
    "gemm_run_noalloc": (_I32, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _I32, _VP]),
    "gemm_run_clocked": (_I32, [_VP, _VP, _VP, _VP, _I64, _I64, _I64, _I32, _VP, _VP]),
}

# Size of the library's own scratch used by gemm_run_noalloc (per device).
NOALLOC_SCRATCH_BYTES = 16 << 20

_lib = None


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{where}: {self.name} ({status_string(status)})")


def lib() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with dense_gemm_run_amd.build "
                "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().gemm_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise GemmError(status, where)


# ------------------------------------------------------------------ C ABI, same names
def gemm_create() -> int:
    h = _VP()
    _check(lib().gemm_create(ctypes.byref(h)), "gemm_create")
    return h.value


def gemm_run(h, A: int, B: int, C: int, M: int, N: int, K: int, dtype: int,
             stream: int | None) -> None:
    _check(lib().gemm_run(h, A, B, C, M, N, K, dtype, stream), "gemm_run")


def gemm_run_config(h, A: int, B: int, C: int, M: int, N: int, K: int, dtype: int,
                    config_id: int, stream: int | None) -> None:
    _check(lib().gemm_run_config(h, A, B, C, M, N, K, dtype, config_id, stream),
           "gemm_run_config")


def gemm_destroy(h) -> None:
    _check(lib().gemm_destroy(h), "gemm_destroy")


def gemm_check_args(A: int, B: int, C: int, M: int, N: int, K: int, dtype: int) -> int:
    return lib().gemm_check_args(A, B, C, M, N, K, dtype)


def gemm_config_count() -> int:
    return lib().gemm_config_count()


def gemm_config_info(config_id: int) -> dict:
    info = ConfigInfo()
    _check(lib().gemm_config_info(config_id, ctypes.byref(info)), "gemm_config_info")
    return {f: (getattr(info, f).decode() if f == "name" else getattr(info, f))
            for f, _ in ConfigInfo._fields_}


def gemm_select_config(A: int, B: int, C: int, M: int, N: int, K: int, dtype: int) -> int:
    return lib().gemm_select_config(A, B, C, M, N, K, dtype)


def gemm_tile_of_block(config_id: int, M: int, N: int, block: int) -> tuple[int, int]:
    tm, tn = _I64(), _I64()
    _check(lib().gemm_tile_of_block(config_id, M, N, block, ctypes.byref(tm), ctypes.byref(tn)),
           "gemm_tile_of_block")
    return tm.value, tn.value


def gemm_run_batched(h, A: int, B: int, C: int, batch: int, M: int, N: int, K: int,
                     stride_a: int, stride_b: int, stride_c: int, dtype: int,
                     stream: int | None) -> None:
    _check(lib().gemm_run_batched(h, A, B, C, batch, M, N, K, stride_a, stride_b, stride_c,
                                  dtype, stream), "gemm_run_batched")


def gemm_run_batched_config(h, A: int, B: int, C: int, batch: int, M: int, N: int, K: int,
                            stride_a: int, stride_b: int, stride_c: int, dtype: int,
                            config_id: int, stream: int | None) -> None:
    _check(lib().gemm_run_batched_config(h, A, B, C, batch, M, N, K, stride_a, stride_b,
                                         stride_c, dtype, config_id, stream),
           "gemm_run_batched_config")


def gemm_check_args_batched(A: int, B: int, C: int, batch: int, M: int, N: int, K: int,
                            stride_a: int, stride_b: int, stride_c: int, dtype: int) -> int:
    return lib().gemm_check_args_batched(A, B, C, batch, M, N, K, stride_a, stride_b, stride_c,
                                         dtype)


def gemm_select_config_batched(A: int, B: int, C: int, batch: int, M: int, N: int, K: int,
                               stride_a: int, stride_b: int, stride_c: int, dtype: int) -> int:
    return lib().gemm_select_config_batched(A, B, C, batch, M, N, K, stride_a, stride_b,
                                            stride_c, dtype)


def gemm_tile_of_block_batched(config_id: int, M: int, N: int, batch: int,
                               block: int) -> tuple[int, int, int]:
    b, tm, tn = _I64(), _I64(), _I64()
    _check(lib().gemm_tile_of_block_batched(config_id, M, N, batch, block, ctypes.byref(b),
                                            ctypes.byref(tm), ctypes.byref(tn)),
           "gemm_tile_of_block_batched")
    return b.value, tm.value, tn.value


def gemm_workspace_size(M: int, N: int, K: int, dtype: int) -> int:
    """Workspace bytes gemm_run_ws uses for this product (0: none; -1: bad sizes)."""
    return lib().gemm_workspace_size(M, N, K, dtype)


def gemm_run_ws(h, A: int, B: int, C: int, M: int, N: int, K: int, dtype: int,
                workspace: int, workspace_bytes: int, stream=None) -> None:
    _check(lib().gemm_run_ws(h, A, B, C, M, N, K, dtype, workspace, workspace_bytes, stream),
           "gemm_run_ws")


def gemm_run_ws_config(h, A: int, B: int, C: int, M: int, N: int, K: int, dtype: int,
                       config_id: int, splits: int, workspace: int, workspace_bytes: int,
                       stream=None) -> None:
    _check(lib().gemm_run_ws_config(h, A, B, C, M, N, K, dtype, config_id, splits, workspace,
                                    workspace_bytes, stream), "gemm_run_ws_config")


def gemm_select_config_ws(A: int, B: int, C: int, M: int, N: int, K: int, dtype: int,
                          workspace_bytes: int) -> tuple[int, int]:
    """(configuration, split count) gemm_run_ws would use; (-1, 1) on bad arguments."""
    s = _I32(1)
    cid = lib().gemm_select_config_ws(A, B, C, M, N, K, dtype, workspace_bytes, ctypes.byref(s))
    return cid, s.value


def gemm_run_noalloc(h, A: int, B: int, C: int, M: int, N: int, K: int, dtype: int,
                     stream=None) -> None:
    """gemm_run_ws with the library's own scratch (allocates nothing)."""
    _check(lib().gemm_run_noalloc(h, A, B, C, M, N, K, dtype, stream), "gemm_run_noalloc")


def gemm_run_clocked(h, A: int, B: int, C: int, M: int, N: int, K: int, dtype: int, clk: int,
                     stream=None) -> None:
    """gemm_run, with the MFMA tile kernels' clock samples written to clk
    (device, 4 x uint64: clock0, clock1, real0, real1)."""
    _check(lib().gemm_run_clocked(h, A, B, C, M, N, K, dtype, clk, stream), "gemm_run_clocked")
