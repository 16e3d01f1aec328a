"""MI355X (gfx950) dense matrix product C = A·B behind a small C ABI.

``gemm(a, b)`` takes two row-major CUDA/ROCm tensors of one dtype (fp32, fp16
or bf16) and returns C = a @ b of that dtype, computed by the library's HIP
kernels on the current stream (fp32 accumulation, round-to-nearest-even
output) through ``gemm_run``, which allocates nothing; ``split_k=True`` opts
into the split-K schedule of ``gemm_run_ws`` with a workspace from torch's
allocator.  8-bit inputs (``torch.float8_e4m3fn`` or ``torch.float8_e5m2``,
the OCP formats) give a bf16 C.  The C-ABI functions are re-exported under their C names.
PyTorch supplies device memory and the stream; nothing else.
"""
from __future__ import annotations

from ._lib import (GEMM_BF16, GEMM_F16, GEMM_F32, GEMM_FP8_E4M3, GEMM_FP8_E5M2, GemmError, gemm_check_args,
                   gemm_check_args_batched, gemm_config_count, gemm_config_info, gemm_create,
                   gemm_destroy, gemm_run, gemm_run_batched, gemm_run_batched_config,
                   gemm_run_config, gemm_run_ws, gemm_run_ws_config, gemm_select_config,
                   gemm_select_config_batched, gemm_select_config_ws, gemm_tile_of_block,
                   gemm_tile_of_block_batched, gemm_workspace_size, gemm_run_noalloc, gemm_run_clocked,
                   status_string)

__all__ = ["gemm", "gemm_batched", "Gemm", "gemm_create", "gemm_run", "gemm_run_config",
           "gemm_run_batched", "gemm_run_batched_config", "gemm_destroy",
           "gemm_check_args", "gemm_check_args_batched", "gemm_config_count",
           "gemm_config_info", "gemm_select_config", "gemm_select_config_batched",
           "gemm_tile_of_block", "gemm_tile_of_block_batched", "status_string", "GemmError",
           "gemm_workspace_size", "gemm_run_ws", "gemm_run_ws_config", "gemm_select_config_ws",
           "gemm_run_noalloc", "gemm_run_clocked",
           "GEMM_F32", "GEMM_F16", "GEMM_BF16", "GEMM_FP8_E4M3", "GEMM_FP8_E5M2",
           "dtype_code", "out_dtype"]


def dtype_code(dt) -> int:
    import torch
    codes = {torch.float32: GEMM_F32, torch.float16: GEMM_F16, torch.bfloat16: GEMM_BF16,
             torch.float8_e4m3fn: GEMM_FP8_E4M3, torch.float8_e5m2: GEMM_FP8_E5M2}
    if dt not in codes:
        raise TypeError("dtype must be float32, float16, bfloat16, float8_e4m3fn or "
                        f"float8_e5m2, got {dt}")
    return codes[dt]


def out_dtype(dt):
    """dtype of C for inputs of dtype ``dt`` (bf16 for the 8-bit formats)."""
    import torch
    dtype_code(dt)
    return torch.bfloat16 if dt in (torch.float8_e4m3fn, torch.float8_e5m2) else dt


class Gemm:
    """A handle bound to one device, plus the tensor-level call."""

    def __init__(self, device=None):
        import torch
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None
                                   else torch.device(device).index or 0)
        with torch.cuda.device(self.device):
            self.handle = gemm_create()

    def close(self):
        if getattr(self, "handle", None):
            gemm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __call__(self, a, b, out=None, config: int | None = None, splits: int | None = None,
                 split_k: bool = False):
        """C = a @ b through gemm_run, which allocates nothing.  With
        ``split_k=True`` the product goes through gemm_run_ws instead: where
        it splits K (few output tiles, long K) its workspace comes from
        torch's allocator on the current stream (stream-ordered, so
        concurrent streams never share one).  ``config`` forces a kernel
        configuration, and with it ``splits`` a split count."""
        import torch
        if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
            raise ValueError("gemm expects [M, K] @ [K, N]")
        if a.dtype != b.dtype:
            raise TypeError(f"a and b must share a dtype ({a.dtype} vs {b.dtype})")
        code = dtype_code(a.dtype)
        if a.device != self.device or b.device != self.device:
            raise ValueError(f"inputs must be on {self.device}")
        if not (a.is_contiguous() and b.is_contiguous()):
            raise ValueError("inputs must be contiguous row-major (no implicit copies)")
        M, K = a.shape
        N = b.shape[1]
        odt = out_dtype(a.dtype)
        if out is None:
            out = torch.empty((M, N), device=self.device, dtype=odt)
        elif (out.shape != (M, N) or out.dtype != odt or out.device != self.device
              or not out.is_contiguous()):
            raise ValueError(f"out must be a contiguous [M, N] tensor of dtype {odt}")
        stream = torch.cuda.current_stream(self.device).cuda_stream
        with torch.cuda.device(self.device):
            if config is None:
                ws = gemm_workspace_size(M, N, K, code) if split_k else 0
                if ws > 0:
                    work = torch.empty(ws, dtype=torch.uint8, device=self.device)
                    gemm_run_ws(self.handle, a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K,
                                code, work.data_ptr(), ws, stream)
                else:
                    gemm_run(self.handle, a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K,
                             code, stream)
            elif splits is not None and splits > 1:
                ws = splits * M * N * 4
                work = torch.empty(ws, dtype=torch.uint8, device=self.device)
                gemm_run_ws_config(self.handle, a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N,
                                   K, code, config, splits, work.data_ptr(), ws, stream)
            else:
                gemm_run_config(self.handle, a.data_ptr(), b.data_ptr(), out.data_ptr(),
                                M, N, K, code, config, stream)
        return out

    def batched(self, a, b, out=None, config: int | None = None):
        """C[i] = a[i] @ b[i].  a is [batch, M, K] or [M, K] (shared by every
        product), b is [batch, K, N] or [K, N]; at least one is 3-D.  Each
        matrix must be contiguous row-major; the batch stride may be anything
        (a 2-D operand has stride 0).  Returns [batch, M, N]."""
        import torch
        if a.ndim not in (2, 3) or b.ndim not in (2, 3) or (a.ndim == 2 and b.ndim == 2):
            raise ValueError("gemm_batched expects [batch, M, K] @ [batch, K, N] "
                             "(one side may be 2-D and shared)")
        if a.shape[-1] != b.shape[-2]:
            raise ValueError("gemm_batched expects [..., M, K] @ [..., K, N]")
        batch = a.shape[0] if a.ndim == 3 else b.shape[0]
        if (a.ndim == 3 and a.shape[0] != batch) or (b.ndim == 3 and b.shape[0] != batch):
            raise ValueError("batch sizes differ")
        if a.dtype != b.dtype:
            raise TypeError(f"a and b must share a dtype ({a.dtype} vs {b.dtype})")
        code = dtype_code(a.dtype)
        if a.device != self.device or b.device != self.device:
            raise ValueError(f"inputs must be on {self.device}")

        def matrix_stride(t):
            # each matrix contiguous row-major; returns the batch stride
            if t.stride(-1) != 1 or (t.shape[-2] > 1 and t.stride(-2) != t.shape[-1]):
                raise ValueError("every matrix must be contiguous row-major (no implicit copies)")
            return 0 if t.ndim == 2 or t.shape[0] == 1 else t.stride(0)

        sa, sb = matrix_stride(a), matrix_stride(b)
        M, K = a.shape[-2], a.shape[-1]
        N = b.shape[-1]
        odt = out_dtype(a.dtype)
        if out is None:
            out = torch.empty((batch, M, N), device=self.device, dtype=odt)
        elif (out.shape != (batch, M, N) or out.dtype != odt or out.device != self.device
              or not out.is_contiguous()):
            raise ValueError(f"out must be a contiguous [batch, M, N] tensor of dtype {odt}")
        stream = torch.cuda.current_stream(self.device).cuda_stream
        with torch.cuda.device(self.device):
            if config is None:
                gemm_run_batched(self.handle, a.data_ptr(), b.data_ptr(), out.data_ptr(), batch,
                                 M, N, K, sa, sb, M * N, code, stream)
            else:
                gemm_run_batched_config(self.handle, a.data_ptr(), b.data_ptr(), out.data_ptr(),
                                        batch, M, N, K, sa, sb, M * N, code, config, stream)
        return out


_default: dict[int, Gemm] = {}


def gemm(a, b, out=None, config: int | None = None, splits: int | None = None,
         split_k: bool = False):
    """C = a @ b on a's device and the current stream (see module docstring
    and Gemm.__call__)."""
    idx = a.device.index if a.device.index is not None else 0
    g = _default.get(idx)
    if g is None:
        g = _default[idx] = Gemm(idx)
    return g(a, b, out=out, config=config, splits=splits, split_k=split_k)


def gemm_batched(a, b, out=None, config: int | None = None):
    """C[i] = a[i] @ b[i] as one launch on a's device and the current stream
    (see Gemm.batched)."""
    idx = a.device.index if a.device.index is not None else 0
    g = _default.get(idx)
    if g is None:
        g = _default[idx] = Gemm(idx)
    return g.batched(a, b, out=out, config=config)
