"""MI355X (gfx950) NVFP4 weight-quantized linear layer.

Thin Python binding over the C ABI of ``libnvfp4.so`` (``include/nvfp4.h``).
Functions take torch tensors that live on the GPU, pass their device pointers
and the current HIP stream to the library, and return torch tensors.  Every
step of the computation runs in the library's HIP kernels; there is no CPU or
PyTorch fallback, and a missing library raises.

bf16 tensors are ``torch.bfloat16``; NVFP4 matrices are a pair of ``uint8``
tensors (codes ``[R, K/2]``, E4M3 scales ``[R, K/16]``).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "library_path", "dequantize", "quantize", "gemm", "gemm_workspace_size", "moe_align",
    "grouped_gemm", "moe_combine", "moe_layer", "topk", "head_topk", "kv_store_e4m3",
    "kv_load_e4m3", "quantize_scaled", "quantize_weight", "gemm_w4a4", "dequantize_scaled",
    "gemm_scaled", "tiled_weight_bytes", "tile_weight", "gemm_tiled", "gemm_tiled_workspace_size",
    "tile_experts", "grouped_gemm_tiled", "moe_layer_tiled",
    "Plan", "make_plan", "BF16", "FP32", "NVFP4", "EPI_NONE", "EPI_SWIGLU",
]

BF16, FP32, NVFP4 = 0, 1, 2
EPI_NONE, EPI_SWIGLU = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libnvfp4.so")
_lib = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_int = ctypes.c_int

_SIGS = {
    "nvfp4_status_string": ([_int], ctypes.c_char_p),
    "nvfp4_version": ([], _int),
    "nvfp4_dequantize": ([_vp, _vp, _i64, _i64, _vp, _vp], _int),
    "nvfp4_quantize": ([_vp, _i64, _i64, _vp, _vp, _vp], _int),
    "nvfp4_gemm_workspace_size": ([_int, _i64, _i64, _i64, _i64], _sz),
    "nvfp4_gemm": ([_int, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _int, _vp, _vp, _sz,
                    _vp], _int),
    "nvfp4_topk_workspace_size": ([_i64, _i64, _i64], _sz),
    "nvfp4_topk": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "nvfp4_head_topk_workspace_size": ([_i64, _i64, _i64, _i64, _i64], _sz),
    "nvfp4_head_topk": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _sz,
                         _vp], _int),
    "nvfp4_gemm_w4a4_bf16_workspace_size": ([_i64, _i64, _i64, _i64], _sz),
    "nvfp4_gemm_w4a4_bf16": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _int, _vp, _vp, _sz,
                              _vp], _int),
    "nvfp4_quantize_scaled": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp], _int),
    "nvfp4_quantize_weight_workspace_size": ([_i64, _i64], _sz),
    "nvfp4_quantize_weight": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "nvfp4_dequantize_scaled": ([_vp, _vp, _vp, _i64, _i64, _vp, _vp], _int),
    "nvfp4_gemm_scaled": ([_int, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _i64,
                           _int, _vp, _vp, _sz, _vp], _int),
    "nvfp4_kv_store_e4m3": ([_vp, _i64, _i64, _vp, ctypes.c_float, _vp, _i64, _vp], _int),
    "nvfp4_kv_load_e4m3": ([_vp, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_float,
                            _vp, _vp], _int),
    "nvfp4_moe_align_workspace_size": ([_i64, _i64, _i64], _sz),
    "nvfp4_moe_align": ([_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "nvfp4_grouped_gemm_workspace_size": ([_i64, _i64, _i64, _i64], _sz),
    "nvfp4_grouped_gemm": ([_vp, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _int,
                            _vp, _vp, _sz, _vp], _int),
    "nvfp4_grouped_gemm_scaled": ([_vp, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp,
                                   _vp, _int, _vp, _vp, _sz, _vp], _int),
    "nvfp4_moe_combine": ([_vp, _vp, _i64, _i64, _i64, _vp, _vp], _int),
    "nvfp4_tiled_weight_bytes": ([_i64, _i64], _sz),
    "nvfp4_tile_weight": ([_vp, _vp, _i64, _i64, _vp, _i64, _vp, _vp], _int),
    "nvfp4_gemm_tiled_workspace_size": ([_int, _i64, _i64, _i64], _sz),
    "nvfp4_gemm_tiled": ([_int, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _vp, _sz, _vp], _int),
    "nvfp4_grouped_gemm_tiled": ([_vp, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp,
                                  _int, _vp, _vp, _sz, _vp], _int),
    "nvfp4_noalloc_scratch_bytes": ([], _sz),
    "nvfp4_gemm_noalloc": ([_int, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _int, _vp,
                            _vp], _int),
}


class Plan(ctypes.Structure):
    """Launch-plan override of the tuning entry points (include/nvfp4_plan.h):
    a field < 0 keeps the library's own choice."""
    _fields_ = [(n, ctypes.c_int) for n in (
        "gemm_min_m", "gemv_small_max", "gemv_tiles", "gemv_waves", "gemv_lds_kib",
        "gemv_splits", "w4a4_fuse", "grouped_mfma_min_rows", "gemv_kparts",
        "grouped_gemv_waves")]


_pp = ctypes.POINTER(Plan)
_SIGS.update({
    "nvfp4_plan_default": ([_pp], None),
    "nvfp4_gemm_workspace_size_planned": ([_pp, _int, _i64, _i64, _i64, _i64], _sz),
    "nvfp4_gemm_planned": ([_pp, _int, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _int, _vp,
                            _vp, _sz, _vp], _int),
    "nvfp4_gemm_w4a4_bf16_workspace_size_planned": ([_pp, _i64, _i64, _i64, _i64], _sz),
    "nvfp4_gemm_w4a4_bf16_planned": ([_pp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _int, _vp,
                                      _vp, _sz, _vp], _int),
    "nvfp4_gemm_tiled_workspace_size_planned": ([_pp, _int, _i64, _i64, _i64], _sz),
    "nvfp4_gemm_tiled_planned": ([_pp, _int, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _vp, _sz,
                                  _vp], _int),
    "nvfp4_grouped_gemm_tiled_planned": ([_pp, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _vp,
                                          _vp, _vp, _int, _vp, _vp, _sz, _vp], _int),
    "nvfp4_grouped_gemm_planned": ([_pp, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _vp, _vp,
                                    _vp, _int, _vp, _vp, _sz, _vp], _int),
    "nvfp4_grouped_gemm_scaled_planned": ([_pp, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _vp,
                                           _vp, _vp, _vp, _int, _vp, _vp, _sz, _vp], _int),
})


def make_plan(**fields) -> Plan:
    """A Plan with the given fields set and every other field -1 (default)."""
    p = Plan()
    for name, _ in Plan._fields_:
        setattr(p, name, -1)
    for name, v in fields.items():
        if name not in dict(Plan._fields_):
            raise ValueError(f"unknown plan field {name!r}")
        setattr(p, name, int(v))
    return p


def _plan_ref(plan):
    if plan is None:
        return None
    if isinstance(plan, dict):
        plan = make_plan(**plan)
    return ctypes.byref(plan)


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded C library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m bit_quantized_gemm_nvfp4_amd.build`"
                " (the NVFP4 layer has no fallback implementation)")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise RuntimeError(lib().nvfp4_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _gpu(*tensors):
    """Every given tensor is a contiguous CUDA tensor, all on one device (checked
    after the shapes and dtypes, so argument errors are reported first)."""
    dev = None
    for t in tensors:
        if t is not None:
            if not t.is_cuda:
                raise RuntimeError("NVFP4 ops run on the GPU only; got a CPU tensor")
            if not t.is_contiguous():
                raise RuntimeError("NVFP4 ops need contiguous tensors")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise RuntimeError(f"NVFP4 ops need one device; got {dev} and {t.device}")


def _arg(t, name, dtype, shape=None, optional=False):
    """Check one tensor argument's dtype and exact shape before any GPU work:
    the kernels trust them (a wrong size reads or writes past the tensor)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dims(t, name, ndim):
    if not isinstance(t, torch.Tensor) or t.dim() != ndim:
        raise ValueError(f"{name} must be a {ndim}-d tensor")
    return tuple(t.shape)


def _workspace(nbytes: int, device, workspace=None):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor")
        if workspace.device != torch.device(device):
            raise RuntimeError(f"workspace on {workspace.device}, expected {device}")
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return workspace, nbytes
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


_OUT_DT = {torch.bfloat16: BF16, torch.float32: FP32}


def _out_dtype(dt):
    if dt not in _OUT_DT:
        raise ValueError(f"out_dtype must be torch.bfloat16 or torch.float32, got {dt}")
    return _OUT_DT[dt]


def _weights(w_codes, w_scales, K=None):
    """NVFP4 weights [N, K/2] + [N, K/16] -> (N, K)."""
    N, half = _dims(w_codes, "w_codes", 2)
    _arg(w_codes, "w_codes", torch.uint8)
    Kw = 2 * half
    if Kw % 32:
        raise ValueError(f"weights K={Kw} is not a multiple of 32")
    if K is not None and Kw != K:
        raise ValueError(f"K mismatch: activations K={K}, weights K={Kw}")
    _arg(w_scales, "w_scales", torch.uint8, (N, Kw // 16))
    return N, Kw


def _rows(row_idx, N):
    if row_idx is None:
        return N
    _dims(row_idx, "row_idx", 1)
    _arg(row_idx, "row_idx", torch.int32)
    n = row_idx.numel()
    if n < 1 or n > N:
        raise ValueError(f"row_idx has {n} entries; 1..{N} allowed")
    return n


# ---- formats -------------------------------------------------------------------------

def dequantize(codes: torch.Tensor, scales: torch.Tensor, out=None) -> torch.Tensor:
    """NVFP4 [N, K/2] codes + [N, K/16] scales -> bf16 [N, K] (exact)."""
    N, K = _weights(codes, scales)
    _arg(out, "out", torch.bfloat16, (N, K), optional=True)
    _gpu(codes, scales, out)
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=codes.device)
    _check(lib().nvfp4_dequantize(_ptr(codes), _ptr(scales), N, K, _ptr(out),
                                  _stream(codes.device)))
    return out


def quantize(x: torch.Tensor, codes=None, scales=None):
    """bf16 [M, K] -> (codes uint8 [M, K/2], scales uint8 [M, K/16])."""
    M, K = _dims(x, "x", 2)
    _arg(x, "x", torch.bfloat16)
    _arg(codes, "codes", torch.uint8, (M, K // 2), optional=True)
    _arg(scales, "scales", torch.uint8, (M, K // 16), optional=True)
    _gpu(x, codes, scales)
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    _check(lib().nvfp4_quantize(_ptr(x), M, K, _ptr(codes), _ptr(scales), _stream(x.device)))
    return codes, scales


# ---- linear layer --------------------------------------------------------------------

def gemm_workspace_size(M: int, N: int, K: int, n_out: int | None = None,
                        w4a4: bool = False, plan=None) -> int:
    n_out = N if n_out is None else n_out
    dt = NVFP4 if w4a4 else BF16
    if plan is not None:
        return int(lib().nvfp4_gemm_workspace_size_planned(_plan_ref(plan), dt, M, N, K, n_out))
    return int(lib().nvfp4_gemm_workspace_size(dt, M, N, K, n_out))


def _activations(a, a_scales):
    """bf16 [M, K] (W4A16) or NVFP4 codes [M, K/2] + scales [M, K/16] -> (M, K, w4a4)."""
    M, c = _dims(a, "a", 2)
    if a_scales is None:
        _arg(a, "a", torch.bfloat16)
        return M, c, False
    _arg(a, "a", torch.uint8)
    _arg(a_scales, "a_scales", torch.uint8, (M, 2 * c // 16))
    return M, 2 * c, True


def gemm(a: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, a_scales=None,
         row_idx=None, out_dtype=torch.bfloat16, out=None, workspace=None,
         plan=None) -> torch.Tensor:
    """y = a . W^T.  a is bf16 [M, K] (W4A16) or NVFP4 codes [M, K/2] with
    a_scales [M, K/16] (W4A4).  row_idx (int32, sorted) restricts the output to
    those weight rows.  plan (dict or Plan) forces a launch plan through the
    tuning entry point (same results)."""
    M, K, w4a4 = _activations(a, a_scales)
    N, _ = _weights(w_codes, w_scales, K)
    n_out = _rows(row_idx, N)
    odt = _out_dtype(out_dtype)
    _arg(out, "out", out_dtype, (M, n_out), optional=True)
    _gpu(a, w_codes, w_scales, a_scales, row_idx, out, workspace)
    if out is None:
        out = torch.empty((M, n_out), dtype=out_dtype, device=a.device)
    ws, wsz = _workspace(gemm_workspace_size(M, N, K, n_out, w4a4, plan), a.device, workspace)
    args = (NVFP4 if w4a4 else BF16, _ptr(a), _ptr(a_scales), M, N, K, _ptr(w_codes),
            _ptr(w_scales), _ptr(row_idx), n_out, odt, _ptr(out), _ptr(ws), wsz,
            _stream(a.device))
    if plan is not None:
        _check(lib().nvfp4_gemm_planned(_plan_ref(plan), *args))
    else:
        _check(lib().nvfp4_gemm(*args))
    return out


# ---- tiled weights (include/nvfp4.h: NF4T) ----------------------------------------------

def tiled_weight_bytes(N: int, K: int) -> int:
    """Bytes of the tiled layout of an N x K NVFP4 matrix (0 for an invalid shape)."""
    return int(lib().nvfp4_tiled_weight_bytes(N, K))


def tile_weight(w_codes: torch.Tensor, w_scales: torch.Tensor, row_idx=None,
                out=None) -> torch.Tensor:
    """The tiled layout (a 1-d uint8 tensor) of NVFP4 weights [N, K/2] + [N, K/16],
    or of the rows row_idx (int32) of them, in that order."""
    N, K = _weights(w_codes, w_scales)
    n_rows = _rows(row_idx, N)
    nbytes = tiled_weight_bytes(n_rows, K)
    _arg(out, "out", torch.uint8, (nbytes,), optional=True)
    _gpu(w_codes, w_scales, row_idx, out)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w_codes.device)
    _check(lib().nvfp4_tile_weight(_ptr(w_codes), _ptr(w_scales), N, K, _ptr(row_idx), n_rows,
                                   _ptr(out), _stream(w_codes.device)))
    return out


def gemm_tiled_workspace_size(M: int, N: int, K: int, w4a4: bool = False, plan=None) -> int:
    dt = NVFP4 if w4a4 else BF16
    if plan is not None:
        return int(lib().nvfp4_gemm_tiled_workspace_size_planned(_plan_ref(plan), dt, M, N, K))
    return int(lib().nvfp4_gemm_tiled_workspace_size(dt, M, N, K))


def gemm_tiled(a: torch.Tensor, w_tiled: torch.Tensor, N: int, a_scales=None,
               out_dtype=torch.bfloat16, out=None, workspace=None, plan=None) -> torch.Tensor:
    """y = a . W^T with W given in the tiled layout (tile_weight) of N rows; a
    as in gemm (bf16 [M, K], or NVFP4 codes with a_scales)."""
    M, K, w4a4 = _activations(a, a_scales)
    if K % 32:
        raise ValueError(f"K={K} is not a multiple of 32")
    if int(N) < 1:
        raise ValueError("N must be positive")
    _arg(w_tiled, "w_tiled", torch.uint8, (tiled_weight_bytes(N, K),))
    odt = _out_dtype(out_dtype)
    _arg(out, "out", out_dtype, (M, N), optional=True)
    _gpu(a, a_scales, w_tiled, out, workspace)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    ws, wsz = _workspace(gemm_tiled_workspace_size(M, N, K, w4a4, plan), a.device, workspace)
    args = (NVFP4 if w4a4 else BF16, _ptr(a), _ptr(a_scales), M, N, K, _ptr(w_tiled), odt,
            _ptr(out), _ptr(ws), wsz, _stream(a.device))
    if plan is not None:
        _check(lib().nvfp4_gemm_tiled_planned(_plan_ref(plan), *args))
    else:
        _check(lib().nvfp4_gemm_tiled(*args))
    return out


# ---- two-level NVFP4 (per-tensor fp32 scale on the device) ------------------------------

def _scalar(g, name, optional=False):
    _arg(g, name, torch.float32, optional=optional)
    if g is not None and g.numel() != 1:
        raise ValueError(f"{name} must hold exactly one float32")


def quantize_scaled(x: torch.Tensor, global_scale: torch.Tensor, codes=None, scales=None):
    """bf16 [M, K] with a per-tensor scale (fp32 tensor of one element on the
    GPU) -> (codes, scales) of fl32(x / g)."""
    M, K = _dims(x, "x", 2)
    _arg(x, "x", torch.bfloat16)
    _scalar(global_scale, "global_scale")
    _arg(codes, "codes", torch.uint8, (M, K // 2), optional=True)
    _arg(scales, "scales", torch.uint8, (M, K // 16), optional=True)
    _gpu(x, global_scale, codes, scales)
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    _check(lib().nvfp4_quantize_scaled(_ptr(x), M, K, _ptr(global_scale), _ptr(codes),
                                       _ptr(scales), _stream(x.device)))
    return codes, scales


def quantize_weight(w: torch.Tensor, workspace=None, codes=None, scales=None,
                    global_scale=None):
    """Offline weight quantizer: bf16 [N, K] -> (codes [N, K/2], scales
    [N, K/16], global_scale fp32 [1]), all on the GPU.  Given outputs are
    written in place (e.g. one expert's slice of a stacked tensor)."""
    N, K = _dims(w, "w", 2)
    _arg(w, "w", torch.bfloat16)
    _arg(codes, "codes", torch.uint8, (N, K // 2), optional=True)
    _arg(scales, "scales", torch.uint8, (N, K // 16), optional=True)
    _scalar(global_scale, "global_scale", optional=True)
    _gpu(w, workspace, codes, scales, global_scale)
    if codes is None:
        codes = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((N, K // 16), dtype=torch.uint8, device=w.device)
    g = global_scale if global_scale is not None else torch.empty(1, dtype=torch.float32,
                                                                  device=w.device)
    ws, wsz = _workspace(int(lib().nvfp4_quantize_weight_workspace_size(N, K)), w.device,
                         workspace)
    _check(lib().nvfp4_quantize_weight(_ptr(w), N, K, _ptr(codes), _ptr(scales), _ptr(g),
                                       _ptr(ws), wsz, _stream(w.device)))
    return codes, scales, g


def dequantize_scaled(codes: torch.Tensor, scales: torch.Tensor, global_scale: torch.Tensor,
                      out=None) -> torch.Tensor:
    """Two-level NVFP4 -> bf16 [N, K]: bf16(fl32(e2m1 * e4m3 * g))."""
    N, K = _weights(codes, scales)
    _scalar(global_scale, "global_scale")
    _arg(out, "out", torch.bfloat16, (N, K), optional=True)
    _gpu(codes, scales, global_scale, out)
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=codes.device)
    _check(lib().nvfp4_dequantize_scaled(_ptr(codes), _ptr(scales), _ptr(global_scale), N, K,
                                         _ptr(out), _stream(codes.device)))
    return out


def gemm_scaled(a: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor,
                w_global_scale=None, a_scales=None, a_global_scale=None, row_idx=None,
                out_dtype=torch.bfloat16, out=None, workspace=None) -> torch.Tensor:
    """gemm() of two-level operands: the output is multiplied by
    a_global_scale * w_global_scale (fp32 device scalars; None stands for 1)."""
    M, K, w4a4 = _activations(a, a_scales)
    N, _ = _weights(w_codes, w_scales, K)
    n_out = _rows(row_idx, N)
    odt = _out_dtype(out_dtype)
    _scalar(w_global_scale, "w_global_scale", optional=True)
    _scalar(a_global_scale, "a_global_scale", optional=True)
    _arg(out, "out", out_dtype, (M, n_out), optional=True)
    _gpu(a, w_codes, w_scales, w_global_scale, a_scales, a_global_scale, row_idx, out, workspace)
    if out is None:
        out = torch.empty((M, n_out), dtype=out_dtype, device=a.device)
    ws, wsz = _workspace(gemm_workspace_size(M, N, K, n_out, w4a4), a.device, workspace)
    _check(lib().nvfp4_gemm_scaled(NVFP4 if w4a4 else BF16, _ptr(a), _ptr(a_scales),
                                   _ptr(a_global_scale), M, N, K, _ptr(w_codes), _ptr(w_scales),
                                   _ptr(w_global_scale), _ptr(row_idx), n_out, odt, _ptr(out),
                                   _ptr(ws), wsz, _stream(a.device)))
    return out


# ---- draft proposal from the masked head ----------------------------------------------

def topk(logits: torch.Tensor, k: int, ids_map=None, workspace=None, values=None, ids=None):
    """Top-k of each row of fp32 logits [M, n], best first (larger value, then
    smaller column; -0 below +0) -> (values fp32 [M, k], ids int32 [M, k]).
    ids are ids_map[column] when ids_map (int32 [n]) is given."""
    M, n = _dims(logits, "logits", 2)
    _arg(logits, "logits", torch.float32)
    _arg(ids_map, "ids_map", torch.int32, (n,), optional=True)
    _arg(values, "values", torch.float32, (M, k), optional=True)
    _arg(ids, "ids", torch.int32, (M, k), optional=True)
    _gpu(logits, ids_map, workspace, values, ids)
    if values is None:
        values = torch.empty((M, k), dtype=torch.float32, device=logits.device)
    if ids is None:
        ids = torch.empty((M, k), dtype=torch.int32, device=logits.device)
    ws, wsz = _workspace(int(lib().nvfp4_topk_workspace_size(M, n, k)), logits.device, workspace)
    _check(lib().nvfp4_topk(_ptr(logits), M, n, k, _ptr(ids_map), _ptr(values), _ptr(ids),
                            _ptr(ws), wsz, _stream(logits.device)))
    return values, ids


def head_topk_workspace_size(M: int, N: int, K: int, n_out: int, k: int) -> int:
    return int(lib().nvfp4_head_topk_workspace_size(M, N, K, n_out, k))


def head_topk(a: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, k: int,
              row_idx=None, workspace=None, values=None, ids=None):
    """Masked draft head and its proposal: fp32 logits of the W4A16 head over
    the rows row_idx (all rows if None), then their top-k -> (values fp32
    [M, k], ids int32 [M, k]); ids are weight-row (token) ids."""
    M, K = _dims(a, "a", 2)
    _arg(a, "a", torch.bfloat16)
    N, _ = _weights(w_codes, w_scales, K)
    n_out = _rows(row_idx, N)
    _arg(values, "values", torch.float32, (M, k), optional=True)
    _arg(ids, "ids", torch.int32, (M, k), optional=True)
    _gpu(a, w_codes, w_scales, row_idx, workspace, values, ids)
    if values is None:
        values = torch.empty((M, k), dtype=torch.float32, device=a.device)
    if ids is None:
        ids = torch.empty((M, k), dtype=torch.int32, device=a.device)
    ws, wsz = _workspace(head_topk_workspace_size(M, N, K, n_out, k), a.device, workspace)
    _check(lib().nvfp4_head_topk(_ptr(a), M, N, K, _ptr(w_codes), _ptr(w_scales), _ptr(row_idx),
                                 n_out, k, _ptr(values), _ptr(ids), _ptr(ws), wsz,
                                 _stream(a.device)))
    return values, ids


# ---- FP8 E4M3 KV cache ------------------------------------------------------------------

def kv_store_e4m3(x: torch.Tensor, slot_mapping: torch.Tensor, scale: float,
                  cache: torch.Tensor) -> torch.Tensor:
    """Write token rows x (bf16 [T, W]) into cache (uint8 [num_slots, W], updated
    in place) at rows slot_mapping (int32 [T]; < 0 skips).  Returns cache."""
    T, W = _dims(x, "x", 2)
    _arg(x, "x", torch.bfloat16)
    _arg(slot_mapping, "slot_mapping", torch.int32, (T,))
    S, Wc = _dims(cache, "cache", 2)
    _arg(cache, "cache", torch.uint8, (S, W))
    _gpu(x, slot_mapping, cache)
    _check(lib().nvfp4_kv_store_e4m3(_ptr(x), T, W, _ptr(slot_mapping), float(scale),
                                     _ptr(cache), S, _stream(x.device)))
    return cache


def kv_load_e4m3(cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                 page_size: int, max_len: int, scale: float, out=None) -> torch.Tensor:
    """Sequences back from the cache through their block tables (int32
    [B, max_pages]) -> bf16 [B, max_len, W]; rows past seq_lens[b] are zero."""
    S, W = _dims(cache, "cache", 2)
    _arg(cache, "cache", torch.uint8)
    B, max_pages = _dims(block_table, "block_table", 2)
    _arg(block_table, "block_table", torch.int32)
    _arg(seq_lens, "seq_lens", torch.int32, (B,))
    _arg(out, "out", torch.bfloat16, (B, max_len, W), optional=True)
    _gpu(cache, block_table, seq_lens, out)
    if out is None:
        out = torch.empty((B, max_len, W), dtype=torch.bfloat16, device=cache.device)
    _check(lib().nvfp4_kv_load_e4m3(_ptr(cache), S, W, _ptr(block_table), _ptr(seq_lens), B,
                                    max_pages, page_size, max_len, float(scale), _ptr(out),
                                    _stream(cache.device)))
    return out


def gemm_w4a4(a: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, row_idx=None,
              out_dtype=torch.bfloat16, out=None, workspace=None, plan=None) -> torch.Tensor:
    """W4A4 product from bf16 activations [M, K]: the activations are quantized
    to NVFP4 inside the call (identical to quantize() then gemm())."""
    M, K = _dims(a, "a", 2)
    _arg(a, "a", torch.bfloat16)
    N, _ = _weights(w_codes, w_scales, K)
    n_out = _rows(row_idx, N)
    odt = _out_dtype(out_dtype)
    _arg(out, "out", out_dtype, (M, n_out), optional=True)
    _gpu(a, w_codes, w_scales, row_idx, out, workspace)
    if out is None:
        out = torch.empty((M, n_out), dtype=out_dtype, device=a.device)
    if plan is not None:
        need = lib().nvfp4_gemm_w4a4_bf16_workspace_size_planned(_plan_ref(plan), M, N, K, n_out)
    else:
        need = lib().nvfp4_gemm_w4a4_bf16_workspace_size(M, N, K, n_out)
    ws, wsz = _workspace(int(need), a.device, workspace)
    args = (_ptr(a), M, N, K, _ptr(w_codes), _ptr(w_scales), _ptr(row_idx), n_out, odt, _ptr(out),
            _ptr(ws), wsz, _stream(a.device))
    if plan is not None:
        _check(lib().nvfp4_gemm_w4a4_bf16_planned(_plan_ref(plan), *args))
    else:
        _check(lib().nvfp4_gemm_w4a4_bf16(*args))
    return out


# ---- routed mixture of experts --------------------------------------------------------

def moe_align(topk_ids: torch.Tensor, num_experts: int, gates=None):
    """int32 [T, topk] expert ids -> (offsets [E+1], gather_idx [T*topk],
    slot_pos [T, topk], row_gates [T*topk] or None).  With gates (fp32 [T, topk])
    the gate weights are also permuted into grouped-row order."""
    T, topk = _dims(topk_ids, "topk_ids", 2)
    _arg(topk_ids, "topk_ids", torch.int32)
    _arg(gates, "gates", torch.float32, (T, topk), optional=True)
    _gpu(topk_ids, gates)
    dev = topk_ids.device
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    gather = torch.empty(T * topk, dtype=torch.int32, device=dev)
    slot = torch.empty((T, topk), dtype=torch.int32, device=dev)
    row_gates = None
    if gates is not None:
        row_gates = torch.empty(T * topk, dtype=torch.float32, device=dev)
    nbytes = int(lib().nvfp4_moe_align_workspace_size(T, topk, num_experts))
    ws, wsz = _workspace(nbytes, dev)
    _check(lib().nvfp4_moe_align(_ptr(topk_ids), _ptr(gates), T, topk, num_experts,
                                 _ptr(offsets), _ptr(gather), _ptr(slot), _ptr(row_gates),
                                 _ptr(ws), wsz, _stream(dev)))
    return offsets, gather, slot, row_gates


def grouped_gemm(a: torch.Tensor, gather_idx, expert_offsets: torch.Tensor,
                 w_codes: torch.Tensor, w_scales: torch.Tensor, rows: int, row_scale=None,
                 epilogue: int = EPI_NONE, out=None, plan=None, w_global=None) -> torch.Tensor:
    """Per-expert W4A16 GEMM over `rows` grouped rows (see nvfp4_grouped_gemm).
    w_global (fp32 [E]) holds the experts' global scales of two-level weights
    (nvfp4_grouped_gemm_scaled).  plan (dict or Plan) forces the kernel choice
    (same results)."""
    a_rows, K = _dims(a, "a", 2)
    _arg(a, "a", torch.bfloat16)
    E, N, half = _dims(w_codes, "w_codes", 3)
    _arg(w_codes, "w_codes", torch.uint8)
    if 2 * half != K:
        raise ValueError(f"K mismatch: activations K={K}, weights K={2 * half}")
    _arg(w_scales, "w_scales", torch.uint8, (E, N, K // 16))
    _arg(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    _arg(gather_idx, "gather_idx", torch.int32, (rows,), optional=True)
    _arg(row_scale, "row_scale", torch.float32, (rows,), optional=True)
    _arg(w_global, "w_global", torch.float32, (E,), optional=True)
    width = N // 2 if epilogue == EPI_SWIGLU else N
    _arg(out, "out", torch.bfloat16, (rows, width), optional=True)
    _gpu(a, gather_idx, expert_offsets, w_codes, w_scales, row_scale, w_global, out)
    if out is None:
        out = torch.empty((rows, width), dtype=torch.bfloat16, device=a.device)
    nbytes = int(lib().nvfp4_grouped_gemm_workspace_size(rows, E, N, K))
    ws, wsz = _workspace(nbytes, a.device)
    head = (_ptr(a), a_rows, K, _ptr(gather_idx), _ptr(expert_offsets), E, rows, N,
            _ptr(w_codes), _ptr(w_scales))
    tail = (_ptr(row_scale), epilogue, _ptr(out), _ptr(ws), wsz, _stream(a.device))
    if w_global is not None:
        args = head + (_ptr(w_global),) + tail
        if plan is not None:
            _check(lib().nvfp4_grouped_gemm_scaled_planned(_plan_ref(plan), *args))
        else:
            _check(lib().nvfp4_grouped_gemm_scaled(*args))
    elif plan is not None:
        _check(lib().nvfp4_grouped_gemm_planned(_plan_ref(plan), *head, *tail))
    else:
        _check(lib().nvfp4_grouped_gemm(*head, *tail))
    return out


def tile_experts(w_codes: torch.Tensor, w_scales: torch.Tensor) -> torch.Tensor:
    """Expert weights [E, N, K/2] + [E, N, K/16] (N % 16 == 0) in the tiled layout:
    the stacked E*N-row matrix tiled, so expert e's N/16 tiles follow expert e-1's."""
    E, N, half = _dims(w_codes, "w_codes", 3)
    if N % 16:
        raise ValueError(f"expert rows N={N} must be a multiple of 16")
    _arg(w_scales, "w_scales", torch.uint8, (E, N, 2 * half // 16))
    return tile_weight(w_codes.view(E * N, half), w_scales.view(E * N, 2 * half // 16))


def grouped_gemm_tiled(a: torch.Tensor, gather_idx, expert_offsets: torch.Tensor,
                       w_tiled: torch.Tensor, E: int, N: int, rows: int, row_scale=None,
                       epilogue: int = EPI_NONE, out=None, plan=None,
                       w_global=None) -> torch.Tensor:
    """grouped_gemm on tiled expert weights (tile_experts) of E experts x N rows."""
    a_rows, K = _dims(a, "a", 2)
    _arg(a, "a", torch.bfloat16)
    if K % 32 or N % 16 or E < 1:
        raise ValueError(f"unsupported grouped shape E={E} N={N} K={K}")
    _arg(w_tiled, "w_tiled", torch.uint8, (tiled_weight_bytes(E * N, K),))
    _arg(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    _arg(gather_idx, "gather_idx", torch.int32, (rows,), optional=True)
    _arg(row_scale, "row_scale", torch.float32, (rows,), optional=True)
    _arg(w_global, "w_global", torch.float32, (E,), optional=True)
    width = N // 2 if epilogue == EPI_SWIGLU else N
    _arg(out, "out", torch.bfloat16, (rows, width), optional=True)
    _gpu(a, gather_idx, expert_offsets, w_tiled, row_scale, w_global, out)
    if out is None:
        out = torch.empty((rows, width), dtype=torch.bfloat16, device=a.device)
    nbytes = int(lib().nvfp4_grouped_gemm_workspace_size(rows, E, N, K))
    ws, wsz = _workspace(nbytes, a.device)
    args = (_ptr(a), a_rows, K, _ptr(gather_idx), _ptr(expert_offsets), E, rows, N,
            _ptr(w_tiled), _ptr(w_global), _ptr(row_scale), epilogue, _ptr(out), _ptr(ws), wsz,
            _stream(a.device))
    if plan is not None:
        _check(lib().nvfp4_grouped_gemm_tiled_planned(_plan_ref(plan), *args))
    else:
        _check(lib().nvfp4_grouped_gemm_tiled(*args))
    return out


def moe_combine(y: torch.Tensor, slot_pos: torch.Tensor, out=None) -> torch.Tensor:
    T, topk = _dims(slot_pos, "slot_pos", 2)
    _arg(slot_pos, "slot_pos", torch.int32)
    R, H = _dims(y, "y", 2)
    _arg(y, "y", torch.bfloat16)
    if R != T * topk:
        raise ValueError(f"y has {R} rows; expected T*topk = {T * topk}")
    _arg(out, "out", torch.bfloat16, (T, H), optional=True)
    _gpu(y, slot_pos, out)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _check(lib().nvfp4_moe_combine(_ptr(y), _ptr(slot_pos), T, topk, H, _ptr(out),
                                   _stream(y.device)))
    return out


def moe_layer(x, topk_ids, gates, w1_codes, w1_scales, w2_codes, w2_scales, w1_global=None,
              w2_global=None):
    """Routed MoE layer: align -> grouped gate+up GEMM with SwiGLU -> grouped down
    GEMM scaled by the gate weights -> combine.  All on the current stream.
    w1_global / w2_global (fp32 [E]): per-expert global scales of two-level
    weights."""
    E = w1_codes.shape[0]
    T, topk = _dims(topk_ids, "topk_ids", 2)
    R = T * topk
    offsets, gather, slot, row_gate = moe_align(topk_ids, E, gates)
    act = grouped_gemm(x, gather, offsets, w1_codes, w1_scales, R, epilogue=EPI_SWIGLU,
                       w_global=w1_global)
    y = grouped_gemm(act, None, offsets, w2_codes, w2_scales, R, row_scale=row_gate,
                     w_global=w2_global)
    return moe_combine(y, slot)


def moe_layer_tiled(x, topk_ids, gates, w1_tiled, w2_tiled, E: int, I: int, w1_global=None,
                    w2_global=None):
    """moe_layer on tiled expert weights: w1_tiled = tile_experts of the gate+up
    weights [E, 2I, H/2], w2_tiled of the down weights [E, H, I/2]."""
    T, topk = _dims(topk_ids, "topk_ids", 2)
    H = x.shape[1]
    R = T * topk
    offsets, gather, slot, row_gate = moe_align(topk_ids, E, gates)
    act = grouped_gemm_tiled(x, gather, offsets, w1_tiled, E, 2 * I, R, epilogue=EPI_SWIGLU,
                             w_global=w1_global)
    y = grouped_gemm_tiled(act, None, offsets, w2_tiled, E, H, R, row_scale=row_gate,
                           w_global=w2_global)
    return moe_combine(y, slot)
