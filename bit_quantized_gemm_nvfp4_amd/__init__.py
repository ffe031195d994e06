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
    "grouped_gemm", "moe_combine", "moe_layer", "topk", "head_topk", "kv_store_e4m3", "kv_load_e4m3", "quantize_scaled", "quantize_weight", "gemm_w4a4",
    "dequantize_scaled", "gemm_scaled", "BF16", "FP32", "NVFP4", "EPI_NONE",
    "EPI_SWIGLU",
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
    "nvfp4_moe_combine": ([_vp, _vp, _i64, _i64, _i64, _vp, _vp], _int),
}


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
    for t in tensors:
        if t is not None:
            if not t.is_cuda:
                raise RuntimeError("NVFP4 ops run on the GPU only; got a CPU tensor")
            if not t.is_contiguous():
                raise RuntimeError("NVFP4 ops need contiguous tensors")


def _workspace(nbytes: int, device, workspace=None):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise RuntimeError(f"workspace too small: need {nbytes} bytes")
        return workspace, nbytes
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


# ---- formats -------------------------------------------------------------------------

def dequantize(codes: torch.Tensor, scales: torch.Tensor, out=None) -> torch.Tensor:
    """NVFP4 [N, K/2] codes + [N, K/16] scales -> bf16 [N, K] (exact)."""
    _gpu(codes, scales, out)
    N, K = codes.shape[0], codes.shape[1] * 2
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=codes.device)
    _check(lib().nvfp4_dequantize(_ptr(codes), _ptr(scales), N, K, _ptr(out),
                                  _stream(codes.device)))
    return out


def quantize(x: torch.Tensor, codes=None, scales=None):
    """bf16 [M, K] -> (codes uint8 [M, K/2], scales uint8 [M, K/16])."""
    _gpu(x, codes, scales)
    if x.dtype != torch.bfloat16:
        raise RuntimeError("quantize expects bf16 activations")
    M, K = x.shape
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    _check(lib().nvfp4_quantize(_ptr(x), M, K, _ptr(codes), _ptr(scales), _stream(x.device)))
    return codes, scales


# ---- linear layer --------------------------------------------------------------------

def gemm_workspace_size(M: int, N: int, K: int, n_out: int | None = None,
                        w4a4: bool = False) -> int:
    return int(lib().nvfp4_gemm_workspace_size(NVFP4 if w4a4 else BF16, M, N, K,
                                               N if n_out is None else n_out))


def gemm(a: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, a_scales=None,
         row_idx=None, out_dtype=torch.bfloat16, out=None, workspace=None) -> torch.Tensor:
    """y = a . W^T.  a is bf16 [M, K] (W4A16) or NVFP4 codes [M, K/2] with
    a_scales [M, K/16] (W4A4).  row_idx (int32, sorted) restricts the output to
    those weight rows."""
    _gpu(a, w_codes, w_scales, a_scales, row_idx, out, workspace)
    w4a4 = a_scales is not None
    M = a.shape[0]
    K = a.shape[1] * (2 if w4a4 else 1)
    N = w_codes.shape[0]
    if w_codes.shape[1] * 2 != K:
        raise RuntimeError(f"K mismatch: activations K={K}, weights K={w_codes.shape[1] * 2}")
    n_out = N if row_idx is None else row_idx.numel()
    odt = {torch.bfloat16: BF16, torch.float32: FP32}[out_dtype]
    if out is None:
        out = torch.empty((M, n_out), dtype=out_dtype, device=a.device)
    ws, wsz = _workspace(gemm_workspace_size(M, N, K, n_out, w4a4), a.device, workspace)
    _check(lib().nvfp4_gemm(NVFP4 if w4a4 else BF16, _ptr(a), _ptr(a_scales), M, N, K,
                            _ptr(w_codes), _ptr(w_scales), _ptr(row_idx), n_out, odt, _ptr(out),
                            _ptr(ws), wsz, _stream(a.device)))
    return out


# ---- two-level NVFP4 (per-tensor fp32 scale on the device) ------------------------------

def quantize_scaled(x: torch.Tensor, global_scale: torch.Tensor, codes=None, scales=None):
    """bf16 [M, K] with a per-tensor scale (fp32 tensor of one element on the
    GPU) -> (codes, scales) of fl32(x / g)."""
    _gpu(x, global_scale, codes, scales)
    M, K = x.shape
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    _check(lib().nvfp4_quantize_scaled(_ptr(x), M, K, _ptr(global_scale), _ptr(codes),
                                       _ptr(scales), _stream(x.device)))
    return codes, scales


def quantize_weight(w: torch.Tensor, workspace=None):
    """Offline weight quantizer: bf16 [N, K] -> (codes [N, K/2], scales
    [N, K/16], global_scale fp32 [1]), all on the GPU."""
    _gpu(w, workspace)
    N, K = w.shape
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, K // 16), dtype=torch.uint8, device=w.device)
    g = torch.empty(1, dtype=torch.float32, device=w.device)
    ws, wsz = _workspace(int(lib().nvfp4_quantize_weight_workspace_size(N, K)), w.device,
                         workspace)
    _check(lib().nvfp4_quantize_weight(_ptr(w), N, K, _ptr(codes), _ptr(scales), _ptr(g),
                                       _ptr(ws), wsz, _stream(w.device)))
    return codes, scales, g


def dequantize_scaled(codes: torch.Tensor, scales: torch.Tensor, global_scale: torch.Tensor,
                      out=None) -> torch.Tensor:
    """Two-level NVFP4 -> bf16 [N, K]: bf16(fl32(e2m1 * e4m3 * g))."""
    _gpu(codes, scales, global_scale, out)
    N, K = codes.shape[0], codes.shape[1] * 2
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
    _gpu(a, w_codes, w_scales, w_global_scale, a_scales, a_global_scale, row_idx, out, workspace)
    w4a4 = a_scales is not None
    M = a.shape[0]
    K = a.shape[1] * (2 if w4a4 else 1)
    N = w_codes.shape[0]
    if w_codes.shape[1] * 2 != K:
        raise RuntimeError(f"K mismatch: activations K={K}, weights K={w_codes.shape[1] * 2}")
    n_out = N if row_idx is None else row_idx.numel()
    odt = {torch.bfloat16: BF16, torch.float32: FP32}[out_dtype]
    if out is None:
        out = torch.empty((M, n_out), dtype=out_dtype, device=a.device)
    ws, wsz = _workspace(gemm_workspace_size(M, N, K, n_out, w4a4), a.device, workspace)
    _check(lib().nvfp4_gemm_scaled(NVFP4 if w4a4 else BF16, _ptr(a), _ptr(a_scales),
                                   _ptr(a_global_scale), M, N, K, _ptr(w_codes), _ptr(w_scales),
                                   _ptr(w_global_scale), _ptr(row_idx), n_out, odt, _ptr(out),
                                   _ptr(ws), wsz, _stream(a.device)))
    return out


# ---- draft proposal from the masked head ----------------------------------------------

def topk(logits: torch.Tensor, k: int, ids_map=None, workspace=None):
    """Top-k of each row of fp32 logits [M, n], best first (larger value, then
    smaller column; -0 below +0) -> (values fp32 [M, k], ids int32 [M, k]).
    ids are ids_map[column] when ids_map (int32 [n]) is given."""
    _gpu(logits, ids_map, workspace)
    if logits.dtype != torch.float32:
        raise RuntimeError("topk expects fp32 logits")
    M, n = logits.shape
    values = torch.empty((M, k), dtype=torch.float32, device=logits.device)
    ids = torch.empty((M, k), dtype=torch.int32, device=logits.device)
    ws, wsz = _workspace(int(lib().nvfp4_topk_workspace_size(M, n, k)), logits.device, workspace)
    _check(lib().nvfp4_topk(_ptr(logits), M, n, k, _ptr(ids_map), _ptr(values), _ptr(ids),
                            _ptr(ws), wsz, _stream(logits.device)))
    return values, ids


def head_topk_workspace_size(M: int, N: int, K: int, n_out: int, k: int) -> int:
    return int(lib().nvfp4_head_topk_workspace_size(M, N, K, n_out, k))


def head_topk(a: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, k: int,
              row_idx=None, workspace=None):
    """Masked draft head and its proposal: fp32 logits of the W4A16 head over
    the rows row_idx (all rows if None), then their top-k -> (values fp32
    [M, k], ids int32 [M, k]); ids are weight-row (token) ids."""
    _gpu(a, w_codes, w_scales, row_idx, workspace)
    M, K = a.shape
    N = w_codes.shape[0]
    if w_codes.shape[1] * 2 != K:
        raise RuntimeError(f"K mismatch: activations K={K}, weights K={w_codes.shape[1] * 2}")
    n_out = N if row_idx is None else row_idx.numel()
    values = torch.empty((M, k), dtype=torch.float32, device=a.device)
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
    _gpu(x, slot_mapping, cache)
    T, W = x.shape
    if cache.dtype != torch.uint8 or cache.shape[1] != W:
        raise RuntimeError("cache must be uint8 [num_slots, W]")
    _check(lib().nvfp4_kv_store_e4m3(_ptr(x), T, W, _ptr(slot_mapping), float(scale),
                                     _ptr(cache), cache.shape[0], _stream(x.device)))
    return cache


def kv_load_e4m3(cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                 page_size: int, max_len: int, scale: float, out=None) -> torch.Tensor:
    """Sequences back from the cache through their block tables (int32
    [B, max_pages]) -> bf16 [B, max_len, W]; rows past seq_lens[b] are zero."""
    _gpu(cache, block_table, seq_lens, out)
    B, max_pages = block_table.shape
    W = cache.shape[1]
    if out is None:
        out = torch.empty((B, max_len, W), dtype=torch.bfloat16, device=cache.device)
    _check(lib().nvfp4_kv_load_e4m3(_ptr(cache), cache.shape[0], W, _ptr(block_table),
                                    _ptr(seq_lens), B, max_pages, page_size, max_len,
                                    float(scale), _ptr(out), _stream(cache.device)))
    return out


def gemm_w4a4(a: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, row_idx=None,
              out_dtype=torch.bfloat16, out=None, workspace=None) -> torch.Tensor:
    """W4A4 product from bf16 activations [M, K]: the activations are quantized
    to NVFP4 inside the call (identical to quantize() then gemm())."""
    _gpu(a, w_codes, w_scales, row_idx, out, workspace)
    M, K = a.shape
    N = w_codes.shape[0]
    if w_codes.shape[1] * 2 != K:
        raise RuntimeError(f"K mismatch: activations K={K}, weights K={w_codes.shape[1] * 2}")
    n_out = N if row_idx is None else row_idx.numel()
    odt = {torch.bfloat16: BF16, torch.float32: FP32}[out_dtype]
    if out is None:
        out = torch.empty((M, n_out), dtype=out_dtype, device=a.device)
    ws, wsz = _workspace(int(lib().nvfp4_gemm_w4a4_bf16_workspace_size(M, N, K, n_out)),
                         a.device, workspace)
    _check(lib().nvfp4_gemm_w4a4_bf16(_ptr(a), M, N, K, _ptr(w_codes), _ptr(w_scales),
                                      _ptr(row_idx), n_out, odt, _ptr(out), _ptr(ws), wsz,
                                      _stream(a.device)))
    return out


# ---- routed mixture of experts --------------------------------------------------------

def moe_align(topk_ids: torch.Tensor, num_experts: int, gates=None):
    """int32 [T, topk] expert ids -> (offsets [E+1], gather_idx [T*topk],
    slot_pos [T, topk], row_gates [T*topk] or None).  With gates (fp32 [T, topk])
    the gate weights are also permuted into grouped-row order."""
    _gpu(topk_ids, gates)
    T, topk = topk_ids.shape
    dev = topk_ids.device
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    gather = torch.empty(T * topk, dtype=torch.int32, device=dev)
    slot = torch.empty((T, topk), dtype=torch.int32, device=dev)
    row_gates = None
    if gates is not None:
        if gates.dtype != torch.float32:
            raise RuntimeError("gates must be float32")
        row_gates = torch.empty(T * topk, dtype=torch.float32, device=dev)
    nbytes = int(lib().nvfp4_moe_align_workspace_size(T, topk, num_experts))
    ws, wsz = _workspace(nbytes, dev)
    _check(lib().nvfp4_moe_align(_ptr(topk_ids), _ptr(gates), T, topk, num_experts,
                                 _ptr(offsets), _ptr(gather), _ptr(slot), _ptr(row_gates),
                                 _ptr(ws), wsz, _stream(dev)))
    return offsets, gather, slot, row_gates


def grouped_gemm(a: torch.Tensor, gather_idx, expert_offsets: torch.Tensor,
                 w_codes: torch.Tensor, w_scales: torch.Tensor, rows: int, row_scale=None,
                 epilogue: int = EPI_NONE, out=None) -> torch.Tensor:
    """Per-expert W4A16 GEMM over `rows` grouped rows (see nvfp4_grouped_gemm)."""
    _gpu(a, gather_idx, expert_offsets, w_codes, w_scales, row_scale, out)
    E, N = w_codes.shape[0], w_codes.shape[1]
    K = w_codes.shape[2] * 2
    width = N // 2 if epilogue == EPI_SWIGLU else N
    if out is None:
        out = torch.empty((rows, width), dtype=torch.bfloat16, device=a.device)
    nbytes = int(lib().nvfp4_grouped_gemm_workspace_size(rows, E, N, K))
    ws, wsz = _workspace(nbytes, a.device)
    _check(lib().nvfp4_grouped_gemm(_ptr(a), a.shape[0], K, _ptr(gather_idx),
                                    _ptr(expert_offsets), E, rows, N, _ptr(w_codes),
                                    _ptr(w_scales), _ptr(row_scale), epilogue, _ptr(out),
                                    _ptr(ws), wsz, _stream(a.device)))
    return out


def moe_combine(y: torch.Tensor, slot_pos: torch.Tensor, out=None) -> torch.Tensor:
    _gpu(y, slot_pos, out)
    T, topk = slot_pos.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _check(lib().nvfp4_moe_combine(_ptr(y), _ptr(slot_pos), T, topk, H, _ptr(out),
                                   _stream(y.device)))
    return out


def moe_layer(x, topk_ids, gates, w1_codes, w1_scales, w2_codes, w2_scales):
    """Routed MoE layer: align -> grouped gate+up GEMM with SwiGLU -> grouped down
    GEMM scaled by the gate weights -> combine.  All on the current stream."""
    _gpu(x, topk_ids, gates)
    E = w1_codes.shape[0]
    T, topk = topk_ids.shape
    R = T * topk
    offsets, gather, slot, row_gate = moe_align(topk_ids, E, gates)
    act = grouped_gemm(x, gather, offsets, w1_codes, w1_scales, R, epilogue=EPI_SWIGLU)
    y = grouped_gemm(act, None, offsets, w2_codes, w2_scales, R, row_scale=row_gate)
    return moe_combine(y, slot)
