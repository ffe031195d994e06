"""CPU oracle for the NVFP4 linear layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 reference (``nvfp4_oracle.c``) plus its ctypes wrapper.  Only
the test suite, the smoke check and the CPU-baseline leg of the benchmark may
import it; the library never does, and the two share no code.

Every function returns plain numpy arrays.  bf16 values travel as ``uint16``
bit patterns.  GEMM-like functions return the unrounded fp64 sums; use
:func:`bf16_round` for the single rounding to a bf16 output.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (host only, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
               "-shared", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None

_p = np.ctypeslib.ndpointer
_i64 = ctypes.c_int64
_U8 = _p(dtype=np.uint8, flags="C_CONTIGUOUS")
_U16 = _p(dtype=np.uint16, flags="C_CONTIGUOUS")
_I32 = _p(dtype=np.int32, flags="C_CONTIGUOUS")
_F32 = _p(dtype=np.float32, flags="C_CONTIGUOUS")
_F64 = _p(dtype=np.float64, flags="C_CONTIGUOUS")


def _nullable(base):
    """ndpointer that also accepts None (passed as NULL)."""

    class _N(base):
        @classmethod
        def from_param(cls, obj):
            if obj is None:
                return None
            return base.from_param(obj)

    return _N


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint]
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_value.restype = ctypes.c_double
        L.oracle_bf16_round.argtypes = [ctypes.c_double]
        L.oracle_bf16_round.restype = ctypes.c_uint16
        L.oracle_bf16_round_array.argtypes = [_F64, _i64, _U16]
        L.oracle_bf16_round_array.restype = None
        L.oracle_scale_code.argtypes = [ctypes.c_double]
        L.oracle_scale_code.restype = ctypes.c_uint
        L.oracle_e2m1_index.argtypes = [ctypes.c_double, ctypes.c_double]
        L.oracle_e2m1_index.restype = ctypes.c_uint
        L.oracle_e2m1_encode.argtypes = [ctypes.c_uint16, ctypes.c_uint]
        L.oracle_e2m1_encode.restype = ctypes.c_uint
        L.oracle_scale_code_array.argtypes = [_F64, _i64, _U8]
        L.oracle_scale_code_array.restype = None
        L.oracle_e2m1_encode_array.argtypes = [_U16, _i64, ctypes.c_uint, _U8]
        L.oracle_e2m1_encode_array.restype = None
        L.oracle_dequantize.argtypes = [_U8, _U8, _i64, _i64, _U16]
        L.oracle_dequantize.restype = None
        L.oracle_tile_weight.argtypes = [_U8, _U8, _i64, _i64, _U8]
        L.oracle_tile_weight.restype = None
        L.oracle_quantize.argtypes = [_U16, _i64, _i64, _U8, _U8]
        L.oracle_quantize.restype = None
        L.oracle_gemm_w4a16.argtypes = [_U16, _i64, _i64, _U8, _U8, _nullable(_I32), _i64, _F64]
        L.oracle_gemm_w4a16.restype = None
        L.oracle_gemm_w4a4.argtypes = [_U8, _U8, _i64, _i64, _U8, _U8, _nullable(_I32), _i64,
                                       _F64]
        L.oracle_gemm_w4a4.restype = None
        L.oracle_moe_align.argtypes = [_I32, _i64, _i64, _i64, _I32, _I32, _I32]
        L.oracle_moe_align.restype = ctypes.c_int
        L.oracle_grouped_gemm.argtypes = [_U16, _i64, _nullable(_I32), _I32, _i64, _i64, _i64,
                                          _U8, _U8, _nullable(_F32), _nullable(_F32),
                                          ctypes.c_int, _F64]
        L.oracle_grouped_gemm.restype = None
        L.oracle_moe_combine.argtypes = [_U16, _I32, _i64, _i64, _i64, _F64]
        L.oracle_moe_combine.restype = None
        L.oracle_moe_layer.argtypes = [_U16, _i64, _i64, _I32, _F32, _i64, _i64, _i64,
                                       _U8, _U8, _U8, _U8, _nullable(_F32), _nullable(_F32),
                                       _F64]
        L.oracle_moe_layer.restype = None
        L.oracle_topk.argtypes = [_F64, _i64, _i64, _i64, _nullable(_I32), _F64, _I32]
        L.oracle_topk.restype = None
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_e4m3_encode.restype = ctypes.c_uint
        L.oracle_kv_store_e4m3.argtypes = [_U16, _i64, _i64, _I32, ctypes.c_float, _U8, _i64]
        L.oracle_kv_store_e4m3.restype = None
        L.oracle_kv_load_e4m3.argtypes = [_U8, _i64, _i64, _I32, _I32, _i64, _i64, _i64, _i64,
                                          ctypes.c_float, _U16]
        L.oracle_kv_load_e4m3.restype = None
        L.oracle_global_scale.argtypes = [ctypes.c_double]
        L.oracle_global_scale.restype = ctypes.c_float
        L.oracle_quantize_scaled.argtypes = [_U16, _i64, _i64, ctypes.c_float, _U8, _U8]
        L.oracle_quantize_scaled.restype = None
        L.oracle_quantize_weight.argtypes = [_U16, _i64, _i64, _U8, _U8]
        L.oracle_quantize_weight.restype = ctypes.c_float
        L.oracle_dequantize_scaled.argtypes = [_U8, _U8, ctypes.c_float, _i64, _i64, _U16]
        L.oracle_dequantize_scaled.restype = None
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- scalar format functions ------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(code)


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(code)


def bf16_value(bits: int) -> float:
    return lib().oracle_bf16_value(bits)


def scale_code(amax: float) -> int:
    return lib().oracle_scale_code(amax)


def e2m1_encode(x_bits: int, scale_code_: int) -> int:
    return lib().oracle_e2m1_encode(x_bits, scale_code_)


def scale_codes(amax) -> np.ndarray:
    """Scale code for every block maximum in amax (fp64 array)."""
    a = np.ascontiguousarray(amax, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint8)
    lib().oracle_scale_code_array(a.reshape(-1), a.size, out.reshape(-1))
    return out


def e2m1_encodes(x_bits, scale_code_: int) -> np.ndarray:
    """4-bit code of every bf16 value in x_bits under one scale code."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_e2m1_encode_array(x.reshape(-1), x.size, scale_code_, out.reshape(-1))
    return out


def num_threads() -> int:
    return lib().oracle_num_threads()


# ---- array functions ---------------------------------------------------------

def bf16_round(v) -> np.ndarray:
    """fp64 array -> bf16 bit patterns (uint16), nearest-even, one rounding."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_bf16_round_array(v.reshape(-1), v.size, out.reshape(-1))
    return out


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> fp64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def tiled_weight_bytes(N: int, K: int) -> int:
    return ((N + 15) // 16) * ((K + 255) // 256) * 2304


def tile_weight(codes, scales, N: int, K: int) -> np.ndarray:
    """The tiled byte order of NF4W(N, K) (uint8, tiled_weight_bytes(N, K))."""
    out = np.empty(tiled_weight_bytes(N, K), dtype=np.uint8)
    lib().oracle_tile_weight(_c(codes, np.uint8), _c(scales, np.uint8), N, K, out)
    return out


def dequantize(codes, scales, N: int, K: int) -> np.ndarray:
    out = np.empty((N, K), dtype=np.uint16)
    lib().oracle_dequantize(_c(codes, np.uint8), _c(scales, np.uint8), N, K, out)
    return out


def quantize(x_bits, M: int, K: int):
    codes = np.empty((M, K // 2), dtype=np.uint8)
    scales = np.empty((M, K // 16), dtype=np.uint8)
    lib().oracle_quantize(_c(x_bits, np.uint16), M, K, codes, scales)
    return codes, scales


def gemm_w4a16(x_bits, M: int, K: int, w_codes, w_scales, row_idx=None, n_out=None):
    if n_out is None:
        n_out = len(row_idx) if row_idx is not None else np.asarray(w_codes).shape[0]
    out = np.empty((M, n_out), dtype=np.float64)
    ri = None if row_idx is None else _c(row_idx, np.int32)
    lib().oracle_gemm_w4a16(_c(x_bits, np.uint16), M, K, _c(w_codes, np.uint8),
                            _c(w_scales, np.uint8), ri, n_out, out)
    return out


def gemm_w4a4(a_codes, a_scales, M: int, K: int, w_codes, w_scales, row_idx=None, n_out=None):
    if n_out is None:
        n_out = len(row_idx) if row_idx is not None else np.asarray(w_codes).shape[0]
    out = np.empty((M, n_out), dtype=np.float64)
    ri = None if row_idx is None else _c(row_idx, np.int32)
    lib().oracle_gemm_w4a4(_c(a_codes, np.uint8), _c(a_scales, np.uint8), M, K,
                           _c(w_codes, np.uint8), _c(w_scales, np.uint8), ri, n_out, out)
    return out


def moe_align(topk_ids, E: int):
    ids = _c(topk_ids, np.int32)
    T, topk = ids.shape
    offsets = np.empty(E + 1, dtype=np.int32)
    gather = np.empty(T * topk, dtype=np.int32)
    slot = np.empty(T * topk, dtype=np.int32)
    rc = lib().oracle_moe_align(ids, T, topk, E, offsets, gather, slot)
    if rc != 0:
        raise ValueError("expert id out of range")
    return offsets, gather, slot.reshape(T, topk)


def grouped_gemm(a_bits, K: int, gather_idx, offsets, E: int, R: int, N: int, w_codes,
                 w_scales, row_scale=None, epilogue: int = 0, w_global=None):
    """Grouped GEMM over experts; w_global (fp32 [E]) is the per-expert global
    scale of two-level weights (None: 1)."""
    width = N // 2 if epilogue == 1 else N
    out = np.empty((R, width), dtype=np.float64)
    gi = None if gather_idx is None else _c(gather_idx, np.int32)
    rs = None if row_scale is None else _c(row_scale, np.float32)
    wg = None if w_global is None else _c(w_global, np.float32)
    if wg is not None and wg.shape != (E,):
        raise ValueError("w_global must hold one scale per expert")
    lib().oracle_grouped_gemm(_c(a_bits, np.uint16), K, gi, _c(offsets, np.int32), E, R, N,
                              _c(w_codes, np.uint8), _c(w_scales, np.uint8), wg, rs, epilogue,
                              out)
    return out


def moe_combine(y_bits, slot_pos, T: int, topk: int, H: int):
    out = np.empty((T, H), dtype=np.float64)
    lib().oracle_moe_combine(_c(y_bits, np.uint16), _c(slot_pos, np.int32), T, topk, H, out)
    return out


def moe_layer(x_bits, ids, gates, E: int, I: int, w1_codes, w1_scales, w2_codes, w2_scales,
              w1_global=None, w2_global=None):
    """The routed-expert layer token by token; w1_global / w2_global (fp32 [E])
    are the per-expert global scales of two-level weights (None: 1)."""
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    topk = np.asarray(ids).shape[1]
    out = np.empty((T, H), dtype=np.float64)
    g1 = None if w1_global is None else _c(w1_global, np.float32)
    g2 = None if w2_global is None else _c(w2_global, np.float32)
    for g in (g1, g2):
        if g is not None and g.shape != (E,):
            raise ValueError("global scales must hold one scale per expert")
    lib().oracle_moe_layer(x, T, H, _c(ids, np.int32), _c(gates, np.float32), topk, E, I,
                           _c(w1_codes, np.uint8), _c(w1_scales, np.uint8),
                           _c(w2_codes, np.uint8), _c(w2_scales, np.uint8), g1, g2, out)
    return out


def topk(v, k: int, ids_map=None):
    """Top-k of each row of v ([M][n], fp64 or fp32) -- best first.

    Returns (values fp64 [M][k], ids int32 [M][k]); ids are ids_map[col] when
    ids_map (the masked head's row indices) is given, else the column.
    Equal values rank the smaller column first; -0 ranks below +0."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    M, n = v.shape
    if not 1 <= k <= n:
        raise ValueError("need 1 <= k <= n")
    out_v = np.empty((M, k), dtype=np.float64)
    out_i = np.empty((M, k), dtype=np.int32)
    im = None if ids_map is None else _c(ids_map, np.int32)
    lib().oracle_topk(v, M, n, k, im, out_v, out_i)
    return out_v, out_i


def head_topk(x_bits, M: int, K: int, w_codes, w_scales, k: int, row_idx=None, n_out=None):
    """Draft proposal of the masked head: fp64 logits of the W4A16 layer over
    the masked rows, then their top-k (ids are weight-row ids)."""
    logits = gemm_w4a16(x_bits, M, K, w_codes, w_scales, row_idx=row_idx, n_out=n_out)
    vals, ids = topk(logits, k, ids_map=row_idx)
    return vals, ids, logits


def e4m3_encode(v: float) -> int:
    """E4M3 code of v: nearest, ties to even code, saturating at +-448."""
    return lib().oracle_e4m3_encode(v)


def kv_store_e4m3(x_bits, slot_mapping, scale: float, cache):
    """Write tokens x (bf16 bits [T][W]) into cache (uint8 [num_slots][W],
    updated in place) at rows slot_mapping[t]; returns cache."""
    x = _c(x_bits, np.uint16)
    T, W = x.shape
    assert cache.dtype == np.uint8 and cache.flags.c_contiguous and cache.shape[1] == W
    lib().oracle_kv_store_e4m3(x, T, W, _c(slot_mapping, np.int32), scale, cache,
                               cache.shape[0])
    return cache


def kv_load_e4m3(cache, block_table, seq_lens, page_size: int, max_len: int, scale: float):
    """Sequences back from the cache: bf16 bits [B][max_len][W]."""
    cache = _c(cache, np.uint8)
    bt = _c(block_table, np.int32)
    B, max_pages = bt.shape
    W = cache.shape[1]
    out = np.empty((B, max_len, W), dtype=np.uint16)
    lib().oracle_kv_load_e4m3(cache, cache.shape[0], W, bt, _c(seq_lens, np.int32), B,
                              max_pages, page_size, max_len, scale, out)
    return out


# ---- two-level NVFP4 (per-tensor fp32 scale) ----------------------------------------

def global_scale(amax: float) -> float:
    """Per-tensor scale of the offline quantizer: fl32(amax / 2688), 1 for 0."""
    return lib().oracle_global_scale(amax)


def quantize_scaled(x_bits, M: int, K: int, g: float):
    """bf16 [M][K] with a given global scale g -> (codes, scales) of fl32(x/g)."""
    codes = np.empty((M, K // 2), dtype=np.uint8)
    scales = np.empty((M, K // 16), dtype=np.uint8)
    lib().oracle_quantize_scaled(_c(x_bits, np.uint16), M, K, g, codes, scales)
    return codes, scales


def quantize_weight(w_bits, N: int, K: int):
    """Offline weight quantizer: bf16 [N][K] -> (codes, scales, g)."""
    codes = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // 16), dtype=np.uint8)
    g = lib().oracle_quantize_weight(_c(w_bits, np.uint16), N, K, codes, scales)
    return codes, scales, float(g)


def dequantize_scaled(codes, scales, g: float, N: int, K: int) -> np.ndarray:
    out = np.empty((N, K), dtype=np.uint16)
    lib().oracle_dequantize_scaled(_c(codes, np.uint8), _c(scales, np.uint8), g, N, K, out)
    return out


def gemm_scaled(x, M: int, K: int, w_codes, w_scales, w_g: float, a_scales=None, a_g: float = 1.0,
                row_idx=None, n_out=None):
    """Two-level product: the single-level sums (W4A16 when a_scales is None,
    else W4A4 with x the activation codes) times a_g * w_g, in fp64."""
    if a_scales is None:
        y = gemm_w4a16(x, M, K, w_codes, w_scales, row_idx=row_idx, n_out=n_out)
    else:
        y = gemm_w4a4(x, a_scales, M, K, w_codes, w_scales, row_idx=row_idx, n_out=n_out)
    return y * (float(a_g) * float(w_g))
