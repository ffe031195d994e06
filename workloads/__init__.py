"""Seeded synthetic inputs shaped like the layers the pages serve.

This module only draws random numbers.  It holds none of the NVFP4 method's
arithmetic, and both the CPU oracle side and the HIP side take their inputs
from it.  Every generator starts a fresh ``numpy.random.default_rng(seed)``
(seed 0 unless told otherwise) and draws its tensors in the order documented
on the function, so any slice of a workload can be regenerated bit for bit.

Shapes stand in for the pages' models:
  - dense 27B layers ("Serving Qwen3.8-27B in 4-bit with a masked speculative
    decoding head"; Prefill Systems' "Qwen3.8-27B" benchmark page): hidden
    5120, MLP 17408, an output head of 248,320 vocabulary rows of which the
    draft head keeps a ranked 32,768 ("The masked head trick");
  - a routed 35B-A3B mixture of experts ("What 350+ Experiments Taught Us
    About Serving Qwen 3.6 35B-A3B", section 1): 128 experts, top-8,
    hidden 2048, expert intermediate 768.
Batch sizes: M = 1, 8 (one stream verifying 7 drafts + 1; concurrency 8) and
32 (4 streams x 8) for decode; M = 8192 for a prefill chunk (an ~8k-token
prompt, below the 16,384 batch-token limit).

bf16 values are returned as uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

HIDDEN = 5120
MLP = 17408
VOCAB = 248320
MASKED_ROWS = 32768
MOE_EXPERTS = 128
MOE_TOPK = 8
MOE_HIDDEN = 2048
MOE_INTER = 768


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 samples to bf16 (nearest, ties to even); used only to turn
    random draws into bf16 inputs."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


@dataclass
class NF4W:
    """An NVFP4 matrix: codes uint8 [R, K/2], scales uint8 [R, K/16]."""
    codes: np.ndarray
    scales: np.ndarray

    @property
    def rows(self) -> int:
        return self.codes.shape[-2]

    @property
    def K(self) -> int:
        return self.codes.shape[-1] * 2


def nvfp4_weight(rng: np.random.Generator, *shape_rows_k, exp_field=(3, 9)) -> NF4W:
    """Random NVFP4 weights.  Draw order: codes, scale exponents, scale
    mantissas.  Codes: every byte uniform over 0..255 (both nibbles uniform
    over all 16 e2m1 codes, negative zero included).  Scales: E4M3 with the
    biased exponent field uniform over exp_field (inclusive; the default 3..9
    gives 2^-4 .. 2^2 before the mantissa) and the 3-bit mantissa uniform;
    sign 0.  A drawn 0x7F (exponent field 15, mantissa 7: the NaN code) is
    replaced by 0x7E (448)."""
    *lead, R, K = shape_rows_k
    codes = rng.integers(0, 256, size=(*lead, R, K // 2), dtype=np.uint8)
    e = rng.integers(exp_field[0], exp_field[1] + 1, size=(*lead, R, K // 16), dtype=np.uint8)
    m = rng.integers(0, 8, size=(*lead, R, K // 16), dtype=np.uint8)
    return NF4W(codes, np.minimum((e << 3) | m, 0x7E).astype(np.uint8))


def normal_bf16(rng: np.random.Generator, M: int, K: int, outlier_frac: float = 0.0) -> np.ndarray:
    """N(0,1) activations rounded to bf16.  With outlier_frac > 0,
    round(outlier_frac*K) channels (columns), drawn without replacement after
    the values, are multiplied by 20 before rounding."""
    x = rng.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(outlier_frac * K))
    if n_out:
        cols = rng.choice(K, size=n_out, replace=False)
        x[:, cols] *= np.float32(20.0)
    return f32_to_bf16_bits(x)


def masked_rows(rng: np.random.Generator, n_rows: int = VOCAB, n_keep: int = MASKED_ROWS) -> np.ndarray:
    """Sorted, unique int32 row indices drawn uniformly without replacement."""
    return np.sort(rng.choice(n_rows, size=n_keep, replace=False)).astype(np.int32)


# ---- the workloads ------------------------------------------------------------

def tiny(seed: int = 0):
    """M=1, K=512, N=1024.  Draws: x, then weights."""
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, 1, 512)
    w = nvfp4_weight(rng, 1024, 512)
    return x, w


DECODE_SHAPES = [(HIDDEN, MLP), (MLP, HIDDEN), (HIDDEN, VOCAB)]  # (K, N)
DECODE_M = [1, 8, 32]


def decode_weights(K: int, N: int, seed: int = 0) -> NF4W:
    """Weights of one decode shape.  Draws: weights only."""
    return nvfp4_weight(np.random.default_rng(seed), N, K)


def decode_activations(M: int, K: int, seed: int = 0) -> np.ndarray:
    """Decode activations, drawn from their own stream (seed + 1000 + M) so that
    every M can be regenerated alone."""
    return normal_bf16(np.random.default_rng(seed + 1000 + M), M, K)


def decode_masked_rows(seed: int = 0) -> np.ndarray:
    """The 32,768 kept head rows, drawn from their own stream (seed + 7)."""
    return masked_rows(np.random.default_rng(seed + 7))


def prefill(K: int, N: int, M: int = 8192, seed: int = 0):
    """Prefill chunk: x [M, K] N(0,1) with 0.1% outlier channels x20, then
    weights NF4W(N, K).  Draws: x values, outlier columns, weights."""
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, M, K, outlier_frac=0.001)
    w = nvfp4_weight(rng, N, K)
    return x, w


def w4a4(M: int = 512, K: int = HIDDEN, N: int = MLP, seed: int = 0):
    """W4A4 path: bf16 activations [M, K] with the outlier profile (quantized
    at run time), then weights NF4W(N, K)."""
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, M, K, outlier_frac=0.001)
    w = nvfp4_weight(rng, N, K)
    return x, w


@dataclass
class MoEWorkload:
    x: np.ndarray        # bf16 bits [T, H]
    ids: np.ndarray      # int32 [T, topk]
    gates: np.ndarray    # float32 [T, topk], softmax-normalised
    w1: NF4W             # [E, 2I, H/2] gate rows 0..I-1, up rows I..2I-1
    w2: NF4W             # [E, H, I/2]


def zipf_routing(rng: np.random.Generator, T: int, E: int, topk: int, s: float = 1.1):
    """Top-k routing with Zipf(s) expert popularity.  Draws: a permutation of the
    experts (popularity ranks 1..E), then a Gumbel(0,1) matrix [T, E].  Scores
    are -s*ln(rank) + Gumbel (Gumbel-top-k sampling without replacement with
    probabilities proportional to rank^-s); each token keeps its topk best
    experts (ties to the lower id) and its gates are the softmax of the kept
    scores (fp64, then float32)."""
    rank = rng.permutation(E).astype(np.float64) + 1.0
    g = rng.gumbel(size=(T, E))
    scores = -s * np.log(rank)[None, :] + g
    order = np.argsort(-scores, axis=1, kind="stable")[:, :topk]
    ids = order.astype(np.int32)
    sel = np.take_along_axis(scores, order, axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    gates = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, gates


# Expert weights look like a trained checkpoint quantized with the amax/6 rule
# and no per-tensor scale: element rms near 1/sqrt(fan-in) puts the E4M3 block
# scales around 2^-9 .. 2^-5 -- exponent fields 0 (subnormal, including the zero
# scale) to 2 -- which keeps the routed layer's activations of order one to ten.
MOE_SCALE_EXP_FIELD = (0, 2)


def moe(T: int, E: int = MOE_EXPERTS, topk: int = MOE_TOPK, H: int = MOE_HIDDEN,
        I: int = MOE_INTER, seed: int = 0, exp_field=MOE_SCALE_EXP_FIELD) -> MoEWorkload:
    """Routed MoE layer.  Draws: x [T, H] N(0,1), routing, W1 NF4W(E x 2I, H),
    W2 NF4W(E x H, I), both with scale exponent fields exp_field (default
    MOE_SCALE_EXP_FIELD; (3, 9) gives the dense layers' 2^-4 .. 2^2 scales)."""
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, T, H)
    ids, gates = zipf_routing(rng, T, E, topk)
    w1 = nvfp4_weight(rng, E, 2 * I, H, exp_field=exp_field)
    w2 = nvfp4_weight(rng, E, H, I, exp_field=exp_field)
    return MoEWorkload(x, ids, gates, w1, w2)


# Two-level expert weights (a per-expert fp32 global scale above the E4M3 block
# scales), as a quantizer that puts each expert's largest block at scale 448
# would leave them: block scales near the top of the E4M3 range (exponent fields
# 11..15, 2^4 .. 448) and global scales around 2^-14 .. 2^-12, so that the
# products scale * g fall near the single-level expert scales above.
MOE_TWO_LEVEL_EXP_FIELD = (11, 15)


def expert_global_scales(rng: np.random.Generator, E: int, exp_range=(-14, -13)) -> np.ndarray:
    """Per-expert fp32 global scales 2^u * (1 + f): u an integer uniform over
    exp_range (inclusive), f uniform in [0, 1); one draw of u, then one of f."""
    u = rng.integers(exp_range[0], exp_range[1] + 1, size=E)
    f = rng.random(E)
    return (np.ldexp(1.0 + f, u)).astype(np.float32)


def moe_two_level(T: int, E: int = MOE_EXPERTS, topk: int = MOE_TOPK, H: int = MOE_HIDDEN,
                  I: int = MOE_INTER, seed: int = 0):
    """Routed MoE layer with two-level expert weights: moe(..., exp_field =
    MOE_TWO_LEVEL_EXP_FIELD), then the W1 and W2 global scales [E] (fp32) from
    the same generator.  Returns (workload, w1_global, w2_global)."""
    wl = moe(T, E=E, topk=topk, H=H, I=I, seed=seed, exp_field=MOE_TWO_LEVEL_EXP_FIELD)
    rng = np.random.default_rng(seed + 7919)
    return wl, expert_global_scales(rng, E), expert_global_scales(rng, E)


# ---- FP8 E4M3 KV cache ------------------------------------------------------------
# Synthetic attention-cache shape: 8 key/value heads of 128 elements, so a token
# row of K (or of V) holds KV_W = 1024 elements; 16-token pages, the default the
# pages report (32-token pages were slower there).
KV_HEADS, KV_HEAD_DIM = 8, 128
KV_W = KV_HEADS * KV_HEAD_DIM
KV_PAGE = 16


@dataclass
class KVWorkload:
    x: np.ndarray             # bf16 bits [T, W]: token rows to store
    slot_mapping: np.ndarray  # int32 [T]: cache slot of each token
    scale: float              # per-cache scale: amax / 448, rounded to fp32
    num_slots: int


def kv_store(T: int, W: int = KV_W, page: int = KV_PAGE, spare_pages: int = 64,
             seed: int = 0) -> KVWorkload:
    """Prefill-shaped KV store: T new tokens of one sequence.  Draws: x [T, W]
    N(0,1) with 0.1% outlier channels x20 (bf16), then a permutation of the
    cache's pages.  The cache has ceil(T/page) + spare_pages pages; token t
    goes to position t % page of the sequence's (t // page)-th page."""
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, T, W, outlier_frac=0.001)
    n_pages = (T + page - 1) // page + spare_pages
    pages = rng.permutation(n_pages)[: (T + page - 1) // page].astype(np.int64)
    t = np.arange(T)
    slot = (pages[t // page] * page + t % page).astype(np.int32)
    amax = float(np.abs(bf16_bits_to_f32(x)).max())
    return KVWorkload(x, slot, float(np.float32(amax / 448.0)), n_pages * page)


def kv_load(B: int, max_len: int, W: int = KV_W, page: int = KV_PAGE, seed: int = 0):
    """Decode-shaped KV read: B sequences of lengths uniform in [1, max_len]
    (the longest set to max_len), pages assigned by one permutation of the
    cache.  Draws: lengths, the page permutation, then the cache codes (uniform
    over the 254 finite E4M3 codes).  Returns (cache uint8 [slots, W],
    block_table int32 [B, max_pages], seq_lens int32 [B], scale)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len + 1, size=B).astype(np.int32)
    lens[0] = max_len
    max_pages = (max_len + page - 1) // page
    n_pages = B * max_pages
    perm = rng.permutation(n_pages).astype(np.int32)
    bt = perm.reshape(B, max_pages)
    codes = rng.integers(0, 254, size=(n_pages * page, W)).astype(np.uint8)
    codes[codes >= 0x7F] += 1            # skip the NaN code 0x7F (0xFF is out of range)
    return codes, bt, lens, 0.0123
