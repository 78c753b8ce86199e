"""FP8 KV cache for the fp64 oracle: code decoding and decode attention over FP8 pools.

TEST INFRASTRUCTURE ONLY (as the rest of ``oracle/``): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import it.

The pages name the two 8-bit float formats ("注意力机制深度优化" (kler.cn), §一.1 loads a model
with ``torch.float8_e4m3fn``; the "H100 FP8 Tensor Core优化" item of the same page uses
``torch.float8_e5m2``) but define neither them nor any scaling.  The formats are the published
OCP 8-bit floating point definitions (OFP8, Open Compute Project, 2023):

  E4M3 ("fn"): sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent field 0 gives
               subnormals 2^-6 * m/8; field 15 with mantissa 7 is NaN (no infinities, so the
               largest finite value is 2^8 * 1.75 = 448).
  E5M2:        sign bit, 5 exponent bits (bias 15), 2 mantissa bits.  Exponent field 0 gives
               subnormals 2^-14 * m/4; field 31 is infinity (mantissa 0) or NaN.

Reading taken for the scaling the pages leave open: one fp32 scale per pool, real value =
scale * decoded code (k_scale for K, v_scale for V), as a per-tensor-scaled FP8 cache stores it.
The attention itself is decode() / decode_paged() / attention() of attention.py on the
dequantized tensors.
"""
from __future__ import annotations

import numpy as np

from .attention import attention, decode, decode_paged

FORMATS = ("e4m3fn", "e5m2")


def decode_e4m3fn(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8), fp64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)
    return sign * val


def decode_e5m2(codes) -> np.ndarray:
    """Value of each E5M2 code (uint8), fp64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    mi = c & 0x3
    m = mi.astype(np.float64)
    val = np.where(e == 0, np.ldexp(m / 4.0, -14), np.ldexp(1.0 + m / 4.0, e - 15))
    val = np.where(e == 31, np.where(mi == 0, np.inf, np.nan), val)
    return sign * val


def dequantize(codes, scale: float, fmt: str) -> np.ndarray:
    """scale * value of each code."""
    if fmt == "e4m3fn":
        return float(scale) * decode_e4m3fn(codes)
    if fmt == "e5m2":
        return float(scale) * decode_e5m2(codes)
    raise ValueError(f"unknown FP8 format {fmt!r}")


def decode_fp8kv(q, k_codes, v_codes, offsets, lens, k_scale: float, v_scale: float, fmt: str,
                 scale: float | None = None, window: int = 0, threads: int | None = None, seqs=None):
    """decode() with the K and V pools held as FP8 codes [T, Hkv, d] (uint8) and per-pool scales."""
    return decode(q, dequantize(k_codes, k_scale, fmt), dequantize(v_codes, v_scale, fmt), offsets, lens,
                  scale=scale, window=window, threads=threads, seqs=seqs)


def decode_paged_fp8kv(q, k_codes, v_codes, block_table, lens, page_size: int, k_scale: float, v_scale: float,
                       fmt: str, scale: float | None = None, window: int = 0, threads: int | None = None,
                       seqs=None):
    """decode_paged() with FP8 pools, as decode_fp8kv()."""
    return decode_paged(q, dequantize(k_codes, k_scale, fmt), dequantize(v_codes, v_scale, fmt), block_table,
                        lens, page_size, scale=scale, window=window, threads=threads, seqs=seqs)


def attention_fp8(q_codes, k_codes, v_codes, q_scale: float, k_scale: float, v_scale: float, fmt: str,
                  scale: float | None = None, causal: bool = False, window: int = 0, threads: int | None = None):
    """attention() of Q, K and V given as FP8 codes [B, H, L, d] (uint8) with one scale per tensor
    ("注意力机制深度优化" §一.1 runs FlashAttention on float8_e4m3fn tensors): the exact attention
    of the dequantized tensors.  Returns O, LSE as attention()."""
    q = dequantize(q_codes, q_scale, fmt)
    k = dequantize(k_codes, k_scale, fmt)
    v = dequantize(v_codes, v_scale, fmt)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    return attention(q, k, v, scale=scale, causal=causal, window=window, threads=threads)
