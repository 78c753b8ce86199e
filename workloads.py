"""Seeded synthetic workloads shared by the oracle tests, the GPU parity tests and bench.py.

This module only draws numbers and lays buffers out. It holds none of the attention
arithmetic, so neither side of a parity comparison borrows the other's maths from here.

Every tensor is drawn as float32 N(0, 1) from a seeded ``torch.Generator`` in the order
q, k, v and then rounded to the working dtype (``Tensor.to`` rounds to nearest even).
The shapes follow the attention articles' own workloads: a 1024-token MHA block, a
4096-token GQA model with 32 query heads over 8 KV heads and head size 128, a 16k
sequence under a 4k sliding window, and a decode batch whose KV caches sit in one pooled
buffer addressed by per-sequence offsets.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    dtype: str          # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    d: int
    causal: bool
    window: int
    seed: int
    return_lse: bool = True

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    n_seq: int
    Hq: int
    Hkv: int
    d: int
    len_lo: int
    len_hi: int
    lens_seed: int
    value_seed: int
    window: int = 0
    max_gap: int = 255  # poisoned rows placed between sequences in the pool

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


# The five workloads the hot path is specified on (the tiny fp32 one in two mask modes).
PREFILL = {
    "mha_f32_L128": PrefillConfig("mha_f32_L128", "f32", 1, 2, 2, 128, 128, 64, False, 0, 1001),
    "mha_f32_L128_causal": PrefillConfig("mha_f32_L128_causal", "f32", 1, 2, 2, 128, 128, 64, True, 0, 1001),
    "mha_bf16_L1024": PrefillConfig("mha_bf16_L1024", "bf16", 4, 16, 16, 1024, 1024, 64, False, 0, 1002),
    "gqa_causal_bf16_L4096": PrefillConfig("gqa_causal_bf16_L4096", "bf16", 2, 32, 8, 4096, 4096, 128, True, 0, 1003),
    "swa_gqa_bf16_L16384_W4096": PrefillConfig("swa_gqa_bf16_L16384_W4096", "bf16", 1, 32, 8, 16384, 16384, 128,
                                               True, 4096, 1004),
}

DECODE = {
    "gqa_decode_bf16": DecodeConfig("gqa_decode_bf16", 64, 32, 8, 128, 1024, 32768, 1005, 1005),
    "mqa_decode_bf16": DecodeConfig("mqa_decode_bf16", 64, 32, 1, 128, 1024, 32768, 1005, 1006),
}


@dataclass(frozen=True)
class VarlenConfig:
    """A ragged chunked-prefill batch: each sequence adds new_lo..new_hi tokens on top of
    cached_lo..cached_hi cached ones (both uniform, seeded)."""
    name: str
    n_seq: int
    Hq: int
    Hkv: int
    d: int
    new_lo: int
    new_hi: int
    cached_lo: int
    cached_hi: int
    seed: int
    causal: bool = True
    window: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def lengths(self):
        """(new tokens, keys) per sequence; keys = cached + new."""
        rng = np.random.default_rng(self.seed)
        lq = rng.integers(self.new_lo, self.new_hi, size=self.n_seq, endpoint=True)
        cached = rng.integers(self.cached_lo, self.cached_hi, size=self.n_seq, endpoint=True)
        return lq.astype(np.int32), (lq + cached).astype(np.int32)


# Continuous batching of chunked prefills against the cache, at the decode batch's head shape.
VARLEN = {
    "chunked_prefill_bf16": VarlenConfig("chunked_prefill_bf16", 16, 32, 8, 128, 512, 2048, 0, 14336, 1007),
}


def normal(shape, gen: torch.Generator, device, dtype) -> torch.Tensor:
    """float32 N(0, 1) from ``gen``, then rounded to ``dtype``."""
    x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(dtype)


def make_generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def prefill_inputs(B, Hq, Hkv, Lq, Lk, d, *, seed, dtype=torch.bfloat16, device="cpu"):
    """q [B, Hq, Lq, d], k and v [B, Hkv, Lk, d], contiguous, drawn in the order q, k, v."""
    g = make_generator(seed, device)
    q = normal((B, Hq, Lq, d), g, device, dtype)
    k = normal((B, Hkv, Lk, d), g, device, dtype)
    v = normal((B, Hkv, Lk, d), g, device, dtype)
    return q, k, v


def backward_inputs(B, Hq, Hkv, Lq, Lk, d, *, seed, dtype=torch.bfloat16, device="cpu"):
    """prefill_inputs plus an upstream gradient dout [B, Hq, Lq, d] ~ N(0, 1), drawn after them."""
    g = make_generator(seed, device)
    q = normal((B, Hq, Lq, d), g, device, dtype)
    k = normal((B, Hkv, Lk, d), g, device, dtype)
    v = normal((B, Hkv, Lk, d), g, device, dtype)
    dout = normal((B, Hq, Lq, d), g, device, dtype)
    return q, k, v, dout


def prefill_inputs_for(cfg: PrefillConfig, device="cpu"):
    return prefill_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.Lq, cfg.Lk, cfg.d, seed=cfg.seed,
                          dtype=cfg.torch_dtype, device=device)


def decode_lens(n_seq: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """KV lengths uniform on [lo, hi] (both ends included)."""
    return np.random.default_rng(seed).integers(lo, hi, size=n_seq, endpoint=True).astype(np.int32)


@dataclass
class PoolLayout:
    lens: np.ndarray        # int32 [n_seq]
    offsets: np.ndarray     # int64 [n_seq], first pool row of each sequence
    total_rows: int         # pool rows T, gaps included
    gaps: list = field(default_factory=list)  # (start, length) of each poisoned gap


def pool_layout(lens: np.ndarray, seed: int, max_gap: int = 255, shuffle: bool = True) -> PoolLayout:
    """Place sequences in one pool in a seeded random order, with a seeded gap of 0..max_gap
    rows before each one and after the last.  Offsets are in token rows."""
    rng = np.random.default_rng(seed + 7919)
    n = len(lens)
    order = rng.permutation(n) if shuffle else np.arange(n)
    gaps = rng.integers(0, max_gap, size=n + 1, endpoint=True) if max_gap > 0 else np.zeros(n + 1, np.int64)
    offsets = np.zeros(n, np.int64)
    pos = 0
    gap_list = []
    for slot, s in enumerate(order):
        if gaps[slot]:
            gap_list.append((pos, int(gaps[slot])))
        pos += int(gaps[slot])
        offsets[s] = pos
        pos += int(lens[s])
    if gaps[n]:
        gap_list.append((pos, int(gaps[n])))
    pos += int(gaps[n])
    return PoolLayout(lens=np.asarray(lens, np.int32), offsets=offsets, total_rows=pos, gaps=gap_list)


def decode_inputs(n_seq, Hq, Hkv, d, lens, *, seed, device="cpu", dtype=torch.bfloat16,
                  max_gap=255, shuffle=True, poison=float("nan")):
    """q [n_seq, Hq, d]; k_pool, v_pool [T, Hkv, d]; offsets int64; lens int32.

    Rows of the pool that belong to no sequence are filled with ``poison`` so that a kernel
    reading outside its sequence shows up as a non-finite output."""
    layout = pool_layout(np.asarray(lens), seed, max_gap=max_gap, shuffle=shuffle)
    g = make_generator(seed, device)
    q = normal((n_seq, Hq, d), g, device, dtype)
    k_pool = normal((layout.total_rows, Hkv, d), g, device, dtype)
    v_pool = normal((layout.total_rows, Hkv, d), g, device, dtype)
    for start, length in layout.gaps:
        k_pool[start:start + length] = poison
        v_pool[start:start + length] = poison
    offsets = torch.from_numpy(layout.offsets).to(device)
    lens_t = torch.from_numpy(layout.lens).to(device)
    return q, k_pool, v_pool, offsets, lens_t, layout


def decode_inputs_for(cfg: DecodeConfig, device="cpu"):
    lens = decode_lens(cfg.n_seq, cfg.len_lo, cfg.len_hi, cfg.lens_seed)
    return decode_inputs(cfg.n_seq, cfg.Hq, cfg.Hkv, cfg.d, lens, seed=cfg.value_seed, device=device,
                         max_gap=cfg.max_gap)


@dataclass
class PagedLayout:
    lens: np.ndarray        # int32 [n_seq]
    page_size: int
    table: np.ndarray       # int32 [n_seq, stride]: page of each sequence's j-th page slot, -1 if none
    pool_pages: int
    row_owner: np.ndarray   # bool [pool_pages * page_size]: the row holds some sequence's token


def paged_layout(lens: np.ndarray, page_size: int, seed: int, extra_pages: int = 0,
                 stride: int | None = None) -> PagedLayout:
    """Give sequence s ceil(lens[s] / page_size) pages, drawn in a seeded random order from a
    pool of (pages needed + extra_pages); page slots a sequence does not use hold -1."""
    rng = np.random.default_rng(seed + 104729)
    need = [-(-int(n) // page_size) for n in lens]
    pool_pages = sum(need) + extra_pages
    perm = rng.permutation(pool_pages)
    stride = max(max(need), 1) if stride is None else stride
    table = np.full((len(lens), stride), -1, np.int32)
    owner = np.zeros(pool_pages * page_size, bool)
    k = 0
    for s, m in enumerate(need):
        for j in range(m):
            page = int(perm[k])
            k += 1
            table[s, j] = page
            owner[page * page_size:page * page_size + min(page_size, int(lens[s]) - j * page_size)] = True
    return PagedLayout(lens=np.asarray(lens, np.int32), page_size=page_size, table=table,
                       pool_pages=pool_pages, row_owner=owner)


def paged_decode_inputs(n_seq, Hq, Hkv, d, lens, page_size, *, seed, device="cpu", dtype=torch.bfloat16,
                        extra_pages=0, stride=None, poison=float("nan")):
    """q [n_seq, Hq, d]; k_pool, v_pool [pool_pages * page_size, Hkv, d]; block table int32;
    lens int32.  Rows that hold no sequence's token (unused pages, the tail of each sequence's
    last page) are filled with ``poison``."""
    layout = paged_layout(np.asarray(lens), page_size, seed, extra_pages=extra_pages, stride=stride)
    g = make_generator(seed, device)
    q = normal((n_seq, Hq, d), g, device, dtype)
    rows = layout.pool_pages * page_size
    k_pool = normal((rows, Hkv, d), g, device, dtype)
    v_pool = normal((rows, Hkv, d), g, device, dtype)
    free = torch.from_numpy(~layout.row_owner).to(device)
    k_pool[free] = poison
    v_pool[free] = poison
    table = torch.from_numpy(layout.table).to(device)
    lens_t = torch.from_numpy(layout.lens).to(device)
    return q, k_pool, v_pool, table, lens_t, layout


# FP8 KV cache: the two formats and their largest finite values (OCP 8-bit floating point).
FP8_DTYPES = {"e4m3fn": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
FP8_MAX = {"e4m3fn": 448.0, "e5m2": 57344.0}


def to_fp8_codes(x: torch.Tensor, fmt: str, scale: float | None = None):
    """Quantise a float tensor to FP8 codes (uint8) with one per-tensor scale: torch's conversion
    (round to nearest even) of x / scale.  The scale defaults to max |x| over the finite entries
    divided by the format's largest finite value, so the largest entry maps to it; NaN stays NaN.
    Returns (codes, scale)."""
    xf = x.to(torch.float32)
    if scale is None:
        fin = torch.isfinite(xf)
        amax = float(xf[fin].abs().max()) if bool(fin.any()) else 1.0
        scale = amax / FP8_MAX[fmt] if amax > 0 else 1.0
    codes = (xf / scale).to(FP8_DTYPES[fmt]).view(torch.uint8)
    return codes, float(scale)


def fp8_decode_inputs(n_seq, Hq, Hkv, d, lens, fmt, *, seed, device="cpu", max_gap=255, shuffle=True):
    """decode_inputs with the pools held as FP8 codes: the same draws in fp32, q rounded to bf16,
    K and V quantised per pool (to_fp8_codes; NaN gap rows become NaN codes).  Returns q,
    k_codes, v_codes, offsets, lens, layout, k_scale, v_scale."""
    q, kp, vp, offs, lens_t, layout = decode_inputs(n_seq, Hq, Hkv, d, lens, seed=seed, device=device,
                                                    dtype=torch.float32, max_gap=max_gap, shuffle=shuffle)
    kc, ks = to_fp8_codes(kp, fmt)
    vc, vs = to_fp8_codes(vp, fmt)
    return q.to(torch.bfloat16), kc, vc, offs, lens_t, layout, ks, vs


def fp8_prefill_inputs(B, Hq, Hkv, Lq, Lk, d, fmt, *, seed, device="cpu"):
    """prefill_inputs drawn in fp32 and quantised per tensor (to_fp8_codes): q, k, v codes
    [B, H, L, d] uint8 and their scales (q_scale, k_scale, v_scale)."""
    q, k, v = prefill_inputs(B, Hq, Hkv, Lq, Lk, d, seed=seed, dtype=torch.float32, device=device)
    (qc, qs), (kc, ks), (vc, vs) = (to_fp8_codes(x, fmt) for x in (q, k, v))
    return qc, kc, vc, qs, ks, vs


def fp8_paged_decode_inputs(n_seq, Hq, Hkv, d, lens, page_size, fmt, *, seed, device="cpu", extra_pages=0,
                            stride=None):
    """paged_decode_inputs with FP8 pools, as fp8_decode_inputs.  Returns q, k_codes, v_codes,
    block table, lens, layout, k_scale, v_scale."""
    q, kp, vp, table, lens_t, layout = paged_decode_inputs(n_seq, Hq, Hkv, d, lens, page_size, seed=seed,
                                                           device=device, dtype=torch.float32,
                                                           extra_pages=extra_pages, stride=stride)
    kc, ks = to_fp8_codes(kp, fmt)
    vc, vs = to_fp8_codes(vp, fmt)
    return q.to(torch.bfloat16), kc, vc, table, lens_t, layout, ks, vs


def varlen_inputs(lq, lk, Hq, Hkv, d, *, seed, device="cpu", dtype=torch.bfloat16, max_gap=37,
                  poison=float("nan")):
    """Ragged prefill inputs: q [sum(lq), Hq, d] packed by cu_seqlens; k_pool, v_pool [T, Hkv, d]
    holding sequence s's lk[s] keys at rows offsets[s] .. (placed by pool_layout: seeded order,
    ``poison`` in the gaps).  Returns q, k_pool, v_pool, cu_seqlens (int32), offsets (int64),
    kv_lens (int32) and the layout."""
    layout = pool_layout(np.asarray(lk), seed, max_gap=max_gap)
    g = make_generator(seed, device)
    q = normal((int(sum(lq)), Hq, d), g, device, dtype)
    k_pool = normal((layout.total_rows, Hkv, d), g, device, dtype)
    v_pool = normal((layout.total_rows, Hkv, d), g, device, dtype)
    for start, length in layout.gaps:
        k_pool[start:start + length] = poison
        v_pool[start:start + length] = poison
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)).to(device)
    offsets = torch.from_numpy(layout.offsets).to(device)
    lens_t = torch.from_numpy(layout.lens).to(device)
    return q, k_pool, v_pool, cu, offsets, lens_t, layout


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a float32 or bfloat16 tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
