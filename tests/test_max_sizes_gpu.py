"""Sizes near the limits the C ABI accepts (per head, K/V byte offsets are 32-bit): long key
ranges in prefill and decode, checked against the oracle on sampled rows / sequences."""
import math

import numpy as np
import pytest
import torch

import attention_attn_fwd_03_amd as af
import oracle
import workloads as wl
from parity import check, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_prefill_two_million_keys():
    """64 query rows at the end of a 2M + 17-key sequence (bottom-right causal: every row sees
    about 2M keys), one KV head shared by two query heads, d = 128: K and V are 512 MB each and the
    tile offsets reach 2^29 bytes."""
    B, Hq, Hkv, Lq, Lk, d = 1, 2, 1, 64, (1 << 21) + 17, 128
    say(f"prefill Lq{Lq} Lk{Lk} Hq{Hq} Hkv{Hkv} d{d}")
    q, k, v = wl.prefill_inputs(B, Hq, Hkv, Lq, Lk, d, seed=41, device=DEV)
    scale = 1.0 / math.sqrt(d)
    o, lse = af.attn_fwd(q, k, v, causal=True, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    rows = [0, 1, 31, 32, 62, 63]
    samples = [(0, h, i) for h in range(Hq) for i in rows]
    O_ref, L_ref = oracle.attention_rows(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), samples, scale=scale, causal=True)
    idx = tuple(np.array(samples).T)
    say(check(wl.to_f64(o)[idx], O_ref, lse.cpu().numpy().astype(np.float64)[idx], L_ref, "bf16", "2M keys"))


def test_decode_one_million_token_sequence():
    """One sequence of 2^20 cached tokens among short ones, Hkv = 8, d = 128 (a 4 GB pool; the
    sequence's rows of one head reach 2^30 bytes), the split spread over every team."""
    lens = np.array([5, (1 << 20) - 3, 77, 1], np.int32)
    Hq, Hkv, d = 32, 8, 128
    say(f"decode lens {lens.tolist()} Hq{Hq} Hkv{Hkv} d{d}")
    q, kp, vp, offs, lens_t, layout = wl.decode_inputs(len(lens), Hq, Hkv, d, lens, seed=43, device=DEV, max_gap=3)
    scale = 1.0 / math.sqrt(d)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((len(lens), Hq), float("nan"), device=DEV, dtype=torch.float32)
    af.attn_decode(q, kp, vp, offs, lens_t, max_len=int(lens.max()), scale=scale, return_lse=True, out=o, lse_out=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    g = Hq // Hkv
    for kh in (0, Hkv - 1):  # one KV head and its query heads at a time keeps the fp64 pool at 2 GB
        hs = slice(kh * g, (kh + 1) * g)
        O_ref, L_ref = oracle.decode(wl.to_f64(q[:, hs]), wl.to_f64(kp[:, kh:kh + 1]), wl.to_f64(vp[:, kh:kh + 1]),
                                     layout.offsets, layout.lens, scale=scale)
        say(kh, check(wl.to_f64(o[:, hs]), O_ref, lse[:, hs].cpu().numpy(), L_ref, "bf16", f"1M-token decode kv{kh}"))
