"""attn_decode_noalloc (the decode entry point that allocates nothing) against attn_decode.

Both run the same kernels with the same split, so on the same inputs their outputs must agree bit
for bit; two calls in a row, the second on a smaller batch, show that what the first call leaves
in the library's fixed workspace does not leak into the second."""
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


def _inputs(lens, Hq, Hkv, d, seed):
    lens = np.asarray(lens, np.int32)
    q, kp, vp, offs, lens_t, layout = wl.decode_inputs(len(lens), Hq, Hkv, d, lens, seed=seed, device=DEV,
                                                       max_gap=19)
    return q, kp, vp, offs, lens_t, layout, int(max(lens.max(), 1))


def _both(q, kp, vp, offs, lens_t, max_len, scale, window=0):
    N, Hq, d = q.shape
    o1 = torch.full_like(q, float("nan"))
    l1 = torch.full((N, Hq), float("nan"), device=DEV, dtype=torch.float32)
    af.attn_decode(q, kp, vp, offs, lens_t, max_len=max_len, window=window, scale=scale, return_lse=True, out=o1,
                   lse_out=l1)
    o2 = torch.full_like(q, float("nan"))
    l2 = torch.full((N, Hq), float("nan"), device=DEV, dtype=torch.float32)
    af.attn_decode_noalloc(q, kp, vp, offs, lens_t, max_len=max_len, window=window, scale=scale, out=o2, lse_out=l2)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


@pytest.mark.parametrize("Hkv", [8, 1])
def test_noalloc_equals_decode_on_two_calls(Hkv):
    """The named decode batch's shape (64 sequences of 1k..32k keys, Hq 32, d 128), then a smaller
    ragged batch: each call equal bit for bit to attn_decode, the second also against the oracle."""
    c = wl.DECODE["gqa_decode_bf16" if Hkv == 8 else "mqa_decode_bf16"]
    lens = wl.decode_lens(c.n_seq, c.len_lo, c.len_hi, c.lens_seed)
    say(f"noalloc decode: {c.name}, then a small batch")
    q, kp, vp, offs, lens_t, _, max_len = _inputs(lens, c.Hq, c.Hkv, c.d, c.value_seed)
    o1, l1, o2, l2 = _both(q, kp, vp, offs, lens_t, max_len, c.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    del q, kp, vp
    small = [5, 0, 700, 33, 1, 2049, 64]
    q, kp, vp, offs, lens_t, layout, max_len = _inputs(small, 8, 2, 128, 3100 + Hkv)
    o1, l1, o2, l2 = _both(q, kp, vp, offs, lens_t, max_len, 1.0 / math.sqrt(128))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    O_ref, L_ref = oracle.decode(q.cpu().float().numpy(), kp.cpu().float().numpy(), vp.cpu().float().numpy(),
                                 layout.offsets, layout.lens, scale=1.0 / math.sqrt(128))
    say(check(wl.to_f64(o2), O_ref, l2.cpu().numpy(), L_ref, "bf16", "noalloc small batch"))


def test_noalloc_window_and_without_lse():
    q, kp, vp, offs, lens_t, _, max_len = _inputs([300, 17, 4000], 16, 4, 64, 3200)
    o1, l1, o2, l2 = _both(q, kp, vp, offs, lens_t, max_len, 0.1, window=129)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3 = torch.full_like(q, float("nan"))
    af.attn_decode_noalloc(q, kp, vp, offs, lens_t, max_len=max_len, window=129, scale=0.1, out=o3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3)
