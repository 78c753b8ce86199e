"""Backward (dQ, dK, dV) of the HIP path against the fp64 oracle's, through the C ABI.

The HIP forward supplies O and the LSE, as a training step would; the oracle differentiates the
definition from q, k, v and dout alone.  Gradients are pre-filled with NaN so that any element
the kernels fail to write fails the test.  The bar is parity.check_grad's."""
import math

import numpy as np
import pytest
import torch

import attention_attn_fwd_03_amd as af
import oracle
import workloads as wl
from parity import check_grad, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_bwd(q, k, v, dout, causal, window, scale, o=None, lse=None):
    if o is None:
        o, lse = af.attn_fwd(q, k, v, causal=causal, window=window, scale=scale, return_lse=True)
    out = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
    af.attn_bwd(q, k, v, o, dout, lse, causal=causal, window=window, scale=scale, out=out)
    torch.cuda.synchronize()
    return out


def bwd_case(B, Hq, Hkv, Lq, Lk, d, causal=True, window=0, seed=0, scale=None):
    label = f"bwd B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} d{d} causal{int(causal)} W{window} seed{seed} scale{scale}"
    say(label)
    q, k, v, do = wl.backward_inputs(B, Hq, Hkv, Lq, Lk, d, seed=seed)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    got = run_bwd(q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), causal, window, scale)
    ref = oracle.attention_backward(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), wl.to_f64(do), scale=scale,
                                    causal=causal, window=window)
    stats = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        stats[name] = check_grad(wl.to_f64(g), r, f"{label} {name}")
    say(stats)
    return got, ref


@pytest.mark.parametrize("L,d", [(1, 64), (31, 128), (33, 64), (128, 128), (129, 64), (300, 128), (517, 64)])
def test_bwd_lengths(L, d):
    bwd_case(1, 4, 2, L, L, d, causal=True, seed=L)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_mask_modes(causal, d):
    bwd_case(2, 4, 4, 389, 389, d, causal=causal, seed=11 + d)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 2), (8, 1), (12, 3)])
def test_bwd_head_groups(Hq, Hkv):
    bwd_case(1, Hq, Hkv, 260, 260, 128, causal=True, seed=Hq * 10 + Hkv)


@pytest.mark.parametrize("Lq,Lk,causal", [(100, 333, True), (100, 333, False), (333, 100, True), (1, 700, True),
                                          (257, 64, True)])
def test_bwd_unequal_lengths(Lq, Lk, causal):
    got, _ = bwd_case(1, 4, 2, Lq, Lk, 64 if Lq % 2 else 128, causal=causal, seed=Lq + Lk)
    if causal and Lq > Lk:
        # rows before position 0 see no key: their gradient is exactly zero
        assert torch.all(got[0][:, :, :Lq - Lk] == 0)


@pytest.mark.parametrize("W,d", [(1, 64), (37, 128), (128, 64), (200, 128), (1000, 64)])
def test_bwd_windows(W, d):
    bwd_case(1, 4, 2, 600, 600, d, causal=True, window=W, seed=W)


def test_bwd_window_unequal_lengths():
    bwd_case(1, 4, 1, 200, 700, 128, causal=True, window=150, seed=5)


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.3])
def test_bwd_scales(scale):
    bwd_case(1, 4, 2, 200, 200, 64, causal=True, seed=7, scale=scale)


def test_bwd_uses_given_o_and_lse():
    """O and LSE computed by the oracle (rounded as the forward would hand them over) instead of
    the HIP forward: the backward alone against the oracle."""
    B, Hq, Hkv, L, d = 1, 4, 2, 300, 128
    q, k, v, do = wl.backward_inputs(B, Hq, Hkv, L, L, d, seed=21)
    scale = 1.0 / math.sqrt(d)
    q64, k64, v64, do64 = (wl.to_f64(t) for t in (q, k, v, do))
    O, LSE = oracle.attention(q64, k64, v64, scale=scale, causal=True)
    o = torch.from_numpy(O).to(torch.bfloat16).to(DEV)
    lse = torch.from_numpy(LSE).to(torch.float32).to(DEV)
    got = run_bwd(q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), True, 0, scale, o=o, lse=lse)
    ref = oracle.attention_backward(q64, k64, v64, do64, scale=scale, causal=True)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        check_grad(wl.to_f64(g), r, f"given O/LSE {name}")


def test_bwd_is_deterministic():
    q, k, v, do = (t.to(DEV) for t in wl.backward_inputs(1, 8, 2, 700, 700, 128, seed=3))
    a = run_bwd(q, k, v, do, True, 0, 1 / math.sqrt(128))
    b = run_bwd(q, k, v, do, True, 0, 1 / math.sqrt(128))
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("name", ["gqa_causal_bf16_L4096", "swa_gqa_bf16_L16384_W4096"])
def test_bwd_named_workload_sampled_heads(name):
    """The full-size launch (every head, the shape the benchmark times); the oracle checks the
    gradients of a sample of (batch, KV head) groups: dq of their query heads, dk and dv."""
    c = wl.PREFILL[name]
    say(f"bwd {name} full size on device")
    q, k, v, do = wl.backward_inputs(c.B, c.Hq, c.Hkv, c.Lq, c.Lk, c.d, seed=c.seed)
    got = run_bwd(q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), c.causal, c.window, c.scale)
    got = [g.cpu() for g in got]
    g = c.Hq // c.Hkv
    rng = np.random.default_rng(c.seed)
    groups = [(0, 0), (c.B - 1, c.Hkv - 1), (int(rng.integers(c.B)), int(rng.integers(c.Hkv)))]
    if c.Lq > 8192:
        groups = groups[1:2]  # the oracle's full L x L backward of one KV group takes seconds at 16k
    for b, kh in groups:
        hs = slice(kh * g, (kh + 1) * g)
        ref = oracle.attention_backward(wl.to_f64(q[b:b + 1, hs]), wl.to_f64(k[b:b + 1, kh:kh + 1]),
                                        wl.to_f64(v[b:b + 1, kh:kh + 1]), wl.to_f64(do[b:b + 1, hs]),
                                        scale=c.scale, causal=c.causal, window=c.window)
        for name_, gg, r in zip(("dq", "dk", "dv"), (got[0][b:b + 1, hs], got[1][b:b + 1, kh:kh + 1],
                                                      got[2][b:b + 1, kh:kh + 1]), ref):
            say(f"  batch {b} kv head {kh} {name_}", check_grad(wl.to_f64(gg), r, f"{name} b{b} kh{kh} {name_}"))
