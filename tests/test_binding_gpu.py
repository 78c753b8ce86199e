"""The Python binding's own checks: caller-supplied outputs and workspaces are validated before any
launch (the library sees only their addresses and writes their full extent), and a valid output
tensor is written in place and returned as is."""
import pytest
import torch

import attention_attn_fwd_03_amd as af
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _prefill():
    return wl.prefill_inputs(1, 4, 2, 96, 96, 64, seed=5, device=DEV)


@pytest.mark.parametrize("bad", ["shape", "dtype", "lse_shape", "lse_dtype", "strided"])
def test_fwd_rejects_bad_outputs(bad):
    q, k, v = _prefill()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], device=DEV, dtype=torch.float32)
    if bad == "shape":
        o = torch.empty((1, 4, 95, 64), device=DEV, dtype=torch.bfloat16)
    elif bad == "dtype":
        o = torch.empty(q.shape, device=DEV, dtype=torch.float32)
    elif bad == "lse_shape":
        lse = torch.empty((1, 4, 95), device=DEV, dtype=torch.float32)
    elif bad == "lse_dtype":
        lse = torch.empty(q.shape[:3], device=DEV, dtype=torch.bfloat16)
    else:
        o = torch.empty((1, 4, 64, 96), device=DEV, dtype=torch.bfloat16).transpose(2, 3)
    with pytest.raises(ValueError):
        af.attn_fwd(q, k, v, causal=True, return_lse=True, out=o, lse_out=lse)


def test_fwd_writes_the_given_output_in_place():
    q, k, v = _prefill()
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device=DEV, dtype=torch.float32)
    o2, lse2 = af.attn_fwd(q, k, v, causal=True, return_lse=True, out=o, lse_out=lse)
    assert o2 is o and lse2 is lse
    ref, ref_lse = af.attn_fwd(q, k, v, causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, ref) and torch.equal(lse, ref_lse)


def test_fp8_fwd_rejects_bad_output():
    q, k, v = _prefill()
    q8, k8, v8 = (torch.zeros(t.shape, device=DEV, dtype=torch.uint8) for t in (q, k, v))
    with pytest.raises(ValueError):
        af.attn_fwd_fp8(q8, k8, v8, qkv_format="e4m3fn", q_scale=1.0, k_scale=1.0, v_scale=1.0,
                        out=torch.empty(q.shape, device=DEV, dtype=torch.float32))


def test_bwd_rejects_bad_gradient_outputs():
    q, k, v = _prefill()
    o, lse = af.attn_fwd(q, k, v, causal=True, return_lse=True)
    dout = torch.ones_like(q)
    wrong = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(v))  # dk shaped like q
    with pytest.raises(ValueError):
        af.attn_bwd(q, k, v, o, dout, lse, causal=True, out=wrong)
    with pytest.raises(RuntimeError, match="ATTN_ERR_WORKSPACE"):
        af.attn_bwd(q, k, v, o, dout, lse, causal=True, workspace=torch.empty(16, device=DEV, dtype=torch.uint8))


def _decode():
    lens = wl.decode_lens(3, 40, 300, 9)
    q, kp, vp, offs, lens_t, _ = wl.decode_inputs(3, 8, 2, 128, lens, seed=9, device=DEV)
    return q, kp, vp, offs, lens_t, int(lens.max())


def test_decode_rejects_bad_outputs_and_workspace():
    q, kp, vp, offs, lens_t, max_len = _decode()
    with pytest.raises(ValueError):
        af.attn_decode(q, kp, vp, offs, lens_t, max_len=max_len, out=torch.empty((3, 8, 64), device=DEV,
                                                                                 dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        af.attn_decode(q, kp, vp, offs, lens_t, max_len=max_len, return_lse=True,
                       lse_out=torch.empty((3, 7), device=DEV, dtype=torch.float32))
    with pytest.raises(RuntimeError, match="ATTN_ERR_WORKSPACE"):
        af.attn_decode(q, kp, vp, offs, lens_t, max_len=max_len, workspace=torch.empty(64, device=DEV,
                                                                                        dtype=torch.uint8))
    with pytest.raises(ValueError):
        af.attn_decode(q, kp, vp, offs, lens_t, max_len=max_len, workspace=torch.empty(1 << 20, dtype=torch.uint8))


def test_decode_writes_the_given_output_in_place():
    q, kp, vp, offs, lens_t, max_len = _decode()
    o = torch.full_like(q, float("nan"))
    assert af.attn_decode(q, kp, vp, offs, lens_t, max_len=max_len, out=o) is o
    ref = af.attn_decode(q, kp, vp, offs, lens_t, max_len=max_len)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)


def test_inputs_on_the_host_are_refused():
    q, k, v = _prefill()
    with pytest.raises(ValueError):
        af.attn_fwd(q, k.cpu(), v, causal=True)
