"""Valid-argument calls into the C ABI, for the host-only sanitizer build (tests/host/launch_stubs.cpp).

Run by tests/test_host_sanitizers.py against that build only: there the kernel launches are stubs,
so argument validation, launch planning, workspace layout and the planner introspection run with
fake device pointers, large sizes and edge values under AddressSanitizer and
UndefinedBehaviorSanitizer.  Against the real library these calls would launch kernels on fake
pointers, so the module refuses to run unless the loaded library is the stub build."""
import ctypes

import numpy as np
import pytest

import attention_attn_fwd_03_amd as af

if not hasattr(af.lib(), "attn_host_stub_build"):
    pytest.skip("only for the host-only stub build of the C ABI", allow_module_level=True)

P = 0x10000
OK = af.ATTN_OK


@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lk,d,causal,window", [
    (1, 1, 1, 1, 1, 64, 0, 0), (2, 32, 8, 4096, 4096, 128, 1, 0), (1, 32, 8, 16384, 16384, 128, 1, 4096),
    (3, 6, 3, 257, 1000, 64, 1, 17), (1, 2, 1, 7, 2 * 1024 * 1024, 128, 0, 0), (1024, 64, 8, 4096, 1, 128, 1, 1)])
def test_fwd_entry_points_accept_valid_shapes(B, Hq, Hkv, Lq, Lk, d, causal, window):
    L = af.lib()
    for scale in (0.0, -0.5, 0.125, 1e30):
        assert L.attn_fwd(P, P, P, P, P, B, Hq, Hkv, Lq, Lk, d, causal, window, scale, None) == OK
        assert L.attn_fwd_f32(P, P, P, P, None, B, Hq, Hkv, Lq, Lk, d, causal, window, scale, None) == OK
    assert L.attn_fwd_fp8(P, P, P, P, P, B, Hq, Hkv, Lq, Lk, d, causal, window, 0.1, 1, 0.5, 2.0, 4.0, None) == OK
    # scales whose product with the score scale overflows fp32 are refused, not folded
    assert L.attn_fwd_fp8(P, P, P, P, P, B, Hq, Hkv, Lq, Lk, d, causal, window, 1e30, 2, 1e20, 1e20, 1.0,
                          None) == af.ATTN_ERR_UNSUPPORTED
    ws = af.bwd_workspace_size(B, Hq, Lq)
    if (B * Hq * Lq) // 16 < (1 << 31):
        assert L.attn_bwd(P, P, P, P, P, P, P, P, P, B, Hq, Hkv, Lq, Lk, d, causal, window, 0.1, P, ws, None) == OK
    info = af.FwdPlanInfo()
    assert L.attn_fwd_plan(B, Hq, Hkv, Lq, min(Lk, 1 << 16), d, causal, window, 0, ctypes.byref(info)) == OK


@pytest.mark.parametrize("n_seq,Hq,Hkv,d,max_len", [(1, 1, 1, 64, 1), (64, 32, 8, 128, 32768), (64, 32, 1, 128, 32768),
                                                     (7, 64, 1, 128, 5000), (300, 48, 1, 64, 999), (65535, 4, 4, 64, 8)])
def test_decode_entry_points_accept_valid_shapes(n_seq, Hq, Hkv, d, max_len):
    L = af.lib()
    ws = af.decode_workspace_size(n_seq, Hq, Hkv, d, max_len)
    assert ws > 0
    args = (P, P, P, P, P, P, P, n_seq, Hq, Hkv, d, 1 << 40, max_len, 0, 0.1)
    assert L.attn_decode(*args, P, ws, None) == OK
    assert L.attn_decode(*args, P, ws - 1, None) == af.ATTN_ERR_WORKSPACE
    assert L.attn_decode_fp8(*args, 1, 0.5, 0.25, P, ws, None) == OK
    expect = OK if ws <= af.DECODE_NOALLOC_BYTES else af.ATTN_ERR_WORKSPACE
    assert L.attn_decode_noalloc(*args, None) == expect
    page = 32
    stride = -(-max_len // page)
    pargs = (P, P, P, P, stride, page, 1 << 20, P, P, P, n_seq, Hq, Hkv, d, max_len, 3, 0.1)
    assert L.attn_decode_paged(*pargs, P, ws, None) == OK
    assert L.attn_decode_paged_fp8(*pargs, 2, 1.0, 1.0, P, ws, None) == OK
    rows = af.decode_rows(Hq, Hkv)
    assert rows.shape[1] == 3


def test_varlen_and_planner_introspection():
    L = af.lib()
    assert L.attn_fwd_varlen(P, P, P, P, P, P, P, P, 16, 32, 8, 128, 2048, 20000, 1 << 30, 1, 0, 0.1, None) == OK
    assert L.attn_fwd_varlen(P, P, P, P, None, P, P, P, 1, 4, 4, 64, 1, 0, 0, 0, 0, 0.1, None) == OK
    for args in ((2, 32, 8, 4096, 4096, 128, 1, 0), (1, 3, 1, 100, 5000, 64, 1, 33), (4, 16, 16, 1024, 1024, 64, 0, 0)):
        sched = af.fwd_schedule(*args)
        assert sched.shape[1] == 3 and len(np.unique(sched, axis=0)) == len(sched)
    for args in ((16, 32, 8, 1888), (1, 4, 1, 900), (40, 8, 2, 128)):
        assert len(af.fwd_varlen_schedule(*args)) > 0
    assert af.decode_plan(64, 32, 8, 128)[0] > 0
    assert L.attn_probe_mfma_ceiling(2, 768, 100, P, 768 * 256 * 4, None) == OK
