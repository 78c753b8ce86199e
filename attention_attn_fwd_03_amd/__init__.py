"""attnfwd: fused exact attention forward and pooled-KV decode for MI355X (gfx950).

A thin ctypes binding over libattnfwd.so (include/attn.h).  Torch tensors supply device
memory and the current stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: without the built library or a GPU the calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ATTNFWD_LIB names another build of the same C ABI (the host-only sanitizer build the CPU tests
# make); by default the in-tree library.
LIB_PATH = os.environ.get("ATTNFWD_LIB") or os.path.join(_HERE, "libattnfwd.so")

ATTN_OK, ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = range(6)
KV_FORMATS = {"e4m3fn": 1, "e5m2": 2}  # attn_kv_format

EXPORTS = ["attn_fwd", "attn_fwd_f32", "attn_fwd_varlen", "attn_decode_workspace_size", "attn_decode",
           "attn_decode_paged", "attn_status_str", "attn_fwd_plan", "attn_fwd_schedule", "attn_fwd_varlen_schedule",
           "attn_decode_plan", "attn_bwd_workspace_size", "attn_bwd", "attn_decode_fp8", "attn_decode_paged_fp8",
           "attn_fwd_fp8", "attn_decode_rows", "attn_decode_noalloc", "attn_probe_mfma_ceiling"]
DECODE_NOALLOC_BYTES = 64 << 20  # ATTN_DECODE_NOALLOC_BYTES
PROBE_SOURCE_BYTES = 64 * (9216 + 10240)  # ATTN_PROBE_SOURCE_BYTES


class FwdPlanInfo(ctypes.Structure):
    _fields_ = [("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("num_q_tiles", ctypes.c_int32), ("heads_per_xcd", ctypes.c_int32),
                ("num_workgroups", ctypes.c_int64), ("tiles_per_head", ctypes.c_int64),
                ("masked_tiles_per_head", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libattnfwd.so (built in-tree by build.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run attention_attn_fwd_03_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64, ctypes.c_size_t
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, vp]
    L.attn_fwd.restype = i32
    L.attn_fwd_f32.argtypes = L.attn_fwd.argtypes
    L.attn_fwd_f32.restype = i32
    L.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i64, i64, i32, i32, f32, vp]
    L.attn_fwd_varlen.restype = i32
    L.attn_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    L.attn_decode_workspace_size.restype = sz
    L.attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i32, i32, f32, vp, sz, vp]
    L.attn_decode.restype = i32
    L.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i32, i32, f32, vp]
    L.attn_decode_noalloc.restype = i32
    L.attn_probe_mfma_ceiling.argtypes = [i32, i32, i32, vp, sz, vp]
    L.attn_probe_mfma_ceiling.restype = i32
    L.attn_decode_paged.argtypes = [vp, vp, vp, vp, i32, i32, i64, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                    vp, sz, vp]
    L.attn_decode_paged.restype = i32
    L.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, f32, f32, f32, vp]
    L.attn_fwd_fp8.restype = i32
    L.attn_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, i32, i32, f32, i32, f32, f32,
                                  vp, sz, vp]
    L.attn_decode_fp8.restype = i32
    L.attn_decode_paged_fp8.argtypes = [vp, vp, vp, vp, i32, i32, i64, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                        i32, f32, f32, vp, sz, vp]
    L.attn_decode_paged_fp8.restype = i32
    L.attn_bwd_workspace_size.argtypes = [i32, i32, i32]
    L.attn_bwd_workspace_size.restype = sz
    L.attn_bwd.argtypes = [vp] * 9 + [i32] * 8 + [f32, vp, sz, vp]
    L.attn_bwd.restype = i32
    L.attn_status_str.argtypes = [i32]
    L.attn_status_str.restype = ctypes.c_char_p
    L.attn_fwd_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(FwdPlanInfo)]
    L.attn_fwd_plan.restype = i32
    L.attn_fwd_schedule.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, i64]
    L.attn_fwd_schedule.restype = i32
    L.attn_fwd_varlen_schedule.argtypes = [i32, i32, i32, i32, vp, i64, ctypes.POINTER(ctypes.c_int64)]
    L.attn_fwd_varlen_schedule.restype = i32
    L.attn_decode_plan.argtypes = [i32, i32, i32, i32] + [ctypes.POINTER(ctypes.c_int32)] * 3
    L.attn_decode_plan.restype = i32
    L.attn_decode_rows.argtypes = [i32, i32, vp, vp, vp, i64]
    L.attn_decode_rows.restype = i32
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().attn_status_str(int(status)).decode()


def _check(status: int):
    if status != ATTN_OK:
        raise RuntimeError(status_str(status))


def _require_gpu(*tensors):
    """Contiguous GPU tensors, all on one device; returns that device."""
    import torch
    for t in tensors:
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError("attnfwd works on GPU tensors only")
        if not t.is_contiguous():
            raise ValueError("attnfwd needs contiguous tensors")
    dev = tensors[0].device
    if any(t.device != dev for t in tensors):
        raise ValueError("attnfwd needs all tensors on one GPU")
    return dev


def _output(t, shape, dtype, device, name: str):
    """A new output tensor, or the caller's ``t`` once it is known to have exactly this shape,
    dtype and device (the library sees only its address and writes the full extent)."""
    import torch
    shape = tuple(int(x) for x in shape)
    if t is None:
        return torch.empty(shape, device=device, dtype=dtype)
    _require_gpu(t)
    if tuple(t.shape) != shape or t.dtype != dtype or t.device != device:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {shape} on {device}")
    return t


def _run(device, fn, *args):
    """Call entry point ``fn`` with ``args`` and the current stream of ``device``, with that device
    current (the library launches on the current device)."""
    import torch
    with torch.cuda.device(device):
        _check(fn(*args, ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)))


def attn_fwd(q, k, v, *, causal: bool = False, window: int = 0, scale: float | None = None,
             return_lse: bool = False, out=None, lse_out=None):
    """Exact attention forward.  q [B, Hq, Lq, d]; k, v [B, Hkv, Lk, d]; bf16 or fp32 (all alike).

    Returns O [B, Hq, Lq, d] (same dtype), and LSE [B, Hq, Lq] fp32 (natural log) when
    ``return_lse``.  ``scale`` defaults to 1/sqrt(d)."""
    import torch
    dev = _require_gpu(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected 4-d tensors [B, H, L, d]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    B, Hq, Lq, d = q.shape
    Bk, Hkv, Lk, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch between q, k and v")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = _output(out, q.shape, q.dtype, dev, "out")
    lse = _output(lse_out, (B, Hq, Lq), torch.float32, dev, "lse_out") if return_lse else None
    fn = lib().attn_fwd if q.dtype == torch.bfloat16 else lib().attn_fwd_f32
    _run(dev, fn, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr() if lse is not None else None,
         B, Hq, Hkv, Lq, Lk, d, int(bool(causal)), int(window), float(scale))
    return (o, lse) if return_lse else o


def bwd_workspace_size(B: int, Hq: int, Lq: int) -> int:
    return int(lib().attn_bwd_workspace_size(B, Hq, Lq))


def attn_bwd(q, k, v, o, dout, lse, *, causal: bool = False, window: int = 0, scale: float | None = None,
             workspace=None, out=None):
    """Gradients (dq, dk, dv) of attn_fwd for an upstream gradient ``dout`` [B, Hq, Lq, d], given
    the forward's output ``o`` and row log-sum-exp ``lse`` [B, Hq, Lq] fp32 (same q, k, v, mask
    and scale).  bf16.  ``workspace``: optional uint8 device tensor of bwd_workspace_size bytes;
    ``out``: optional (dq, dk, dv) tensors to write."""
    import torch
    dev = _require_gpu(q, k, v, o, dout, lse)
    if any(t.dtype != torch.bfloat16 for t in (q, k, v, o, dout)) or lse.dtype != torch.float32:
        raise ValueError("attn_bwd takes bfloat16 q, k, v, o, dout and float32 lse")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("expected 4-d tensors [B, H, L, d]")
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if (tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != d or tuple(o.shape) != tuple(q.shape)
            or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, Lq)):
        raise ValueError("shape mismatch between q, k, v, o, dout and lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = bwd_workspace_size(B, Hq, Lq)
    if workspace is None:
        workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    if _require_gpu(workspace) != dev:
        raise ValueError("the workspace must be on the tensors' GPU")
    dq, dk, dv = (None, None, None) if out is None else out
    dq = _output(dq, q.shape, torch.bfloat16, dev, "dq")
    dk = _output(dk, k.shape, torch.bfloat16, dev, "dk")
    dv = _output(dv, v.shape, torch.bfloat16, dev, "dv")
    _run(dev, lib().attn_bwd, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
         dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Lq, Lk, d, int(bool(causal)), int(window),
         float(scale), workspace.data_ptr(), workspace.numel() * workspace.element_size())
    return dq, dk, dv


def attn_fwd_fp8(q, k, v, *, qkv_format: str, q_scale: float, k_scale: float, v_scale: float, causal: bool = False,
                 window: int = 0, scale: float | None = None, return_lse: bool = False, out=None, lse_out=None):
    """Exact attention over FP8 inputs: q [B, Hq, Lq, d], k, v [B, Hkv, Lk, d] uint8 codes of
    ``qkv_format`` ('e4m3fn' / 'e5m2') with per-tensor scales (real value = scale * code value).
    Returns O [B, Hq, Lq, d] bf16 and, when ``return_lse``, LSE [B, Hq, Lq] fp32."""
    import torch
    dev = _require_gpu(q, k, v)
    if q.dtype != torch.uint8 or k.dtype != torch.uint8 or v.dtype != torch.uint8:
        raise ValueError("attn_fwd_fp8 takes uint8 FP8 codes")
    if qkv_format not in KV_FORMATS:
        raise ValueError("qkv_format must be 'e4m3fn' or 'e5m2'")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected 4-d tensors [B, H, L, d]")
    B, Hq, Lq, d = q.shape
    Bk, Hkv, Lk, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch between q, k and v")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = _output(out, (B, Hq, Lq, d), torch.bfloat16, dev, "out")
    lse = _output(lse_out, (B, Hq, Lq), torch.float32, dev, "lse_out") if return_lse else None
    _run(dev, lib().attn_fwd_fp8, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
         lse.data_ptr() if lse is not None else None, B, Hq, Hkv, Lq, Lk, d, int(bool(causal)), int(window),
         float(scale), KV_FORMATS[qkv_format], float(q_scale), float(k_scale), float(v_scale))
    return (o, lse) if return_lse else o


def decode_workspace_size(n_seq: int, Hq: int, Hkv: int, d: int, max_len: int) -> int:
    return int(lib().attn_decode_workspace_size(n_seq, Hq, Hkv, d, max_len))


def attn_fwd_varlen(q, k_pool, v_pool, cu_seqlens_q, kv_offsets, kv_lens, *, max_seqlen_q: int, causal: bool = True,
                    window: int = 0, scale: float | None = None, return_lse: bool = False, out=None, lse_out=None):
    """Ragged prefill: new tokens of several sequences packed in q [total_q, Hq, d] (sequence s's
    rows cu_seqlens_q[s] .. cu_seqlens_q[s+1] - 1), each attending to its kv_lens[s] keys at pool
    rows kv_offsets[s] .. (pools [T, Hkv, d]), bottom-right aligned.  bf16; cu_seqlens_q and
    kv_lens int32, kv_offsets int64, all on the device; max_seqlen_q >= every sequence's new
    tokens.  Returns O [total_q, Hq, d] and, when ``return_lse``, LSE [total_q, Hq] fp32."""
    import torch
    dev = _require_gpu(q, k_pool, v_pool, cu_seqlens_q, kv_offsets, kv_lens)
    if q.dim() != 3 or k_pool.dim() != 3:
        raise ValueError("expected q [total_q, Hq, d] and pools [T, Hkv, d]")
    if q.dtype != torch.bfloat16 or k_pool.dtype != torch.bfloat16 or v_pool.dtype != torch.bfloat16:
        raise ValueError("ragged prefill takes bfloat16 q and pools")
    if cu_seqlens_q.dtype != torch.int32 or kv_lens.dtype != torch.int32 or kv_offsets.dtype != torch.int64:
        raise ValueError("cu_seqlens_q and kv_lens must be int32, kv_offsets int64")
    total_q, Hq, d = q.shape
    T, Hkv, dk = k_pool.shape
    n_seq = kv_lens.numel()
    if (dk != d or tuple(v_pool.shape) != tuple(k_pool.shape) or cu_seqlens_q.numel() != n_seq + 1
            or kv_offsets.numel() != n_seq):
        raise ValueError("shape mismatch between q, pools, cu_seqlens_q, kv_offsets and kv_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = _output(out, q.shape, torch.bfloat16, dev, "out")
    lse = _output(lse_out, (total_q, Hq), torch.float32, dev, "lse_out") if return_lse else None
    _run(dev, lib().attn_fwd_varlen, q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), o.data_ptr(),
         lse.data_ptr() if lse is not None else None, cu_seqlens_q.data_ptr(), kv_offsets.data_ptr(),
         kv_lens.data_ptr(), n_seq, Hq, Hkv, d, int(max_seqlen_q), total_q, T, int(bool(causal)), int(window),
         float(scale))
    return (o, lse) if return_lse else o


def _decode_workspace(workspace, N, Hq, Hkv, d, max_len, dev):
    """The caller's workspace (its size is checked by the library), or a new one of the size the
    library asks for."""
    import torch
    if workspace is None:
        return torch.empty(max(decode_workspace_size(N, Hq, Hkv, d, max_len), 16), device=dev, dtype=torch.uint8)
    if _require_gpu(workspace) != dev:
        raise ValueError("the workspace must be on the tensors' GPU")
    return workspace


def _kv_format(q, k_pool, v_pool, kv_format, k_scale, v_scale):
    """0 for bf16 pools; the attn_kv_format code for uint8 (FP8 code) pools."""
    import torch
    if q.dtype != torch.bfloat16:
        raise ValueError("decode takes a bfloat16 q")
    if k_pool.dtype == torch.bfloat16 and v_pool.dtype == torch.bfloat16:
        if kv_format is not None:
            raise ValueError("kv_format applies to uint8 (FP8 code) pools")
        return 0
    if k_pool.dtype == torch.uint8 and v_pool.dtype == torch.uint8:
        if kv_format not in KV_FORMATS or k_scale is None or v_scale is None:
            raise ValueError("FP8 pools need kv_format ('e4m3fn' or 'e5m2'), k_scale and v_scale")
        return KV_FORMATS[kv_format]
    raise ValueError("pools must both be bfloat16, or both uint8 FP8 codes")


def attn_decode(q, k_pool, v_pool, offsets, lens, *, max_len: int, window: int = 0, scale: float | None = None,
                return_lse: bool = False, workspace=None, out=None, lse_out=None, kv_format: str | None = None,
                k_scale: float | None = None, v_scale: float | None = None):
    """Decode one query token per sequence against a pooled KV cache.

    q [N, Hq, d] bf16; k_pool, v_pool [T, Hkv, d] bf16, or uint8 FP8 codes with ``kv_format``
    ('e4m3fn' / 'e5m2') and per-pool ``k_scale`` / ``v_scale`` (real value = scale * code value);
    offsets int64 [N] (first pool row of each sequence); lens int32 [N]; max_len >= max(lens).
    Returns O [N, Hq, d] bf16 and, when ``return_lse``, LSE [N, Hq] fp32."""
    import torch
    dev = _require_gpu(q, k_pool, v_pool, offsets, lens)
    fmt = _kv_format(q, k_pool, v_pool, kv_format, k_scale, v_scale)
    if offsets.dtype != torch.int64 or lens.dtype != torch.int32:
        raise ValueError("offsets must be int64 and lens int32")
    if q.dim() != 3 or k_pool.dim() != 3:
        raise ValueError("expected q [N, Hq, d] and pools [T, Hkv, d]")
    N, Hq, d = q.shape
    T, Hkv, dk = k_pool.shape
    if dk != d or tuple(v_pool.shape) != tuple(k_pool.shape) or offsets.numel() != N or lens.numel() != N:
        raise ValueError("shape mismatch between q, pools, offsets and lens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    workspace = _decode_workspace(workspace, N, Hq, Hkv, d, max_len, dev)
    o = _output(out, q.shape, torch.bfloat16, dev, "out")
    lse = _output(lse_out, (N, Hq), torch.float32, dev, "lse_out") if return_lse else None
    args = (q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), offsets.data_ptr(), lens.data_ptr(), o.data_ptr(),
            lse.data_ptr() if lse is not None else None, N, Hq, Hkv, d, T, int(max_len), int(window), float(scale))
    tail = (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    if fmt == 0:
        _run(dev, lib().attn_decode, *args, *tail)
    else:
        _run(dev, lib().attn_decode_fp8, *args, fmt, float(k_scale), float(v_scale), *tail)
    return (o, lse) if return_lse else o


def attn_decode_noalloc(q, k_pool, v_pool, offsets, lens, *, max_len: int, out, lse_out=None, window: int = 0,
                        scale: float | None = None):
    """attn_decode (bf16 pools) through the entry point that allocates nothing: the library's fixed
    per-GPU workspace of DECODE_NOALLOC_BYTES replaces the caller's, and the outputs ``out``
    [N, Hq, d] bf16 and optional ``lse_out`` [N, Hq] fp32 must be given.  Calls that overlap in
    time on one GPU race (they share that workspace)."""
    import torch
    dev = _require_gpu(q, k_pool, v_pool, offsets, lens)
    if _kv_format(q, k_pool, v_pool, None, None, None) != 0:
        raise ValueError("attn_decode_noalloc takes bfloat16 pools")
    if offsets.dtype != torch.int64 or lens.dtype != torch.int32:
        raise ValueError("offsets must be int64 and lens int32")
    if q.dim() != 3 or k_pool.dim() != 3:
        raise ValueError("expected q [N, Hq, d] and pools [T, Hkv, d]")
    N, Hq, d = q.shape
    T, Hkv, dk = k_pool.shape
    if dk != d or tuple(v_pool.shape) != tuple(k_pool.shape) or offsets.numel() != N or lens.numel() != N:
        raise ValueError("shape mismatch between q, pools, offsets and lens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = _output(out, q.shape, torch.bfloat16, dev, "out")
    lse = _output(lse_out, (N, Hq), torch.float32, dev, "lse_out") if lse_out is not None else None
    _run(dev, lib().attn_decode_noalloc, q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), offsets.data_ptr(),
         lens.data_ptr(), o.data_ptr(), lse.data_ptr() if lse is not None else None, N, Hq, Hkv, d, T, int(max_len),
         int(window), float(scale))
    return o


def attn_decode_paged(q, k_pool, v_pool, block_table, lens, *, page_size: int, max_len: int, window: int = 0,
                      scale: float | None = None, return_lse: bool = False, workspace=None, out=None,
                      lse_out=None, kv_format: str | None = None, k_scale: float | None = None,
                      v_scale: float | None = None):
    """Decode one query token per sequence against a paged KV cache.

    q [N, Hq, d] bf16; k_pool, v_pool [pool_pages * page_size, Hkv, d] bf16 (physical page p
    is rows p * page_size .. + page_size - 1); block_table int32 [N, table_stride] (entry j of
    sequence s: the page holding its tokens j * page_size .. + page_size - 1); lens int32 [N];
    max_len >= max(lens).  FP8 pools as attn_decode.  Returns O [N, Hq, d] bf16 and, when
    ``return_lse``, LSE [N, Hq]."""
    import torch
    dev = _require_gpu(q, k_pool, v_pool, block_table, lens)
    fmt = _kv_format(q, k_pool, v_pool, kv_format, k_scale, v_scale)
    if q.dim() != 3 or k_pool.dim() != 3:
        raise ValueError("expected q [N, Hq, d] and pools [pool_pages * page_size, Hkv, d]")
    if block_table.dtype != torch.int32 or lens.dtype != torch.int32:
        raise ValueError("block_table and lens must be int32")
    if block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [N, table_stride] tensor")
    N, Hq, d = q.shape
    T, Hkv, dk = k_pool.shape
    if page_size < 1 or T % page_size != 0:
        raise ValueError("the pools must hold a whole number of pages")
    if (dk != d or tuple(v_pool.shape) != tuple(k_pool.shape) or block_table.shape[0] != N
            or lens.numel() != N):
        raise ValueError("shape mismatch between q, pools, block_table and lens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    workspace = _decode_workspace(workspace, N, Hq, Hkv, d, max_len, dev)
    o = _output(out, q.shape, torch.bfloat16, dev, "out")
    lse = _output(lse_out, (N, Hq), torch.float32, dev, "lse_out") if return_lse else None
    args = (q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(), int(block_table.shape[1]),
            int(page_size), T // page_size, lens.data_ptr(), o.data_ptr(), lse.data_ptr() if lse is not None else None,
            N, Hq, Hkv, d, int(max_len), int(window), float(scale))
    tail = (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    if fmt == 0:
        _run(dev, lib().attn_decode_paged, *args, *tail)
    else:
        _run(dev, lib().attn_decode_paged_fp8, *args, fmt, float(k_scale), float(v_scale), *tail)
    return (o, lse) if return_lse else o


def probe_mfma_ceiling(workgroups: int, steps: int, sink, mode: int = 1) -> None:
    """Enqueue the matrix-core ceiling probe (include/attn_probe.h; mode 0: MFMAs alone, 1: with
    LDS operands, 2: with the softmax's vector work too, 3: with the per-step barrier, 4: with the
    per-step global->LDS loads) on the current stream of the sink's GPU; ``sink`` is a float32
    device tensor of at least workgroups * 256 elements, plus PROBE_SOURCE_BYTES / 4 in front
    (the source blocks) for mode 4."""
    import torch
    dev = _require_gpu(sink)
    if sink.dtype != torch.float32:
        raise ValueError("sink must be float32")
    _run(dev, lib().attn_probe_mfma_ceiling, int(mode), int(workgroups), int(steps), sink.data_ptr(), sink.numel() * 4)


def fwd_plan(B, Hq, Hkv, Lq, Lk, d, causal=False, window=0, f32=False) -> dict:
    info = FwdPlanInfo()
    _check(lib().attn_fwd_plan(B, Hq, Hkv, Lq, Lk, d, int(bool(causal)), int(window), int(bool(f32)),
                               ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in FwdPlanInfo._fields_}


def fwd_schedule(B, Hq, Hkv, Lq, Lk, d, causal=False, window=0, f32=False) -> np.ndarray:
    """[num_workgroups, 3] array of (batch, query head, query tile) per workgroup index."""
    n = fwd_plan(B, Hq, Hkv, Lq, Lk, d, causal, window, f32)["num_workgroups"]
    out = np.zeros((n, 3), dtype=np.int32)
    _check(lib().attn_fwd_schedule(B, Hq, Hkv, Lq, Lk, d, int(bool(causal)), int(window), int(bool(f32)),
                                   out.ctypes.data, out.size))
    return out


def fwd_varlen_schedule(n_seq, Hq, Hkv, max_seqlen_q) -> np.ndarray:
    """[num_blocks, 3] (sequence, query head, query tile) per block of attn_fwd_varlen; sequence
    n_seq marks a block without work."""
    n = ctypes.c_int64()
    _check(lib().attn_fwd_varlen_schedule(n_seq, Hq, Hkv, max_seqlen_q, None, 0, ctypes.byref(n)))
    out = np.zeros((n.value, 3), dtype=np.int32)
    _check(lib().attn_fwd_varlen_schedule(n_seq, Hq, Hkv, max_seqlen_q, out.ctypes.data, out.size, ctypes.byref(n)))
    return out


def decode_plan(n_seq: int, Hq: int, Hkv: int, d: int) -> tuple[int, int, int]:
    """(teams, rows per sequence, tokens per block) of the decode split on the current device."""
    t, r, b = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().attn_decode_plan(int(n_seq), int(Hq), int(Hkv), int(d), ctypes.byref(t), ctypes.byref(r),
                                  ctypes.byref(b)))
    return t.value, r.value, b.value


def decode_rows(Hq: int, Hkv: int) -> np.ndarray:
    """[rows_per_seq, 3] (KV head, first query head, query heads) of each row of the decode split."""
    n = max(1, int(Hkv)) * max(1, -(-(int(Hq) // max(1, int(Hkv))) // 32))  # enough for either layout
    kv, first, nh = (np.zeros(n, np.int32) for _ in range(3))
    _check(lib().attn_decode_rows(int(Hq), int(Hkv), kv.ctypes.data, first.ctypes.data, nh.ctypes.data, n))
    rows = 1 if (Hq <= 32 and 32 % Hkv == 0) else n
    return np.stack([kv[:rows], first[:rows], nh[:rows]], axis=1)


def decode_pieces(lens, teams: int, tokens_per_block: int = 32, window: int = 0, max_len: int | None = None,
                  pool_rows: int | None = None, offsets=None, aligned: bool = False) -> list[tuple[int, int, int, int]]:
    """The (team, sequence, first block, blocks) pieces of one row of the decode split, in the
    order the split computes them (host-side restatement of the plan for tests and tools).
    ``aligned`` (paged caches): block 0 starts at the tokens_per_block boundary at or below the
    first visible key instead of at the key itself."""
    nb = []
    for s, n in enumerate(lens):
        n = int(n)
        ok = n >= 0 and (max_len is None or n <= max_len)
        if offsets is not None:
            ok = ok and int(offsets[s]) >= 0 and (pool_rows is None or int(offsets[s]) + n <= pool_rows)
        vis = min(n, window) if (window > 0 and n > window) else n
        org = n - vis
        if aligned:
            org -= org % tokens_per_block
        nb.append(-(-(n - org) // tokens_per_block) if ok and n > org else 0)
    total = sum(nb)
    share = -(-total // teams) if total else 0
    out, p = [], 0
    for s, b in enumerate(nb):
        if b:
            for t in range(p // share, (p + b - 1) // share + 1):
                lo, hi = max(p, t * share), min(p + b, (t + 1) * share)
                out.append((t, s, lo - p, hi - lo))
        p += b
    return out
