"""Decode over an FP8 KV cache (attn_decode_fp8, attn_decode_paged_fp8) against the fp64 oracle.

Pools hold E4M3 or E5M2 codes with one scale per pool (workloads.to_fp8_codes); the oracle decodes
the same codes itself (oracle.fp8) and attends exactly.  Codes convert exactly to bf16, so the bar
is the bf16 decode bar (parity.check).  With power-of-two scales the FP8 path must also equal the
bf16 path bit for bit on the same values, since every scaling is then exact."""
import math

import numpy as np
import pytest
import torch

import attention_attn_fwd_03_amd as af
import oracle
import workloads as wl
from parity import FP8_MFMA_EPS, check, record, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
FMTS = ["e4m3fn", "e5m2"]


def gather_codes(kc, vc, offsets, lens, seqs):
    ks, vs, offs, ls, pos = [], [], [], [], 0
    for s in seqs:
        a, n = int(offsets[s]), int(lens[s])
        ks.append(kc[a:a + n].cpu().numpy())
        vs.append(vc[a:a + n].cpu().numpy())
        offs.append(pos)
        ls.append(n)
        pos += n
    return np.concatenate(ks), np.concatenate(vs), np.array(offs, np.int64), np.array(ls, np.int32)


def run(q, kc, vc, offs, lens, max_len, window, scale, fmt, ks, vs):
    N, Hq, d = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((N, Hq), float("nan"), device=q.device, dtype=torch.float32)
    af.attn_decode(q, kc, vc, offs, lens, max_len=max_len, window=window, scale=scale, return_lse=True, out=o,
                   lse_out=lse, kv_format=fmt, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    return o, lse


def fp8_case(lens, Hq, Hkv, d, fmt, window=0, seed=0, scale=None, seqs=None, scale_mult=None, max_gap=37):
    """scale_mult = (a, b) multiplies the pools' quantisation scales (the keys by a, the values by
    b); O grows by b and is compared after dividing by b, so the unit-scale bar applies."""
    lens = np.asarray(lens, np.int32)
    label = f"fp8 decode {fmt} N{len(lens)} Hq{Hq} Hkv{Hkv} d{d} W{window} seed{seed} lens[:8]={lens[:8].tolist()}"
    say(label)
    q, kc, vc, offs, lens_t, layout, ks, vs = wl.fp8_decode_inputs(len(lens), Hq, Hkv, d, lens, fmt, seed=seed,
                                                                   max_gap=max_gap)
    vmul = 1.0
    if scale_mult is not None:
        ks, vs, vmul = ks * scale_mult[0], vs * scale_mult[1], scale_mult[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o, lse = run(q.to(DEV), kc.to(DEV), vc.to(DEV), offs.to(DEV), lens_t.to(DEV), int(max(lens.max(), 1)), window,
                 scale, fmt, ks, vs)
    seqs = list(range(len(lens))) if seqs is None else seqs
    kg, vg, po, pl = gather_codes(kc, vc, layout.offsets, layout.lens, seqs)
    O_ref, L_ref = oracle.decode_fp8kv(wl.to_f64(q)[seqs], kg, vg, po, pl, ks, vs, fmt, scale=scale, window=window)
    return check(wl.to_f64(o)[seqs] / vmul, O_ref / vmul, lse.cpu().numpy()[seqs], L_ref, "bf16", label)


MIXED = [1, 31, 32, 33, 0, 64, 5, 100, 1000, 2049, 3, 777]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (32, 1), (8, 8), (40, 8), (64, 1)])
def test_fp8_decode_shapes(fmt, d, Hq, Hkv):
    fp8_case(MIXED, Hq, Hkv, d, fmt, seed=Hq + Hkv + d)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("W", [1, 33, 500])
def test_fp8_decode_window(fmt, W):
    fp8_case(MIXED, 32, 8, 128, fmt, window=W, seed=W)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mult", [(0.37, 2.9), (2.0 ** -2, 2.0 ** 3), (1.7, 0.011)])
def test_fp8_decode_scales(fmt, mult):
    fp8_case(MIXED, 32, 4, 128, fmt, seed=9, scale_mult=mult)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("Hkv", [8, 1])
def test_fp8_equals_bf16_path_with_power_of_two_scales(fmt, Hkv):
    """Codes convert exactly to bf16 and power-of-two scales are exact, so the FP8 kernel and the
    bf16 kernel on the dequantized pool (exact in bf16) produce the same bits."""
    lens = np.array(MIXED, np.int32)
    q, kc, vc, offs, lens_t, layout, _, _ = wl.fp8_decode_inputs(len(lens), 32, Hkv, 128, lens, fmt, seed=4)
    ks, vs = 2.0 ** -3, 2.0 ** 2
    dt = wl.FP8_DTYPES[fmt]
    kb = (kc.view(dt).to(torch.float32) * ks).to(torch.bfloat16)
    vb = (vc.view(dt).to(torch.float32) * vs).to(torch.bfloat16)
    kb = torch.where(torch.isnan(kb), torch.zeros_like(kb), kb)  # NaN gap rows: never read by either path
    vb = torch.where(torch.isnan(vb), torch.zeros_like(vb), vb)
    max_len = int(lens.max())
    o8, l8 = run(q.to(DEV), kc.to(DEV), vc.to(DEV), offs.to(DEV), lens_t.to(DEV), max_len, 0, 0.0884, fmt, ks, vs)
    o = torch.full_like(o8, float("nan"))
    lse = torch.full_like(l8, float("nan"))
    af.attn_decode(q.to(DEV), kb.to(DEV), vb.to(DEV), offs.to(DEV), lens_t.to(DEV), max_len=max_len, scale=0.0884,
                   return_lse=True, out=o, lse_out=lse)
    torch.cuda.synchronize()
    assert torch.equal(o8.view(torch.int16), o.view(torch.int16)) and torch.equal(l8, lse)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", ["gqa_decode_bf16", "mqa_decode_bf16"])
def test_fp8_named_decode(fmt, name):
    """The full decode batch (64 sequences, lengths 1k..32k, NaN codes in the pool's gaps) with an
    FP8 cache: every sequence against the oracle."""
    c = wl.DECODE[name]
    lens = wl.decode_lens(c.n_seq, c.len_lo, c.len_hi, c.lens_seed)
    say(f"fp8 decode {fmt} {name} full size on device")
    q, kc, vc, offs, lens_t, layout, ks, vs = wl.fp8_decode_inputs(c.n_seq, c.Hq, c.Hkv, c.d, lens, fmt,
                                                                   seed=c.value_seed, device=DEV, max_gap=c.max_gap)
    o, lse = run(q, kc, vc, offs, lens_t, int(lens.max()), 0, c.scale, fmt, ks, vs)
    seqs = list(range(c.n_seq))
    kg, vg, po, pl = gather_codes(kc, vc, layout.offsets, layout.lens, seqs)
    O_ref, L_ref = oracle.decode_fp8kv(wl.to_f64(q)[seqs], kg, vg, po, pl, ks, vs, fmt, scale=c.scale)
    record(name.replace("_bf16", f"_fp8_{fmt}"), check(wl.to_f64(o)[seqs], O_ref, lse.cpu().numpy()[seqs], L_ref,
                                                         "bf16", name + " " + fmt))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("W,Hkv", [(1, 8), (45, 2), (700, 1)])
def test_fp8_decode_paged_window(fmt, W, Hkv):
    """An FP8 paged cache under a window: block 0 starts at the block boundary below the first
    visible key (masked up to it), and table entries of pages wholly before the window are -1, so
    reading one would turn the sequence's output into NaN."""
    P = 32
    lens = np.array([1, 50, 1031, 3 * 1024 + 1, 2000, 33, 64, 0], np.int32)
    label = f"fp8 paged window {fmt} W{W} Hkv{Hkv}"
    say(label)
    q, kc, vc, table, lens_t, layout, ks, vs = wl.fp8_paged_decode_inputs(len(lens), 16, Hkv, 128, lens, P, fmt,
                                                                          seed=W + Hkv, extra_pages=2)
    ktab = table.clone()  # the kernel's table; the oracle gathers every token, so it gets the full one
    for s_, n in enumerate(layout.lens):
        ktab[s_, :max(int(n) - W, 0) // P] = -1
    o = torch.full((len(lens), 16, 128), float("nan"), device=DEV, dtype=torch.bfloat16)
    lse = torch.full((len(lens), 16), float("nan"), device=DEV, dtype=torch.float32)
    af.attn_decode_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), ktab.to(DEV), lens_t.to(DEV), page_size=P,
                         max_len=int(lens.max()), window=W, scale=0.0884, return_lse=True, out=o, lse_out=lse,
                         kv_format=fmt, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.decode_paged_fp8kv(wl.to_f64(q), kc.numpy(), vc.numpy(), layout.table, layout.lens, P,
                                             ks, vs, fmt, scale=0.0884, window=W)
    check(wl.to_f64(o), O_ref, lse.cpu().numpy(), L_ref, "bf16", label)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("Hkv,P,d", [(8, 16, 128), (8, 64, 128), (1, 32, 128), (2, 48, 128), (8, 32, 64), (1, 64, 64)])
def test_fp8_decode_paged(fmt, Hkv, P, d):
    lens = np.array(MIXED, np.int32)
    label = f"fp8 paged {fmt} Hkv{Hkv} P{P} d{d}"
    say(label)
    q, kc, vc, table, lens_t, layout, ks, vs = wl.fp8_paged_decode_inputs(len(lens), 32, Hkv, d, lens, P, fmt,
                                                                          seed=P + Hkv + d, extra_pages=3)
    o = torch.full((len(lens), 32, d), float("nan"), device=DEV, dtype=torch.bfloat16)
    lse = torch.full((len(lens), 32), float("nan"), device=DEV, dtype=torch.float32)
    af.attn_decode_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), table.to(DEV), lens_t.to(DEV), page_size=P,
                         max_len=int(lens.max()), scale=0.0884, return_lse=True, out=o, lse_out=lse, kv_format=fmt,
                         k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.decode_paged_fp8kv(wl.to_f64(q), kc.numpy(), vc.numpy(), layout.table, layout.lens, P, ks,
                                             vs, fmt, scale=0.0884)
    check(wl.to_f64(o), O_ref, lse.cpu().numpy(), L_ref, "bf16", label)


@pytest.mark.parametrize("fmt", FMTS)
def test_fp8_invalid_sequences_report_nan(fmt):
    """A sequence whose range leaves the pool is not read and reports NaN; the others are exact."""
    lens = np.array([40, 70, 5, 33], np.int32)
    q, kc, vc, offs, lens_t, layout, ks, vs = wl.fp8_decode_inputs(4, 16, 4, 64, lens, fmt, seed=3)
    bad = offs.clone()
    bad[1] = layout.total_rows - 10  # runs past the end of the pool
    o, lse = run(q.to(DEV), kc.to(DEV), vc.to(DEV), bad.to(DEV), lens_t.to(DEV), 70, 0, 0.125, fmt, ks, vs)
    assert torch.isnan(o[1]).all().item() and torch.isnan(lse[1]).all().item()
    good = [0, 2, 3]
    kg, vg, po, pl = gather_codes(kc, vc, layout.offsets, layout.lens, good)
    O_ref, L_ref = oracle.decode_fp8kv(wl.to_f64(q)[good], kg, vg, po, pl, ks, vs, fmt, scale=0.125)
    check(wl.to_f64(o)[good], O_ref, lse.cpu().numpy()[good], L_ref, "bf16", "fp8 invalid")


# ---------------------------------------------------------------------------------------------
# Prefill over FP8 Q, K, V (attn_fwd_fp8).  The oracle attends exactly over the dequantized
# tensors; P is rounded to bf16 as in the bf16 kernel, so the bf16 bar applies to O; the LSE bar
# adds the FP8 matrix cores' accumulation error (parity.FP8_MFMA_EPS).

def fp8_lse_allowance(qd, kd, scale, rows=None):
    """Per query row: FP8_MFMA_EPS * |scale| * max_j sum_i |q_i k_ji| (every key j, an upper bound)
    for dequantized q [B, Hq, Lq, d], k [B, Hkv, Lk, d]; ``rows`` picks (b, h, i) samples."""
    B, Hq, Lq, d = qd.shape
    g = Hq // kd.shape[1]
    if rows is None:
        out = np.empty((B, Hq, Lq))
        for b in range(B):
            for h in range(Hq):
                out[b, h] = (np.abs(qd[b, h]) @ np.abs(kd[b, h // g]).T).max(axis=1)
    else:
        out = np.array([(np.abs(qd[b, h, i]) @ np.abs(kd[b, h // g]).T).max() for b, h, i in rows])
    return FP8_MFMA_EPS * abs(scale) * out


def fp8_fwd_case(B, Hq, Hkv, Lq, Lk, d, causal, window, fmt, seed, scale=None, scale_mult=(1.0, 1.0, 1.0)):
    label = f"fp8 fwd {fmt} B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} d{d} causal{int(causal)} W{window} seed{seed} scale{scale}"
    say(label)
    qc, kc, vc, qs, ks, vs = wl.fp8_prefill_inputs(B, Hq, Hkv, Lq, Lk, d, fmt, seed=seed)
    qs, ks, vs = qs * scale_mult[0], ks * scale_mult[1], vs * scale_mult[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o = torch.full((B, Hq, Lq, d), float("nan"), device=DEV, dtype=torch.bfloat16)
    lse = torch.full((B, Hq, Lq), float("nan"), device=DEV, dtype=torch.float32)
    af.attn_fwd_fp8(qc.to(DEV), kc.to(DEV), vc.to(DEV), qkv_format=fmt, q_scale=qs, k_scale=ks, v_scale=vs,
                    causal=causal, window=window, scale=scale, return_lse=True, out=o, lse_out=lse)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_fp8(qc.numpy(), kc.numpy(), vc.numpy(), qs, ks, vs, fmt, scale=scale,
                                        causal=causal, window=window)
    vm = scale_mult[2]
    extra = fp8_lse_allowance(oracle.dequantize(qc.numpy(), qs, fmt), oracle.dequantize(kc.numpy(), ks, fmt), scale)
    stats = check(wl.to_f64(o) / vm, O_ref / vm, lse.cpu().numpy(), L_ref, "bf16", label, lse_abs_extra=extra)
    say(stats)
    return stats


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,causal", [(1, True), (33, False), (128, True), (129, True), (300, False), (517, True)])
def test_fp8_fwd_lengths(fmt, d, L, causal):
    fp8_fwd_case(1, 4, 2, L, L, d, causal, 0, fmt, seed=L + d)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 1), (12, 4)])
def test_fp8_fwd_head_groups(fmt, Hq, Hkv):
    fp8_fwd_case(2, Hq, Hkv, 200, 200, 128, True, 0, fmt, seed=Hq * Hkv)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("Lq,Lk", [(100, 333), (333, 100), (1, 700), (257, 64)])
def test_fp8_fwd_unequal_lengths(fmt, Lq, Lk):
    fp8_fwd_case(1, 4, 2, Lq, Lk, 128, True, 0, fmt, seed=Lq + Lk)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("W,d", [(1, 64), (37, 128), (64, 128), (500, 64)])
def test_fp8_fwd_windows(fmt, W, d):
    fp8_fwd_case(1, 4, 2, 600, 600, d, True, W, fmt, seed=W)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("scale,mult", [(0.0, (1.0, 1.0, 1.0)), (-0.1, (1.0, 1.0, 1.0)), (0.05, (3.0, 0.5, 7.0))])
def test_fp8_fwd_scales(fmt, scale, mult):
    fp8_fwd_case(1, 4, 2, 300, 300, 128, True, 0, fmt, seed=11, scale=scale, scale_mult=mult)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", ["gqa_causal_bf16_L4096", "swa_gqa_bf16_L16384_W4096"])
def test_fp8_fwd_named_workload_full_size(fmt, name):
    """The causal GQA L4096 workload (B2 Hq32 Hkv8 d128) and the window workload (L16384, W4096)
    with FP8 inputs, full-size launch, against the oracle over the whole output."""
    c = wl.PREFILL[name]
    say(f"fp8 fwd {fmt} {name} full size on device")
    qc, kc, vc, qs, ks, vs = wl.fp8_prefill_inputs(c.B, c.Hq, c.Hkv, c.Lq, c.Lk, c.d, fmt, seed=c.seed, device=DEV)
    o, lse = af.attn_fwd_fp8(qc, kc, vc, qkv_format=fmt, q_scale=qs, k_scale=ks, v_scale=vs, causal=True,
                             window=c.window, scale=c.scale, return_lse=True)
    torch.cuda.synchronize()
    og, lg = wl.to_f64(o), lse.cpu().numpy()
    del o, lse
    qd, kd, vd = (oracle.dequantize(x.cpu().numpy(), s_, fmt) for x, s_ in ((qc, qs), (kc, ks), (vc, vs)))
    O_ref, L_ref = oracle.attention(qd, kd, vd, scale=c.scale, causal=True, window=c.window)
    extra = fp8_lse_allowance(qd, kd, c.scale)
    record(name.replace("_bf16_", f"_fp8_{fmt}_"), check(og, O_ref, lg, L_ref, "bf16", f"fp8 {name}",
                                                          lse_abs_extra=extra))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_score_accumulation_error(fmt, d):
    """Measures the bound the FP8 LSE bar rests on.  With one key per row (Lk = 1, no mask) the
    row's probability is exactly 1, so its LSE is the score itself, scale * q . k, read back
    through fp32 (a few ulps).  Over 32768 scores of uniformly random finite codes (the full range
    of the format, both signs) the error of each must stay within FP8_MFMA_EPS * |scale| *
    sum_i |q_i k_i|; the largest measured ratio is printed."""
    rng = np.random.default_rng(77 + d)
    B, H, Lq = 2, 16, 1024
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.dequantize(codes, 1.0, fmt)
    finite = codes[np.isfinite(vals)]
    qc = rng.choice(finite, size=(B, H, Lq, d)).astype(np.uint8)
    kc = rng.choice(finite, size=(B, H, 1, d)).astype(np.uint8)
    vc = rng.choice(finite, size=(B, H, 1, d)).astype(np.uint8)
    qd, kd = oracle.dequantize(qc, 1.0, fmt), oracle.dequantize(kc, 1.0, fmt)
    scale = 1.0 / math.sqrt(d)
    _, lse = af.attn_fwd_fp8(torch.from_numpy(qc).to(DEV), torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV),
                             qkv_format=fmt, q_scale=1.0, k_scale=1.0, v_scale=1.0, causal=False, scale=scale,
                             return_lse=True)
    torch.cuda.synchronize()
    exact = scale * np.einsum("bhid,bhd->bhi", qd, kd[:, :, 0])
    mag = abs(scale) * np.einsum("bhid,bhd->bhi", np.abs(qd), np.abs(kd[:, :, 0]))
    err = np.abs(lse.cpu().numpy().astype(np.float64) - exact)
    # what fp32 itself costs: the fold of the scale into log2(e) units and back (a few ulps)
    fp32_part = 8 * np.finfo(np.float32).eps * np.abs(exact)
    ratio = np.maximum(err - fp32_part, 0.0) / np.maximum(mag, 1e-30)
    record(f"fp8_{fmt}_score_accumulation_d{d}",
           {"max_err_over_abs_sum": float(ratio.max()), "bound": FP8_MFMA_EPS, "scores": int(ratio.size)})
    assert np.all(np.isfinite(lse.cpu().numpy()))
    assert ratio.max() <= FP8_MFMA_EPS


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", ["gqa_decode_bf16", "mqa_decode_bf16"])
def test_fp8_named_decode_paged(fmt, name):
    """The full decode batch with an FP8 cache in 64-token pages scattered over the pool (spare
    pages and page tails NaN codes): every sequence against the oracle."""
    c = wl.DECODE[name]
    P = 64
    lens = wl.decode_lens(c.n_seq, c.len_lo, c.len_hi, c.lens_seed)
    say(f"fp8 paged decode {fmt} {name} full size on device, P{P}")
    q, kc, vc, table, lens_t, layout, ks, vs = wl.fp8_paged_decode_inputs(c.n_seq, c.Hq, c.Hkv, c.d, lens, P, fmt,
                                                                          seed=c.value_seed, device=DEV, extra_pages=97)
    o, lse = af.attn_decode_paged(q, kc, vc, table, lens_t, page_size=P, max_len=int(lens.max()), scale=c.scale,
                                  return_lse=True, kv_format=fmt, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    seqs = list(range(c.n_seq))
    tab = layout.table
    used = sorted({int(tab[s_, j]) for s_ in seqs for j in range(-(-int(lens[s_]) // P))})
    new_id = {p_: i for i, p_ in enumerate(used)}
    rows = torch.tensor([p_ * P + r for p_ in used for r in range(P)], dtype=torch.int64, device=DEV)
    kcomp, vcomp = kc.index_select(0, rows).cpu().numpy(), vc.index_select(0, rows).cpu().numpy()
    sub = np.full((len(seqs), tab.shape[1]), -1, np.int64)
    for i, s_ in enumerate(seqs):
        for j in range(-(-int(lens[s_]) // P)):
            sub[i, j] = new_id[int(tab[s_, j])]
    O_ref, L_ref = oracle.decode_paged_fp8kv(wl.to_f64(q)[seqs], kcomp, vcomp, sub, lens[seqs], P, ks, vs, fmt,
                                             scale=c.scale)
    record(name.replace("_bf16", f"_fp8_{fmt}") + "_paged_P64",
           check(wl.to_f64(o)[seqs], O_ref, lse.cpu().numpy()[seqs], L_ref, "bf16", f"{name} {fmt} paged"))
