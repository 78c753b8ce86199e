"""Plant plausible mistakes in the oracle (on the CPU) and require that each one fails at
least one pin.  This shows the pins can tell a wrong oracle from a right one."""
import importlib

import numpy as np
import pytest

import oracle_pins as pins

mod = importlib.import_module("oracle.attention")


def _interleaved_kv_head(h, Hq, Hkv):
    return h % Hkv


def _window_one_too_wide(rows, Lq, Lk, causal, window):
    p = rows[:, None] + (Lk - Lq)
    j = np.arange(Lk)[None, :]
    vis = np.ones((len(rows), Lk), dtype=bool)
    if causal:
        vis &= j <= p
    if window > 0:
        vis &= j >= p - window
    return vis


def _causal_top_left(rows, Lq, Lk, causal, window):
    p = rows[:, None]
    j = np.arange(Lk)[None, :]
    vis = np.ones((len(rows), Lk), dtype=bool)
    if causal:
        vis &= j <= p
    if window > 0:
        vis &= j > p - window
    return vis


def _scale_dropped(q, k, scale):
    return np.asarray(q, np.float64) @ np.asarray(k, np.float64).T


def _scale_squared(q, k, scale):
    return scale * scale * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)


def _make_softmax(variant):
    orig = mod.masked_softmax

    def f(S, vis):
        if variant == "bias":       # large negative bias instead of exclusion
            S2 = np.where(vis, S, S - 1e4)
            m = S2.max(axis=1)
            E = np.exp(S2 - m[:, None])
            l = E.sum(axis=1)
            return E / l[:, None], m + np.log(l)
        P, lse = orig(S, vis)
        if variant == "lse_no_max":  # dropped the max term of the LSE
            m = np.where(vis.any(axis=1), np.where(vis, S, -np.inf).max(axis=1), 0.0)
            return P, lse - m
        if variant == "no_normalise":
            E = np.where(vis, np.exp(S - np.where(vis, S, -np.inf).max(axis=1, keepdims=True)), 0.0)
            return E, lse
        if variant == "log2_lse":
            return P, lse / np.log(2.0)
        raise AssertionError(variant)
    return f


def _merge_unweighted(outs, lses):
    outs, lses = np.asarray(outs, np.float64), np.asarray(lses, np.float64)
    return outs.mean(axis=0), np.log(np.exp(lses).sum(axis=0))


def _decode_window_from_start(q, k_pool, v_pool, offsets, lens, scale=None, window=0, threads=None, seqs=None):
    # the window counted from the oldest key instead of the newest
    N, Hq, d = np.asarray(q).shape
    scale = 1 / np.sqrt(d) if scale is None else scale
    O = np.zeros((N, Hq, d)); L = np.zeros((N, Hq))
    for s in range(N):
        a, n = int(offsets[s]), int(lens[s])
        nn = min(n, window) if window else n
        for h in range(Hq):
            kh = h // (Hq // k_pool.shape[1])
            o, l = mod.attention_head(np.asarray(q)[s, h][None], k_pool[a:a + nn, kh], v_pool[a:a + nn, kh], scale,
                                      False, 0)
            O[s, h], L[s, h] = o[0], l[0]
    return O, L


def _paged_rows_unscaled(table_row, n, page_size):
    # forgot to multiply the page number by the page size
    t = np.arange(n)
    return np.asarray(table_row, np.int64)[t // page_size] + t % page_size


def _paged_rows_swapped(table_row, n, page_size):
    # page slot and offset inside the page exchanged
    t = np.arange(n)
    return np.asarray(table_row, np.int64)[t % page_size % len(table_row)] * page_size + t // page_size


def _seq_rows_from_zero(pool, start, n):
    # the sequence's offset into the pool forgotten
    return np.asarray(pool[:n], np.float64)


def _softmax_backward_no_rowsum(P, dP, O, dO):
    # the rowsum(dO * O) term of the softmax Jacobian dropped
    return P * dP


def _key_grads_unscaled(dS, P, q, dO, scale):
    # dK without the score scale
    return dS.T @ q, P.T @ dO


def _rows_reversed(q, k, v, samples, scale=None, causal=False, window=0, threads=None):
    # the rows come back in the reverse of the requested order
    O, L = _orig_rows(q, k, v, samples, scale=scale, causal=causal, window=window, threads=threads)
    return O[::-1].copy(), L[::-1].copy()


def _rows_offset_dropped(q, k, v, samples, scale=None, causal=False, window=0, threads=None):
    # the requested row index ignored: the n-th sample computes row n of its head
    samples = [(b, h, min(n, np.asarray(q).shape[2] - 1)) for n, (b, h, _) in enumerate(samples)]
    return _orig_rows(q, k, v, samples, scale=scale, causal=causal, window=window, threads=threads)


def _rows_mask_dropped(q, k, v, samples, scale=None, causal=False, window=0, threads=None):
    # the causal mask (and window) not applied to sampled rows
    return _orig_rows(q, k, v, samples, scale=scale, causal=False, window=0, threads=threads)


_orig_rows = mod.attention_rows


MUTANTS = {
    "gqa_interleaved": ("kv_head", _interleaved_kv_head),
    "window_off_by_one": ("_visibility_rows", _window_one_too_wide),
    "causal_top_left": ("_visibility_rows", _causal_top_left),
    "scale_dropped": ("scores", _scale_dropped),
    "scale_squared": ("scores", _scale_squared),
    "mask_as_bias": ("masked_softmax", "bias"),
    "lse_missing_max": ("masked_softmax", "lse_no_max"),
    "softmax_not_normalised": ("masked_softmax", "no_normalise"),
    "lse_base2": ("masked_softmax", "log2_lse"),
    "merge_unweighted": ("merge_partials", _merge_unweighted),
    "paged_rows_unscaled": ("paged_rows", _paged_rows_unscaled),
    "paged_rows_swapped": ("paged_rows", _paged_rows_swapped),
    "varlen_offsets_ignored": ("_seq_rows", _seq_rows_from_zero),
    "backward_no_rowsum": ("_softmax_backward", _softmax_backward_no_rowsum),
    "backward_dk_unscaled": ("_key_grads", _key_grads_unscaled),
    "rows_order_reversed": ("attention_rows", _rows_reversed),
    "rows_offset_dropped": ("attention_rows", _rows_offset_dropped),
    "rows_mask_dropped": ("attention_rows", _rows_mask_dropped),
}


def _run_all_checks():
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check()
        except Exception as e:  # AssertionError or a shape error from a broken oracle
            failed.append(check.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, repl = MUTANTS[name]
    if attr == "masked_softmax":
        repl = _make_softmax(repl)
    monkeypatch.setattr(mod, attr, repl)
    import oracle
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, repl)
    failed = _run_all_checks()
    assert failed, f"mutant {name} passed every pin"


def test_decode_window_mutant_is_caught(monkeypatch):
    import oracle
    monkeypatch.setattr(oracle, "decode", _decode_window_from_start)
    monkeypatch.setattr(mod, "decode", _decode_window_from_start)
    failed = _run_all_checks()
    assert failed


# ---- FP8 KV cache (oracle/fp8.py) -----------------------------------------------------------

fp8mod = importlib.import_module("oracle.fp8")


def _e4m3_bias8(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m / 8.0, -7), np.ldexp(1.0 + m / 8.0, e - 8))
    return sign * np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)


def _e4m3_flush_subnormals(codes):
    c = np.asarray(codes, dtype=np.uint8)
    return np.where(((c >> 3) & 0xF) == 0, 0.0, fp8mod.__dict__["_orig_e4m3"](codes))


def _fp8kv_scales_swapped(q, k_codes, v_codes, offsets, lens, k_scale, v_scale, fmt, **kw):
    return fp8mod.decode(q, fp8mod.dequantize(k_codes, v_scale, fmt), fp8mod.dequantize(v_codes, k_scale, fmt),
                         offsets, lens, **kw)


def _fp8_attention_v_unscaled(q_codes, k_codes, v_codes, q_scale, k_scale, v_scale, fmt, **kw):
    return fp8mod.attention(fp8mod.dequantize(q_codes, q_scale, fmt), fp8mod.dequantize(k_codes, k_scale, fmt),
                            fp8mod.dequantize(v_codes, 1.0, fmt), **kw)


def _paged_fp8kv_scales_swapped(q, k_codes, v_codes, block_table, lens, page_size, k_scale, v_scale, fmt, **kw):
    return fp8mod.decode_paged(q, fp8mod.dequantize(k_codes, v_scale, fmt), fp8mod.dequantize(v_codes, k_scale, fmt),
                               block_table, lens, page_size, **kw)


def _paged_fp8kv_as_e4m3(q, k_codes, v_codes, block_table, lens, page_size, k_scale, v_scale, fmt, **kw):
    # the format argument ignored
    return fp8mod.decode_paged(q, fp8mod.dequantize(k_codes, k_scale, "e4m3fn"),
                               fp8mod.dequantize(v_codes, v_scale, "e4m3fn"), block_table, lens, page_size, **kw)


FP8_MUTANTS = {
    "fp8_attention_v_scale_dropped": ("attention_fp8", _fp8_attention_v_unscaled),
    "e4m3_bias_8": ("decode_e4m3fn", _e4m3_bias8),
    "e4m3_subnormals_flushed": ("decode_e4m3fn", _e4m3_flush_subnormals),
    "e5m2_read_as_e4m3": ("decode_e5m2", fp8mod.decode_e4m3fn),
    "fp8kv_scales_swapped": ("decode_fp8kv", _fp8kv_scales_swapped),
    "paged_fp8kv_scales_swapped": ("decode_paged_fp8kv", _paged_fp8kv_scales_swapped),
    "paged_fp8kv_format_ignored": ("decode_paged_fp8kv", _paged_fp8kv_as_e4m3),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_planted_fp8_mistake_is_caught(name, monkeypatch):
    import oracle
    attr, repl = FP8_MUTANTS[name]
    monkeypatch.setitem(fp8mod.__dict__, "_orig_e4m3", fp8mod.decode_e4m3fn)
    monkeypatch.setattr(fp8mod, attr, repl)
    monkeypatch.setattr(oracle, attr, repl)
    failed = _run_all_checks()
    assert failed, f"mutant {name} passed every pin"
