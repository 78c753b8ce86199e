"""Seeded random shapes through the C ABI against the fp64 oracle, element by element.

The parametrized parity tests pick their edge cases by hand; these draw batch, head counts and
grouping, lengths (equal and unequal, ragged against every tile size), head dimension, masking,
window, scale and dtype at random from one fixed seed, so that combinations nobody listed are
covered too.  Every case is reproducible from its id."""
import numpy as np
import pytest

from test_backward_gpu import bwd_case
from test_fp8_gpu import fp8_case, fp8_fwd_case
from test_parity_gpu import decode_case, decode_paged_case, full_case, varlen_case


def _prefill_cases(n=24, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = "f32" if i % 4 == 3 else "bf16"
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 3, 4]))
        Hq = Hkv * int(rng.choice([1, 2, 3, 5, 8]))
        B = int(rng.integers(1, 4))
        lmax = 300 if dtype == "f32" else 700
        Lq = int(rng.integers(1, lmax))
        Lk = Lq if rng.random() < 0.5 else int(rng.integers(1, lmax))
        causal = bool(rng.random() < 0.7)
        window = int(rng.integers(1, Lk + 20)) if causal and rng.random() < 0.5 else 0
        # Other scales for fp32 only: the bf16 bars hold for unit-variance scores (peaked softmax in
        # bf16 has its own test, test_peaked_softmax_bf16_within_rounding).
        draw = rng.random() < 0.25
        scale = round(float(rng.uniform(-1.0, 1.0)), 4) if draw and dtype == "f32" else None
        cases.append((B, Hq, Hkv, Lq, Lk, d, causal, window, dtype, scale, 9000 + i))
    return cases


def _decode_cases(n=12, seed=20261204):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        n_seq = int(rng.integers(1, 70))
        kind = rng.random(n_seq)
        lens = np.where(kind < 0.1, 0,
                        np.where(kind < 0.4, rng.integers(1, 40, n_seq), rng.integers(40, 3000, n_seq)))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
        if i % 4 == 0:  # more query heads per KV head than one 32-column block holds, not a multiple
            Hkv, Hq = (1, 48) if i % 8 == 0 else (2, 80)
        d = int(rng.choice([64, 128]))
        window = 0 if rng.random() < 0.6 else int(rng.integers(1, 2000))
        cases.append((lens.astype(np.int32).tolist(), Hq, Hkv, d, window, 9100 + i))
    return cases


def _varlen_cases(n=8, seed=20261205):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        n_seq = int(rng.integers(2, 7))
        lq = rng.integers(0, 400, n_seq)
        if i % 2 == 0:
            lq[int(rng.integers(0, n_seq))] = 0  # a sequence with no new tokens
        lk = lq + rng.integers(0, 1500, n_seq)
        Hkv = int(rng.choice([1, 2, 4]))
        Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
        d = int(rng.choice([64, 128]))
        causal = i % 3 != 2 and bool(rng.random() < 0.8)
        window = int(rng.integers(1, 600)) if causal and rng.random() < 0.4 else 0
        cases.append((lq.tolist(), lk.tolist(), Hq, Hkv, d, causal, window, 9200 + i))
    return cases


def _backward_cases(n=10, seed=20261206):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4]))
        Hq = Hkv * int(rng.choice([1, 2, 3, 4]))
        B = int(rng.integers(1, 3))
        Lq = int(rng.integers(1, 400))
        Lk = Lq if rng.random() < 0.5 else int(rng.integers(1, 400))
        causal = i % 4 != 1 and bool(rng.random() < 0.85)
        window = int(rng.integers(1, Lk + 20)) if causal and i % 3 == 0 else 0
        cases.append((B, Hq, Hkv, Lq, Lk, d, causal, window, 9300 + i))
    return cases


def _fp8_cases(n=10, seed=20261207):
    """FP8 prefill (even draws) and FP8 KV decode (odd draws), both formats."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        fmt = "e4m3fn" if i % 4 < 2 else "e5m2"
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        if i % 2 == 0:
            Lq = int(rng.integers(1, 500))
            Lk = Lq if rng.random() < 0.5 else int(rng.integers(1, 500))
            causal = bool(rng.random() < 0.7)
            window = int(rng.integers(1, Lk + 20)) if causal and rng.random() < 0.5 else 0
            cases.append(("prefill", fmt, int(rng.integers(1, 3)), Hq, Hkv, Lq, Lk, d, causal, window, 9400 + i))
        else:
            n_seq = int(rng.integers(1, 50))
            lens = rng.integers(0, 2500, n_seq)
            lens[0] = max(int(lens[0]), 1)
            window = 0 if rng.random() < 0.6 else int(rng.integers(1, 1500))
            cases.append(("decode", fmt, lens.astype(np.int32).tolist(), Hq, Hkv, d, window, 9400 + i))
    return cases


def _paged_cases(n=8, seed=20261208):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        n_seq = int(rng.integers(1, 40))
        lens = rng.integers(0, 2500, n_seq)
        lens[0] = max(int(lens[0]), 1)
        if i % 2 == 0:
            lens = np.append(lens, 0)  # an empty sequence
        Hkv = int(rng.choice([1, 2, 4, 8]))
        Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
        d = int(rng.choice([64, 128]))
        page = int(rng.choice([32, 64, 128, 256]))  # multiples of every layout's block
        window = 0 if rng.random() < 0.6 else int(rng.integers(1, 1500))
        cases.append((lens.astype(np.int32).tolist(), Hq, Hkv, d, page, window, 9500 + i))
    return cases


def _id(c):
    return "-".join(str(x) if not isinstance(x, list) else f"n{len(x)}" for x in c)


@pytest.mark.gpu
@pytest.mark.parametrize("case", _prefill_cases(), ids=_id)
def test_random_prefill(case):
    B, Hq, Hkv, Lq, Lk, d, causal, window, dtype, scale, seed = case
    full_case(B, Hq, Hkv, Lq, Lk, d, causal, window, dtype, seed=seed, scale=scale)


@pytest.mark.gpu
@pytest.mark.parametrize("case", _decode_cases(), ids=_id)
def test_random_decode(case):
    lens, Hq, Hkv, d, window, seed = case
    if max(lens) == 0:
        lens = lens[:-1] + [1]  # max_len must be at least 1
    decode_case(lens, Hq, Hkv, d, window=window, seed=seed)


@pytest.mark.gpu
@pytest.mark.parametrize("case", _varlen_cases(), ids=_id)
def test_random_varlen(case):
    lq, lk, Hq, Hkv, d, causal, window, seed = case
    varlen_case(lq, lk, Hq, Hkv, d, causal=causal, window=window, seed=seed)


@pytest.mark.gpu
@pytest.mark.parametrize("case", _backward_cases(), ids=_id)
def test_random_backward(case):
    B, Hq, Hkv, Lq, Lk, d, causal, window, seed = case
    bwd_case(B, Hq, Hkv, Lq, Lk, d, causal=causal, window=window, seed=seed)


@pytest.mark.gpu
@pytest.mark.parametrize("case", _fp8_cases(), ids=_id)
def test_random_fp8(case):
    if case[0] == "prefill":
        _, fmt, B, Hq, Hkv, Lq, Lk, d, causal, window, seed = case
        fp8_fwd_case(B, Hq, Hkv, Lq, Lk, d, causal, window, fmt, seed=seed)
    else:
        _, fmt, lens, Hq, Hkv, d, window, seed = case
        fp8_case(lens, Hq, Hkv, d, fmt, window=window, seed=seed)


@pytest.mark.gpu
@pytest.mark.parametrize("case", _paged_cases(), ids=_id)
def test_random_paged_decode(case):
    lens, Hq, Hkv, d, page, window, seed = case
    decode_paged_case(lens, Hq, Hkv, d, page, window=window, seed=seed)


@pytest.mark.gpu
@pytest.mark.parametrize("Hkv,d", [(8, 128), (1, 64)])
def test_decode_many_short_sequences(Hkv, d):
    """Thousands of sequences, most shorter than one block and some empty: far more sequences than
    teams, so shares span many sequences and most pieces are whole short sequences."""
    rng = np.random.default_rng(9600 + Hkv + d)
    lens = rng.integers(0, 90, 3000).astype(np.int32)
    lens[::7] = 0
    lens[1] = 700
    decode_case(lens.tolist(), 8 * Hkv if Hkv > 1 else 16, Hkv, d, seed=9600 + Hkv + d)
    paged = rng.integers(0, 300, 1500).astype(np.int32)
    paged[0] = 1
    decode_paged_case(paged.tolist(), 8 * Hkv if Hkv > 1 else 16, Hkv, d, 64, seed=9650 + Hkv + d)


def test_the_draws_cover_the_space():
    """(Host only.)  The seeded draws include each kind of case at least once, so that a change of
    seed that loses one shows here."""
    pre = _prefill_cases()
    assert {c[5] for c in pre} == {64, 128} and {c[8] for c in pre} == {"bf16", "f32"}
    assert any(c[6] and c[7] for c in pre) and any(not c[6] for c in pre) and any(c[9] is not None for c in pre)
    assert any(c[3] != c[4] for c in pre) and any(c[1] != c[2] for c in pre)
    dec = _decode_cases()
    assert any(0 in c[0] for c in dec) and any(c[4] for c in dec) and any(c[1] % 32 and c[1] > 32 for c in dec)
    var = _varlen_cases()
    assert any(0 in c[0] for c in var) and any(c[6] for c in var) and any(not c[5] for c in var)
    bwd = _backward_cases()
    assert any(c[7] for c in bwd) and any(not c[6] for c in bwd) and any(c[3] != c[4] for c in bwd)
    assert {c[5] for c in bwd} == {64, 128}
    f8 = _fp8_cases()
    assert {c[0] for c in f8} == {"prefill", "decode"} and {c[1] for c in f8} == {"e4m3fn", "e5m2"}
    pg = _paged_cases()
    assert len({c[4] for c in pg}) >= 3 and any(c[5] for c in pg) and any(0 in c[0] for c in pg)
