"""Checks that pin the fp64 oracle to facts fixed by the attention articles and by
mathematics, independently of the oracle's own code.

Each ``check_*`` raises AssertionError on a mismatch.  ``test_oracle.py`` runs every check;
``test_oracle_mutants.py`` plants plausible mistakes in the oracle and requires that each
one trips at least one check.

Articles cited (by title and section):
  [DS-Attn]  "003-注意力机制详解：从基础Attention到DeepSeek的优化策略" (lakecityint.com)
  [LLM-Attn] "LLM中的Attention实现及优化" (zeeklog.com)
  [MQA-GQA]  tqpw.cn article on MQA → GQA → FlashAttention
  [Deep-Opt] "注意力机制深度优化" (kler.cn)
  [FlashMLA] "高效多头潜在注意力解码技术：Flash MLA深度解析" (developer.baidu.com)
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_example.json")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------------------------
# Pure-Python brute force: a triple loop written from the definition with math.exp / math.fsum.
# Visibility is spelled differently from the oracle on purpose (distance from the query's
# position instead of index comparisons).

def brute_force(q, k, v, scale, causal, window):
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    group = Hq // Hkv
    O = np.zeros((B, Hq, Lq, v.shape[3]))
    LSE = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            kh = h // group
            for i in range(Lq):
                pos = i + Lk - Lq
                keys = []
                for j in range(Lk):
                    dist = pos - j                   # how far back key j lies
                    if causal and dist < 0:
                        continue
                    if window and dist >= window:
                        continue
                    keys.append(j)
                if not keys:
                    O[b, h, i] = 0.0
                    LSE[b, h, i] = -math.inf
                    continue
                s = [scale * math.fsum(float(q[b, h, i, c]) * float(k[b, kh, j, c]) for c in range(d)) for j in keys]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                for c in range(v.shape[3]):
                    O[b, h, i, c] = math.fsum(wj * float(v[b, kh, j, c]) for wj, j in zip(w, keys)) / tot
                LSE[b, h, i] = mx + math.log(tot)
    return O, LSE


TINY_SHAPES = [
    # (Hq, Hkv, Lq, Lk, d)
    (1, 1, 1, 1, 1),
    (2, 1, 3, 5, 3),
    (4, 2, 5, 3, 4),
    (2, 2, 7, 7, 8),
    (4, 1, 12, 12, 2),
    (2, 1, 12, 9, 5),
]
TINY_MODES = [(False, 0), (True, 0), (True, 1), (True, 2), (True, 5)]


def check_brute_force(seed=11):
    rng = _rng(seed)
    for (Hq, Hkv, Lq, Lk, d) in TINY_SHAPES:
        q = rng.standard_normal((1, Hq, Lq, d))
        k = rng.standard_normal((1, Hkv, Lk, d))
        v = rng.standard_normal((1, Hkv, Lk, d))
        scale = 0.7
        for causal, window in TINY_MODES:
            O, L = oracle.attention(q, k, v, scale=scale, causal=causal, window=window)
            Ob, Lb = brute_force(q, k, v, scale, causal, window)
            assert np.array_equal(np.isneginf(L), np.isneginf(Lb)), (Hq, Hkv, Lq, Lk, d, causal, window)
            fin = np.isfinite(Lb)
            assert np.max(np.abs(O - Ob)) <= 1e-12, (Hq, Hkv, Lq, Lk, d, causal, window)
            assert np.max(np.abs(L[fin] - Lb[fin]), initial=0) <= 1e-12, (Hq, Hkv, Lq, Lk, d, causal, window)


# ---------------------------------------------------------------------------------------------
# Library routine: torch's CPU scaled_dot_product_attention in float64 (square shapes only,
# because its is_causal is aligned top-left; GQA through enable_gqa, which expands KV heads
# to consecutive query heads).

def check_torch_sdpa(seed=12):
    import torch
    import torch.nn.functional as F
    rng = _rng(seed)
    for (B, Hq, Hkv, L, d) in [(2, 4, 4, 33, 16), (1, 8, 2, 40, 8), (1, 6, 1, 17, 32)]:
        q = rng.standard_normal((B, Hq, L, d))
        k = rng.standard_normal((B, Hkv, L, d))
        v = rng.standard_normal((B, Hkv, L, d))
        for causal in (False, True):
            scale = 1.0 / math.sqrt(d)
            O, _ = oracle.attention(q, k, v, scale=scale, causal=causal)
            ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                                 is_causal=causal, scale=scale, enable_gqa=(Hq != Hkv)).numpy()
            assert np.max(np.abs(O - ref)) <= 1e-12, (B, Hq, Hkv, L, d, causal)


# ---------------------------------------------------------------------------------------------
# Invariants and closed forms.

def check_softmax_rows(seed=13):
    """Rows of P sum to one, P >= 0, P is exactly 0 where masked ([DS-Attn §一] safe softmax)."""
    rng = _rng(seed)
    for (Lq, Lk, causal, window) in [(9, 9, False, 0), (9, 9, True, 0), (9, 14, True, 3), (14, 9, True, 0)]:
        S = rng.standard_normal((Lq, Lk)) * 5
        vis = oracle.visibility(Lq, Lk, causal, window)
        P, lse = oracle.masked_softmax(S, vis)
        nonempty = vis.any(axis=1)
        assert np.all(P >= 0)
        assert np.all(P[~vis] == 0.0)
        assert np.max(np.abs(P[nonempty].sum(axis=1) - 1.0), initial=0) <= 1e-13
        assert np.all(P[~nonempty] == 0.0) and np.all(np.isneginf(lse[~nonempty]))
        # LSE is the log of the visible sum of exp(S) (direct evaluation; scores are small here)
        direct = np.array([math.log(math.fsum(math.exp(S[i, j]) for j in range(Lk) if vis[i, j]))
                           for i in range(Lq) if nonempty[i]])
        assert np.max(np.abs(lse[nonempty] - direct)) <= 1e-12


def check_constant_scores(seed=14):
    """scale = 0 makes every visible weight equal: O_i = mean of the visible V rows and
    LSE_i = ln(number of visible keys)."""
    rng = _rng(seed)
    B, Hq, Hkv, L, d = 1, 4, 2, 11, 6
    q = rng.standard_normal((B, Hq, L, d))
    k = rng.standard_normal((B, Hkv, L, d))
    v = rng.standard_normal((B, Hkv, L, d))
    O, LSE = oracle.attention(q, k, v, scale=0.0)
    for h in range(Hq):
        assert np.allclose(O[0, h], np.broadcast_to(v[0, h // 2].mean(axis=0), (L, d)), atol=1e-13)
        assert np.allclose(LSE[0, h], math.log(L), atol=1e-13)
    O, LSE = oracle.attention(q, k, v, scale=0.0, causal=True)
    for h in range(Hq):
        for i in range(L):
            assert np.allclose(O[0, h, i], v[0, h // 2, :i + 1].mean(axis=0), atol=1e-13)
            assert abs(LSE[0, h, i] - math.log(i + 1)) <= 1e-13
    O, LSE = oracle.attention(q, k, v, scale=0.0, causal=True, window=4)
    for i in range(L):
        lo = max(0, i - 3)
        assert np.allclose(O[0, 0, i], v[0, 0, lo:i + 1].mean(axis=0), atol=1e-13)
        assert abs(LSE[0, 0, i] - math.log(i + 1 - lo)) <= 1e-13


def check_causal_boundary(seed=15):
    """Causal row 0 sees only key 0: O = V_0 and LSE = scale q_0.k_0.  With one key and no
    mask every row returns V_0.  With Lq > Lk (bottom-right alignment) the first Lq - Lk rows
    see nothing: O = 0 and LSE = -inf."""
    rng = _rng(seed)
    q = rng.standard_normal((1, 2, 8, 5))
    k = rng.standard_normal((1, 2, 8, 5))
    v = rng.standard_normal((1, 2, 8, 5))
    O, LSE = oracle.attention(q, k, v, scale=0.3, causal=True)
    for h in range(2):
        assert np.allclose(O[0, h, 0], v[0, h, 0], atol=1e-15)
        assert abs(LSE[0, h, 0] - 0.3 * float(q[0, h, 0] @ k[0, h, 0])) <= 1e-13
    O, LSE = oracle.attention(q, k[:, :, :1], v[:, :, :1], scale=0.3)
    assert np.allclose(O, np.broadcast_to(v[:, :, :1], O.shape), atol=1e-15)
    O, LSE = oracle.attention(q, k[:, :, :3], v[:, :, :3], scale=0.3, causal=True)
    assert np.all(O[:, :, :5] == 0.0) and np.all(np.isneginf(LSE[:, :, :5]))
    assert np.allclose(O[0, 0, 5], v[0, 0, 0], atol=1e-15)       # position 0: key 0 only
    assert np.all(np.isfinite(LSE[:, :, 5:]))


def check_window_convention(seed=16):
    """[LLM-Attn] each token attends to at most the previous W tokens, read as W keys counting
    itself: W = 1 gives O_i = V_i and LSE_i = scale q_i.k_i; W >= L equals plain causal;
    W = L - 1 differs from causal only in the last row."""
    rng = _rng(seed)
    L = 10
    q = rng.standard_normal((1, 2, L, 4))
    k = rng.standard_normal((1, 2, L, 4))
    v = rng.standard_normal((1, 2, L, 4))
    O, LSE = oracle.attention(q, k, v, scale=0.5, causal=True, window=1)
    assert np.allclose(O, v, atol=1e-15)
    assert np.allclose(LSE, 0.5 * np.einsum("bhid,bhid->bhi", q, k), atol=1e-13)
    Oc, Lc = oracle.attention(q, k, v, scale=0.5, causal=True)
    for W in (L, L + 5):
        Ow, Lw = oracle.attention(q, k, v, scale=0.5, causal=True, window=W)
        assert np.array_equal(Ow, Oc) and np.array_equal(Lw, Lc)
    Ow, Lw = oracle.attention(q, k, v, scale=0.5, causal=True, window=L - 1)
    assert np.array_equal(Ow[:, :, :L - 1], Oc[:, :, :L - 1])
    assert np.all(np.abs(Ow[:, :, L - 1] - Oc[:, :, L - 1]) > 0)


def check_gqa_mapping(seed=17):
    """Hkv = Hq is plain MHA; GQA/MQA equal MHA over K/V repeated to consecutive query heads
    ([LLM-Attn] repeat_kv; [MQA-GQA §2.1] MQA broadcasts one K/V to every head)."""
    rng = _rng(seed)
    B, Hq, L, d = 2, 8, 9, 4
    q = rng.standard_normal((B, Hq, L, d))
    for Hkv in (8, 4, 2, 1):
        k = rng.standard_normal((B, Hkv, L, d))
        v = rng.standard_normal((B, Hkv, L, d))
        g = Hq // Hkv
        for causal in (False, True):
            O, LSE = oracle.attention(q, k, v, scale=0.4, causal=causal)
            krep, vrep = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
            Om, Lm = oracle.attention(q, krep, vrep, scale=0.4, causal=causal)
            assert np.array_equal(O, Om) and np.array_equal(LSE, Lm)
            # per-head restatement: head h uses K/V head h // g, checked head by head
            for h in range(Hq):
                Oh, _ = oracle.attention(q[:, h:h + 1], k[:, h // g:h // g + 1], v[:, h // g:h // g + 1],
                                         scale=0.4, causal=causal)
                assert np.array_equal(Oh[:, 0], O[:, h])


def check_pv_invariants(seed=18):
    """O(V + 1 c^T) = O(V) + c; O(alpha V) = alpha O(V); without a mask, permuting the keys and
    values together leaves O unchanged."""
    rng = _rng(seed)
    q = rng.standard_normal((1, 2, 7, 5))
    k = rng.standard_normal((1, 2, 7, 5))
    v = rng.standard_normal((1, 2, 7, 5))
    c = rng.standard_normal(5)
    for causal, window in [(False, 0), (True, 0), (True, 3)]:
        O, _ = oracle.attention(q, k, v, scale=0.6, causal=causal, window=window)
        O2, _ = oracle.attention(q, k, v + c, scale=0.6, causal=causal, window=window)
        assert np.allclose(O2, O + c, atol=1e-13)
        O3, _ = oracle.attention(q, k, -2.5 * v, scale=0.6, causal=causal, window=window)
        assert np.allclose(O3, -2.5 * O, atol=1e-13)
    perm = rng.permutation(7)
    O, L = oracle.attention(q, k, v, scale=0.6)
    Op, Lp = oracle.attention(q, k[:, :, perm], v[:, :, perm], scale=0.6)
    assert np.allclose(O, Op, atol=1e-13) and np.allclose(L, Lp, atol=1e-13)


def check_lse_identity(seed=19):
    """sum over visible j of exp(S_ij - LSE_i) = 1 and O_i = sum_j exp(S_ij - LSE_i) V_j."""
    rng = _rng(seed)
    Lq, Lk, d = 6, 10, 3
    q = rng.standard_normal((1, 1, Lq, d))
    k = rng.standard_normal((1, 1, Lk, d))
    v = rng.standard_normal((1, 1, Lk, d))
    for causal, window in [(False, 0), (True, 0), (True, 4)]:
        O, LSE = oracle.attention(q, k, v, scale=0.8, causal=causal, window=window)
        for i in range(Lq):
            pos = i + Lk - Lq
            js = [j for j in range(Lk) if (not causal or j <= pos) and (window == 0 or pos - j < window)]
            s = [0.8 * float(q[0, 0, i] @ k[0, 0, j]) for j in js]
            w = [math.exp(x - LSE[0, 0, i]) for x in s]
            assert abs(math.fsum(w) - 1.0) <= 1e-13
            assert np.allclose(O[0, 0, i], sum(wj * v[0, 0, j] for wj, j in zip(w, js)), atol=1e-13)


def check_split_merge(seed=20):
    """Attention over disjoint key chunks, merged by their LSEs, equals attention over all
    keys (the cross-chunk form of the rescale step of [DS-Attn §二])."""
    rng = _rng(seed)
    Lq, Lk, d = 5, 23, 4
    q = rng.standard_normal((1, 2, Lq, d))
    k = rng.standard_normal((1, 2, Lk, d))
    v = rng.standard_normal((1, 2, Lk, d))
    O, LSE = oracle.attention(q, k, v, scale=0.5)
    for bounds in ([0, 8, 16, 23], [0, 1, 23], [0, 11, 12, 20, 23]):
        parts = [oracle.attention(q, k[:, :, a:b], v[:, :, a:b], scale=0.5) for a, b in zip(bounds, bounds[1:])]
        Om, Lm = oracle.merge_partials([p[0] for p in parts], [p[1] for p in parts])
        assert np.max(np.abs(Om - O)) <= 1e-12 and np.max(np.abs(Lm - LSE)) <= 1e-12
    # a chunk that sees nothing (LSE = -inf) does not change the result
    empty_o = np.zeros_like(O)
    empty_l = np.full_like(LSE, -np.inf)
    Om, Lm = oracle.merge_partials([O, empty_o], [LSE, empty_l])
    assert np.max(np.abs(Om - O)) <= 1e-15 and np.max(np.abs(Lm - LSE)) <= 1e-15
    Om, Lm = oracle.merge_partials([empty_o], [empty_l])
    assert np.all(Om == 0) and np.all(np.isneginf(Lm))


def check_decode_is_last_row(seed=21):
    """A decode query is the newest token: its result equals the last row of causal prefill
    over the same sequence, with or without a window."""
    rng = _rng(seed)
    Hq, Hkv, d = 4, 2, 6
    lens = [1, 5, 9, 13]
    N = len(lens)
    T = sum(lens) + 7
    kp = rng.standard_normal((T, Hkv, d))
    vp = rng.standard_normal((T, Hkv, d))
    offs = [2, 3 + 1, 3 + 5 + 1, 3 + 5 + 9 + 2]
    qd = rng.standard_normal((N, Hq, d))
    for W in (0, 1, 4, 100):
        O, LSE = oracle.decode(qd, kp, vp, offs, lens, scale=0.35, window=W)
        for s, (o, n) in enumerate(zip(offs, lens)):
            ks = kp[o:o + n].transpose(1, 0, 2)[None]
            vs = vp[o:o + n].transpose(1, 0, 2)[None]
            qs = np.zeros((1, Hq, n, d))
            qs[0, :, n - 1] = qd[s]
            Op, Lp = oracle.attention(qs, ks, vs, scale=0.35, causal=True, window=W)
            assert np.max(np.abs(O[s] - Op[0, :, n - 1])) <= 1e-13
            assert np.max(np.abs(LSE[s] - Lp[0, :, n - 1])) <= 1e-13


def check_pool_addressing(seed=22):
    """Sequences placed in any order, with NaN rows between them, give the same result as a
    packed pool ([DS-Attn §三.3]: sequences in one pool told apart by offset)."""
    rng = _rng(seed)
    Hq, Hkv, d = 2, 1, 3
    lens = np.array([4, 1, 6])
    kseq = [rng.standard_normal((n, Hkv, d)) for n in lens]
    vseq = [rng.standard_normal((n, Hkv, d)) for n in lens]
    qd = rng.standard_normal((3, Hq, d))
    packed_k, packed_v = np.concatenate(kseq), np.concatenate(vseq)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    O1, L1 = oracle.decode(qd, packed_k, packed_v, offs, lens, scale=0.9)
    order, gaps = [2, 0, 1], [3, 0, 5, 2]
    T = int(lens.sum()) + sum(gaps)
    pk = np.full((T, Hkv, d), np.nan)
    pv = np.full((T, Hkv, d), np.nan)
    offs2 = np.zeros(3, np.int64)
    pos = 0
    for slot, s in enumerate(order):
        pos += gaps[slot]
        offs2[s] = pos
        pk[pos:pos + lens[s]], pv[pos:pos + lens[s]] = kseq[s], vseq[s]
        pos += lens[s]
    O2, L2 = oracle.decode(qd, pk, pv, offs2, lens, scale=0.9)
    assert np.all(np.isfinite(O2)) and np.array_equal(O1, O2) and np.array_equal(L1, L2)
    # an empty sequence yields O = 0 and LSE = -inf
    O3, L3 = oracle.decode(qd, pk, pv, offs2, np.array([4, 0, 6]), scale=0.9)
    assert np.all(O3[1] == 0) and np.all(np.isneginf(L3[1]))


def paged_pool(kseq, vseq, page_size, n_pages, rng):
    """Scatter each sequence's rows over pages picked at random from a pool of n_pages (unused
    pages hold NaN).  Returns the pool and the [N, max pages] table (unused entries -1)."""
    N = len(kseq)
    Hkv, d = kseq[0].shape[1], kseq[0].shape[2]
    need = [-(-len(k) // page_size) for k in kseq]
    order = rng.permutation(n_pages)[:sum(need)]
    pk = np.full((n_pages * page_size, Hkv, d), np.nan)
    pv = np.full((n_pages * page_size, Hkv, d), np.nan)
    table = np.full((N, max(max(need), 1)), -1, np.int64)
    used = 0
    for s in range(N):
        for j in range(need[s]):
            page = int(order[used])
            used += 1
            table[s, j] = page
            lo, hi = j * page_size, min((j + 1) * page_size, len(kseq[s]))
            pk[page * page_size:page * page_size + hi - lo] = kseq[s][lo:hi]
            pv[page * page_size:page * page_size + hi - lo] = vseq[s][lo:hi]
    return pk, pv, table


def check_paged_matches_contiguous(seed=23):
    """A paged cache ([LLM-Attn], PagedAttention: the cache in small pieces that need not be
    contiguous) holds the same keys as a contiguous pool: scattering every sequence over pages
    in random order, with NaN in unused pages and unused page slots, changes nothing."""
    rng = _rng(seed)
    Hq, Hkv, d = 4, 2, 5
    lens = np.array([1, 7, 8, 13, 0, 21])
    kseq = [rng.standard_normal((n, Hkv, d)) for n in lens]
    vseq = [rng.standard_normal((n, Hkv, d)) for n in lens]
    qd = rng.standard_normal((len(lens), Hq, d))
    packed_k, packed_v = np.concatenate(kseq), np.concatenate(vseq)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    for P in (1, 3, 4, 8, 32):
        pk, pv, table = paged_pool(kseq, vseq, P, int(sum(-(-n // P) for n in lens)) + 3, rng)
        for W in (0, 1, 5):
            O1, L1 = oracle.decode(qd, packed_k, packed_v, offs, lens, scale=0.6, window=W)
            O2, L2 = oracle.decode_paged(qd, pk, pv, table, lens, P, scale=0.6, window=W)
            assert np.array_equal(O1, O2) and np.array_equal(L1, L2), (P, W)
            assert np.all(np.isfinite(O2[lens > 0]))


def check_paged_brute_force(seed=24):
    """Pure-Python walk of the page table, page by page: for page slot j of sequence s and
    offset r inside it, token j * P + r (if it exists) lives in pool row table[s][j] * P + r."""
    rng = _rng(seed)
    Hq, Hkv, d, P = 2, 1, 3, 4
    lens = [3, 9, 4]
    kseq = [rng.standard_normal((n, Hkv, d)) for n in lens]
    vseq = [rng.standard_normal((n, Hkv, d)) for n in lens]
    qd = rng.standard_normal((len(lens), Hq, d))
    pk, pv, table = paged_pool(kseq, vseq, P, 9, rng)
    for W in (0, 2):
        O, LSE = oracle.decode_paged(qd, pk, pv, table, np.array(lens), P, scale=0.8, window=W)
        for s, n in enumerate(lens):
            keys = []
            for j in range(table.shape[1]):
                for r in range(P):
                    t = j * P + r
                    if t < n and (W == 0 or t >= n - W):
                        keys.append(int(table[s, j]) * P + r)
            for h in range(Hq):
                sc = [0.8 * math.fsum(float(qd[s, h, c]) * float(pk[row, 0, c]) for c in range(d)) for row in keys]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                tot = math.fsum(w)
                for c in range(d):
                    ref = math.fsum(wi * float(pv[row, 0, c]) for wi, row in zip(w, keys)) / tot
                    assert abs(O[s, h, c] - ref) <= 1e-12, (s, h, c, W)
                assert abs(LSE[s, h] - (mx + math.log(tot))) <= 1e-12, (s, h, W)


def varlen_pool(seq_k, seq_v, rng, max_gap=4):
    """Sequences' key rows placed in a token-major pool in random order with NaN gaps."""
    n = len(seq_k)
    Hkv, d = seq_k[0].shape[1], seq_k[0].shape[2]
    gaps = rng.integers(0, max_gap + 1, size=n + 1)
    T = sum(len(k) for k in seq_k) + int(gaps.sum())
    pk = np.full((T, Hkv, d), np.nan)
    pv = np.full((T, Hkv, d), np.nan)
    offs = np.zeros(n, np.int64)
    pos = 0
    for slot, s in enumerate(rng.permutation(n)):
        pos += int(gaps[slot])
        offs[s] = pos
        pk[pos:pos + len(seq_k[s])], pv[pos:pos + len(seq_k[s])] = seq_k[s], seq_v[s]
        pos += len(seq_k[s])
    return pk, pv, offs


def check_varlen_brute_force(seed=25):
    """Ragged prefill against a pool ([Deep-Opt §二.1] continuous batching; [FlashMLA §一, §2.2]
    variable lengths): every sequence's rows equal the pure-Python triple loop on that sequence
    alone (new tokens as the last Lq_s of its Lk_s positions), with NaN between sequences."""
    rng = _rng(seed)
    Hq, Hkv, d = 4, 2, 3
    lq = [3, 1, 0, 5, 2]
    lk = [7, 1, 4, 5, 9]
    seq_k = [rng.standard_normal((n, Hkv, d)) for n in lk]
    seq_v = [rng.standard_normal((n, Hkv, d)) for n in lk]
    pk, pv, offs = varlen_pool(seq_k, seq_v, rng)
    cu = np.concatenate([[0], np.cumsum(lq)])
    q = rng.standard_normal((int(cu[-1]), Hq, d))
    for causal, W in ((True, 0), (True, 2), (False, 0)):
        O, LSE = oracle.prefill_varlen(q, pk, pv, cu, offs, lk, scale=0.45, causal=causal, window=W)
        for s in range(len(lq)):
            if lq[s] == 0:
                continue
            qs = q[cu[s]:cu[s + 1]].transpose(1, 0, 2)[None]
            ks = seq_k[s].transpose(1, 0, 2)[None]
            vs = seq_v[s].transpose(1, 0, 2)[None]
            Ob, Lb = brute_force(qs, ks, vs, 0.45, causal, W)
            o, l = O[cu[s]:cu[s + 1]].transpose(1, 0, 2)[None], LSE[cu[s]:cu[s + 1]].T[None]
            fin = np.isfinite(Lb)
            assert np.array_equal(np.isneginf(l), np.isneginf(Lb)), (s, causal, W)
            assert np.max(np.abs(o - Ob)) <= 1e-12, (s, causal, W)
            assert np.max(np.abs(l[fin] - Lb[fin]), initial=0) <= 1e-12, (s, causal, W)


def check_varlen_chunks(seed=26):
    """Chunked prefill: feeding a sequence's new tokens in two chunks (the first against the keys up
    to its end, the second against all of them) gives the same rows as one prefill of all of them,
    which holds only with bottom-right alignment and correct pool addressing."""
    rng = _rng(seed)
    Hq, Hkv, d = 2, 1, 4
    cached, new1, new2 = 6, 3, 4
    L = cached + new1 + new2
    k = rng.standard_normal((L, Hkv, d))
    v = rng.standard_normal((L, Hkv, d))
    pk, pv, offs = varlen_pool([k], [v], rng)
    q = rng.standard_normal((new1 + new2, Hq, d))
    for W in (0, 3):
        O, LSE = oracle.prefill_varlen(q, pk, pv, [0, new1 + new2], offs, [L], scale=0.7, window=W)
        O1, L1 = oracle.prefill_varlen(q[:new1], pk, pv, [0, new1], offs, [cached + new1], scale=0.7, window=W)
        O2, L2 = oracle.prefill_varlen(q[new1:], pk, pv, [0, new2], offs, [L], scale=0.7, window=W)
        assert np.max(np.abs(np.concatenate([O1, O2]) - O)) <= 1e-13, W
        assert np.max(np.abs(np.concatenate([L1, L2]) - LSE)) <= 1e-13, W
    # one new token per sequence is decode
    lens = [5, 9, 1]
    seq_k = [rng.standard_normal((n, 2, 3)) for n in lens]
    seq_v = [rng.standard_normal((n, 2, 3)) for n in lens]
    pk, pv, offs = varlen_pool(seq_k, seq_v, rng)
    qd = rng.standard_normal((3, 4, 3))
    Ov, Lv = oracle.prefill_varlen(qd, pk, pv, [0, 1, 2, 3], offs, lens, scale=0.5, window=4)
    Od, Ld = oracle.decode(qd, pk, pv, offs, lens, scale=0.5, window=4)
    assert np.max(np.abs(Ov - Od)) <= 1e-14 and np.max(np.abs(Lv - Ld)) <= 1e-14


def _vis_by_distance(Lq, Lk, causal, window):
    """Visibility spelled as distance back from the query's position (independent of the oracle)."""
    dist = (np.arange(Lq)[:, None] + (Lk - Lq)) - np.arange(Lk)[None, :]
    vis = np.ones((Lq, Lk), bool)
    if causal:
        vis &= dist >= 0
    if window:
        vis &= dist < window
    return vis


def check_backward_autograd(seed=27):
    """The backward oracle ([MQA-GQA §4]: the backward pass recomputes the forward) against torch's
    float64 autograd through the plain formula softmax(scale q k^T + mask) v, GQA by repeating K/V
    (whose gradients autograd sums back)."""
    import torch
    rng = _rng(seed)
    for (Hq, Hkv, Lq, Lk, d, causal, W) in [(4, 2, 7, 9, 5, True, 0), (2, 2, 6, 6, 3, False, 0),
                                            (4, 1, 5, 8, 4, True, 3), (3, 3, 8, 8, 2, True, 1)]:
        q = rng.standard_normal((1, Hq, Lq, d))
        k = rng.standard_normal((1, Hkv, Lk, d))
        v = rng.standard_normal((1, Hkv, Lk, d))
        do = rng.standard_normal((1, Hq, Lq, d))
        scale = 0.6
        qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        g = Hq // Hkv
        kk, vv = kt.repeat_interleave(g, dim=1), vt.repeat_interleave(g, dim=1)
        vis = torch.from_numpy(_vis_by_distance(Lq, Lk, causal, W))
        S = (scale * qt @ kk.transpose(-1, -2)).masked_fill(~vis, -math.inf)
        O = torch.softmax(S, dim=-1) @ vv
        (O * torch.from_numpy(do)).sum().backward()
        dQ, dK, dV = oracle.attention_backward(q, k, v, do, scale=scale, causal=causal, window=W)
        for got, ref, nm in ((dQ, qt.grad, "dq"), (dK, kt.grad, "dk"), (dV, vt.grad, "dv")):
            assert np.max(np.abs(got - ref.numpy())) <= 1e-12, (nm, Hq, Hkv, Lq, Lk, causal, W)


def check_backward_finite_differences(seed=28):
    """Central differences of L = sum(attention(q, k, v) * dO), taken with the forward oracle, match
    the backward oracle's gradients for every input element of a tiny causal GQA window case."""
    rng = _rng(seed)
    Hq, Hkv, Lq, Lk, d, W, scale = 2, 1, 3, 4, 2, 3, 0.9
    q = rng.standard_normal((1, Hq, Lq, d))
    k = rng.standard_normal((1, Hkv, Lk, d))
    v = rng.standard_normal((1, Hkv, Lk, d))
    do = rng.standard_normal((1, Hq, Lq, d))
    dQ, dK, dV = oracle.attention_backward(q, k, v, do, scale=scale, causal=True, window=W)
    eps = 1e-6

    def loss(q_, k_, v_):
        return float(np.sum(oracle.attention(q_, k_, v_, scale=scale, causal=True, window=W)[0] * do))

    for which, x, grad in ((0, q, dQ), (1, k, dK), (2, v, dV)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (which, idx, fd, grad[idx])


def check_backward_closed_forms(seed=29):
    """Equal value rows make the output constant in q and k: dQ = dK = 0.  Equal key rows give
    uniform rows of P whose dS sums to zero per row: dQ = 0.  Rows that see no key (Lq > Lk,
    causal) get dQ = 0 and their dO does not reach dK or dV."""
    rng = _rng(seed)
    Hq, Hkv, Lq, Lk, d = 2, 1, 5, 6, 3
    q = rng.standard_normal((1, Hq, Lq, d))
    k = rng.standard_normal((1, Hkv, Lk, d))
    v = np.repeat(rng.standard_normal((1, Hkv, 1, d)), Lk, axis=2)
    do = rng.standard_normal((1, Hq, Lq, d))
    dQ, dK, _ = oracle.attention_backward(q, k, v, do, scale=0.8, causal=True)
    assert np.max(np.abs(dQ)) <= 1e-13 and np.max(np.abs(dK)) <= 1e-13
    k_eq = np.repeat(rng.standard_normal((1, Hkv, 1, d)), Lk, axis=2)
    v2 = rng.standard_normal((1, Hkv, Lk, d))
    dQ, _, _ = oracle.attention_backward(q, k_eq, v2, do, scale=0.8)
    assert np.max(np.abs(dQ)) <= 1e-13
    Lq2, Lk2 = 6, 3                              # rows 0..2 see no key
    q2 = rng.standard_normal((1, Hq, Lq2, d))
    k2 = rng.standard_normal((1, Hkv, Lk2, d))
    v3 = rng.standard_normal((1, Hkv, Lk2, d))
    do2 = rng.standard_normal((1, Hq, Lq2, d))
    dQa, dKa, dVa = oracle.attention_backward(q2, k2, v3, do2, scale=0.8, causal=True)
    assert np.all(dQa[:, :, :3] == 0)
    do3 = do2.copy()
    do3[:, :, :3] = rng.standard_normal((1, Hq, 3, d))
    _, dKb, dVb = oracle.attention_backward(q2, k2, v3, do3, scale=0.8, causal=True)
    assert np.array_equal(dKa, dKb) and np.array_equal(dVa, dVb)


def check_fp8_decoders():
    """The FP8 decoders against the OCP 8-bit float definitions, by hand-worked codes, and against
    torch's own float8 dtypes (an independent conversion) for all 256 codes of each format."""
    import torch
    e4 = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
          0x40: 2.0, 0x78: 256.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0, 0x81: -(2.0 ** -9)}
    e5 = {0x00: 0.0, 0x01: 2.0 ** -16, 0x03: 3 * 2.0 ** -16, 0x04: 2.0 ** -14, 0x3C: 1.0, 0x3E: 1.5,
          0x7B: 57344.0, 0x7C: math.inf, 0xFC: -math.inf, 0xBC: -1.0}
    for table, f in ((e4, oracle.decode_e4m3fn), (e5, oracle.decode_e5m2)):
        for code, want in table.items():
            got = float(f(np.array([code], np.uint8))[0])
            assert got == want, (f.__name__, hex(code), got, want)
    assert math.copysign(1.0, float(oracle.decode_e4m3fn(np.array([0x80], np.uint8))[0])) == -1.0
    for code in (0x7F, 0xFF):
        assert math.isnan(float(oracle.decode_e4m3fn(np.array([code], np.uint8))[0]))
    for code in (0x7D, 0x7E, 0x7F, 0xFD):
        assert math.isnan(float(oracle.decode_e5m2(np.array([code], np.uint8))[0]))
    codes = np.arange(256, dtype=np.uint8)
    for f, dt in ((oracle.decode_e4m3fn, torch.float8_e4m3fn), (oracle.decode_e5m2, torch.float8_e5m2)):
        a = f(codes)
        b = torch.from_numpy(codes).view(dt).to(torch.float64).numpy()
        assert np.array_equal(np.isnan(a), np.isnan(b)), f.__name__
        ok = ~np.isnan(a)
        assert np.array_equal(a[ok], b[ok]), f.__name__


def check_fp8kv_decode(seed=30):
    """Decode over FP8 pools: equal to decode() over the pools that torch's float8 conversion
    dequantizes (an independent route), for both formats; v_scale scales O and leaves the LSE;
    k_scale acts as a factor on the scores."""
    import torch
    rng = _rng(seed)
    N, Hq, Hkv, d = 3, 4, 2, 8
    lens = np.array([5, 1, 9], np.int32)
    T = 20
    offsets = np.array([0, 6, 10], np.int64)
    q = rng.standard_normal((N, Hq, d))
    for fmt, dt in (("e4m3fn", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        kc = torch.from_numpy(rng.standard_normal((T, Hkv, d)) * 3).to(dt).view(torch.uint8).numpy()
        vc = torch.from_numpy(rng.standard_normal((T, Hkv, d)) * 3).to(dt).view(torch.uint8).numpy()
        ks, vs = 0.37, 1.9
        O, L = oracle.decode_fp8kv(q, kc, vc, offsets, lens, ks, vs, fmt, scale=0.5)
        kt = torch.from_numpy(kc).view(dt).to(torch.float64).numpy() * ks
        vt = torch.from_numpy(vc).view(dt).to(torch.float64).numpy() * vs
        O2, L2 = oracle.decode(q, kt, vt, offsets, lens, scale=0.5)
        assert np.allclose(O, O2, rtol=1e-13, atol=1e-13) and np.allclose(L, L2, rtol=1e-13, atol=1e-13), fmt
        O3, L3 = oracle.decode_fp8kv(q, kc, vc, offsets, lens, ks, 2 * vs, fmt, scale=0.5)
        assert np.allclose(O3, 2 * O, rtol=1e-13, atol=1e-13) and np.allclose(L3, L, rtol=1e-13, atol=1e-13)
        O4, L4 = oracle.decode_fp8kv(q, kc, vc, offsets, lens, 1.0, vs, fmt, scale=0.5 * ks)
        assert np.allclose(O4, O, rtol=1e-12, atol=1e-13) and np.allclose(L4, L, rtol=1e-12, atol=1e-13)
    # the two formats read the same codes differently
    Oe4, _ = oracle.decode_fp8kv(q, kc, vc, offsets, lens, 1.0, 1.0, "e4m3fn", scale=0.5)
    assert not np.allclose(Oe4, oracle.decode_fp8kv(q, kc, vc, offsets, lens, 1.0, 1.0, "e5m2", scale=0.5)[0])


def check_fp8_attention(seed=31):
    """Attention over FP8 Q, K, V: equal to attention() of the tensors torch's float8 conversion
    dequantizes (an independent route), for both formats; q_scale * k_scale act as one factor on
    the scores and v_scale scales O."""
    import torch
    rng = _rng(seed)
    B, Hq, Hkv, L, d = 1, 4, 2, 9, 8
    for fmt, dt in (("e4m3fn", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        codes = [torch.from_numpy(rng.standard_normal(shape) * 4).to(dt).view(torch.uint8).numpy()
                 for shape in ((B, Hq, L, d), (B, Hkv, L, d), (B, Hkv, L, d))]
        qs, ks, vs = 0.21, 0.7, 1.3
        O, L_ = oracle.attention_fp8(*codes, qs, ks, vs, fmt, scale=0.4, causal=True, window=5)
        ref = [torch.from_numpy(c).view(dt).to(torch.float64).numpy() * s_ for c, s_ in zip(codes, (qs, ks, vs))]
        O2, L2 = oracle.attention(*ref, scale=0.4, causal=True, window=5)
        assert np.allclose(O, O2, rtol=1e-13, atol=1e-13) and np.allclose(L_, L2, rtol=1e-13, atol=1e-13), fmt
        O3, L3 = oracle.attention_fp8(*codes, 1.0, qs * ks, 2 * vs, fmt, scale=0.4, causal=True, window=5)
        assert np.allclose(O3, 2 * O, rtol=1e-12, atol=1e-13) and np.allclose(L3, L_, rtol=1e-12, atol=1e-13)


def check_decode_paged_fp8kv(seed=32):
    """Paged decode over FP8 pools: the code pools scattered over pages in random order (unused
    pages and page tails hold NaN codes) give what decode() gives over contiguous pools that
    torch's float8 conversion dequantizes (an independent route), for both formats and with a
    window; v_scale scales O and leaves the LSE; k_scale acts as a factor on the scores."""
    import torch
    rng = _rng(seed)
    N, Hq, Hkv, d, P = 4, 4, 2, 8, 4
    lens = np.array([5, 1, 11, 0], np.int32)
    q = rng.standard_normal((N, Hq, d))
    for fmt, dt, nan_code in (("e4m3fn", torch.float8_e4m3fn, 0x7F), ("e5m2", torch.float8_e5m2, 0x7F)):
        kseq = [torch.from_numpy(rng.standard_normal((n, Hkv, d)) * 3).to(dt).view(torch.uint8).numpy() for n in lens]
        vseq = [torch.from_numpy(rng.standard_normal((n, Hkv, d)) * 3).to(dt).view(torch.uint8).numpy() for n in lens]
        need = [-(-int(n) // P) for n in lens]
        n_pages = sum(need) + 3
        order = rng.permutation(n_pages)
        kp = np.full((n_pages * P, Hkv, d), nan_code, np.uint8)
        vp = np.full((n_pages * P, Hkv, d), nan_code, np.uint8)
        table = np.full((N, max(need)), -1, np.int64)
        used = 0
        for s_, n in enumerate(lens):
            for j in range(need[s_]):
                page = int(order[used])
                used += 1
                table[s_, j] = page
                lo, hi = j * P, min((j + 1) * P, int(n))
                kp[page * P:page * P + hi - lo] = kseq[s_][lo:hi]
                vp[page * P:page * P + hi - lo] = vseq[s_][lo:hi]
        ks, vs = 0.29, 1.7
        kc = np.concatenate(kseq) if lens.sum() else np.zeros((0, Hkv, d), np.uint8)
        vc = np.concatenate(vseq)
        offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
        kt = torch.from_numpy(kc).view(dt).to(torch.float64).numpy() * ks
        vt = torch.from_numpy(vc).view(dt).to(torch.float64).numpy() * vs
        for W in (0, 3):
            O, L = oracle.decode_paged_fp8kv(q, kp, vp, table, lens, P, ks, vs, fmt, scale=0.5, window=W)
            O2, L2 = oracle.decode(q, kt, vt, offs, lens, scale=0.5, window=W)
            assert np.allclose(O, O2, rtol=1e-13, atol=1e-13) and np.allclose(L, L2, rtol=1e-13, atol=1e-13), (fmt, W)
            assert np.all(np.isneginf(L[lens == 0])) and np.all(O[lens == 0] == 0.0)
        O3, L3 = oracle.decode_paged_fp8kv(q, kp, vp, table, lens, P, ks, 2 * vs, fmt, scale=0.5)
        O, L = oracle.decode_paged_fp8kv(q, kp, vp, table, lens, P, ks, vs, fmt, scale=0.5)
        assert np.allclose(O3, 2 * O, rtol=1e-13, atol=1e-13) and np.allclose(L3, L, rtol=1e-13, atol=1e-13)
        O4, L4 = oracle.decode_paged_fp8kv(q, kp, vp, table, lens, P, 1.0, vs, fmt, scale=0.5 * ks)
        assert np.allclose(O4, O, rtol=1e-12, atol=1e-13) and np.allclose(L4, L, rtol=1e-12, atol=1e-13)


def check_attention_rows(seed=33):
    """attention_rows() returns, for each requested (b, h, i) in the order given (repeats allowed),
    row i of head h of batch b of the full result: against attention() on causal, windowed,
    non-causal, Lq != Lk (rows that see no key included) and GQA/MQA shapes, and against the
    pure-Python brute force on a tiny shape."""
    rng = _rng(seed)
    for (B, Hq, Hkv, Lq, Lk, d) in [(2, 4, 2, 37, 37, 16), (1, 6, 1, 20, 45, 8), (2, 2, 2, 45, 20, 8)]:
        q = rng.standard_normal((B, Hq, Lq, d))
        k = rng.standard_normal((B, Hkv, Lk, d))
        v = rng.standard_normal((B, Hkv, Lk, d))
        for causal, W in ((False, 0), (True, 0), (True, 7)):
            O, L = oracle.attention(q, k, v, scale=0.3, causal=causal, window=W)
            n = 25
            samples = list(zip(rng.integers(0, B, n).tolist(), rng.integers(0, Hq, n).tolist(),
                               rng.integers(0, Lq, n).tolist()))
            samples += [samples[3], (B - 1, Hq - 1, Lq - 1), (0, 0, 0)]
            Or, Lr = oracle.attention_rows(q, k, v, samples, scale=0.3, causal=causal, window=W)
            for m, (b, h, i) in enumerate(samples):
                assert np.max(np.abs(Or[m] - O[b, h, i])) <= 1e-13, (b, h, i, causal, W)
                if np.isneginf(L[b, h, i]):
                    assert np.isneginf(Lr[m]), (b, h, i)
                else:
                    assert abs(Lr[m] - L[b, h, i]) <= 1e-13, (b, h, i, causal, W)
    q = rng.standard_normal((1, 4, 9, 3))
    k = rng.standard_normal((1, 2, 11, 3))
    v = rng.standard_normal((1, 2, 11, 3))
    Ob, Lb = brute_force(q, k, v, 0.9, True, 4)
    samples = [(0, 3, 8), (0, 0, 2), (0, 2, 5), (0, 1, 0), (0, 3, 1)]
    Or, Lr = oracle.attention_rows(q, k, v, samples, scale=0.9, causal=True, window=4)
    for m, (b, h, i) in enumerate(samples):
        assert np.max(np.abs(Or[m] - Ob[b, h, i])) <= 1e-12 and abs(Lr[m] - Lb[b, h, i]) <= 1e-12, (h, i)


def check_useful_flops():
    """4 * d per visible pair per query head: the closed forms L*L*4d*B*Hq without a mask and
    L(L+1)/2 * 4d * B*Hq under causal masking, and the mask count otherwise."""
    assert oracle.useful_flops(2, 3, 64, 64, 16, False, 0) == 4 * 16 * 2 * 3 * 64 * 64
    assert oracle.useful_flops(1, 32, 4096, 4096, 128, True, 0) == 4 * 128 * 32 * 4096 * 4097 // 2
    assert oracle.useful_flops(1, 2, 9, 30, 8, True, 5) == 4 * 8 * 2 * int(oracle.visibility(9, 30, True, 5).sum())


def check_golden():
    """Hand-derived exact values (tests/golden/worked_example.json)."""
    g = json.load(open(GOLDEN))
    scale = math.log(2.0)
    q, k, v = (np.array(g[x], dtype=np.float64) for x in ("q", "k", "v"))
    fr = np.vectorize(lambda s: float(Fraction(s)))
    for case in g["cases"]:
        O, LSE = oracle.attention(q, k, v, scale=scale, causal=case["causal"], window=case["window"])
        assert np.max(np.abs(O - fr(np.array(case["o"])))) <= 1e-14, case
        assert np.max(np.abs(LSE - np.log(fr(np.array(case["lse_exp"]))))) <= 1e-14, case
    dec = g["decode"]
    kp = np.array([[float(x) for x in row] for row in dec["pool_k"]])[:, None, :]
    vp = np.array([[float(x) for x in row] for row in dec["pool_v"]])[:, None, :]
    qd = np.array(dec["q"], dtype=np.float64)[:, None, :]
    for case in dec["cases"]:
        O, LSE = oracle.decode(qd, kp, vp, dec["offsets"], dec["lens"], scale=scale, window=case["window"])
        assert np.max(np.abs(O[:, 0] - fr(np.array(case["o"])))) <= 1e-14, case
        assert np.max(np.abs(LSE[:, 0] - np.log(fr(np.array(case["lse_exp"]))))) <= 1e-14, case


def check_visible_pairs():
    """The pair count used for useful FLOPs equals the number of True entries of the mask,
    and the closed forms: Lq*Lk; L(L+1)/2 causal; W(W+1)/2 + (L-W)W with a window W < L."""
    for (Lq, Lk, causal, W) in [(7, 7, False, 0), (7, 7, True, 0), (9, 5, True, 0), (5, 9, True, 0),
                                (20, 20, True, 6), (20, 20, True, 25), (13, 20, True, 4)]:
        assert oracle.visible_pairs(Lq, Lk, causal, W) == int(oracle.visibility(Lq, Lk, causal, W).sum())
    assert oracle.visible_pairs(64, 64, False, 0) == 64 * 64
    assert oracle.visible_pairs(64, 64, True, 0) == 64 * 65 // 2
    assert oracle.visible_pairs(64, 64, True, 16) == 16 * 17 // 2 + (64 - 16) * 16


ALL_CHECKS = [check_golden, check_brute_force, check_torch_sdpa, check_softmax_rows, check_constant_scores,
              check_causal_boundary, check_window_convention, check_gqa_mapping, check_pv_invariants,
              check_lse_identity, check_split_merge, check_decode_is_last_row, check_pool_addressing,
              check_paged_matches_contiguous, check_paged_brute_force, check_varlen_brute_force,
              check_varlen_chunks, check_backward_autograd, check_backward_finite_differences,
              check_backward_closed_forms, check_visible_pairs, check_fp8_decoders, check_fp8kv_decode,
              check_fp8_attention, check_decode_paged_fp8kv, check_attention_rows, check_useful_flops]
