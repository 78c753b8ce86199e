"""Plain fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU package never imports
it, and it imports nothing from the GPU package; both sides share only the seeded input
generators in ``workloads.py``.

Sources (web articles on attention optimisation, cited by title and section):

  [DS-Attn]  "003-注意力机制详解：从基础Attention到DeepSeek的优化策略" (lakecityint.com):
             §一 the plain scaled dot-product and the max-subtracted ("safe") softmax;
             §二 FlashAttention's tiled online-softmax pseudo-code; §三.1 mixed precision;
             §三.2 sliding-window attention; §三.3 KV-cache pool addressed by offsets.
  [LLM-Attn] "LLM中的Attention实现及优化" (zeeklog.com): MQA and GQA with repeat_kv;
             the KV-cache size formula; sliding-window attention (each token sees at most
             the previous W tokens).
  [MQA-GQA]  tqpw.cn article on MQA → GQA → FlashAttention: §2.1 MQA shares one K/V over
             all heads; §3.1 uniform GQA grouping; §5.3 tunable sm_scale.
  [Deep-Opt] "注意力机制深度优化" (kler.cn): §一.2 causal mask, upper-right triangle skipped.
  [FlashMLA] "高效多头潜在注意力解码技术：Flash MLA深度解析" (developer.baidu.com): §3.2
             performance tuning, paged GPU memory for long sequences.

What it computes (the plain definition, [DS-Attn §一]): for every batch b and query head h,
with kh = floor(h / (Hq / Hkv)) ([LLM-Attn] repeat_kv copies each KV head to consecutive
query heads) and delta = Lk - Lq,

    S = scale * Q[b,h] K[b,kh]^T                          (Lq x Lk, fp64, materialised)
    visible(i, j) = (not causal or j <= i + delta) and (W == 0 or j > i + delta - W)
    P = softmax over the visible entries of each row (max subtracted first)
    O = P V[b,kh],   LSE_i = log(sum over visible j of exp(S_ij))   (natural log)

Readings taken where the articles are silent (each is checked by a pin in tests/):
  * causal alignment when Lq != Lk is bottom-right: query i sits at position i + Lk - Lq;
  * a window of W keeps W keys including the query's own position (p - W < j <= p);
  * masked entries are excluded (probability exactly 0), not given a large negative bias;
  * a row that sees no key gets O = 0 and LSE = -inf.

Everything is fp64.  Inputs of any float dtype are upcast exactly.  There is no tiling, no
online softmax and no reordering beyond processing query rows in blocks to bound memory.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

try:  # keep BLAS single-threaded inside the worker threads
    from threadpoolctl import threadpool_limits
except ImportError:  # pragma: no cover - optional
    threadpool_limits = None


def host_cores() -> int:
    return len(os.sched_getaffinity(0))


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def visibility(Lq: int, Lk: int, causal: bool, window: int) -> np.ndarray:
    """Boolean [Lq, Lk]: may query i attend to key j?

    Query i is at absolute position p = i + (Lk - Lq).  Causal ([Deep-Opt §一.2]) keeps
    j <= p.  A sliding window of W ([LLM-Attn] sliding window; [DS-Attn §三.2]) keeps only
    the W most recent positions, p - W < j.  W = 0 means no window."""
    p = np.arange(Lq)[:, None] + (Lk - Lq)
    j = np.arange(Lk)[None, :]
    vis = np.ones((Lq, Lk), dtype=bool)
    if causal:
        vis &= j <= p
    if window > 0:
        vis &= j > p - window
    return vis


def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * q k^T for one head ([DS-Attn §一]: Q times K transposed, divided by sqrt(d))."""
    return scale * (_f64(q) @ _f64(k).T)


def masked_softmax(S: np.ndarray, vis: np.ndarray):
    """Max-subtracted softmax over the visible entries of each row ([DS-Attn §一], safe_softmax).

    Returns (P, LSE): P is exactly 0 where invisible and its visible entries of each row sum
    to one; LSE is the natural log of the row's sum of exp(S) over visible entries.  A row
    with no visible entry gets P = 0 and LSE = -inf."""
    S = np.where(vis, S, -np.inf)
    empty = ~vis.any(axis=1)
    m = np.where(empty, 0.0, S.max(axis=1, initial=-np.inf))
    E = np.exp(S - m[:, None])          # exp(-inf) = 0 on masked entries
    l = E.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(empty[:, None], 0.0, E / np.where(empty, 1.0, l)[:, None])
        lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))
    return P, lse


def attention_head(q, k, v, scale: float, causal: bool, window: int, rows=None, block: int = 1024):
    """O [n, d] and LSE [n] for one (batch, head): q [Lq, d], k and v [Lk, d].

    ``rows`` selects query indices (default: all).  Rows are processed ``block`` at a time so
    that one head of a long sequence does not need its whole Lq x Lk score matrix at once."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Lq, Lk = q.shape[0], k.shape[0]
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), v.shape[1]))
    lse = np.empty(len(rows))
    for s in range(0, len(rows), block):
        r = rows[s:s + block]
        S = scores(q[r], k, scale)
        vis = _visibility_rows(r, Lq, Lk, causal, window)
        P, lse[s:s + block] = masked_softmax(S, vis)
        out[s:s + block] = P @ v
    return out, lse


def _visibility_rows(rows: np.ndarray, Lq: int, Lk: int, causal: bool, window: int) -> np.ndarray:
    """The rows ``rows`` of visibility(Lq, Lk, causal, window), without building all of it."""
    p = rows[:, None] + (Lk - Lq)
    j = np.arange(Lk)[None, :]
    vis = np.ones((len(rows), Lk), dtype=bool)
    if causal:
        vis &= j <= p
    if window > 0:
        vis &= j > p - window
    return vis


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """KV head serving query head h: consecutive query heads share one KV head
    ([LLM-Attn] repeat_kv; [MQA-GQA §3.1] uniform grouping, e.g. 8 heads as 2 groups of 4)."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def _pool(n_jobs: int, threads):
    n = host_cores() if threads is None else threads
    return max(1, min(n, n_jobs))


def _run(jobs, fn, threads):
    workers = _pool(len(jobs), threads)
    if workers == 1:
        return [fn(j) for j in jobs]
    if threadpool_limits is None:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, jobs))
    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, jobs))


def attention(q, k, v, scale: float | None = None, causal: bool = False, window: int = 0,
              threads: int | None = None):
    """Full attention: q [B, Hq, Lq, d], k and v [B, Hkv, Lk, d] -> O [B, Hq, Lq, d], LSE [B, Hq, Lq].

    ``scale`` defaults to 1/sqrt(d) ([DS-Attn §一]).  Work is spread over (b, h) pairs on a
    thread pool as wide as the host's cores."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if window and not causal:
        raise ValueError("a sliding window is defined only together with causal masking")
    O = np.empty((B, Hq, Lq, v.shape[3]))
    LSE = np.empty((B, Hq, Lq))

    def one(bh):
        b, h = bh
        kh = kv_head(h, Hq, Hkv)
        O[b, h], LSE[b, h] = attention_head(q[b, h], k[b, kh], v[b, kh], scale, causal, window)

    _run([(b, h) for b in range(B) for h in range(Hq)], one, threads)
    return O, LSE


def attention_rows(q, k, v, samples, scale: float | None = None, causal: bool = False, window: int = 0,
                   threads: int | None = None):
    """Selected output rows only.  ``samples`` is a sequence of (b, h, i); returns
    O [n, d] and LSE [n] in the same order.  Used where the whole output is too large for
    the oracle but single rows are cheap."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    groups: dict = {}
    for n, (b, h, i) in enumerate(samples):
        groups.setdefault((int(b), int(h)), []).append((n, int(i)))
    O = np.empty((len(samples), v.shape[3]))
    LSE = np.empty(len(samples))

    def one(key):
        b, h = key
        idx = groups[key]
        rows = np.array([i for _, i in idx])
        kh = kv_head(h, Hq, Hkv)
        o, l = attention_head(q[b, h], k[b, kh], v[b, kh], scale, causal, window, rows=rows)
        for (n, _), orow, lrow in zip(idx, o, l):
            O[n], LSE[n] = orow, lrow

    _run(list(groups), one, threads)
    return O, LSE


def decode(q, k_pool, v_pool, offsets, lens, scale: float | None = None, window: int = 0,
           threads: int | None = None, seqs=None):
    """One new token per sequence against its KV cache in a shared pool.

    q [N, Hq, d]; k_pool and v_pool [T, Hkv, d]; sequence s owns pool rows
    offsets[s] .. offsets[s] + lens[s] - 1 ([DS-Attn §三.3]: one preallocated pool, sequences
    told apart by offset).  The query is the newest token, at position lens[s] - 1, so it sees
    every cached key, or only the last W with a window.  Returns O [N, Hq, d], LSE [N, Hq]
    (or only the sequences in ``seqs``, in that order)."""
    q = np.asarray(q)
    N, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seqs = list(range(N)) if seqs is None else [int(s) for s in seqs]
    O = np.empty((len(seqs), Hq, v_pool.shape[2]))
    LSE = np.empty((len(seqs), Hq))

    def one(n_s):
        n, s = n_s
        start, n_tok = int(offsets[s]), int(lens[s])
        kseq = _f64(k_pool[start:start + n_tok])      # [n_tok, Hkv, d]
        vseq = _f64(v_pool[start:start + n_tok])
        for h in range(Hq):
            kh = kv_head(h, Hq, Hkv)
            o, l = attention_head(q[s, h][None, :], kseq[:, kh], vseq[:, kh], scale, True, window)
            O[n, h], LSE[n, h] = o[0], l[0]

    _run(list(enumerate(seqs)), one, threads)
    return O, LSE


def paged_rows(table_row, n: int, page_size: int) -> np.ndarray:
    """Pool rows of tokens 0 .. n-1 of one sequence in a paged cache: token t sits at offset
    t mod page_size of the page listed at index floor(t / page_size) of the sequence's table."""
    t = np.arange(n)
    pages = np.asarray(table_row, dtype=np.int64)[t // page_size]
    return pages * page_size + t % page_size


def decode_paged(q, k_pool, v_pool, block_table, lens, page_size: int, scale: float | None = None,
                 window: int = 0, threads: int | None = None, seqs=None):
    """decode() over a paged KV cache.

    [LLM-Attn], PagedAttention: the cache is handed out in small fixed-size pieces, so one
    sequence's keys need not be contiguous; [FlashMLA §3.2]: paged GPU memory for long
    sequences.  Reading taken for the layout the articles leave open: k_pool and v_pool are
    [pool_pages * page_size, Hkv, d], physical page p is rows p * page_size ..
    (p + 1) * page_size - 1, and block_table[s][j] names the page holding tokens
    j * page_size .. (j + 1) * page_size - 1 of sequence s.  The sequence's keys are gathered
    in token order and attended exactly as in decode(): the query is the newest token, it sees
    every key, or only the last W with a window.  Returns O [N, Hq, d], LSE [N, Hq]."""
    q = np.asarray(q)
    N, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seqs = list(range(N)) if seqs is None else [int(s) for s in seqs]
    O = np.empty((len(seqs), Hq, v_pool.shape[2]))
    LSE = np.empty((len(seqs), Hq))

    def one(n_s):
        n, s = n_s
        rows = paged_rows(block_table[s], int(lens[s]), page_size)
        kseq = _f64(k_pool[rows])      # [n_tok, Hkv, d], in token order
        vseq = _f64(v_pool[rows])
        for h in range(Hq):
            kh = kv_head(h, Hq, Hkv)
            o, l = attention_head(q[s, h][None, :], kseq[:, kh], vseq[:, kh], scale, True, window)
            O[n, h], LSE[n, h] = o[0], l[0]

    _run(list(enumerate(seqs)), one, threads)
    return O, LSE


def _seq_rows(pool, start: int, n: int) -> np.ndarray:
    """Rows start .. start + n - 1 of a token-major pool, upcast."""
    return _f64(pool[start:start + n])


def prefill_varlen(q, k_pool, v_pool, cu_seqlens_q, offsets, lens_k, scale: float | None = None,
                   causal: bool = True, window: int = 0, threads: int | None = None):
    """Prefill of new tokens of several sequences, packed end to end, against each one's keys in a
    shared pool.

    [Deep-Opt §二.1]: continuous batching puts requests of different lengths in one batch;
    [FlashMLA §一, §2.2]: variable-length sequences, processed chunk by chunk against their
    history.  q [total_q, Hq, d]: rows cu_seqlens_q[s] .. cu_seqlens_q[s+1] - 1 are the Lq_s new
    tokens of sequence s.  k_pool, v_pool [T, Hkv, d]: its Lk_s = lens_k[s] keys (the cached ones
    followed by the new tokens' own) are rows offsets[s] .. offsets[s] + Lk_s - 1 ([DS-Attn
    §三.3]).  Query i of sequence s sits at position i + Lk_s - Lq_s (bottom-right, the KV-cache
    convention), and is attended exactly as in attention().  Returns O [total_q, Hq, d] and
    LSE [total_q, Hq]."""
    q = np.asarray(q)
    total, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if window and not causal:
        raise ValueError("a sliding window is defined only together with causal masking")
    cu = [int(x) for x in cu_seqlens_q]
    O = np.zeros((total, Hq, v_pool.shape[2]))
    LSE = np.zeros((total, Hq))

    def one(s):
        a, b = cu[s], cu[s + 1]
        if b <= a:
            return
        ks = _seq_rows(k_pool, int(offsets[s]), int(lens_k[s]))
        vs = _seq_rows(v_pool, int(offsets[s]), int(lens_k[s]))
        for h in range(Hq):
            kh = kv_head(h, Hq, Hkv)
            o, l = attention_head(q[a:b, h], ks[:, kh], vs[:, kh], scale, causal, window)
            O[a:b, h], LSE[a:b, h] = o, l

    _run(list(range(len(cu) - 1)), one, threads)
    return O, LSE


def _softmax_backward(P, dP, O, dO):
    """dS = P * (dP - rowsum(dO * O)): the row-wise softmax Jacobian applied to dP (rowsum(dO * O)
    equals rowsum(P * dP), since O = P V and dP = dO V^T)."""
    D = (dO * O).sum(axis=1)
    return P * (dP - D[:, None])


def _key_grads(dS, P, q, dO, scale):
    """dK = scale * dS^T q and dV = P^T dO for one query head's rows."""
    return scale * (dS.T @ q), P.T @ dO


def attention_backward(q, k, v, dout, scale: float | None = None, causal: bool = False, window: int = 0,
                       threads: int | None = None, block: int = 512):
    """Gradients of attention() with respect to q, k and v, for an upstream gradient dout = dL/dO.

    [MQA-GQA §4]: FlashAttention's backward pass recomputes the forward results rather than
    keeping the score matrix ([DS-Attn §一]: the softmax matrix would otherwise have to be stored
    for back-propagation).  Here the plain definition is differentiated, everything materialised
    in fp64 (query rows ``block`` at a time):
        S = scale * q k^T on the visible entries, P = row softmax of S, O = P v
        dV = P^T dO,   dP = dO v^T,   dS = P * (dP - rowsum(dO * O))
        dQ = scale * dS k,   dK = scale * dS^T q
    With GQA the gradient of a KV head is the sum over the query heads sharing it ([LLM-Attn]
    repeat_kv: the copies' gradients flow back to the shared head).  Rows that see no key have
    P = 0 and contribute nothing.  Returns dQ, dK, dV shaped like q, k, v."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if window and not causal:
        raise ValueError("a sliding window is defined only together with causal masking")
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)

    def one(b_kh):
        b, kh = b_kh
        for h in range(Hq):
            if kv_head(h, Hq, Hkv) != kh:
                continue
            for s0 in range(0, Lq, block):
                r = np.arange(s0, min(s0 + block, Lq))
                S = scores(q[b, h, r], k[b, kh], scale)
                P, _ = masked_softmax(S, _visibility_rows(r, Lq, Lk, causal, window))
                O = P @ v[b, kh]
                dO = dout[b, h, r]
                dS = _softmax_backward(P, dO @ v[b, kh].T, O, dO)
                dQ[b, h, r] = scale * (dS @ k[b, kh])
                gk, gv = _key_grads(dS, P, q[b, h, r], dO, scale)
                dK[b, kh] += gk
                dV[b, kh] += gv

    _run([(b, kh) for b in range(B) for kh in range(Hkv)], one, threads)
    return dQ, dK, dV


def merge_partials(outs, lses):
    """Combine attention results taken over disjoint key subsets into the result over their
    union.  outs [C, ..., d] are the per-subset normalised outputs, lses [C, ...] their
    natural-log sums.  This is the rescale-by-exp(old max - new max) step of [DS-Attn §二]
    applied across whole subsets:
        M = max_c LSE_c,  w_c = exp(LSE_c - M),  O = sum_c w_c O_c / sum_c w_c,
        LSE = M + log(sum_c w_c).
    Subsets with LSE = -inf (no visible key) get weight 0; if all do, O = 0 and LSE = -inf."""
    outs, lses = _f64(outs), _f64(lses)
    M = lses.max(axis=0)
    none = ~np.isfinite(M) & (M < 0)
    Ms = np.where(none, 0.0, M)
    w = np.exp(lses - Ms[None])
    wsum = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        O = np.where(none[..., None], 0.0, (w[..., None] * outs).sum(axis=0) / np.where(none, 1.0, wsum)[..., None])
        LSE = np.where(none, -np.inf, Ms + np.log(np.where(none, 1.0, wsum)))
    return O, LSE


def useful_flops(B, Hq, Lq, Lk, d, causal, window) -> int:
    """4·d per visible (query, key) pair per query head: 2·d for the score, 2·d for P·V."""
    return 4 * d * B * Hq * visible_pairs(Lq, Lk, causal, window)


def visible_pairs(Lq: int, Lk: int, causal: bool, window: int) -> int:
    """Number of visible (i, j) pairs of one head, counted row by row without the matrix."""
    p = np.arange(Lq, dtype=np.int64) + (Lk - Lq)
    hi = np.minimum(p, Lk - 1) if causal else np.full(Lq, Lk - 1, np.int64)
    lo = np.maximum(p - window + 1, 0) if window > 0 else np.zeros(Lq, np.int64)
    return int(np.clip(hi - lo + 1, 0, None).sum())
