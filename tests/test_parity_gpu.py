"""HIP path vs the fp64 oracle, element by element, through the C ABI (Python binding).

Inputs are seeded N(0, 1) draws from workloads.py; the oracle sees the same bf16/fp32 values
upcast exactly to fp64.  Every named workload is compared in full (every output element and
every LSE) with the launch configuration the benchmark times, and its max abs error, relative
RMS and LSE error are printed.  Outputs are pre-filled with NaN so that any row the kernel fails
to write fails the test."""
import math

import numpy as np
import pytest
import torch

import attention_attn_fwd_03_amd as af
import oracle
import workloads as wl
from parity import check, record, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def to64(t):
    return wl.to_f64(t)


def run_fwd(q, k, v, causal, window, scale):
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device=q.device, dtype=torch.float32)
    af.attn_fwd(q, k, v, causal=causal, window=window, scale=scale, return_lse=True, out=o, lse_out=lse)
    torch.cuda.synchronize()
    return o, lse


def full_case(B, Hq, Hkv, Lq, Lk, d, causal, window, dtype, seed, scale=None):
    """Whole output against the oracle.  Scores are N(0, (scale*sqrt(d))^2); the fp32 bound
    grows with that magnitude when a test departs from scale = 1/sqrt(d)."""
    label = f"fwd B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} d{d} causal{int(causal)} W{window} {dtype} seed{seed}"
    say(label)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k, v = wl.prefill_inputs(B, Hq, Hkv, Lq, Lk, d, seed=seed, dtype=tdt, device="cpu")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o, lse = run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal, window, scale)
    O_ref, L_ref = oracle.attention(to64(q), to64(k), to64(v), scale=scale, causal=causal, window=window)
    magnitude = abs(scale) * math.sqrt(d)
    return check(to64(o), O_ref, lse.cpu().numpy(), L_ref, dtype, label, magnitude=magnitude,
                 lse_relative=magnitude > 1.0)


# ---------------------------------------------------------------------------------------------
# The named workloads.

@pytest.mark.parametrize("name", ["mha_f32_L128", "mha_f32_L128_causal", "mha_bf16_L1024"])
def test_named_workload_full(name):
    c = wl.PREFILL[name]
    record(name, full_case(c.B, c.Hq, c.Hkv, c.Lq, c.Lk, c.d, c.causal, c.window, c.dtype, c.seed))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["gqa_causal_bf16_L4096", "swa_gqa_bf16_L16384_W4096"])
def test_named_workload_full_size(name):
    """The full-size launch (the configuration the benchmark times) against the oracle over the
    whole output: every element of O and every LSE."""
    c = wl.PREFILL[name]
    say(f"fwd {name} full size on device")
    q, k, v = wl.prefill_inputs_for(c, device=DEV)
    o, lse = run_fwd(q, k, v, c.causal, c.window, c.scale)
    og, lg = to64(o), lse.cpu().numpy()
    del o, lse
    O_ref, L_ref = oracle.attention(to64(q), to64(k), to64(v), scale=c.scale, causal=c.causal, window=c.window)
    record(name, check(og, O_ref, lg, L_ref, "bf16", name))


# ---------------------------------------------------------------------------------------------
# Edge shapes.

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 127, 129, 1000, 4097])
@pytest.mark.parametrize("causal", [False, True])
def test_lengths(L, causal, dtype):
    full_case(1, 2, 1, L, L, 128, causal, 0, dtype, seed=100 + L)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Lq,Lk", [(1, 300), (65, 200), (200, 65), (300, 70), (128, 1), (5, 4097)])
@pytest.mark.parametrize("causal", [False, True])
def test_unequal_lengths(Lq, Lk, causal, d):
    """Bottom-right causal alignment; Lq > Lk leaves the first Lq - Lk rows with no key."""
    full_case(2, 4, 2, Lq, Lk, d, causal, 0, "bf16", seed=200 + Lq + Lk)


@pytest.mark.parametrize("W", [1, 2, 63, 64, 65, 299, 300, 305])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_windows(W, dtype):
    full_case(1, 4, 2, 300, 300, 128, True, W, dtype, seed=300 + W)


@pytest.mark.parametrize("W", [7, 128, 1000])
def test_windows_unequal_lengths(W):
    full_case(1, 2, 1, 333, 1200, 64, True, W, "bf16", seed=400 + W)
    full_case(1, 2, 1, 1200, 333, 64, True, W, "bf16", seed=401 + W)


@pytest.mark.parametrize("Hkv", [32, 16, 8, 4, 1])
def test_head_groups(Hkv):
    """GQA/MQA head sharing, g = Hq / Hkv from 1 to 32."""
    full_case(1, 32, Hkv, 200, 200, 128, True, 0, "bf16", seed=500 + Hkv)


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.0, 1e-3])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scales(scale, dtype):
    full_case(1, 2, 2, 150, 150, 64, True, 0, dtype, seed=600, scale=scale)
    full_case(1, 2, 2, 150, 150, 64, False, 0, dtype, seed=601, scale=scale)


@pytest.mark.parametrize("scale,d", [(-0.6144, 128), (0.6, 128), (0.9, 64)])
def test_peaked_softmax_bf16_within_rounding(scale, d):
    """Scores far from unit variance (|scale| * sqrt(d) about 7): each row's softmax is peaked and O
    approaches single rows of V, |O| up to max|V|.  Then the bf16 rounding of O (half an ulp, up to
    2^-8 |O|) and of the probabilities (up to 2^-8 of each weight) allow max-abs errors up to
    2^-7 max|V| -- beyond the 2e-2 bar, which holds for unit-variance scores, where O averages many
    rows.  The bar here is that arithmetic bound; the relative RMS bar is unchanged."""
    B, Hq, Hkv, Lq, Lk = 3, 20, 4, 508, 276
    label = f"fwd peaked B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} d{d} scale{scale}"
    say(label)
    q, k, v = wl.prefill_inputs(B, Hq, Hkv, Lq, Lk, d, seed=9018, dtype=torch.bfloat16, device="cpu")
    o, lse = run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), False, 0, scale)
    O_ref, L_ref = oracle.attention(to64(q), to64(k), to64(v), scale=scale, causal=False, window=0)
    og = to64(o)
    bound = 2.0 ** -7 * float(np.abs(to64(v)).max())
    err = float(np.abs(og - O_ref).max())
    rms = float(np.linalg.norm(og - O_ref) / np.linalg.norm(O_ref))
    say(f"  max_abs {err:.4g} (bound {bound:.4g}), rel_rms {rms:.3g}")
    assert err <= bound, (label, err, bound)
    assert rms <= 5e-3, (label, rms)
    lse_err = float(np.abs(lse.cpu().numpy().astype(np.float64) - L_ref).max())
    assert lse_err <= 1e-4 * max(1.0, float(np.abs(L_ref).max())), (label, lse_err)


@pytest.mark.parametrize("d", [64, 128])
def test_batches_and_odd_heads(d):
    full_case(3, 6, 3, 257, 257, d, True, 0, "bf16", seed=700)
    full_case(3, 6, 3, 257, 257, d, False, 0, "f32", seed=701)
    full_case(5, 3, 1, 64, 64, d, True, 17, "bf16", seed=702)


def test_without_lse_and_repeatability():
    """lse = NULL is accepted; repeated calls give bit-identical results."""
    q, k, v = wl.prefill_inputs(2, 8, 2, 700, 700, 128, seed=800, device=DEV)
    o1 = af.attn_fwd(q, k, v, causal=True)
    o2, _ = af.attn_fwd(q, k, v, causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_large_values_and_nan_propagation():
    q, k, v = wl.prefill_inputs(1, 2, 1, 130, 130, 64, seed=900, dtype=torch.float32, device="cpu")
    q = q * 30  # scores up to a few hundred: exercises the rescale path
    o, lse = run_fwd(q.to(DEV), k.to(DEV), v.to(DEV), True, 0, 0.125)
    O_ref, L_ref = oracle.attention(to64(q), to64(k), to64(v), scale=0.125, causal=True)
    check(to64(o), O_ref, lse.cpu().numpy(), L_ref, "f32", "large scores", magnitude=30.0, lse_relative=True)
    k2 = k.clone()
    k2[0, 0, 5, 3] = float("nan")
    o, _ = run_fwd(q.to(DEV), k2.to(DEV), v.to(DEV), True, 0, 0.125)
    on = o.cpu()
    assert torch.isnan(on[0, :, 5:]).any(dim=-1).all() and torch.isfinite(on[0, :, :5]).all()


# ---------------------------------------------------------------------------------------------
# Ragged (chunked) prefill against a pooled KV cache.

def run_varlen(q, kp, vp, cu, offs, lens, max_q, causal, window, scale):
    total, Hq, d = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((total, Hq), float("nan"), device=q.device, dtype=torch.float32)
    af.attn_fwd_varlen(q, kp, vp, cu, offs, lens, max_seqlen_q=max_q, causal=causal, window=window, scale=scale,
                       return_lse=True, out=o, lse_out=lse)
    torch.cuda.synchronize()
    return o, lse


def varlen_case(lq, lk, Hq, Hkv, d, causal=True, window=0, seed=0, scale=None, max_gap=37):
    lq, lk = np.asarray(lq, np.int32), np.asarray(lk, np.int32)
    label = f"varlen N{len(lq)} Hq{Hq} Hkv{Hkv} d{d} causal{causal} W{window} seed{seed} lq[:6]={lq[:6].tolist()}"
    say(label)
    q, kp, vp, cu, offs, lens, layout = wl.varlen_inputs(lq, lk, Hq, Hkv, d, seed=seed, device="cpu", max_gap=max_gap)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o, lse = run_varlen(q.to(DEV), kp.to(DEV), vp.to(DEV), cu.to(DEV), offs.to(DEV), lens.to(DEV),
                        int(max(lq.max(), 1)), causal, window, scale)
    O_ref, L_ref = oracle.prefill_varlen(q.float().numpy(), kp.float().numpy(), vp.float().numpy(), cu.numpy(),
                                         layout.offsets, layout.lens, scale=scale, causal=causal, window=window)
    return check(to64(o), O_ref, lse.cpu().numpy(), L_ref, "bf16", label)


VARLEN_LQ = [1, 17, 128, 129, 300, 0, 64, 1000, 33, 256]
VARLEN_CACHED = [0, 100, 500, 0, 4000, 10, 64, 2000, 1, 255]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 1), (True, 100), (True, 777)])
def test_varlen_chunked_prefill(causal, window, d):
    """New tokens of ten sequences (0 to 1000 each, ragged against the 128-row tiles) over caches
    of 0 to 4000 keys, NaN between the sequences in the pool."""
    lk = [a + b for a, b in zip(VARLEN_LQ, VARLEN_CACHED)]
    varlen_case(VARLEN_LQ, lk, 8, 2, d, causal=causal, window=window, seed=2200 + d + window)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 1), (12, 4)])
def test_varlen_head_groups(Hq, Hkv):
    varlen_case([70, 200, 5], [70, 600, 5], Hq, Hkv, 128, seed=2300 + Hq + Hkv)


def test_varlen_more_queries_than_keys():
    """Lq_s > Lk_s with causal masking: the first rows see no key (O = 0, LSE = -inf)."""
    varlen_case([50, 10], [20, 10], 4, 2, 128, seed=2400)


def test_varlen_matches_dense_per_sequence():
    """Every sequence of the batch gives bit for bit what attn_fwd gives on that sequence alone
    (same tiles, same arithmetic; only the addressing differs)."""
    lq = [300, 1, 129, 700]
    lk = [300, 2000, 129, 1500]
    Hq, Hkv, d = 8, 2, 128
    q, kp, vp, cu, offs, lens, layout = wl.varlen_inputs(lq, lk, Hq, Hkv, d, seed=2500, device=DEV)
    o, lse = run_varlen(q, kp, vp, cu, offs, lens, max(lq), True, 0, 0.1)
    for s, (a, n_q, n_k) in enumerate(zip(cu.tolist()[:-1], lq, lk)):
        off = int(layout.offsets[s])
        qs = q[a:a + n_q].transpose(0, 1).contiguous()[None]          # [1, Hq, Lq, d]
        ks = kp[off:off + n_k].transpose(0, 1).contiguous()[None]     # [1, Hkv, Lk, d]
        vs = vp[off:off + n_k].transpose(0, 1).contiguous()[None]
        od, ld = af.attn_fwd(qs, ks, vs, causal=True, scale=0.1, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o[a:a + n_q], od[0].transpose(0, 1)), s
        assert torch.equal(lse[a:a + n_q], ld[0].transpose(0, 1)), s


def test_varlen_invalid_sequences_report_nan():
    """A sequence whose keys fall outside the pool, whose length is negative or whose query count
    exceeds max_seqlen_q is not read; its rows are NaN and the others are unaffected."""
    lq, lk = [40, 30, 20, 60], [100, 80, 20, 60]
    q, kp, vp, cu, offs, lens, layout = wl.varlen_inputs(lq, lk, 8, 2, 128, seed=2600, device="cpu")
    T = kp.shape[0]
    bad_offs, bad_lens = offs.clone(), lens.clone()
    bad_offs[1] = T - 10          # keys run past the pool
    bad_lens[2] = -1
    o, lse = run_varlen(q.to(DEV), kp.to(DEV), vp.to(DEV), cu.to(DEV), bad_offs.to(DEV), bad_lens.to(DEV), 50,
                        True, 0, 0.1)      # max_seqlen_q = 50 < 60: sequence 3 is rejected too
    o, lse = o.cpu().float(), lse.cpu()
    c = cu.tolist()
    assert torch.isnan(o[c[1]:]).all() and torch.isnan(lse[c[1]:]).all()
    O_ref, L_ref = oracle.prefill_varlen(q[:c[1]].float().numpy(), kp.float().numpy(), vp.float().numpy(),
                                         [0, c[1]], layout.offsets[:1], layout.lens[:1], scale=0.1)
    check(o[:c[1]].double().numpy(), O_ref, lse[:c[1]].numpy(), L_ref, "bf16", "valid neighbour")


def test_named_varlen_chunked_prefill():
    """The chunked-prefill batch at full size (16 sequences, 512-2048 new tokens over 0-14k cached
    keys, Hq 32 / Hkv 8, d 128): all outputs finite, every sequence bit-identical to attn_fwd on it
    alone, and sampled rows of three sequences against the oracle."""
    c = wl.VARLEN["chunked_prefill_bf16"]
    lq, lk = c.lengths()
    say(f"varlen {c.name} full size on device: lq {lq.tolist()}")
    q, kp, vp, cu, offs, lens, layout = wl.varlen_inputs(lq, lk, c.Hq, c.Hkv, c.d, seed=c.seed, device=DEV)
    o, lse = run_varlen(q, kp, vp, cu, offs, lens, int(lq.max()), c.causal, c.window, c.scale)
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    rng = np.random.default_rng(c.seed)
    cl = cu.tolist()
    for s in range(c.n_seq):
        off, n_q, n_k = int(layout.offsets[s]), int(lq[s]), int(lk[s])
        qs = q[cl[s]:cl[s] + n_q].transpose(0, 1).contiguous()[None]
        ks = kp[off:off + n_k].transpose(0, 1).contiguous()[None]
        vs = vp[off:off + n_k].transpose(0, 1).contiguous()[None]
        od, ld = af.attn_fwd(qs, ks, vs, causal=c.causal, window=c.window, scale=c.scale, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o[cl[s]:cl[s] + n_q], od[0].transpose(0, 1)), s
        if s in (0, int(np.argmax(lk)), int(np.argmin(lq))):
            rows = sorted(set(rng.integers(0, n_q, 6).tolist()) | {0, n_q - 1})
            samples = [(0, h, i) for h in (0, 5, c.Hq - 1) for i in rows]
            O_ref, L_ref = oracle.attention_rows(qs.cpu().float().numpy(), ks.cpu().float().numpy(),
                                                 vs.cpu().float().numpy(), samples, scale=c.scale, causal=c.causal,
                                                 window=c.window)
            got_o = np.stack([to64(o[cl[s] + i, h]) for (_, h, i) in samples])
            got_l = np.array([float(lse[cl[s] + i, h]) for (_, h, i) in samples])
            check(got_o, O_ref, got_l, L_ref, "bf16", f"{c.name} seq {s}")


# ---------------------------------------------------------------------------------------------
# Decode over a pooled KV cache.

def gather_pool(kp, vp, offsets, lens, seqs):
    """Copy the rows of the chosen sequences into packed fp32 host arrays for the oracle."""
    ks, vs, offs, ls, pos = [], [], [], [], 0
    for s in seqs:
        a, n = int(offsets[s]), int(lens[s])
        ks.append(kp[a:a + n].cpu().float().numpy())
        vs.append(vp[a:a + n].cpu().float().numpy())
        offs.append(pos)
        ls.append(n)
        pos += n
    return np.concatenate(ks), np.concatenate(vs), np.array(offs, np.int64), np.array(ls, np.int32)


def oracle_decode(q, kp, vp, offsets, lens, seqs, scale, window=0):
    kg, vg, offs, ls = gather_pool(kp, vp, offsets, lens, seqs)
    qs = q.cpu().float().numpy()[seqs]
    return oracle.decode(qs, kg, vg, offs, ls, scale=scale, window=window)


def run_decode(q, kp, vp, offs, lens, max_len, window, scale):
    N, Hq, d = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((N, Hq), float("nan"), device=q.device, dtype=torch.float32)
    af.attn_decode(q, kp, vp, offs, lens, max_len=max_len, window=window, scale=scale, return_lse=True, out=o,
                   lse_out=lse)
    torch.cuda.synchronize()
    return o, lse


def decode_case(lens, Hq, Hkv, d, window=0, seed=0, scale=None, max_len=None, device_gen=False, seqs=None,
                max_gap=37):
    lens = np.asarray(lens, np.int32)
    label = f"decode N{len(lens)} Hq{Hq} Hkv{Hkv} d{d} W{window} seed{seed} lens[:8]={lens[:8].tolist()}"
    say(label)
    dev = DEV if device_gen else "cpu"
    q, kp, vp, offs, lens_t, layout = wl.decode_inputs(len(lens), Hq, Hkv, d, lens, seed=seed, device=dev,
                                                       max_gap=max_gap)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    max_len = int(lens.max()) if max_len is None else max_len
    o, lse = run_decode(q.to(DEV), kp.to(DEV), vp.to(DEV), offs.to(DEV), lens_t.to(DEV), max_len, window, scale)
    seqs = list(range(len(lens))) if seqs is None else seqs
    O_ref, L_ref = oracle_decode(q, kp, vp, layout.offsets, layout.lens, seqs, scale, window)
    return check(to64(o)[seqs], O_ref, lse.cpu().numpy()[seqs], L_ref, "bf16", label)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["gqa_decode_bf16", "mqa_decode_bf16"])
def test_named_decode(name):
    """Full-size decode batch (64 sequences, lengths 1k..32k, NaN-poisoned gaps in the pool)
    against the oracle: every sequence, every query head, every element."""
    c = wl.DECODE[name]
    lens = wl.decode_lens(c.n_seq, c.len_lo, c.len_hi, c.lens_seed)
    say(f"decode {name} full size on device")
    q, kp, vp, offs, lens_t, layout = wl.decode_inputs(c.n_seq, c.Hq, c.Hkv, c.d, lens, seed=c.value_seed,
                                                       device=DEV, max_gap=c.max_gap)
    o, lse = run_decode(q, kp, vp, offs, lens_t, int(lens.max()), 0, c.scale)
    seqs = list(range(c.n_seq))
    O_ref, L_ref = oracle_decode(q, kp, vp, layout.offsets, layout.lens, seqs, c.scale)
    record(name, check(to64(o), O_ref, lse.cpu().numpy(), L_ref, "bf16", name))


def edge_lens(n_seq, share_blocks):
    """Lengths that put team boundaries at, just before and just after sequence boundaries and
    inside the last partial block, mixed with empty and one-token sequences."""
    base = [1, 31, 32, 33, 0, 64, 5, 100]
    lens = []
    for i in range(n_seq):
        if i % 3 == 0:
            lens.append(share_blocks * 32 - (i % 5))  # a share's worth of keys, give or take a few
        else:
            lens.append(base[i % len(base)])
    return lens


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hkv", [8, 2, 1])
def test_decode_split_edges(Hkv, d):
    """Lengths chosen against the actual split: the batch holds about `teams` shares, so pieces
    start and end on every kind of boundary, including single-block pieces."""
    Hq = 8
    teams, rows, tpb = af.decode_plan(40, Hq, Hkv, d)
    lens = edge_lens(40, 3)
    total = sum(-(-n // tpb) for n in lens)
    # scale the long sequences so that the total is a few blocks per team
    target = 3 * teams
    k = max(1, target // max(total, 1))
    lens = [n * k if n > 100 else n for n in lens]
    say(f"split edges: teams {teams} rows {rows} tpb {tpb} total blocks {sum(-(-n // tpb) for n in lens)}")
    decode_case(lens, Hq, Hkv, d, seed=1000 + Hkv + d)


def test_decode_one_long_sequence_over_all_teams():
    """One sequence long enough that every team takes a share of it, next to tiny ones."""
    teams, _, tpb = af.decode_plan(3, 8, 2, 128)
    lens = [5, teams * tpb * 2 + 17, 1]
    decode_case(lens, 8, 2, 128, seed=1050)


def test_decode_more_teams_than_blocks():
    """Fewer blocks than teams: most teams get no work; every block is still computed."""
    decode_case([1, 40, 3], 8, 8, 128, seed=1060)


@pytest.mark.parametrize("W", [1, 31, 100, 600, 5000])
def test_decode_window(W):
    lens = [1, 50, 1031, 3 * 1024 + 1, 2000]
    decode_case(lens, 8, 2, 128, window=W, seed=1100 + W)


@pytest.mark.parametrize("Hq,Hkv", [(64, 1), (48, 1), (40, 8), (4, 4)])
def test_decode_head_blocks(Hq, Hkv):
    """More than 32 query heads per KV head take several head blocks."""
    decode_case([700, 33, 1500], Hq, Hkv, 128, seed=1200 + Hq)


@pytest.mark.parametrize("scale", [0.0, -0.2, 1.5])
def test_decode_scales(scale):
    decode_case([100, 1000, 7], 8, 2, 128, scale=scale, seed=1300)


def test_decode_max_len_larger_than_needed():
    decode_case([100, 200], 4, 1, 128, max_len=5000, seed=1400)


def test_decode_invalid_sequences_report_nan():
    """A sequence whose rows fall outside the pool (or whose length exceeds max_len, or is
    negative) is not read; its outputs are NaN while the other sequences are unaffected."""
    lens = np.array([40, 60, 80, 30], np.int32)
    q, kp, vp, offs, lens_t, layout = wl.decode_inputs(4, 8, 2, 128, lens, seed=1500, device="cpu")
    T = kp.shape[0]
    bad_offs = offs.clone()
    bad_offs[1] = T - 10            # runs past the end of the pool
    bad_lens = lens_t.clone()
    bad_lens[2] = 100               # longer than max_len = 90
    bad_lens[3] = -1
    o, lse = run_decode(q.to(DEV), kp.to(DEV), vp.to(DEV), bad_offs.to(DEV), bad_lens.to(DEV), 90, 0, 0.1)
    o, lse = o.cpu().float(), lse.cpu()
    assert torch.isnan(o[1:]).all() and torch.isnan(lse[1:]).all()
    O_ref, L_ref = oracle_decode(q, kp, vp, layout.offsets, layout.lens, [0], 0.1)
    check(o[:1].double().numpy(), O_ref, lse[:1].numpy(), L_ref, "bf16", "valid neighbour")


# ---------------------------------------------------------------------------------------------
# Decode over a paged KV cache.

def run_decode_paged(q, kp, vp, table, lens, page_size, max_len, window, scale):
    N, Hq, d = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((N, Hq), float("nan"), device=q.device, dtype=torch.float32)
    af.attn_decode_paged(q, kp, vp, table, lens, page_size=page_size, max_len=max_len, window=window, scale=scale,
                         return_lse=True, out=o, lse_out=lse)
    torch.cuda.synchronize()
    return o, lse


def oracle_decode_paged(q, kp, vp, table, lens, page_size, seqs, scale, window=0):
    """The paged oracle on a compact pool holding only the pages of the chosen sequences (each
    page copied once, the table renumbered)."""
    table, lens = np.asarray(table), np.asarray(lens)
    used = sorted({int(table[s, j]) for s in seqs for j in range(-(-int(lens[s]) // page_size))})
    new = {p: i for i, p in enumerate(used)}
    rows = torch.tensor([p * page_size + r for p in used for r in range(page_size)], dtype=torch.int64)
    kc = kp.index_select(0, rows.to(kp.device)).cpu().float().numpy()
    vc = vp.index_select(0, rows.to(vp.device)).cpu().float().numpy()
    sub = np.full((len(seqs), table.shape[1]), -1, np.int64)
    for i, s in enumerate(seqs):
        for j in range(-(-int(lens[s]) // page_size)):
            sub[i, j] = new[int(table[s, j])]
    qs = q.cpu().float().numpy()[seqs]
    return oracle.decode_paged(qs, kc, vc, sub, lens[seqs], page_size, scale=scale, window=window)


def decode_paged_case(lens, Hq, Hkv, d, page_size, window=0, seed=0, scale=None, extra_pages=5, table_fn=None,
                      seqs=None):
    lens = np.asarray(lens, np.int32)
    label = f"paged decode N{len(lens)} Hq{Hq} Hkv{Hkv} d{d} P{page_size} W{window} seed{seed} lens[:8]={lens[:8].tolist()}"
    say(label)
    q, kp, vp, table, lens_t, layout = wl.paged_decode_inputs(len(lens), Hq, Hkv, d, lens, page_size, seed=seed,
                                                              device="cpu", extra_pages=extra_pages)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    ktab = table.clone() if table_fn is None else table_fn(table.clone(), layout)
    o, lse = run_decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), ktab.to(DEV), lens_t.to(DEV), page_size,
                              int(max(lens.max(), 1)), window, scale)
    seqs = list(range(len(lens))) if seqs is None else seqs
    O_ref, L_ref = oracle_decode_paged(q, kp, vp, layout.table, layout.lens, page_size, seqs, scale, window)
    return check(to64(o)[seqs], O_ref, lse.cpu().numpy()[seqs], L_ref, "bf16", label)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["gqa_decode_bf16", "mqa_decode_bf16"])
def test_named_decode_paged(name):
    """The full decode batch with its cache in 64-token pages scattered over the pool (unused
    pages and page tails NaN): every sequence against the oracle, and the result bit-identical
    to the contiguous entry point on the same keys (same split, same arithmetic)."""
    c = wl.DECODE[name]
    P = 64
    lens = wl.decode_lens(c.n_seq, c.len_lo, c.len_hi, c.lens_seed)
    say(f"paged decode {name} full size on device, P{P}")
    q, kp, vp, table, lens_t, layout = wl.paged_decode_inputs(c.n_seq, c.Hq, c.Hkv, c.d, lens, P, seed=c.value_seed,
                                                              device=DEV, extra_pages=97)
    o, lse = run_decode_paged(q, kp, vp, table, lens_t, P, int(lens.max()), 0, c.scale)
    seqs = list(range(c.n_seq))
    O_ref, L_ref = oracle_decode_paged(q, kp, vp, layout.table, layout.lens, P, seqs, c.scale)
    record(name + "_paged_P64", check(to64(o)[seqs], O_ref, lse.cpu().numpy()[seqs], L_ref, "bf16", name + " paged"))
    # the same keys laid out contiguously, through attn_decode
    rows = np.concatenate([(layout.table[s, :-(-int(n) // P)].astype(np.int64)[:, None] * P
                            + np.arange(P)[None, :]).ravel()[:int(n)] for s, n in enumerate(lens)])
    rows = torch.from_numpy(rows).to(DEV)
    kc, vc = kp.index_select(0, rows), vp.index_select(0, rows)
    offs = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)).to(DEV)
    o2, lse2 = run_decode(q, kc, vc, offs, lens_t, int(lens.max()), 0, c.scale)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hkv", [8, 2, 1])
def test_decode_paged_page_sizes(Hkv, d):
    """Page sizes from one block up to 256 tokens, lengths on both sides of block and page
    boundaries, against the split's real share size."""
    Hq = 8
    teams, rows, tpb = af.decode_plan(24, Hq, Hkv, d)
    lens = [0, 1, tpb - 1, tpb, tpb + 1, 63, 64, 65, 255, 256, 257, 1000, 3 * teams * tpb + 11, 7, 2, 500,
            129, 130, 31, 33, 4096, 17, 900, 1]
    for P in sorted({tpb, 2 * tpb, max(64, tpb), 256}):
        decode_paged_case(lens, Hq, Hkv, d, P, seed=1800 + P + Hkv + d)


@pytest.mark.parametrize("W,Hkv", [(1, 2), (31, 2), (100, 2), (600, 2), (5000, 2), (700, 1), (45, 8)])
def test_decode_paged_window(W, Hkv):
    """Under a window the first block starts at the page boundary below the first visible key
    (masked up to it); table entries of pages wholly before the window are set to -1 for the
    kernel, which must not read them."""
    P = 32

    def drop_early_pages(table, layout):
        for s, n in enumerate(layout.lens):
            lo = max(int(n) - W, 0)
            table[s, :lo // P] = -1
        return table

    decode_paged_case([1, 50, 1031, 3 * 1024 + 1, 2000, 33, 64], 8, Hkv, 128, P, window=W, seed=1900 + W + Hkv,
                      table_fn=drop_early_pages)


def test_decode_paged_shared_pages():
    """Pages shared between sequences (a common prefix held once) and pages listed out of order."""
    P = 32
    lens = np.array([300, 500, 64, 200], np.int32)

    def share_prefix(table, layout):
        table[1, :4] = table[0, :4]      # sequence 1 starts with sequence 0's first 128 tokens
        table[3, :3] = table[3, :3].flip(0)
        return table

    say("paged decode shared pages")
    q, kp, vp, table, lens_t, layout = wl.paged_decode_inputs(4, 8, 2, 128, lens, P, seed=2000, device="cpu")
    ktab = share_prefix(table.clone(), layout)
    o, lse = run_decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), ktab.to(DEV), lens_t.to(DEV), P, 500, 0, 0.1)
    O_ref, L_ref = oracle_decode_paged(q, kp, vp, ktab.numpy(), layout.lens, P, [0, 1, 2, 3], 0.1)
    check(to64(o), O_ref, lse.cpu().numpy(), L_ref, "bf16", "shared pages")


def test_decode_paged_bad_entries_report_nan():
    """A sequence whose visible keys lie on a page entry outside [0, pool_pages) reads nothing from
    it and reports NaN; so do lengths past max_len or negative; other sequences are unaffected."""
    P = 32
    lens = np.array([100, 90, 70, 60, 80], np.int32)
    q, kp, vp, table, lens_t, layout = wl.paged_decode_inputs(5, 8, 2, 128, lens, P, seed=2100, device="cpu")
    bad = table.clone()
    bad[1, 2] = layout.pool_pages          # one past the last page
    bad[2, 0] = -5
    bad_lens = lens_t.clone()
    bad_lens[3] = 101                      # longer than max_len = 100
    bad_lens[4] = -1
    o, lse = run_decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), bad.to(DEV), bad_lens.to(DEV), P, 100, 0, 0.1)
    o, lse = o.cpu().float(), lse.cpu()
    assert torch.isnan(o[1:]).all() and torch.isnan(lse[1:]).all()
    O_ref, L_ref = oracle_decode_paged(q, kp, vp, layout.table, layout.lens, P, [0], 0.1)
    check(o[:1].double().numpy(), O_ref, lse[:1].numpy(), L_ref, "bf16", "valid neighbour")


def test_decode_matches_prefill_last_row():
    """Decode of a sequence equals the last row of causal prefill over it (GPU vs GPU, both
    checked against the oracle elsewhere)."""
    L, Hq, Hkv, d = 777, 8, 2, 128
    q, k, v = wl.prefill_inputs(1, Hq, Hkv, L, L, d, seed=1600, device=DEV)
    o_pref = af.attn_fwd(q, k, v, causal=True)
    kp = k[0].transpose(0, 1).contiguous()  # [L, Hkv, d]
    vp = v[0].transpose(0, 1).contiguous()
    qd = q[0, :, L - 1].contiguous()[None]
    offs = torch.zeros(1, dtype=torch.int64, device=DEV)
    lens = torch.full((1,), L, dtype=torch.int32, device=DEV)
    o_dec = af.attn_decode(qd, kp, vp, offs, lens, max_len=L)
    torch.cuda.synchronize()
    diff = (o_dec[0].float() - o_pref[0, :, L - 1].float()).abs().max().item()
    assert diff <= 2e-2


@pytest.mark.parametrize("Lk", [65, 129, 1000, 4097])
@pytest.mark.parametrize("d", [64, 128])
def test_reads_stay_inside_k_and_v(Lk, d):
    """K and V sit directly in front of NaN-filled memory; a kernel reading rows past Lk (for
    the last head, whose rows end the tensor) would turn O into NaN through 0 * NaN."""
    B, Hq, Hkv, Lq = 1, 4, 2, 77
    say(f"tail reads Lk{Lk} d{d}")
    q, k, v = wl.prefill_inputs(B, Hq, Hkv, Lq, Lk, d, seed=1700 + Lk, device="cpu")

    def fenced(t):
        store = torch.full((t.numel() + 128 * d,), float("nan"), dtype=t.dtype, device=DEV)
        view = store[: t.numel()].view(t.shape)
        view.copy_(t.to(DEV))
        return view

    kk, vv = fenced(k), fenced(v)
    for causal in (False, True):
        o, lse = run_fwd(q.to(DEV), kk, vv, causal, 0, 1.0 / math.sqrt(d))
        O_ref, L_ref = oracle.attention(to64(q), to64(k), to64(v), scale=1.0 / math.sqrt(d), causal=causal)
        check(to64(o), O_ref, lse.cpu().numpy(), L_ref, "bf16", f"fenced Lk{Lk} d{d} causal{causal}")
