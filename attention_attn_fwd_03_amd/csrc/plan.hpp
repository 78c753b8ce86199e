// Tile scheduler: which query tile a workgroup owns, which K/V tiles it must visit, and which
// of those need a mask.  Host and device share these functions, so the host planner, the
// CPU tests (through attn_fwd_plan / attn_fwd_schedule) and the kernels agree by construction.
//
// Visibility follows the plain definition: query row i sits at absolute position
// p = i + (Lk - Lq) (bottom-right alignment); causal keeps keys j <= p ("注意力机制深度优化",
// §一.2, skip the upper-right triangle); a window of W keeps j > p - W, the W most recent
// positions ("LLM中的Attention实现及优化", sliding-window section).  Tiles that hold no visible
// pair for any row of the workgroup are never visited; only tiles that mix visible and
// invisible pairs are masked ("003-注意力机制详解…", §三.2: compute the band, do not build the
// full matrix and mask it).
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define ATTN_HD __host__ __device__ __forceinline__
#else
#define ATTN_HD inline
#endif

namespace attnfwd {

struct KeyRange {
  int kt_lo, kt_hi;  // inclusive K-tile range; empty when kt_lo > kt_hi
  int k_begin, k_end;  // visible key span [k_begin, k_end) of the union of the tile's rows
};

// K tiles touched by query rows [q_start, q_start + bq) ∩ [0, Lq).
ATTN_HD KeyRange key_range(int q_start, int bq, int Lq, int Lk, int bk, int causal, int window) {
  const int delta = Lk - Lq;
  const int q_last = (q_start + bq < Lq ? q_start + bq : Lq) - 1;
  int k_end = Lk;
  if (causal) {
    const int hi = q_last + delta + 1;
    k_end = hi < k_end ? hi : k_end;
  }
  int k_begin = 0;
  if (window > 0) {
    const int lo = q_start + delta - window + 1;
    k_begin = lo > 0 ? lo : 0;
  }
  KeyRange r;
  r.k_begin = k_begin;
  r.k_end = k_end;
  if (k_end <= k_begin) {
    r.kt_lo = 0;
    r.kt_hi = -1;
  } else {
    r.kt_lo = k_begin / bk;
    r.kt_hi = (k_end - 1) / bk;
  }
  return r;
}

// True when every (row, key) pair of the tile [k0, k0 + bk) is visible for all rows
// [q_start, q_last], so the kernel can skip masking it.
ATTN_HD bool tile_full(int k0, int q_start, int bq, int Lq, int Lk, int bk, int causal, int window) {
  const int delta = Lk - Lq;
  const int q_last = (q_start + bq < Lq ? q_start + bq : Lq) - 1;
  if (k0 + bk > Lk) return false;
  if (causal && k0 + bk - 1 > q_start + delta) return false;
  if (window > 0 && k0 <= q_last + delta - window) return false;
  return true;
}

// Keys a query row sees, relative to kbase = k0 + 4*(lane/32) (the first key of the lane's rows in
// an S^T accumulator block): key kbase + ci is visible iff lo <= ci <= hi.  Query q sits at
// position q + Lk - Lq (bottom-right), sees keys up to it under causal masking, the last `window`
// positions under a window, and nothing past Lk - 1.
ATTN_HD void edge_key_limits(int k0, int h, int q, int Lq, int Lk, int causal, int window, int& lo, int& hi) {
  const int pos = q + (Lk - Lq);
  int hk = Lk - 1;
  if (causal && pos < hk) hk = pos;
  int lk = 0;
  if (window > 0 && pos - window + 1 > lk) lk = pos - window + 1;
  const int kbase = k0 + 4 * h;
  lo = lk - kbase;
  hi = hk - kbase;
}

// Per-pair visibility, used inside masked tiles.
ATTN_HD bool visible(int key, int q, int Lq, int Lk, int causal, int window) {
  const int p = q + (Lk - Lq);
  return key < Lk && key >= 0 && (!causal || key <= p) && (window <= 0 || key > p - window);
}

struct PrefillTile {
  int b, hq, hkv, qt;
};

// Block index -> (batch, query head, KV head, query tile).
//  * Workgroups are dispatched to the chip's 8 XCDs round-robin by block index and each XCD has
//    its own L2.  When B*Hq is a multiple of 8, block bid goes to band bid % 8 of B*Hq/8
//    consecutive heads, so the query heads that share a KV head (consecutive heads) read it
//    from the same L2.
//  * Causal tiles are handed out heaviest first (the last query tile sees the most keys), which
//    evens out the tail of the launch.
ATTN_HD PrefillTile prefill_tile(int bid, int B, int Hq, int group, int n_qt, int causal, int heads_per_xcd) {
  const int bh_total = B * Hq;
  int qt_rank, bh;
  if (heads_per_xcd > 0) {
    const int xcd = bid & 7, slot = bid >> 3;
    qt_rank = slot / heads_per_xcd;
    bh = xcd * heads_per_xcd + slot % heads_per_xcd;
  } else {
    qt_rank = bid / bh_total;
    bh = bid % bh_total;
  }
  PrefillTile t;
  t.qt = causal ? n_qt - 1 - qt_rank : qt_rank;
  t.b = bh / Hq;
  t.hq = bh % Hq;
  t.hkv = t.hq / group;
  return t;
}

ATTN_HD int prefill_heads_per_xcd(int B, int Hq) { return (B * Hq) % 8 == 0 ? (B * Hq) / 8 : 0; }

// Block index -> work item for ragged batches, whose sequences' keys (a cached prefix of up to
// tens of thousands of rows) outgrow one XCD's L2.  All workgroups of one (sequence, KV head) --
// its g query heads times its query tiles -- go to the same XCD (bid % 8) in consecutive slots,
// so they stream the same keys together through that L2; groups g = b * Hkv + hkv are dealt to
// the XCDs round-robin (with Hkv a multiple of 8 every XCD gets one KV head of every sequence,
// hence equal work), and inside a group query tiles come heaviest first.  With fewer than 32
// groups each is cut into `parts` contiguous pieces dealt out the same way, so that every XCD
// has work.  The launch holds prefill_grouped_blocks(...) blocks; b >= B marks a block without
// work.
struct GroupedOrder {
  int g_heads, items, parts, part_size, per_xcd;
};
ATTN_HD GroupedOrder prefill_grouped_order(int B, int Hq, int Hkv, int n_qt) {
  GroupedOrder o;
  o.g_heads = Hq / Hkv;
  o.items = o.g_heads * n_qt;
  const int groups = B * Hkv;
  int parts = groups >= 32 ? 1 : (32 + groups - 1) / groups;
  if (parts > o.items) parts = o.items;
  o.parts = parts;
  o.part_size = (o.items + parts - 1) / parts;
  o.per_xcd = (groups * parts + 7) / 8;
  return o;
}
ATTN_HD int prefill_grouped_blocks(int B, int Hq, int Hkv, int n_qt) {
  const GroupedOrder o = prefill_grouped_order(B, Hq, Hkv, n_qt);
  return 8 * o.per_xcd * o.part_size;
}
ATTN_HD PrefillTile prefill_tile_grouped(int bid, int B, int Hq, int Hkv, int n_qt) {
  const GroupedOrder o = prefill_grouped_order(B, Hq, Hkv, n_qt);
  const int xcd = bid & 7, slot = bid >> 3;
  const int piece = xcd + 8 * (slot / o.part_size);  // (group, part)
  const int g = piece / o.parts;
  const int within = (piece % o.parts) * o.part_size + slot % o.part_size;
  PrefillTile t;
  t.b = within < o.items ? g / Hkv : B;  // >= B: no work
  t.hkv = g % Hkv;
  t.qt = n_qt - 1 - within / o.g_heads;
  t.hq = t.hkv * o.g_heads + within % o.g_heads;
  return t;
}

// Decode work decomposition.  A block is 32 K (and V) rows, the M dimension of one MFMA tile.
//  * Packed layout (Hq <= 32 and Hkv divides 32): a block holds P = Hkv heads of 32 / Hkv
//    consecutive tokens, i.e. 32 consecutive pool rows, and a worker serves every query head of
//    the sequence; a row of the block only meets the query heads of its own group (the others
//    are masked).  Each block is one contiguous stretch of the pool, whatever Hkv is.
//  * Row layout (otherwise): a block holds 32 consecutive tokens of one KV head (P = 1), and a
//    worker serves one "row" (a KV head and up to 32 of its query heads); U = Hkv * head_blocks
//    rows per sequence.
// The launch holds `teams` teams of U single-wave workers.  The blocks of all sequences,
// concatenated in sequence order, are cut into `teams` equal shares of q = ceil(T / teams)
// blocks (T = blocks of one row per sequence, summed); team t takes share t and its member u
// runs row u over every sequence the share touches.  A (team, sequence) pair produces at most
// one partial per row, stored in slot (t + s) * U + u: consecutive sequences' team ranges overlap
// in at most one team, so slots never collide and at most U * (teams + n_seq) exist.
constexpr int kDecodeBlockRows = 32;
constexpr int kDecodeMaxWorkers = 2048;  // workers per launch, at most (one resident round)
// Workers per CU, at most.  Packed layout (GQA): three single-wave workers per CU stream the pool
// about 2% faster than four and 3% faster than two (d = 128; counts that are not a multiple of the
// CU count load the CUs unevenly and are slower still).  One-head layout (MQA, large groups): two
// per CU, about 1% faster than three on the MQA batch (fewer partials to write and merge, the
// stream no slower).
constexpr int kDecodeWorkersPerCu = 3;
constexpr int kDecodeWorkersPerCuOneHead = 2;
// An FP8 pool halves the bytes per block while the per-block work grows (the codes are converted
// to bf16 in registers): four workers per CU, one per SIMD, are about 9% faster than three on the
// GQA batch (equal on MQA).
constexpr int kDecodeWorkersPerCuFp8 = 4;

ATTN_HD int decode_head_blocks(int group) { return (group + 31) / 32; }
// KV heads per block: Hkv in the packed layout, 1 in the row layout.
ATTN_HD int decode_pack(int Hq, int Hkv) { return (Hq <= 32 && 32 % Hkv == 0) ? Hkv : 1; }
ATTN_HD int decode_tokens_per_block(int Hq, int Hkv) { return kDecodeBlockRows / decode_pack(Hq, Hkv); }
ATTN_HD int decode_rows_per_seq(int Hq, int Hkv) {
  return decode_pack(Hq, Hkv) > 1 ? 1 : Hkv * decode_head_blocks(Hq / Hkv);
}
// Row u of a sequence: its KV head, the first query head it serves and how many it serves.  In
// the packed layout the one row serves all Hq heads; otherwise row u is KV head u / head_blocks
// and head block u % head_blocks of that head's group, whose last block may hold fewer than 32.
ATTN_HD int decode_row_kv_head(int Hq, int Hkv, int u) {
  return decode_pack(Hq, Hkv) > 1 ? 0 : u / decode_head_blocks(Hq / Hkv);
}
ATTN_HD int decode_row_first_head(int Hq, int Hkv, int u) {
  if (decode_pack(Hq, Hkv) > 1) return 0;
  const int group = Hq / Hkv, hb = decode_head_blocks(group);
  return (u / hb) * group + (u % hb) * 32;
}
ATTN_HD int decode_row_heads(int Hq, int Hkv, int u) {
  if (decode_pack(Hq, Hkv) > 1) return Hq;
  const int group = Hq / Hkv, left = group - (u % decode_head_blocks(group)) * 32;
  return left < 32 ? left : 32;
}
// Query heads per partial slot.
ATTN_HD int decode_heads_per_slot(int Hq, int Hkv) {
  const int group = Hq / Hkv;
  return decode_pack(Hq, Hkv) > 1 ? Hq : (group < 32 ? group : 32);
}
ATTN_HD int decode_teams(int workers, int rows_per_seq) {
  const int t = workers / rows_per_seq;
  return t > 0 ? t : 1;
}
// Keys the query of a sequence with n cached tokens sees: all of them, or the last `window`.
ATTN_HD int decode_visible_keys(int n, int window) { return window > 0 && n > window ? window : n; }
// First token of a sequence's block 0: its first visible key, or, in a paged cache (aligned),
// the start of the tokens_per_block group holding it, so that no block straddles a page (the
// page size is a multiple of tokens_per_block); keys before the first visible one are masked.
ATTN_HD int decode_block_origin(int n, int window, int tokens_per_block, int aligned) {
  const int lo = n - decode_visible_keys(n, window);
  return aligned ? lo - lo % tokens_per_block : lo;
}
ATTN_HD int decode_key_blocks(int n, int window, int tokens_per_block, int aligned) {
  const int org = decode_block_origin(n, window, tokens_per_block, aligned);
  return n > org ? (n - org + tokens_per_block - 1) / tokens_per_block : 0;
}
ATTN_HD long long decode_max_slots(int n_seq, int rows_per_seq) {
  return (long long)rows_per_seq * (decode_teams(kDecodeMaxWorkers, rows_per_seq) + n_seq);
}

// Decode workspace (host side): the blocks-per-team share (one int, 256-byte region), the
// exclusive prefix of per-sequence block counts (n_seq + 1 ints), then for every partial slot
// the (m, l) pair and the unnormalised fp32 O of its query heads.
struct DecWorkspaceLayout {
  size_t share, prefix, ml, o, total;  // byte offsets of each region, and the size
};
inline DecWorkspaceLayout decode_workspace_layout(int n_seq, int Hq, int Hkv, int d) {
  const size_t slots = (size_t)decode_max_slots(n_seq, decode_rows_per_seq(Hq, Hkv));
  const size_t nh = (size_t)decode_heads_per_slot(Hq, Hkv);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  DecWorkspaceLayout l;
  l.share = 0;
  l.prefix = 256;
  l.ml = l.prefix + up(sizeof(int) * ((size_t)n_seq + 1));
  l.o = l.ml + up(slots * nh * 2 * sizeof(float));
  l.total = l.o + slots * nh * (size_t)d * sizeof(float);
  return l;
}

}  // namespace attnfwd
