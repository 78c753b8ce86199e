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

// Decode: each workgroup handles one chunk of keys of one (sequence, KV head, block of up to 32
// query heads); a second pass merges the chunks.
ATTN_HD int decode_head_blocks(int group) { return (group + 31) / 32; }

// Keys per chunk: the largest power of two in [128, 1024] that still gives about 8192 work units
// at the longest sequence (units = n_seq * KV heads * head blocks * chunks), so that every CU
// has work, while long chunks keep the number of partials small.
ATTN_HD int decode_chunk_keys(int n_seq, int units_per_chunk_row, int max_len) {
  int ck = 1024;
  while (ck > 128 && (long long)n_seq * units_per_chunk_row * ((max_len + ck - 1) / ck) < 8192) ck /= 2;
  return ck;
}

ATTN_HD int decode_num_chunks(int max_len, int chunk_keys) { return (max_len + chunk_keys - 1) / chunk_keys; }

}  // namespace attnfwd
