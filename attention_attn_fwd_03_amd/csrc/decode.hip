// Decode attention over a pooled KV cache: one new query token per sequence, its keys and
// values read from rows offsets[s] .. offsets[s] + lens[s] - 1 of one shared pool
// ("003-注意力机制详解：从基础Attention到DeepSeek的优化策略", §三.3: one preallocated pool,
// sequences told apart by offset).  The query is the newest token, so every cached key is
// visible, or only the last W under a sliding window.
//
// The pass is bound by reading K and V once from HBM ("LLM中的Attention实现及优化": the KV
// cache makes attention memory-bound, and GQA/MQA cut its size by Hq/Hkv).  It is split over
// the key length, with equal work per worker whatever the mix of lengths:
//   1. decode_split_kernel: one resident round of single-wave workers, in teams of U = Hkv *
//      head_blocks (plan.hpp).  Each team takes an equal share of the 32-key blocks of all
//      sequences laid end to end; member u runs the online softmax of the tiled algorithm
//      ("003-…", §二) for row u (a KV head and up to 32 query heads sharing it) over the blocks
//      of each sequence the share touches, and writes one unnormalised partial (O, m, l) in fp32
//      per sequence touched.  The U members of a team read the same tokens of every KV head at
//      the same time, so together they sweep contiguous pool rows.  K and V reach LDS by
//      wave-wide buffer loads (each load instruction fetches whole rows) into a two-stage ring;
//      K comes back as the MFMA A operand, V transposed through ds_read_b64_tr_b16.
//   2. decode_merge_kernel: per (sequence, query head), rescales its partials to a common
//      maximum and writes O (bf16) and the natural-log LSE (fp32).
// A paged cache ("LLM中的Attention实现及优化", PagedAttention: the cache in small fixed-size pages
// that need not be contiguous) uses the same two passes; only the split's addressing changes:
// each block is looked up in the sequence's row of the page table and read from its page (the
// page size is a multiple of the block's token count, and a sequence's blocks start on a block
// boundary, so no block straddles two pages).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "attn_device.hpp"
#include "fp8_device.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace attnfwd {

typedef __attribute__((address_space(3))) void lds_void_d;

template <int D, int KV = kKvBf16>
struct DecCfg {
  static constexpr bool FP8 = KV != kKvBf16;
  static constexpr int ROWB = FP8 ? D : D * 2;  // bytes of one head's K or V row
  static constexpr int CH = ROWB / 16;          // 16-byte chunks per row
  // Row pitches in LDS are whole 16-byte chunks (each lane of a wave-wide load fills one chunk).
  // K: the bf16 A-operand reads of 16 rows x 16 bytes hit distinct banks (the fp8 reads of 32 rows
  // x 8 bytes meet in pairs, rows r and r + 16; K is a small share of the LDS reads).  V: the
  // transposed reads of a half-wave (bf16: 4 rows x 64 bytes; fp8: 8 rows x 32 bytes) cover the
  // 256-byte bank space once.
  static constexpr int KPB = ROWB + 16;
  static constexpr int VPB = FP8 ? ROWB + 32 : ROWB + 64;
  static_assert(KPB % 16 == 0 && VPB % 16 == 0, "whole chunks per LDS row");
  static constexpr int K_STAGE = (kDecodeBlockRows * KPB + 1023) / 1024 * 1024;
  static constexpr int V_STAGE = kDecodeBlockRows * VPB;
  static constexpr int K_LOADS = K_STAGE / 1024;  // wave-wide 16-byte-per-lane loads per stage
  static constexpr int V_LOADS = V_STAGE / 1024;
  static_assert(V_STAGE % 1024 == 0, "a V stage must be whole wave-wide loads");
  static_assert(2 * (K_LOADS + V_LOADS) <= 63, "two blocks' loads must fit the vmcnt counter");
};

// Pipeline stages of the split: three (up to two blocks in flight per worker) for the one-head
// bf16 layout at d = 128, which runs two workers per CU (2 x 57 KB of LDS), else two.  Measured
// (three alternating A/B rounds): MQA 1-2% faster, MQA over a paged cache 3-6% faster; FP8 pools
// (four workers per CU, 4 x 30 KB) were 5% slower on GQA and unchanged on MQA with three, and the
// packed bf16 layout runs three workers per CU, for which three stages do not fit (3 x 57 KB).
template <int D, int KV, bool PACKED>
struct DecStages {
  static constexpr int value = D == 128 && !PACKED && KV == kKvBf16 ? 3 : 2;
};

__device__ __forceinline__ bool decode_seq_valid(const DecArgs& a, int n, int64_t base, bool paged) {
  if (paged) return n >= 0 && n <= a.max_len;  // page entries are checked as they are read
  return n >= 0 && n <= a.max_len && base >= 0 && base + n <= a.pool_rows;
}

// Blocks of one row of sequence s; 0 for a sequence that is not read (invalid or empty).
__device__ __forceinline__ int seq_blocks(const DecArgs& a, int s, int tpb, bool paged) {
  const int n = a.lens[s];
  const int64_t base = paged ? 0 : a.offsets[s];
  return decode_seq_valid(a, n, base, paged) ? decode_key_blocks(n, a.window, tpb, paged) : 0;
}

__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
  return (int64_t)(((uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((int)(x >> 32)) << 32) |
                   (unsigned)__builtin_amdgcn_readfirstlane((int)x));
}

// Buffer over tokens [k0, end) of one sequence, KV heads kvh .. kvh + pack - 1: view byte 0 is
// head kvh of pool row base + k0, and the view ends after head kvh + pack - 1 of token end - 1.
// Anything at or past the end reads as zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t seq_rsrc(const void* pool, int64_t base, int k0, int end, int kvh,
                                                           int Hkv, int pack, int rowb) {
  const int left = end - k0;
  // Every input is wave-uniform; passing the address and size through readfirstlane keeps the
  // descriptor in scalar registers whatever registers the compiler chose for its inputs (a
  // descriptor it cannot prove uniform would be wrapped in a per-lane loop).
  const uint64_t addr = (uint64_t)pool + ((uint64_t)(base + k0) * Hkv + kvh) * rowb;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)addr);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(addr >> 32));
  const int bytes = __builtin_amdgcn_readfirstlane(left > 0 ? ((left - 1) * Hkv + pack) * rowb : 0);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), 0, bytes, 0x00020000);
}

// Cache policy of the K/V stream: non-temporal.  Every cached row is read exactly once per call,
// so it should not displace anything in L2; marking the loads as streaming lifts the decode pass
// from about 74% to about 80% of HBM peak on MI355X.
constexpr int kStreamPolicy = 2;

// N wave-wide loads straight into LDS: load j fills bytes [j*1024, +1024) of `stage`, lane l's
// 16 bytes at j*1024 + 16*l coming from buffer offset voff[j].
template <int N>
__device__ __forceinline__ void load_to_lds(__amdgpu_buffer_rsrc_t rs, unsigned char* stage,
                                            const unsigned (&voff)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_d*)(stage + j * 1024), 16, voff[j], 0, 0, kStreamPolicy);
}

// Per-lane source offsets of the loads that fill a stage of 32 block rows at pitch PITCH: lane
// slot o = j*1024 + 16*lane holds row r = o / PITCH, chunk (o % PITCH) / 16.  Block row r is
// token r / pack, KV head r % pack, i.e. byte (r / pack) * token_bytes + (r % pack) * ROWB of the
// block's buffer.  Pad slots take an offset past any buffer (the hardware returns zeros and
// reads nothing).
// With SWAP23, LDS row r holds block row r with bits 2 and 3 exchanged (the fp8 V stage: an
// 8-row transposed read then returns the rows in the order of the P operand, see below).
template <int N, int PITCH, int CH, int ROWB, bool SWAP23 = false>
__device__ __forceinline__ void stage_offsets(unsigned (&voff)[N], int lane, int pack, int token_bytes) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int o = j * 1024 + 16 * lane;
    const int r = o / PITCH, ch = (o % PITCH) / 16;
    const int src = SWAP23 ? fp8_v_row(r) : r;
    voff[j] = (r < kDecodeBlockRows && ch < CH)
                  ? (unsigned)((src / pack) * token_bytes + (src % pack) * ROWB + ch * 16)
                  : 0x80000000u;
  }
}

// PAGED selects the pool addressing, KV the pool's element format and PACKED the block layout
// (all Hkv heads of 32 / Hkv tokens, or 32 tokens of one head) at compile time, so the contiguous
// bf16 kernel carries none of the page-table or conversion code, and the one-head layout (MQA,
// large groups) none of the packed layout's masking.
template <int D, bool PAGED, int KV, bool PACKED>
// At d = 128 at most four waves share a CU (one per SIMD), so the wave may use the whole register
// file; at d = 64 two waves per SIMD fit.
__global__ __launch_bounds__(64, D == 128 ? 1 : 2) void decode_split_kernel(DecArgs a) {
  using C = DecCfg<D, KV>;
  constexpr int NST = DecStages<D, KV, PACKED>::value;
  // Each pipeline stage (K rows, then V rows) is its own LDS object, so reading one does not wait
  // for loads into another.
  __shared__ __attribute__((aligned(1024))) unsigned char kv_lds0[C::K_STAGE + C::V_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char kv_lds1[C::K_STAGE + C::V_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char kv_lds2[NST == 3 ? C::K_STAGE + C::V_STAGE : 1024];
  auto k_stage = [&](auto stage_c) -> unsigned char* {
    constexpr int S = decltype(stage_c)::value;
    if constexpr (S == 0) return kv_lds0;
    else if constexpr (S == 1) return kv_lds1;
    else return kv_lds2;
  };
  auto v_stage = [&](auto stage_c) -> unsigned char* { return k_stage(stage_c) + C::K_STAGE; };

  const int lane = threadIdx.x, h = lane >> 5, col = lane & 31;
  const int team = blockIdx.x / a.rows, u = blockIdx.x % a.rows;
  const int pack = PACKED ? a.pack : 1, tpb = PACKED ? a.tpb : kDecodeBlockRows;
  const int pack_log2 = PACKED ? __builtin_ctz((unsigned)a.pack) : 0;
  const int kvh0 = decode_row_kv_head(a.Hq, a.Hkv, u);      // KV head of block row 0
  const int qbase = decode_row_first_head(a.Hq, a.Hkv, u);  // query head of column 0
  const bool writer = blockIdx.x == 0;  // publishes the share and the prefix for the merge pass

  // ---- This team's share of the blocks: [start, stop) of the concatenated block order. ----
  int total = 0, s_cur = -1, b_cur = 0, start = 0, stop = 0;
  int n_cur = 0;          // length and first pool row of sequence s_cur
  int64_t base_cur = 0;
  if (a.n_seq <= 64) {
    int n_l = 0;
    int64_t base_l = 0;
    if (lane < a.n_seq) {
      n_l = a.lens[lane];
      base_l = PAGED ? 0 : a.offsets[lane];
    }
    const int nbv =
        lane < a.n_seq && decode_seq_valid(a, n_l, base_l, PAGED) ? decode_key_blocks(n_l, a.window, tpb, PAGED) : 0;
    const int incl = wave_inclusive_scan(nbv, lane);
    total = __builtin_amdgcn_readlane(incl, 63);
    const int share = (total + a.teams - 1) / a.teams;
    start = team * share;
    stop = start + share < total ? start + share : total;
    const int excl = incl - nbv;
    if (writer) {
      if (lane < a.n_seq) a.ws_prefix[lane] = excl;
      if (lane == 0) {
        a.ws_prefix[a.n_seq] = total;
        a.ws_share[0] = share;
      }
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(nbv > 0 && excl <= start && start < excl + nbv);
    if (start < stop && hit != 0) {
      const int l = __builtin_ctzll(hit);
      s_cur = l;
      b_cur = start - __builtin_amdgcn_readlane(excl, l);
      n_cur = __builtin_amdgcn_readlane(n_l, l);
      base_cur = (int64_t)(((uint64_t)(unsigned)__builtin_amdgcn_readlane((int)(base_l >> 32), l) << 32) |
                           (unsigned)__builtin_amdgcn_readlane((int)base_l, l));
    }
  } else {
    for (int g = 0; g < a.n_seq; g += 64) {
      const int s = g + lane;
      total += wave_sum_i32(s < a.n_seq ? seq_blocks(a, s, tpb, PAGED) : 0);
    }
    total = __builtin_amdgcn_readfirstlane(total);
    const int share = (total + a.teams - 1) / a.teams;
    start = team * share;
    stop = start + share < total ? start + share : total;
    if (writer || start < stop) {
      int run = 0;
      for (int g = 0; g < a.n_seq; g += 64) {
        const int s = g + lane;
        const int nbv = s < a.n_seq ? seq_blocks(a, s, tpb, PAGED) : 0;
        const int incl = wave_inclusive_scan(nbv, lane);
        const int excl = run + incl - nbv;
        if (writer && s < a.n_seq) a.ws_prefix[s] = excl;
        const uint64_t hit = __builtin_amdgcn_ballot_w64(nbv > 0 && excl <= start && start < excl + nbv);
        if (s_cur < 0 && start < stop && hit != 0) {
          const int l = __builtin_ctzll(hit);
          s_cur = g + l;
          b_cur = start - __builtin_amdgcn_readlane(excl, l);
        }
        run += __builtin_amdgcn_readlane(incl, 63);
        if (!writer && s_cur >= 0) break;
      }
      if (writer && lane == 0) {
        a.ws_prefix[a.n_seq] = total;
        a.ws_share[0] = share;
      }
    }
  }
  if (start >= stop || s_cur < 0) return;

  const int token_bytes = a.Hkv * C::ROWB;  // bytes between consecutive tokens of the pool
  unsigned k_voff[C::K_LOADS], v_voff[C::V_LOADS];
  stage_offsets<C::K_LOADS, C::KPB, C::CH, C::ROWB>(k_voff, lane, pack, token_bytes);
  stage_offsets<C::V_LOADS, C::VPB, C::CH, C::ROWB, C::FP8>(v_voff, lane, pack, token_bytes);
  // K A operand: lane holds K[row = col][16*ks + 8*h .. +7], at LDS byte col*KPB + 32*ks + 16*h
  // (bf16) or col*KPB + 16*ks + 8*h (fp8 codes, converted in registers).
  const int k_lane = col * C::KPB + h * (C::FP8 ? 8 : 16);
  // V^T operand.  bf16: ds_read_b64_tr_b16 addressing (see attn_device.hpp).  fp8: one
  // ds_read_b64_tr_b8 per operand, group g = lane/16 reading rows 8*(g/2) .. +7 and columns
  // 16*(g%2) .. +15 of the 32-column slice: lane l gets rows 16*j + 8*h .. +7 of column l%32.  The
  // stage holds block row swap23(r) at LDS row r, so these are block rows 16*j + 8*(e/4) + 4*h +
  // e%4 for byte e -- the rows the P operand holds at k = 8*h + e.
  const int v_lane = C::FP8 ? (8 * (lane >> 5) + ((lane & 15) >> 1)) * C::VPB + ((lane >> 4) & 1) * 16 + (lane & 1) * 8
                            : (4 * h + ((lane & 15) >> 2)) * C::VPB + ((lane >> 4) & 1) * 32 + (lane & 3) * 8;
  // S^T register i of this lane holds block row r(i) = 8*(i/4) + 4*h + i%4 against query head
  // qbase + col.  In the packed layout only rows of the head's own KV group count.
  unsigned head_ok = 0xFFFFu;
  if constexpr (PACKED) {
    head_ok = 0u;
    const int g = col / a.group;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (((8 * (i >> 2) + 4 * h + (i & 3)) % pack) == g) head_ok |= 1u << i;
  }
  const float c = a.c;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  constexpr int QL = D / 16;  // Q loads per lane
  constexpr unsigned kWaitBlock = vmcnt_at_most(C::K_LOADS + C::V_LOADS);

  const auto* lens_c = kernel_constant(a.lens);
  const auto* offs_c = kernel_constant(a.offsets);
  const QTransform qt = q_transform(a.qmode);
  // Columns past the row's own heads (the last head block of a group may hold fewer than 32)
  // read head qbase instead, are zeroed and never stored.
  const bool q_ok = col < decode_row_heads(a.Hq, a.Hkv, u);

  if (a.n_seq > 64) {
    n_cur = lens_c[s_cur];
    base_cur = PAGED ? 0 : offs_c[s_cur];
  }

  // One piece per iteration: blocks [b, b + take) of sequence s.
  int pos = start, s = s_cur, b = b_cur;
  int n = n_cur;
  int64_t base = base_cur;
  for (;;) {
    const int nb = decode_key_blocks(n, a.window, tpb, PAGED);  // > 0: the sequence holds block `pos`
    const int take = nb - b < stop - pos ? nb - b : stop - pos;
    const int vis_lo = n - decode_visible_keys(n, a.window);           // first visible key
    const int org = decode_block_origin(n, a.window, tpb, PAGED);       // first token of block 0
    const int t_begin = org + b * tpb;                                        // first token
    const int t_end = org + (b + take) * tpb < n ? org + (b + take) * tpb : n;  // one past the last

    // Paged: the table entries of the piece's first 64 pages, lane i holding page slot pg0 + i
    // (loaded next to Q, one round trip for both); entries past the table row read as -1.
    int pg0 = 0, pg_win = -1;
    auto load_window = [&](int j) {
      pg0 = j;
      pg_win = j + lane < a.table_stride ? a.block_table[(size_t)s * a.table_stride + j + lane] : -1;
    };
    if constexpr (PAGED) load_window(t_begin / a.page_size);

    // Q is loaded raw here and transformed only after the first block's loads are issued (below),
    // so all its loads are in flight together and the K/V loads start without waiting for them.
    u32x4 qraw[QL];
    {
      const unsigned short* Qg =
          (const unsigned short*)a.q + ((size_t)s * a.Hq + qbase + (q_ok ? col : 0)) * D;
#pragma unroll
      for (int ks = 0; ks < QL; ++ks) qraw[ks] = *(const u32x4*)(Qg + ks * 16 + h * 8);
    }
    bf16x8 qf[QL];
    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    RowState st = {-INFINITY, 0.f, 0.f};

    // Loads of the block starting at token t0 into stage STAGE.  Contiguous pool: a buffer over
    // the piece's remaining tokens.  Paged pool: the block lies inside one page (t0 is a multiple
    // of tpb, the page size a multiple of tpb); its entry is looked up and the buffer covers the
    // block's tokens in that page.  An entry outside [0, pool_pages) reads nothing and marks the
    // piece bad.  A block past the piece's end reads nothing and looks nothing up.
    bool bad = false;
    auto issue = [&](int t0, auto stage_c) {
      int64_t rbase = base;  // pool row of token 0 of the sequence, as if it were contiguous
      int end = t_end;
      if constexpr (PAGED) {
        rbase = 0;
        end = t0;
        if (t0 < t_end) {
          const int j = t0 / a.page_size;
          if (j - pg0 >= 64) load_window(j);  // pages are visited in order
          const int64_t pg = __builtin_amdgcn_readlane(pg_win, j - pg0);
          if (pg >= 0 && pg < a.pool_pages) {
            rbase = (pg - j) * a.page_size;  // rbase + t0 = pg * page_size + t0 % page_size
            end = t0 + tpb < t_end ? t0 + tpb : t_end;
          } else {
            bad = true;
          }
        }
      }
      load_to_lds(seq_rsrc(a.k_pool, rbase, t0, end, kvh0, a.Hkv, pack, C::ROWB), k_stage(stage_c), k_voff);
      load_to_lds(seq_rsrc(a.v_pool, rbase, t0, end, kvh0, a.Hkv, pack, C::ROWB), v_stage(stage_c), v_voff);
    };
    // One block (first token t0) held in stage STAGE.
    auto block = [&](int t0, auto stage_c) {
      const unsigned char* Ks = k_stage(stage_c) + k_lane;
      f32x16 sv[1];
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[0][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < QL; ++ks) {
        bf16x8 kf;
        if constexpr (C::FP8)
          kf = fp8x8_to_bf16<KV>(*(const u32x2*)(Ks + ks * 16));
        else
          kf = __builtin_bit_cast(bf16x8, *(const u32x4*)(Ks + ks * 32));
        sv[0] = mfma_32x32x16(kf, qf[ks], sv[0]);
      }
      // The piece ends inside this block (only at the sequence's end), or the block starts
      // before the first visible key (only a paged cache under a window).
      if (t0 + tpb > t_end || (PAGED && t0 < vis_lo)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * h + (i & 3);
          const int tok = t0 + (r >> pack_log2);
          const bool ok = ((head_ok >> i) & 1u) && tok < t_end && (!PAGED || tok >= vis_lo);
          sv[0][i] = ok ? sv[0][i] : -INFINITY;
        }
      } else if constexpr (PACKED) {  // rows of other KV groups
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[0][i] = ((head_ok >> i) & 1u) ? sv[0][i] : -INFINITY;
      }
      const float mb = update_max(sv, st, o, c);
      unsigned pk[8];
      exp_block(sv[0], c, mb, st, pk);
      const unsigned char* Vs = v_stage(stage_c) + v_lane;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 pw = {pk[4 * j], pk[4 * j + 1], pk[4 * j + 2], pk[4 * j + 3]};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          bf16x8 vf;
          if constexpr (C::FP8) {
            vf = fp8x8_to_bf16<KV>(lds_read_tr8(Vs + 16 * j * C::VPB + dt * 32));
          } else {
            const u32x2 r0 = lds_read_tr16(Vs + 16 * j * C::VPB + dt * 64);
            const u32x2 r1 = lds_read_tr16(Vs + (16 * j + 8) * C::VPB + dt * 64);
            vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3));
          }
          o[dt] = mfma_32x32x16(vf, pb, o[dt]);
        }
      }
    };

    // The blocks after the current one are always issued, even past the piece's end (they then
    // read nothing), which keeps the loop free of branches around the loads.
    issue(t_begin, S0{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < QL; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, q_word(qraw[ks], qt, q_ok));
    if constexpr (NST == 2) {
      for (int t0 = t_begin;; t0 += 2 * tpb) {
        issue(t0 + tpb, S1{});
        __builtin_amdgcn_s_waitcnt(kWaitBlock);
        block(t0, S0{});
        if (t0 + tpb >= t_end) break;
        issue(t0 + 2 * tpb, S0{});
        __builtin_amdgcn_s_waitcnt(kWaitBlock);
        block(t0 + tpb, S1{});
        if (t0 + 2 * tpb >= t_end) break;
      }
    } else {
      // Two blocks in flight while one is computed, except during the third block of each round:
      // at the top of the loop only the block read first may be in flight.  The compiler's record
      // of which LDS stage a global->LDS load writes does not survive the loop's back edge, so a
      // load still in flight there into another stage would make the first read wait for it.
      constexpr unsigned kWaitTwo = vmcnt_at_most(2 * (C::K_LOADS + C::V_LOADS));
      using S2 = std::integral_constant<int, 2>;
      for (int t0 = t_begin;; t0 += 3 * tpb) {
        issue(t0 + tpb, S1{});
        issue(t0 + 2 * tpb, S2{});
        __builtin_amdgcn_s_waitcnt(kWaitTwo);
        block(t0, S0{});
        if (t0 + tpb >= t_end) break;
        issue(t0 + 3 * tpb, S0{});
        __builtin_amdgcn_s_waitcnt(kWaitTwo);
        block(t0 + tpb, S1{});
        if (t0 + 2 * tpb >= t_end) break;
        __builtin_amdgcn_s_waitcnt(kWaitBlock);
        block(t0 + 2 * tpb, S2{});
        if (t0 + 3 * tpb >= t_end) break;
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));  // no load may still target LDS past this point

    // Partial of this (team, sequence, row): unnormalised O relative to m, plus (m, l).  An fp8
    // pool's V scale is applied here (the K scale is folded into c).
    const float l_tot = pair_sum(st.l);
    if (q_ok) {
      const size_t idx = ((size_t)(team + s) * a.rows + u) * a.nh + col;
      float* wo = a.ws_o + idx * D;
      const float vs = C::FP8 ? a.v_scale : 1.f;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4*)(wo + dt * 32 + g * 8 + h * 4) =
              f32x4{o[dt][4 * g] * vs, o[dt][4 * g + 1] * vs, o[dt][4 * g + 2] * vs, o[dt][4 * g + 3] * vs};
      if (h == 0) {  // a piece that met a bad page entry is marked with NaN for the merge
        a.ws_ml[2 * idx] = bad ? NAN : st.m;
        a.ws_ml[2 * idx + 1] = bad ? NAN : l_tot;
      }
    }

    pos += take;
    if (pos >= stop) break;
    // The next sequence that holds blocks starts exactly at `pos` (it exists while blocks remain
    // in the share; the bound only guards the lens/offsets reads).
    b = 0;
    for (++s; s < a.n_seq; ++s) {
      n = lens_c[s];
      base = PAGED ? 0 : offs_c[s];
      if (decode_seq_valid(a, n, base, PAGED) && decode_key_blocks(n, a.window, tpb, PAGED) > 0) break;
    }
    if (s >= a.n_seq) break;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));  // no load may still target LDS past this point
}

// One 64-lane workgroup per (query head, sequence).  Lane j holds piece j's (m, l) (64 pieces at a
// time); the maximum and the sum of weights come from wave reductions; each lane accumulates
// D/64 output columns over the pieces, the piece weight broadcast from the lane that holds it.
// The kernel is two memory round trips with no branch around a load: the sequence's length and
// offset and the split's share and prefix (scalar loads, all issued together), then the pieces'
// (m, l) and the O slices of the first MB pieces (unconditional loads at clamped piece indices,
// whose surplus values are dropped by selects).
// Wave-wide maximum and sum in VALU steps: within each 16-lane row by DPP (swap neighbours, swap
// pairs, mirror halves of 8, mirror the row), then across the four rows by readlane.
#define ATTN_DPP(v, ctrl) \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (v)), (ctrl), 0xF, 0xF, false))
__device__ __forceinline__ float wave_max_f(float x) {
  x = fmaxf(x, ATTN_DPP(x, 0xB1));   // quad_perm [1, 0, 3, 2]
  x = fmaxf(x, ATTN_DPP(x, 0x4E));   // quad_perm [2, 3, 0, 1]
  x = fmaxf(x, ATTN_DPP(x, 0x141));  // row_half_mirror
  x = fmaxf(x, ATTN_DPP(x, 0x140));  // row_mirror
  const int b = __builtin_bit_cast(int, x);
  return fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))),
               fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48))));
}
__device__ __forceinline__ float wave_sum_f(float x) {
  x += ATTN_DPP(x, 0xB1);
  x += ATTN_DPP(x, 0x4E);
  x += ATTN_DPP(x, 0x141);
  x += ATTN_DPP(x, 0x140);
  const int b = __builtin_bit_cast(int, x);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}
#undef ATTN_DPP

template <int PER>
__device__ __forceinline__ void load_slice(const float* p, float (&v)[PER]) {
  if constexpr (PER == 2) {
    const f32x2 w = *(const f32x2*)p;
    v[0] = w.x;
    v[1] = w.y;
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) v[e] = p[e];
  }
}

template <int D, bool PACKED, bool PAGED>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecArgs a) {
  constexpr int PER = D / 64;
  constexpr int MB = 16;
  const int hq = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  // Wave-uniform and constant while the merge runs (the split kernel before it wrote the share and
  // the prefix): through the scalar cache, none of them behind a branch.
  const int n = kernel_constant(a.lens)[s];
  const int64_t base = PAGED ? 0 : kernel_constant(a.offsets)[s];
  const int share = kernel_constant(a.ws_share)[0];
  const int p0 = kernel_constant(a.ws_prefix)[s];
  const bool valid = decode_seq_valid(a, n, base, PAGED);  // else the outputs become NaN
  const int nb = valid ? decode_key_blocks(n, a.window, a.tpb, PAGED) : 0;
  const int kvh = hq / a.group, within = hq % a.group;
  // Slot row and column of this query head: one row holding every head in the packed layout,
  // else row (KV head, block of 32 heads).
  const int u = PACKED ? 0 : kvh * a.hblocks + within / 32;
  const int col = PACKED ? hq : within % 32;
  // Teams t0 .. t0 + np - 1 met this sequence; piece j is slot (t0 + j + s) * rows + u, head col.
  const int sh = share > 0 ? share : 1;
  const int t0 = p0 / sh;
  const int np = nb > 0 ? (p0 + nb - 1) / sh - t0 + 1 : 0;
  const size_t idx0 = ((size_t)(t0 + s) * a.rows + u) * a.nh + col;
  const size_t step = (size_t)a.rows * a.nh;
  const float* wo0 = a.ws_o + idx0 * D + lane * PER;

  float M = -INFINITY, L = 0.f;
  bool bad = !valid;  // also set when a piece read a page entry outside the pool (its m is NaN)
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int j0 = 0; j0 < np; j0 += 64) {
    const int cnt = np - j0 < 64 ? np - j0 : 64;
    const int jl = lane < cnt ? lane : cnt - 1;
    const f32x2 ml = *(const f32x2*)(a.ws_ml + 2 * (idx0 + (size_t)(j0 + jl) * step));
    float ov[MB][PER];
    auto fetch = [&](int jb) {
#pragma unroll
      for (int jj = 0; jj < MB; ++jj) {
        const int jc = jb + jj < cnt ? jb + jj : cnt - 1;
        load_slice<PER>(wo0 + (size_t)(j0 + jc) * step * D, ov[jj]);
      }
#pragma unroll
      for (int jj = 0; jj < MB; ++jj)
#pragma unroll
        for (int e = 0; e < PER; ++e) ov[jj][e] = jb + jj < cnt ? ov[jj][e] : 0.f;
    };
    fetch(0);
    // Keep the first batch's loads next to the (m, l) load (one round trip for both) rather than
    // behind the reductions that follow.
#pragma unroll
    for (int jj = 0; jj < MB; ++jj)
#pragma unroll
      for (int e = 0; e < PER; ++e) asm volatile("" : "+v"(ov[jj][e]));
    const float mj = lane < cnt ? ml.x : -INFINITY;
    const float lj = lane < cnt ? ml.y : 0.f;
    // Rescale what is accumulated so far to the new maximum, then add these pieces.
    if (__builtin_amdgcn_ballot_w64(__builtin_isnan(mj)) != 0) bad = true;
    const float Mn = fmaxf(M, wave_max_f(mj));
    if (Mn != -INFINITY) {
      const float alpha = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      L *= alpha;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] *= alpha;
      M = Mn;
      const float w = lane < cnt ? __builtin_amdgcn_exp2f(mj - M) : 0.f;
      L += w * lj;
      for (int jb = 0; jb < cnt; jb += MB) {
        if (jb > 0) fetch(jb);
#pragma unroll
        for (int jj = 0; jj < MB; ++jj) {
          const float wj =
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), (jb + jj) & 63));
#pragma unroll
          for (int e = 0; e < PER; ++e) acc[e] += wj * ov[jj][e];
        }
      }
    }
  }
  L = wave_sum_f(L);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  unsigned short* O = (unsigned short*)a.o + ((size_t)s * a.Hq + hq) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e)
    O[lane * PER + e] = __builtin_bit_cast(unsigned short, (__bf16)(bad ? NAN : acc[e] * inv));
  if (a.lse != nullptr && lane == 0)
    a.lse[(size_t)s * a.Hq + hq] = bad ? NAN : L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
}

#define ATTN_DECODE_VARIANTS(KV)                                                 \
  template __global__ void decode_split_kernel<64, false, KV, false>(DecArgs);  \
  template __global__ void decode_split_kernel<128, false, KV, false>(DecArgs); \
  template __global__ void decode_split_kernel<64, true, KV, false>(DecArgs);   \
  template __global__ void decode_split_kernel<128, true, KV, false>(DecArgs);  \
  template __global__ void decode_split_kernel<64, false, KV, true>(DecArgs);   \
  template __global__ void decode_split_kernel<128, false, KV, true>(DecArgs);  \
  template __global__ void decode_split_kernel<64, true, KV, true>(DecArgs);    \
  template __global__ void decode_split_kernel<128, true, KV, true>(DecArgs);
ATTN_DECODE_VARIANTS(kKvBf16)
ATTN_DECODE_VARIANTS(kKvE4M3)
ATTN_DECODE_VARIANTS(kKvE5M2)
#undef ATTN_DECODE_VARIANTS
template __global__ void decode_merge_kernel<64, false, false>(DecArgs);
template __global__ void decode_merge_kernel<128, false, false>(DecArgs);
template __global__ void decode_merge_kernel<64, true, false>(DecArgs);
template __global__ void decode_merge_kernel<128, true, false>(DecArgs);
template __global__ void decode_merge_kernel<64, false, true>(DecArgs);
template __global__ void decode_merge_kernel<128, false, true>(DecArgs);
template __global__ void decode_merge_kernel<64, true, true>(DecArgs);
template __global__ void decode_merge_kernel<128, true, true>(DecArgs);

// Workspace of attn_decode_noalloc, for callers that cannot allocate device memory: a fixed array
// in the library's code object.  Each GPU the library runs on holds its own copy (at its own
// address) until the process ends.  Host code never uses the array's name as an address; the
// device address comes from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

void* decode_scratch() {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> ptrs[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = ptrs[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    ptrs[dev].store(p, std::memory_order_release);
  }
  return p;
}

int decode_workers(int d, bool fp8, bool packed) {
  static std::atomic<int> cache[2][2][2][64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  std::atomic<int>& slot = cache[d == 128 ? 1 : 0][fp8 ? 1 : 0][packed ? 1 : 0][dev];
  int w = slot.load(std::memory_order_relaxed);
  if (w > 0) return w;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  // the occupancy of the variant that will run (its stage count sets its LDS)
  auto occ = [&](auto kernel) { return hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64, 0); };
  hipError_t e;
  if (d == 128)
    e = fp8 ? (packed ? occ(decode_split_kernel<128, false, kKvE4M3, true>)
                      : occ(decode_split_kernel<128, false, kKvE4M3, false>))
            : (packed ? occ(decode_split_kernel<128, false, kKvBf16, true>)
                      : occ(decode_split_kernel<128, false, kKvBf16, false>));
  else
    e = fp8 ? (packed ? occ(decode_split_kernel<64, false, kKvE4M3, true>)
                      : occ(decode_split_kernel<64, false, kKvE4M3, false>))
            : (packed ? occ(decode_split_kernel<64, false, kKvBf16, true>)
                      : occ(decode_split_kernel<64, false, kKvBf16, false>));
  if (e != hipSuccess || cus <= 0 || per_cu <= 0) return -1;
  const int cap = fp8 ? kDecodeWorkersPerCuFp8 : packed ? kDecodeWorkersPerCu : kDecodeWorkersPerCuOneHead;
  if (per_cu > cap) per_cu = cap;
  w = cus * per_cu < kDecodeMaxWorkers ? cus * per_cu : kDecodeMaxWorkers;
  slot.store(w, std::memory_order_relaxed);
  return w;
}

template <int D, int KV>
void launch_split(const DecArgs& a, dim3 grid, hipStream_t stream) {
  if (a.pack > 1) {
    if (a.paged) hipLaunchKernelGGL((decode_split_kernel<D, true, KV, true>), grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL((decode_split_kernel<D, false, KV, true>), grid, dim3(64), 0, stream, a);
  } else {
    if (a.paged) hipLaunchKernelGGL((decode_split_kernel<D, true, KV, false>), grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL((decode_split_kernel<D, false, KV, false>), grid, dim3(64), 0, stream, a);
  }
}

template <int D>
void launch_decode_d(const DecArgs& a, hipStream_t stream) {
  const dim3 g1((unsigned)(a.teams * a.rows));
  const dim3 g2((unsigned)a.Hq, (unsigned)a.n_seq);
  if (a.kv_fmt == kKvE4M3)
    launch_split<D, kKvE4M3>(a, g1, stream);
  else if (a.kv_fmt == kKvE5M2)
    launch_split<D, kKvE5M2>(a, g1, stream);
  else
    launch_split<D, kKvBf16>(a, g1, stream);
  if (a.pack > 1) {
    if (a.paged) hipLaunchKernelGGL((decode_merge_kernel<D, true, true>), g2, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL((decode_merge_kernel<D, true, false>), g2, dim3(64), 0, stream, a);
  } else {
    if (a.paged) hipLaunchKernelGGL((decode_merge_kernel<D, false, true>), g2, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL((decode_merge_kernel<D, false, false>), g2, dim3(64), 0, stream, a);
  }
}

hipError_t launch_decode(const DecArgs& a, int d, hipStream_t stream) {
  if (d == 64)
    launch_decode_d<64>(a, stream);
  else
    launch_decode_d<128>(a, stream);
  return hipGetLastError();
}

}  // namespace attnfwd
