// Fused attention forward (prefill) for gfx950: O = softmax(scale * Q K^T + mask) V and the
// row log-sum-exp, without ever writing the score matrix to memory.
//
// Sources, cited by title and section:
//   [DS-Attn]  "003-注意力机制详解：从基础Attention到DeepSeek的优化策略": §一 plain scaled
//              dot product and max-subtracted softmax; §二 tiling with an online softmax
//              (running row max and sum, accumulator rescaled by exp(old max - new max));
//              §三.1 mixed precision (products in 16-bit, softmax in fp32, result back to 16-bit).
//   [MQA-GQA]  tqpw.cn article on MQA → GQA → FlashAttention, §4.2: tiles sized for on-chip
//              memory, running statistics, one fused kernel.
//   [LLM-Attn] "LLM中的Attention实现及优化": GQA shares one K/V head among consecutive query
//              heads (repeat_kv semantics, but the copy is never made).
//
// Design (one workgroup = 4 waves = 128 query rows of one (batch, query head); three workgroups
// share a CU, so each SIMD runs three waves):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K (A operand) from LDS, Q (B operand) held in
//     registers for the whole key loop.  Computing the transpose puts one query row per lane
//     (rows = keys), so a row's max and sum need one exchange between lanes l and l ^ 32.
//   * The fp32 S^T accumulator, rounded to bf16, is already the B operand of O^T = V^T P^T;
//     V^T (the A operand) comes from row-major V in LDS through ds_read_b64_tr_b16.
//   * K/V tiles are double-buffered in LDS; the next tile's global loads are in flight while
//     the current one is computed.
//   * Tiles beyond the causal diagonal or outside the window are not visited; only tiles that
//     straddle a boundary are masked.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "attn_device.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace attnfwd {

template <int D, int BK>
struct Bf16Cfg {
  static constexpr int THREADS = 256, WAVES = 4, BQ = 128, NB = BK / 32;
  static constexpr int ROWB = D * 2;    // bytes of one K/V row in memory
  static constexpr int CH = D / 8;      // 16-byte chunks per row
  // LDS row pitches.  K rows sit 16 bytes apart modulo the 256-byte bank space, so the A-operand
  // reads (16 consecutive rows, one chunk each) hit 16 distinct slots; V rows sit 64 bytes apart,
  // so a transposed read (4 consecutive rows x 64 bytes per half-wave) covers the bank space once.
  static constexpr int KPB = ROWB + 16, VPB = ROWB + 64;
  // LDS bytes per stage, rounded up to whole wave-wide loads (the rows past BK are never read).
  static constexpr int K_TILE = (BK * KPB + 1023) / 1024 * 1024, V_TILE = (BK * VPB + 1023) / 1024 * 1024;
  static constexpr int K_LOADS = (K_TILE + 1023) / 1024;      // wave-wide 16-byte loads per tile
  static constexpr int V_LOADS = (V_TILE + 1023) / 1024;
  static constexpr int KL_PER_WAVE = (K_LOADS + WAVES - 1) / WAVES;
  static constexpr int VL_PER_WAVE = (V_LOADS + WAVES - 1) / WAVES;
  static constexpr int LDS_BYTES = 2 * K_TILE + 2 * V_TILE;
  static_assert(K_TILE % 1024 == 0 && V_TILE % 1024 == 0, "stages must be whole wave-wide loads");
};

// Buffer descriptor over at most max_rows rows, from row0 on, of nrows rows stride_bytes apart
// (each row_bytes long) at `base`: the rows of one head of a token-major pool.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t strided_rows_rsrc(const unsigned short* base, int row0, int nrows,
                                                                    int stride_bytes, int row_bytes, int max_rows) {
  int left = nrows - row0 > 0 ? nrows - row0 : 0;
  if (left > max_rows) left = max_rows;
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned char*)base + (size_t)row0 * stride_bytes), 0,
                                           left > 0 ? (left - 1) * stride_bytes + row_bytes : 0, 0x00020000);
}

// Three workgroups share a CU: each SIMD runs three waves, one from each.  That needs at most
// 168 VGPRs and 53 KB of LDS per workgroup, which is why d = 128 walks the keys in tiles of 32
// (two stages of K and V take 38 KB; tiles of 64 would take 74 KB) and d = 64 in tiles of 64 (42 KB).
// VARLEN: a ragged batch against a pool (see FwdArgs): each workgroup finds its sequence's query
// rows and keys, rows are strided by the head count, and tiles past a sequence's end exit at once.
// MASK (kMaskNone, kMaskCausal, kMaskWindow) is the mask mode, fixed at compile time: a kernel
// without a window carries none of its tests.
template <int D, int BK, bool VARLEN, int MASK>
__global__ __launch_bounds__(256, 3) void fwd_bf16_kernel(FwdArgs a) {
  using C = Bf16Cfg<D, BK>;
  constexpr int NB = C::NB;
  constexpr int causal = MASK != kMaskNone;
  const int window = MASK == kMaskWindow ? a.window : 0;
  // Two K stages and two V stages, filled straight from global memory by buffer loads while the
  // other stage is being computed on.  Each stage is its own LDS object, so the compiler can see
  // that reads of one stage do not depend on the loads still landing in the other and does not
  // wait for them.
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds0[C::K_TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds1[C::K_TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds0[C::V_TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds1[C::V_TILE];
  auto k_stage = [&](auto st_c) -> unsigned char* {
    if constexpr (decltype(st_c)::value == 0) return k_lds0;
    else return k_lds1;
  };
  auto v_stage = [&](auto st_c) -> unsigned char* {
    if constexpr (decltype(st_c)::value == 0) return v_lds0;
    else return v_lds1;
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x, lane = tid & 63;
  // Uniform (kept in an SGPR), and visibly below WAVES, so load guards that always hold fold away.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (C::WAVES - 1);
  const int h = lane >> 5, col = lane & 31;
  const PrefillTile t = VARLEN ? prefill_tile_grouped(blockIdx.x, a.B, a.Hq, a.Hkv, a.n_qt)
                               : prefill_tile(blockIdx.x, a.B, a.Hq, a.group, a.n_qt, causal, a.heads_per_xcd);
  if (VARLEN && t.b >= a.B) return;  // padding block of the grouped order
  const int q_start = t.qt * C::BQ;
  const int q = q_start + wave * 32 + col;  // query row of this lane

  // Rows of this (batch, head): Q and O rows q_rs elements apart, K and V rows kv_rs apart.
  const unsigned short* Qg;
  size_t kv_off;
  int q_rs = D, kv_rs = D;
  int64_t row0 = 0;  // ragged: first packed query row of the sequence
  if constexpr (VARLEN) {
    const auto* cu = kernel_constant(a.cu_q);
    const int64_t c0 = cu[t.b], c1 = cu[t.b + 1];
    const int n_k = kernel_constant(a.kv_lens)[t.b];
    const int64_t off = kernel_constant(a.kv_offs)[t.b];
    const bool rows_ok = c0 >= 0 && c0 <= c1 && c1 <= a.total_q;
    const bool ok = rows_ok && c1 - c0 <= a.Lq && n_k >= 0 && off >= 0 && off + n_k <= a.pool_rows;
    if (!ok) {
      // A sequence that is not read: its rows (when they can be told) report NaN.
      if (rows_ok && q_start < c1 - c0) {
        const int n_q = (int)(c1 - c0);
        const __bf16 nanb = (__bf16)NAN;
        unsigned short* Or = (unsigned short*)a.o + ((size_t)c0 * a.Hq + t.hq) * D;
        for (int r = tid >> 3; r < C::BQ; r += C::THREADS >> 3)
          if (q_start + r < n_q)
            for (int e = (tid & 7); e < D; e += 8)
              Or[(size_t)(q_start + r) * a.Hq * D + e] = __builtin_bit_cast(unsigned short, nanb);
        if (a.lse != nullptr && tid < C::BQ && q_start + tid < n_q)
          a.lse[(size_t)(c0 + q_start + tid) * a.Hq + t.hq] = NAN;
      }
      return;
    }
    a.Lq = (int)(c1 - c0);
    a.Lk = n_k;
    if (q_start >= a.Lq) return;  // this tile lies past the sequence's queries
    row0 = c0;
    q_rs = a.Hq * D;
    kv_rs = a.Hkv * D;
    Qg = (const unsigned short*)a.q + ((size_t)c0 * a.Hq + t.hq) * D;
    kv_off = ((size_t)off * a.Hkv + t.hkv) * D;
  } else {
    Qg = (const unsigned short*)a.q + ((size_t)(t.b * a.Hq + t.hq) * a.Lq) * D;
    kv_off = ((size_t)(t.b * a.Hkv + t.hkv) * a.Lk) * D;
  }
  const KeyRange kr = key_range(q_start, C::BQ, a.Lq, a.Lk, BK, causal, window);
  const unsigned short* Kh = (const unsigned short*)a.k + kv_off;  // this head's K and V rows
  const unsigned short* Vh = (const unsigned short*)a.v + kv_off;

  // Q rows as the B operand: lane holds Q[q][16*ks + 8*h .. +7] for every ks.
  bf16x8 qf[D / 16];
  {
    const QTransform qt = q_transform(a.qmode);
    const bool q_ok = q < a.Lq;
    const unsigned short* Qr = Qg + (size_t)(q_ok ? q : 0) * q_rs;  // rows past Lq read row 0, then zero
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, q_word(*(const u32x4*)(Qr + ks * 16 + h * 8), qt, q_ok));
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  RowState st = {-INFINITY, 0.f, 0.f};
  const float c = a.c;

  // Global -> LDS.  Wave-wide load j of a tile writes 16 bytes per lane at LDS offset
  // j*1024 + 16*lane of the stage; that slot is row o / pitch, chunk (o % pitch) / 16 of the padded
  // layout.  The per-lane byte offsets inside a tile are the same for every tile.
  // An offset past any buffer (and past any gbase it is added to) for pad slots.
  constexpr unsigned kPastEnd = 0x80000000u;
  unsigned k_voff[C::KL_PER_WAVE], v_voff[C::VL_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::KL_PER_WAVE; ++i) {
    const int o = (wave + C::WAVES * i) * 1024 + 16 * lane;
    const int row = o / C::KPB, chunk = (o % C::KPB) / 16;
    k_voff[i] = (row < BK && chunk < C::CH) ? (unsigned)(row * kv_rs * 2 + chunk * 16) : kPastEnd;
  }
#pragma unroll
  for (int i = 0; i < C::VL_PER_WAVE; ++i) {
    const int o = (wave + C::WAVES * i) * 1024 + 16 * lane;
    const int row = o / C::VPB, chunk = (o % C::VPB) / 16;
    v_voff[i] = (row < BK && chunk < C::CH) ? (unsigned)(row * kv_rs * 2 + chunk * 16) : kPastEnd;
  }
  auto issue_k = [&](auto st_c, int kt) {
    if constexpr (VARLEN)
      issue_loads(strided_rows_rsrc(Kh, kt * BK, a.Lk, kv_rs * 2, C::ROWB, BK), k_stage(st_c), wave, C::WAVES,
                  C::K_LOADS, k_voff);
    else
      issue_loads(rows_rsrc(Kh, kt * BK, a.Lk, C::ROWB), k_stage(st_c), wave, C::WAVES, C::K_LOADS, k_voff);
  };
  auto issue_v = [&](auto st_c, int kt) {
    if constexpr (VARLEN)
      issue_loads(strided_rows_rsrc(Vh, kt * BK, a.Lk, kv_rs * 2, C::ROWB, BK), v_stage(st_c), wave, C::WAVES,
                  C::V_LOADS, v_voff);
    else
      issue_loads(rows_rsrc(Vh, kt * BK, a.Lk, C::ROWB), v_stage(st_c), wave, C::WAVES, C::V_LOADS, v_voff);
  };

  // K reads for S^T = K Q^T: lane reads row 32*kb + col, elements 16*ks + 8*h .. +7.
  const int k_lane = col * C::KPB + h * 16;
  auto qk = [&](auto st_c, f32x16 (&s)[NB]) {
    const unsigned char* Ks = k_stage(st_c) + k_lane;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        const bf16x8 kf = *(const bf16x8*)(Ks + kb * 32 * C::KPB + ks * 32);
        s[kb] = mfma_32x32x16(kf, qf[ks], s[kb]);
      }
  };
  // V^T operand through ds_read_b64_tr_b16 (see attn_device.hpp): lane reads 8 bytes at row
  // 16*j + 8*rr + 4*h + (lane&15)/4, columns 32*dt + 16*((lane>>4)&1) + 4*(lane&3) .. +3.
  const int v_lane = (4 * h + ((lane & 15) >> 2)) * C::VPB + ((lane >> 4) & 1) * 32 + (lane & 3) * 8;
  auto pv = [&](auto st_c, int kb, const u32x4 (&pw)[2]) {
    const unsigned char* Vs = v_stage(st_c) + v_lane;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int j = 2 * kb + half;
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw[half]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const u32x2 r0 = lds_read_tr16(Vs + 16 * j * C::VPB + dt * 64);
        const u32x2 r1 = lds_read_tr16(Vs + (16 * j + 8) * C::VPB + dt * 64);
        const u32x4 vw = __builtin_shufflevector(r0, r1, 0, 1, 2, 3);
        o[dt] = mfma_32x32x16(__builtin_bit_cast(bf16x8, vw), pb, o[dt]);
      }
    }
  };
  const int lo = kr.kt_lo, hi = kr.kt_hi;
  const int w_start = q_start + wave * 32;  // this wave's rows: [w_start, w_start + 32)
  const KeyRange wkr = key_range(w_start, 32, a.Lq, a.Lk, BK, causal, window);
  const int w_lo = wkr.kt_lo, w_hi = wkr.kt_hi;
  // One tile on stage `stage` (a compile-time constant after the unroll below): start the loads of
  // tile kt+1 into the other stage, S = K Q^T, mask (edge tiles only), the online softmax of S,
  // O += P V, then wait for the loads and synchronise.
  auto step = [&](int kt, auto stage_c) {
    constexpr int STAGE = decltype(stage_c)::value;
    using Cur = std::integral_constant<int, STAGE>;
    using Oth = std::integral_constant<int, STAGE ^ 1>;
    if (kt + 1 <= hi) {
      issue_k(Oth{}, kt + 1);
      issue_v(Oth{}, kt + 1);
    }
    // A wave skips tiles that no row of its own 32 sees (above its diagonal, before its window);
    // skipping equals running them fully masked.  Tiles all its rows see fully are not masked.
    if (kt >= w_lo && kt <= w_hi) {
      f32x16 sc[NB];
      qk(Cur{}, sc);
      const int k0 = kt * BK;
      if (!tile_full(k0, w_start, 32, a.Lq, a.Lk, BK, causal, window)) {
        int elo, ehi;
        edge_key_limits(k0, h, q, a.Lq, a.Lk, causal, window, elo, ehi);
        mask_tile(sc, elo, ehi);
      }
      const float mb = update_max(sc, st, o, c);
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        unsigned pk[8];
        exp_block(sc[kb], c, mb, st, pk);
        const u32x4 pw[2] = {u32x4{pk[0], pk[1], pk[2], pk[3]}, u32x4{pk[4], pk[5], pk[6], pk[7]}};
        pv(Cur{}, kb, pw);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's global->LDS loads have landed
    __syncthreads();
  };

  if (lo <= hi) {
    issue_k(S0{}, lo);
    issue_v(S0{}, lo);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = lo; kt <= hi; kt += 2) {
      step(kt, S0{});
      if (kt + 1 <= hi) step(kt + 1, S1{});
    }
  }

  // ---- epilogue: O = acc / l (bf16, round to nearest even), LSE in natural log ----
  const float l_tot = pair_sum(st.l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // O leaves through LDS so that each store instruction writes whole rows: the accumulator layout
  // gives every lane 8 bytes of one row, four times per 32 columns.  All LDS stages are free here
  // (the last step ended with a barrier and no loads in flight); each wave stages its 32 rows in
  // a stage of its own.
  constexpr int OPB = D * 2 + 8;  // LDS row pitch of the staged O tile
  static_assert(32 * OPB <= C::K_TILE && 32 * OPB <= C::V_TILE, "a stage holds one wave's O tile");
  unsigned char* ot = wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 w = {pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                       pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv)};
      *(u32x2*)(ot + col * OPB + (dt * 32 + g * 8 + h * 4) * 2) = w;
    }
  // The reads see the writes above: LDS executes one wave's instructions in order.  Each
  // wave-wide read takes 16 bytes per lane, RPI whole rows.
  constexpr int RPI = 1024 / (D * 2);
  const int r_in = lane / (D / 8), chunk = lane % (D / 8);
  unsigned short* Oh = (unsigned short*)a.o + (VARLEN ? ((size_t)row0 * a.Hq + t.hq) * D
                                                      : ((size_t)(t.b * a.Hq + t.hq) * a.Lq) * D);
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + r_in;
    const u32x4 w = *(const u32x4*)(ot + r * OPB + chunk * 16);
    const int qr = q_start + wave * 32 + r;
    if (qr < a.Lq) *(u32x4*)(Oh + (size_t)qr * q_rs + chunk * 8) = w;
  }
  if (a.lse != nullptr && h == 0 && q < a.Lq)
    a.lse[VARLEN ? (size_t)(row0 + q) * a.Hq + t.hq : (size_t)(t.b * a.Hq + t.hq) * a.Lq + q] =
        l_tot > 0.f ? (st.m + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------------------------
// fp32 inputs: the same schedule on v_mfma_f32_32x32x2_f32, with P kept in fp32.

template <int D>
struct F32Cfg {
  static constexpr int THREADS = 256, BQ = 128, BK = 32;
  static constexpr int KP = D + 4, VP = D + 4;  // row pitches (floats)
  static constexpr int K_ELEMS = BK * KP, V_ELEMS = BK * VP, STAGE = K_ELEMS + V_ELEMS;
  static constexpr int CHUNKS = D / 4;  // 16-byte pieces per row
  static constexpr int LOADS = BK * CHUNKS / THREADS;
  static_assert(BK * CHUNKS % THREADS == 0, "tile must split evenly over the threads");
};

template <int D>
__global__ __launch_bounds__(256, 1) void fwd_f32_kernel(FwdArgs a) {
  using C = F32Cfg<D>;
  constexpr int BK = C::BK;
  __shared__ __attribute__((aligned(16))) float smem[2 * C::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const PrefillTile t = prefill_tile(blockIdx.x, a.B, a.Hq, a.group, a.n_qt, a.causal, a.heads_per_xcd);
  const int q_start = t.qt * C::BQ;
  const int q = q_start + wave * 32 + col;
  const KeyRange kr = key_range(q_start, C::BQ, a.Lq, a.Lk, BK, a.causal, a.window);

  const float* Qg = (const float*)a.q + ((size_t)(t.b * a.Hq + t.hq) * a.Lq) * D;
  const float* Kg = (const float*)a.k + ((size_t)(t.b * a.Hkv + t.hkv) * a.Lk) * D;
  const float* Vg = (const float*)a.v + ((size_t)(t.b * a.Hkv + t.hkv) * a.Lk) * D;

  // Contraction index of MFMA step (ks2, e) in half-wave h is d = 4*ks2 + 2*h + e.
  float qf[D / 2];
  {
    const float sgn = a.qmode == kQNegate ? -1.f : (a.qmode == kQZero ? 0.f : 1.f);
    for (int ks2 = 0; ks2 < D / 4; ++ks2) {
      float2 w = make_float2(0.f, 0.f);
      if (q < a.Lq) w = *(const float2*)(Qg + (size_t)q * D + 4 * ks2 + 2 * h);
      qf[2 * ks2] = a.qmode == kQZero ? 0.f : w.x * sgn;
      qf[2 * ks2 + 1] = a.qmode == kQZero ? 0.f : w.y * sgn;
    }
  }

  f32x16 o[D / 32];
  for (int dt = 0; dt < D / 32; ++dt)
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  RowState st = {-INFINITY, 0.f, 0.f};

  float4 kreg[C::LOADS], vreg[C::LOADS];
  auto load_tile = [&](int kt) {
    const int k0 = kt * BK;
    for (int i = 0; i < C::LOADS; ++i) {
      const int idx = tid + i * C::THREADS;
      const int row = idx / C::CHUNKS, ch = idx % C::CHUNKS;
      const int key = k0 + row;
      if (key < a.Lk) {
        kreg[i] = *(const float4*)(Kg + (size_t)key * D + ch * 4);
        vreg[i] = *(const float4*)(Vg + (size_t)key * D + ch * 4);
      } else {
        kreg[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        vreg[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  auto store_tile = [&](int stage) {
    float* Ks = smem + stage * C::STAGE;
    float* Vs = Ks + C::K_ELEMS;
    for (int i = 0; i < C::LOADS; ++i) {
      const int idx = tid + i * C::THREADS;
      const int row = idx / C::CHUNKS, ch = idx % C::CHUNKS;
      *(float4*)(Ks + row * C::KP + ch * 4) = kreg[i];
      *(float4*)(Vs + row * C::VP + ch * 4) = vreg[i];
    }
  };

  if (kr.kt_lo <= kr.kt_hi) {
    load_tile(kr.kt_lo);
    store_tile(0);
    __syncthreads();
  }
  const float c = a.c;

  for (int kt = kr.kt_lo; kt <= kr.kt_hi; ++kt) {
    const int stage = (kt - kr.kt_lo) & 1;
    const bool more = kt < kr.kt_hi;
    if (more) load_tile(kt + 1);
    const float* Ks = smem + stage * C::STAGE;
    const float* Vs = Ks + C::K_ELEMS;
    const int k0 = kt * BK;

    f32x16 s[1];
    for (int i = 0; i < 16; ++i) s[0][i] = 0.f;
    for (int ks2 = 0; ks2 < D / 4; ++ks2) {
      const float2 kf = *(const float2*)(Ks + col * C::KP + 4 * ks2 + 2 * h);
      s[0] = mfma_32x32x2(kf.x, qf[2 * ks2], s[0]);
      s[0] = mfma_32x32x2(kf.y, qf[2 * ks2 + 1], s[0]);
    }
    float p[16];
    const bool full = tile_full(k0, q_start, C::BQ, a.Lq, a.Lk, BK, a.causal, a.window);
    if (!full) {
      int elo, ehi;
      edge_key_limits(k0, h, q, a.Lq, a.Lk, a.causal, a.window, elo, ehi);
      mask_tile(s, elo, ehi);
    }
    const float mb = update_max(s, st, o, c);
    exp_block_f32(s[0], c, mb, st, p);
    // O^T += V^T P^T: MFMA i pairs key (8*(i/4) + i%4) of half-wave 0 with key +4 of half 1.
    for (int i = 0; i < 16; ++i) {
      const int key = (i >> 2) * 8 + h * 4 + (i & 3);
      for (int dt = 0; dt < D / 32; ++dt) o[dt] = mfma_32x32x2(Vs[key * C::VP + dt * 32 + col], p[i], o[dt]);
    }

    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  const float l_tot = pair_sum(st.l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q < a.Lq) {
    float* Og = (float*)a.o + ((size_t)(t.b * a.Hq + t.hq) * a.Lq + q) * D;
    for (int dt = 0; dt < D / 32; ++dt)
      for (int g = 0; g < 4; ++g) {
        const float4 w = make_float4(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv, o[dt][4 * g + 2] * inv,
                                     o[dt][4 * g + 3] * inv);
        *(float4*)(Og + dt * 32 + g * 8 + h * 4) = w;
      }
    if (a.lse != nullptr && h == 0)
      a.lse[(size_t)(t.b * a.Hq + t.hq) * a.Lq + q] =
          l_tot > 0.f ? (st.m + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------------

// Explicit instantiations: the host pass must emit a launch stub for every variant.
#define ATTN_FWD_BF16_VARIANTS(VARLEN, MASK)                          \
  template __global__ void fwd_bf16_kernel<64, 64, VARLEN, MASK>(FwdArgs); \
  template __global__ void fwd_bf16_kernel<128, 32, VARLEN, MASK>(FwdArgs);
ATTN_FWD_BF16_VARIANTS(false, kMaskNone)
ATTN_FWD_BF16_VARIANTS(false, kMaskCausal)
ATTN_FWD_BF16_VARIANTS(false, kMaskWindow)
ATTN_FWD_BF16_VARIANTS(true, kMaskNone)
ATTN_FWD_BF16_VARIANTS(true, kMaskCausal)
ATTN_FWD_BF16_VARIANTS(true, kMaskWindow)
#undef ATTN_FWD_BF16_VARIANTS
template __global__ void fwd_f32_kernel<64>(FwdArgs);
template __global__ void fwd_f32_kernel<128>(FwdArgs);

int prefill_block_q(bool f32) { return f32 ? F32Cfg<64>::BQ : Bf16Cfg<128, 32>::BQ; }
int prefill_block_k(bool f32, int d) { return f32 ? F32Cfg<64>::BK : (d == 128 ? 32 : 64); }
int prefill_threads(bool) { return 256; }
int prefill_lds_bytes(bool f32, int d) {
  if (f32) return d == 64 ? 2 * F32Cfg<64>::STAGE * 4 : 2 * F32Cfg<128>::STAGE * 4;
  return d == 64 ? Bf16Cfg<64, 64>::LDS_BYTES : Bf16Cfg<128, 32>::LDS_BYTES;
}

int mask_mode(const FwdArgs& a) { return a.causal ? (a.window > 0 ? kMaskWindow : kMaskCausal) : kMaskNone; }

template <bool VARLEN, int MASK>
void launch_bf16(const FwdArgs& a, int d, dim3 g, hipStream_t stream) {
  if (d == 64) hipLaunchKernelGGL((fwd_bf16_kernel<64, 64, VARLEN, MASK>), g, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((fwd_bf16_kernel<128, 32, VARLEN, MASK>), g, dim3(256), 0, stream, a);
}

template <bool VARLEN>
void launch_bf16_masked(const FwdArgs& a, int d, dim3 g, hipStream_t stream) {
  switch (mask_mode(a)) {
    case kMaskNone: launch_bf16<VARLEN, kMaskNone>(a, d, g, stream); break;
    case kMaskCausal: launch_bf16<VARLEN, kMaskCausal>(a, d, g, stream); break;
    default: launch_bf16<VARLEN, kMaskWindow>(a, d, g, stream); break;
  }
}

hipError_t launch_prefill(const FwdArgs& a, bool f32, int d, hipStream_t stream) {
  const int64_t grid = (int64_t)a.n_qt * a.B * a.Hq;
  const dim3 g((unsigned)grid), b(256);
  if (f32) {
    if (d == 64) hipLaunchKernelGGL(fwd_f32_kernel<64>, g, b, 0, stream, a);
    else hipLaunchKernelGGL(fwd_f32_kernel<128>, g, b, 0, stream, a);
  } else {
    launch_bf16_masked<false>(a, d, g, stream);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_varlen(const FwdArgs& a, int d, hipStream_t stream) {
  const int64_t grid = prefill_grouped_blocks(a.B, a.Hq, a.Hkv, a.n_qt);
  launch_bf16_masked<true>(a, d, dim3((unsigned)grid), stream);
  return hipGetLastError();
}

}  // namespace attnfwd
