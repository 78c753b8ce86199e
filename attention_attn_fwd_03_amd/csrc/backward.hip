// Attention backward for gfx950: dQ, dK, dV of O = softmax(scale * Q K^T + mask) V, given O, the
// upstream gradient dO and the forward's row log-sum-exp.
//
// Source, cited by title and section: the MQA -> GQA -> FlashAttention article (tqpw.cn), §4:
// the backward pass recomputes the forward's intermediate results from the tiles instead of
// storing them; "003-注意力机制详解：从基础Attention到DeepSeek的优化策略" §一: the full softmax
// matrix would otherwise have to be kept for back-propagation.  With P = exp(scale*S - LSE):
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D = rowsum(dO * O)
//     dQ = scale * dS K,   dK = scale * dS^T Q,
// and with GQA a KV head's gradient sums the query heads that share it.
//
// Three passes, no atomics (the result does not depend on scheduling):
//   1. bwd_rowdot_kernel: D for every query row.
//   2. bwd_dq_kernel: one workgroup per 128 query rows of one head, as the forward: S^T = K Q^T and
//      dP^T = V dO^T with Q and dO held as MFMA B operands, P^T rebuilt from the LSE (no running
//      maximum is needed), dS^T in registers, dQ^T += K^T dS^T with K^T read transposed from LDS.
//   3. bwd_dkdv_kernel: one workgroup per 128 keys of one KV head (a wave per 32 keys, its K and
//      V rows held as B operands), walking the query rows that see those keys, 32 at a time, for
//      every query head of the group: S = Q K^T, dP = dO V^T, then dV^T += dO^T P and
//      dK^T += Q^T dS with dO^T and Q^T read transposed from LDS.
// The lane layouts are those of the forward kernel (attn_device.hpp): an fp32 accumulator block
// rounded to bf16 is directly the B operand of the next product, and the transposed LDS reads
// take rows in the matching order.  Probabilities and dS enter the products in bf16; every
// accumulation is fp32.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "attn_device.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace attnfwd {

template <int D>
struct BwdCfg {
  static constexpr int ROWB = D * 2;    // bytes of one row
  static constexpr int CH = D / 8;      // 16-byte chunks per row
  static constexpr int NPB = ROWB + 16; // LDS pitch of tiles read only as the A operand
};

// Query rows per step of the dK/dV kernel.  Its three Q and three dO stages, each its own LDS
// object, must lie within the 64 KB an LDS instruction's offset reaches, or the compiler keeps a
// separate address per stage and runs out of registers: at d = 128 that allows 32 rows (6 x 8 KB).
// (64-row steps at d = 64 measured 14% slower than 32.)
constexpr int kBwdQStep = 32;

// s_waitcnt immediate that waits for this wave's LDS (and scalar) operations only.
constexpr unsigned kLgkmDone = 0xC07Fu;

// Workgroup barrier for a loop whose global->LDS loads stay in flight across it.
// __syncthreads() also fences memory, which makes the compiler wait for every outstanding
// vector-memory load first; here each wave has already waited (s_waitcnt) for what the others
// will read.  The "memory" clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_after_waits() { asm volatile("s_barrier" ::: "memory"); }

constexpr int round1k(int x) { return (x + 1023) / 1024 * 1024; }

// Tiles read both as the MFMA A operand (16 consecutive rows, one 16-byte chunk each, per
// quarter-wave) and transposed (4 consecutive rows, 64 contiguous bytes each, per half-wave) are
// stored unpadded with their 16-byte chunks permuted per row: chunk c of row r sits at chunk
// c ^ swz(r).  The LDS bank space is 256 bytes.  At d = 128 a row fills it and swz(r) =
// 4 (r mod 4) + (r / 4 mod 4): the 16 rows of an A read land on 16 distinct chunks, and the 4 rows
// of a transposed read on 4 distinct 64-byte quarters.  At d = 64 two rows share it (r mod 2 picks
// the half) and swz(r) = 4 (r / 2 mod 2) + (r / 4 mod 4), which gives the same two properties.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128)
    return ((row & 3) << 2) | ((row >> 2) & 3);
  else
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Per-lane byte offsets of the wave-wide loads that fill a tile of `rows` rows at LDS pitch
// `pitch`: load j (of those given to this wave) fills LDS bytes [j*1024, +1024); lane slot
// o = j*1024 + 16*lane is row o / pitch, chunk (o % pitch) / 16.  Pad slots get an offset past
// any buffer (zeros, nothing read).
template <int N>
__device__ __forceinline__ void tile_offsets(unsigned (&voff)[N], int wave, int waves, int lane, int rows, int pitch,
                                             int chunks, int row_bytes) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int o = (wave + waves * i) * 1024 + 16 * lane;
    const int row = o / pitch, chunk = (o % pitch) / 16;
    voff[i] = (row < rows && chunk < chunks) ? (unsigned)(row * row_bytes + chunk * 16) : 0x80000000u;
  }
}

// The same for a swizzled tile (pitch = row bytes): LDS chunk p of row r receives memory chunk
// p ^ swz(r).
template <int D, int N>
__device__ __forceinline__ void tile_offsets_swz(unsigned (&voff)[N], int wave, int waves, int lane, int rows) {
  constexpr int ROWB = D * 2;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int o = (wave + waves * i) * 1024 + 16 * lane;
    const int row = o / ROWB, chunk = (o % ROWB) / 16;
    voff[i] = row < rows ? (unsigned)(row * ROWB + (chunk ^ swz<D>(row)) * 16) : 0x80000000u;
  }
}

// The MFMA A operand "row r, 16*ks + 8*(lane/32) .. +7" of a padded tile at pitch `pitch`, for
// the 32 rows starting at `row0`: lane reads row row0 + lane%32.
__device__ __forceinline__ bf16x8 a_frag(const unsigned char* tile, int row0, int pitch, int ks, int lane) {
  return __builtin_bit_cast(bf16x8, *(const u32x4*)(tile + (row0 + (lane & 31)) * pitch + ks * 32 + (lane >> 5) * 16));
}

// The same from a swizzled tile (row0 a multiple of 16).
template <int D>
__device__ __forceinline__ bf16x8 a_frag_swz(const unsigned char* tile, int row0, int ks, int lane) {
  const int row = row0 + (lane & 31);
  const int chunk = (2 * ks + (lane >> 5)) ^ swz<D>(row);
  return __builtin_bit_cast(bf16x8, *(const u32x4*)(tile + row * (2 * D) + chunk * 16));
}

// Transposed A operand from a swizzled tile: columns 32*dt .. +31 of the tile as rows, tile rows
// 16*j .. 16*j + 15 as the k dimension, in the row order that matches an accumulator block used
// as the B operand (see the lane layout of ds_read_b64_tr_b16 in attn_device.hpp).
template <int D>
__device__ __forceinline__ bf16x8 at_frag_swz(const unsigned char* tile, int j, int dt, int lane) {
  const int r = 16 * j + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int chunk = 4 * dt + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int byte = (lane & 1) * 8;
  const u32x2 r0 = lds_read_tr16(tile + r * (2 * D) + (chunk ^ swz<D>(r)) * 16 + byte);
  const u32x2 r1 = lds_read_tr16(tile + (r + 8) * (2 * D) + (chunk ^ swz<D>(r + 8)) * 16 + byte);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3));
}

// Accumulator block -> the two bf16 B operands of its 16-row halves.
__device__ __forceinline__ void to_b_operands(const f32x16& x, bf16x8 (&b)[2]) {
  u32x4 w[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j >> 2][j & 3] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
  b[0] = __builtin_bit_cast(bf16x8, w[0]);
  b[1] = __builtin_bit_cast(bf16x8, w[1]);
}

// The forward's row LSE (natural log) as the base-2 offset of P = exp2(c * s - lse2); a row that
// saw no key (LSE = -inf) gets +inf, so its P is exactly 0.
__device__ __forceinline__ float lse_offset(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// Store a wave's 32 x D output block, held as D/32 accumulator blocks of its transpose (lane
// column = output row, rows = output columns), scaled by `mul` and rounded to bf16, through an
// LDS scratch of 32 * (2D + 8) bytes so that each store instruction writes whole rows.  Rows
// past `nrows` are not stored.
template <int D>
__device__ __forceinline__ void store_rows_t(const f32x16 (&acc)[D / 32], float mul, unsigned char* scratch,
                                             unsigned short* out, int nrows, int lane) {
  constexpr int OPB = D * 2 + 8;
  const int h = lane >> 5, col = lane & 31;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 w = {pack_bf16x2(acc[dt][4 * g] * mul, acc[dt][4 * g + 1] * mul),
                       pack_bf16x2(acc[dt][4 * g + 2] * mul, acc[dt][4 * g + 3] * mul)};
      *(u32x2*)(scratch + col * OPB + (dt * 32 + g * 8 + h * 4) * 2) = w;
    }
  constexpr int RPI = 1024 / (D * 2);
  const int r_in = lane / (D / 8), chunk = lane % (D / 8);
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + r_in;
    const u32x4 w = *(const u32x4*)(scratch + r * OPB + chunk * 16);
    if (r < nrows) *(u32x4*)(out + (size_t)r * D + chunk * 8) = w;
  }
}

// ---------------------------------------------------------------------------------------------
// 1. D = rowsum(dO * O), fp32, for rows of two [rows, D] bf16 matrices.

template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const unsigned short* o, const unsigned short* dout,
                                                         float* dvec, int64_t rows) {
  constexpr int LPR = D / 8;        // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;    // rows per workgroup
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int part = tid % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 x = *(const u32x4*)(o + row * D + part * 8);
    const u32x4 y = *(const u32x4*)(dout + row * D + part * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(bf16_bits_to_float((unsigned short)(x[w] & 0xFFFF)), bf16_bits_to_float((unsigned short)(y[w] & 0xFFFF)), acc);
      acc = fmaf(bf16_bits_to_float((unsigned short)(x[w] >> 16)), bf16_bits_to_float((unsigned short)(y[w] >> 16)), acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) dvec[row] = acc;
}

// ---------------------------------------------------------------------------------------------
// 2. dQ.  One workgroup = 4 waves = 128 query rows of one (batch, query head); keys in tiles of BK.
// Blocks are ordered as the forward's (plan.hpp prefill_tile): heaviest query tiles first, query
// heads that share a KV head banded onto one XCD.

template <int D, int BK>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  constexpr int NB = BK / 32;
  constexpr int K_TILE = BK * C::ROWB;                  // swizzled, read both ways
  constexpr int V_TILE = round1k(BK * C::NPB);          // padded, read as the A operand
  constexpr int K_LOADS = K_TILE / 1024, V_LOADS = V_TILE / 1024;
  constexpr int KLW = (K_LOADS + 3) / 4, VLW = (V_LOADS + 3) / 4;
  constexpr int OPB = 2 * D + 8;                        // epilogue scratch pitch
  static_assert(K_TILE % 1024 == 0, "whole wave-wide loads");
  // Each stage is its own LDS object, so the compiler can see that reading one does not depend on
  // the loads still landing in the other and does not wait for them in the middle of a step.  Each
  // also holds one wave's 32 output rows for the epilogue.
  constexpr int K_BYTES = K_TILE > 32 * OPB ? K_TILE : round1k(32 * OPB);
  static_assert(V_TILE >= 32 * OPB, "a V stage holds one wave's output rows");
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds0[K_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds1[K_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds0[V_TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds1[V_TILE];
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  auto k_stage = [&](auto st) -> unsigned char* {
    if constexpr (decltype(st)::value == 0) return k_lds0;
    else return k_lds1;
  };
  auto v_stage = [&](auto st) -> unsigned char* {
    if constexpr (decltype(st)::value == 0) return v_lds0;
    else return v_lds1;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 3;
  const int h = lane >> 5, col = lane & 31;
  const PrefillTile t = prefill_tile(blockIdx.x, a.B, a.Hq, a.group, a.n_qt, a.causal, a.heads_per_xcd);
  const int b = t.b, hq = t.hq, hkv = t.hkv;
  const int q_start = t.qt * 128, w_start = q_start + wave * 32;
  const int q = w_start + col;
  const bool q_ok = q < a.Lq;

  const size_t q_off = ((size_t)(b * a.Hq + hq) * a.Lq) * D;
  const size_t kv_off = ((size_t)(b * a.Hkv + hkv) * a.Lk) * D;
  const unsigned short* Kh = (const unsigned short*)a.k + kv_off;
  const unsigned short* Vh = (const unsigned short*)a.v + kv_off;

  // Q and dO rows as B operands; this row's LSE offset and D.
  bf16x8 qf[D / 16], df[D / 16];
  {
    const unsigned short* Qr = (const unsigned short*)a.q + q_off + (size_t)(q_ok ? q : 0) * D;
    const unsigned short* Dr = (const unsigned short*)a.dout + q_off + (size_t)(q_ok ? q : 0) * D;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 wq = *(const u32x4*)(Qr + ks * 16 + h * 8);
      const u32x4 wd = *(const u32x4*)(Dr + ks * 16 + h * 8);
      qf[ks] = __builtin_bit_cast(bf16x8, q_ok ? wq : zero);
      df[ks] = __builtin_bit_cast(bf16x8, q_ok ? wd : zero);
    }
  }
  const size_t row_idx = (size_t)(b * a.Hq + hq) * a.Lq + (q_ok ? q : 0);
  const float lse2 = q_ok ? lse_offset(a.lse[row_idx]) : INFINITY;
  const float drow = q_ok ? a.dvec[row_idx] : 0.f;
  const float c = a.c2;

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

  unsigned k_voff[KLW], v_voff[VLW];
  tile_offsets_swz<D>(k_voff, wave, 4, lane, BK);
  tile_offsets(v_voff, wave, 4, lane, BK, C::NPB, C::CH, C::ROWB);
  auto issue = [&](auto st, int kt) {
    issue_loads(rows_rsrc(Kh, kt * BK, a.Lk, C::ROWB), k_stage(st), wave, 4, K_LOADS, k_voff);
    issue_loads(rows_rsrc(Vh, kt * BK, a.Lk, C::ROWB), v_stage(st), wave, 4, V_LOADS, v_voff);
  };

  const KeyRange kr = key_range(q_start, 128, a.Lq, a.Lk, BK, a.causal, a.window);
  const KeyRange wr = key_range(w_start, 32, a.Lq, a.Lk, BK, a.causal, a.window);
  const int lo = kr.kt_lo, hi = kr.kt_hi;

  auto step = [&](int kt, auto st) {
    using Cur = decltype(st);
    using Oth = std::integral_constant<int, Cur::value ^ 1>;
    if (kt + 1 <= hi) issue(Oth{}, kt + 1);
    if (kt >= wr.kt_lo && kt <= wr.kt_hi) {
      const unsigned char* Ks = k_stage(Cur{});
      const unsigned char* Vs = v_stage(Cur{});
      f32x16 x[NB], dp[NB];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) x[kb][i] = dp[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
          x[kb] = mfma_32x32x16(a_frag_swz<D>(Ks, kb * 32, ks, lane), qf[ks], x[kb]);
          dp[kb] = mfma_32x32x16(a_frag(Vs, kb * 32, C::NPB, ks, lane), df[ks], dp[kb]);
        }
      // Exponent argument c*s - lse2, masked on edge tiles (after scaling: c may be negative).
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) x[kb][i] = fmaf(x[kb][i], c, -lse2);
      const int k0 = kt * BK;
      if (!tile_full(k0, w_start, 32, a.Lq, a.Lk, BK, a.causal, a.window)) {
        int elo, ehi;
        edge_key_limits(k0, h, q, a.Lq, a.Lk, a.causal, a.window, elo, ehi);
        mask_tile(x, elo, ehi);
      }
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        f32x16 ds;
#pragma unroll
        for (int i = 0; i < 16; ++i) ds[i] = __builtin_amdgcn_exp2f(x[kb][i]) * (dp[kb][i] - drow);
        bf16x8 db[2];
        to_b_operands(ds, db);
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
            acc[dt] = mfma_32x32x16(at_frag_swz<D>(Ks, 2 * kb + half, dt, lane), db[half], acc[dt]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  if (lo <= hi) {
    issue(S0{}, lo);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = lo; kt <= hi; kt += 2) {
      step(kt, S0{});
      if (kt + 1 <= hi) step(kt + 1, S1{});
    }
  }
  // The stages are free (the last step ended with a barrier, no loads in flight): each wave
  // stages its rows in a stage of its own.
  const int nrows = a.Lq - w_start;
  unsigned char* scratch = wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1;
  if (nrows > 0)
    store_rows_t<D>(acc, a.scale, scratch, (unsigned short*)a.dq + q_off + (size_t)w_start * D, nrows, lane);
}

// ---------------------------------------------------------------------------------------------
// 3. dK and dV.  One workgroup = 4 waves = 128 keys of one (batch, KV head); a step is BQS query
// rows of one query head of the group.  Steps run over the query rows from the last down, and
// over the group's heads inside each stretch of rows, so that the workgroups of one KV head read
// the same rows at about the same time.  Blocks are ordered key tile first (the first key tiles
// see the most query rows under a causal mask: heaviest first), KV groups second; with B * Hkv
// a multiple of 8 all key tiles of a KV group run on one XCD (block index mod 8), sharing its L2.

template <int D, int BQS>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  constexpr int NQB = BQS / 32;                         // 32-row query blocks per step
  constexpr int T_TILE = BQS * C::ROWB;                 // swizzled Q or dO rows of one step
  constexpr int T_LOADS = T_TILE / 1024, TLW = (T_LOADS + 3) / 4;
  constexpr int OPB = 2 * D + 8;
  static_assert(T_TILE % 1024 == 0, "whole wave-wide loads");
  // Three stages of Q and dO rows, each its own LDS object, the stage of every step known at
  // compile time (the loop below is unrolled three times): the compiler can then see that reading
  // one stage does not depend on the loads still landing in another.  The loop is rotated so that
  // at its top no load is in flight (the compiler's record of which object a global->LDS load
  // writes does not survive the back edge): per round of three steps, the first two compute with
  // the next two steps' loads in flight, the third with the next one's.  A stage array also holds
  // one wave's 32 output rows for the epilogue.
  constexpr int ST_BYTES = T_TILE > 32 * OPB ? T_TILE : round1k(32 * OPB);
  static_assert(6 * ST_BYTES + 2 * 2 * BQS * 4 <= 65536, "the stages stay within an LDS offset's reach");
  __shared__ __attribute__((aligned(1024))) unsigned char q_lds0[ST_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char q_lds1[ST_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char q_lds2[ST_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char d_lds0[ST_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char d_lds1[ST_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char d_lds2[ST_BYTES];
  __shared__ __attribute__((aligned(16))) float row_lds[2][2][BQS];  // [step parity][lse offset, D][row]
  auto q_stage = [&](auto st_c) -> unsigned char* {
    constexpr int S = decltype(st_c)::value;
    if constexpr (S == 0) return q_lds0;
    else if constexpr (S == 1) return q_lds1;
    else return q_lds2;
  };
  auto d_stage = [&](auto st_c) -> unsigned char* {
    constexpr int S = decltype(st_c)::value;
    if constexpr (S == 0) return d_lds0;
    else if constexpr (S == 1) return d_lds1;
    else return d_lds2;
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  // Every wave issues T_LOADS / 4 loads per tile, two tiles per step.
  static_assert(T_LOADS % 4 == 0, "every wave issues the same number of loads");
  constexpr int STEP_LOADS = 2 * (T_LOADS / 4);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 3;
  const int h = lane >> 5, col = lane & 31;
  const int n_groups = a.B * a.Hkv;
  const int kt = blockIdx.x / n_groups, bkv = blockIdx.x % n_groups;
  const int b = bkv / a.Hkv, hkv = bkv % a.Hkv;
  const int k_start = kt * 128, kw = k_start + wave * 32;
  const int key = kw + col;
  const bool k_ok = key < a.Lk;
  const int delta = a.Lk - a.Lq;

  const size_t kv_off = ((size_t)(b * a.Hkv + hkv) * a.Lk) * D;
  // This wave's keys and values as B operands.
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const unsigned short* Kr = (const unsigned short*)a.k + kv_off + (size_t)(k_ok ? key : 0) * D;
    const unsigned short* Vr = (const unsigned short*)a.v + kv_off + (size_t)(k_ok ? key : 0) * D;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 wk = *(const u32x4*)(Kr + ks * 16 + h * 8);
      const u32x4 wv = *(const u32x4*)(Vr + ks * 16 + h * 8);
      kf[ks] = __builtin_bit_cast(bf16x8, k_ok ? wk : zero);
      vf[ks] = __builtin_bit_cast(bf16x8, k_ok ? wv : zero);
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[dt][i] = dv[dt][i] = 0.f;

  // Query rows that see some key of [k0, k1): i >= k0 - delta (causal), i < k1 - 1 - delta + W
  // (window), 0 <= i < Lq.
  auto q_range = [&](int k0, int k1, int& qlo, int& qhi) {
    qlo = 0;
    qhi = a.Lq;
    if (a.causal && k0 - delta > qlo) qlo = k0 - delta;
    if (a.window > 0 && k1 - 1 - delta + a.window < qhi) qhi = k1 - 1 - delta + a.window;
  };
  const int k_end = k_start + 128 < a.Lk ? k_start + 128 : a.Lk;
  int qlo, qhi;
  q_range(k_start, k_end, qlo, qhi);
  const int kw_end = kw + 32 < a.Lk ? kw + 32 : a.Lk;
  int wqlo = 0, wqhi = 0;  // this wave's query range (empty when its keys are past Lk)
  if (kw < a.Lk) q_range(kw, kw_end, wqlo, wqhi);
  // This lane's key sees queries [klo, khi] (inclusive).
  int klo = 0, khi = a.Lq - 1;
  if (a.causal && key - delta > klo) klo = key - delta;
  if (a.window > 0 && key - delta + a.window - 1 < khi) khi = key - delta + a.window - 1;
  if (!k_ok) khi = klo - 1;

  const int q0_first = qlo > 0 ? qlo / BQS * BQS : 0;
  const int n_qsteps = qhi > q0_first ? (qhi - q0_first + BQS - 1) / BQS : 0;
  const int n_steps = n_qsteps * a.group;

  unsigned t_voff[TLW];
  tile_offsets_swz<D>(t_voff, wave, 4, lane, BQS);
  // Step (qi, hd): query head hkv * group + hd, rows q_top - qi * BQS .. + BQS - 1.
  const int q_top = q0_first + (n_qsteps - 1) * BQS;
  // Row (over batch, head and position) of position 0 of the group's first query head: the rows
  // of Q, dO, the LSE and D are addressed from it with one scalar product per step.
  const int64_t grp_row0 = (int64_t)(b * a.Hq + hkv * a.group) * a.Lq;
  // Loads of step (qi, hd) into a stage.  Past the last step (`live` false) the same loads run over
  // an empty buffer and fill the stage with zeros that nothing reads, so every step issues the
  // same loads and the compiler can count them.
  auto issue = [&](auto st_c, int qi, int hd, bool live) {
    const int q0 = live ? q_top - qi * BQS : a.Lq;
    const uint64_t byte = (uint64_t)(grp_row0 + (int64_t)(live ? hd : 0) * a.Lq + q0) * C::ROWB;
    const int bytes = (a.Lq - q0 > 0 ? a.Lq - q0 : 0) * C::ROWB;
    issue_loads(__builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned char*)a.q + byte), 0, bytes, 0x00020000),
                q_stage(st_c), wave, 4, T_LOADS, t_voff);
    issue_loads(__builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned char*)a.dout + byte), 0, bytes, 0x00020000),
                d_stage(st_c), wave, 4, T_LOADS, t_voff);
  };
  // LSE offsets (threads 0 .. BQS-1) and D (threads BQS .. 2*BQS-1) of a step's rows, fetched
  // before that step's predecessor computes and written to LDS before the barrier that precedes
  // their use.  Every thread loads (clamped; the others discard theirs), and the value is
  // converted only when it is stored, so no wave waits for the load before computing.
  auto fetch_rows = [&](int qi, int hd, float& raw, bool& valid) {
    const int r = q_top - qi * BQS + (tid % BQS);
    valid = r < a.Lq && qi < n_qsteps;
    const size_t idx = (size_t)(grp_row0 + (int64_t)(qi < n_qsteps ? hd : 0) * a.Lq) + (valid ? r : 0);
    raw = (tid < BQS ? a.lse : a.dvec)[idx];
  };
  auto row_value = [&](float raw, bool valid) {
    return tid < BQS ? (valid ? lse_offset(raw) : INFINITY) : (valid ? raw : 0.f);
  };
  const float c = a.c2;

  // Steps s, s + 1 and s + 2 as (qi, hd): heads inside each stretch of rows.
  auto advance = [&](int& qi_, int& hd_) {
    if (++hd_ == a.group) {
      hd_ = 0;
      ++qi_;
    }
  };
  int qi = 0, qi1 = 0, hd1 = 0;  // (the current step's head is implicit in its stage)
  advance(qi1, hd1);
  int qi2 = qi1, hd2 = hd1;
  advance(qi2, hd2);
  // One step on stage ST: fetch the next step's rows, issue the loads given (`ahead`: how many
  // steps' loads follow it in flight when it ends), compute, wait until only those are in flight,
  // store the next step's rows, barrier.
  auto step = [&](int s, auto st_c, auto issue_c, auto ahead_c) {
    float next_raw;
    bool next_valid;
    fetch_rows(qi1, hd1, next_raw, next_valid);
    __builtin_amdgcn_sched_barrier(0);  // the row load goes out before the tile loads
    issue_c();
    const int q0 = q_top - qi * BQS;
    const unsigned char* Qs = q_stage(st_c);
    const unsigned char* Ds = d_stage(st_c);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qb0 = q0 + 32 * qb;
      if (qb0 + 32 > wqlo && qb0 < wqhi) {  // some of these rows see this wave's keys
        f32x16 x, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = dp[i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          x = mfma_32x32x16(a_frag_swz<D>(Qs, 32 * qb, ks, lane), kf[ks], x);
          dp = mfma_32x32x16(a_frag_swz<D>(Ds, 32 * qb, ks, lane), vf[ks], dp);
        }
        // Rows of the S block are queries qb0 + 8*(i/4) + 4h + i%4.
        const float* lr = row_lds[s & 1][0] + 32 * qb + 4 * h;
        const float* dr = row_lds[s & 1][1] + 32 * qb + 4 * h;
        f32x16 xs[1], dd;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 lv = *(const f32x4*)(lr + 8 * g);
          const f32x4 dv4 = *(const f32x4*)(dr + 8 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xs[0][4 * g + e] = fmaf(x[4 * g + e], c, -lv[e]);
            dd[4 * g + e] = dv4[e];
          }
        }
        const bool full = k_ok && kw_end == kw + 32 && qb0 + 32 <= a.Lq && (!a.causal || qb0 >= kw + 31 - delta) &&
                          (a.window <= 0 || qb0 + 31 <= kw - delta + a.window - 1);
        if (!full) mask_tile(xs, klo - (qb0 + 4 * h), khi - (qb0 + 4 * h));
        f32x16 p, ds;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[i] = __builtin_amdgcn_exp2f(xs[0][i]);
          ds[i] = p[i] * (dp[i] - dd[i]);
        }
        bf16x8 pb[2], db[2];
        to_b_operands(p, pb);
        to_b_operands(ds, db);
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            dv[dt] = mfma_32x32x16(at_frag_swz<D>(Ds, 2 * qb + half, dt, lane), pb[half], dv[dt]);
            dk[dt] = mfma_32x32x16(at_frag_swz<D>(Qs, 2 * qb + half, dt, lane), db[half], dk[dt]);
          }
      }
    }
    // The next step's tiles have landed (only `ahead` steps' loads may still be in flight), and
    // so has its row fetch, which was issued before them.
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(decltype(ahead_c)::value * STEP_LOADS));
    const float rv = row_value(next_raw, next_valid);
    if (tid < 2 * BQS) row_lds[(s + 1) & 1][tid / BQS][tid % BQS] = rv;
    qi = qi1;
    qi1 = qi2;
    hd1 = hd2;
    advance(qi2, hd2);
    // This wave's LDS reads of the stage and its row_lds writes are done before the others pass.
    __builtin_amdgcn_s_waitcnt(kLgkmDone);
    barrier_after_waits();
  };
  using A0 = std::integral_constant<int, 0>;
  using A1 = std::integral_constant<int, 1>;

  if (n_steps > 0) {
    issue(S0{}, 0, 0, true);
    {
      float raw;
      bool valid;
      fetch_rows(0, 0, raw, valid);
      const float rv = row_value(raw, valid);
      if (tid < 2 * BQS) row_lds[0][tid / BQS][tid % BQS] = rv;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // (qi, hd) of steps s + 1 and s + 2 are (qi1, hd1) and (qi2, hd2) at the start of step s.
    for (int s = 0; s < n_steps; s += 3) {
      // top of the round: nothing in flight; step s's tiles are in stage 0
      step(s, S0{}, [&] {
        issue(S1{}, qi1, hd1, s + 1 < n_steps);
        issue(S2{}, qi2, hd2, s + 2 < n_steps);
      }, A1{});
      if (s + 1 >= n_steps) break;
      step(s + 1, S1{}, [&] { issue(S0{}, qi2, hd2, s + 3 < n_steps); }, A1{});
      if (s + 2 >= n_steps) break;
      step(s + 2, S2{}, [] {}, A0{});
    }
    // The zero-filling loads past the last step land in stages the epilogue reuses.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  const int nrows = a.Lk - kw;
  if (nrows > 0) {
    // Wave w stages its rows in a stage of its own (all are free after the loop).
    unsigned char* scratch = wave == 0 ? q_lds0 : wave == 1 ? q_lds1 : wave == 2 ? q_lds2 : d_lds0;
    store_rows_t<D>(dk, a.scale, scratch, (unsigned short*)a.dk + kv_off + (size_t)kw * D, nrows, lane);
    store_rows_t<D>(dv, 1.f, scratch, (unsigned short*)a.dv + kv_off + (size_t)kw * D, nrows, lane);
  }
}

template __global__ void bwd_rowdot_kernel<64>(const unsigned short*, const unsigned short*, float*, int64_t);
template __global__ void bwd_rowdot_kernel<128>(const unsigned short*, const unsigned short*, float*, int64_t);
template __global__ void bwd_dq_kernel<64, 64>(BwdArgs);
template __global__ void bwd_dq_kernel<128, 32>(BwdArgs);
template __global__ void bwd_dkdv_kernel<64, kBwdQStep>(BwdArgs);
template __global__ void bwd_dkdv_kernel<128, kBwdQStep>(BwdArgs);

hipError_t launch_backward(const BwdArgs& a, int d, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Hq * a.Lq;
  const int rpb = 256 / (d / 8);
  const dim3 g1((unsigned)((rows + rpb - 1) / rpb)), blk(256);
  const dim3 g2((unsigned)((int64_t)a.n_qt * a.B * a.Hq)), g3((unsigned)((int64_t)a.n_kt * a.B * a.Hkv));
  const unsigned short* o = (const unsigned short*)a.o;
  const unsigned short* dout = (const unsigned short*)a.dout;
  if (d == 64) {
    hipLaunchKernelGGL(bwd_rowdot_kernel<64>, g1, blk, 0, stream, o, dout, a.dvec, rows);
    hipLaunchKernelGGL((bwd_dq_kernel<64, 64>), g2, blk, 0, stream, a);
    hipLaunchKernelGGL((bwd_dkdv_kernel<64, kBwdQStep>), g3, blk, 0, stream, a);
  } else {
    hipLaunchKernelGGL(bwd_rowdot_kernel<128>, g1, blk, 0, stream, o, dout, a.dvec, rows);
    hipLaunchKernelGGL((bwd_dq_kernel<128, 32>), g2, blk, 0, stream, a);
    hipLaunchKernelGGL((bwd_dkdv_kernel<128, kBwdQStep>), g3, blk, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attnfwd
