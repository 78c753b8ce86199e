// Fused attention forward (prefill) over 8-bit float inputs for gfx950: Q, K and V are E4M3 or
// E5M2 codes with one scale per tensor, O (bf16) = softmax(scale * Q K^T + mask) V of the
// dequantized tensors, and the row log-sum-exp.
//
// Sources, cited by title and section: "注意力机制深度优化" (kler.cn), §一.1 runs FlashAttention
// with float8_e4m3fn tensors, and its FP8 tensor-core item with float8_e5m2; the tiled online
// softmax is that of "003-注意力机制详解：从基础Attention到DeepSeek的优化策略", §二, as in the bf16
// kernel.
//
// Design: the bf16 kernel's schedule (4 waves x 32 query rows, K/V tiles double-buffered in LDS
// by wave-wide DMA loads, per-wave tile skip and edge masking, lazy rescale, LDS-staged epilogue)
// with
//   * S^T = K Q^T on v_mfma_f32_32x32x64_f8f6f4: each lane holds 32 codes of its query row per 64
//     head dimensions (half the registers of bf16 Q) and reads 32 codes of a K row from LDS; the
//     codes enter the product unconverted, products accumulate in fp32 and the two scales are
//     folded into the score scale;
//   * P stays as in the bf16 kernel (fp32 softmax, rounded to bf16), and O^T = V^T P^T runs on
//     the bf16 MFMA: each V^T operand is one ds_read_b64_tr_b8 of the stage (rows in the order
//     fp8_v_row gives them) converted to bf16 in registers, which is exact;
//   * 64-key tiles at both head sizes: the stages take 38 KB at d = 128, as the bf16 kernel's
//     32-key tiles do, so three workgroups still share a CU.
// Quantisation of P (FP8 for both products) is not done: it would need a scaling of P that the
// pages do not give, and it changes the result beyond the bf16 bar.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "attn_device.hpp"
#include "fp8_device.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace attnfwd {

template <int D, int BK>
struct Fp8Cfg {
  static constexpr int THREADS = 256, WAVES = 4, BQ = 128, NB = BK / 32;
  static constexpr int ROWB = D;         // bytes of one row of codes
  static constexpr int CH = D / 16;      // 16-byte chunks per row
  // K: the A-operand reads of a quarter-wave (16 rows, one 16-byte chunk each) hit distinct 16-byte
  // slots of the 256-byte bank space.  V: the transposed reads of a half-wave (8 rows x 32 bytes)
  // cover it once.  Both pitches are whole chunks, as the DMA loads fill one chunk per lane.
  static constexpr int KPB = ROWB + 16, VPB = ROWB + 32;
  static constexpr int K_TILE = (BK * KPB + 1023) / 1024 * 1024, V_TILE = (BK * VPB + 1023) / 1024 * 1024;
  static constexpr int K_LOADS = K_TILE / 1024, V_LOADS = V_TILE / 1024;
  static constexpr int KL_PER_WAVE = (K_LOADS + WAVES - 1) / WAVES;
  static constexpr int VL_PER_WAVE = (V_LOADS + WAVES - 1) / WAVES;
  static constexpr int OPB = D * 2 + 8;  // LDS row pitch of the staged bf16 O tile
  static_assert(BK % 32 == 0 && D % 64 == 0, "64-dimension MFMA steps and 32-key blocks");
};

template <int D, int BK, int FMT>
__global__ __launch_bounds__(256, 3) void fwd_fp8_kernel(FwdArgs a) {
  using C = Fp8Cfg<D, BK>;
  constexpr int NB = C::NB;
  constexpr int KS = D / 64;  // MFMA steps over the head dimension
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (C::WAVES - 1);
  const int h = lane >> 5, col = lane & 31;
  const PrefillTile t = prefill_tile(blockIdx.x, a.B, a.Hq, a.group, a.n_qt, a.causal, a.heads_per_xcd);
  const int q_start = t.qt * C::BQ;
  const int q = q_start + wave * 32 + col;

  const unsigned char* Qg = (const unsigned char*)a.q + ((size_t)(t.b * a.Hq + t.hq) * a.Lq) * D;
  const size_t kv_off = ((size_t)(t.b * a.Hkv + t.hkv) * a.Lk) * D;
  const unsigned short* Kh = (const unsigned short*)((const unsigned char*)a.k + kv_off);
  const unsigned short* Vh = (const unsigned short*)((const unsigned char*)a.v + kv_off);
  const KeyRange kr = key_range(q_start, C::BQ, a.Lq, a.Lk, BK, a.causal, a.window);

  // Q as the B operand: for step ks the lane holds codes 64*ks + 32*h .. +31 of its row; a
  // negative scale flips every code's sign bit, a zero scale (or a row past Lq) zeroes them.
  i32x8 qf[KS];
  {
    const bool q_ok = q < a.Lq;
    const unsigned keep = (q_ok && a.qmode != kQZero) ? 0xFFFFFFFFu : 0u;
    const unsigned flip = (q_ok && a.qmode == kQNegate) ? 0x80808080u : 0u;
    const unsigned char* Qr = Qg + (size_t)(q_ok ? q : 0) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 w0 = *(const u32x4*)(Qr + ks * 64 + h * 32);
      const u32x4 w1 = *(const u32x4*)(Qr + ks * 64 + h * 32 + 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[ks][e] = (int)((w0[e] & keep) ^ flip);
        qf[ks][4 + e] = (int)((w1[e] & keep) ^ flip);
      }
    }
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  RowState st = {-INFINITY, 0.f, 0.f};
  const float c = a.c;

  // Global -> LDS, as the bf16 kernel: wave-wide load j writes 16 bytes per lane at j*1024 +
  // 16*lane of the stage, which is row o / pitch, chunk (o % pitch) / 16; V rows in fp8_v_row order.
  constexpr unsigned kPastEnd = 0x80000000u;
  unsigned k_voff[C::KL_PER_WAVE], v_voff[C::VL_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::KL_PER_WAVE; ++i) {
    const int o = (wave + C::WAVES * i) * 1024 + 16 * lane;
    const int row = o / C::KPB, chunk = (o % C::KPB) / 16;
    k_voff[i] = (row < BK && chunk < C::CH) ? (unsigned)(row * C::ROWB + chunk * 16) : kPastEnd;
  }
#pragma unroll
  for (int i = 0; i < C::VL_PER_WAVE; ++i) {
    const int o = (wave + C::WAVES * i) * 1024 + 16 * lane;
    const int row = o / C::VPB, chunk = (o % C::VPB) / 16;
    v_voff[i] = (row < BK && chunk < C::CH) ? (unsigned)(fp8_v_row(row) * C::ROWB + chunk * 16) : kPastEnd;
  }
  auto issue = [&](auto st_c, int kt) {
    issue_loads(rows_rsrc(Kh, kt * BK, a.Lk, C::ROWB), k_stage(st_c), wave, C::WAVES, C::K_LOADS, k_voff);
    issue_loads(rows_rsrc(Vh, kt * BK, a.Lk, C::ROWB), v_stage(st_c), wave, C::WAVES, C::V_LOADS, v_voff);
  };

  // K reads: lane reads row 32*kb + col, codes 64*ks + 32*h .. +31.
  const int k_lane = col * C::KPB + h * 32;
  auto qk = [&](auto st_c, f32x16 (&s)[NB]) {
    const unsigned char* Ks = k_stage(st_c) + k_lane;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        const u32x4 w0 = *(const u32x4*)(Ks + kb * 32 * C::KPB + ks * 64);
        const u32x4 w1 = *(const u32x4*)(Ks + kb * 32 * C::KPB + ks * 64 + 16);
        const i32x8 kf = {(int)w0[0], (int)w0[1], (int)w0[2], (int)w0[3],
                          (int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
        s[kb] = mfma_32x32x64_f8<FMT>(kf, qf[ks], s[kb]);
      }
  };
  // V^T operand: group g = lane/16 reads rows 8*(g/2) .. +7 and bytes 16*(g%2) .. +15 of a
  // 32-column slice; lane l receives stage rows 16*j + 8*h .. +7 of column 32*dt + l%32.
  const int v_lane = (8 * h + ((lane & 15) >> 1)) * C::VPB + ((lane >> 4) & 1) * 16 + (lane & 1) * 8;
  auto pv = [&](auto st_c, int kb, const u32x4 (&pw)[2]) {
    const unsigned char* Vs = v_stage(st_c) + v_lane;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int j = 2 * kb + half;
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw[half]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        o[dt] = mfma_32x32x16(fp8x8_to_bf16<FMT>(lds_read_tr8(Vs + 16 * j * C::VPB + dt * 32)), pb, o[dt]);
    }
  };
  const int lo = kr.kt_lo, hi = kr.kt_hi;
  const int w_start = q_start + wave * 32;
  const KeyRange wkr = key_range(w_start, 32, a.Lq, a.Lk, BK, a.causal, a.window);
  const int w_lo = wkr.kt_lo, w_hi = wkr.kt_hi;
  auto step = [&](int kt, auto stage_c) {
    constexpr int STAGE = decltype(stage_c)::value;
    using Cur = std::integral_constant<int, STAGE>;
    using Oth = std::integral_constant<int, STAGE ^ 1>;
    if (kt + 1 <= hi) issue(Oth{}, kt + 1);
    if (kt >= w_lo && kt <= w_hi) {
      f32x16 sc[NB];
      qk(Cur{}, sc);
      const int k0 = kt * BK;
      if (!tile_full(k0, w_start, 32, a.Lq, a.Lk, BK, a.causal, a.window)) {
        int elo, ehi;
        edge_key_limits(k0, h, q, a.Lq, a.Lk, a.causal, a.window, elo, ehi);
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

  // ---- epilogue: O = v_scale * acc / l (bf16), LSE in natural log; O staged through LDS ----
  const float l_tot = pair_sum(st.l);
  const float inv = l_tot > 0.f ? a.v_scale / l_tot : 0.f;
  constexpr int OPB = C::OPB;
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
  constexpr int RPI = 1024 / (D * 2);
  const int r_in = lane / (D / 8), chunk = lane % (D / 8);
  unsigned short* Oh = (unsigned short*)a.o + ((size_t)(t.b * a.Hq + t.hq) * a.Lq) * D;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + r_in;
    const u32x4 w = *(const u32x4*)(ot + r * OPB + chunk * 16);
    const int qr = w_start + r;
    if (qr < a.Lq) *(u32x4*)(Oh + (size_t)qr * D + chunk * 8) = w;
  }
  if (a.lse != nullptr && h == 0 && q < a.Lq)
    a.lse[(size_t)(t.b * a.Hq + t.hq) * a.Lq + q] =
        l_tot > 0.f ? (st.m + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
}

template __global__ void fwd_fp8_kernel<64, 64, kKvE4M3>(FwdArgs);
template __global__ void fwd_fp8_kernel<128, 64, kKvE4M3>(FwdArgs);
template __global__ void fwd_fp8_kernel<64, 64, kKvE5M2>(FwdArgs);
template __global__ void fwd_fp8_kernel<128, 64, kKvE5M2>(FwdArgs);

hipError_t launch_prefill_fp8(const FwdArgs& a, int d, int fmt, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.n_qt * a.B * a.Hq)), block(256);
  if (d == 64) {
    if (fmt == kKvE4M3) hipLaunchKernelGGL((fwd_fp8_kernel<64, 64, kKvE4M3>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((fwd_fp8_kernel<64, 64, kKvE5M2>), grid, block, 0, stream, a);
  } else {
    if (fmt == kKvE4M3) hipLaunchKernelGGL((fwd_fp8_kernel<128, 64, kKvE4M3>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((fwd_fp8_kernel<128, 64, kKvE5M2>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attnfwd
