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
// Design (one workgroup = 4 waves = 128 query rows of one (batch, query head)):
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

#include "attn_device.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace attnfwd {

template <int D, int BK>
struct Bf16Cfg {
  static constexpr int THREADS = 256, BQ = 128, NB = BK / 32;
  static constexpr int KP = D + 8;    // K row pitch (elements): rows land 16 bytes apart mod 256
  static constexpr int VP = D + 32;   // V row pitch (elements): rows land 64 bytes apart mod 256
  static constexpr int K_ELEMS = BK * KP, V_ELEMS = BK * VP, STAGE = K_ELEMS + V_ELEMS;
  static constexpr int CHUNKS = D / 8;                   // 16-byte pieces per row
  static constexpr int LOADS = BK * CHUNKS / THREADS;    // pieces per thread per tensor
  static_assert(BK * CHUNKS % THREADS == 0, "tile must split evenly over the threads");
};

template <int D, int BK>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a) {
  using C = Bf16Cfg<D, BK>;
  __shared__ __attribute__((aligned(16))) unsigned short smem[2 * C::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const PrefillTile t = prefill_tile(blockIdx.x, a.B, a.Hq, a.group, a.n_qt, a.causal, a.heads_per_xcd);
  const int q_start = t.qt * C::BQ;
  const int q = q_start + wave * 32 + col;  // query row of this lane
  const KeyRange kr = key_range(q_start, C::BQ, a.Lq, a.Lk, BK, a.causal, a.window);

  const unsigned short* Qg = (const unsigned short*)a.q + ((size_t)(t.b * a.Hq + t.hq) * a.Lq) * D;
  const unsigned short* Kg = (const unsigned short*)a.k + ((size_t)(t.b * a.Hkv + t.hkv) * a.Lk) * D;
  const unsigned short* Vg = (const unsigned short*)a.v + ((size_t)(t.b * a.Hkv + t.hkv) * a.Lk) * D;

  // Q rows as the B operand: lane holds Q[q][16*ks + 8*h .. +7] for every ks.
  bf16x8 qf[D / 16];
  {
    const unsigned flip = a.negate ? 0x80008000u : 0u;  // negative scale: flip the sign of Q exactly
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (q < a.Lq) w = *(const u32x4*)(Qg + (size_t)q * D + ks * 16 + h * 8);
      w ^= flip;
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x16 o[D / 32];
  for (int dt = 0; dt < D / 32; ++dt)
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  RowState st = {-INFINITY, 0.f};

  u32x4 kreg[C::LOADS], vreg[C::LOADS];
  auto load_tile = [&](int kt) {
    const int k0 = kt * BK;
    for (int i = 0; i < C::LOADS; ++i) {
      const int idx = tid + i * C::THREADS;
      const int row = idx / C::CHUNKS, ch = idx % C::CHUNKS;
      const int key = k0 + row;
      if (key < a.Lk) {
        kreg[i] = *(const u32x4*)(Kg + (size_t)key * D + ch * 8);
        vreg[i] = *(const u32x4*)(Vg + (size_t)key * D + ch * 8);
      } else {
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int stage) {
    unsigned short* Ks = smem + stage * C::STAGE;
    unsigned short* Vs = Ks + C::K_ELEMS;
    for (int i = 0; i < C::LOADS; ++i) {
      const int idx = tid + i * C::THREADS;
      const int row = idx / C::CHUNKS, ch = idx % C::CHUNKS;
      *(u32x4*)(Ks + row * C::KP + ch * 8) = kreg[i];
      *(u32x4*)(Vs + row * C::VP + ch * 8) = vreg[i];
    }
  };

  if (kr.kt_lo <= kr.kt_hi) {
    load_tile(kr.kt_lo);
    store_tile(0);
    __syncthreads();
  }
  const float c = a.c;
  // ds_read_b64_tr_b16 addressing for the V^T operand (see attn_device.hpp): 16-lane group G
  // covers columns 16*(G%2) .. +15 of a 32-column block, half-wave h covers keys 4h.. of each
  // 8-key group.
  const int trG = lane >> 4, tri = lane & 15;
  const int tr_row = 4 * h + (tri >> 2);
  const int tr_col = (trG & 1) * 16 + (tri & 3) * 4;

  for (int kt = kr.kt_lo; kt <= kr.kt_hi; ++kt) {
    const int stage = (kt - kr.kt_lo) & 1;
    const bool more = kt < kr.kt_hi;
    if (more) load_tile(kt + 1);

    const unsigned short* Ks = smem + stage * C::STAGE;
    const unsigned short* Vs = Ks + C::K_ELEMS;
    const int k0 = kt * BK;

    // ---- S^T = K Q^T (fp32 accumulate); scale is applied later, in fp32 ----
    f32x16 s[C::NB];
    for (int kb = 0; kb < C::NB; ++kb)
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
    for (int ks = 0; ks < D / 16; ++ks) {
      for (int kb = 0; kb < C::NB; ++kb) {
        const bf16x8 kf = *(const bf16x8*)(Ks + (kb * 32 + col) * C::KP + ks * 16 + h * 8);
        s[kb] = mfma_32x32x16(kf, qf[ks], s[kb]);
      }
    }

    // ---- mask (only tiles that straddle a boundary) ----
    const bool edge = !tile_full(k0, q_start, C::BQ, a.Lq, a.Lk, BK, a.causal, a.window);
    if (edge) {
      for (int kb = 0; kb < C::NB; ++kb)
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
          if (!visible(key, q, a.Lq, a.Lk, a.causal, a.window)) s[kb][i] = -INFINITY;
        }
    }

    // ---- online softmax ([DS-Attn §二]) with a lazily raised reference maximum ----
    float mx = -INFINITY;
    for (int kb = 0; kb < C::NB; ++kb)
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = pair_max(mx);
    const float tmax = (mx == -INFINITY) ? -INFINITY : mx * c;
    const bool need = tmax > st.m + kRescaleSlack;
    if (wave_any(need)) {
      const float m_new = need ? tmax : st.m;
      const float alpha = need ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.f;
      st.l *= alpha;
      for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
      st.m = m_new;
    }
    const float mb = (st.m == -INFINITY) ? 0.f : st.m;

    // P = exp2(S * c - m), rounded to bf16 for the MFMA; the row sum takes the fp32 values so
    // that the LSE keeps fp32 accuracy.
    unsigned pk[C::NB * 8];
    float lsum = 0.f;
    for (int kb = 0; kb < C::NB; ++kb) {
      for (int pi = 0; pi < 8; ++pi) {
        const float s0 = s[kb][2 * pi], s1 = s[kb][2 * pi + 1];
        float p0 = __builtin_amdgcn_exp2f(fmaf(s0, c, -mb));
        float p1 = __builtin_amdgcn_exp2f(fmaf(s1, c, -mb));
        if (edge) {
          p0 = (s0 == -INFINITY) ? 0.f : p0;
          p1 = (s1 == -INFINITY) ? 0.f : p1;
        }
        pk[kb * 8 + pi] = pack_bf16x2(p0, p1);
        lsum += p0 + p1;
      }
    }
    st.l += lsum;

    // ---- O^T += V^T P^T ----
    for (int j = 0; j < BK / 16; ++j) {
      const int kb = j >> 1, half = j & 1;
      const u32x4 pw = {pk[kb * 8 + half * 4 + 0], pk[kb * 8 + half * 4 + 1], pk[kb * 8 + half * 4 + 2],
                        pk[kb * 8 + half * 4 + 3]};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
      const unsigned short* vrow = Vs + (16 * j + tr_row) * C::VP + tr_col;
      for (int dt = 0; dt < D / 32; ++dt) {
        const u32x2 r0 = lds_read_tr16(vrow + dt * 32);
        const u32x2 r1 = lds_read_tr16(vrow + 8 * C::VP + dt * 32);
        const u32x4 vw = {r0[0], r0[1], r1[0], r1[1]};
        o[dt] = mfma_32x32x16(__builtin_bit_cast(bf16x8, vw), pb, o[dt]);
      }
    }

    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l (bf16, round to nearest even), LSE in natural log ----
  const float l_tot = pair_sum(st.l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q < a.Lq) {
    unsigned short* Og = (unsigned short*)a.o + ((size_t)(t.b * a.Hq + t.hq) * a.Lq + q) * D;
    for (int dt = 0; dt < D / 32; ++dt)
      for (int g = 0; g < 4; ++g) {
        const u32x2 w = {pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                         pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv)};
        *(u32x2*)(Og + dt * 32 + g * 8 + h * 4) = w;
      }
    if (a.lse != nullptr && h == 0)
      a.lse[(size_t)(t.b * a.Hq + t.hq) * a.Lq + q] =
          l_tot > 0.f ? (st.m + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
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
    const float sgn = a.negate ? -1.f : 1.f;
    for (int ks2 = 0; ks2 < D / 4; ++ks2) {
      float2 w = make_float2(0.f, 0.f);
      if (q < a.Lq) w = *(const float2*)(Qg + (size_t)q * D + 4 * ks2 + 2 * h);
      qf[2 * ks2] = w.x * sgn;
      qf[2 * ks2 + 1] = w.y * sgn;
    }
  }

  f32x16 o[D / 32];
  for (int dt = 0; dt < D / 32; ++dt)
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  RowState st = {-INFINITY, 0.f};

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

    f32x16 s;
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
    for (int ks2 = 0; ks2 < D / 4; ++ks2) {
      const float2 kf = *(const float2*)(Ks + col * C::KP + 4 * ks2 + 2 * h);
      s = mfma_32x32x2(kf.x, qf[2 * ks2], s);
      s = mfma_32x32x2(kf.y, qf[2 * ks2 + 1], s);
    }

    const bool edge = !tile_full(k0, q_start, C::BQ, a.Lq, a.Lk, BK, a.causal, a.window);
    if (edge) {
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + (i >> 2) * 8 + h * 4 + (i & 3);
        if (!visible(key, q, a.Lq, a.Lk, a.causal, a.window)) s[i] = -INFINITY;
      }
    }
    float mx = -INFINITY;
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = pair_max(mx);
    const float tmax = (mx == -INFINITY) ? -INFINITY : mx * c;
    const bool need = tmax > st.m + kRescaleSlack;
    if (wave_any(need)) {
      const float m_new = need ? tmax : st.m;
      const float alpha = need ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.f;
      st.l *= alpha;
      for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
      st.m = m_new;
    }
    const float mb = (st.m == -INFINITY) ? 0.f : st.m;
    float p[16];
    for (int i = 0; i < 16; ++i) {
      float pi = __builtin_amdgcn_exp2f(fmaf(s[i], c, -mb));
      if (edge) pi = (s[i] == -INFINITY) ? 0.f : pi;
      p[i] = pi;
      st.l += pi;
    }
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

int prefill_block_q(bool f32) { return f32 ? F32Cfg<64>::BQ : Bf16Cfg<128, 64>::BQ; }
int prefill_block_k(bool f32) { return f32 ? F32Cfg<64>::BK : 64; }
int prefill_threads(bool) { return 256; }
int prefill_lds_bytes(bool f32, int d) {
  if (f32) return d == 64 ? 2 * F32Cfg<64>::STAGE * 4 : 2 * F32Cfg<128>::STAGE * 4;
  return d == 64 ? 2 * Bf16Cfg<64, 64>::STAGE * 2 : 2 * Bf16Cfg<128, 64>::STAGE * 2;
}

hipError_t launch_prefill(const FwdArgs& a, bool f32, int d, hipStream_t stream) {
  const int64_t grid = (int64_t)a.n_qt * a.B * a.Hq;
  const dim3 g((unsigned)grid), b(256);
  if (f32) {
    if (d == 64) hipLaunchKernelGGL(fwd_f32_kernel<64>, g, b, 0, stream, a);
    else hipLaunchKernelGGL(fwd_f32_kernel<128>, g, b, 0, stream, a);
  } else {
    if (d == 64) hipLaunchKernelGGL((fwd_bf16_kernel<64, 64>), g, b, 0, stream, a);
    else hipLaunchKernelGGL((fwd_bf16_kernel<128, 64>), g, b, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attnfwd
