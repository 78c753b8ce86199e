// Decode attention over a pooled KV cache: one new query token per sequence, its keys and
// values read from rows offsets[s] .. offsets[s] + lens[s] - 1 of one shared pool
// ("003-注意力机制详解：从基础Attention到DeepSeek的优化策略", §三.3: one preallocated pool,
// sequences told apart by offset).  The query is the newest token, so every cached key is
// visible, or only the last W under a sliding window.
//
// The pass is bound by reading K and V once from HBM ("LLM中的Attention实现及优化": the KV
// cache makes attention memory-bound, and GQA/MQA cut its size by Hq/Hkv).  It is split over
// the key length:
//   1. decode_split_kernel: one 64-lane workgroup per (sequence, KV head, block of <= 32 query
//      heads, chunk of keys) streams the chunk in 32-key blocks and runs the online softmax of
//      the tiled algorithm ("003-…", §二) for all query heads that share the KV head at once on
//      MFMA, writing an unnormalised partial (O, m, l) in fp32.  K goes straight from memory into
//      MFMA A-operand registers (double-buffered); V goes into a two-stage LDS ring by
//      wave-wide buffer loads and comes back transposed through ds_read_b64_tr_b16.  The next
//      32-key block (16 KB at d = 128) is in flight while the current one is computed.
//   2. decode_merge_kernel: per (sequence, query head), rescales the chunk partials to a
//      common maximum and writes O (bf16) and the natural-log LSE (fp32).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "attn_device.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace attnfwd {

typedef __attribute__((address_space(3))) void lds_void_d;

template <int D>
struct DecCfg {
  static constexpr int BKD = 32;              // keys per block
  static constexpr int ROWB = D * 2;          // bytes of one head's K or V row
  static constexpr int CH = D / 8;            // 16-byte chunks per row
  static constexpr int VPB = ROWB + 64;       // V row pitch in LDS (rows 64 bytes apart mod 256)
  static constexpr int V_STAGE = BKD * VPB;   // bytes per V stage
  static constexpr int V_LOADS = V_STAGE / 1024;
  static constexpr int K_LOADS = D / 16;      // 16-byte A-operand loads per lane per block
  static_assert(V_STAGE % 1024 == 0, "a V stage must be whole wave-wide loads");
};

// s_waitcnt immediate that waits until at most n vector-memory instructions are outstanding and
// leaves the LDS/scalar and export counters unconstrained (vmcnt split over bits 3:0 and 15:14).
constexpr unsigned vmcnt_at_most(unsigned n) { return 0x0F70u | (n & 0xFu) | ((n >> 4) << 14); }

__device__ __forceinline__ bool decode_seq_valid(const DecArgs& a, int n, int64_t base) {
  return n >= 0 && n <= a.max_len && base >= 0 && base + n <= a.pool_rows;
}

// Buffer over one KV head of one sequence's keys [k0, end): view byte r * row_bytes + c is byte c
// of pool row base + k0 + r, head kvh.  Keys at or past `end` read as zeros without touching
// memory, so a block issued past the end of the chunk costs no bandwidth.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t seq_rsrc(const void* pool, int64_t base, int k0, int end, int kvh,
                                                           int Hkv, int rowb) {
  const unsigned char* p = (const unsigned char*)pool + ((size_t)(base + k0) * Hkv + kvh) * rowb;
  const int left = end - k0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, left > 0 ? ((left - 1) * Hkv + 1) * rowb : 0, 0x00020000);
}

template <int N>
__device__ __forceinline__ void load_k_block(__amdgpu_buffer_rsrc_t rs, unsigned voff, u32x4 (&dst)[N]) {
#pragma unroll
  for (int ks = 0; ks < N; ++ks) dst[ks] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + ks * 32, 0, 0);
}

template <int N>
__device__ __forceinline__ void load_v_block(__amdgpu_buffer_rsrc_t rs, unsigned char* stage,
                                             const unsigned (&voff)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_d*)(stage + j * 1024), 16, voff[j], 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(64, 2) void decode_split_kernel(DecArgs a) {
  using C = DecCfg<D>;
  constexpr int BKD = C::BKD;
  // Two V stages as separate LDS objects, so reading one does not wait for loads into the other.
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds0[C::V_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds1[C::V_STAGE];

  const int lane = threadIdx.x, h = lane >> 5, col = lane & 31;
  const int chunk = blockIdx.x, kvh = blockIdx.y / a.hblocks, hb = blockIdx.y % a.hblocks, s = blockIdx.z;
  // Scalar (wave-uniform) copies of the sequence's length and first row: the buffer descriptors
  // built from them then live in scalar registers.
  const int n = __builtin_amdgcn_readfirstlane(a.lens[s]);
  const int64_t base_raw = a.offsets[s];
  const int64_t base = (int64_t)(((uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((int)(base_raw >> 32)) << 32) |
                                 (unsigned)__builtin_amdgcn_readfirstlane((int)base_raw));
  if (!decode_seq_valid(a, n, base)) return;  // the merge pass reports the sequence as NaN
  const int lo = a.window > 0 ? (n - a.window > 0 ? n - a.window : 0) : 0;
  const int start = lo + chunk * a.chunk_keys;
  if (start >= n) return;
  const int end = start + a.chunk_keys < n ? start + a.chunk_keys : n;

  const int h0 = kvh * a.group + hb * 32;                          // first query head of this block
  const int nh = a.group - hb * 32 < 32 ? a.group - hb * 32 : 32;  // query heads in this block

  // Query heads as the B operand of S^T = K Q^T (columns beyond nh are zero).
  bf16x8 qf[D / 16];
  {
    const unsigned short* Qg = (const unsigned short*)a.q + ((size_t)s * a.Hq + h0 + col) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (col < nh) w = *(const u32x4*)(Qg + ks * 16 + h * 8);
      qf[ks] = __builtin_bit_cast(bf16x8, q_word(w, a.qmode));
    }
  }

  const int row_bytes = a.Hkv * C::ROWB;  // bytes between consecutive tokens of one head
  // K A operand: lane holds K[key = kb0 + col][16*ks + 8*h .. +7], byte col*row_bytes + 32*ks + 16*h.
  const unsigned k_voff = (unsigned)(col * row_bytes + h * 16);
  // V: wave-wide load j fills LDS bytes [j*1024, +1024) of a stage; lane slot o = j*1024 + 16*lane
  // is row o / VPB, chunk (o % VPB) / 16; pad slots take an offset past the buffer (zeros).
  unsigned v_voff[C::V_LOADS];
#pragma unroll
  for (int j = 0; j < C::V_LOADS; ++j) {
    const int o = j * 1024 + 16 * lane;
    const int row = o / C::VPB, ch = (o % C::VPB) / 16;
    v_voff[j] = ch < C::CH ? (unsigned)(row * row_bytes + ch * 16) : 0x80000000u;
  }
  // ds_read_b64_tr_b16 addressing of the V^T operand (see attn_device.hpp).
  const int v_lane = (4 * h + ((lane & 15) >> 2)) * C::VPB + ((lane >> 4) & 1) * 32 + (lane & 3) * 8;

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  RowState st = {-INFINITY, 0.f};
  const float c = a.c;

  // One 32-key block whose K is in kc and whose V is in LDS stage STAGE.
  auto block = [&](int kb0, const u32x4 (&kc)[D / 16], auto stage_c) {
    constexpr int STAGE = decltype(stage_c)::value;
    f32x16 sv[1];
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[0][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) sv[0] = mfma_32x32x16(__builtin_bit_cast(bf16x8, kc[ks]), qf[ks], sv[0]);
    if (kb0 + BKD > end) mask_tile(sv, -(1 << 30), end - 1 - (kb0 + 4 * h));  // keys at or past `end`
    const float mb = update_max(sv, st, o, c);
    unsigned pk[8];
    exp_block(sv[0], c, mb, st, pk);
    const unsigned char* Vs = (STAGE == 0 ? v_lds0 : v_lds1) + v_lane;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u32x4 pw = {pk[4 * j], pk[4 * j + 1], pk[4 * j + 2], pk[4 * j + 3]};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const u32x2 r0 = lds_read_tr16(Vs + 16 * j * C::VPB + dt * 64);
        const u32x2 r1 = lds_read_tr16(Vs + (16 * j + 8) * C::VPB + dt * 64);
        const u32x4 vw = __builtin_shufflevector(r0, r1, 0, 1, 2, 3);
        o[dt] = mfma_32x32x16(__builtin_bit_cast(bf16x8, vw), pb, o[dt]);
      }
    }
  };
  // Loads of the block starting at kb0: K into registers, V into LDS stage `stage`.
  auto issue = [&](int kb0, u32x4 (&kdst)[D / 16], auto stage_c) {
    constexpr int STAGE = decltype(stage_c)::value;
    load_k_block(seq_rsrc(a.k_pool, base, kb0, end, kvh, a.Hkv, C::ROWB), k_voff, kdst);
    load_v_block(seq_rsrc(a.v_pool, base, kb0, end, kvh, a.Hkv, C::ROWB), STAGE == 0 ? v_lds0 : v_lds1, v_voff);
  };
  // After the next block's loads are issued, wait until only they are outstanding: the current
  // block's K registers and V stage have then landed (loads complete in issue order).  The next
  // block is issued even past the chunk's end (it reads nothing there), which keeps the loop
  // free of branches around the loads.
  constexpr unsigned kWaitCurrent = vmcnt_at_most(C::K_LOADS + C::V_LOADS);

  u32x4 ka[D / 16], kb[D / 16];
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  issue(start, ka, S0{});
  for (int kb0 = start;; kb0 += 2 * BKD) {
    issue(kb0 + BKD, kb, S1{});
    __builtin_amdgcn_s_waitcnt(kWaitCurrent);
    block(kb0, ka, S0{});
    if (kb0 + BKD >= end) break;
    issue(kb0 + 2 * BKD, ka, S0{});
    __builtin_amdgcn_s_waitcnt(kWaitCurrent);
    block(kb0 + BKD, kb, S1{});
    if (kb0 + 2 * BKD >= end) break;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));  // no load may still target LDS when the wave ends

  // Partial for this chunk: unnormalised O relative to m, plus (m, l).
  const float l_tot = pair_sum(st.l);
  if (col < nh) {
    const size_t slot = ((size_t)s * a.Hq + h0 + col) * a.n_chunks + chunk;
    float* wo = a.ws + slot * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(wo + dt * 32 + g * 8 + h * 4) =
            f32x4{o[dt][4 * g], o[dt][4 * g + 1], o[dt][4 * g + 2], o[dt][4 * g + 3]};
    if (h == 0) {
      float* wml = a.ws + (size_t)a.n_seq * a.Hq * a.n_chunks * D + slot * 2;
      wml[0] = st.m;
      wml[1] = l_tot;
    }
  }
}

// One 64-lane workgroup per (sequence, query head).  Lane j reads chunk j's (m, l) (64 chunks at a
// time); the maximum and the sum of weights come from wave reductions; each lane accumulates
// D/64 output columns over the chunks, the chunk weight broadcast from the lane that holds it.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecArgs a) {
  const int hq = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const int n = a.lens[s];
  const int64_t base = a.offsets[s];
  unsigned short* O = (unsigned short*)a.o + ((size_t)s * a.Hq + hq) * D;
  constexpr int PER = D / 64;
  if (!decode_seq_valid(a, n, base)) {
    const __bf16 nanb = (__bf16)NAN;
    for (int e = 0; e < PER; ++e) O[lane * PER + e] = __builtin_bit_cast(unsigned short, nanb);
    if (a.lse != nullptr && lane == 0) a.lse[(size_t)s * a.Hq + hq] = NAN;
    return;
  }
  const int lo = a.window > 0 ? (n - a.window > 0 ? n - a.window : 0) : 0;
  const int nch = (n - lo + a.chunk_keys - 1) / a.chunk_keys;
  const size_t slot0 = ((size_t)s * a.Hq + hq) * a.n_chunks;
  const float* wml = a.ws + (size_t)a.n_seq * a.Hq * a.n_chunks * D + slot0 * 2;

  float M = -INFINITY;
  for (int j = lane; j < nch; j += 64) M = fmaxf(M, wml[2 * j]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float L = 0.f;
  if (M != -INFINITY) {
    for (int j0 = 0; j0 < nch; j0 += 64) {
      const int j = j0 + lane;
      const float w = j < nch ? __builtin_amdgcn_exp2f(wml[2 * j] - M) : 0.f;
      if (j < nch) L += w * wml[2 * j + 1];
      const int cnt = nch - j0 < 64 ? nch - j0 : 64;
      const float* wo = a.ws + (slot0 + j0) * D + lane * PER;
      for (int jj = 0; jj < cnt; ++jj) {
        const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), jj));
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += wj * wo[(size_t)jj * D + e];
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int e = 0; e < PER; ++e) O[lane * PER + e] = __builtin_bit_cast(unsigned short, (__bf16)(acc[e] * inv));
  if (a.lse != nullptr && lane == 0)
    a.lse[(size_t)s * a.Hq + hq] = L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
}

template __global__ void decode_split_kernel<64>(DecArgs);
template __global__ void decode_split_kernel<128>(DecArgs);
template __global__ void decode_merge_kernel<64>(DecArgs);
template __global__ void decode_merge_kernel<128>(DecArgs);

size_t decode_workspace_bytes(int n_seq, int Hq, int Hkv, int d, int max_len) {
  const int ck = decode_chunk_keys(n_seq, Hkv * decode_head_blocks(Hq / Hkv), max_len);
  return (size_t)n_seq * Hq * ((max_len + ck - 1) / ck) * (size_t)(d + 2) * sizeof(float);
}

hipError_t launch_decode(const DecArgs& a, int d, hipStream_t stream) {
  const dim3 g1((unsigned)a.n_chunks, (unsigned)(a.Hkv * a.hblocks), (unsigned)a.n_seq);
  const dim3 g2((unsigned)a.Hq, (unsigned)a.n_seq);
  if (d == 64) {
    hipLaunchKernelGGL(decode_split_kernel<64>, g1, dim3(64), 0, stream, a);
    hipLaunchKernelGGL(decode_merge_kernel<64>, g2, dim3(64), 0, stream, a);
  } else {
    hipLaunchKernelGGL(decode_split_kernel<128>, g1, dim3(64), 0, stream, a);
    hipLaunchKernelGGL(decode_merge_kernel<128>, g2, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attnfwd
