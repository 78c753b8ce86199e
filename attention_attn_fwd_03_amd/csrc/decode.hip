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
//      heads, chunk of kDecodeChunk keys) streams the chunk in 32-key blocks, runs the
//      online softmax of the tiled algorithm ("003-…", §二) for all query heads that share the
//      KV head at once on MFMA, and writes an unnormalised partial (O, m, l) in fp32.
//   2. decode_merge_kernel: per (sequence, query head), rescales the chunk partials to a
//      common maximum and writes O (bf16) and the natural-log LSE (fp32).
#include <hip/hip_runtime.h>

#include "attn_device.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace attnfwd {

__device__ __forceinline__ bool decode_seq_valid(const DecArgs& a, int n, int64_t base) {
  return n >= 0 && n <= a.max_len && base >= 0 && base + n <= a.pool_rows;
}

template <int D>
__global__ __launch_bounds__(64) void decode_split_kernel(DecArgs a) {
  constexpr int BKD = 32;            // keys per block
  constexpr int VP = D + 32;         // LDS row pitch of V (elements)
  constexpr int CH = D / 8;          // 16-byte pieces per row
  constexpr int VPIECES = BKD * CH / 64;
  __shared__ __attribute__((aligned(16))) unsigned short vs[BKD * VP];

  const int lane = threadIdx.x, h = lane >> 5, col = lane & 31;
  const int chunk = blockIdx.x, kvh = blockIdx.y / a.hblocks, hb = blockIdx.y % a.hblocks, s = blockIdx.z;
  const int n = a.lens[s];
  const int64_t base = a.offsets[s];
  if (!decode_seq_valid(a, n, base)) return;  // the merge pass reports the sequence as NaN
  const int lo = a.window > 0 ? (n - a.window > 0 ? n - a.window : 0) : 0;
  const int start = lo + chunk * kDecodeChunk;
  if (start >= n) return;
  const int end = start + kDecodeChunk < n ? start + kDecodeChunk : n;

  const int h0 = kvh * a.group + hb * 32;                      // first query head of this block
  const int nh = a.group - hb * 32 < 32 ? a.group - hb * 32 : 32;  // query heads in this block

  // Query heads as the B operand of S^T = K Q^T (columns beyond nh are zero).
  bf16x8 qf[D / 16];
  {
    const unsigned short* Qg = (const unsigned short*)a.q + ((size_t)s * a.Hq + h0 + col) * D;
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (col < nh) w = *(const u32x4*)(Qg + ks * 16 + h * 8);
      qf[ks] = __builtin_bit_cast(bf16x8, q_word(w, a.qmode));
    }
  }

  const unsigned short* Kp = (const unsigned short*)a.k_pool;
  const unsigned short* Vp = (const unsigned short*)a.v_pool;
  const size_t row_stride = (size_t)a.Hkv * D;  // elements between consecutive pool rows
  const size_t head_off = (size_t)kvh * D;

  // K block straight into A-operand registers: lane holds K[key = kb0 + col][16*ks + 8*h ..].
  u32x4 kc[D / 16], kn[D / 16], vn[VPIECES];
  auto load_k = [&](int kb0, u32x4* dst) {
    const int key = kb0 + col;
    const bool ok = key < end;
    const unsigned short* src = Kp + (size_t)(base + (ok ? key : start)) * row_stride + head_off + h * 8;
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (ok) w = *(const u32x4*)(src + ks * 16);
      dst[ks] = w;
    }
  };
  // V block as row-major 16-byte pieces, later stored to LDS.
  auto load_v = [&](int kb0) {
    for (int i = 0; i < VPIECES; ++i) {
      const int idx = lane + 64 * i, row = idx / CH, ch = idx % CH;
      const int key = kb0 + row;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (key < end) w = *(const u32x4*)(Vp + (size_t)(base + key) * row_stride + head_off + ch * 8);
      vn[i] = w;
    }
  };
  auto store_v = [&]() {
    for (int i = 0; i < VPIECES; ++i) {
      const int idx = lane + 64 * i, row = idx / CH, ch = idx % CH;
      *(u32x4*)(vs + row * VP + ch * 8) = vn[i];
    }
  };

  f32x16 o[D / 32];
  for (int dt = 0; dt < D / 32; ++dt)
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  RowState st = {-INFINITY, 0.f};
  const float c = a.c;
  const int trG = lane >> 4, tri = lane & 15;
  const int tr_row = 4 * h + (tri >> 2);
  const int tr_col = (trG & 1) * 16 + (tri & 3) * 4;

  load_k(start, kc);
  load_v(start);
  store_v();
  __syncthreads();

  for (int kb0 = start; kb0 < end; kb0 += BKD) {
    const bool more = kb0 + BKD < end;
    if (more) {
      load_k(kb0 + BKD, kn);
      load_v(kb0 + BKD);
    }
    f32x16 sv;
    for (int i = 0; i < 16; ++i) sv[i] = 0.f;
    for (int ks = 0; ks < D / 16; ++ks) sv = mfma_32x32x16(__builtin_bit_cast(bf16x8, kc[ks]), qf[ks], sv);

    f32x16 sa[1] = {sv};
    const bool full = kb0 + BKD <= end;
    if (!full) mask_tile(sa, -(1 << 30), end - 1 - (kb0 + 4 * h));  // keys at or past `end`
    const float mb = update_max(sa, st, o, c);
    unsigned pk[8];
    exp_block(sa[0], c, mb, st, pk);
    for (int j = 0; j < 2; ++j) {
      const u32x4 pw = {pk[4 * j], pk[4 * j + 1], pk[4 * j + 2], pk[4 * j + 3]};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
      const unsigned short* vrow = vs + (16 * j + tr_row) * VP + tr_col;
      for (int dt = 0; dt < D / 32; ++dt) {
        const u32x2 r0 = lds_read_tr16(vrow + dt * 32);
        const u32x2 r1 = lds_read_tr16(vrow + 8 * VP + dt * 32);
        const u32x4 vw = {r0[0], r0[1], r1[0], r1[1]};
        o[dt] = mfma_32x32x16(__builtin_bit_cast(bf16x8, vw), pb, o[dt]);
      }
    }
    __syncthreads();
    if (more) {
      store_v();
      for (int ks = 0; ks < D / 16; ++ks) kc[ks] = kn[ks];
    }
    __syncthreads();
  }

  // Partial for this chunk: unnormalised O relative to m, plus (m, l).
  const float l_tot = pair_sum(st.l);
  if (col < nh) {
    const size_t slot = ((size_t)s * a.Hq + h0 + col) * a.n_chunks + chunk;
    float* wo = a.ws + slot * D;
    for (int dt = 0; dt < D / 32; ++dt)
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
  const int nch = (n - lo + kDecodeChunk - 1) / kDecodeChunk;
  const size_t slot0 = ((size_t)s * a.Hq + hq) * a.n_chunks;
  const float* wml = a.ws + (size_t)a.n_seq * a.Hq * a.n_chunks * D + slot0 * 2;
  float M = -INFINITY;
  for (int j = 0; j < nch; ++j) M = fmaxf(M, wml[2 * j]);
  float acc[PER];
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float L = 0.f;
  if (M != -INFINITY) {
    for (int j = 0; j < nch; ++j) {
      const float w = __builtin_amdgcn_exp2f(wml[2 * j] - M);
      L += w * wml[2 * j + 1];
      const float* wo = a.ws + (slot0 + j) * D + lane * PER;
      for (int e = 0; e < PER; ++e) acc[e] += w * wo[e];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int e = 0; e < PER; ++e) O[lane * PER + e] = __builtin_bit_cast(unsigned short, (__bf16)(acc[e] * inv));
  if (a.lse != nullptr && lane == 0)
    a.lse[(size_t)s * a.Hq + hq] = L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
}

size_t decode_workspace_bytes(int n_seq, int Hq, int d, int max_len) {
  return (size_t)n_seq * Hq * decode_num_chunks(max_len) * (size_t)(d + 2) * sizeof(float);
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
