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
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "attn_device.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace attnfwd {

typedef __attribute__((address_space(3))) void lds_void_d;

template <int D>
struct DecCfg {
  static constexpr int BKD = kDecodeBlockKeys;  // keys per block
  static constexpr int ROWB = D * 2;            // bytes of one head's K or V row
  static constexpr int CH = D / 8;              // 16-byte chunks per row
  static constexpr int KPB = ROWB + 16;         // K row pitch in LDS: A-operand reads of 16 rows hit distinct banks
  static constexpr int VPB = ROWB + 64;         // V row pitch: transposed reads of 4 rows hit distinct banks
  static constexpr int K_STAGE = (BKD * KPB + 1023) / 1024 * 1024;
  static constexpr int V_STAGE = BKD * VPB;
  static constexpr int K_LOADS = K_STAGE / 1024;  // wave-wide 16-byte-per-lane loads per stage
  static constexpr int V_LOADS = V_STAGE / 1024;
  static_assert(V_STAGE % 1024 == 0, "a V stage must be whole wave-wide loads");
  static_assert(K_LOADS + V_LOADS <= 63, "one block's loads must fit the vmcnt counter");
};

// s_waitcnt immediate that waits until at most n vector-memory instructions are outstanding and
// leaves the LDS/scalar and export counters unconstrained (vmcnt split over bits 3:0 and 15:14).
constexpr unsigned vmcnt_at_most(unsigned n) { return 0x0F70u | (n & 0xFu) | ((n >> 4) << 14); }

__device__ __forceinline__ bool decode_seq_valid(const DecArgs& a, int n, int64_t base) {
  return n >= 0 && n <= a.max_len && base >= 0 && base + n <= a.pool_rows;
}

// 32-key blocks of one row of sequence s; 0 for a sequence that is not read (invalid or empty).
__device__ __forceinline__ int seq_blocks(const DecArgs& a, int s) {
  const int n = a.lens[s];
  const int64_t base = a.offsets[s];
  return decode_seq_valid(a, n, base) ? decode_key_blocks(n, a.window) : 0;
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

// Buffer over one KV head of one sequence's keys [k0, end): view byte r * row_bytes + c is byte c
// of pool row base + k0 + r, head kvh.  Keys at or past `end` read as zeros without touching
// memory, so a block issued past the end of a piece costs no bandwidth.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t seq_rsrc(const void* pool, int64_t base, int k0, int end, int kvh,
                                                           int Hkv, int rowb) {
  const unsigned char* p = (const unsigned char*)pool + ((size_t)(base + k0) * Hkv + kvh) * rowb;
  const int left = end - k0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, left > 0 ? ((left - 1) * Hkv + 1) * rowb : 0, 0x00020000);
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

// Per-lane source offsets of the loads that fill a stage of `rows` rows at pitch PITCH: lane slot
// o = j*1024 + 16*lane holds row o / PITCH, chunk (o % PITCH) / 16; pad slots take an offset
// past any buffer (the hardware returns zeros and reads nothing).
template <int N, int PITCH, int CH>
__device__ __forceinline__ void stage_offsets(unsigned (&voff)[N], int lane, int rows, int row_bytes) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int o = j * 1024 + 16 * lane;
    const int row = o / PITCH, ch = (o % PITCH) / 16;
    voff[j] = (row < rows && ch < CH) ? (unsigned)(row * row_bytes + ch * 16) : 0x80000000u;
  }
}

template <int D>
__global__ __launch_bounds__(64, 2) void decode_split_kernel(DecArgs a) {
  using C = DecCfg<D>;
  constexpr int BKD = C::BKD;
  // Each pipeline stage is its own LDS object, so reading one does not wait for loads into the other.
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds0[C::K_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds1[C::K_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds0[C::V_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds1[C::V_STAGE];

  const int lane = threadIdx.x, h = lane >> 5, col = lane & 31;
  const int team = blockIdx.x / a.rows, u = blockIdx.x % a.rows;
  const int kvh = u / a.hblocks, hb = u % a.hblocks;
  const bool writer = blockIdx.x == 0;  // publishes the share and the prefix for the merge pass

  // Blocks of one row per sequence, summed over the batch; this team's share of them.
  int total = 0;
  for (int g = 0; g < a.n_seq; g += 64) {
    const int s = g + lane;
    total += wave_sum_i32(s < a.n_seq ? seq_blocks(a, s) : 0);
  }
  total = __builtin_amdgcn_readfirstlane(total);
  const int share = (total + a.teams - 1) / a.teams;
  const int start = team * share;
  const int stop = start + share < total ? start + share : total;

  // The sequence holding block `start` and the block's index in it.  The writer stores the
  // exclusive prefix of block counts on the way.
  int s_cur = -1, b_cur = 0;
  if (writer || start < stop) {
    int run = 0;
    for (int g = 0; g < a.n_seq; g += 64) {
      const int s = g + lane;
      const int nbv = s < a.n_seq ? seq_blocks(a, s) : 0;
      const int incl = wave_inclusive_scan(nbv, lane);
      const int excl = run + incl - nbv;
      if (writer && s < a.n_seq) a.ws_prefix[s] = excl;
      const uint64_t hit = __builtin_amdgcn_ballot_w64(nbv > 0 && excl <= start && start < excl + nbv);
      if (s_cur < 0 && hit != 0) {
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
  if (start >= stop || s_cur < 0) return;

  const int h0 = kvh * a.group + hb * 32;                          // first query head of this row
  const int nh = a.group - hb * 32 < 32 ? a.group - hb * 32 : 32;  // query heads in this row
  const int row_bytes = a.Hkv * C::ROWB;  // bytes between consecutive tokens of one head

  unsigned k_voff[C::K_LOADS], v_voff[C::V_LOADS];
  stage_offsets<C::K_LOADS, C::KPB, C::CH>(k_voff, lane, BKD, row_bytes);
  stage_offsets<C::V_LOADS, C::VPB, C::CH>(v_voff, lane, BKD, row_bytes);
  // K A operand: lane holds K[key = col][16*ks + 8*h .. +7] at LDS byte col*KPB + 32*ks + 16*h.
  const int k_lane = col * C::KPB + h * 16;
  // ds_read_b64_tr_b16 addressing of the V^T operand (see attn_device.hpp).
  const int v_lane = (4 * h + ((lane & 15) >> 2)) * C::VPB + ((lane >> 4) & 1) * 32 + (lane & 3) * 8;
  const float c = a.c;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // After the next block's loads are issued, wait until only they are outstanding: the current
  // block's stages have then landed (loads complete in issue order).
  constexpr unsigned kWaitCurrent = vmcnt_at_most(C::K_LOADS + C::V_LOADS);

  int pos = start, s = s_cur, b = b_cur;
  for (;;) {
    const int n = __builtin_amdgcn_readfirstlane(a.lens[s]);
    const int64_t base = uniform_i64(a.offsets[s]);
    const int nb = decode_key_blocks(n, a.window);  // > 0: the sequence holds block `pos`
    const int take = nb - b < stop - pos ? nb - b : stop - pos;
    const int lo = n - decode_visible_keys(n, a.window);
    const int k_begin = lo + b * BKD;
    const int k_end = lo + (b + take) * BKD < n ? lo + (b + take) * BKD : n;

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
    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    RowState st = {-INFINITY, 0.f};

    // Loads of the block starting at key kb0 into stage STAGE.
    auto issue = [&](int kb0, auto stage_c) {
      constexpr int STAGE = decltype(stage_c)::value;
      load_to_lds(seq_rsrc(a.k_pool, base, kb0, k_end, kvh, a.Hkv, C::ROWB), STAGE == 0 ? k_lds0 : k_lds1, k_voff);
      load_to_lds(seq_rsrc(a.v_pool, base, kb0, k_end, kvh, a.Hkv, C::ROWB), STAGE == 0 ? v_lds0 : v_lds1, v_voff);
    };
    // One 32-key block held in stage STAGE.
    auto block = [&](int kb0, auto stage_c) {
      constexpr int STAGE = decltype(stage_c)::value;
      const unsigned char* Ks = (STAGE == 0 ? k_lds0 : k_lds1) + k_lane;
      f32x16 sv[1];
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[0][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        sv[0] = mfma_32x32x16(__builtin_bit_cast(bf16x8, *(const u32x4*)(Ks + ks * 32)), qf[ks], sv[0]);
      if (kb0 + BKD > k_end) mask_tile(sv, -(1 << 30), k_end - 1 - (kb0 + 4 * h));  // keys at or past the end
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

    // The block after the current one is always issued, even past the piece's end (it then
    // reads nothing), which keeps the loop free of branches around the loads.
    issue(k_begin, S0{});
    for (int kb0 = k_begin;; kb0 += 2 * BKD) {
      issue(kb0 + BKD, S1{});
      __builtin_amdgcn_s_waitcnt(kWaitCurrent);
      block(kb0, S0{});
      if (kb0 + BKD >= k_end) break;
      issue(kb0 + 2 * BKD, S0{});
      __builtin_amdgcn_s_waitcnt(kWaitCurrent);
      block(kb0 + BKD, S1{});
      if (kb0 + 2 * BKD >= k_end) break;
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));  // no load may still target LDS past this point

    // Partial of this (team, sequence, row): unnormalised O relative to m, plus (m, l).
    const float l_tot = pair_sum(st.l);
    if (col < nh) {
      const size_t idx = ((size_t)(team + s) * a.rows + u) * a.nh + col;
      float* wo = a.ws_o + idx * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4*)(wo + dt * 32 + g * 8 + h * 4) =
              f32x4{o[dt][4 * g], o[dt][4 * g + 1], o[dt][4 * g + 2], o[dt][4 * g + 3]};
      if (h == 0) {
        a.ws_ml[2 * idx] = st.m;
        a.ws_ml[2 * idx + 1] = l_tot;
      }
    }

    pos += take;
    if (pos >= stop) break;
    // The next sequence that holds blocks starts exactly at `pos`.
    b = 0;
    do {
      ++s;
    } while (s < a.n_seq && __builtin_amdgcn_readfirstlane(seq_blocks(a, s)) == 0);
    if (s >= a.n_seq) break;
  }
}

// One 64-lane workgroup per (query head, sequence).  Lane j holds piece j's (m, l) (64 pieces at a
// time); the maximum and the sum of weights come from wave reductions; each lane accumulates
// D/64 output columns over the pieces, the piece weight broadcast from the lane that holds it.
// The partial O rows are fetched MB pieces at a time, all loads of a batch issued before any of
// them is used, so a sequence with few pieces costs about two memory round trips.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecArgs a) {
  constexpr int PER = D / 64;
  constexpr int MB = 16;
  const int hq = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const int n = a.lens[s];
  const int64_t base = a.offsets[s];
  unsigned short* O = (unsigned short*)a.o + ((size_t)s * a.Hq + hq) * D;
  if (!decode_seq_valid(a, n, base)) {
    const __bf16 nanb = (__bf16)NAN;
    for (int e = 0; e < PER; ++e) O[lane * PER + e] = __builtin_bit_cast(unsigned short, nanb);
    if (a.lse != nullptr && lane == 0) a.lse[(size_t)s * a.Hq + hq] = NAN;
    return;
  }
  const int nb = decode_key_blocks(n, a.window);
  const int kvh = hq / a.group, within = hq % a.group;
  const int u = kvh * a.hblocks + within / 32, col = within % 32;

  float M = -INFINITY, L = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  if (nb > 0) {
    const int share = a.ws_share[0];
    const int p0 = a.ws_prefix[s];
    const int t0 = p0 / share;
    const int np = (p0 + nb - 1) / share - t0 + 1;  // teams whose share meets this sequence
    // Partial index of piece j: slot (t0 + j + s) * rows + u, head col.
    const size_t idx0 = ((size_t)(t0 + s) * a.rows + u) * a.nh + col;
    const size_t step = (size_t)a.rows * a.nh;
    const float* wo0 = a.ws_o + idx0 * D + lane * PER;
    for (int j = lane; j < np; j += 64) M = fmaxf(M, a.ws_ml[2 * (idx0 + j * step)]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if (M != -INFINITY) {
      for (int j0 = 0; j0 < np; j0 += 64) {
        const int j = j0 + lane;
        float w = 0.f;
        if (j < np) {
          const size_t idx = idx0 + j * step;
          w = __builtin_amdgcn_exp2f(a.ws_ml[2 * idx] - M);
          L += w * a.ws_ml[2 * idx + 1];
        }
        const int cnt = np - j0 < 64 ? np - j0 : 64;
        for (int jb = 0; jb < cnt; jb += MB) {
          float ov[MB][PER];
#pragma unroll
          for (int jj = 0; jj < MB; ++jj)
#pragma unroll
            for (int e = 0; e < PER; ++e)
              ov[jj][e] = jb + jj < cnt ? wo0[((size_t)(j0 + jb + jj) * step) * D + e] : 0.f;
#pragma unroll
          for (int jj = 0; jj < MB; ++jj) {
            const float wj =
                __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), (jb + jj) & 63));
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] += wj * ov[jj][e];
          }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    }
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

DecWorkspaceLayout decode_workspace_layout(int n_seq, int Hq, int Hkv, int d) {
  const int group = Hq / Hkv;
  const size_t slots = (size_t)decode_max_slots(n_seq, decode_rows_per_seq(Hkv, group));
  const size_t nh = (size_t)decode_heads_per_block(group);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  DecWorkspaceLayout l;
  l.share = 0;
  l.prefix = 256;
  l.ml = l.prefix + up(sizeof(int) * ((size_t)n_seq + 1));
  l.o = l.ml + up(slots * nh * 2 * sizeof(float));
  l.total = l.o + slots * nh * (size_t)d * sizeof(float);
  return l;
}

int decode_workers(int d) {
  static std::atomic<int> cache[2][64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  std::atomic<int>& slot = cache[d == 128 ? 1 : 0][dev];
  int w = slot.load(std::memory_order_relaxed);
  if (w > 0) return w;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  const hipError_t e = d == 128 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<128>, 64, 0)
                                : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<64>, 64, 0);
  if (e != hipSuccess || cus <= 0 || per_cu <= 0) return -1;
  w = cus * per_cu < kDecodeMaxWorkers ? cus * per_cu : kDecodeMaxWorkers;
  slot.store(w, std::memory_order_relaxed);
  return w;
}

hipError_t launch_decode(const DecArgs& a, int d, hipStream_t stream) {
  const dim3 g1((unsigned)(a.teams * a.rows));
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
