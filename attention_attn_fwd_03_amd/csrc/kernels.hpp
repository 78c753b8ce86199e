// Host-side view of the kernels: argument blocks and launch entry points.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnfwd {

// Mask modes of the prefill kernels (a compile-time parameter): no mask, causal, causal with a
// sliding window.
enum MaskMode : int { kMaskNone = 0, kMaskCausal = 1, kMaskWindow = 2 };

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Lq, Lk;
  int group;          // Hq / Hkv
  int causal, window;
  float c;            // |scale| * log2(e), or 1 when scale = 0
  int qmode;          // kQAsIs, kQNegate (scale < 0) or kQZero (scale = 0): c is always > 0
  int n_qt;           // query tiles per head (ragged batches: of the longest sequence)
  int heads_per_xcd;  // > 0: XCD-banded block order (see plan.hpp)
  // Ragged batches against a pool (fwd_bf16_kernel<..., true, ...>): B is the number of sequences;
  // q and o are [total_q, Hq, d] with sequence b's rows cu_q[b] .. cu_q[b+1] - 1; k and v are the
  // pools [pool_rows, Hkv, d] with its keys at rows kv_offs[b] .. + kv_lens[b] - 1; lse is
  // [total_q, Hq].  Lq and Lk are the largest query count (max_seqlen_q) and unused.
  const int32_t* cu_q;
  const int64_t* kv_offs;
  const int32_t* kv_lens;
  int64_t total_q, pool_rows;
  // FP8 inputs (fwd_fp8_kernel): the V scale, applied to the result (the Q and K scales are folded
  // into c).
  float v_scale;
};

struct DecArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int64_t* offsets;
  const int32_t* lens;
  void* o;
  float* lse;
  // Workspace regions (see decode_workspace_layout): the blocks-per-team share, the exclusive
  // prefix of per-sequence block counts, and the partials' (m, l) and unnormalised O.
  int* ws_share;
  int* ws_prefix;
  float* ws_ml;
  float* ws_o;
  int64_t pool_rows;
  // Paged cache (paged != 0): token t of sequence s is pool row
  // block_table[s * table_stride + t / page_size] * page_size + t % page_size; offsets is unused.
  const int32_t* block_table;
  int64_t pool_pages;
  int table_stride, page_size, paged;
  int n_seq, Hq, Hkv, group, hblocks, max_len, window;
  int pack;   // KV heads per 32-row block (Hkv in the packed layout, else 1)
  int tpb;    // tokens per block: 32 / pack
  int rows;   // rows per sequence (1 in the packed layout, else Hkv * hblocks)
  int nh;     // query heads per partial slot
  int teams;  // teams of `rows` workers in the split launch
  float c;       // |scale| * log2(e) (times an fp8 pool's K scale), or 1 when scale = 0
  int qmode;
  int kv_fmt;    // pool element format: 0 bf16, 1 E4M3, 2 E5M2
  float v_scale; // fp8 pools: V scale (real value = v_scale * code value)
};

// Backward (bf16): q, o, dout, dq are [B, Hq, Lq, d]; k, v, dk, dv are [B, Hkv, Lk, d]; lse is
// the forward's natural-log row sum [B, Hq, Lq]; dvec is [B, Hq, Lq] fp32 scratch for
// D = rowsum(dO * O).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* dvec;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, Lq, Lk;
  int group;  // Hq / Hkv
  int causal, window;
  float scale;
  float c2;   // scale * log2(e), signed
  int n_qt;   // 128-row query tiles per head
  int n_kt;   // 128-row key tiles per KV head
  int heads_per_xcd;  // dQ block order, as the forward's (plan.hpp)
};


int prefill_block_q(bool f32);
int prefill_block_k(bool f32, int d);
int prefill_threads(bool f32);
int prefill_lds_bytes(bool f32, int d);
hipError_t launch_prefill(const FwdArgs& a, bool f32, int d, hipStream_t stream);
hipError_t launch_prefill_varlen(const FwdArgs& a, int d, hipStream_t stream);
hipError_t launch_prefill_fp8(const FwdArgs& a, int d, int fmt, hipStream_t stream);

// The static decode workspace of the current device (attn_decode_noalloc): its device address,
// looked up once per device, or nullptr if the runtime refuses.
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
void* decode_scratch();

// One resident round of split workers on the current device for a bf16 or fp8 pool in the packed
// or one-head block layout (plan.hpp), or < 0.
int decode_workers(int d, bool fp8, bool packed);
hipError_t launch_decode(const DecArgs& a, int d, hipStream_t stream);

hipError_t launch_backward(const BwdArgs& a, int d, hipStream_t stream);

// Matrix-core ceiling probe (probe.hip): `workgroups` workgroups of four waves, each running
// `steps` 32-key steps of the prefill loop's MFMA work (mode 0), with its LDS operand reads
// (mode 1), and with the softmax's vector work (mode 2); sink holds workgroups * 256 floats.
// Ceiling probe: mode 4 reads its tiles from the first kProbeSrcBytes of the sink (kProbeSrcBlocks
// blocks of one K and one V stage) and writes its results after them.
constexpr int kProbeSrcBlocks = 64;
constexpr size_t kProbeSrcBytes = (size_t)kProbeSrcBlocks * (9216 + 10240);
hipError_t launch_probe_mfma(int mode, int workgroups, int steps, float* sink, hipStream_t stream);

}  // namespace attnfwd
