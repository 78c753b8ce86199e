// Host-side view of the kernels: argument blocks and launch entry points.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnfwd {

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
  int n_qt;           // query tiles per head
  int heads_per_xcd;  // > 0: XCD-banded block order (see plan.hpp)
};

struct DecArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int64_t* offsets;
  const int32_t* lens;
  void* o;
  float* lse;
  float* ws;  // per-chunk partials: O [n_seq][Hq][n_chunks][d], then (m, l) [n_seq][Hq][n_chunks][2]
  int64_t pool_rows;
  int n_seq, Hq, Hkv, group, hblocks, max_len, window, n_chunks, chunk_keys;
  float c;
  int qmode;
};

int prefill_block_q(bool f32);
int prefill_block_k(bool f32);
int prefill_threads(bool f32);
int prefill_lds_bytes(bool f32, int d);
hipError_t launch_prefill(const FwdArgs& a, bool f32, int d, hipStream_t stream);

size_t decode_workspace_bytes(int n_seq, int Hq, int Hkv, int d, int max_len);
hipError_t launch_decode(const DecArgs& a, int d, hipStream_t stream);

}  // namespace attnfwd
