// C ABI: argument validation, launch planning and kernel launches.  Nothing here touches the
// device before every argument has been checked.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/attn.h"
#include "../../include/attn_probe.h"
#include "kernels.hpp"
#include "plan.hpp"

using namespace attnfwd;

namespace {

constexpr float kLog2eHost = 1.4426950408889634f;

// The kernels scale scores by c = |scale| * log2(e) > 0.  A negative scale flips the sign of Q
// (exact); a zero scale zeroes Q and uses c = 1, which gives the same all-zero scores.
void set_scale(float scale, float& c, int& qmode) {
  if (scale == 0.f) {
    c = 1.f;
    qmode = 2;
  } else {
    c = std::fabs(scale) * kLog2eHost;
    qmode = scale < 0.f ? 1 : 0;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// FP8 tensor scales are folded into the kernels' score scale c in fp32 (set_scale, then c *= f);
// a product that overflows would turn every score into inf or NaN, so it is refused instead.
bool scale_folds(float scale, float f) {
  if (scale == 0.f) return true;  // run as Q = 0 with c = 1: nothing is folded
  return std::isfinite(f) && std::isfinite(std::fabs(scale) * kLog2eHost * f);
}

int check_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int Hq,
              int Hkv, int Lq, int Lk, int d, int causal, int window, float scale) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lq <= 0 || Lk <= 0 || d <= 0 || window < 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (causal != 0 && causal != 1) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (window > 0 && !causal) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_UNSUPPORTED;
  (void)lse;
  // Element offsets are computed in size_t on the device, block indices and per-head buffer
  // byte ranges in 32 bits.
  const int64_t n_qt = (Lq + 127) / 128;
  if ((int64_t)B * Hq * n_qt >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  if ((int64_t)Lk * d * 4 >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

FwdArgs make_fwd_args(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                      int Lq, int Lk, int d, int causal, int window, float scale, bool f32) {
  (void)d;
  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Lq = Lq;
  a.Lk = Lk;
  a.group = Hq / Hkv;
  a.causal = causal;
  a.window = window;
  set_scale(scale, a.c, a.qmode);
  const int bq = prefill_block_q(f32);
  a.n_qt = (Lq + bq - 1) / bq;
  a.heads_per_xcd = prefill_heads_per_xcd(B, Hq);
  return a;
}

int fwd_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Lq,
               int Lk, int d, int causal, int window, float scale, void* stream, bool f32) {
  const int st = check_fwd(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d, causal, window, scale);
  if (st != ATTN_OK) return st;
  const FwdArgs a = make_fwd_args(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d, causal, window, scale, f32);
  const hipError_t e = launch_prefill(a, f32, d, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Lq,
             int Lk, int d, int causal, int window, float scale, void* stream) {
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d, causal, window, scale, stream, false);
}

int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int Hq, int Hkv,
                 int Lq, int Lk, int d, int causal, int window, float scale, void* stream) {
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d, causal, window, scale, stream, true);
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Lq,
                 int Lk, int d, int causal, int window, float scale, int qkv_format, float q_scale, float k_scale,
                 float v_scale, void* stream) {
  const int st = check_fwd(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d, causal, window, scale);
  if (st != ATTN_OK) return st;
  if (qkv_format != ATTN_KV_E4M3 && qkv_format != ATTN_KV_E5M2) return ATTN_ERR_UNSUPPORTED;
  if (!(std::isfinite(q_scale) && q_scale > 0.f && std::isfinite(k_scale) && k_scale > 0.f &&
        std::isfinite(v_scale) && v_scale > 0.f))
    return ATTN_ERR_UNSUPPORTED;
  if (!scale_folds(scale, q_scale * k_scale)) return ATTN_ERR_UNSUPPORTED;
  FwdArgs a = make_fwd_args(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d, causal, window, scale, false);
  if (a.qmode != 2) a.c *= q_scale * k_scale;  // scores: scale * q_scale * k_scale * (q . k codes); 2: zero scale
  a.v_scale = v_scale;
  const hipError_t e = launch_prefill_fp8(a, d, qkv_format, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_varlen(const void* q, const void* k_pool, const void* v_pool, void* o, float* lse,
                    const int32_t* cu_seqlens_q, const int64_t* kv_offsets, const int32_t* kv_lens, int n_seq, int Hq,
                    int Hkv, int d, int max_seqlen_q, int64_t total_q, int64_t pool_rows, int causal, int window,
                    float scale, void* stream) {
  if (!cu_seqlens_q || !kv_offsets || !kv_lens) return ATTN_ERR_NULL;
  if (n_seq <= 0 || max_seqlen_q <= 0 || total_q < 0 || pool_rows < 0) return ATTN_ERR_SHAPE;
  // The per-sequence key counts live on the device; their tiles are addressed one BK-row buffer at
  // a time, so only the row pitch of the pool bounds the 32-bit offsets here.
  const int st = check_fwd(q, k_pool, v_pool, o, lse, n_seq, Hq, Hkv, max_seqlen_q, 1, d, causal, window, scale);
  if (st != ATTN_OK) return st;
  if ((int64_t)Hkv * d * 2 * 64 >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  if (total_q == 0) return ATTN_OK;  // no query rows: nothing to write
  FwdArgs a = make_fwd_args(q, k_pool, v_pool, o, lse, n_seq, Hq, Hkv, max_seqlen_q, 1, d, causal, window, scale,
                            false);
  a.cu_q = cu_seqlens_q;
  a.kv_offs = kv_offsets;
  a.kv_lens = kv_lens;
  a.total_q = total_q;
  a.pool_rows = pool_rows;
  const hipError_t e = launch_prefill_varlen(a, d, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t attn_decode_workspace_size(int n_seq, int Hq, int Hkv, int d, int max_len) {
  if (n_seq <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_len < 1 || (d != 64 && d != 128)) return 0;
  return decode_workspace_layout(n_seq, Hq, Hkv, d).total;
}

}  // extern "C"

namespace {

// Shared by the contiguous and the paged entry points: everything but the addressing of the pool.
// a.kv_fmt selects the pool's element format; k_scale and v_scale apply to fp8 pools only.
int decode_common(const void* q, const void* k_pool, const void* v_pool, const int32_t* lens, void* o,
                  float* lse, int n_seq, int Hq, int Hkv, int d, int max_len, int window, float scale,
                  float k_scale, float v_scale, void* workspace, size_t workspace_bytes, void* stream, DecArgs& a,
                  bool static_scratch = false) {
  if (!q || !k_pool || !v_pool || !lens || !o) return ATTN_ERR_NULL;
  if (n_seq <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || max_len < 1 || window < 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return ATTN_ERR_UNSUPPORTED;
  if (a.kv_fmt < 0 || a.kv_fmt > 2) return ATTN_ERR_UNSUPPORTED;
  if (a.kv_fmt != 0 && !(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return ATTN_ERR_UNSUPPORTED;
  if (a.kv_fmt != 0 && !scale_folds(scale, k_scale)) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o)) return ATTN_ERR_UNSUPPORTED;
  if (n_seq > 65535) return ATTN_ERR_SHAPE;
  const int group = Hq / Hkv;
  const int rows = decode_rows_per_seq(Hq, Hkv);
  const int tpb = decode_tokens_per_block(Hq, Hkv);
  if (rows > 65535) return ATTN_ERR_SHAPE;
  // one sequence's rows of one head are addressed with 32-bit byte offsets
  if ((int64_t)max_len * Hkv * d * 2 >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  // block counts summed over the batch are kept in 32 bits
  if ((int64_t)n_seq * ((max_len + tpb - 1) / tpb) >= (int64_t)1 << 30)
    return ATTN_ERR_SHAPE;
  if (a.paged && a.page_size % tpb != 0) return ATTN_ERR_UNSUPPORTED;
  const DecWorkspaceLayout lay = decode_workspace_layout(n_seq, Hq, Hkv, d);
  if (static_scratch) {  // the library's own fixed workspace (attn_decode_noalloc)
    if (lay.total > kDecodeScratchBytes) return ATTN_ERR_WORKSPACE;
    workspace = decode_scratch();
    if (workspace == nullptr) return ATTN_ERR_HIP;
    workspace_bytes = kDecodeScratchBytes;
  }
  if (workspace == nullptr || workspace_bytes < lay.total) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_UNSUPPORTED;
  const int workers = decode_workers(d, a.kv_fmt != 0, decode_pack(Hq, Hkv) > 1);
  if (workers <= 0) return ATTN_ERR_HIP;

  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.lens = lens;
  a.o = o;
  a.lse = lse;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  a.ws_share = reinterpret_cast<int*>(ws + lay.share);
  a.ws_prefix = reinterpret_cast<int*>(ws + lay.prefix);
  a.ws_ml = reinterpret_cast<float*>(ws + lay.ml);
  a.ws_o = reinterpret_cast<float*>(ws + lay.o);
  a.n_seq = n_seq;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = group;
  a.hblocks = decode_head_blocks(group);
  a.max_len = max_len;
  a.window = window;
  a.pack = decode_pack(Hq, Hkv);
  a.tpb = tpb;
  a.rows = rows;
  a.nh = decode_heads_per_slot(Hq, Hkv);
  a.teams = decode_teams(workers, rows);
  set_scale(scale, a.c, a.qmode);
  if (a.kv_fmt != 0) {
    if (a.qmode != 2) a.c *= k_scale;  // scores of an fp8 pool: scale * k_scale * (q . code values)
    a.v_scale = v_scale;
  } else {
    a.v_scale = 1.f;
  }
  const hipError_t e = launch_decode(a, d, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

int attn_decode(const void* q, const void* k_pool, const void* v_pool, const int64_t* offsets,
                const int32_t* lens, void* o, float* lse, int n_seq, int Hq, int Hkv, int d, int64_t pool_rows,
                int max_len, int window, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (!offsets) return ATTN_ERR_NULL;
  if (pool_rows < 0) return ATTN_ERR_SHAPE;
  DecArgs a{};
  a.offsets = offsets;
  a.pool_rows = pool_rows;
  a.paged = 0;
  return decode_common(q, k_pool, v_pool, lens, o, lse, n_seq, Hq, Hkv, d, max_len, window, scale, 1.f, 1.f,
                       workspace, workspace_bytes, stream, a);
}

int attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool, const int64_t* offsets,
                        const int32_t* lens, void* o, float* lse, int n_seq, int Hq, int Hkv, int d,
                        int64_t pool_rows, int max_len, int window, float scale, void* stream) {
  if (!offsets) return ATTN_ERR_NULL;
  if (pool_rows < 0) return ATTN_ERR_SHAPE;
  DecArgs a{};
  a.offsets = offsets;
  a.pool_rows = pool_rows;
  a.paged = 0;
  return decode_common(q, k_pool, v_pool, lens, o, lse, n_seq, Hq, Hkv, d, max_len, window, scale, 1.f, 1.f,
                       nullptr, 0, stream, a, true);
}

int attn_decode_fp8(const void* q, const void* k_pool, const void* v_pool, const int64_t* offsets,
                    const int32_t* lens, void* o, float* lse, int n_seq, int Hq, int Hkv, int d, int64_t pool_rows,
                    int max_len, int window, float scale, int kv_format, float k_scale, float v_scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!offsets) return ATTN_ERR_NULL;
  if (pool_rows < 0) return ATTN_ERR_SHAPE;
  if (kv_format != ATTN_KV_E4M3 && kv_format != ATTN_KV_E5M2) return ATTN_ERR_UNSUPPORTED;
  DecArgs a{};
  a.offsets = offsets;
  a.pool_rows = pool_rows;
  a.paged = 0;
  a.kv_fmt = kv_format;
  return decode_common(q, k_pool, v_pool, lens, o, lse, n_seq, Hq, Hkv, d, max_len, window, scale, k_scale,
                       v_scale, workspace, workspace_bytes, stream, a);
}

}  // extern "C"

namespace {

int decode_paged_common(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                        int table_stride, int page_size, int64_t pool_pages, const int32_t* lens, void* o, float* lse,
                        int n_seq, int Hq, int Hkv, int d, int max_len, int window, float scale, int kv_format,
                        float k_scale, float v_scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (!block_table) return ATTN_ERR_NULL;
  if (page_size < 1 || pool_pages < 0 || max_len < 1 || table_stride < 1) return ATTN_ERR_SHAPE;
  // every token a valid sequence may hold has a table entry
  if ((int64_t)table_stride < ((int64_t)max_len + page_size - 1) / page_size) return ATTN_ERR_SHAPE;
  if ((int64_t)n_seq * table_stride >= (int64_t)1 << 40) return ATTN_ERR_SHAPE;
  // one page of one head is addressed with 32-bit byte offsets
  if ((int64_t)page_size * Hkv * d * 2 >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  DecArgs a{};
  a.offsets = nullptr;
  a.block_table = block_table;
  a.table_stride = table_stride;
  a.page_size = page_size;
  a.pool_pages = pool_pages;
  a.pool_rows = pool_pages * page_size;
  a.paged = 1;
  a.kv_fmt = kv_format;
  return decode_common(q, k_pool, v_pool, lens, o, lse, n_seq, Hq, Hkv, d, max_len, window, scale, k_scale,
                       v_scale, workspace, workspace_bytes, stream, a);
}

}  // namespace

extern "C" {

int attn_decode_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                      int table_stride, int page_size, int64_t pool_pages, const int32_t* lens, void* o, float* lse,
                      int n_seq, int Hq, int Hkv, int d, int max_len, int window, float scale, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return decode_paged_common(q, k_pool, v_pool, block_table, table_stride, page_size, pool_pages, lens, o, lse,
                             n_seq, Hq, Hkv, d, max_len, window, scale, 0, 1.f, 1.f, workspace, workspace_bytes,
                             stream);
}

int attn_decode_paged_fp8(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                          int table_stride, int page_size, int64_t pool_pages, const int32_t* lens, void* o,
                          float* lse, int n_seq, int Hq, int Hkv, int d, int max_len, int window, float scale,
                          int kv_format, float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (kv_format != ATTN_KV_E4M3 && kv_format != ATTN_KV_E5M2) return ATTN_ERR_UNSUPPORTED;
  return decode_paged_common(q, k_pool, v_pool, block_table, table_stride, page_size, pool_pages, lens, o, lse,
                             n_seq, Hq, Hkv, d, max_len, window, scale, kv_format, k_scale, v_scale, workspace,
                             workspace_bytes, stream);
}

size_t attn_bwd_workspace_size(int B, int Hq, int Lq) {
  if (B <= 0 || Hq <= 0 || Lq <= 0) return 0;
  const size_t bytes = (size_t)B * Hq * Lq * sizeof(float);
  return (bytes + 255) / 256 * 256;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
             void* dk, void* dv, int B, int Hq, int Hkv, int Lq, int Lk, int d, int causal, int window, float scale,
             void* workspace, size_t workspace_bytes, void* stream) {
  if (!dout || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL;
  const int st = check_fwd(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d, causal, window, scale);
  if (st != ATTN_OK) return st;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(lse))
    return ATTN_ERR_UNSUPPORTED;
  // query rows of one head are addressed with 32-bit byte offsets; block counts fit the grid
  if ((int64_t)Lq * d * 4 >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  if ((int64_t)B * Hkv * ((Lk + 127) / 128) >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  if ((int64_t)B * Hq * Lq / 16 >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  const size_t need = attn_bwd_workspace_size(B, Hq, Lq);
  if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_UNSUPPORTED;
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dvec = static_cast<float*>(workspace);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Lq = Lq;
  a.Lk = Lk;
  a.group = Hq / Hkv;
  a.causal = causal;
  a.window = window;
  a.scale = scale;
  a.c2 = scale * kLog2eHost;
  a.n_qt = (Lq + 127) / 128;
  a.n_kt = (Lk + 127) / 128;
  a.heads_per_xcd = prefill_heads_per_xcd(B, Hq);
  const hipError_t e = launch_backward(a, d, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL: a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE: invalid size (non-positive, Hq % Hkv != 0, or too large)";
    case ATTN_ERR_UNSUPPORTED:
      return "ATTN_ERR_UNSUPPORTED: unsupported head size, window without causal, non-finite scale or "
             "misaligned pointer";
    case ATTN_ERR_WORKSPACE:
      return "ATTN_ERR_WORKSPACE: workspace missing or too small (attn_decode_noalloc: the call needs more than "
             "the library's fixed ATTN_DECODE_NOALLOC_BYTES of decode workspace)";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: kernel launch failed";
    default: return "unknown attn status";
  }
}

int attn_fwd_plan(int B, int Hq, int Hkv, int Lq, int Lk, int d, int causal, int window, int dtype_f32,
                  attn_fwd_plan_info* out) {
  static const int kDummy[4] = {0, 0, 0, 0};  // aligned stand-in pointers: validation only
  const void* p = kDummy;
  if (!out) return ATTN_ERR_NULL;
  const int st = check_fwd(p, p, p, p, nullptr, B, Hq, Hkv, Lq, Lk, d, causal, window, 1.0f);
  if (st != ATTN_OK) return st;
  const bool f32 = dtype_f32 != 0;
  const int bq = prefill_block_q(f32), bk = prefill_block_k(f32, d);
  out->block_q = bq;
  out->block_k = bk;
  out->threads = prefill_threads(f32);
  out->lds_bytes = prefill_lds_bytes(f32, d);
  out->num_q_tiles = (Lq + bq - 1) / bq;
  out->heads_per_xcd = prefill_heads_per_xcd(B, Hq);
  out->num_workgroups = (int64_t)out->num_q_tiles * B * Hq;
  int64_t tiles = 0, masked = 0;
  for (int qt = 0; qt < out->num_q_tiles; ++qt) {
    const KeyRange r = key_range(qt * bq, bq, Lq, Lk, bk, causal, window);
    for (int kt = r.kt_lo; kt <= r.kt_hi; ++kt) {
      ++tiles;
      if (!tile_full(kt * bk, qt * bq, bq, Lq, Lk, bk, causal, window)) ++masked;
    }
  }
  out->tiles_per_head = tiles;
  out->masked_tiles_per_head = masked;
  return ATTN_OK;
}

int attn_fwd_schedule(int B, int Hq, int Hkv, int Lq, int Lk, int d, int causal, int window, int dtype_f32,
                      int32_t* out, int64_t out_len) {
  attn_fwd_plan_info info;
  const int st = attn_fwd_plan(B, Hq, Hkv, Lq, Lk, d, causal, window, dtype_f32, &info);
  if (st != ATTN_OK) return st;
  if (!out) return ATTN_ERR_NULL;
  if (out_len < 3 * info.num_workgroups) return ATTN_ERR_SHAPE;
  for (int64_t bid = 0; bid < info.num_workgroups; ++bid) {
    const PrefillTile t =
        prefill_tile((int)bid, B, Hq, Hq / Hkv, info.num_q_tiles, causal, info.heads_per_xcd);
    out[3 * bid + 0] = t.b;
    out[3 * bid + 1] = t.hq;
    out[3 * bid + 2] = t.qt;
  }
  return ATTN_OK;
}

int attn_fwd_varlen_schedule(int n_seq, int Hq, int Hkv, int max_seqlen_q, int32_t* out, int64_t out_len,
                             int64_t* num_blocks) {
  if (!num_blocks) return ATTN_ERR_NULL;
  if (n_seq <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_seqlen_q <= 0) return ATTN_ERR_SHAPE;
  const int bq = prefill_block_q(false);
  const int n_qt = (max_seqlen_q + bq - 1) / bq;
  const int64_t n = prefill_grouped_blocks(n_seq, Hq, Hkv, n_qt);
  *num_blocks = n;
  if (!out) return ATTN_OK;  // size query
  if (out_len < 3 * n) return ATTN_ERR_SHAPE;
  for (int64_t bid = 0; bid < n; ++bid) {
    const PrefillTile t = prefill_tile_grouped((int)bid, n_seq, Hq, Hkv, n_qt);
    out[3 * bid + 0] = t.b;  // n_seq: a block without work
    out[3 * bid + 1] = t.hq;
    out[3 * bid + 2] = t.qt;
  }
  return ATTN_OK;
}

static_assert(ATTN_DECODE_NOALLOC_BYTES == kDecodeScratchBytes, "the header states the scratch size");

int attn_decode_rows(int Hq, int Hkv, int32_t* kv_head, int32_t* first_head, int32_t* n_heads, int64_t out_len) {
  if (!kv_head || !first_head || !n_heads) return ATTN_ERR_NULL;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  const int rows = decode_rows_per_seq(Hq, Hkv);
  if (out_len < rows) return ATTN_ERR_SHAPE;
  for (int u = 0; u < rows; ++u) {
    kv_head[u] = decode_row_kv_head(Hq, Hkv, u);
    first_head[u] = decode_row_first_head(Hq, Hkv, u);
    n_heads[u] = decode_row_heads(Hq, Hkv, u);
  }
  return ATTN_OK;
}

int attn_decode_plan(int n_seq, int Hq, int Hkv, int d, int32_t* teams, int32_t* rows_per_seq,
                     int32_t* tokens_per_block) {
  if (!teams || !rows_per_seq || !tokens_per_block) return ATTN_ERR_NULL;
  if (n_seq <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  const int workers = decode_workers(d, false, decode_pack(Hq, Hkv) > 1);
  if (workers <= 0) return ATTN_ERR_HIP;
  *rows_per_seq = decode_rows_per_seq(Hq, Hkv);
  *tokens_per_block = decode_tokens_per_block(Hq, Hkv);
  *teams = decode_teams(workers, *rows_per_seq);
  return ATTN_OK;
}

int attn_probe_mfma_ceiling(int mode, int workgroups, int steps, float* sink, size_t sink_bytes, void* stream) {
  if (!sink) return ATTN_ERR_NULL;
  if (workgroups <= 0 || steps <= 0) return ATTN_ERR_SHAPE;
  if (mode < 0 || mode > 4) return ATTN_ERR_UNSUPPORTED;
  if (sink_bytes < (size_t)workgroups * 256 * sizeof(float) + (mode == 4 ? kProbeSrcBytes : 0))
    return ATTN_ERR_WORKSPACE;
  static_assert(ATTN_PROBE_SOURCE_BYTES == kProbeSrcBytes, "header and kernel agree on the probe's source size");
  const hipError_t e = launch_probe_mfma(mode, workgroups, steps, sink, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
