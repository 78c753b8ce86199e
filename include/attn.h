/* attnfwd — fused exact attention forward and pooled-KV decode for AMD MI355X (gfx950).
 *
 * Computes O = softmax(scale * Q K^T + mask) V and the row log-sum-exp without writing the
 * score matrix to memory.  The operation is the plain scaled dot-product attention of
 * "003-注意力机制详解：从基础Attention到DeepSeek的优化策略" (§一), evaluated with the tiled
 * online softmax of its §二, with:
 *   - GQA / MQA: query head h reads KV head h / (Hq / Hkv), i.e. consecutive query heads share
 *     a KV head, as repeat_kv expands them in "LLM中的Attention实现及优化" — without copying;
 *     Hq must be a multiple of Hkv (the tqpw.cn MQA/GQA article, §3.1, asserts h % g == 0);
 *   - causal masking ("注意力机制深度优化", §一.2), aligned bottom-right when Lq != Lk: query row
 *     i sits at position i + (Lk - Lq) and sees keys j <= i + (Lk - Lq);
 *   - a sliding window of W ("LLM中的Attention实现及优化": each token sees at most the previous
 *     W tokens), read as the W most recent positions counting the query's own;
 *   - decode against a KV cache pool shared by many sequences and addressed by offsets
 *     ("003-注意力机制详解…", §三.3).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, 16-byte aligned, row-major
 *     and contiguous.  The library allocates nothing and frees nothing; besides its kernel code
 *     it keeps only the decode worker count of each device, computed on first use from the
 *     occupancy query and read-only afterwards.  Inputs are not modified; outputs must not
 *     alias inputs.
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the default stream) and return
 *     without synchronising.  Argument errors are detected on the host, before any device work,
 *     and returned as a status.  Device faults surface at the caller's next synchronisation.
 *     A call only launches kernels on `stream` (no copies, memsets or allocations), so it may be
 *     captured into a HIP graph and replayed; sizes and pointers are fixed at capture, while the
 *     contents of device arrays (lens, offsets, block tables, q, ...) are read at each replay.
 *   - scale is explicit (1/sqrt(d) is the usual choice); any finite value, including 0 and
 *     negative values, is accepted.
 *   - A query row that sees no key gets O = 0 and LSE = -inf.  NaN/Inf inputs propagate.
 *   - Head dimension d must be 64 or 128.
 */
#ifndef ATTNFWD_ATTN_H
#define ATTNFWD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* a size <= 0 (n_seq may not be 0 either), Hq % Hkv != 0, window < 0,
                               max_len < 1, pool_rows < 0, or a size too large to index (per head,
                               Lk*d*4 and max_len*Hkv*d*2 must stay below 2^31 bytes) */
  ATTN_ERR_UNSUPPORTED = 3, /* d not in {64, 128}; window > 0 without causal; scale not finite;
                               a pointer not 16-byte aligned; an unknown FP8 format, an FP8
                               tensor scale that is not finite and > 0, or FP8 scales whose
                               product with |scale| * log2(e) overflows fp32 (they are folded
                               into the score scale) */
  ATTN_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than attn_decode_workspace_size / attn_bwd_workspace_size */
  ATTN_ERR_HIP = 5          /* the HIP runtime refused a launch */
} attn_status;

/* Element formats of an FP8 KV cache (attn_decode_fp8, attn_decode_paged_fp8): the OCP 8-bit
 * floating point formats that "注意力机制深度优化" (§一.1 and its FP8 tensor-core item) loads
 * models in, torch.float8_e4m3fn and torch.float8_e5m2. */
typedef enum {
  ATTN_KV_E4M3 = 1,  /* 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities, max 448 */
  ATTN_KV_E5M2 = 2   /* 1 sign, 5 exponent (bias 15), 2 mantissa bits; IEEE-style inf / NaN */
} attn_kv_format;

/* Prefill / full attention, bfloat16 tensors (uint16 storage, round-to-nearest-even results).
 *   q [B, Hq, Lq, d], k and v [B, Hkv, Lk, d], o [B, Hq, Lq, d]  (bf16)
 *   lse [B, Hq, Lq] fp32, natural log; may be NULL (not written).
 *   causal: 0 or 1.  window: 0 = none, W > 0 keeps keys p - W < j <= p (requires causal).
 * Scores and the softmax are fp32; probabilities are rounded to bf16 for the P.V product,
 * which accumulates in fp32 ("003-注意力机制详解…", §三.1 mixed precision). */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Lq, int Lk, int d,
             int causal, int window, float scale, void* stream);

/* Same as attn_fwd with fp32 tensors throughout (q, k, v, o are float*). */
int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                 int B, int Hq, int Hkv, int Lq, int Lk, int d,
                 int causal, int window, float scale, void* stream);

/* attn_fwd over 8-bit float inputs ("注意力机制深度优化" §一.1 runs FlashAttention on float8_e4m3fn
 * tensors, its FP8 tensor-core item on float8_e5m2): q [B, Hq, Lq, d], k and v [B, Hkv, Lk, d] hold
 * codes of format qkv_format (attn_kv_format, one byte per element), with one scale per tensor
 * (real value = scale * code value; finite and > 0).  o [B, Hq, Lq, d] is bf16, lse as attn_fwd.
 * S = Q K^T runs on the FP8 matrix cores (v_mfma_f32_32x32x64_f8f6f4, fp32 accumulation, the Q and
 * K scales folded into the score scale); the softmax is fp32, P is rounded to bf16 and P V runs on
 * the bf16 matrix cores with V's codes converted exactly.  The result is attn_fwd's arithmetic on
 * the dequantized tensors.  Masking, scale, rules and status codes as attn_fwd. */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Lq, int Lk, int d, int causal, int window, float scale,
                 int qkv_format, float q_scale, float k_scale, float v_scale, void* stream);

/* Ragged prefill against a pooled KV cache (continuous batching: "注意力机制深度优化" §二.1;
 * variable-length sequences processed in chunks against their history: "高效多头潜在注意力解码技术：
 * Flash MLA深度解析" §一, §2.2).  bf16.
 *   q, o [total_q, Hq, d]: rows cu_seqlens_q[s] .. cu_seqlens_q[s+1] - 1 are the Lq_s new tokens
 *   of sequence s (cu_seqlens_q[n_seq + 1] int32, device memory).
 *   k_pool, v_pool [pool_rows, Hkv, d]: sequence s's Lk_s = kv_lens[s] keys are pool rows
 *   kv_offsets[s] .. kv_offsets[s] + Lk_s - 1 (int64 / int32 arrays in device memory); they
 *   include the new tokens' own keys, last.
 *   Query i of sequence s sits at position i + Lk_s - Lq_s (bottom-right, as in attn_fwd), so a
 *   chunk of new tokens sees the whole cache and, with causal, the new tokens before it.
 *   lse [total_q, Hq] fp32, natural log; may be NULL.  max_seqlen_q >= every Lq_s sizes the grid.
 * Sequences are checked on the device: one with cu_seqlens_q[s] > cu_seqlens_q[s+1], a row past
 * total_q, Lq_s > max_seqlen_q, kv_lens < 0, kv_offsets < 0 or offsets + lens > pool_rows is not
 * read; its rows (when its query range lies inside [0, total_q]) are set to NaN.  Other rules
 * and status codes as attn_fwd; total_q = 0 returns ATTN_OK without device work. */
int attn_fwd_varlen(const void* q, const void* k_pool, const void* v_pool, void* o, float* lse,
                    const int32_t* cu_seqlens_q, const int64_t* kv_offsets, const int32_t* kv_lens,
                    int n_seq, int Hq, int Hkv, int d, int max_seqlen_q, int64_t total_q, int64_t pool_rows,
                    int causal, int window, float scale, void* stream);

/* Bytes of device workspace attn_decode needs for these sizes (0 if a size is invalid).  The size
 * does not depend on max_len or on the device: with U rows per sequence and H query heads per
 * row (attn_decode_plan), about U * (2048 / U + n_seq) * H * (d + 2) * 4 bytes. */
size_t attn_decode_workspace_size(int n_seq, int Hq, int Hkv, int d, int max_len);

/* Decode: one new query token per sequence against its cached keys and values.
 *   q, o [n_seq, Hq, d] bf16;  k_pool, v_pool [pool_rows, Hkv, d] bf16.
 *   offsets[n_seq] int64: pool row of each sequence's first token (any order, gaps allowed).
 *   lens[n_seq] int32: cached tokens of each sequence, 0 <= lens[s] <= max_len, counting the
 *   query token itself (its K/V are the last row).  The query sees all lens[s] keys, or only
 *   the last `window` of them when window > 0.
 *   lse [n_seq, Hq] fp32, natural log; may be NULL.
 *   workspace: caller-owned device memory of at least attn_decode_workspace_size(...) bytes,
 *   fully rewritten by each call; calls that share a workspace must not overlap in time.
 * offsets and lens live in device memory and are checked on the device: a sequence with
 * lens < 0, lens > max_len, offsets < 0 or offsets + lens > pool_rows is not read, and its
 * outputs (o rows and lse) are set to NaN.  `stream` must belong to the current device.
 * Work is split evenly over one resident round of workers whatever the mix of lengths (see
 * attn_decode_plan); n_seq * ceil(max_len / tokens_per_block) must stay below 2^30. */
int attn_decode(const void* q, const void* k_pool, const void* v_pool,
                const int64_t* offsets, const int32_t* lens, void* o, float* lse,
                int n_seq, int Hq, int Hkv, int d, int64_t pool_rows, int max_len, int window,
                float scale, void* workspace, size_t workspace_bytes, void* stream);

/* Decode against a paged KV cache ("LLM中的Attention实现及优化", PagedAttention: the cache is
 * handed out in small fixed-size pages that need not be contiguous; "高效多头潜在注意力解码技术：
 * Flash MLA深度解析" §3.2: paged GPU memory for long sequences).  As attn_decode, except for the
 * addressing of the pool:
 *   k_pool, v_pool [pool_pages * page_size, Hkv, d] bf16: physical page p is pool rows
 *   p * page_size .. (p + 1) * page_size - 1.
 *   block_table [n_seq, table_stride] int32 (device memory): block_table[s * table_stride + j]
 *   is the page holding tokens j * page_size .. (j + 1) * page_size - 1 of sequence s.  Only
 *   the entries of pages holding keys the query sees are read; table_stride must be at least
 *   ceil(max_len / page_size).  Pages may be shared between sequences and appear in any order.
 *   page_size must be a multiple of the decode block's token count (attn_decode_plan's
 *   tokens_per_block: 32 / Hkv in the packed layout, else 32); ATTN_ERR_UNSUPPORTED otherwise.
 * A sequence with lens < 0 or lens > max_len is not read, and one whose visible keys lie on a
 * page entry outside [0, pool_pages) reads nothing from that page; the outputs of both are set
 * to NaN.  Uses the same workspace (attn_decode_workspace_size). */
int attn_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_table, int table_stride, int page_size, int64_t pool_pages,
                      const int32_t* lens, void* o, float* lse,
                      int n_seq, int Hq, int Hkv, int d, int max_len, int window,
                      float scale, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace attn_bwd needs: B * Hq * Lq fp32 values (rounded up to 256). */
size_t attn_bwd_workspace_size(int B, int Hq, int Lq);

/* Backward of attn_fwd (bf16): the gradients of O = softmax(scale * Q K^T + mask) V with respect
 * to q, k and v for an upstream gradient dout = dL/dO.  FlashAttention's backward pass recomputes
 * the probabilities tile by tile from the forward's row log-sum-exp instead of storing them (the
 * tqpw.cn MQA/GQA article, §4; the stored softmax matrix is what "003-注意力机制详解…" §一 says
 * back-propagation would otherwise need).  With P = exp(scale * S - lse) on the visible entries:
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),  dQ = scale * dS K,
 *   dK = scale * dS^T Q;  with GQA a KV head's gradient sums its query heads' contributions.
 *   q, o, dout, dq [B, Hq, Lq, d]; k, v, dk, dv [B, Hkv, Lk, d] (bf16, results rounded to nearest
 *   even); lse [B, Hq, Lq] fp32 as written by attn_fwd with the same q, k, v, mask and scale.
 *   dq, dk and dv are fully overwritten (not accumulated into).  Masking, scale and status codes
 *   as attn_fwd; rows with lse = -inf contribute nothing and get dq = 0.
 * P and dS enter the products rounded to bf16; everything accumulates in fp32.  The result does
 * not depend on scheduling (no atomics).  workspace: caller-owned device memory of at least
 * attn_bwd_workspace_size(B, Hq, Lq) bytes, 16-byte aligned, overwritten by each call; calls that
 * share a workspace must not overlap in time (ATTN_ERR_WORKSPACE if NULL or too small). */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Lq, int Lk, int d,
             int causal, int window, float scale, void* workspace, size_t workspace_bytes, void* stream);

/* attn_decode for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, layout, results and status
 * codes as attn_decode, without the workspace: the decode workspace is a fixed array of
 * ATTN_DECODE_NOALLOC_BYTES (64 MiB) inside the library, one per GPU, which that GPU holds until
 * the process ends.  A call whose attn_decode_workspace_size(...) exceeds it returns
 * ATTN_ERR_WORKSPACE before any device work (at Hq = 32, d = 128: up to about 1900 sequences).
 * The call allocates nothing and calls no allocating routine; its device address is looked up
 * on its first call on each device (ATTN_ERR_HIP if the runtime refuses).  Every call on one GPU
 * shares that GPU's array, whatever the stream: calls that overlap in time on one GPU race and
 * their results are undefined; calls in order on one stream, or separated by synchronisation,
 * are independent (nothing in the array needs to start at zero). */
#define ATTN_DECODE_NOALLOC_BYTES ((size_t)64 << 20)
int attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                        const int64_t* offsets, const int32_t* lens, void* o, float* lse,
                        int n_seq, int Hq, int Hkv, int d, int64_t pool_rows, int max_len, int window,
                        float scale, void* stream);

/* attn_decode over an FP8 KV cache: k_pool and v_pool [pool_rows, Hkv, d] hold 8-bit codes of
 * format kv_format (one byte per element, same layout as the bf16 pools), with one scale per pool:
 * the key is k_scale * K(code), the value v_scale * V(code) (k_scale, v_scale finite and > 0).
 * q, o, lse and every other argument as attn_decode; the same workspace.  Codes convert exactly to
 * bf16, so the arithmetic is attn_decode's: scores in fp32 (k_scale folded into the score scale),
 * P rounded to bf16 for P.V, fp32 accumulation, v_scale applied to the fp32 result.  NaN codes
 * propagate like NaN values. */
int attn_decode_fp8(const void* q, const void* k_pool, const void* v_pool,
                    const int64_t* offsets, const int32_t* lens, void* o, float* lse,
                    int n_seq, int Hq, int Hkv, int d, int64_t pool_rows, int max_len, int window,
                    float scale, int kv_format, float k_scale, float v_scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/* attn_decode_paged over an FP8 KV cache (pools [pool_pages * page_size, Hkv, d] of 8-bit codes),
 * with kv_format, k_scale and v_scale as attn_decode_fp8. */
int attn_decode_paged_fp8(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, int table_stride, int page_size, int64_t pool_pages,
                          const int32_t* lens, void* o, float* lse,
                          int n_seq, int Hq, int Hkv, int d, int max_len, int window,
                          float scale, int kv_format, float k_scale, float v_scale,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* attn_status_str(int status);

/* ---- planner introspection (host only, no device work; used by tests and tooling) ---- */

typedef struct {
  int32_t block_q;            /* query rows per workgroup */
  int32_t block_k;            /* keys per K/V tile */
  int32_t threads;            /* threads per workgroup */
  int32_t lds_bytes;          /* LDS per workgroup */
  int32_t num_q_tiles;        /* ceil(Lq / block_q) */
  int32_t heads_per_xcd;      /* > 0 when blocks are banded by XCD */
  int64_t num_workgroups;     /* grid size */
  int64_t tiles_per_head;     /* K/V tiles visited, summed over the query tiles of one head */
  int64_t masked_tiles_per_head; /* of which straddle a mask boundary */
} attn_fwd_plan_info;

/* Fill *out with the launch plan attn_fwd (dtype_f32 = 0) or attn_fwd_f32 (dtype_f32 = 1)
 * would use.  Returns the same status the call itself would return for these sizes. */
int attn_fwd_plan(int B, int Hq, int Hkv, int Lq, int Lk, int d, int causal, int window,
                  int dtype_f32, attn_fwd_plan_info* out);

/* Write, for every workgroup index bid < num_workgroups, the (batch, query head, query tile)
 * it computes: out[3*bid + 0..2].  `out` is host memory of 3 * num_workgroups int32. */
int attn_fwd_schedule(int B, int Hq, int Hkv, int Lq, int Lk, int d, int causal, int window,
                      int dtype_f32, int32_t* out, int64_t out_len);

/* Block order of attn_fwd_varlen for these sizes: *num_blocks blocks, and (if out is not NULL)
 * out[3*i .. 3*i+2] = (sequence, query head, query tile) of block i; sequence = n_seq marks a
 * block without work.  The blocks of one (sequence, KV head) share an XCD (i % 8) and
 * consecutive slots. */
int attn_fwd_varlen_schedule(int n_seq, int Hq, int Hkv, int max_seqlen_q, int32_t* out, int64_t out_len,
                             int64_t* num_blocks);

/* Decode work split on the current device.  A block is 32 rows of K/V: when Hq <= 32 and Hkv
 * divides 32 it holds all Hkv heads of 32/Hkv consecutive tokens (one contiguous stretch of the
 * pool; *rows_per_seq = 1 and one worker serves every query head), otherwise 32 tokens of one KV
 * head (*rows_per_seq = Hkv * ceil((Hq/Hkv) / 32) rows, each a KV head and up to 32 of its query
 * heads).  *tokens_per_block = 32/Hkv or 32.  *teams = teams of rows_per_seq single-wave
 * workers launched.  With nb(s) = ceil(visible keys of s / tokens_per_block) blocks per row (0
 * for a sequence that is not read) and T = sum of nb(s), the blocks of all sequences laid end
 * to end are cut into shares of ceil(T / teams) blocks; team t computes share t for every row,
 * one partial per (row, sequence) it meets.  ATTN_ERR_HIP without a usable device.  The plan is
 * that of bf16 pools (three workers per CU in the packed layout, two in the one-head layout);
 * FP8 pools (attn_decode_fp8) run four per CU. */
int attn_decode_plan(int n_seq, int Hq, int Hkv, int d, int32_t* teams, int32_t* rows_per_seq,
                     int32_t* tokens_per_block);

/* The rows of one sequence in the decode split (host only, no device work): for each row u <
 * attn_decode_plan's rows_per_seq, kv_head[u] is the KV head its blocks hold (0 in the packed
 * layout, whose blocks hold every KV head), and the row serves query heads first_head[u] ..
 * first_head[u] + n_heads[u] - 1 of each sequence; the kernels read and write q and o rows of
 * those heads only.  out_len is the length of each output array (host memory); ATTN_ERR_SHAPE
 * if it is below rows_per_seq or the head counts are invalid. */
int attn_decode_rows(int Hq, int Hkv, int32_t* kv_head, int32_t* first_head, int32_t* n_heads,
                     int64_t out_len);

#ifdef __cplusplus
}
#endif

#endif /* ATTNFWD_ATTN_H */
