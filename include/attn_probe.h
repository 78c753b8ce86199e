/* attnfwd measurement probe (not part of the attention computation).
 *
 * The prefill kernel's fraction of the nominal bf16 matrix-core peak is read against what the
 * matrix cores sustain on this part when fed the same way: the pages' own efficiency metric is
 * FLOPs utilisation ("高效多头潜在注意力解码技术：Flash MLA深度解析", §3.3 monitoring table), and
 * under sustained matrix load the engine clock drops below the 2.4 GHz the nominal peak assumes.
 */
#ifndef ATTNFWD_ATTN_PROBE_H
#define ATTNFWD_ATTN_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launch `workgroups` workgroups shaped like the d = 128 prefill kernel's (256 threads, three per
 * CU, the same two LDS stages), each of whose four waves runs `steps` steps of that kernel's
 * matrix work: 16 v_mfma_f32_32x32x16_bf16 per step (2 * 32 * 32 * 16 * 16 = 524288 FLOP per
 * wave), and, by `mode`:
 *   0  nothing else (operands held in registers);
 *   1  the operand reads from LDS (K rows for S^T = K Q^T, V^T by ds_read_b64_tr_b16);
 *   2  mode 1 plus the softmax's vector work per step (row maximum, one fma, exp2 and add per
 *      score, bf16 packing of P).
 * No global loads, no barriers.  sink: device memory of at least workgroups * 256 floats,
 * overwritten (keeps the results live).  Enqueued on `stream`; the caller times it.  Status codes
 * as attn.h: ATTN_ERR_NULL, ATTN_ERR_SHAPE (a count <= 0), ATTN_ERR_UNSUPPORTED (mode not 0-2),
 * ATTN_ERR_WORKSPACE (sink too small), ATTN_ERR_HIP. */
int attn_probe_mfma_ceiling(int mode, int workgroups, int steps, float* sink, size_t sink_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTNFWD_ATTN_PROBE_H */
