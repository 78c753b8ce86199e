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
 *   2  mode 1 plus the softmax's vector work per step (the lane's row maximum tested against the
 *      reference, one fma, exp2 and add per score, bf16 packing of P);
 *   3  mode 2 plus the end of the kernel's step: wait for the wave's loads, workgroup barrier;
 *   4  mode 3 plus the kernel's loads: each step fills the other K and V LDS stages (19 KB per
 *      workgroup) from global memory with wave-wide global->LDS loads; Q rows come from the same
 *      source, so all operands carry the caller's data.
 * Modes 0-3 load nothing from global memory.  sink: device memory of at least workgroups * 256
 * floats, overwritten (keeps the results live); in mode 4 it must hold ATTN_PROBE_SOURCE_BYTES
 * more, in front: 64 blocks of 19 KB (one K and one V stage each) that the workgroups read in
 * turn (block = workgroup index % 64), e.g. small bf16 values; the results go after them.
 * Enqueued on `stream`; the caller times it.  Status codes as attn.h: ATTN_ERR_NULL,
 * ATTN_ERR_SHAPE (a count <= 0), ATTN_ERR_UNSUPPORTED (mode not 0-4), ATTN_ERR_WORKSPACE (sink
 * too small), ATTN_ERR_HIP. */
#define ATTN_PROBE_SOURCE_BYTES ((size_t)64 * (9216 + 10240))
int attn_probe_mfma_ceiling(int mode, int workgroups, int steps, float* sink, size_t sink_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTNFWD_ATTN_PROBE_H */
