"""fp64 CPU oracle for exact scaled-dot-product attention — TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
package.  It shares no code with the GPU path and imports nothing from it.
"""
from .attention import (attention, attention_backward, attention_head, attention_rows, decode, decode_paged, host_cores, kv_head,
                        masked_softmax, merge_partials, paged_rows, prefill_varlen, scores, useful_flops,
                        visibility, visible_pairs)
from .fp8 import attention_fp8, decode_e4m3fn, decode_e5m2, decode_fp8kv, decode_paged_fp8kv, dequantize

__all__ = ["attention", "attention_backward", "attention_head", "attention_rows", "decode", "decode_paged", "host_cores", "kv_head",
           "masked_softmax", "merge_partials", "paged_rows", "prefill_varlen", "scores", "useful_flops",
           "visibility", "visible_pairs", "decode_e4m3fn", "decode_e5m2", "decode_fp8kv", "decode_paged_fp8kv",
           "dequantize", "attention_fp8"]
