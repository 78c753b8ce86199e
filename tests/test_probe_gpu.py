"""The ceiling probe (include/attn_probe.h) runs in every mode and leaves finite results.

It is a measurement kernel, not part of attention: this only checks that each mode launches with
the documented sink layout (mode 4 reads its source blocks from the front of the sink and writes
its results after them) and completes."""
import numpy as np
import pytest
import torch

import attention_attn_fwd_03_amd as af

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4])
def test_probe_modes_run(mode):
    wgs, steps = 16, 8
    src_floats = af.PROBE_SOURCE_BYTES // 4
    sink = torch.empty(src_floats + wgs * 256, device=DEV, dtype=torch.float32)
    # source blocks: bf16 pairs of 0.01 (0x3C24), as bench.py fills them
    sink.view(torch.int32).fill_(0x3C243C24)
    af.probe_mfma_ceiling(wgs, steps, sink, mode=mode)
    torch.cuda.synchronize()
    res = sink.cpu().numpy()
    out = res[src_floats:] if mode == 4 else res[: wgs * 256]
    assert np.all(np.isfinite(out)), mode
    if mode == 4:  # the source blocks are read, not written
        assert np.all(sink[:src_floats].view(torch.int32).cpu().numpy() == 0x3C243C24)


def test_probe_rejects_a_sink_without_source_blocks():
    wgs = 16
    sink = torch.empty(wgs * 256, device=DEV, dtype=torch.float32)
    with pytest.raises(RuntimeError):
        af.probe_mfma_ceiling(wgs, 4, sink, mode=4)
