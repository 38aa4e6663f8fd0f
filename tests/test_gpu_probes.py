"""The measurement probes on the GPU: the copy copies, the read and the
MFMA loop run and leave their sink untouched (its only write is guarded by
a condition that does not occur)."""
import pytest
import torch

import mixture_experts_layer_counting_amd as m
from tests.gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def test_probes_run_and_copy_copies():
    say("case: probes on 64 MiB")
    n = 16 << 20
    src = torch.arange(n, dtype=torch.int32, device=DEV)
    dst = torch.zeros_like(src)
    sink = torch.full((64,), 7.0, dtype=torch.float32, device=DEV)
    m.check(m.moe_probe_copy(dst, src, n * 4), "moe_probe_copy")
    m.check(m.moe_probe_read(src, n * 4, sink), "moe_probe_read")
    m.check(m.moe_probe_mfma(sink, 64), "moe_probe_mfma")
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert torch.all(sink == 7.0)
