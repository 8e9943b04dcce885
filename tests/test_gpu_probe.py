"""The streaming-read probe the benchmark uses for its "achievable read"
figure: it runs on buffers of every size class and leaves them unchanged."""

import pytest
import torch

from bit_nf4_quantized_quantize_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, (64 << 20) + 48])
def test_probe_read_runs_and_leaves_the_buffer(nbytes):
    buf = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
    ref = buf.clone()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    B.qlora_probe_read(buf, sink)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)
