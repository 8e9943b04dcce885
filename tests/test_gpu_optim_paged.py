"""GPU parity of the paged optimizer step (QLoRA section 3 "Paged
Optimizers", reading G16): AdamW states in pinned host memory, paged through
a small device staging buffer chunk by chunk, on one stream and with a
separate copy stream.  The update kernel is the device-resident one, so
parameters, their bf16 copy and both states must be bit-identical to
qlora_adamw_step with device-resident states after several steps, for a
ragged number of elements spanning several chunks (and one chunk)."""

import sys

import pytest
import torch

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_nf4_quantized_quantize_amd import binding
    binding.lib()
    return binding


@pytest.mark.parametrize("n,staging_kib,copy_stream", [(100_003, 16, False), (100_003, 16, True),
                                                       (524_288, 256, True), (777, 64, True), (1_000_000, 1024, False)])
def test_paged_equals_device_states(B, n, staging_kib, copy_stream):
    _log(f"paged AdamW n={n} staging={staging_kib} KiB copy_stream={copy_stream}")
    g = torch.Generator(device="cuda").manual_seed(n + staging_kib)
    p0 = (torch.randn(n, generator=g, device="cuda") * 0.01).float()
    grads = [(torch.randn(n, generator=g, device="cuda") * (1.0 if k % 2 == 0 else 1e-3)).to(torch.bfloat16)
             for k in range(3)]
    # reference: device-resident states
    p_d, m_d, v_d = p0.clone(), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    pb_d = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    # paged: pinned host states
    p_h = p0.clone()
    m_h, v_h = torch.zeros(n).pin_memory(), torch.zeros(n).pin_memory()
    pb_h = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    staging = torch.empty(staging_kib << 10, dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream() if copy_stream else None
    sc = torch.empty(4, dtype=torch.float32, device="cuda")
    for t, gr in enumerate(grads, start=1):
        B.qlora_clip_scale(gr, 0.3, scale=sc)
        B.qlora_adamw_step(p_d, gr, m_d, v_d, t, 2e-4, (0.9, 0.999), 1e-8, 0.01, grad_scale=sc, param_bf16=pb_d)
        B.qlora_adamw_step_paged(p_h, gr, m_h, v_h, t, 2e-4, staging, (0.9, 0.999), 1e-8, 0.01, grad_scale=sc,
                                 param_bf16=pb_h, copy_stream=cs)
    torch.cuda.synchronize()
    assert torch.equal(p_d.view(torch.int32), p_h.view(torch.int32))
    assert torch.equal(pb_d.view(torch.int16), pb_h.view(torch.int16))
    assert torch.equal(m_d.cpu().view(torch.int32), m_h.view(torch.int32))
    assert torch.equal(v_d.cpu().view(torch.int32), v_h.view(torch.int32))
    assert float(m_h.abs().sum()) > 0
