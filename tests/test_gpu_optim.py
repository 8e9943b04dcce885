"""GPU parity: the LoRA optimizer step (global gradient-norm clipping and
AdamW, reading G16) through the C ABI against the fp64 CPU oracle.

Tolerance: the GPU step is fp32 arithmetic (one rounding per operation), the
oracle fp64.  After a few steps the parameters agree to a relative 1e-5 of
the parameter scale (fp32 has 2^-24 ~ 6e-8 per operation, and each step
adds about ten operations); the clip scale to 1e-6.  The bf16 copy of the
parameters is checked bit-exactly against the rounding of the GPU's own
fp32 parameters, and keeping the states in pinned host memory must give
bit-identical results to keeping them on the device."""

import sys

import numpy as np
import pytest
import torch

from oracle import optim

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


def _f(x):
    """The fp32 value an fp32 argument of the ABI carries."""
    return float(np.float32(x))


def _bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _run(B, n, steps, host_states, seed, lr=2e-4, wd=0.01):
    g = torch.Generator(device="cuda").manual_seed(seed)
    p0 = (torch.randn(n, generator=g, device="cuda") * 0.01).float()
    grads = [(torch.randn(n, generator=g, device="cuda") * (2.0 if k % 2 == 0 else 1e-3)).to(torch.bfloat16)
             for k in range(steps)]
    p = p0.clone()
    if host_states:
        m = torch.zeros(n, dtype=torch.float32).pin_memory()
        v = torch.zeros(n, dtype=torch.float32).pin_memory()
    else:
        m = torch.zeros(n, dtype=torch.float32, device="cuda")
        v = torch.zeros(n, dtype=torch.float32, device="cuda")
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    scales = []
    for t in range(1, steps + 1):
        sc = B.qlora_clip_scale(grads[t - 1], 0.3)
        B.qlora_adamw_step(p, grads[t - 1], m, v, t, lr, (0.9, 0.999), 1e-8, wd, grad_scale=sc, param_bf16=pb)
        scales.append(sc[:1].clone())
    torch.cuda.synchronize()
    return p0, grads, p, m, v, pb, [float(s.item()) for s in scales]


@pytest.mark.parametrize("n", [5, 4096 * 64 * 2 + 37, 1 << 20])
def test_clip_and_adamw_parity(B, n):
    _log(f"optim n={n}")
    steps = 4
    p0, grads, p, m, v, pb, scales = _run(B, n, steps, False, seed=n)
    ref_p = p0.cpu().numpy().astype(np.float64)
    ref_m, ref_v = np.zeros(n), np.zeros(n)
    for t in range(1, steps + 1):
        gr = grads[t - 1].float().cpu().numpy().astype(np.float64)
        sc = optim.clip_scale([gr], 0.3)
        assert abs(scales[t - 1] - sc) <= 1e-6 * sc, (t, scales[t - 1], sc)
        ref_p, ref_m, ref_v = optim.adamw_step(ref_p, gr, ref_m, ref_v, t, _f(2e-4), _f(0.9), _f(0.999), _f(1e-8),
                                               _f(0.01), sc)
    pn = p.cpu().numpy().astype(np.float64)  # (hyperparameters below are the fp32 values the kernel receives)
    err = np.max(np.abs(pn - ref_p)) / np.max(np.abs(ref_p))
    _log(f"  max param error / max |param| = {err:.2e}")
    assert err <= 1e-5
    assert np.allclose(m.cpu().numpy(), ref_m, rtol=1e-5, atol=1e-9)
    assert np.allclose(v.cpu().numpy(), ref_v, rtol=1e-5, atol=1e-12)
    assert np.array_equal(_bf16_bits(pb), _bf16_bits(p.to(torch.bfloat16)))


def test_unclipped_scale_is_one(B):
    _log("optim clip scale 1")
    g = (torch.ones(1000, device="cuda") * 1e-3).to(torch.bfloat16)
    assert float(B.qlora_clip_scale(g, 0.3)[0].item()) == 1.0


def test_states_in_pinned_host_memory_match_device(B):
    """The paged reading: the states evicted to (pinned) host memory and used
    in place by the step give the same bits as device-resident states."""
    _log("optim host-resident states")
    n = 300007
    a = _run(B, n, 3, False, seed=9)
    b = _run(B, n, 3, True, seed=9)
    assert torch.equal(a[2], b[2])
    assert torch.equal(a[3], b[3].cuda()) and torch.equal(a[4], b[4].cuda())
    assert torch.equal(a[5], b[5])
