"""GPU parity of qlora_dropout_mask (reading G19: the LoRA dropout keep mask of
QLoRA Appendix B.2 drawn from Philox4x64-10) against the oracle's generator:
the packed mask bytes are bit-exact on ragged and workload shapes, and the
dropout forward and backward driven by a device-drawn mask match the fp64
oracle driven by the oracle's mask."""

import sys

import numpy as np
import pytest
import torch

from oracle import dropout_rng, linear
from test_gpu_linear import OracleWeight

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


@pytest.mark.parametrize("seed,offset,M,K,p", [(0, 0, 1, 8, 0.1), (1, 2, 3, 40, 0.5), (2 ** 64 - 1, 2 ** 63 + 5, 7, 264, 0.05),
                                               (12345, 77, 130, 1000, 0.999), (99, 3, 64, 4096, 0.0),
                                               (2024, 1, 4096, 4096, 0.1), (7, 9, 2048, 11008, 0.05)])
def test_mask_bit_exact(B, seed, offset, M, K, p):
    _log(f"dropout mask seed={seed} offset={offset} M={M} K={K} p={p}")
    got = B.qlora_dropout_mask(seed, offset, M, K, p)
    torch.cuda.synchronize()
    want = dropout_rng.keep_mask_packed(seed, offset, M, K, p)
    g = got.cpu().numpy()
    if not np.array_equal(g, want):
        bad = np.argwhere(g != want)[:5].tolist()
        raise AssertionError(f"mask bytes differ at {bad} (of {(g != want).sum()})")


def test_device_mask_drives_the_dropout_layer(B):
    M, N, K, r, p = 300, 256, 576, 64, 0.1
    s = 16.0 / r
    g = torch.Generator(device="cuda").manual_seed(31)
    W = torch.randn(N, K, generator=g, device="cuda") * 0.02
    X = torch.randn(M, K, generator=g, device="cuda").to(torch.bfloat16)
    A = (torch.randn(K, r, generator=g, device="cuda") * 0.01).to(torch.bfloat16)
    Bm = (torch.randn(r, N, generator=g, device="cuda") * 0.01).to(torch.bfloat16)
    dY = torch.randn(M, N, generator=g, device="cuda").to(torch.bfloat16)
    km = B.qlora_dropout_mask(5, 11, M, K, p)
    qw = B.qlora_nf4_quantize(W)
    Y, XA = B.qlora_linear_fwd(X, qw, A, Bm, s, keep=km, p=p)
    dX, dA, dB = B.qlora_linear_bwd(dY, X, None, qw, A, Bm, s, keep=km, p=p)
    torch.cuda.synchronize()
    keep = dropout_rng.keep_mask(5, 11, M, K, p)
    Wb = OracleWeight(W.cpu().numpy()).full()
    f = lambda t: t.float().cpu().numpy()  # noqa: E731
    Yr, XAr = linear.forward_dropout(f(X), Wb, f(A), f(Bm), s, keep, p)
    dXr, dAr, dBr = linear.backward_dropout(f(dY), f(X), Wb, f(A), f(Bm), s, keep, p)
    for name, o, ref in (("Y", Y, Yr), ("XA", XA, XAr), ("dX", dX, dXr), ("dA", dA, dAr), ("dB", dB, dBr)):
        e = linear.rel_l2(f(o), ref)
        _log(f"  {name}: rel_l2={e:.3e}")
        assert e <= 5e-3
