"""GPU parity: the decoder block with QLoRA adapters on all seven linear
layers (the library's linears, fp32 glue) against the fp64 oracle block,
with and without gradient checkpointing."""

import sys

import numpy as np
import pytest
import torch

from oracle import block as oblock
from oracle import blockwise

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def BL():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_nf4_quantized_quantize_amd import binding, block
    binding.lib()
    return block


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def _setup(BL, hidden, mlp, heads, r, batch, seq, seed):
    g = torch.Generator().manual_seed(seed)
    shapes = BL.linear_shapes(hidden, mlp)
    W = {n: torch.randn(sh, generator=g) * 0.02 for n, sh in shapes.items()}
    A = {n: (torch.randn(shapes[n][1], r, generator=g) * 0.05).to(torch.bfloat16) for n in BL.LINEARS}
    Bm = {n: (torch.randn(r, shapes[n][0], generator=g) * 0.05).to(torch.bfloat16) for n in BL.LINEARS}
    g1 = 1 + 0.1 * torch.randn(hidden, generator=g)
    g2 = 1 + 0.1 * torch.randn(hidden, generator=g)
    x = torch.randn(batch, seq, hidden, generator=g)
    dy = torch.randn(batch, seq, hidden, generator=g)
    s = 16.0 / r
    blk = BL.QLoraBlock({n: W[n].cuda() for n in W}, {n: A[n].cuda() for n in A}, {n: Bm[n].cuda() for n in Bm},
                        g1.cuda(), g2.cuda(), s, heads)
    # the oracle sees the BF16 dequantised weights (Eq. 6) and the same values
    Wo = {n: blockwise.bf16_round(blockwise.quantize(W[n].numpy(), True).dequantize()).astype(np.float64)
          for n in W}
    ref = oblock.forward_backward(x.numpy(), Wo, {n: A[n].float().numpy() for n in A},
                                  {n: Bm[n].float().numpy() for n in Bm}, g1.numpy(), g2.numpy(), s, heads,
                                  dy.numpy())
    return blk, x, dy, ref


def _run(blk, x, dy, checkpoint):
    for p in blk.parameters():
        p.grad = None
    xg = x.cuda().requires_grad_(True)
    y = blk(xg, checkpoint=checkpoint)
    y.backward(dy.cuda())
    torch.cuda.synchronize()
    return (y.detach().cpu().numpy(), xg.grad.cpu().numpy(),
            {n: blk.lin[n].A.grad.float().cpu().numpy() for n in blk.lin},
            {n: blk.lin[n].B.grad.float().cpu().numpy() for n in blk.lin})


# Tolerance: each linear rounds its input and output to bf16 (relative
# error up to 2^-9 each) and the adapter gradients come out in bf16; a path
# through the block crosses at most four linears (q/k/v, o, gate/up, down),
# so a few tenths of a percent rel-L2 are expected.  The gate is 2e-2 for
# the output and the input gradient, 3e-2 for the adapter gradients.
@pytest.mark.parametrize("hidden,mlp,heads,r,batch,seq", [(256, 512, 4, 16, 2, 32), (128, 320, 2, 64, 1, 48)])
def test_block_matches_oracle(BL, hidden, mlp, heads, r, batch, seq):
    _log(f"block hidden={hidden} mlp={mlp} heads={heads} r={r} batch={batch} seq={seq}")
    blk, x, dy, ref = _setup(BL, hidden, mlp, heads, r, batch, seq, seed=hidden + seq)
    y, dx, dA, dB = _run(blk, x, dy, checkpoint=False)
    y_ref, dx_ref, dA_ref, dB_ref = ref
    assert _rel(y, y_ref) < 2e-2
    assert _rel(dx, dx_ref) < 2e-2
    for n in BL.LINEARS:
        assert _rel(dA[n], dA_ref[n]) < 3e-2, n
        assert _rel(dB[n], dB_ref[n]) < 3e-2, n


def test_block_checkpointing_recomputes_the_same(BL):
    """With gradient checkpointing the forward runs again inside the
    backward on the same deterministic kernels: output and gradients equal
    those of the plain run."""
    _log("block checkpointing")
    blk, x, dy, _ = _setup(BL, 256, 512, 4, 16, 2, 32, seed=7)
    plain = _run(blk, x, dy, checkpoint=False)
    ckpt = _run(blk, x, dy, checkpoint=True)
    assert np.array_equal(plain[0], ckpt[0]) and np.array_equal(plain[1], ckpt[1])
    for n in BL.LINEARS:
        assert np.array_equal(plain[2][n], ckpt[2][n]) and np.array_equal(plain[3][n], ckpt[3][n]), n


def test_block_checkpointing_keeps_less(BL):
    """After the forward, checkpointing holds only the block input for the
    backward, far less than the plain forward's saved activations."""
    _log("block saved activations")
    blk, x, dy, _ = _setup(BL, 256, 512, 4, 16, 4, 64, seed=8)
    held = {}
    for ck in (False, True, False):
        xg = x.cuda().requires_grad_(True)
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        y = blk(xg, checkpoint=ck)
        torch.cuda.synchronize()
        held[ck] = torch.cuda.memory_allocated() - base - y.numel() * y.element_size()
        del y, xg
    assert held[True] < 0.2 * held[False], held
