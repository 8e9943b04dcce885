"""GPU parity of qlora_nf4_quantize_batched: every weight of a batch gets the
same codes, FP8 constants, second-level scales and mean, bit for bit, as its
own qlora_nf4_quantize call (QLoRA section 2 Eq. 1 and section 3 "Double
Quantization", one tensor at a time), across batches of more than one launch
(more than 32 tensors), ragged sizes, empty tensors, both input dtypes,
without double quantisation, and for the other storage types; the NF4 codes
are also checked against the oracle."""

import sys

import numpy as np
import pytest
import torch

from oracle import blockwise

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


def _shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = i % 5
        if kind == 0:
            out.append((int(rng.integers(1, 40)), 64 * int(rng.integers(1, 30))))
        elif kind == 1:
            out.append((1, int(rng.integers(1, 5000))))           # ragged tail block and group
        elif kind == 2:
            out.append((0, 128))                                  # empty
        elif kind == 3:
            out.append((int(rng.integers(100, 600)), 256))
        else:
            out.append((64, 64 * int(rng.integers(40, 200))))
    return out


def _same(a, b):
    for k in a:
        if not np.array_equal(a[k], b[k]):
            return k
    return None


@pytest.mark.parametrize("count,dtype,dq,ct", [(7, torch.float32, True, 0), (70, torch.float32, True, 0),
                                                (45, torch.bfloat16, True, 0), (33, torch.float32, False, 0),
                                                (40, torch.float32, True, 1), (36, torch.bfloat16, True, 4),
                                                (34, torch.float32, False, 4)])
def test_batched_equals_single_calls(B, count, dtype, dq, ct):
    _log(f"batched quantize count={count} dtype={dtype} dq={dq} code_type={ct}")
    g = torch.Generator(device="cuda").manual_seed(count * 7 + ct)
    ws, singles, batch = [], [], []
    for i, (r, c) in enumerate(_shapes(count, count + ct)):
        w = (torch.randn(r, c, generator=g, device="cuda") * (0.02 * (1 + i % 3))).to(dtype)
        if r * c and i % 11 == 4:
            w[0, :min(c, 64)] = 0.0                               # an all-zero block
        ws.append(w)
        singles.append(B.qlora_nf4_quantize(w, double_quant=dq, code_type=ct) if r * c else None)
        batch.append(B.NF4Weight(r, c, dq, code_type=ct))
    nonempty = [(w, q) for w, q in zip(ws, batch)]
    B.qlora_nf4_quantize_batched([w for w, _ in nonempty], [q for _, q in nonempty])
    torch.cuda.synchronize()
    for i, (w, s, q) in enumerate(zip(ws, singles, batch)):
        if s is None:
            continue
        k = _same(s.host(), q.host())
        assert k is None, f"tensor {i} ({tuple(w.shape)}): {k} differs from its own call"
        if ct == 0 and dq and i % 9 == 0:
            st = blockwise.quantize(w.float().cpu().numpy(), double_quant=True)
            assert np.array_equal(q.host()["codes"], st.packed)
            assert np.array_equal(q.host()["absmax_q"], st.absmax_q)


def test_batched_sweep_layer_shapes(B):
    """One layer of the 32-layer 7B sweep (4 x 4096^2, 2 x 11008 x 4096,
    4096 x 11008) in one call, against single calls."""
    from bit_nf4_quantized_quantize_amd import synth
    shapes = synth.sweep_7b_shapes()[:7]
    ws = [synth.sweep_weight(i, "cuda") for i in range(7)]
    singles = [B.qlora_nf4_quantize(w) for w in ws]
    batch = [B.NF4Weight(n, k, True) for n, k in shapes]
    B.qlora_nf4_quantize_batched(ws, batch)
    torch.cuda.synchronize()
    for i, (s, q) in enumerate(zip(singles, batch)):
        assert _same(s.host(), q.host()) is None, f"matrix {i}"
