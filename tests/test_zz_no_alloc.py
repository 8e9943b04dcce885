"""GPU check of qlora_linear_fwd_noalloc (the forward for callers that cannot
allocate): through the C ABI, its outputs equal qlora_linear_fwd's bit for
bit, on two calls in a row (the second with a smaller input, so it runs on
what the first left in the shared scratch array), on the tiled path and
on the small-token path; a call whose workspace exceeds the fixed capacity
is refused before anything is enqueued."""

import ctypes
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


def _noalloc_fwd(B, X, q, A, Bm, s, Y, XA):
    d = q.desc()
    M = X.shape[0]
    r = A.shape[1]
    st = B.lib().qlora_linear_fwd_noalloc(B._ptr(X), M, ctypes.byref(d), B._ptr(A), B._ptr(Bm), r, float(s),
                                         B._ptr(Y), B._ptr(XA), B._stream())
    return st


def _inputs(M, N, K, r, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    W = torch.randn(N, K, generator=g, device="cuda") * 0.02
    X = torch.randn(M, K, generator=g, device="cuda").to(torch.bfloat16)
    A = (torch.randn(K, r, generator=g, device="cuda") * 0.01).to(torch.bfloat16)
    Bm = (torch.randn(r, N, generator=g, device="cuda") * 0.01).to(torch.bfloat16)
    return W, X, A, Bm


@pytest.mark.parametrize("shapes", [((4096, 4096, 4096, 64), (512, 4096, 4096, 64)),
                                    ((2048, 4096, 11008, 64), (300, 4096, 11008, 64)),
                                    ((16, 8192, 22016, 64), (3, 8192, 22016, 64)),
                                    ((600, 640, 320, 17), (77, 640, 320, 17))])
def test_noalloc_equals_workspace_forward(B, shapes):
    for M, N, K, r in shapes:
        _log(f"noalloc fwd M={M} N={N} K={K} r={r}")
        s = 16.0 / r
        W, X, A, Bm = _inputs(M, N, K, r, seed=M + N + K + r)
        qw = B.qlora_nf4_quantize(W)
        Y0, XA0 = B.qlora_linear_fwd(X, qw, A, Bm, s)
        Y1 = torch.full_like(Y0, 3.0)
        XA1 = torch.full_like(XA0, 3.0)
        st = _noalloc_fwd(B, X, qw, A, Bm, s, Y1, XA1)
        assert st == B.QLORA_OK, B.lib().qlora_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))
        assert torch.equal(XA0.view(torch.int16), XA1.view(torch.int16))


def test_noalloc_refuses_beyond_capacity(B):
    """400000 tokens on 11008 x 4096 need more than the 96 MiB of scratch:
    refused with WORKSPACE_TOO_SMALL on the host, nothing enqueued (the
    buffers passed are small and never touched)."""
    N, K, r, M = 11008, 4096, 64, 400000
    nws, _ = B.qlora_linear_workspace(M, N, K, r)
    assert nws > 96 << 20
    qw = B.NF4Weight(N, K, True)
    small = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    Y = torch.full((64,), 2.0, dtype=torch.bfloat16, device="cuda")
    d = qw.desc()
    st = B.lib().qlora_linear_fwd_noalloc(B._ptr(small), M, ctypes.byref(d), B._ptr(small), B._ptr(small), r, 1.0,
                                         B._ptr(Y), None, B._stream())
    assert st == B.QLORA_ERR_WORKSPACE_TOO_SMALL
    assert "capacity" in B.lib().qlora_last_error().decode()
    torch.cuda.synchronize()
    assert torch.all(Y == 2.0)
