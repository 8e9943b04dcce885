"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, answers host queries, and rejects bad arguments on the
host before anything is enqueued (the pointers passed here are never
dereferenced because validation fails first)."""

import ctypes
import os
import re

import numpy as np
import pytest

from bit_nf4_quantized_quantize_amd import binding as B
from oracle import blockwise, codebook

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("qlora_nf4.h", "qlora_nf4_profile.h")]
FAKE = 0x10000          # 16-byte aligned, never dereferenced
FAKE_MIS = 0x10004      # misaligned


def header_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(qlora_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_library_loads_and_exports_every_declared_symbol():
    L = B.lib()
    names = header_functions()
    assert len(names) == 24, names
    assert sorted(B.EXPORTED) == names
    for n in names:
        assert hasattr(L, n), n


def test_storage_bytes_match_closed_form():
    for numel in (1, 63, 64, 65, 4096 * 4096, 11008 * 4096, 22016 * 8192):
        for dq in (True, False):
            got = B.qlora_nf4_storage_bytes(numel, dq)
            want = blockwise.storage_bytes(numel, dq)
            assert {k: v for k, v in got.items() if v} == want
    numel = 4096 * 4096
    bits = 8 * sum(B.qlora_nf4_storage_bytes(numel, True).values()) / numel
    assert bits == 4 + 8 / 64 + 32 / (64 * 256) + 32 / numel
    for ct in (*B.CODE_TYPES.values(), B.QLORA_CODE_INT8):
        for numel in (1, 63, 65, 4096 * 4096):
            for dq in (True, False):
                got = B.qlora_storage_bytes(numel, dq, ct)
                assert {k: v for k, v in got.items() if v} == blockwise.storage_bytes(numel, dq, ct)
    bits8 = 8 * sum(B.qlora_storage_bytes(numel, True, B.QLORA_CODE_INT8).values()) / numel
    assert bits8 == 8 + 8 / 64 + 32 / (64 * 256) + 32 / numel
    out = (ctypes.c_int64 * 5)()
    assert B.lib().qlora_storage_bytes(64, 1, 5, out) == B.QLORA_ERR_INVALID_ARG
    assert B.lib().qlora_storage_bytes(64, 2, 4, out) == B.QLORA_ERR_INVALID_ARG
    assert B.lib().qlora_storage_bytes(-1, 1, 4, out) == B.QLORA_ERR_INVALID_ARG
    assert B.lib().qlora_storage_bytes(64, 1, 4, None) == B.QLORA_ERR_INVALID_ARG


def test_library_codebook_is_appendix_e():
    assert np.array_equal(np.array(B.qlora_nf4_codebook(), np.float32).view(np.uint32),
                          codebook.NF4.view(np.uint32))


def test_library_codebooks_equal_oracle_bit_exact():
    """Every codebook the library quantises against equals the oracle's
    (built independently from the format definitions), sign of zero included."""
    for name, ct in B.CODE_TYPES.items():
        got = np.array(B.qlora_codebook(ct), np.float32)
        assert np.array_equal(got.view(np.uint32), codebook.CODEBOOKS[ct].view(np.uint32)), name
    got = np.array(B.qlora_codebook(B.QLORA_CODE_INT8), np.float32)
    assert np.array_equal(got.view(np.uint32), codebook.INT8.view(np.uint32))
    out = (ctypes.c_float * 256)()
    assert B.lib().qlora_codebook(5, out) == B.QLORA_ERR_INVALID_ARG
    assert B.lib().qlora_codebook(-1, out) == B.QLORA_ERR_INVALID_ARG


def test_status_strings():
    L = B.lib()
    for s in range(-6, 1):
        assert L.qlora_status_string(s).decode() != "unknown status"
    assert L.qlora_status_string(-99).decode() == "unknown status"


def _desc(rows=256, cols=256, dq=1, codes=FAKE, bs=64, bs2=256):
    d = B.qlora_nf4_t()
    d.rows, d.cols, d.blocksize, d.blocksize2, d.double_quant = rows, cols, bs, bs2, dq
    d.codes, d.absmax_q, d.scale2, d.offset, d.absmax = codes, FAKE, FAKE, FAKE, FAKE
    return d


def _quant(d, w=FAKE, dtype=0, ws=FAKE, nws=1 << 30):
    return B.lib().qlora_nf4_quantize(w, dtype, ctypes.byref(d) if d is not None else None, ws, nws, None)


def test_quantize_validation():
    L = B.lib()
    assert _quant(None) == B.QLORA_ERR_INVALID_ARG
    assert "descriptor" in L.qlora_last_error().decode()
    assert _quant(_desc(bs=32)) == B.QLORA_ERR_INVALID_ARG
    assert _quant(_desc(bs2=128)) == B.QLORA_ERR_INVALID_ARG
    assert _quant(_desc(dq=2)) == B.QLORA_ERR_INVALID_ARG
    d = _desc()
    d.code_type = 5
    assert _quant(d) == B.QLORA_ERR_INVALID_ARG
    assert "code_type" in L.qlora_last_error().decode()
    assert _quant(_desc(rows=-1)) == B.QLORA_ERR_INVALID_ARG
    assert _quant(_desc(rows=1 << 20, cols=1 << 20)) == B.QLORA_ERR_INVALID_ARG
    assert _quant(_desc(codes=None)) == B.QLORA_ERR_INVALID_ARG
    assert _quant(_desc(codes=FAKE_MIS)) == B.QLORA_ERR_MISALIGNED
    assert _quant(_desc(), dtype=7) == B.QLORA_ERR_UNSUPPORTED_DTYPE
    assert _quant(_desc(), w=None) == B.QLORA_ERR_INVALID_ARG
    assert _quant(_desc(), w=FAKE_MIS) == B.QLORA_ERR_MISALIGNED
    assert _quant(_desc(), nws=16) == B.QLORA_ERR_WORKSPACE_TOO_SMALL
    assert _quant(_desc(), ws=None) == B.QLORA_ERR_INVALID_ARG
    d = _desc(dq=1)
    d.offset = None
    assert _quant(d) == B.QLORA_ERR_INVALID_ARG
    d = _desc(dq=0)
    d.absmax = None
    assert _quant(d) == B.QLORA_ERR_INVALID_ARG
    # an empty weight is a successful no-op
    assert _quant(_desc(rows=0), w=None, ws=None, nws=0) == B.QLORA_OK


def test_batched_quantize_validation():
    """The batched call validates every descriptor and pointer before any
    launch: mixed code types or double_quant, a null weight pointer, a small
    workspace, a bad count."""
    L = B.lib()
    n = 3
    descs = (B.qlora_nf4_t * n)(*[_desc() for _ in range(n)])
    ptrs = (ctypes.c_void_p * n)(FAKE, FAKE, FAKE)
    need = ctypes.c_int64(0)
    assert L.qlora_nf4_quantize_batched_workspace(descs, n, ctypes.byref(need)) == B.QLORA_OK
    assert need.value == 3 * B.qlora_nf4_quantize_workspace(256 * 256, True)
    assert L.qlora_nf4_quantize_batched(ptrs, 0, descs, n, FAKE, need.value - 1, None) == \
        B.QLORA_ERR_WORKSPACE_TOO_SMALL
    assert L.qlora_nf4_quantize_batched(ptrs, 0, descs, -1, FAKE, need.value, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_nf4_quantize_batched(ptrs, 0, descs, 5000, FAKE, need.value, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_nf4_quantize_batched(ptrs, 3, descs, n, FAKE, need.value, None) == B.QLORA_ERR_UNSUPPORTED_DTYPE
    assert L.qlora_nf4_quantize_batched(None, 0, None, 0, None, 0, None) == B.QLORA_OK
    descs[1].code_type = 4
    assert L.qlora_nf4_quantize_batched(ptrs, 0, descs, n, FAKE, need.value, None) == B.QLORA_ERR_INVALID_ARG
    descs[1].code_type = 0
    descs[2].double_quant = 0
    assert L.qlora_nf4_quantize_batched(ptrs, 0, descs, n, FAKE, need.value, None) == B.QLORA_ERR_INVALID_ARG
    descs[2].double_quant = 1
    ptrs[1] = None
    assert L.qlora_nf4_quantize_batched(ptrs, 0, descs, n, FAKE, need.value, None) == B.QLORA_ERR_INVALID_ARG
    ptrs[1] = FAKE_MIS
    assert L.qlora_nf4_quantize_batched(ptrs, 0, descs, n, FAKE, need.value, None) == B.QLORA_ERR_MISALIGNED


def test_dequantize_validation():
    L = B.lib()
    d = _desc()
    assert L.qlora_nf4_dequantize(ctypes.byref(d), FAKE, 5, None) == B.QLORA_ERR_UNSUPPORTED_DTYPE
    assert L.qlora_nf4_dequantize(ctypes.byref(d), None, 0, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_nf4_dequantize(ctypes.byref(d), FAKE_MIS, 0, None) == B.QLORA_ERR_MISALIGNED
    assert L.qlora_nf4_dequantize(None, FAKE, 0, None) == B.QLORA_ERR_INVALID_ARG


def test_workspace_queries():
    assert B.qlora_nf4_quantize_workspace(4096 * 4096, False) == 0
    assert B.qlora_nf4_quantize_workspace(4096 * 4096, True) >= 4 * 4096 * 4096 // 64
    f, b = B.qlora_linear_workspace(4096, 4096, 4096, 64)
    assert f >= 2 * 4096 * 64 * 3 and b >= 2 * 4096 * 64 * 3
    # every token count, including none, has a defined workspace
    for M in (0, 1, 15, 4096, 1 << 20):
        for r in (1, 8, 64, 100, 256):
            f, b = B.qlora_linear_workspace(M, 256, 512, r)
            assert f >= 0 and b >= 0
    assert B.qlora_nf4_quantize_workspace(0, True) == 0
    with pytest.raises(B.QLoraError):
        B.qlora_linear_workspace(16, 100, 256, 8)
    with pytest.raises(B.QLoraError):
        B.qlora_linear_workspace(16, 256, 256, 0)


def _fwd(d, M=16, r=8, X=FAKE, A=FAKE, Bp=FAKE, Y=FAKE, XA=FAKE, ws=FAKE, nws=1 << 30):
    return B.lib().qlora_linear_fwd(X, M, ctypes.byref(d), A, Bp, r, 2.0, Y, XA, ws, nws, None)


def _bwd(d, M=16, r=8, dY=FAKE, X=FAKE, XA=FAKE, A=FAKE, Bp=FAKE, dX=FAKE, dA=FAKE, dB=FAKE, acc=0, ws=FAKE,
         nws=1 << 30):
    return B.lib().qlora_linear_bwd(dY, X, XA, M, ctypes.byref(d), A, Bp, r, 2.0, dX, dA, dB, acc, ws, nws, None)


def test_linear_validation():
    assert _fwd(_desc(cols=200)) == B.QLORA_ERR_INVALID_ARG       # K % 64
    assert _fwd(_desc(rows=100)) == B.QLORA_ERR_INVALID_ARG       # N % 64
    assert _fwd(_desc(), r=0) == B.QLORA_ERR_INVALID_ARG
    assert _fwd(_desc(), r=257) == B.QLORA_ERR_INVALID_ARG
    assert _fwd(_desc(), M=-1) == B.QLORA_ERR_INVALID_ARG
    assert _fwd(_desc(), X=None) == B.QLORA_ERR_INVALID_ARG
    assert _fwd(_desc(), Y=FAKE_MIS) == B.QLORA_ERR_MISALIGNED
    assert _fwd(_desc(), XA=FAKE_MIS) == B.QLORA_ERR_MISALIGNED
    assert _fwd(_desc(), nws=1024) == B.QLORA_ERR_WORKSPACE_TOO_SMALL
    assert _fwd(_desc(bs=128)) == B.QLORA_ERR_INVALID_ARG
    # M = 0: nothing to compute, nothing enqueued
    assert _fwd(_desc(), M=0, X=None, Y=None, ws=None, nws=0) == B.QLORA_OK
    assert _bwd(_desc(cols=100)) == B.QLORA_ERR_INVALID_ARG
    assert _bwd(_desc(), dA=None) == B.QLORA_ERR_INVALID_ARG
    # XA may be NULL (recomputed); a bad one is still refused, before any launch
    assert _bwd(_desc(), XA=None, nws=1024) == B.QLORA_ERR_WORKSPACE_TOO_SMALL
    assert _bwd(_desc(), XA=FAKE_MIS) == B.QLORA_ERR_MISALIGNED
    assert _bwd(_desc(), X=None, XA=None) == B.QLORA_ERR_INVALID_ARG
    assert _bwd(_desc(), acc=2) == B.QLORA_ERR_INVALID_ARG
    assert "accumulate" in B.lib().qlora_last_error().decode()
    assert _bwd(_desc(), acc=-1) == B.QLORA_ERR_INVALID_ARG
    # no tokens and accumulate: nothing to add, nothing enqueued
    assert _bwd(_desc(), M=0, acc=1, dY=None, X=None, XA=None, ws=None, nws=0) == B.QLORA_OK
    assert _bwd(_desc(), dX=FAKE_MIS) == B.QLORA_ERR_MISALIGNED
    assert _bwd(_desc(), nws=1024) == B.QLORA_ERR_WORKSPACE_TOO_SMALL
    assert _bwd(_desc(), r=300) == B.QLORA_ERR_INVALID_ARG
    # Int8 weights take the same validation (the shape checks still apply)
    d8 = _desc(cols=200)
    d8.code_type = B.QLORA_CODE_INT8
    assert _fwd(d8) == B.QLORA_ERR_INVALID_ARG
    assert _bwd(d8) == B.QLORA_ERR_INVALID_ARG


def _fwd_do(d, keep=FAKE, p=0.1, M=16, r=8, nws=1 << 30):
    return B.lib().qlora_linear_fwd_dropout(FAKE, M, ctypes.byref(d), FAKE, FAKE, r, 2.0, keep, p, FAKE, FAKE, FAKE,
                                            nws, None)


def _bwd_do(d, keep=FAKE, p=0.1, M=16, r=8, nws=1 << 30):
    return B.lib().qlora_linear_bwd_dropout(FAKE, FAKE, FAKE, M, ctypes.byref(d), FAKE, FAKE, r, 2.0, keep, p, FAKE,
                                            FAKE, FAKE, 0, FAKE, nws, None)


def test_dropout_validation():
    """The dropout entry points reject a missing or misaligned mask and p
    outside [0, 1) on the host; shape errors as for the plain ones."""
    for call in (_fwd_do, _bwd_do):
        assert call(_desc(), keep=None) == B.QLORA_ERR_INVALID_ARG
        assert "keep_mask" in B.lib().qlora_last_error().decode()
        assert call(_desc(), keep=FAKE_MIS) == B.QLORA_ERR_MISALIGNED
        assert call(_desc(), p=1.0) == B.QLORA_ERR_INVALID_ARG
        assert call(_desc(), p=-0.1) == B.QLORA_ERR_INVALID_ARG
        assert call(_desc(), p=float("nan")) == B.QLORA_ERR_INVALID_ARG
        assert call(_desc(cols=200)) == B.QLORA_ERR_INVALID_ARG
        assert call(_desc(), r=0) == B.QLORA_ERR_INVALID_ARG
        assert call(_desc(), nws=1024) == B.QLORA_ERR_WORKSPACE_TOO_SMALL


def test_dropout_mask_validation():
    """The mask generator rejects bad sizes, p outside [0, 1) and a missing or
    misaligned buffer on the host; no tokens is a no-op."""
    L = B.lib()
    assert L.qlora_dropout_mask(1, 0, 16, 60, 0.1, FAKE, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_dropout_mask(1, 0, -1, 64, 0.1, FAKE, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_dropout_mask(1, 0, 16, 64, 1.0, FAKE, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_dropout_mask(1, 0, 16, 64, -0.5, FAKE, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_dropout_mask(1, 0, 16, 64, float("nan"), FAKE, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_dropout_mask(1, 0, 16, 64, 0.1, None, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_dropout_mask(1, 0, 16, 64, 0.1, FAKE_MIS, None) == B.QLORA_ERR_MISALIGNED
    assert L.qlora_dropout_mask(1, 0, 0, 64, 0.1, None, None) == B.QLORA_OK


def test_profile_hook_validation():
    L = B.lib()
    assert L.qlora_profile_events(9, None, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_profile_events(0, FAKE, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_profile_events(0, None, None) == B.QLORA_OK


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        B.qlora_nf4_quantize(torch.zeros(64))


def test_optimizer_validation():
    """The clip and AdamW entry points reject bad arguments on the host."""
    L = B.lib()
    ws = ctypes.c_int64(0)
    assert L.qlora_clip_scale_workspace(1000, ctypes.byref(ws)) == B.QLORA_OK and ws.value >= 8
    assert L.qlora_clip_scale_workspace(-1, ctypes.byref(ws)) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_clip_scale(FAKE, -1, 0.3, FAKE, FAKE, 1 << 20, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_clip_scale(FAKE, 100, 0.0, FAKE, FAKE, 1 << 20, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_clip_scale(FAKE, 100, 0.3, None, FAKE, 1 << 20, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_clip_scale(None, 100, 0.3, FAKE, FAKE, 1 << 20, None) == B.QLORA_ERR_INVALID_ARG
    assert L.qlora_clip_scale(FAKE, 100, 0.3, FAKE, FAKE, 1, None) == B.QLORA_ERR_WORKSPACE_TOO_SMALL

    def step(**kw):
        a = dict(param=FAKE, pbf=None, grad=FAKE, m=FAKE, v=FAKE, n=100, gs=None, lr=1e-4, b1=0.9, b2=0.999,
                 eps=1e-8, wd=0.0, t=1)
        a.update(kw)
        return L.qlora_adamw_step(a["param"], a["pbf"], a["grad"], a["m"], a["v"], a["n"], a["gs"], a["lr"],
                                  a["b1"], a["b2"], a["eps"], a["wd"], a["t"], None)
    assert step(t=0) == B.QLORA_ERR_INVALID_ARG
    assert step(b2=1.0) == B.QLORA_ERR_INVALID_ARG
    assert step(eps=0.0) == B.QLORA_ERR_INVALID_ARG
    assert step(lr=-1.0) == B.QLORA_ERR_INVALID_ARG
    assert step(n=-5) == B.QLORA_ERR_INVALID_ARG
    assert step(m=None) == B.QLORA_ERR_INVALID_ARG
    assert step(param=FAKE_MIS) == B.QLORA_ERR_MISALIGNED
    assert step(pbf=FAKE_MIS) == B.QLORA_ERR_MISALIGNED
    assert step(n=0, param=None, grad=None, m=None, v=None) == B.QLORA_OK

    def paged(**kw):
        a = dict(param=FAKE, pbf=None, grad=FAKE, m=FAKE, v=FAKE, n=100, gs=None, lr=1e-4, b1=0.9, b2=0.999,
                 eps=1e-8, wd=0.0, t=1, st=FAKE, sb=1 << 20)
        a.update(kw)
        return L.qlora_adamw_step_paged(a["param"], a["pbf"], a["grad"], a["m"], a["v"], a["n"], a["gs"], a["lr"],
                                        a["b1"], a["b2"], a["eps"], a["wd"], a["t"], a["st"], a["sb"], None, None)
    assert paged(sb=4095) == B.QLORA_ERR_WORKSPACE_TOO_SMALL
    assert paged(st=None) == B.QLORA_ERR_INVALID_ARG
    assert paged(st=FAKE_MIS) == B.QLORA_ERR_MISALIGNED
    assert paged(t=0) == B.QLORA_ERR_INVALID_ARG
    assert paged(m=None) == B.QLORA_ERR_INVALID_ARG
    assert paged(n=0, param=None, grad=None, m=None, v=None, st=FAKE) == B.QLORA_OK


def test_block_module_matches_oracle_layout():
    """The decoder block's seven linears and their [out, in] shapes are the
    oracle block's (host logic only; the block itself runs on the GPU)."""
    from bit_nf4_quantized_quantize_amd import block
    from oracle import block as oblock
    assert block.LINEARS == oblock.LINEARS
    assert block.linear_shapes(4096, 11008) == oblock.shapes(4096, 11008)
    assert block.EPS == oblock.EPS


def test_probe_read_validates_on_host():
    L = B.lib()
    bad = B.QLORA_ERR_INVALID_ARG
    assert L.qlora_probe_read(FAKE, 15, FAKE, None) == bad          # not a multiple of 16 bytes
    assert L.qlora_probe_read(FAKE_MIS, 16, FAKE, None) == bad      # misaligned source
    assert L.qlora_probe_read(None, 16, FAKE, None) == bad
    assert L.qlora_probe_read(FAKE, 16, None, None) == bad
    assert L.qlora_probe_read(FAKE, -16, FAKE, None) == bad
    assert L.qlora_probe_read(None, 0, None, None) == B.QLORA_OK     # nothing to read: nothing enqueued
