"""The reference streaming pass (ce_stream_reference) on the GPU, through the C ABI.

A benchmark aid, not a step of the method: it reads and writes a buffer with
the fused kernel's own 16-byte non-temporal buffer instructions in 64 KiB
workgroup spans.  In place it XORs every 32-bit word with 0x80008000 (two
passes restore the buffer); otherwise it copies.  The checks are bit-exact
against torch's own bitwise ops, over sizes that end inside a vector span,
exactly on a workgroup span and past it, with guard bytes after the buffer
that must stay untouched.
"""
import ctypes

import pytest
import torch

import vocab_cross_entropy_amd as vce
from vocab_cross_entropy_amd import _abi

pytestmark = pytest.mark.gpu

SIZES = [16, 4096, 65536 - 16, 65536, 65536 + 16, (1 << 20) + 48, 3 << 20]
GUARD = 4096  # bytes after the buffer, filled with a pattern the pass must not touch


def _words(nbytes, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(-(2**31), 2**31 - 1, ((nbytes + GUARD) // 4,), generator=g, dtype=torch.int32).cuda()


def _raw(src_ptr, dst_ptr, nbytes):
    return vce.lib.ce_stream_reference(ctypes.c_void_p(src_ptr), ctypes.c_void_p(dst_ptr), nbytes,
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("nbytes", SIZES)
def test_in_place_flips_and_restores(nbytes):
    buf = _words(nbytes, 11 + nbytes)
    before = buf.clone()
    w = nbytes // 4
    assert _raw(buf.data_ptr(), buf.data_ptr(), nbytes) == _abi.CE_OK
    torch.cuda.synchronize()
    flip = torch.tensor(0x80008000 - (1 << 32), dtype=torch.int32, device="cuda")
    assert torch.equal(buf[:w], before[:w] ^ flip)
    assert torch.equal(buf[w:], before[w:])
    assert _raw(buf.data_ptr(), buf.data_ptr(), nbytes) == _abi.CE_OK
    torch.cuda.synchronize()
    assert torch.equal(buf, before)


@pytest.mark.parametrize("nbytes", SIZES)
def test_copy(nbytes):
    src = _words(nbytes, 101 + nbytes)
    src_before = src.clone()
    dst = _words(nbytes, 202 + nbytes)
    dst_before = dst.clone()
    w = nbytes // 4
    assert _raw(src.data_ptr(), dst.data_ptr(), nbytes) == _abi.CE_OK
    torch.cuda.synchronize()
    assert torch.equal(dst[:w], src_before[:w])
    assert torch.equal(dst[w:], dst_before[w:])
    assert torch.equal(src, src_before)


def test_binding_forms():
    x = torch.randn(4096, 33, dtype=torch.bfloat16, device="cuda")
    x0 = x.clone()
    vce.ce_stream_reference(x)
    torch.cuda.synchronize()
    assert torch.equal(x, -x0)  # the XOR flips the sign of both BF16 halves of every word
    y = torch.empty_like(x)
    vce.ce_stream_reference(x, y)
    torch.cuda.synchronize()
    assert torch.equal(y, -x0)
    with pytest.raises(vce.CeArgumentError):
        vce.ce_stream_reference(x, torch.empty(7, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(vce.CeArgumentError):
        vce.ce_stream_reference(x.t())
