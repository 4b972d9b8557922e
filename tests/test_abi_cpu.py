"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments on the host before any HIP call (nothing is enqueued and
no buffer is touched).  No compute call is made here.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from vocab_cross_entropy_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ce.h")


@pytest.fixture(scope="module")
def lib():
    return _abi.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ce_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("ce_forward", "ce_backward_inplace", "ce_fwd_bwd_fused", "ce_shard_partial_stats",
              "ce_shard_combine"):
        assert n in names


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _abi.SIGNATURES, f"binding lacks {name}"


def test_version_and_strings(lib):
    assert lib.ce_abi_version() == _abi.CE_ABI_VERSION
    for s in range(7):
        assert lib.ce_status_string(s).startswith(b"CE_")


# -- host-side validation with host buffers (never dereferenced) ------------
class Host:
    """Host stand-ins for device buffers; validation must reject the call
    before anything reads or writes them."""

    def __init__(self, N=6, V=16, dtype=_abi.CE_BF16):
        self.x = np.zeros(N * V * 2, np.uint16 if dtype == _abi.CE_BF16 else np.float32)
        self.t = np.zeros(N, np.int64)
        self.loss = np.full(N, 7.0, np.float32)
        self.lse = np.full(N, 7.0, np.float32)
        self.n = np.full(1, 7, np.int32)
        self.stats = np.full(N * 4, 7.0, np.float32)
        self.ws = np.zeros(1 << 16, np.uint8)
        self.N, self.V, self.dtype = N, V, dtype

    def logits(self, **kw):
        d = dict(data=self.x.ctypes.data, dtype=self.dtype, reserved=0, d0=2, d1=self.N // 2, s0=self.N // 2 * self.V,
                 s1=self.V, v_local=self.V, vocab_start=0, vocab_total=self.V)
        d.update(kw)
        return _abi.CeLogits(**d)

    def targets(self, **kw):
        d = dict(data=self.t.ctypes.data, s0=self.N // 2, s1=1)
        d.update(kw)
        return _abi.CeTargets(**d)

    @staticmethod
    def params(**kw):
        d = dict(label_smoothing=0.0, reduce_loss=0, ignore_idx=-100, split_chunks=0, smoothing=0)
        d.update(kw)
        return _abi.CeParams(**d)

    def untouched(self):
        return (np.all(self.loss == 7.0) and np.all(self.lse == 7.0) and self.n[0] == 7
                and np.all(self.stats == 7.0) and not self.x.any())


def _fused(lib, h, x=None, t=None, p=None, ws=True, ws_bytes=None):
    x = x or h.logits()
    t = t or h.targets()
    p = p or h.params()
    return lib.ce_fwd_bwd_fused(ctypes.byref(x), ctypes.byref(t), ctypes.byref(p), None, h.loss.ctypes.data,
                                h.n.ctypes.data, h.ws.ctypes.data if ws else None,
                                h.ws.nbytes if ws_bytes is None else ws_bytes, None)


BAD_FUSED = [
    ("dtype", dict(x=dict(dtype=7)), _abi.CE_EDTYPE),
    ("reserved", dict(x=dict(reserved=1)), _abi.CE_EINVAL),
    ("v_local_zero", dict(x=dict(v_local=0, vocab_total=0)), _abi.CE_EINVAL),
    ("d1_zero", dict(x=dict(d1=0)), _abi.CE_EINVAL),
    ("d0_negative", dict(x=dict(d0=-1)), _abi.CE_EINVAL),
    ("null_data", dict(x=dict(data=None)), _abi.CE_EINVAL),
    ("misaligned_bf16", dict(x=dict(data="odd")), _abi.CE_ELAYOUT),
    ("negative_stride", dict(x=dict(s0=-16)), _abi.CE_ELAYOUT),
    ("rows_overlap", dict(x=dict(s1=8)), _abi.CE_ELAYOUT),
    ("rows_overlap_outer", dict(x=dict(s0=16)), _abi.CE_ELAYOUT),
    ("sharded_for_fused", dict(x=dict(vocab_start=16, vocab_total=32)), _abi.CE_ELAYOUT),
    ("shard_past_vocab", dict(x=dict(vocab_start=8, vocab_total=20)), _abi.CE_ELAYOUT),
    # a row of 4 GiB or more: beyond the kernels' 32-bit buffer ranges
    ("row_of_4gib_f32", dict(x=dict(dtype=_abi.CE_F32, d0=1, d1=1, s0=1 << 30, s1=1 << 30, v_local=1 << 30,
                                    vocab_total=1 << 30)), _abi.CE_ELAYOUT),
    ("row_of_4gib_bf16", dict(x=dict(d0=1, d1=1, s0=1 << 31, s1=1 << 31, v_local=1 << 31,
                                     vocab_total=1 << 31)), _abi.CE_ELAYOUT),
    ("smoothing_negative", dict(p=dict(label_smoothing=-0.1)), _abi.CE_EINVAL),
    ("smoothing_above_one", dict(p=dict(label_smoothing=1.5)), _abi.CE_EINVAL),
    ("smoothing_nan", dict(p=dict(label_smoothing=float("nan"))), _abi.CE_EINVAL),
    ("reduce_unknown", dict(p=dict(reduce_loss=3)), _abi.CE_EINVAL),
    ("reduce_negative", dict(p=dict(reduce_loss=-1)), _abi.CE_EINVAL),
    ("split_chunks_too_many", dict(p=dict(split_chunks=65)), _abi.CE_EINVAL),
    ("smoothing_unknown", dict(p=dict(smoothing=2)), _abi.CE_EINVAL),
    # a over the other classes of a one-class vocabulary: nowhere to put it
    ("smoothing_others_one_class", dict(x=dict(d0=1, d1=1, s0=1, s1=1, v_local=1, vocab_total=1),
                                        p=dict(smoothing=1, label_smoothing=0.1)), _abi.CE_EINVAL),
    ("null_targets", dict(t=dict(data=None)), _abi.CE_EINVAL),
    ("target_negative_stride", dict(t=dict(s1=-1)), _abi.CE_ELAYOUT),
    ("no_workspace", dict(ws=False), _abi.CE_EWORKSPACE),
    ("small_workspace", dict(ws_bytes=16), _abi.CE_EWORKSPACE),
]


@pytest.mark.parametrize("name,change,status", BAD_FUSED, ids=[b[0] for b in BAD_FUSED])
def test_fused_rejects_before_any_hip_call(lib, name, change, status):
    h = Host()
    xkw = dict(change.get("x", {}))
    if xkw.get("data") == "odd":
        xkw["data"] = h.x.ctypes.data + 1
    x = h.logits(**xkw)
    t = h.targets(**change.get("t", {}))
    p = h.params(**change.get("p", {}))
    rc = _fused(lib, h, x, t, p, ws=change.get("ws", True), ws_bytes=change.get("ws_bytes"))
    assert rc == status, (rc, lib.ce_last_error())
    assert lib.ce_last_error()
    assert h.untouched()


def test_noalloc_rejects_before_any_hip_call(lib):
    """The allocation-free fused call refuses bad arguments, and a call whose
    workspace would not fit its 16 MiB static scratch, on the host."""
    h = Host()
    t, p = h.targets(), h.params()

    def call(x, pp=p):
        return lib.ce_fwd_bwd_fused_noalloc(ctypes.byref(x), ctypes.byref(t), ctypes.byref(pp), None,
                                            h.loss.ctypes.data, h.n.ctypes.data, None)

    assert call(h.logits(dtype=7)) == _abi.CE_EDTYPE
    assert call(h.logits(vocab_start=16, vocab_total=32)) == _abi.CE_ELAYOUT
    assert call(h.logits(), h.params(split_chunks=65)) == _abi.CE_EINVAL
    # 131072 rows of 128000 BF16 columns in 8 chunks: 256 + (12 + 256) N bytes, above 16 MiB
    big = h.logits(d0=1, d1=131072, s0=131072 * 128000, s1=128000, v_local=128000, vocab_total=128000)
    assert call(big, h.params(reduce_loss=1)) == _abi.CE_EWORKSPACE
    assert b"16777216" in lib.ce_last_error()
    assert h.untouched()


def test_other_calls_reject(lib):
    h = Host()
    p = h.params()
    bad_x = h.logits(dtype=5)
    t = h.targets()
    assert lib.ce_forward(ctypes.byref(bad_x), ctypes.byref(t), ctypes.byref(p), h.loss.ctypes.data, None, None,
                          h.ws.ctypes.data, h.ws.nbytes, None) == _abi.CE_EDTYPE
    # forward needs unsharded logits
    sx = h.logits(vocab_start=16, vocab_total=64)
    assert lib.ce_forward(ctypes.byref(sx), ctypes.byref(t), ctypes.byref(p), h.loss.ctypes.data, None, None,
                          h.ws.ctypes.data, h.ws.nbytes, None) == _abi.CE_ELAYOUT
    # backward: lse required, n_valid required when reducing
    x = h.logits()
    assert lib.ce_backward_inplace(ctypes.byref(x), ctypes.byref(t), ctypes.byref(p), None, None, None,
                                   None) == _abi.CE_EINVAL
    pr = h.params(reduce_loss=1)
    assert lib.ce_backward_inplace(ctypes.byref(x), ctypes.byref(t), ctypes.byref(pr), h.lse.ctypes.data, None,
                                   None, None) == _abi.CE_EINVAL
    # smoothing over the other classes of one class: backward and combine reject it too
    po = h.params(smoothing=1, label_smoothing=0.2)
    x1 = h.logits(d0=1, d1=1, s0=1, s1=1, v_local=1, vocab_total=1)
    assert lib.ce_backward_inplace(ctypes.byref(x1), ctypes.byref(t), ctypes.byref(po), h.lse.ctypes.data, None,
                                   None, None) == _abi.CE_EINVAL
    assert lib.ce_shard_combine(h.stats.ctypes.data, 1, 2, 3, 1, ctypes.byref(t), ctypes.byref(po),
                                h.loss.ctypes.data, None, None, h.ws.ctypes.data, h.ws.nbytes, None) == _abi.CE_EINVAL
    # shard stats: misaligned stats, shard past the vocabulary
    assert lib.ce_shard_partial_stats(ctypes.byref(x), ctypes.byref(t), ctypes.byref(p), h.stats.ctypes.data + 4,
                                      None) == _abi.CE_ELAYOUT
    bad_shard = h.logits(vocab_start=60, vocab_total=64)
    assert lib.ce_shard_partial_stats(ctypes.byref(bad_shard), ctypes.byref(t), ctypes.byref(p),
                                      h.stats.ctypes.data, None) == _abi.CE_ELAYOUT
    # combine: S < 1, vocab_total < 1, small workspace
    assert lib.ce_shard_combine(h.stats.ctypes.data, 0, 2, 3, 64, ctypes.byref(t), ctypes.byref(p),
                                h.loss.ctypes.data, None, None, h.ws.ctypes.data, h.ws.nbytes, None) == _abi.CE_EINVAL
    assert lib.ce_shard_combine(h.stats.ctypes.data, 1, 2, 3, 0, ctypes.byref(t), ctypes.byref(p),
                                h.loss.ctypes.data, None, None, h.ws.ctypes.data, h.ws.nbytes, None) == _abi.CE_EINVAL
    assert lib.ce_shard_combine(h.stats.ctypes.data, 1, 2, 3, 64, ctypes.byref(t), ctypes.byref(p),
                                h.loss.ctypes.data, None, None, h.ws.ctypes.data, 8, None) == _abi.CE_EWORKSPACE
    assert h.untouched()


def test_workspace_sizes(lib):
    h = Host(N=8192, V=128000)
    x = h.logits(d0=4, d1=2048, s0=2048 * 128000, s1=128000)
    p = h.params(reduce_loss=1, label_smoothing=0.1)
    n = lib.ce_workspace_bytes(ctypes.byref(x), ctypes.byref(p))
    # header + FP32 losses of the split calls + the fused call's tagged losses
    # + 8 chunks (of 2000 of the 2048 vectors of a 256 x 8 workgroup) x 4 tagged words per row
    assert n == 256 + 8192 * 4 + 8192 * 8 + 8192 * 8 * 4 * 8
    # the sum keeps the same per-row losses as the mean
    assert lib.ce_workspace_bytes(ctypes.byref(x), ctypes.byref(h.params(reduce_loss=2, smoothing=1))) == n
    p0 = h.params()
    x1 = h.logits(d0=2, d1=512, s0=512 * 32000, s1=32000, v_local=32000, vocab_total=32000)
    # without the mean: header + the fused call's tagged losses (every call collects them)
    assert lib.ce_workspace_bytes(ctypes.byref(x1), ctypes.byref(p0)) == 256 + 1024 * 8
    assert lib.ce_workspace_bytes(ctypes.byref(h.logits(dtype=9)), ctypes.byref(p0)) == 0
    assert lib.ce_combine_workspace_bytes(512, ctypes.byref(h.params(reduce_loss=1))) == 256 + 2048
    # forced split: chunks of at most one workgroup
    p3 = h.params(split_chunks=3)
    x2 = h.logits(d0=1, d1=10, s0=40960, s1=4096, v_local=4096, vocab_total=4096)
    assert lib.ce_workspace_bytes(ctypes.byref(x2), ctypes.byref(p3)) == 256 + 256 + (10 * 3 * 4 * 8 + 255) // 256 * 256


def test_workspace_init_validates(lib):
    # rejected before any HIP call (no GPU needed): NULL, misaligned, too small, not a multiple of 8
    assert lib.ce_workspace_init(None, 4096, None) == _abi.CE_EINVAL
    assert lib.ce_workspace_init(ctypes.c_void_p(0x10000 + 8), 4096, None) == _abi.CE_EWORKSPACE
    assert lib.ce_workspace_init(ctypes.c_void_p(0x10000), 128, None) == _abi.CE_EWORKSPACE
    assert lib.ce_workspace_init(ctypes.c_void_p(0x10000), 4100, None) == _abi.CE_EWORKSPACE


# The automatic chunk count of a split row (the workspace holds 4 tagged 8-byte words per row and chunk): the
# count whose chunks fill their workgroup's registers best; between options within 1%, BF16 takes the
# 256-thread chunks while K stays at most 8, FP32 the fewer chunks.
AUTO_CHUNKS = [(_abi.CE_BF16, 49152, 3), (_abi.CE_BF16, 65536, 4), (_abi.CE_BF16, 100000, 7),
               (_abi.CE_BF16, 128000, 8), (_abi.CE_BF16, 152064, 5), (_abi.CE_BF16, 256000, 8),
               (_abi.CE_BF16, 32768, 1), (_abi.CE_F32, 65536, 4), (_abi.CE_F32, 128000, 8),
               (_abi.CE_F32, 16384, 1)]


@pytest.mark.parametrize("dtype,V,K", AUTO_CHUNKS, ids=[f"{'bf16' if d == _abi.CE_BF16 else 'f32'}-V{v}"
                                                        for d, v, _ in AUTO_CHUNKS])
def test_automatic_chunk_count(lib, dtype, V, K):
    h = Host(N=64, V=V)
    x = h.logits(dtype=dtype, d0=1, d1=64, s0=64 * V, s1=V)
    p = h.params()  # no reduction: header + tagged losses + the exchange words
    n = lib.ce_workspace_bytes(ctypes.byref(x), ctypes.byref(p))
    tagged = (256 + 64 * 8 + 255) // 256 * 256
    assert n == tagged + (64 * K * 4 * 8 if K > 1 else 0), (n, K)


def test_split_chunks_too_few_rejected(lib):
    # V = 600000 BF16 rows need at least 5 chunks of 16384 vectors; 4 cannot hold them
    h = Host()
    x = h.logits(d0=1, d1=2, s0=1200000, s1=600000, v_local=600000, vocab_total=600000)
    p = h.params(split_chunks=4)
    rc = lib.ce_fwd_bwd_fused(ctypes.byref(x), ctypes.byref(h.targets()), ctypes.byref(p), None,
                              h.loss.ctypes.data, None, h.ws.ctypes.data, h.ws.nbytes, None)
    assert rc == _abi.CE_ELAYOUT
    assert h.untouched()


def test_profile_calls_validate(lib):
    assert lib.ce_profile_stop(None, 0, None) == _abi.CE_EINVAL
    assert lib.ce_profile_start(0) == _abi.CE_EINVAL


def test_scale_grad_validates(lib):
    # rejected before any HIP call: NULL factor with rows, bad mode, bad dtype, NULL descriptor
    h = Host()
    g = np.full(h.N, 2.0, np.float32)
    assert lib.ce_scale_grad_inplace(ctypes.byref(h.logits()), None, 1, None) == _abi.CE_EINVAL
    assert lib.ce_scale_grad_inplace(ctypes.byref(h.logits()), g.ctypes.data, 2, None) == _abi.CE_EINVAL
    assert lib.ce_scale_grad_inplace(ctypes.byref(h.logits(dtype=9)), g.ctypes.data, 1, None) == _abi.CE_EDTYPE
    assert lib.ce_scale_grad_inplace(None, g.ctypes.data, 1, None) == _abi.CE_EINVAL
    assert h.untouched()


def test_stream_reference_validates(lib):
    # rejected before any HIP call (the pointers are never dereferenced on the host): a size that is
    # not a multiple of 16, NULL, misaligned and partly overlapping buffers; no bytes is a no-op
    a, b = 0x100000, 0x200000
    vp = ctypes.c_void_p
    assert lib.ce_stream_reference(vp(a), vp(b), 0, None) == _abi.CE_OK
    assert lib.ce_stream_reference(None, None, 0, None) == _abi.CE_OK
    assert lib.ce_stream_reference(vp(a), vp(b), 24, None) == _abi.CE_EINVAL
    assert lib.ce_stream_reference(vp(a), vp(b), -16, None) == _abi.CE_EINVAL
    assert lib.ce_stream_reference(None, vp(b), 32, None) == _abi.CE_EINVAL
    assert lib.ce_stream_reference(vp(a), None, 32, None) == _abi.CE_EINVAL
    assert lib.ce_stream_reference(vp(a + 8), vp(b), 32, None) == _abi.CE_EINVAL
    assert lib.ce_stream_reference(vp(a), vp(b + 4), 32, None) == _abi.CE_EINVAL
    assert lib.ce_stream_reference(vp(a), vp(a + 16), 32, None) == _abi.CE_EINVAL
    assert lib.ce_stream_reference(vp(a + 16), vp(a), 32, None) == _abi.CE_EINVAL
    assert b"overlap" in lib.ce_last_error()


def _linear_host(N=16, D=8, V=32):
    h = np.zeros((N, D), np.uint16)
    w = np.zeros((V, D), np.uint16)
    t = np.zeros(N, np.int64)
    return h, w, t


def test_linear_rejects_before_any_hip_call(lib):
    """ce_linear_cross_entropy checks everything on the host first."""
    h, w, t = _linear_host()
    loss = np.full(16, 7.0, np.float32)
    ws = np.zeros(1 << 12, np.uint8)

    def call(lin=None, p=None, t_ptr=t.ctypes.data, ts=1, dh=None, dh_ld=8, dw=None, dw_ld=8, acc=0, chunk=0,
             wsp=ws.ctypes.data, wsb=ws.nbytes):
        d = dict(h=h.ctypes.data, w=w.ctypes.data, dtype=_abi.CE_BF16, gemm=0, N=16, D=8, V=32, h_ld=8, w_ld=8)
        d.update(lin or {})
        q = dict(label_smoothing=0.0, reduce_loss=1, ignore_idx=-100, split_chunks=0, smoothing=0)
        q.update(p or {})
        return lib.ce_linear_cross_entropy(ctypes.byref(_abi.CeLinear(**d)), t_ptr, ts,
                                           ctypes.byref(_abi.CeParams(**q)), None, loss.ctypes.data, None, dh,
                                           dh_ld, dw, dw_ld, acc, chunk, wsp, wsb, None)

    assert call(lin=dict(dtype=3)) == _abi.CE_EDTYPE
    assert call(lin=dict(gemm=3)) == _abi.CE_EINVAL
    assert call(lin=dict(gemm=-1)) == _abi.CE_EINVAL
    assert call(lin=dict(D=0)) == _abi.CE_EINVAL
    assert call(lin=dict(h_ld=4)) == _abi.CE_ELAYOUT
    assert call(lin=dict(w=None)) == _abi.CE_EINVAL
    assert call(lin=dict(h=h.ctypes.data + 1)) == _abi.CE_ELAYOUT
    assert call(p=dict(split_chunks=2)) == _abi.CE_EINVAL
    assert call(p=dict(reduce_loss=7)) == _abi.CE_EINVAL
    assert call(p=dict(label_smoothing=2.0)) == _abi.CE_EINVAL
    assert call(lin=dict(V=1), p=dict(smoothing=1, label_smoothing=0.1)) == _abi.CE_EINVAL
    assert call(t_ptr=None) == _abi.CE_EINVAL
    assert call(dh=h.ctypes.data, dh_ld=4) == _abi.CE_ELAYOUT
    assert call(dw=w.ctypes.data, dw_ld=2) == _abi.CE_ELAYOUT
    assert call(acc=2) == _abi.CE_EINVAL
    assert call(wsb=64) == _abi.CE_EWORKSPACE
    assert call(wsp=None) == _abi.CE_EWORKSPACE
    assert lib.ce_last_error()
    assert np.all(loss == 7.0)


def test_linear_workspace_sizes(lib):
    h, w, t = _linear_host()
    lin = _abi.CeLinear(h.ctypes.data, w.ctypes.data, _abi.CE_BF16, 0, 8192, 4096, 128000, 4096, 4096)
    p = _abi.CeParams(0.1, 1, -100, 0, 0)
    rows = ctypes.c_int64(0)
    n = lib.ce_linear_workspace_bytes(ctypes.byref(lin), ctypes.byref(p), 0, ctypes.byref(rows))
    # automatic chunks of 4096 rows (about 1 GiB of BF16 logits), plus the fused call's words and GEMM scratch
    assert rows.value == 4096
    assert 4096 * 128000 * 2 < n < 4096 * 128000 * 2 + (128 << 20)
    n2 = lib.ce_linear_workspace_bytes(ctypes.byref(lin), ctypes.byref(p), 100, ctypes.byref(rows))
    assert rows.value == 100 and n2 < n
    lin.dtype = 9
    assert lib.ce_linear_workspace_bytes(ctypes.byref(lin), ctypes.byref(p), 0, None) == 0


def test_linear_tune_rejects_before_any_hip_call(lib):
    h, w, t = _linear_host()
    ws = np.zeros(1 << 12, np.uint8)
    lin = _abi.CeLinear(h.ctypes.data, w.ctypes.data, _abi.CE_BF16, 0, 16, 8, 32, 8, 8)
    p = _abi.CeParams(0.0, 1, -100, 0, 0)
    assert lib.ce_linear_tune(ctypes.byref(lin), ctypes.byref(p), None, 0, None, 0, 0, ws.ctypes.data, 64,
                              None) == _abi.CE_EWORKSPACE
    assert lib.ce_linear_tune(ctypes.byref(lin), ctypes.byref(p), h.ctypes.data, 4, None, 0, 0, ws.ctypes.data,
                              ws.nbytes, None) == _abi.CE_ELAYOUT
    bad = _abi.CeLinear(h.ctypes.data, w.ctypes.data, 5, 0, 16, 8, 32, 8, 8)
    assert lib.ce_linear_tune(ctypes.byref(bad), ctypes.byref(p), None, 0, None, 0, 0, ws.ctypes.data, ws.nbytes,
                              None) == _abi.CE_EDTYPE


def _shard_set(h, widths, change=None):
    """Shard descriptors over the host buffer: consecutive column ranges of widths."""
    V = sum(widths)
    arr = (_abi.CeLogits * len(widths))()
    start = 0
    for i, w in enumerate(widths):
        d = dict(data=h.x.ctypes.data + 2 * start, dtype=_abi.CE_BF16, reserved=0, d0=2, d1=h.N // 2,
                 s0=h.N // 2 * V, s1=V, v_local=w, vocab_start=start, vocab_total=V)
        d.update((change or {}).get(i, {}))
        arr[i] = _abi.CeLogits(**d)
        start += w
    return arr


BAD_SHARDS = [
    ("no_shards", dict(S=0), _abi.CE_EINVAL),
    ("too_many_shards", dict(widths=[1] * 17), _abi.CE_EINVAL),
    ("gap", dict(change={1: dict(vocab_start=9)}), _abi.CE_ELAYOUT),
    ("overlap", dict(change={1: dict(vocab_start=7)}), _abi.CE_ELAYOUT),
    ("short_cover", dict(change={1: dict(v_local=7)}), _abi.CE_ELAYOUT),
    ("dtype_mismatch", dict(change={1: dict(dtype=_abi.CE_F32)}), _abi.CE_ELAYOUT),
    ("rows_mismatch", dict(change={1: dict(d1=2)}), _abi.CE_ELAYOUT),
    ("vocab_total_mismatch", dict(change={1: dict(vocab_total=32)}), _abi.CE_ELAYOUT),
    ("bad_shard_stride", dict(change={1: dict(s1=4)}), _abi.CE_ELAYOUT),
    ("split_chunks", dict(p=dict(split_chunks=2)), _abi.CE_EINVAL),
    ("reduce_unknown", dict(p=dict(reduce_loss=5)), _abi.CE_EINVAL),
    ("small_workspace", dict(ws_bytes=16), _abi.CE_EWORKSPACE),
    ("no_workspace", dict(ws=False), _abi.CE_EWORKSPACE),
    ("null_targets", dict(t=dict(data=None)), _abi.CE_EINVAL),
]


@pytest.mark.parametrize("name,case,status", BAD_SHARDS, ids=[b[0] for b in BAD_SHARDS])
def test_shards_fused_rejects_before_any_hip_call(lib, name, case, status):
    h = Host()
    widths = case.get("widths", [8, 8])
    arr = _shard_set(h, widths, case.get("change"))
    S = case.get("S", len(arr))
    p = h.params(**case.get("p", {}))
    t = h.targets(**case.get("t", {}))
    rc = lib.ce_shards_fwd_bwd_fused(arr, S, ctypes.byref(t), ctypes.byref(p), None, h.loss.ctypes.data,
                                     h.n.ctypes.data, h.ws.ctypes.data if case.get("ws", True) else None,
                                     case.get("ws_bytes", h.ws.nbytes), None)
    assert rc == status, (rc, lib.ce_last_error())
    assert lib.ce_last_error()
    assert h.untouched()
    if "ws" not in case and "ws_bytes" not in case and "t" not in case:  # the shard set itself is refused
        assert lib.ce_shards_workspace_bytes(arr, S, ctypes.byref(p)) == 0


def test_shards_workspace_sizes(lib):
    h = Host(V=200)
    p = h.params()
    one = lib.ce_shards_workspace_bytes(_shard_set(h, [200]), 1, ctypes.byref(p))
    two = lib.ce_shards_workspace_bytes(_shard_set(h, [100, 100]), 2, ctypes.byref(p))
    assert 0 < one < two  # a second shard adds exchange slots per row
    # a vocabulary of at most 64 columns is one item per row (FP64, gathered): no exchange slots
    h = Host()
    assert (lib.ce_shards_workspace_bytes(_shard_set(h, [8, 8]), 2, ctypes.byref(p))
            == lib.ce_shards_workspace_bytes(_shard_set(h, [16]), 1, ctypes.byref(p)) > 0)
    # 16 shards is the most; up to 64 chunks per row in all
    assert lib.ce_shards_workspace_bytes(_shard_set(h, [1] * 16), 16, ctypes.byref(p)) > 0


def test_last_error_is_per_thread(lib):
    """ce_last_error's text belongs to the calling thread: two threads that
    fail differently at the same time each read their own message (ctypes
    releases the interpreter lock during the calls, so they interleave)."""
    import threading

    results = {}
    barrier = threading.Barrier(2)

    def worker(name, change, expect_status, expect_text):
        h = Host()
        x = h.logits(**change.get("x", {}))
        p = h.params(**change.get("p", {}))
        ok = True
        barrier.wait()
        for _ in range(2000):
            rc = _fused(lib, h, x=x, p=p)
            msg = lib.ce_last_error().decode()
            ok &= rc == expect_status and expect_text in msg
        results[name] = ok

    threads = [threading.Thread(target=worker, args=("dtype", dict(x=dict(dtype=7)), _abi.CE_EDTYPE, "dtype")),
               threading.Thread(target=worker, args=("reduce", dict(p=dict(reduce_loss=9)), _abi.CE_EINVAL,
                                                      "reduce"))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert results == {"dtype": True, "reduce": True}


def test_device_build_contracts_within_expressions_only():
    """The kernels round m log2(e) once and reuse that value so its rounding
    cancels between the sum's terms and its rescaling; hipcc's default
    contraction across statements would fuse the product, unrounded, into a
    later subtraction.  The device build must keep -ffp-contract=on."""
    import importlib.util
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "vocab_cross_entropy_amd", "csrc", "build.py")
    spec = importlib.util.spec_from_file_location("vce_build_flags", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert "-ffp-contract=on" in mod.DEVICE
    assert not any(f.startswith("-ffp-contract=") and f != "-ffp-contract=on" for f in mod.DEVICE + mod.COMMON)


def test_linear_gemm_plan(lib):
    """Which products run on the native MFMA kernel: every one for a BF16 head
    with 16-byte rows under CE_GEMM_NATIVE, dh and dW under CE_GEMM_AUTO; none
    under the library engine, for FP32 heads, or when D or a row stride is not
    a multiple of 8 or a base pointer not 16-byte aligned; -1 for an invalid
    descriptor."""
    h = np.zeros(16 * 64 + 8, np.uint16)
    w = np.zeros(32 * 64 + 8, np.uint16)
    hp = h.ctypes.data + (-h.ctypes.data) % 16
    wp = w.ctypes.data + (-w.ctypes.data) % 16

    def plan(**kw):
        d = dict(h=hp, w=wp, dtype=_abi.CE_BF16, gemm=_abi.CE_GEMM_NATIVE, N=16, D=64, V=32, h_ld=64, w_ld=64)
        d.update(kw)
        return lib.ce_linear_gemm_plan(ctypes.byref(_abi.CeLinear(**d)))

    assert plan() == 7
    assert plan(V=30001) == 7  # the logits stride is padded to a multiple of 8
    assert plan(N=0) == 7
    assert plan(gemm=_abi.CE_GEMM_LIBRARY) == 0
    assert plan(dtype=_abi.CE_F32) == 0
    assert plan(D=60, h_ld=64, w_ld=64) == 0
    assert plan(h_ld=68) == 0
    assert plan(w_ld=72) == 7
    assert plan(h=hp + 2) == 0
    assert plan(w=wp + 8) == 0
    assert plan(gemm=3) == -1
    assert plan(D=0) == -1
    assert plan(h_ld=32) == -1
    assert lib.ce_linear_gemm_plan(None) == -1
    # the automatic choice: the native kernel for dh and dW (bits 1 and 2), where it applies
    assert plan(gemm=_abi.CE_GEMM_AUTO) == 6
    assert plan(gemm=_abi.CE_GEMM_AUTO, dtype=_abi.CE_F32) == 0
    assert plan(gemm=_abi.CE_GEMM_AUTO, h=hp + 2) == 0
