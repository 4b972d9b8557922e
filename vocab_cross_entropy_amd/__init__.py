"""MI355X-native fused (vocabulary-parallel) cross-entropy.

Thin Python binding of the C ABI in ``include/ce.h`` (``libce.so``, built by
``vocab_cross_entropy_amd/csrc/build.py``).  The functions below only marshal torch
device tensors into the ABI's descriptors and pass torch's current HIP stream;
every step of the computation runs in the library's gfx950 kernels.  PyTorch
provides device memory and streams.

Entry points with the C names:
    ce_forward, ce_backward_inplace, ce_fwd_bwd_fused,
    ce_shard_partial_stats, ce_shard_combine
    (and ce_forward_ex, ce_backward_inplace_ex, ce_shard_combine_ex, which
    also hand the backward the lse residual and 1 - p_t)
and the interface of the TransformerEngineNPU issue #29 page (section 1):
    parallel_cross_entropy(inp, target, label_smoothing=0.0, reduce_loss=False,
                           dist_process_group=None, ignore_idx=-100)

``reduce_loss`` is False / True (the page's flag: per-row losses / their mean
over non-ignored rows) or one of "none", "mean", "sum".  ``smoothing`` (a
keyword) is "all" (a / V on every class, torch's convention) or "others"
(a / (V - 1) on every class but the target, the CANN ops-nn page's kernel).
"""
from __future__ import annotations

import ctypes
import functools
import weakref

import torch

from . import _abi
from ._abi import CE_BF16, CE_F32, CeArgumentError, CeError

__all__ = [
    "ce_forward", "ce_backward_inplace", "ce_fwd_bwd_fused", "ce_forward_ex", "ce_backward_inplace_ex",
    "ce_shard_combine_ex", "ce_fwd_bwd_fused_noalloc", "ce_scale_grad_inplace", "ce_shard_partial_stats",
    "ce_shard_combine", "ce_shards_fwd_bwd_fused", "ce_shards_workspace_bytes",
    "ce_workspace_bytes", "ce_combine_workspace_bytes", "ce_workspace_init", "ce_workspace_check",
    "ce_linear_workspace_bytes", "ce_linear_cross_entropy", "ce_linear_tune", "ce_linear_gemm_plan",
    "ce_stream_reference",
    "parallel_cross_entropy", "linear_cross_entropy",
    "Profiler", "CeError", "CeArgumentError", "lib", "ShardedCrossEntropy", "sharded_cross_entropy",
]

lib = _abi.load()

_ARG_ERRORS = {_abi.CE_EINVAL, _abi.CE_EDTYPE, _abi.CE_ELAYOUT, _abi.CE_EWORKSPACE}


def _check(status: int):
    if status != _abi.CE_OK:
        detail = lib.ce_last_error().decode(errors="replace")
        cls = CeArgumentError if status in _ARG_ERRORS else CeError
        raise cls(status, detail)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# torch's current HIP stream of a device as a raw handle: the raw accessor
# costs ~0.1 us a call against ~2 us for building a torch Stream object
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device):
    if _raw_stream is not None:
        idx = device.index if device.index is not None else torch.cuda.current_device()
        return ctypes.c_void_p(_raw_stream(idx))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _device_of(x, what="logits") -> torch.device:
    """The GPU device of ``x``; anything else is refused before the library
    sees a pointer (a host pointer handed to a kernel would fault the GPU)."""
    if not isinstance(x, torch.Tensor):
        raise CeArgumentError(_abi.CE_EINVAL, f"{what} must be a torch tensor")
    if x.device.type != "cuda":
        raise CeArgumentError(_abi.CE_EINVAL, f"{what} must be a GPU tensor, got one on {x.device}")
    return x.device


def _need(dev: torch.device, what: str, v, dtype=None, numel=0, contiguous=True):
    """``v`` (a tensor or None) lives on ``dev``, has ``dtype`` and holds at
    least ``numel`` elements (contiguous ones, for the flat buffers)."""
    if v is None:
        return
    # the common case in one test (the integer device index: a host tensor's is -1); the detailed
    # checks below only name what failed
    if (isinstance(v, torch.Tensor) and v.get_device() == dev.index and (dtype is None or v.dtype == dtype)
            and v.numel() >= numel and (not contiguous or v.is_contiguous())):
        return
    if not isinstance(v, torch.Tensor):
        raise CeArgumentError(_abi.CE_EINVAL, f"{what} must be a torch tensor")
    if v.device != dev:
        raise CeArgumentError(_abi.CE_EINVAL, f"{what} is on {v.device}, the logits on {dev}")
    if dtype is not None and v.dtype != dtype:
        raise CeArgumentError(_abi.CE_EINVAL, f"{what} must be {dtype}, got {v.dtype}")
    if v.numel() < numel:
        raise CeArgumentError(_abi.CE_EINVAL, f"{what} holds {v.numel()} elements, {numel} needed")
    if contiguous and not v.is_contiguous():
        raise CeArgumentError(_abi.CE_ELAYOUT, f"{what} must be contiguous")


def _need_targets(dev: torch.device, t, d0: int, d1: int):
    _need(dev, "targets", t, torch.int64, contiguous=False)
    if t is None or t.shape != (d0, d1):
        raise CeArgumentError(_abi.CE_EINVAL, f"targets must be a ({d0}, {d1}) int64 tensor")


def _need_ws(dev: torch.device, ws):
    _need(dev, "workspace", ws, torch.uint8)


def _dtype_code(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return CE_F32
    if x.dtype == torch.bfloat16:
        return CE_BF16
    return -1  # rejected by the library with CE_EDTYPE


def logits_desc(x: torch.Tensor, vocab_start: int = 0, vocab_total: int | None = None) -> _abi.CeLogits:
    """Descriptor of a (d0, d1, V) logits view; columns must be contiguous."""
    sh, st = x.shape, x.stride()
    if len(sh) != 3:
        raise CeArgumentError(_abi.CE_EINVAL, "logits must be a 3-d (d0, d1, V) tensor")
    d0, d1, v = sh
    if st[2] != 1 and v > 1:
        raise CeArgumentError(_abi.CE_ELAYOUT, "logits columns must be contiguous (stride 1)")
    return _abi.CeLogits(x.data_ptr(), _dtype_code(x), 0, d0, d1, st[0], st[1], v, vocab_start,
                         v if vocab_total is None else vocab_total)


def targets_desc(t: torch.Tensor) -> _abi.CeTargets:
    st = t.stride()
    if len(st) != 2 or t.dtype != torch.int64:
        raise CeArgumentError(_abi.CE_EINVAL, "targets must be a 2-d int64 tensor")
    return _abi.CeTargets(t.data_ptr(), st[0], st[1])


_REDUCTIONS = {"none": _abi.CE_REDUCE_NONE, "mean": _abi.CE_REDUCE_MEAN, "sum": _abi.CE_REDUCE_SUM}
_SMOOTHINGS = {"all": _abi.CE_SMOOTH_ALL, "others": _abi.CE_SMOOTH_OTHERS}


def reduction_code(reduce_loss) -> int:
    """False / True / "none" / "mean" / "sum" -> CE_REDUCE_*."""
    if isinstance(reduce_loss, str):
        if reduce_loss not in _REDUCTIONS:
            raise CeArgumentError(_abi.CE_EINVAL, f"reduce_loss {reduce_loss!r} is not one of {sorted(_REDUCTIONS)}")
        return _REDUCTIONS[reduce_loss]
    return _abi.CE_REDUCE_MEAN if reduce_loss else _abi.CE_REDUCE_NONE


def _smoothing_code(smoothing: str) -> int:
    if smoothing not in _SMOOTHINGS:
        raise CeArgumentError(_abi.CE_EINVAL, f"smoothing {smoothing!r} is not one of {sorted(_SMOOTHINGS)}")
    return _SMOOTHINGS[smoothing]


def params(label_smoothing=0.0, reduce_loss=False, ignore_idx=-100, split_chunks=0, smoothing="all") -> _abi.CeParams:
    """A parameter block (shared per distinct value; the library only reads it)."""
    return _params(float(label_smoothing), reduction_code(reduce_loss), int(ignore_idx), int(split_chunks),
                   _smoothing_code(smoothing))


@functools.lru_cache(maxsize=256)
def _params(label_smoothing: float, reduce_code: int, ignore_idx: int, split_chunks: int,
            smoothing_code: int) -> _abi.CeParams:
    return _abi.CeParams(label_smoothing, reduce_code, ignore_idx, split_chunks, smoothing_code)


def _f32(n, device):
    return torch.empty(n, dtype=torch.float32, device=device)


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# Workspace tensors this binding has prepared with ce_workspace_init, by
# object identity (id -> weak reference; a new tensor over reused memory is
# prepared again).  Not a WeakSet: that compares tensors with ==.
_prepared: dict[int, weakref.ref] = {}


def _is_prepared(ws: torch.Tensor) -> bool:
    r = _prepared.get(id(ws))
    return r is not None and r() is ws


def ce_workspace_init(ws: torch.Tensor) -> torch.Tensor:
    """Prepare ``ws`` (uint8 device tensor) for ce_fwd_bwd_fused; once is enough."""
    _need_ws(_device_of(ws, "workspace"), ws)
    _check(lib.ce_workspace_init(_ptr(ws), ws.numel(), _stream(ws.device)))
    for k in [k for k, r in _prepared.items() if r() is None]:
        del _prepared[k]
    _prepared[id(ws)] = weakref.ref(ws)
    return ws


def ce_workspace_bytes(x: torch.Tensor, label_smoothing=0.0, reduce_loss=False, ignore_idx=-100,
                       split_chunks=0, smoothing="all") -> int:
    n = lib.ce_workspace_bytes(ctypes.byref(logits_desc(x)),
                               ctypes.byref(params(label_smoothing, reduce_loss, ignore_idx, split_chunks,
                                                   smoothing)))
    if n == 0:
        _check(_abi.CE_EINVAL)
    return int(n)


def ce_combine_workspace_bytes(rows: int, reduce_loss=False) -> int:
    n = lib.ce_combine_workspace_bytes(int(rows), ctypes.byref(params(reduce_loss=reduce_loss)))
    if n == 0:
        _check(_abi.CE_EINVAL)
    return int(n)


def _forward(x, t, label_smoothing, reduce_loss, ignore_idx, loss, lse, lse_aux, n_valid, ws, want_lse, want_aux,
             smoothing):
    dev = _device_of(x)
    N = x.shape[0] * x.shape[1]
    _need_targets(dev, t, x.shape[0], x.shape[1])
    p = params(label_smoothing, reduce_loss, ignore_idx, smoothing=smoothing)
    loss = _f32(1 if p.reduce_loss else N, dev) if loss is None else loss
    if lse is None and want_lse:
        lse = _f32(N, dev)
    if lse_aux is None and want_aux:
        lse_aux = torch.empty((N, 2), dtype=torch.float32, device=dev)
    n_valid = torch.empty(1, dtype=torch.int32, device=dev) if n_valid is None else n_valid
    _need(dev, "loss", loss, torch.float32, 1 if p.reduce_loss else N)
    _need(dev, "lse", lse, torch.float32, N)
    _need(dev, "lse_aux", lse_aux, torch.float32, 2 * N)
    _need(dev, "n_valid", n_valid, torch.int32, 1)
    xd = logits_desc(x)
    if ws is None:
        ws = _workspace(lib.ce_workspace_bytes(ctypes.byref(xd), ctypes.byref(p)), dev)
    _need_ws(dev, ws)
    _check(lib.ce_forward_ex(ctypes.byref(xd), ctypes.byref(targets_desc(t)), ctypes.byref(p), _ptr(loss),
                             _ptr(lse), _ptr(lse_aux), _ptr(n_valid), _ptr(ws), ws.numel(), _stream(dev)))
    return loss, lse, lse_aux, n_valid


def ce_forward(x, t, label_smoothing=0.0, reduce_loss=False, ignore_idx=-100, *, loss=None, lse=None,
               n_valid=None, ws=None, want_lse=True, smoothing="all"):
    """Forward only.  Returns (loss [N] or [1], lse [N] or None, n_valid [1])."""
    loss, lse, _, n_valid = _forward(x, t, label_smoothing, reduce_loss, ignore_idx, loss, lse, None, n_valid, ws,
                                     want_lse, False, smoothing)
    return loss, lse, n_valid


def ce_forward_ex(x, t, label_smoothing=0.0, reduce_loss=False, ignore_idx=-100, *, loss=None, lse=None,
                  lse_aux=None, n_valid=None, ws=None, smoothing="all"):
    """Forward with the backward hand-off.  Returns (loss, lse [N], lse_aux
    [N, 2] = (lse residual, 1 - p_t), n_valid [1]); ce_backward_inplace_ex
    takes lse and lse_aux."""
    return _forward(x, t, label_smoothing, reduce_loss, ignore_idx, loss, lse, lse_aux, n_valid, ws, True, True,
                    smoothing)


def ce_backward_inplace_ex(x, t, lse, lse_aux, label_smoothing=0.0, reduce_loss=False, ignore_idx=-100, *,
                           grad_out=None, n_valid=None, vocab_start=0, vocab_total=None, smoothing="all"):
    """Writes the gradient over ``x`` (which may be a vocabulary shard) from
    the forward's lse and, when not None, its lse_aux pair."""
    dev = _device_of(x)
    N = x.shape[0] * x.shape[1]
    _need_targets(dev, t, x.shape[0], x.shape[1])
    p = params(label_smoothing, reduce_loss, ignore_idx, smoothing=smoothing)
    _need(dev, "lse", lse, torch.float32, N)
    _need(dev, "lse_aux", lse_aux, torch.float32, 2 * N)
    _need(dev, "grad_out", grad_out, torch.float32, N if p.reduce_loss == _abi.CE_REDUCE_NONE else 1)
    _need(dev, "n_valid", n_valid, torch.int32, 1)
    _check(lib.ce_backward_inplace_ex(ctypes.byref(logits_desc(x, vocab_start, vocab_total)),
                                      ctypes.byref(targets_desc(t)), ctypes.byref(p), _ptr(lse), _ptr(lse_aux),
                                      _ptr(grad_out), _ptr(n_valid), _stream(dev)))
    return x


def ce_backward_inplace(x, t, lse, label_smoothing=0.0, reduce_loss=False, ignore_idx=-100, *, grad_out=None,
                        n_valid=None, vocab_start=0, vocab_total=None, smoothing="all"):
    """Writes the gradient over ``x`` (which may be a vocabulary shard) from the lse alone."""
    return ce_backward_inplace_ex(x, t, lse, None, label_smoothing, reduce_loss, ignore_idx, grad_out=grad_out,
                                  n_valid=n_valid, vocab_start=vocab_start, vocab_total=vocab_total,
                                  smoothing=smoothing)


def ce_fwd_bwd_fused(x, t, label_smoothing=0.0, reduce_loss=False, ignore_idx=-100, *, grad_out=None, loss=None,
                     n_valid=None, ws=None, split_chunks=0, smoothing="all"):
    """Loss and, in place over ``x``, the gradient.  Returns (loss, n_valid).

    The sum over a global count of valid tokens (data-parallel training):
    ``reduce_loss="sum"`` with ``grad_out`` = [1 / count] gives that gradient
    with one rounding; ``loss / count`` is the normalised loss."""
    dev = _device_of(x)
    N = x.shape[0] * x.shape[1]
    _need_targets(dev, t, x.shape[0], x.shape[1])
    p = params(label_smoothing, reduce_loss, ignore_idx, split_chunks, smoothing)
    loss = _f32(1 if p.reduce_loss else N, dev) if loss is None else loss
    n_valid = torch.empty(1, dtype=torch.int32, device=dev) if n_valid is None else n_valid
    _need(dev, "grad_out", grad_out, torch.float32, N if p.reduce_loss == _abi.CE_REDUCE_NONE else 1)
    _need(dev, "loss", loss, torch.float32, 1 if p.reduce_loss else N)
    _need(dev, "n_valid", n_valid, torch.int32, 1)
    xd = logits_desc(x)
    if ws is None:
        nb = lib.ce_workspace_bytes(ctypes.byref(xd), ctypes.byref(p))
        if nb == 0:
            _check(_abi.CE_EINVAL)
        ws = _workspace(nb, dev)
    _need_ws(dev, ws)
    if not _is_prepared(ws):
        ce_workspace_init(ws)
    _check(lib.ce_fwd_bwd_fused(ctypes.byref(xd), ctypes.byref(targets_desc(t)), ctypes.byref(p), _ptr(grad_out),
                                _ptr(loss), _ptr(n_valid), _ptr(ws), ws.numel(), _stream(dev)))
    return loss, n_valid


def ce_fwd_bwd_fused_noalloc(x, t, label_smoothing=0.0, reduce_loss=False, ignore_idx=-100, *, grad_out=None,
                             loss, n_valid, split_chunks=0, smoothing="all"):
    """ce_fwd_bwd_fused with the library's static per-device scratch as its
    workspace: nothing is allocated, so ``loss`` and ``n_valid`` must be
    given.  Returns (loss, n_valid)."""
    dev = _device_of(x)
    N = x.shape[0] * x.shape[1]
    _need_targets(dev, t, x.shape[0], x.shape[1])
    p = params(label_smoothing, reduce_loss, ignore_idx, split_chunks, smoothing)
    _need(dev, "grad_out", grad_out, torch.float32, N if p.reduce_loss == _abi.CE_REDUCE_NONE else 1)
    _need(dev, "loss", loss, torch.float32, 1 if p.reduce_loss else N)
    _need(dev, "n_valid", n_valid, torch.int32, 1)
    _check(lib.ce_fwd_bwd_fused_noalloc(ctypes.byref(logits_desc(x)), ctypes.byref(targets_desc(t)),
                                        ctypes.byref(p), _ptr(grad_out), _ptr(loss), _ptr(n_valid), _stream(dev)))
    return loss, n_valid


def _shard_descs(shards):
    """(d0, d1, V_s) shard views in vocabulary order -> a ctypes array of descriptors."""
    if not shards:
        raise CeArgumentError(_abi.CE_EINVAL, "at least one shard is needed")
    total = sum(int(x.shape[2]) for x in shards)
    arr = (_abi.CeLogits * len(shards))()
    start = 0
    for i, x in enumerate(shards):
        arr[i] = logits_desc(x, start, total)
        start += int(x.shape[2])
    return arr


def ce_shards_workspace_bytes(shards, label_smoothing=0.0, reduce_loss=False, ignore_idx=-100,
                              smoothing="all") -> int:
    arr = _shard_descs(shards)
    n = lib.ce_shards_workspace_bytes(arr, len(shards), ctypes.byref(params(label_smoothing, reduce_loss,
                                                                             ignore_idx, 0, smoothing)))
    if n == 0:
        _check(_abi.CE_EINVAL)
    return int(n)


def ce_shards_fwd_bwd_fused(shards, t, label_smoothing=0.0, reduce_loss=False, ignore_idx=-100, *, grad_out=None,
                            loss=None, n_valid=None, ws=None, smoothing="all"):
    """The shard flow in one launch: ``shards`` are the (d0, d1, V_s) pieces of
    the logits in vocabulary order (separate tensors); each is read once and
    receives its gradient in place.  Returns (loss, n_valid)."""
    arr = _shard_descs(shards)
    d0, d1, _ = shards[0].shape
    N = d0 * d1
    dev = _device_of(shards[0], "shard 0")
    for i, x in enumerate(shards):
        _need(dev, f"shard {i}", x, contiguous=False)
    _need_targets(dev, t, d0, d1)
    p = params(label_smoothing, reduce_loss, ignore_idx, 0, smoothing)
    loss = _f32(1 if p.reduce_loss else N, dev) if loss is None else loss
    n_valid = torch.empty(1, dtype=torch.int32, device=dev) if n_valid is None else n_valid
    _need(dev, "grad_out", grad_out, torch.float32, N if p.reduce_loss == _abi.CE_REDUCE_NONE else 1)
    _need(dev, "loss", loss, torch.float32, 1 if p.reduce_loss else N)
    _need(dev, "n_valid", n_valid, torch.int32, 1)
    _need_ws(dev, ws)
    if ws is None:
        nb = lib.ce_shards_workspace_bytes(arr, len(shards), ctypes.byref(p))
        if nb == 0:
            _check(_abi.CE_EINVAL)
        ws = _workspace(nb, dev)
    if not _is_prepared(ws):
        ce_workspace_init(ws)
    _check(lib.ce_shards_fwd_bwd_fused(arr, len(shards), ctypes.byref(targets_desc(t)), ctypes.byref(p),
                                       _ptr(grad_out), _ptr(loss), _ptr(n_valid), _ptr(ws), ws.numel(), _stream(dev)))
    return loss, n_valid


def ce_scale_grad_inplace(x, grad_out: torch.Tensor, per_row: bool):
    """Multiply the gradient staged in ``x`` by ``grad_out`` ([N] per row, or
    [1]) in place; rows whose factor is exactly 1 are not touched."""
    dev = _device_of(x)
    g = grad_out.to(device=dev, dtype=torch.float32).reshape(-1).contiguous()
    _need(dev, "grad_out", g, torch.float32, x.shape[0] * x.shape[1] if per_row else 1)
    _check(lib.ce_scale_grad_inplace(ctypes.byref(logits_desc(x)), _ptr(g), int(bool(per_row)), _stream(dev)))
    return x


def ce_stream_reference(src: torch.Tensor, dst: torch.Tensor | None = None):
    """The library's reference streaming pass over ``src``'s bytes (a benchmark
    aid): with ``dst`` None every 32-bit word is XORed with 0x80008000 in
    place, else ``src`` is copied into ``dst`` (same byte count, no overlap).
    Contiguous tensors on one GPU, a multiple of 16 bytes, 16-byte aligned."""
    dev = _device_of(src, "src")
    if not src.is_contiguous():
        raise CeArgumentError(_abi.CE_EINVAL, "src must be contiguous")
    nbytes = src.numel() * src.element_size()
    if dst is not None:
        if _device_of(dst, "dst") != dev or not dst.is_contiguous():
            raise CeArgumentError(_abi.CE_EINVAL, "dst must be contiguous on src's device")
        if dst.numel() * dst.element_size() != nbytes:
            raise CeArgumentError(_abi.CE_EINVAL, "dst must hold as many bytes as src")
    _check(lib.ce_stream_reference(_ptr(src), _ptr(src if dst is None else dst), nbytes, _stream(dev)))
    return src if dst is None else dst


def ce_shard_partial_stats(shard, t, vocab_start, vocab_total, ignore_idx=-100, *, stats=None):
    """(m, d, y, r) per row of one vocabulary shard, as a [N, 4] FP32 tensor."""
    dev = _device_of(shard, "shard")
    N = shard.shape[0] * shard.shape[1]
    _need_targets(dev, t, shard.shape[0], shard.shape[1])
    stats = torch.empty((N, 4), dtype=torch.float32, device=dev) if stats is None else stats
    _need(dev, "stats", stats, torch.float32, 4 * N)
    p = params(ignore_idx=ignore_idx)
    _check(lib.ce_shard_partial_stats(ctypes.byref(logits_desc(shard, vocab_start, vocab_total)),
                                      ctypes.byref(targets_desc(t)), ctypes.byref(p), _ptr(stats), _stream(dev)))
    return stats


def _combine(stats, t, vocab_total, label_smoothing, reduce_loss, ignore_idx, loss, lse, lse_aux, n_valid, ws,
             want_aux, smoothing):
    dev = _device_of(stats, "stats")
    if stats.dim() != 3 or stats.shape[2] != 4:
        raise CeArgumentError(_abi.CE_EINVAL, "stats must be an [S, N, 4] tensor")
    S = stats.shape[0]
    _need(dev, "targets", t, torch.int64, contiguous=False)
    if t is None or t.dim() != 2:
        raise CeArgumentError(_abi.CE_EINVAL, "targets must be a 2-d int64 tensor")
    d0, d1 = t.shape
    N = d0 * d1
    p = params(label_smoothing, reduce_loss, ignore_idx, smoothing=smoothing)
    loss = _f32(1 if p.reduce_loss else N, dev) if loss is None else loss
    lse = _f32(N, dev) if lse is None else lse
    if lse_aux is None and want_aux:
        lse_aux = torch.empty((N, 2), dtype=torch.float32, device=dev)
    n_valid = torch.empty(1, dtype=torch.int32, device=dev) if n_valid is None else n_valid
    if ws is None:
        ws = _workspace(ce_combine_workspace_bytes(N, reduce_loss), dev)
    _need(dev, "stats", stats, torch.float32, 4 * S * N)
    _need(dev, "loss", loss, torch.float32, 1 if p.reduce_loss else N)
    _need(dev, "lse", lse, torch.float32, N)
    _need(dev, "lse_aux", lse_aux, torch.float32, 2 * N)
    _need(dev, "n_valid", n_valid, torch.int32, 1)
    _need_ws(dev, ws)
    _check(lib.ce_shard_combine_ex(_ptr(stats), S, d0, d1, int(vocab_total), ctypes.byref(targets_desc(t)),
                                   ctypes.byref(p), _ptr(loss), _ptr(lse), _ptr(lse_aux), _ptr(n_valid), _ptr(ws),
                                   ws.numel(), _stream(dev)))
    return loss, lse, lse_aux, n_valid


def ce_shard_combine(stats, t, vocab_total, label_smoothing=0.0, reduce_loss=False, ignore_idx=-100, *, loss=None,
                     lse=None, n_valid=None, ws=None, smoothing="all"):
    """Combine stats [S, N, 4] into (loss, lse [N], n_valid [1])."""
    loss, lse, _, n_valid = _combine(stats, t, vocab_total, label_smoothing, reduce_loss, ignore_idx, loss, lse,
                                     None, n_valid, ws, False, smoothing)
    return loss, lse, n_valid


def ce_shard_combine_ex(stats, t, vocab_total, label_smoothing=0.0, reduce_loss=False, ignore_idx=-100, *,
                        loss=None, lse=None, lse_aux=None, n_valid=None, ws=None, smoothing="all"):
    """Combine stats [S, N, 4] into (loss, lse [N], lse_aux [N, 2], n_valid
    [1]); lse and lse_aux are the per-shard backward's hand-off."""
    return _combine(stats, t, vocab_total, label_smoothing, reduce_loss, ignore_idx, loss, lse, lse_aux, n_valid,
                    ws, True, smoothing)


_GEMM = {"auto": _abi.CE_GEMM_AUTO, "native": _abi.CE_GEMM_NATIVE, "library": _abi.CE_GEMM_LIBRARY}


def _gemm_code(gemm: str) -> int:
    if gemm not in _GEMM:
        raise CeArgumentError(_abi.CE_EINVAL, f"gemm must be one of {sorted(_GEMM)}, got {gemm!r}")
    return _GEMM[gemm]


def linear_desc(h: torch.Tensor, w: torch.Tensor, gemm: str = "auto") -> _abi.CeLinear:
    """[N, D] hidden states and the [V, D] head weight (rows may be strided, columns contiguous); ``gemm``
    picks the products' engine: "auto", "native" (the library's MFMA kernel where it applies) or
    "library" (hipBLASLt)."""
    if h.dim() != 2 or w.dim() != 2 or h.shape[1] != w.shape[1]:
        raise CeArgumentError(_abi.CE_EINVAL, f"need h [N, D] and w [V, D], got {tuple(h.shape)} and {tuple(w.shape)}")
    if h.dtype != w.dtype:
        raise CeArgumentError(_abi.CE_EDTYPE, f"h is {h.dtype}, w is {w.dtype}")
    if (h.shape[0] > 1 and h.stride(1) != 1) or w.stride(1) != 1:
        raise CeArgumentError(_abi.CE_ELAYOUT, "h and w need contiguous columns")
    N, D = h.shape
    return _abi.CeLinear(_ptr(h), _ptr(w), _dtype_code(h), _gemm_code(gemm), N, D, w.shape[0], max(h.stride(0), D),
                         max(w.stride(0), D))


def ce_linear_gemm_plan(h, w, gemm="auto") -> int:
    """Bit mask of the products ce_linear_cross_entropy runs on the library's MFMA kernel for these
    operands and engine: 1 logits, 2 dh, 4 dW."""
    plan = lib.ce_linear_gemm_plan(ctypes.byref(linear_desc(h, w, gemm)))
    if plan < 0:
        _check(_abi.CE_EINVAL)
    return int(plan)


def ce_linear_workspace_bytes(h, w, reduce_loss=False, chunk_rows=0, label_smoothing=0.0, ignore_idx=-100,
                              smoothing="all"):
    """(bytes, chunk rows) of ce_linear_cross_entropy's workspace."""
    got = ctypes.c_int64(0)
    n = lib.ce_linear_workspace_bytes(ctypes.byref(linear_desc(h, w)),
                                      ctypes.byref(params(label_smoothing, reduce_loss, ignore_idx, 0, smoothing)),
                                      int(chunk_rows), ctypes.byref(got))
    if n == 0:
        _check(_abi.CE_EINVAL)
    return int(n), int(got.value)


def ce_linear_cross_entropy(h, w, t, label_smoothing=0.0, reduce_loss=False, ignore_idx=-100, *, grad_out=None,
                            loss=None, n_valid=None, dh=None, dw=None, want_dh=True, want_dw=True,
                            accumulate_dw=False, chunk_rows=0, ws=None, smoothing="all", gemm="auto"):
    """Loss of the head h W^T over row chunks, with dh = dL/dh (input dtype) and
    dw = dL/dW (FP32, or added to ``dw`` with ``accumulate_dw``).  ``t`` is
    the [N] int64 targets (any stride); ``gemm`` the products' engine (see
    linear_desc).  Returns (loss, dh, dw, n_valid)."""
    N, D = h.shape
    V = w.shape[0]
    dev = _device_of(h, "h")
    _need(dev, "w", w, contiguous=False)
    _need(dev, "targets", t, torch.int64, contiguous=False)
    p = params(label_smoothing, reduce_loss, ignore_idx, 0, smoothing)
    loss = _f32(1 if p.reduce_loss else N, dev) if loss is None else loss
    n_valid = torch.empty(1, dtype=torch.int32, device=dev) if n_valid is None else n_valid
    _need(dev, "grad_out", grad_out, torch.float32, N if p.reduce_loss == _abi.CE_REDUCE_NONE else 1)
    _need(dev, "loss", loss, torch.float32, 1 if p.reduce_loss else N)
    _need(dev, "n_valid", n_valid, torch.int32, 1)
    _need(dev, "dh", dh, contiguous=False)
    _need(dev, "dw", dw, contiguous=False)
    _need_ws(dev, ws)
    if dh is None and want_dh:
        dh = torch.empty((N, D), dtype=h.dtype, device=dev)
    if dw is None and want_dw:
        dw = torch.empty((V, D), dtype=torch.float32, device=dev)
    if dh is not None and (dh.dtype != h.dtype or dh.shape != h.shape or dh.stride(1) != 1):
        raise CeArgumentError(_abi.CE_ELAYOUT, "dh must be [N, D] in h's dtype with contiguous columns")
    if dw is not None and (dw.dtype != torch.float32 or tuple(dw.shape) != (V, D) or dw.stride(1) != 1):
        raise CeArgumentError(_abi.CE_ELAYOUT, "dw must be an FP32 [V, D] tensor with contiguous columns")
    if t.dim() != 1 or t.numel() != N or t.dtype != torch.int64:
        raise CeArgumentError(_abi.CE_EINVAL, "targets must be an int64 [N] tensor")
    desc = linear_desc(h, w, gemm)
    if ws is None:
        nb = lib.ce_linear_workspace_bytes(ctypes.byref(desc), ctypes.byref(p), int(chunk_rows), None)
        if nb == 0:
            _check(_abi.CE_EINVAL)
        ws = _workspace(nb, dev)
    if not _is_prepared(ws):
        ce_workspace_init(ws)
    _check(lib.ce_linear_cross_entropy(ctypes.byref(desc), _ptr(t), t.stride(0) if N > 1 else 1, ctypes.byref(p),
                                       _ptr(grad_out), _ptr(loss), _ptr(n_valid), _ptr(dh),
                                       dh.stride(0) if dh is not None else 0, _ptr(dw),
                                       dw.stride(0) if dw is not None else 0, int(bool(accumulate_dw)),
                                       int(chunk_rows), _ptr(ws), ws.numel(), _stream(dev)))
    return loss, dh, dw, n_valid


def ce_linear_tune(h, w, reduce_loss="mean", *, dh=None, dw=None, want_dh=True, want_dw=True, chunk_rows=0,
                   ws=None, label_smoothing=0.0, smoothing="all", gemm="auto"):
    """Time the GEMM library's candidates for the chunked call's shapes on
    these buffers and keep the fastest (synchronises; dh and dw receive
    scratch values).  Returns the workspace it used, which the calls can share."""
    N, D = h.shape
    V = w.shape[0]
    dev = _device_of(h, "h")
    _need(dev, "w", w, contiguous=False)
    _need(dev, "dh", dh, contiguous=False)
    _need(dev, "dw", dw, contiguous=False)
    _need_ws(dev, ws)
    p = params(label_smoothing, reduce_loss, -100, 0, smoothing)
    if dh is None and want_dh:
        dh = torch.empty((N, D), dtype=h.dtype, device=dev)
    if dw is None and want_dw:
        dw = torch.empty((V, D), dtype=torch.float32, device=dev)
    desc = linear_desc(h, w, gemm)
    if ws is None:
        nb = lib.ce_linear_workspace_bytes(ctypes.byref(desc), ctypes.byref(p), int(chunk_rows), None)
        if nb == 0:
            _check(_abi.CE_EINVAL)
        ws = _workspace(nb, dev)
    if not _is_prepared(ws):
        ce_workspace_init(ws)
    _check(lib.ce_linear_tune(ctypes.byref(desc), ctypes.byref(p), _ptr(dh), dh.stride(0) if dh is not None else 0,
                              _ptr(dw), dw.stride(0) if dw is not None else 0, int(chunk_rows), _ptr(ws), ws.numel(),
                              _stream(dev)))
    return ws


def ce_workspace_check(ws: torch.Tensor):
    """Raises CeError(CE_EDEADLOCK) if a call since the last check gave up
    waiting, CeArgumentError(CE_EWORKSPACE) if a fused call found ``ws``
    unprepared; clears that record.  Synchronises the stream."""
    _device_of(ws, "workspace")
    _check(lib.ce_workspace_check(_ptr(ws), _stream(ws.device)))


class ParallelCrossEntropy(torch.autograd.Function):
    """Autograd form of the fused call (TENPU #29 sections 1 and 6).

    Forward: one ce_fwd_bwd_fused call computes the FP32 loss and writes the
    gradient for an upstream gradient of 1 over ``inp`` (in its dtype, in
    place: no N x V gradient buffer is allocated).  Backward: the staged
    gradient times the upstream gradient, in place, through
    ce_scale_grad_inplace, which leaves rows whose factor is exactly 1
    untouched (no host synchronisation to find them); ``inp``'s storage is
    returned as the gradient.  After the forward, ``inp`` holds the gradient,
    not the logits.
    """

    @staticmethod
    def forward(ctx, inp, target, label_smoothing=0.0, reduce_loss=False, ignore_idx=-100, smoothing="all"):
        buf = inp.detach()
        loss, _ = ce_fwd_bwd_fused(buf, target, label_smoothing, reduce_loss, ignore_idx, smoothing=smoothing)
        ctx.reduced = reduction_code(reduce_loss) != _abi.CE_REDUCE_NONE
        ctx.save_for_backward(buf)
        return loss[0] if ctx.reduced else loss.view(target.shape)

    @staticmethod
    def backward(ctx, grad_loss):
        (buf,) = ctx.saved_tensors
        ce_scale_grad_inplace(buf, grad_loss, per_row=not ctx.reduced)
        return buf, None, None, None, None, None


def parallel_cross_entropy(inp, target, label_smoothing=0.0, reduce_loss=False, dist_process_group=None,
                           ignore_idx=-100, *, smoothing="all"):
    """The issue #29 interface: FP32 loss (per row in ``target``'s shape, or
    their mean over non-ignored rows, or with ``reduce_loss="sum"`` their
    sum); the gradient is staged in place in ``inp`` (in its dtype) and
    reaches autograd through ParallelCrossEntropy.

    ``inp`` is (B, SQ, V) or (SQ, B, V) (any row strides, contiguous
    columns); ``target`` the matching (B, SQ) / (SQ, B) int64 global indices.
    """
    if dist_process_group is not None:
        raise NotImplementedError("vocabulary-parallel process groups need more than one GPU; on one GPU use "
                                  "ce_shards_fwd_bwd_fused, or ce_shard_partial_stats / ce_shard_combine / "
                                  "ce_backward_inplace per shard")
    return ParallelCrossEntropy.apply(inp, target, label_smoothing, reduce_loss, ignore_idx, smoothing)


class ShardedCrossEntropy(torch.autograd.Function):
    """Autograd form of the one-launch shard call (ce_shards_fwd_bwd_fused):
    the logits arrive as S vocabulary shards, separate (d0, d1, V_s) tensors
    in vocabulary order (hyper-parallel #269 section 3.1's ceil(V / S) split,
    as a tensor-parallel rank would hold them).  Forward: each shard is read
    once and receives its gradient for an upstream gradient of 1 in place.
    Backward: every shard's staged gradient times the upstream gradient
    (ce_scale_grad_inplace, nothing touched when it is 1); the shards'
    storage is returned as their gradients.  After the forward the shards
    hold gradients, not logits."""

    @staticmethod
    def forward(ctx, target, label_smoothing, reduce_loss, ignore_idx, smoothing, *shards):
        bufs = [x.detach() for x in shards]
        loss, _ = ce_shards_fwd_bwd_fused(bufs, target, label_smoothing, reduce_loss, ignore_idx,
                                          smoothing=smoothing)
        ctx.reduced = reduction_code(reduce_loss) != _abi.CE_REDUCE_NONE
        ctx.save_for_backward(*bufs)
        return loss[0] if ctx.reduced else loss.view(target.shape)

    @staticmethod
    def backward(ctx, grad_loss):
        bufs = ctx.saved_tensors
        for buf in bufs:
            ce_scale_grad_inplace(buf, grad_loss, per_row=not ctx.reduced)
        return (None, None, None, None, None, *bufs)


def sharded_cross_entropy(shards, target, label_smoothing=0.0, reduce_loss=False, ignore_idx=-100, *,
                          smoothing="all"):
    """Cross-entropy over logits held as vocabulary shards (a list of (d0, d1,
    V_s) tensors in vocabulary order, at most 16), with the same options and
    result as parallel_cross_entropy over their concatenation; one launch."""
    return ShardedCrossEntropy.apply(target, label_smoothing, reduce_loss, ignore_idx, smoothing, *shards)


class LinearCrossEntropy(torch.autograd.Function):
    """Autograd form of the chunked head + loss (ce_linear_cross_entropy).

    Mean or sum: the forward computes the loss and both gradients for an
    upstream gradient of 1 (dh in h's dtype, dW in FP32; no logits are kept);
    the backward scales them in place by the upstream gradient
    (ce_scale_grad_inplace: nothing is read or written when it is 1, and no
    host synchronisation finds out).  Per-row losses: dW needs every row's
    upstream gradient, so the forward computes only the losses and the
    backward runs the chunked call again with the upstream gradients (one
    logits product more).  dW is returned in FP32; autograd casts it to the
    weight's dtype."""

    @staticmethod
    def forward(ctx, h, weight, target, label_smoothing=0.0, reduce_loss="mean", ignore_idx=-100,
                smoothing="all", chunk_rows=0, gemm="auto"):
        ctx.per_row = reduction_code(reduce_loss) == _abi.CE_REDUCE_NONE
        ctx.args = (label_smoothing, reduce_loss, ignore_idx, smoothing, chunk_rows, gemm)
        if ctx.per_row:
            loss, _, _, _ = ce_linear_cross_entropy(h.detach(), weight.detach(), target, label_smoothing,
                                                    reduce_loss, ignore_idx, want_dh=False, want_dw=False,
                                                    chunk_rows=chunk_rows, smoothing=smoothing, gemm=gemm)
            ctx.save_for_backward(h.detach(), weight.detach(), target)
            return loss
        loss, dh, dw, _ = ce_linear_cross_entropy(h.detach(), weight.detach(), target, label_smoothing,
                                                  reduce_loss, ignore_idx, want_dh=ctx.needs_input_grad[0],
                                                  want_dw=ctx.needs_input_grad[1], chunk_rows=chunk_rows,
                                                  smoothing=smoothing, gemm=gemm)
        ctx.save_for_backward(dh if dh is not None else torch.empty(0),
                              dw if dw is not None else torch.empty(0))
        ctx.has = (dh is not None, dw is not None)
        return loss[0]

    @staticmethod
    def backward(ctx, grad_loss):
        if ctx.per_row:
            h, weight, target = ctx.saved_tensors
            label_smoothing, reduce_loss, ignore_idx, smoothing, chunk_rows, gemm = ctx.args
            g = grad_loss.to(dtype=torch.float32).reshape(-1).contiguous()
            _, dh, dw, _ = ce_linear_cross_entropy(h, weight, target, label_smoothing, reduce_loss, ignore_idx,
                                                   grad_out=g, want_dh=ctx.needs_input_grad[0],
                                                   want_dw=ctx.needs_input_grad[1], chunk_rows=chunk_rows,
                                                   smoothing=smoothing, gemm=gemm)
            return dh, dw, None, None, None, None, None, None, None
        dh, dw = ctx.saved_tensors
        g = grad_loss.reshape(1)
        if ctx.has[0]:
            ce_scale_grad_inplace(dh.view(1, *dh.shape), g, per_row=False)
        if ctx.has[1]:
            ce_scale_grad_inplace(dw.view(1, *dw.shape), g, per_row=False)
        return (dh if ctx.has[0] else None, dw if ctx.has[1] else None, None, None, None, None, None, None, None)


def linear_cross_entropy(h, weight, target, label_smoothing=0.0, reduce_loss="mean", ignore_idx=-100, *,
                         smoothing="all", chunk_rows=0, gemm="auto"):
    """Cross-entropy of the head ``h @ weight.T`` without whole logits: the
    rows go through ce_linear_cross_entropy in chunks.  ``h`` [N, D],
    ``weight`` [V, D] (torch Linear layout), ``target`` [N] int64.  Returns
    the FP32 mean or sum, or the [N] per-row losses with
    ``reduce_loss="none"``, and reaches autograd through LinearCrossEntropy.
    ``gemm`` picks the products' engine (see linear_desc)."""
    return LinearCrossEntropy.apply(h, weight, target, label_smoothing, reduce_loss, ignore_idx, smoothing,
                                    chunk_rows, gemm)


class Profiler:
    """Collects the main-kernel duration (ms) of each of the next calls."""

    def __init__(self, capacity: int):
        self.capacity = capacity
        self.ms: list[float] = []

    def __enter__(self):
        _check(lib.ce_profile_start(self.capacity))
        return self

    def __exit__(self, *exc):
        buf = (ctypes.c_float * self.capacity)()
        n = ctypes.c_int32(0)
        _check(lib.ce_profile_stop(buf, self.capacity, ctypes.byref(n)))
        self.ms = [buf[i] for i in range(n.value)]
        return False
