"""ctypes declarations of include/ce.h (argument marshalling only).

The shared library is the one built in-tree by ``vocab_cross_entropy_amd/csrc/build.py``;
there is no fallback: if it is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libce.so")
# the same library with phase stamps compiled in; loaded only when
# VCE_PHASE_CLOCK=1 (bench.py --phases sets it)
PHASES_LIB_PATH = os.path.join(PKG, "libce_phases.so")

CE_OK, CE_EINVAL, CE_EDTYPE, CE_ELAYOUT, CE_EWORKSPACE, CE_EHIP, CE_EDEADLOCK = range(7)
CE_F32, CE_BF16 = 0, 1
CE_REDUCE_NONE, CE_REDUCE_MEAN, CE_REDUCE_SUM = 0, 1, 2
CE_SMOOTH_ALL, CE_SMOOTH_OTHERS = 0, 1
CE_GEMM_AUTO, CE_GEMM_NATIVE, CE_GEMM_LIBRARY = 0, 1, 2
CE_ABI_VERSION = 7


class CeLogits(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("d0", ctypes.c_int64),
        ("d1", ctypes.c_int64),
        ("s0", ctypes.c_int64),
        ("s1", ctypes.c_int64),
        ("v_local", ctypes.c_int64),
        ("vocab_start", ctypes.c_int64),
        ("vocab_total", ctypes.c_int64),
    ]


class CeTargets(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("s0", ctypes.c_int64), ("s1", ctypes.c_int64)]


class CeParams(ctypes.Structure):
    _fields_ = [
        ("label_smoothing", ctypes.c_float),
        ("reduce_loss", ctypes.c_int32),
        ("ignore_idx", ctypes.c_int64),
        ("split_chunks", ctypes.c_int32),
        ("smoothing", ctypes.c_int32),
    ]


class CeLinear(ctypes.Structure):
    _fields_ = [
        ("h", ctypes.c_void_p),
        ("w", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("gemm", ctypes.c_int32),
        ("N", ctypes.c_int64),
        ("D", ctypes.c_int64),
        ("V", ctypes.c_int64),
        ("h_ld", ctypes.c_int64),
        ("w_ld", ctypes.c_int64),
    ]


# Every symbol include/ce.h declares, with its ctypes signature.
_P = ctypes.POINTER
_vp = ctypes.c_void_p
SIGNATURES = {
    "ce_workspace_bytes": (ctypes.c_size_t, [_P(CeLogits), _P(CeParams)]),
    "ce_combine_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, _P(CeParams)]),
    "ce_forward": (ctypes.c_int, [_P(CeLogits), _P(CeTargets), _P(CeParams), _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                  _vp]),
    "ce_forward_ex": (ctypes.c_int, [_P(CeLogits), _P(CeTargets), _P(CeParams), _vp, _vp, _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp]),
    "ce_backward_inplace": (ctypes.c_int, [_P(CeLogits), _P(CeTargets), _P(CeParams), _vp, _vp, _vp, _vp]),
    "ce_backward_inplace_ex": (ctypes.c_int, [_P(CeLogits), _P(CeTargets), _P(CeParams), _vp, _vp, _vp, _vp,
                                              _vp]),
    "ce_fwd_bwd_fused": (ctypes.c_int, [_P(CeLogits), _P(CeTargets), _P(CeParams), _vp, _vp, _vp, _vp,
                                        ctypes.c_size_t, _vp]),
    "ce_fwd_bwd_fused_noalloc": (ctypes.c_int, [_P(CeLogits), _P(CeTargets), _P(CeParams), _vp, _vp, _vp, _vp]),
    "ce_shards_workspace_bytes": (ctypes.c_size_t, [_P(CeLogits), ctypes.c_int32, _P(CeParams)]),
    "ce_shards_fwd_bwd_fused": (ctypes.c_int, [_P(CeLogits), ctypes.c_int32, _P(CeTargets), _P(CeParams), _vp, _vp,
                                               _vp, _vp, ctypes.c_size_t, _vp]),
    "ce_scale_grad_inplace": (ctypes.c_int, [_P(CeLogits), _vp, ctypes.c_int32, _vp]),
    "ce_stream_reference": (ctypes.c_int, [_vp, _vp, ctypes.c_int64, _vp]),
    "ce_shard_partial_stats": (ctypes.c_int, [_P(CeLogits), _P(CeTargets), _P(CeParams), _vp, _vp]),
    "ce_shard_combine": (ctypes.c_int, [_vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        _P(CeTargets), _P(CeParams), _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "ce_shard_combine_ex": (ctypes.c_int, [_vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                           _P(CeTargets), _P(CeParams), _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                           _vp]),
    "ce_workspace_init": (ctypes.c_int, [_vp, ctypes.c_size_t, _vp]),
    "ce_linear_gemm_plan": (ctypes.c_int32, [_P(CeLinear)]),
    "ce_linear_workspace_bytes": (ctypes.c_size_t, [_P(CeLinear), _P(CeParams), ctypes.c_int64,
                                                    _P(ctypes.c_int64)]),
    "ce_linear_tune": (ctypes.c_int, [_P(CeLinear), _P(CeParams), _vp, ctypes.c_int64, _vp, ctypes.c_int64,
                                      ctypes.c_int64, _vp, ctypes.c_size_t, _vp]),
    "ce_linear_cross_entropy": (ctypes.c_int, [_P(CeLinear), _vp, ctypes.c_int64, _P(CeParams), _vp, _vp, _vp, _vp,
                                               ctypes.c_int64, _vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                               _vp, ctypes.c_size_t, _vp]),
    "ce_workspace_check": (ctypes.c_int, [_vp, _vp]),
    "ce_profile_start": (ctypes.c_int, [ctypes.c_int32]),
    "ce_profile_stop": (ctypes.c_int, [_vp, ctypes.c_int32, _P(ctypes.c_int32)]),
    "ce_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ce_last_error": (ctypes.c_char_p, []),
    "ce_abi_version": (ctypes.c_int32, []),
}


def load(path: str | None = None) -> ctypes.CDLL:
    phases = path is None and os.environ.get("VCE_PHASE_CLOCK") == "1"
    if path is None:
        path = PHASES_LIB_PATH if phases else LIB_PATH
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python vocab_cross_entropy_amd/csrc/build.py"
            f"{' --phases' if phases else ''}` (hipcc, gfx950) first")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if phases:
        lib.ce_phase_clock.restype = ctypes.c_int
        lib.ce_phase_clock.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    if lib.ce_abi_version() != CE_ABI_VERSION:
        raise ImportError(f"{path} has ABI version {lib.ce_abi_version()}, expected {CE_ABI_VERSION}")
    return lib


class CeError(RuntimeError):
    """A non-OK ce_status; ``status`` holds the code."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} [status {status}]")
        self.status = status


class CeArgumentError(CeError, ValueError):
    """Argument, dtype, layout or workspace error (nothing was enqueued)."""
