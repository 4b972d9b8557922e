"""FP64 CPU oracle for fused (vocabulary-parallel) cross-entropy.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package; the product path
(``vocab_cross_entropy_amd``) never does and shares no code with it.

This module is a thin ctypes layer over ``ce_oracle.c`` (see that file's header
for the definitions computed and the passages they follow).  Inputs are torch
CPU tensors of any strides; the C code reads their exact stored bits through
``data_ptr()`` and the element strides, so a transposed view is read in place.
Outputs are float64 numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ce_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libce_oracle.so")

OR_F32 = 0
OR_BF16 = 1

# smoothing conventions and reductions (ce_oracle.c)
SMOOTHING = {"all": 0, "others": 1}
REDUCTION = {"none": 0, "mean": 1, "sum": 2}


def reduction_code(reduce_loss) -> int:
    """False / True / "none" / "mean" / "sum" -> 0 / 1 / 0 / 1 / 2."""
    if isinstance(reduce_loss, str):
        return REDUCTION[reduce_loss]
    return int(bool(reduce_loss))


def smoothing_code(smoothing: str) -> int:
    return SMOOTHING[smoothing]


class OracleError(ValueError):
    """A non-ignored target is outside [0, V), or an argument is malformed."""


class _Logits(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("pad_", ctypes.c_int32),
        ("d0", ctypes.c_int64),
        ("d1", ctypes.c_int64),
        ("s0", ctypes.c_int64),
        ("s1", ctypes.c_int64),
        ("v_local", ctypes.c_int64),
        ("vocab_start", ctypes.c_int64),
        ("vocab_total", ctypes.c_int64),
    ]


class _Targets(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("s0", ctypes.c_int64), ("s1", ctypes.c_int64)]


def build(force: bool = False) -> str:
    """Compile ce_oracle.c with gcc (-O2, no fast-math, OpenMP over rows)."""
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "ce_oracle.h")))
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest:
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-I", _HERE,
             "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.POINTER
    i64, i32, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    vp = ctypes.c_void_p
    lib.or_count_valid.argtypes = [P(_Targets), i64, i64, i64]
    lib.or_count_valid.restype = i64
    lib.or_loss_rows.argtypes = [P(_Logits), P(_Targets), dbl, i32, i64, vp, i64, vp, vp]
    lib.or_grad_rows.argtypes = [P(_Logits), P(_Targets), dbl, i32, i64, i32, vp, dbl, i64, vp, i64, vp]
    lib.or_mean_loss.argtypes = [vp, i64, i64]
    lib.or_mean_loss.restype = dbl
    lib.or_sum_loss.argtypes = [vp, i64]
    lib.or_sum_loss.restype = dbl
    lib.or_shard_stats.argtypes = [P(_Logits), P(_Targets), i64, vp, i64, vp]
    lib.or_shard_combine.argtypes = [vp, i32, i64, i64, P(_Targets), i64, dbl, i32, i64, vp, vp, vp]
    lib.or_shard_grad.argtypes = [P(_Logits), P(_Targets), dbl, i32, i64, i32, vp, dbl, i64, vp, i64, vp, vp]
    lib.or_linear_ce.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, vp, i64, dbl, i32, i64, i32, vp, dbl, i64,
                                 i32, vp, vp, vp, vp]
    for f in ("or_loss_rows", "or_grad_rows", "or_shard_stats", "or_shard_combine", "or_shard_grad", "or_linear_ce"):
        getattr(lib, f).restype = ctypes.c_int
    lib.or_max_threads.restype = ctypes.c_int
    return lib


def load(lib_path: str | None = None) -> ctypes.CDLL:
    """Load the oracle library (building it first if nothing is built)."""
    global _lib
    if lib_path is not None:
        return _declare(ctypes.CDLL(lib_path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


class Oracle:
    """Oracle bound to one compiled library (the default one, or a test copy)."""

    def __init__(self, lib: ctypes.CDLL | None = None):
        self.lib = lib if lib is not None else load()

    # -- argument marshalling -------------------------------------------------
    @staticmethod
    def _logits(x: torch.Tensor, vocab_start: int = 0, vocab_total: int | None = None) -> _Logits:
        if x.device.type != "cpu" or x.dim() != 3 or x.stride(2) != 1:
            raise OracleError("logits must be a CPU (d0, d1, V) tensor with unit column stride")
        if x.dtype == torch.float32:
            code = OR_F32
        elif x.dtype == torch.bfloat16:
            code = OR_BF16
        else:
            raise OracleError(f"unsupported dtype {x.dtype}")
        d0, d1, v = x.shape
        return _Logits(x.data_ptr(), code, 0, d0, d1, x.stride(0), x.stride(1), v,
                       vocab_start, v if vocab_total is None else vocab_total)

    @staticmethod
    def _targets(t: torch.Tensor) -> _Targets:
        if t.device.type != "cpu" or t.dtype != torch.int64 or t.dim() != 2:
            raise OracleError("targets must be a CPU int64 (d0, d1) tensor")
        return _Targets(t.data_ptr(), t.stride(0), t.stride(1))

    @staticmethod
    def _rows(rows, n: int) -> np.ndarray:
        r = np.arange(n, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        if r.size and (r.min() < 0 or r.max() >= n):
            raise OracleError("row index out of range")
        return r

    @staticmethod
    def _check(rc: int):
        if rc == -1:
            raise OracleError("a non-ignored target lies outside [0, V)")
        if rc != 0:
            raise OracleError(f"oracle rejected its arguments (code {rc})")

    # -- definitions ------------------------------------------------------------
    def count_valid(self, t: torch.Tensor, ignore_idx: int = -100) -> int:
        d0, d1 = t.shape
        return int(self.lib.or_count_valid(ctypes.byref(self._targets(t)), d0, d1, ignore_idx))

    def loss_rows(self, x, t, alpha=0.0, ignore_idx=-100, rows=None, smoothing="all"):
        """Per-row loss and lse (float64) of the listed logical rows (all if None).
        ``smoothing``: "all" (a / V on every class) or "others" (a / (V - 1)
        on every class but the target)."""
        lx, lt = self._logits(x), self._targets(t)
        r = self._rows(rows, lx.d0 * lx.d1)
        loss = np.empty(r.size, np.float64)
        lse = np.empty(r.size, np.float64)
        self._check(self.lib.or_loss_rows(ctypes.byref(lx), ctypes.byref(lt), float(alpha), smoothing_code(smoothing),
                                          int(ignore_idx), r.ctypes.data, r.size, loss.ctypes.data,
                                          lse.ctypes.data))
        return loss, lse

    def grad_rows(self, x, t, alpha=0.0, ignore_idx=-100, reduce_loss=False, g=None, rows=None,
                  n_valid=None, smoothing="all"):
        """Unrounded float64 gradient rows [len(rows), V].

        ``reduce_loss``: False / "none", True / "mean", or "sum".  ``g``:
        per-row upstream gradient [d0*d1] (not reducing) or a scalar
        (reducing); None means 1.  ``n_valid`` defaults to the count of
        non-ignored targets.
        """
        lx, lt = self._logits(x), self._targets(t)
        N = lx.d0 * lx.d1
        r = self._rows(rows, N)
        if n_valid is None:
            n_valid = self.count_valid(t, ignore_idx)
        g_row_ptr, g_scalar = None, 1.0
        g_keep = None
        if g is not None:
            if reduction_code(reduce_loss):
                g_scalar = float(g)
            else:
                g_keep = np.ascontiguousarray(np.asarray(g, dtype=np.float64).reshape(-1))
                if g_keep.size != N:
                    raise OracleError("per-row g must have d0*d1 entries")
                g_row_ptr = g_keep.ctypes.data
        out = np.empty((r.size, lx.v_local), np.float64)
        self._check(self.lib.or_grad_rows(ctypes.byref(lx), ctypes.byref(lt), float(alpha), smoothing_code(smoothing),
                                          int(ignore_idx), reduction_code(reduce_loss), g_row_ptr, g_scalar,
                                          int(n_valid), r.ctypes.data, r.size, out.ctypes.data))
        return out

    def mean_loss(self, loss: np.ndarray, n_valid: int) -> float:
        loss = np.ascontiguousarray(loss, dtype=np.float64)
        return float(self.lib.or_mean_loss(loss.ctypes.data, loss.size, int(n_valid)))

    def sum_loss(self, loss: np.ndarray) -> float:
        loss = np.ascontiguousarray(loss, dtype=np.float64)
        return float(self.lib.or_sum_loss(loss.ctypes.data, loss.size))

    def reduce(self, loss: np.ndarray, reduce_loss, n_valid: int):
        """The per-row losses as the given reduction returns them."""
        code = reduction_code(reduce_loss)
        if code == 1:
            return self.mean_loss(loss, n_valid)
        if code == 2:
            return self.sum_loss(loss)
        return loss

    def shard_stats(self, shard, t, vocab_start, vocab_total, ignore_idx=-100, rows=None):
        """(m, d, y, r) float64 [len(rows), 4] of one vocabulary shard."""
        lx, lt = self._logits(shard, vocab_start, vocab_total), self._targets(t)
        r = self._rows(rows, lx.d0 * lx.d1)
        out = np.empty((r.size, 4), np.float64)
        self._check(self.lib.or_shard_stats(ctypes.byref(lx), ctypes.byref(lt), int(ignore_idx),
                                            r.ctypes.data, r.size, out.ctypes.data))
        return out

    def shard_combine(self, stats, t, vocab_total, alpha=0.0, ignore_idx=-100, rows=None, smoothing="all"):
        """Combine stats [S, len(rows), 4] into (loss, lse) for the listed rows."""
        st = np.ascontiguousarray(stats, dtype=np.float64)
        S, nr, four = st.shape
        if four != 4:
            raise OracleError("stats must be [S, rows, 4]")
        lt = self._targets(t)
        d0, d1 = t.shape
        r = self._rows(rows, d0 * d1)
        if r.size != nr:
            raise OracleError("stats rows do not match the row list")
        loss = np.empty(nr, np.float64)
        lse = np.empty(nr, np.float64)
        self._check(self.lib.or_shard_combine(st.ctypes.data, S, nr, int(vocab_total), ctypes.byref(lt), d1,
                                              float(alpha), smoothing_code(smoothing), int(ignore_idx),
                                              r.ctypes.data, loss.ctypes.data, lse.ctypes.data))
        return loss, lse

    def shard_grad(self, shard, t, vocab_start, vocab_total, lse, alpha=0.0, ignore_idx=-100,
                   reduce_loss=False, g=None, rows=None, n_valid=None, smoothing="all"):
        """Unrounded float64 gradient of one shard's listed rows, given combined lse."""
        lx, lt = self._logits(shard, vocab_start, vocab_total), self._targets(t)
        N = lx.d0 * lx.d1
        r = self._rows(rows, N)
        lse = np.ascontiguousarray(lse, dtype=np.float64)
        if lse.size != r.size:
            raise OracleError("lse must have one entry per listed row")
        if n_valid is None:
            n_valid = self.count_valid(t, ignore_idx)
        g_row_ptr, g_scalar, g_keep = None, 1.0, None
        if g is not None:
            if reduction_code(reduce_loss):
                g_scalar = float(g)
            else:
                g_keep = np.ascontiguousarray(np.asarray(g, dtype=np.float64).reshape(-1))
                g_row_ptr = g_keep.ctypes.data
        out = np.empty((r.size, lx.v_local), np.float64)
        self._check(self.lib.or_shard_grad(ctypes.byref(lx), ctypes.byref(lt), float(alpha),
                                           smoothing_code(smoothing), int(ignore_idx), reduction_code(reduce_loss),
                                           g_row_ptr, g_scalar, int(n_valid), r.ctypes.data, r.size,
                                           lse.ctypes.data, out.ctypes.data))
        return out

    def linear_ce(self, h, w, t, alpha=0.0, ignore_idx=-100, reduce_loss=False, g=None, n_valid=None,
                  smoothing="all", round_logits=True, want_dh=True, want_dw=True, want_g=False):
        """Head + loss of h [N, D] and w [V, D] (CPU, FP32 or BF16, contiguous
        columns), targets t [N] int64.  Returns (loss rows [N], dh [N, D],
        dw [V, D]) in float64, and G [N, V] after them with ``want_g``; the
        reduction of the loss is left to ``reduce``."""
        if h.dtype != w.dtype or h.dim() != 2 or w.dim() != 2 or h.shape[1] != w.shape[1]:
            raise OracleError("h [N, D] and w [V, D] of one dtype")
        if h.device.type != "cpu" or w.device.type != "cpu" or t.device.type != "cpu":
            raise OracleError("CPU tensors only")
        if (h.shape[0] > 1 and h.stride(1) != 1) or w.stride(1) != 1:
            raise OracleError("contiguous columns only")
        code = OR_F32 if h.dtype == torch.float32 else OR_BF16 if h.dtype == torch.bfloat16 else None
        if code is None:
            raise OracleError(f"unsupported dtype {h.dtype}")
        N, D = h.shape
        V = w.shape[0]
        if t.dtype != torch.int64 or t.dim() != 1 or t.numel() != N:
            raise OracleError("targets must be int64 [N]")
        if n_valid is None:
            n_valid = int((t != ignore_idx).sum())
        red = reduction_code(reduce_loss)
        g_row_ptr, g_scalar, g_keep = None, 1.0, None
        if g is not None:
            if red:
                g_scalar = float(g)
            else:
                g_keep = np.ascontiguousarray(np.asarray(g, dtype=np.float64).reshape(-1))
                if g_keep.size != N:
                    raise OracleError("per-row g must have N entries")
                g_row_ptr = g_keep.ctypes.data
        loss = np.empty(N, np.float64)
        dh = np.empty((N, D), np.float64) if want_dh else None
        dw = np.empty((V, D), np.float64) if want_dw else None
        G = np.empty((N, V), np.float64) if want_g else None
        self._check(self.lib.or_linear_ce(h.data_ptr(), w.data_ptr(), code, N, D, V, max(h.stride(0), D),
                                          max(w.stride(0), D), t.data_ptr(), t.stride(0) if N > 1 else 1,
                                          float(alpha), smoothing_code(smoothing), int(ignore_idx), red,
                                          g_row_ptr, g_scalar, int(n_valid), 1 if round_logits else 0,
                                          loss.ctypes.data, None if dh is None else dh.ctypes.data,
                                          None if dw is None else dw.ctypes.data,
                                          None if G is None else G.ctypes.data))
        return (loss, dh, dw, G) if want_g else (loss, dh, dw)

    def linear_ce_blocked(self, h, w, t, alpha=0.0, ignore_idx=-100, reduce_loss=False, g=None, n_valid=None,
                          smoothing="all", dw_cols=(), block=512, on_block=None):
        """The head + loss of every row, for heads whose logits are too large
        for or_linear_ce's loops (hyper-parallel #269's chunked lm_head at full
        size).  Per block of rows: the logits as a float64 matrix product of
        the exact stored values (a library matmul as the step; exact whenever
        every partial sum is, as for grid-valued inputs), materialised as the
        library does (FP32, then BF16 by nearest even for BF16 inputs), then
        that block's loss rows and gradient G by or_loss_rows / or_grad_rows
        on the materialised logits, and dW's columns ``dw_cols`` accumulated as
        G^T h[:, cols] in float64.  ``on_block(rows, G)`` sees each block's G.
        Returns (loss rows [N], dW[:, dw_cols] [V, len(dw_cols)])."""
        if h.dtype != w.dtype or h.dim() != 2 or w.dim() != 2 or h.shape[1] != w.shape[1]:
            raise OracleError("h [N, D] and w [V, D] of one dtype")
        if h.dtype not in (torch.float32, torch.bfloat16):
            raise OracleError(f"unsupported dtype {h.dtype}")
        N, D = h.shape
        V = w.shape[0]
        if t.dtype != torch.int64 or t.dim() != 1 or t.numel() != N:
            raise OracleError("targets must be int64 [N]")
        if n_valid is None:
            n_valid = int((t != ignore_idx).sum())
        cols = np.asarray(dw_cols, dtype=np.int64)
        wt = w.to(torch.float64).T.contiguous()
        hc = h.to(torch.float64)[:, torch.as_tensor(cols)].numpy() if cols.size else None
        loss = np.empty(N, np.float64)
        dwc = np.zeros((V, cols.size), np.float64)
        red = reduction_code(reduce_loss)
        for r0 in range(0, N, block):
            r1 = min(N, r0 + block)
            logits = (h[r0:r1].to(torch.float64) @ wt).to(torch.float32)
            if h.dtype == torch.bfloat16:
                logits = logits.to(torch.bfloat16)
            x = logits.reshape(1, r1 - r0, V)
            tb = t[r0:r1].reshape(1, r1 - r0).contiguous()
            loss[r0:r1], _ = self.loss_rows(x, tb, alpha, ignore_idx, smoothing=smoothing)
            gb = None
            if g is not None:
                gb = float(g) if red else np.asarray(g, np.float64).reshape(-1)[r0:r1]
            G = self.grad_rows(x, tb, alpha, ignore_idx, reduce_loss=reduce_loss, g=gb, n_valid=n_valid,
                               smoothing=smoothing)
            if cols.size:
                dwc += G.T @ hc[r0:r1]
            if on_block is not None:
                on_block(np.arange(r0, r1), G)
        return loss, dwc

    def max_threads(self) -> int:
        return int(self.lib.or_max_threads())


def default() -> Oracle:
    return Oracle()
