"""CPU oracle for the decode-time MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports it and
it never imports the GPU library.

``moe_oracle.c`` holds the fp64 reference (router logits, top-k selection,
routing weights, SwiGLU experts, shared expert, residual); this module only
compiles it with gcc, loads it with ctypes and marshals NumPy arrays.  The
brute-force dense formulation that pins it lives in ``oracle.brute``; the
score-gap enforcement for generated inputs in ``oracle.gap``.

bf16 tensors cross this boundary as ``numpy.uint16`` arrays of bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

SOFTMAX = 0
SIGMOID = 1


def build(force: bool = True, src: str = _SRC, dst: str = _LIB) -> str:
    """Compile ``moe_oracle.c`` (or ``src``) into ``liboracle.so`` (or ``dst``)."""
    if force or not os.path.exists(dst):
        tmp = dst + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, dst)
    return dst


class _Cfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("score_fn", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("routed_scale", ctypes.c_double), ("add_residual", ctypes.c_int32)]


@dataclass
class LayerShape:
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    score_fn: int = SIGMOID
    renormalize: int = 1
    routed_scale: float = 1.0
    add_residual: int = 1

    def cfg(self, batch: int) -> _Cfg:
        return _Cfg(self.hidden, self.n_experts, self.top_k, self.inter, self.shared_inter,
                    batch, self.score_fn, self.renormalize, float(self.routed_scale),
                    self.add_residual)


class Oracle:
    """ctypes view of one build of the oracle library (the default one, or a
    mutated copy built by the pin tests to show that the pins catch it)."""

    def __init__(self, path: str):
        self.path = path
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        L.oracle_router_logits.argtypes = [ctypes.POINTER(_Cfg), P, P, P, P]
        L.oracle_select.argtypes = [ctypes.POINTER(_Cfg), P, P, P]
        L.oracle_swiglu.argtypes = [ctypes.c_int32] * 3 + [P] * 4
        L.oracle_forward.argtypes = [ctypes.POINTER(_Cfg), P, P, P, P, P, P, P, P, P, P]
        for f in (L.oracle_router_logits, L.oracle_select, L.oracle_swiglu,
                  L.oracle_forward, L.oracle_max_threads):
            f.restype = ctypes.c_int
        self.L = L

    def router_logits(self, shape: LayerShape, x, wr, bias=None) -> np.ndarray:
        """fp64 router logits z[B][E] (step 1)."""
        x, wr = _u16(x), _u16(wr)
        B = x.shape[0]
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        z = np.empty((B, shape.n_experts), np.float64)
        cfg = shape.cfg(B)
        rc = self.L.oracle_router_logits(ctypes.byref(cfg), _ptr(x), _ptr(wr), _ptr(b), _ptr(z))
        if rc:
            raise RuntimeError("oracle_router_logits failed (%d)" % rc)
        return z

    def select(self, shape: LayerShape, z) -> tuple:
        """Top-k indices (rank order) and routing weights from fp64 logits (steps 2-3)."""
        z = np.ascontiguousarray(z, dtype=np.float64)
        B = z.shape[0]
        idx = np.empty((B, shape.top_k), np.int32)
        w = np.empty((B, shape.top_k), np.float64)
        cfg = shape.cfg(B)
        rc = self.L.oracle_select(ctypes.byref(cfg), _ptr(z), _ptr(idx), _ptr(w))
        if rc:
            raise RuntimeError("oracle_select failed (%d)" % rc)
        return idx, w

    def swiglu(self, w13, w2, x) -> np.ndarray:
        """Dense SwiGLU FFN per token, fp64: W2 (silu(W1 x) * (W3 x))."""
        w13, w2, x = _u16(w13), _u16(w2), _u16(x)
        n2, H = w13.shape
        B = x.shape[0]
        y = np.empty((B, H), np.float64)
        rc = self.L.oracle_swiglu(H, n2 // 2, B, _ptr(w13), _ptr(w2), _ptr(x), _ptr(y))
        if rc:
            raise RuntimeError("oracle_swiglu failed (%d)" % rc)
        return y

    def forward(self, shape: LayerShape, x, wr, w13, w2, s13=None, s2=None, bias=None):
        """Whole layer in fp64.

        ``w13``/``w2`` are either full arrays [E][2I][H] / [E][H][I] or sequences of
        per-expert arrays (``None`` for experts the caller did not supply).
        Returns (out64 [B][H] float64, idx [B][k] int32, w [B][k] float64).
        """
        x, wr = _u16(x), _u16(wr)
        B = x.shape[0]
        E = shape.n_experts
        keep = []
        t13 = (ctypes.c_void_p * E)()
        t2 = (ctypes.c_void_p * E)()
        for e in range(E):
            a13 = w13[e]
            a2 = w2[e]
            if a13 is not None:
                a13 = _u16(a13)
                keep.append(a13)
                t13[e] = a13.ctypes.data
            if a2 is not None:
                a2 = _u16(a2)
                keep.append(a2)
                t2[e] = a2.ctypes.data
        if shape.shared_inter > 0:
            s13, s2 = _u16(s13), _u16(s2)
        else:
            s13 = s2 = None
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        out = np.empty((B, shape.hidden), np.float64)
        idx = np.empty((B, shape.top_k), np.int32)
        w = np.empty((B, shape.top_k), np.float64)
        cfg = shape.cfg(B)
        rc = self.L.oracle_forward(ctypes.byref(cfg), _ptr(x), _ptr(wr), _ptr(b),
                                   ctypes.cast(t13, ctypes.c_void_p), ctypes.cast(t2, ctypes.c_void_p),
                                   _ptr(s13), _ptr(s2), _ptr(out), _ptr(idx), _ptr(w))
        if rc == -3:
            raise KeyError("oracle_forward: a selected expert's weights were not supplied")
        if rc:
            raise RuntimeError("oracle_forward failed (%d)" % rc)
        return out, idx, w

    def max_threads(self) -> int:
        return int(self.L.oracle_max_threads())


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 operands are passed as uint16 bit patterns, got %s" % a.dtype)
    return a


def _ptr(a) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data) if a is not None else ctypes.c_void_p(0)


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _default = Oracle(_LIB)
    return _default


def router_logits(shape, x, wr, bias=None):
    return default().router_logits(shape, x, wr, bias)


def select(shape, z):
    return default().select(shape, z)


def swiglu(w13, w2, x):
    return default().swiglu(w13, w2, x)


def forward(shape, x, wr, w13, w2, s13=None, s2=None, bias=None):
    return default().forward(shape, x, wr, w13, w2, s13, s2, bias)


def max_threads() -> int:
    return default().max_threads()
