"""Python binding of the MI355X decode-time MoE layer library.

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmoe_decode.so`` (built from ``csrc/`` by :func:`build`).  PyTorch supplies
device memory and streams.  The names mirror the C ABI in
``include/moe_decode.h``.  Importing this package raises if the library has
not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
LIB_PATH = os.path.join(_HERE, "libmoe_decode.so")
HEADER = os.path.join(_ROOT, "include", "moe_decode.h")
_CSRC = os.path.join(_HERE, "csrc")
SOURCES = [os.path.join(_CSRC, f) for f in ("moe_kernels.hip", "moe_layer_tb1.hip", "moe_layer_tb2.hip",
                                             "moe_layer_tb4.hip", "moe_scratch.hip", "moe_fused.hip",
                                             "moe_decode.cpp")]

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_NOMEM, MOE_ERR_STATE = range(6)
STATUS_NAMES = ["MOE_OK", "MOE_ERR_INVALID", "MOE_ERR_UNSUPPORTED", "MOE_ERR_HIP", "MOE_ERR_NOMEM",
                "MOE_ERR_STATE"]
SOFTMAX, SIGMOID = 0, 1
VARIANT_AUTO, VARIANT_SMALL_M, VARIANT_SPLIT_K = 0, 1, 2
VARIANT_NAMES = {0: "AUTO", 1: "SMALL_M", 2: "SPLIT_K"}
SINGLE_AUTO, SINGLE_OFF, SINGLE_REQUIRED = 0, 1, 2

EXPORTS = ["moe_decode_plan", "moe_decode_forward", "moe_decode_forward_prefetch", "moe_decode_forward_noalloc",
           "moe_decode_routing",
           "moe_decode_read_stats",
           "moe_decode_plan_info", "moe_decode_set_profiling", "moe_decode_profile_read",
           "moe_decode_destroy", "moe_decode_last_error"]


def build(arch: str = "gfx950", out: str = LIB_PATH, jobs: int = 8) -> str:
    """Compile the HIP kernels and the host library into ``libmoe_decode.so``
    (one hipcc process per source file, ``jobs`` at a time, then one link)."""
    from concurrent.futures import ThreadPoolExecutor

    bdir = os.path.join(_HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    flags = ["--offload-arch=" + arch, "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
             "-I", os.path.join(_ROOT, "include")]

    def compile_one(src):
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        subprocess.run(["hipcc", *flags, "-c", src, "-o", obj], check=True)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["hipcc", "--offload-arch=" + arch, "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, out)
    return out


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        self.status = status
        super().__init__("%s: %s" % (STATUS_NAMES[status] if 0 <= status < 6 else status, msg))


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("score_fn", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("routed_scale", ctypes.c_float), ("add_residual", ctypes.c_int32),
                ("router_bias", ctypes.c_void_p), ("force_variant", ctypes.c_int32),
                ("mfma_min_tokens", ctypes.c_int32), ("shared_stream", ctypes.c_int32),
                ("topk_launch", ctypes.c_int32), ("single_launch", ctypes.c_int32)]


class Info(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("n_kernels", ctypes.c_int32),
                ("mfma_min_tokens", ctypes.c_int32), ("shared_mfma", ctypes.c_int32),
                ("shared_stream", ctypes.c_int32), ("router_mfma", ctypes.c_int32),
                ("single_launch", ctypes.c_int32), ("layer_grid", ctypes.c_int32),
                ("topk_launch", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t),
                ("shared_gateup_in", ctypes.c_int32)]


class Stats(ctypes.Structure):
    _fields_ = [("n_unique", ctypes.c_int32), ("gemv_tiles", ctypes.c_int32),
                ("mfma_tiles", ctypes.c_int32), ("error_flags", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmoe_decode.so is not built (run __graft_entry__.build() or "
                              "mixture_experts_layer_29_amd.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.moe_decode_plan.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(P)]
        L.moe_decode_forward.argtypes = [P, P, P, P, P, P, P]
        L.moe_decode_forward_noalloc.argtypes = [P, P, P, P, P, P, P]
        L.moe_decode_forward_prefetch.argtypes = [P, P, P, P, P, P, P, P, P]
        L.moe_decode_routing.argtypes = [P, P, P, P, P, P]
        L.moe_decode_read_stats.argtypes = [P, ctypes.POINTER(Stats)]
        L.moe_decode_plan_info.argtypes = [P, ctypes.POINTER(Info)]
        L.moe_decode_set_profiling.argtypes = [P, ctypes.c_int32]
        L.moe_decode_profile_read.argtypes = [P, ctypes.c_int32, ctypes.POINTER(ctypes.c_double),
                                              ctypes.POINTER(ctypes.c_int32),
                                              ctypes.POINTER(ctypes.c_char_p),
                                              ctypes.POINTER(ctypes.c_int32)]
        L.moe_decode_destroy.argtypes = [P]
        for name in EXPORTS[:-1]:
            getattr(L, name).restype = ctypes.c_int
        L.moe_decode_last_error.restype = ctypes.c_char_p
        L.moe_decode_last_error.argtypes = []
        _lib = L
    return _lib


def last_error() -> str:
    return lib().moe_decode_last_error().decode()


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, last_error())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(hidden, n_experts, top_k, inter, shared_inter, batch, score_fn=SIGMOID, renormalize=1,
                routed_scale=1.0, add_residual=1, router_bias=None, force_variant=VARIANT_AUTO,
                mfma_min_tokens=0, shared_stream=0, topk_launch=0, single_launch=SINGLE_AUTO) -> Config:
    return Config(hidden, n_experts, top_k, inter, shared_inter, batch, score_fn, renormalize,
                  float(routed_scale), add_residual, _ptr(router_bias), force_variant, mfma_min_tokens,
                  shared_stream, topk_launch, single_launch)


class Plan:
    """Owns one ``moe_decode_plan_t``."""

    def __init__(self, cfg: Config):
        h = ctypes.c_void_p()
        _check(lib().moe_decode_plan(ctypes.byref(cfg), ctypes.byref(h)))
        self.cfg = cfg
        self.handle = h

    def forward(self, x, router_w, expert_w, shared_w, out, stream=None):
        _check(lib().moe_decode_forward(self.handle, _ptr(x), _ptr(router_w), _ptr(expert_w),
                                        _ptr(shared_w), _ptr(out), _stream(stream)))
        return out

    def forward_prefetch(self, x, router_w, expert_w, shared_w, out, next_router_w, next_shared_w, stream=None):
        _check(lib().moe_decode_forward_prefetch(self.handle, _ptr(x), _ptr(router_w), _ptr(expert_w),
                                                 _ptr(shared_w), _ptr(out), _ptr(next_router_w),
                                                 _ptr(next_shared_w), _stream(stream)))
        return out

    def forward_noalloc(self, x, router_w, expert_w, shared_w, out, stream=None):
        _check(lib().moe_decode_forward_noalloc(self.handle, _ptr(x), _ptr(router_w), _ptr(expert_w),
                                                _ptr(shared_w), _ptr(out), _stream(stream)))
        return out

    def routing(self, topk_idx=None, topk_w=None, n_unique=None, logits=None, stream=None):
        _check(lib().moe_decode_routing(self.handle, _ptr(topk_idx), _ptr(topk_w), _ptr(n_unique),
                                        _ptr(logits), _stream(stream)))

    def stats(self) -> Stats:
        s = Stats()
        _check(lib().moe_decode_read_stats(self.handle, ctypes.byref(s)))
        return s

    def info(self) -> Info:
        i = Info()
        _check(lib().moe_decode_plan_info(self.handle, ctypes.byref(i)))
        return i

    def set_profiling(self, enable: bool):
        _check(lib().moe_decode_set_profiling(self.handle, 1 if enable else 0))

    def profile_read(self) -> dict:
        cap = 16
        ms = (ctypes.c_double * cap)()
        cnt = (ctypes.c_int32 * cap)()
        names = (ctypes.c_char_p * cap)()
        n = ctypes.c_int32()
        _check(lib().moe_decode_profile_read(self.handle, cap, ms, cnt, names, ctypes.byref(n)))
        return {names[i].decode(): (ms[i], cnt[i]) for i in range(n.value)}

    def destroy(self):
        if self.handle is not None and self.handle.value is not None:
            _check(lib().moe_decode_destroy(self.handle))
        self.handle = None

    def __del__(self):
        try:
            if getattr(self, "handle", None) is not None and self.handle.value is not None:
                lib().moe_decode_destroy(self.handle)
        except Exception:
            pass
