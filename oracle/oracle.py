"""Python access to the fp64 CPU oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the package smoke check
and the benchmark's CPU-baseline leg, never by the library's product path.
It shares no code with the HIP library; the only thing both sides use is the
seeded input generator.

Every function takes and returns numpy arrays in the plain layout documented
in moe_oracle.h (bf16 as uint16 bit patterns, double results).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
# MOE_ORACLE_LIB names another build of moe_oracle.c to load instead (the
# mutation test loads deliberately broken copies this way, in a child process).
LIB_PATH = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "libmoe_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc -O2 -fopenmp (no -ffast-math)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Cfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("has_shared", ctypes.c_int32)]


_P = ctypes.c_void_p


class _Experts(ctypes.Structure):
    _fields_ = [("w13_q", _P), ("w13_s", _P), ("w2_q", _P), ("w2_s", _P),
                ("sh_w13", _P), ("sh_w2", _P)]


class _ExpertsFmt(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("w13_q", _P), ("w13_s", _P), ("w2_q", _P), ("w2_s", _P),
                ("sh_w13", _P), ("sh_w2", _P)]


# routed-expert weight formats (oracle_forward_fmt)
FMT_INT4_G32, FMT_MXFP4, FMT_FP8_BLOCK = 0, 1, 2
_SCALE_DTYPE = {FMT_INT4_G32: np.uint16, FMT_MXFP4: np.uint8, FMT_FP8_BLOCK: np.float32}


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                build(force=True)
            L = ctypes.CDLL(LIB_PATH)
            L.oracle_bf16_to_f64.restype = ctypes.c_double
            L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
            L.oracle_f64_to_bf16.restype = ctypes.c_uint16
            L.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
            L.oracle_f64_to_bf16_array.argtypes = [_P, _P, ctypes.c_int64]
            L.oracle_dequant.argtypes = [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P]
            L.oracle_route.argtypes = [ctypes.POINTER(_Cfg), _P, _P, ctypes.c_int32, _P, _P, _P, _P]
            L.oracle_expert_q.argtypes = [ctypes.POINTER(_Cfg), _P, _P, _P, _P, _P, _P, _P]
            L.oracle_expert_dense.argtypes = [ctypes.POINTER(_Cfg), _P, _P, _P, _P, _P]
            L.oracle_forward.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_Experts), _P,
                                         ctypes.c_int32, _P, _P, _P]
            L.oracle_permute.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
            L.oracle_rmsnorm.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_double, _P]
            L.oracle_num_threads.restype = ctypes.c_int
            L.oracle_e4m3_to_f64.restype = ctypes.c_double
            L.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
            L.oracle_f32_to_e4m3.restype = ctypes.c_uint8
            L.oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
            L.oracle_lmhead_quantize.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, _P, _P]
            L.oracle_lmhead_gemv_fp8.argtypes = [_P, _P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P]
            L.oracle_lmhead_gemv_bf16.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P]
            L.oracle_e2m1_to_f64.restype = ctypes.c_double
            L.oracle_e2m1_to_f64.argtypes = [ctypes.c_uint8]
            L.oracle_e8m0_to_f64.restype = ctypes.c_double
            L.oracle_e8m0_to_f64.argtypes = [ctypes.c_uint8]
            L.oracle_dequant_fmt.argtypes = [ctypes.c_int32, _P, _P, ctypes.c_int32, ctypes.c_int32, _P]
            L.oracle_forward_fmt.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_ExpertsFmt), _P,
                                             ctypes.c_int32, _P, _P, _P]
            _lib = L
        return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def _cfg(shape) -> _Cfg:
    return _Cfg(shape.hidden, shape.n_experts, shape.top_k, shape.inter,
                shape.group_size, int(shape.has_shared))


def num_threads() -> int:
    return lib().oracle_num_threads()


def bf16_to_f64(bits) -> np.ndarray:
    b = _c(bits, np.uint16)
    return np.array([lib().oracle_bf16_to_f64(int(v)) for v in b.ravel()]).reshape(b.shape)


def f64_to_bf16(v) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_f64_to_bf16_array(_ptr(v), _ptr(out), v.size)
    return out


def dequant(q, s, group_size: int = 32) -> np.ndarray:
    q, s = _c(q, np.uint8), _c(s, np.uint16)
    N, K = q.shape[0], q.shape[1] * 2
    W = np.empty((N, K), np.float64)
    if lib().oracle_dequant(_ptr(q), _ptr(s), N, K, group_size, _ptr(W)) != 0:
        raise ValueError("oracle_dequant: bad arguments")
    return W


def route(shape, router_w, x):
    """Returns (ids int32 [M][k], w float64 [M][k], gap float64 [M], logits float64 [M][E])."""
    x = _c(x, np.uint16).reshape(-1, shape.hidden)
    rw = _c(router_w, np.float32)
    M = x.shape[0]
    ids = np.empty((M, shape.top_k), np.int32)
    w = np.empty((M, shape.top_k), np.float64)
    gap = np.empty(M, np.float64)
    logits = np.empty((M, shape.n_experts), np.float64)
    c = _cfg(shape)
    if lib().oracle_route(ctypes.byref(c), _ptr(rw), _ptr(x), M, _ptr(ids), _ptr(w), _ptr(gap), _ptr(logits)) != 0:
        raise ValueError("oracle_route: bad arguments")
    return ids, w, gap, logits


def expert_q(shape, w13_q, w13_s, w2_q, w2_s, x_f64):
    """One quantized expert on one token (x as float64 [H]); returns (h [I], y [H])."""
    arrs = [_c(w13_q, np.uint8), _c(w13_s, np.uint16), _c(w2_q, np.uint8), _c(w2_s, np.uint16)]
    x = _c(x_f64, np.float64)
    h = np.empty(shape.inter, np.float64)
    y = np.empty(shape.hidden, np.float64)
    c = _cfg(shape)
    if lib().oracle_expert_q(ctypes.byref(c), *[_ptr(a) for a in arrs], _ptr(x), _ptr(h), _ptr(y)) != 0:
        raise ValueError("oracle_expert_q: bad arguments")
    return h, y


def expert_dense(shape, sh_w13, sh_w2, x_f64):
    a, b = _c(sh_w13, np.uint16), _c(sh_w2, np.uint16)
    x = _c(x_f64, np.float64)
    h = np.empty(shape.inter, np.float64)
    y = np.empty(shape.hidden, np.float64)
    c = _cfg(shape)
    if lib().oracle_expert_dense(ctypes.byref(c), _ptr(a), _ptr(b), _ptr(x), _ptr(h), _ptr(y)) != 0:
        raise ValueError("oracle_expert_dense: bad arguments")
    return h, y


def forward(shape, experts, x, ids, w):
    """experts: an object with w13_q/w13_s/w2_q/w2_s (full [E]-leading arrays, or
    dicts {expert id: array}) and sh_w13/sh_w2.  Returns (out float64 [M][H],
    number of slots with an out-of-range id)."""
    E = shape.n_experts
    x = _c(x, np.uint16).reshape(-1, shape.hidden)
    ids = _c(ids, np.int32).reshape(x.shape[0], shape.top_k)
    w = _c(w, np.float64).reshape(x.shape[0], shape.top_k)
    keep = []

    def table(name, dtype):
        src = getattr(experts, name) if not isinstance(experts, dict) else experts[name]
        arr = (ctypes.c_void_p * E)()
        for e in range(E):
            a = None
            if isinstance(src, dict):
                a = src.get(e)
            elif src is not None:
                a = src[e]
            if a is not None:
                a = _c(a, dtype)
                keep.append(a)
                arr[e] = a.ctypes.data
        keep.append(arr)
        return ctypes.cast(arr, ctypes.c_void_p)

    def get(name):
        return getattr(experts, name) if not isinstance(experts, dict) else experts.get(name)

    sh13 = get("sh_w13")
    sh2 = get("sh_w2")
    sh13 = None if sh13 is None else _c(sh13, np.uint16)
    sh2 = None if sh2 is None else _c(sh2, np.uint16)
    ex = _Experts(table("w13_q", np.uint8), table("w13_s", np.uint16),
                  table("w2_q", np.uint8), table("w2_s", np.uint16),
                  _ptr(sh13), _ptr(sh2))
    out = np.empty((x.shape[0], shape.hidden), np.float64)
    c = _cfg(shape)
    rc = lib().oracle_forward(ctypes.byref(c), ctypes.byref(ex), _ptr(x), x.shape[0],
                              _ptr(ids), _ptr(w), _ptr(out))
    if rc < 0:
        raise ValueError(f"oracle_forward: error {rc}")
    return out, rc


def permute(ids, E: int):
    ids = _c(ids, np.int32)
    M, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.full(M * k, -1, np.int32)
    rc = lib().oracle_permute(_ptr(ids), M, k, E, _ptr(counts), _ptr(offsets), _ptr(perm))
    if rc < 0:
        raise ValueError("oracle_permute: bad arguments")
    return counts, offsets, perm, rc


def rmsnorm(y_bits, eps: float = 1e-6):
    y = _c(y_bits, np.uint16)
    M, H = y.shape
    out = np.empty_like(y)
    if lib().oracle_rmsnorm(_ptr(y), M, H, eps, _ptr(out)) != 0:
        raise ValueError("oracle_rmsnorm: bad arguments")
    return out


def e4m3_to_f64(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    return np.array([lib().oracle_e4m3_to_f64(int(v)) for v in c.ravel()]).reshape(c.shape)


def f32_to_e4m3(v) -> np.ndarray:
    v = _c(v, np.float32)
    return np.array([lib().oracle_f32_to_e4m3(float(a)) for a in v.ravel()], np.uint8).reshape(v.shape)


def e2m1_to_f64(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    return np.array([lib().oracle_e2m1_to_f64(int(v)) for v in c.ravel()]).reshape(c.shape)


def e8m0_to_f64(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    return np.array([lib().oracle_e8m0_to_f64(int(v)) for v in c.ravel()]).reshape(c.shape)


def lmhead_quantize(w_bits):
    """w bf16 [V][H] -> (q uint8 E4M3 [V][H], s float32 [V])."""
    w = _c(w_bits, np.uint16)
    V, H = w.shape
    q = np.empty((V, H), np.uint8)
    sc = np.empty(V, np.float32)
    if lib().oracle_lmhead_quantize(_ptr(w), V, H, _ptr(q), _ptr(sc)) != 0:
        raise ValueError("oracle_lmhead_quantize: bad arguments")
    return q, sc


def lmhead_gemv_fp8(q, sc, x_bits) -> np.ndarray:
    q, sc = _c(q, np.uint8), _c(sc, np.float32)
    V, H = q.shape
    x = _c(x_bits, np.uint16).reshape(-1, H)
    out = np.empty((x.shape[0], V), np.float64)
    if lib().oracle_lmhead_gemv_fp8(_ptr(q), _ptr(sc), V, H, _ptr(x), x.shape[0], _ptr(out)) != 0:
        raise ValueError("oracle_lmhead_gemv_fp8: bad arguments")
    return out


def lmhead_gemv_bf16(w_bits, x_bits) -> np.ndarray:
    w = _c(w_bits, np.uint16)
    V, H = w.shape
    x = _c(x_bits, np.uint16).reshape(-1, H)
    out = np.empty((x.shape[0], V), np.float64)
    if lib().oracle_lmhead_gemv_bf16(_ptr(w), V, H, _ptr(x), x.shape[0], _ptr(out)) != 0:
        raise ValueError("oracle_lmhead_gemv_bf16: bad arguments")
    return out


def dequant_fmt(fmt: int, q, s, N: int, K: int) -> np.ndarray:
    q, s = _c(q, np.uint8), _c(s, _SCALE_DTYPE[fmt])
    W = np.empty((N, K), np.float64)
    if lib().oracle_dequant_fmt(fmt, _ptr(q), _ptr(s), N, K, _ptr(W)) != 0:
        raise ValueError("oracle_dequant_fmt: bad arguments")
    return W


def forward_fmt(shape, fmt: int, experts, x, ids, w):
    """oracle_forward with the routed experts in format fmt: experts maps
    w13_q/w13_s/w2_q/w2_s to {expert id: array} (or [E]-leading arrays) and
    holds sh_w13/sh_w2.  Returns (out float64 [M][H], bad-id count)."""
    E = shape.n_experts
    x = _c(x, np.uint16).reshape(-1, shape.hidden)
    ids = _c(ids, np.int32).reshape(x.shape[0], shape.top_k)
    w = _c(w, np.float64).reshape(x.shape[0], shape.top_k)
    keep = []

    def table(name, dtype):
        src = experts[name]
        arr = (ctypes.c_void_p * E)()
        for e in range(E):
            a = src.get(e) if isinstance(src, dict) else src[e]
            if a is not None:
                a = _c(a, dtype)
                keep.append(a)
                arr[e] = a.ctypes.data
        keep.append(arr)
        return ctypes.cast(arr, ctypes.c_void_p)

    sh13, sh2 = experts.get("sh_w13"), experts.get("sh_w2")
    sh13 = None if sh13 is None else _c(sh13, np.uint16)
    sh2 = None if sh2 is None else _c(sh2, np.uint16)
    sd = _SCALE_DTYPE[fmt]
    ex = _ExpertsFmt(fmt, table("w13_q", np.uint8), table("w13_s", sd), table("w2_q", np.uint8),
                     table("w2_s", sd), _ptr(sh13), _ptr(sh2))
    out = np.empty((x.shape[0], shape.hidden), np.float64)
    c = _cfg(shape)
    rc = lib().oracle_forward_fmt(ctypes.byref(c), ctypes.byref(ex), _ptr(x), x.shape[0], _ptr(ids), _ptr(w),
                                  _ptr(out))
    if rc < 0:
        raise ValueError(f"oracle_forward_fmt: error {rc}")
    return out, rc
