"""ctypes binding of libmoe_w4a16.so (include/moe_w4a16.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  The library
must be built (``python -m w4a16_grouped_quantized_amd.build``); a missing
library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_w4a16.so")

MOE_F_INPUT_RMSNORM = 0x1
MOE_F_ONE_LAUNCH = 0x2
MOE_ERR_WORKSPACE = -4
MOE_FMT_MXFP4 = 1
MOE_FMT_FP8_BLOCK = 2
# bytes of the static workspace of moe_layer_w4a16_noalloc (MOE_NOALLOC_WS_BYTES)
MOE_NOALLOC_WS_BYTES = 16 << 20

MOE_OK = 0
STATUS_NAMES = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_ALIGN",
                -4: "MOE_ERR_WORKSPACE", -5: "MOE_ERR_UNSUPPORTED", -6: "MOE_ERR_LAUNCH",
                -7: "MOE_ERR_DEVICE"}

# Every symbol include/moe_w4a16.h declares.
EXPORTS = ("moe_packed_size", "moe_pack_weights", "moe_workspace_size", "moe_workspace_init",
           "moe_route", "moe_forward_w4a16", "moe_layer_w4a16", "moe_gate_up_w4a16", "moe_down_w4a16", "moe_permute",
           "moe_get_device_error", "moe_status_string", "moe_build_info", "moe_probe_read",
           "moe_layer_w4a16_noalloc", "moe_lmhead_quantize_fp8", "moe_lmhead_fp8", "moe_lmhead_bf16",
           "moe_forward_fmt", "moe_packed_size_mxfp4", "moe_pack_weights_mxfp4", "moe_layer_mxfp4")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


class MoeConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("has_shared", ctypes.c_int32)]


class MoeWeightsFmt(ctypes.Structure):
    """moe_weights_fmt: device pointers of routed experts in MXFP4 or block FP8."""
    _fields_ = [("w13_q", ctypes.c_void_p), ("w13_s", ctypes.c_void_p), ("w2_q", ctypes.c_void_p),
                ("w2_s", ctypes.c_void_p), ("sh_w13", ctypes.c_void_p), ("sh_w2", ctypes.c_void_p)]


_P = ctypes.c_void_p


class MoeWeightsPlain(ctypes.Structure):
    _fields_ = [("w13_q", _P), ("w13_s", _P), ("w2_q", _P), ("w2_s", _P),
                ("sh_w13", _P), ("sh_w2", _P)]


_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built; run python -m w4a16_grouped_quantized_amd.build")
            L = ctypes.CDLL(LIB_PATH)
            cfgp = ctypes.POINTER(MoeConfig)
            L.moe_packed_size.restype = ctypes.c_size_t
            L.moe_packed_size.argtypes = [cfgp]
            L.moe_pack_weights.argtypes = [cfgp, ctypes.POINTER(MoeWeightsPlain), _P, ctypes.c_size_t, _P]
            L.moe_workspace_size.restype = ctypes.c_size_t
            L.moe_workspace_size.argtypes = [cfgp, ctypes.c_int32]
            L.moe_workspace_init.argtypes = [_P, ctypes.c_size_t, _P]
            L.moe_route.argtypes = [cfgp, _P, _P, ctypes.c_int32, ctypes.c_uint32, _P, _P, _P, _P,
                                    ctypes.c_size_t, _P]
            L.moe_forward_w4a16.argtypes = [cfgp, _P, _P, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_size_t, _P]
            L.moe_layer_w4a16.argtypes = [cfgp, _P, _P, _P, ctypes.c_int32, ctypes.c_uint32, _P, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]
            L.moe_layer_w4a16_noalloc.argtypes = [cfgp, _P, _P, _P, ctypes.c_int32, ctypes.c_uint32, _P, _P, _P,
                                                  _P, _P]
            L.moe_forward_fmt.argtypes = [cfgp, ctypes.c_int32, ctypes.POINTER(MoeWeightsFmt), _P, ctypes.c_int32,
                                          _P, _P, _P, _P, ctypes.c_size_t, _P]
            L.moe_packed_size_mxfp4.restype = ctypes.c_size_t
            L.moe_packed_size_mxfp4.argtypes = [cfgp]
            L.moe_pack_weights_mxfp4.argtypes = [cfgp, ctypes.POINTER(MoeWeightsFmt), _P, ctypes.c_size_t, _P]
            L.moe_layer_mxfp4.argtypes = [cfgp, _P, _P, _P, ctypes.c_int32, ctypes.c_uint32, _P, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]
            L.moe_lmhead_quantize_fp8.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
            L.moe_lmhead_fp8.argtypes = [_P, _P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P, _P]
            L.moe_lmhead_bf16.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P, _P]
            L.moe_gate_up_w4a16.argtypes = [cfgp, _P, _P, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]
            L.moe_down_w4a16.argtypes = [cfgp, _P, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_size_t, _P]
            L.moe_permute.argtypes = [cfgp, _P, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_size_t, _P]
            L.moe_get_device_error.argtypes = [_P, _P, ctypes.POINTER(ctypes.c_int32)]
            L.moe_status_string.restype = ctypes.c_char_p
            L.moe_status_string.argtypes = [ctypes.c_int]
            L.moe_build_info.restype = ctypes.c_char_p
            L.moe_build_info.argtypes = []
            L.moe_probe_read.argtypes = [_P, ctypes.c_size_t, _P, ctypes.c_int32, _P]
            _lib = L
        return _lib


def config(shape) -> MoeConfig:
    return MoeConfig(shape.hidden, shape.n_experts, shape.top_k, shape.inter, shape.group_size,
                     int(shape.has_shared))


def _check(fn: str, rc: int):
    if rc != MOE_OK:
        raise MoeError(fn, rc, lib().moe_status_string(rc).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def build_info() -> str:
    return lib().moe_build_info().decode()


def status_string(rc: int) -> str:
    return lib().moe_status_string(rc).decode()


def packed_size(cfg: MoeConfig) -> int:
    return lib().moe_packed_size(ctypes.byref(cfg))


def workspace_size(cfg: MoeConfig, max_tokens: int) -> int:
    return lib().moe_workspace_size(ctypes.byref(cfg), max_tokens)


def pack_weights(cfg, w13_q, w13_s, w2_q, w2_s, sh_w13, sh_w2, packed, stream=None):
    src = MoeWeightsPlain(_ptr(w13_q), _ptr(w13_s), _ptr(w2_q), _ptr(w2_s), _ptr(sh_w13), _ptr(sh_w2))
    _check("moe_pack_weights", lib().moe_pack_weights(ctypes.byref(cfg), ctypes.byref(src), _ptr(packed),
                                                      packed.numel() * packed.element_size(), _stream(stream)))


def workspace_init(ws, stream=None):
    _check("moe_workspace_init", lib().moe_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def route(cfg, router_w, x, topk_ids, topk_w, ws, flags: int = 0, x_norm=None, stream=None):
    M = x.shape[0]
    _check("moe_route", lib().moe_route(ctypes.byref(cfg), _ptr(router_w), _ptr(x), M, flags, _ptr(x_norm),
                                        _ptr(topk_ids), _ptr(topk_w), _ptr(ws), ws.numel() * ws.element_size(),
                                        _stream(stream)))


def forward(cfg, packed, x, topk_ids, topk_w, out, ws, stream=None):
    M = x.shape[0]
    _check("moe_forward_w4a16", lib().moe_forward_w4a16(ctypes.byref(cfg), _ptr(packed), _ptr(x), M,
                                                        _ptr(topk_ids), _ptr(topk_w), _ptr(out), _ptr(ws),
                                                        ws.numel() * ws.element_size(), _stream(stream)))


def layer(cfg, router_w, packed, x, topk_ids, topk_w, out, ws, flags: int = 0, x_norm=None, stream=None):
    M = x.shape[0]
    _check("moe_layer_w4a16", lib().moe_layer_w4a16(ctypes.byref(cfg), _ptr(router_w), _ptr(packed), _ptr(x), M,
                                                    flags, _ptr(x_norm), _ptr(topk_ids), _ptr(topk_w), _ptr(out),
                                                    _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def layer_noalloc(cfg, router_w, packed, x, topk_ids, topk_w, out, flags: int = 0, x_norm=None, stream=None):
    """moe_layer_w4a16 on the library's own static workspace (no allocation)."""
    M = x.shape[0]
    _check("moe_layer_w4a16_noalloc",
           lib().moe_layer_w4a16_noalloc(ctypes.byref(cfg), _ptr(router_w), _ptr(packed), _ptr(x), M, flags,
                                         _ptr(x_norm), _ptr(topk_ids), _ptr(topk_w), _ptr(out), _stream(stream)))


def gate_up(cfg, packed, x, topk_ids, ws, stream=None):
    M = x.shape[0]
    _check("moe_gate_up_w4a16", lib().moe_gate_up_w4a16(ctypes.byref(cfg), _ptr(packed), _ptr(x), M,
                                                        _ptr(topk_ids), _ptr(ws), ws.numel() * ws.element_size(),
                                                        _stream(stream)))


def down(cfg, packed, topk_ids, topk_w, out, ws, stream=None):
    M = topk_ids.shape[0]
    _check("moe_down_w4a16", lib().moe_down_w4a16(ctypes.byref(cfg), _ptr(packed), M, _ptr(topk_ids),
                                                  _ptr(topk_w), _ptr(out), _ptr(ws),
                                                  ws.numel() * ws.element_size(), _stream(stream)))


def permute(cfg, topk_ids, counts, offsets, perm, ws, stream=None):
    M = topk_ids.shape[0]
    _check("moe_permute", lib().moe_permute(ctypes.byref(cfg), _ptr(topk_ids), M, _ptr(counts), _ptr(offsets),
                                            _ptr(perm), _ptr(ws), ws.numel() * ws.element_size(),
                                            _stream(stream)))


def probe_read(buf, sink, blocks: int, stream=None):
    _check("moe_probe_read", lib().moe_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                                  blocks, _stream(stream)))


def get_device_error(ws, stream=None) -> int:
    code = ctypes.c_int32(0)
    rc = lib().moe_get_device_error(_ptr(ws), _stream(stream), ctypes.byref(code))
    if rc not in (MOE_OK, -7):
        _check("moe_get_device_error", rc)
    return code.value


class MoeLayer:
    """One layer resident on the GPU: router (fp32, plain layout) and the
    packed expert blob, built from a synth.Layer (numpy, plain layout)."""

    def __init__(self, layer, device="cuda"):
        import torch
        self.shape = layer.shape
        self.cfg = config(layer.shape)
        dev = torch.device(device)

        def up(a, dtype):
            return torch.from_numpy(np.ascontiguousarray(a).view(dtype)).to(dev)

        self.router_w = up(layer.router_w, np.float32)
        n = packed_size(self.cfg)
        if n == 0:
            raise MoeError("moe_packed_size", -2, "invalid config")
        self.packed = torch.empty(n, dtype=torch.uint8, device=dev)
        w13_q, w13_s = up(layer.w13_q, np.uint8), up(layer.w13_s, np.int16)
        w2_q, w2_s = up(layer.w2_q, np.uint8), up(layer.w2_s, np.int16)
        sh13 = up(layer.sh_w13, np.int16) if layer.shape.has_shared else None
        sh2 = up(layer.sh_w2, np.int16) if layer.shape.has_shared else None
        pack_weights(self.cfg, w13_q, w13_s, w2_q, w2_s, sh13, sh2, self.packed)
        torch.cuda.current_stream().synchronize()
        del w13_q, w13_s, w2_q, w2_s, sh13, sh2


class Workspace:
    def __init__(self, cfg: MoeConfig, max_tokens: int, device="cuda"):
        import torch
        n = workspace_size(cfg, max_tokens)
        if n == 0:
            raise MoeError("moe_workspace_size", -2, "invalid config or max_tokens")
        self.buf = torch.empty(n, dtype=torch.uint8, device=device)
        workspace_init(self.buf)


def lmhead_quantize_fp8(w, q, scale, stream=None):
    """w bf16 [V][H] -> q uint8 [V][H] (E4M3 codes), scale float32 [V]."""
    V, H = w.shape
    _check("moe_lmhead_quantize_fp8", lib().moe_lmhead_quantize_fp8(_ptr(w), V, H, _ptr(q), _ptr(scale), _stream(stream)))


def lmhead_fp8(q, scale, x, logits, stream=None):
    """logits float32 [M][V] from the FP8 head q [V][H], scale [V] and x bf16 [M][H]."""
    V, H = q.shape
    _check("moe_lmhead_fp8", lib().moe_lmhead_fp8(_ptr(q), _ptr(scale), V, H, _ptr(x), x.shape[0], _ptr(logits),
                                                  _stream(stream)))


def lmhead_bf16(w, x, logits, stream=None):
    """logits float32 [M][V] from the BF16 head w [V][H] and x bf16 [M][H]."""
    V, H = w.shape
    _check("moe_lmhead_bf16", lib().moe_lmhead_bf16(_ptr(w), V, H, _ptr(x), x.shape[0], _ptr(logits), _stream(stream)))



class FmtLayerDev:
    """A synth.FmtLayer (MXFP4 or block-FP8 routed experts) resident on the
    GPU in its plain layout, with its router."""

    def __init__(self, layer, device="cuda"):
        import torch
        self.shape, self.fmt = layer.shape, layer.fmt
        self.cfg = config(layer.shape)
        dev = torch.device(device)

        def up(a):
            a = np.ascontiguousarray(a)
            return torch.from_numpy(a.view(np.uint8).reshape(-1)).to(dev)

        self.router_w = torch.from_numpy(np.ascontiguousarray(layer.router_w)).to(dev)
        self.w13_q, self.w13_s, self.w2_q, self.w2_s = (up(layer.w13_q), up(layer.w13_s), up(layer.w2_q),
                                                        up(layer.w2_s))
        self.sh_w13 = up(layer.sh_w13) if layer.shape.has_shared else None
        self.sh_w2 = up(layer.sh_w2) if layer.shape.has_shared else None
        self.weights = MoeWeightsFmt(_ptr(self.w13_q), _ptr(self.w13_s), _ptr(self.w2_q), _ptr(self.w2_s),
                                     _ptr(self.sh_w13), _ptr(self.sh_w2))


class MxLayerDev:
    """An MXFP4 synth.FmtLayer packed into the tiled layout of the one-launch
    layer (moe_pack_weights_mxfp4), with its router; the plain device copy is
    released after packing unless keep_plain."""

    def __init__(self, layer, device="cuda", keep_plain: bool = False):
        import torch
        if layer.fmt != MOE_FMT_MXFP4:
            raise ValueError("MxLayerDev takes an MXFP4 layer")
        plain = FmtLayerDev(layer, device)
        self.shape, self.cfg, self.router_w = plain.shape, plain.cfg, plain.router_w
        n = lib().moe_packed_size_mxfp4(ctypes.byref(self.cfg))
        if n == 0:
            raise MoeError("moe_packed_size_mxfp4", -2, "invalid config")
        self.packed = torch.empty(n, dtype=torch.uint8, device=device)
        _check("moe_pack_weights_mxfp4",
               lib().moe_pack_weights_mxfp4(ctypes.byref(self.cfg), ctypes.byref(plain.weights), _ptr(self.packed),
                                            n, _stream(None)))
        torch.cuda.current_stream().synchronize()
        self.plain = plain if keep_plain else None


def layer_mxfp4(cfg, router_w, packed, x, topk_ids, topk_w, out, ws, flags: int = 0, x_norm=None, stream=None):
    """moe_layer_mxfp4: the MXFP4 layer in one launch (packed by MxLayerDev)."""
    M = x.shape[0]
    _check("moe_layer_mxfp4", lib().moe_layer_mxfp4(ctypes.byref(cfg), _ptr(router_w), _ptr(packed), _ptr(x), M,
                                                    flags, _ptr(x_norm), _ptr(topk_ids), _ptr(topk_w), _ptr(out),
                                                    _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def forward_fmt(dl: FmtLayerDev, x, topk_ids, topk_w, out, ws, stream=None):
    """moe_forward_fmt: out bf16 [M][H] with the routed experts of dl."""
    _check("moe_forward_fmt", lib().moe_forward_fmt(ctypes.byref(dl.cfg), dl.fmt, ctypes.byref(dl.weights), _ptr(x),
                                                    x.shape[0], _ptr(topk_ids), _ptr(topk_w), _ptr(out), _ptr(ws),
                                                    ws.numel() * ws.element_size(), _stream(stream)))
