"""The C-ABI library loads, exports every symbol include/moe_w4a16.h declares,
and rejects bad arguments before launching anything (no GPU needed: every case
here fails validation, so no HIP call is made)."""
import ctypes
import os
import re

import pytest

from w4a16_grouped_quantized_amd import binding as B
from w4a16_grouped_quantized_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4a16.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmoe_w4a16.so is not built (python -m w4a16_grouped_quantized_amd.build)")
    return B.lib()


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert set(declared) == set(B.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_build_info_and_status_strings(lib):
    info = B.build_info()
    assert "gfx950" in info and "layout=" in info
    for rc in range(0, -8, -1):
        assert B.status_string(rc) and B.status_string(rc) != "unknown status"
    assert B.status_string(-99) == "unknown status"


def _cfg(**kw):
    d = dict(hidden=2560, n_experts=512, top_k=8, inter=768, group_size=32, has_shared=1)
    d.update(kw)
    return B.MoeConfig(**d)


def test_sizes(lib):
    c = B.config(synth.LING)
    # packed blob = plain bytes (routed codes + scales + shared) + 16 bytes of
    # range data per expert, each section 256-aligned
    E, H, I = 512, 2560, 768
    plain = E * (2 * I * H // 2 + 2 * I * (H // 32) * 2 + H * I // 2 + H * (I // 32) * 2) + (2 * I * H + H * I) * 2
    assert B.packed_size(c) == plain + E * 16
    assert B.workspace_size(c, 1) > 0
    assert B.workspace_size(c, 4) > B.workspace_size(c, 1)
    assert B.packed_size(_cfg(group_size=64)) == 0
    assert B.workspace_size(_cfg(hidden=100), 1) == 0
    assert B.workspace_size(c, -1) == 0


@pytest.mark.parametrize("kw,rc", [
    (dict(group_size=64), -5),
    (dict(hidden=100), -2),
    (dict(hidden=0), -2),
    (dict(inter=40), -2),
    (dict(top_k=0), -2),
    (dict(top_k=600, n_experts=512), -2),
    (dict(n_experts=1024, top_k=8), -5),
    (dict(top_k=65, n_experts=128), -5),
    (dict(has_shared=2), -2),
    (dict(hidden=8192), -5),
])
def test_config_validation(lib, kw, rc):
    c = _cfg(**kw)
    fake = ctypes.c_void_p(0x10000)
    got = lib.moe_route(ctypes.byref(c), fake, fake, 1, 0, None, fake, fake, fake, 1 << 30, None)
    assert got == rc
    got = lib.moe_forward_w4a16(ctypes.byref(c), fake, fake, 1, fake, fake, fake, fake, 1 << 30, None)
    assert got == rc


def test_pointer_and_size_validation(lib):
    c = _cfg()
    a = ctypes.c_void_p(0x10000)     # aligned, never dereferenced: every call below fails a check
    odd = ctypes.c_void_p(0x10001)
    big = 1 << 40
    assert lib.moe_route(None, a, a, 1, 0, None, a, a, a, big, None) == -1
    assert lib.moe_route(ctypes.byref(c), None, a, 1, 0, None, a, a, a, big, None) == -1
    assert lib.moe_route(ctypes.byref(c), a, a, 1, B.MOE_F_INPUT_RMSNORM, None, a, a, a, big, None) == -1
    assert lib.moe_route(ctypes.byref(c), a, a, 1, 0x8, None, a, a, a, big, None) == -2
    assert lib.moe_route(ctypes.byref(c), a, a, -1, 0, None, a, a, a, big, None) == -2
    assert lib.moe_route(ctypes.byref(c), a, odd, 1, 0, None, a, a, a, big, None) == -3
    assert lib.moe_route(ctypes.byref(c), a, a, 1, 0, None, a, a, a, 16, None) == -4
    # M = 0 is a no-op and succeeds without touching any pointer
    assert lib.moe_route(ctypes.byref(c), None, None, 0, 0, None, None, None, None, 0, None) == 0
    assert lib.moe_forward_w4a16(ctypes.byref(c), None, None, 0, None, None, None, None, 0, None) == 0
    assert lib.moe_forward_w4a16(ctypes.byref(c), a, a, 1, a, a, None, a, big, None) == -1
    assert lib.moe_forward_w4a16(ctypes.byref(c), odd, a, 1, a, a, a, a, big, None) == -3
    assert lib.moe_forward_w4a16(ctypes.byref(c), a, a, 1, a, a, a, a, 64, None) == -4
    # more (token, slot) pairs than the small-M kernels take, for a shape the
    # many-token kernels are not compiled for (the tiny layer)
    tiny = B.config(synth.TINY)
    assert lib.moe_forward_w4a16(ctypes.byref(tiny), a, a, 2049, a, a, a, a, big, None) == -5
    assert lib.moe_permute(ctypes.byref(c), a, 4, None, a, a, a, big, None) == -1
    assert lib.moe_permute(ctypes.byref(c), a, 4, a, a, a, a, 8, None) == -4
    w = B.MoeWeightsPlain(a, a, a, a, None, None)   # shared expert missing while has_shared = 1
    assert lib.moe_pack_weights(ctypes.byref(c), ctypes.byref(w), a, big, None) == -1
    w = B.MoeWeightsPlain(a, a, a, a, a, a)
    assert lib.moe_pack_weights(ctypes.byref(c), ctypes.byref(w), a, 1024, None) == -4
    assert lib.moe_workspace_init(None, 64, None) == -1
    assert lib.moe_workspace_init(odd, 64, None) == -3
    code = ctypes.c_int32(0)
    assert lib.moe_get_device_error(None, None, ctypes.byref(code)) == -1


def test_rmsnorm_output_must_not_overlap_input(lib):
    """With MOE_F_INPUT_RMSNORM the call writes x_norm while other
    workgroups of the same launch still read x: an overlap is refused before
    anything is launched (moe_route and moe_layer_w4a16)."""
    c = _cfg()
    H = c.hidden
    base = 0x100000
    a = ctypes.c_void_p(base)
    big = 1 << 40
    rms = B.MOE_F_INPUT_RMSNORM
    for M in (1, 4):
        row = H * 2
        for xn in (base, base + 16, base + M * row - 16):       # in place, shifted inside x
            p = ctypes.c_void_p(xn)
            assert lib.moe_route(ctypes.byref(c), a, a, M, rms, p, a, a, a, big, None) == -2, (M, xn)
            assert lib.moe_layer_w4a16(ctypes.byref(c), a, a, a, M, rms, p, a, a, a, a, big, None) == -2, (M, xn)
        # adjacent but disjoint buffers pass this check (and then fail the
        # workspace-size check, so nothing is launched)
        after = ctypes.c_void_p(base + M * row)
        assert lib.moe_route(ctypes.byref(c), a, a, M, rms, after, a, a, a, 16, None) == -4
        before = ctypes.c_void_p(base - M * row)
        assert lib.moe_layer_w4a16(ctypes.byref(c), a, a, a, M, rms, before, a, a, a, a, 16, None) == -4


def test_read_probe_validation(lib):
    a = ctypes.c_void_p(0x10000)
    assert lib.moe_probe_read(None, 64, a, 8, None) == -1
    assert lib.moe_probe_read(a, 64, None, 8, None) == -1
    assert lib.moe_probe_read(ctypes.c_void_p(0x10004), 64, a, 8, None) == -3
    assert lib.moe_probe_read(a, 65, a, 8, None) == -3
    assert lib.moe_probe_read(a, 64, a, 0, None) == -2
    assert lib.moe_probe_read(a, 0, a, 8, None) == 0


def test_noalloc_limits_checked_on_the_host(lib):
    """moe_layer_w4a16_noalloc: the static workspace size the binding uses is
    the header's, and sizes are refused before the device is touched."""
    hdr = open(HEADER).read()
    m = re.search(r"#define MOE_NOALLOC_WS_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == B.MOE_NOALLOC_WS_BYTES
    cfg = B.config(synth.LING)
    a = ctypes.c_void_p(0x10000)
    big = 1
    while lib.moe_workspace_size(ctypes.byref(cfg), big) <= B.MOE_NOALLOC_WS_BYTES:
        big += 1
    assert big > 64
    args = (0, None, a, a, a, None)  # flags, x_norm, ids, weights, out, stream
    assert lib.moe_layer_w4a16_noalloc(ctypes.byref(cfg), a, a, a, big, *args) == B.MOE_ERR_WORKSPACE
    assert lib.moe_layer_w4a16_noalloc(ctypes.byref(cfg), a, a, a, -1, *args) == -2
    assert lib.moe_layer_w4a16_noalloc(ctypes.byref(cfg), a, a, a, 0, *args) == 0
    assert lib.moe_layer_w4a16_noalloc(None, a, a, a, 1, *args) == -1


def test_mxfp4_layer_host_checks(lib):
    """The MXFP4 one-launch entry points refuse bad arguments on the host
    (nothing is launched): the packed size counts one byte per E8M0 scale,
    and the layer covers only what the one-launch kernel covers."""
    cfg = B.config(synth.LING)
    E, H, I = 512, 2560, 768
    plain = E * (2 * I * H // 2 + 2 * I * (H // 32) + H * I // 2 + H * (I // 32)) + (2 * I * H + H * I) * 2
    assert lib.moe_packed_size_mxfp4(ctypes.byref(cfg)) == plain + E * 16
    assert lib.moe_packed_size_mxfp4(ctypes.byref(cfg)) < lib.moe_packed_size(ctypes.byref(cfg))
    a = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10001)
    w = B.MoeWeightsFmt(a, a, a, a, a, a)
    n = lib.moe_packed_size_mxfp4(ctypes.byref(cfg))
    assert lib.moe_pack_weights_mxfp4(ctypes.byref(cfg), None, a, n, None) == -1
    assert lib.moe_pack_weights_mxfp4(ctypes.byref(cfg), ctypes.byref(w), a, n - 1, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_pack_weights_mxfp4(ctypes.byref(cfg), ctypes.byref(w), odd, n, None) == -3
    nos = B.MoeWeightsFmt(a, a, a, a, None, None)
    assert lib.moe_pack_weights_mxfp4(ctypes.byref(cfg), ctypes.byref(nos), a, n, None) == -1
    ws = 1 << 30

    def call(M, flags=0, x=a, x_norm=None, out=a):
        return lib.moe_layer_mxfp4(ctypes.byref(cfg), a, a, x, M, flags, x_norm, a, a, out, a, ws, None)

    assert call(0) == 0
    assert call(-1) == -2
    assert call(1, flags=B.MOE_F_ONE_LAUNCH) == -2  # only MOE_F_INPUT_RMSNORM
    assert call(1, flags=B.MOE_F_INPUT_RMSNORM) == -1  # x_norm missing
    assert call(1, flags=B.MOE_F_INPUT_RMSNORM, x_norm=a) == -2  # x_norm overlaps x
    assert call(1, out=odd) == -3
    assert call(5) == -5  # more tokens than the one launch takes
    assert lib.moe_layer_mxfp4(None, a, a, a, 1, 0, None, a, a, a, a, ws, None) == -1
