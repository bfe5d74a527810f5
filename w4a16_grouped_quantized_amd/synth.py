"""Seeded synthetic inputs for the W4A16 grouped-quantized MoE layer.

This module only draws random numbers and encodes them into the storage
formats the layer consumes. It holds none of the layer's arithmetic (no
dequantisation, routing, matmul or activation) and serves both the HIP path
and the CPU oracle, which otherwise share no code.

Shapes (hidden 2560, 512 routed experts, top-8, moe_intermediate_size 768,
one BF16 shared expert) follow the Ling-3.0-flash descriptions: the vLLM
recipe page "inclusionAI/Ling-3.0-flash" (Overview: 512 routed experts,
8 active, one shared expert) and the bpdata.com article on Ling-3.0-flash MoE
inference (model section: hidden 2,560; Humming section:
moe_intermediate_size = 768).  The weight format follows the recipe page's
"Single-GPU int4" section: symmetric W4, group_size 32, routed experts only.

Plain ("checkpoint") layout produced here, all row-major, K contiguous:

  router_w  float32 [E][H]
  w13_q     uint8   [E][2I][H/2]   code u = q + 8, low nibble = even k
  w13_s     uint16  [E][2I][H/G]   bf16 bit patterns; rows [0,I) gate, [I,2I) up
  w2_q      uint8   [E][H][I/2]
  w2_s      uint16  [E][H][I/G]
  sh_w13    uint16  [2I][H]        bf16
  sh_w2     uint16  [H][I]         bf16

Distributions: router N(0, 0.02^2) in fp32; q uniform over the 15 integers
-7..7 (code -8 is never drawn); scales bf16(|N(0,1)| * 0.02); shared weights
bf16(N(0,1) * 0.02); x bf16(N(0,1)).  bf16(v) means: round v to float32
(round-to-nearest-even), then to bf16 (round-to-nearest-even).

Seeding: numpy PCG64 via SeedSequence(seed).spawn(8) in the fixed order
[router, w13_q, w13_s, w2_q, w2_s, sh_w13, sh_w2, x]; the four routed streams
are split again per expert (child.spawn(E)), so any single expert can be
regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "LayerShape", "TINY", "LING", "Layer", "make_layer", "make_expert",
    "make_tokens", "bf16_bits", "bf16_bits_to_f32", "pack_codes",
    "unpack_codes_reference_free", "FMT_INT4_G32", "FMT_MXFP4", "FMT_FP8_BLOCK",
    "FmtLayer", "make_layer_fmt", "make_lmhead", "LM_VOCAB",
]


@dataclasses.dataclass(frozen=True)
class LayerShape:
    hidden: int        # H
    n_experts: int     # E
    top_k: int         # k
    inter: int         # I  (moe_intermediate_size)
    group_size: int = 32
    has_shared: bool = True

    def __post_init__(self):
        if self.hidden % self.group_size or self.inter % self.group_size:
            raise ValueError("hidden and inter must be multiples of group_size")
        if not (1 <= self.top_k <= self.n_experts):
            raise ValueError("need 1 <= top_k <= n_experts")


# Tiny layer: hidden 256, 16 experts, top-2, intermediate 64, no shared expert.
TINY = LayerShape(hidden=256, n_experts=16, top_k=2, inter=64, has_shared=False)
# Ling-3.0-flash MoE layer shape.
LING = LayerShape(hidden=2560, n_experts=512, top_k=8, inter=768, has_shared=True)

_STREAMS = ("router", "w13_q", "w13_s", "w2_q", "w2_s", "sh_w13", "sh_w2", "x")


def bf16_bits(v) -> np.ndarray:
    """bf16 bit patterns (uint16) of v: round to float32, then to bf16 (RNE)."""
    f = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes [..., K] (values 0..15) two per byte along the last
    axis: element 2j in the low nibble, element 2j+1 in the high nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2:
        raise ValueError("last axis must be even")
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes_reference_free(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_codes (codes, not values): used only to check that
    packing is lossless."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def _seeds(seed: int, shape: LayerShape):
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    d = dict(zip(_STREAMS, kids))
    per_expert = {n: d[n].spawn(shape.n_experts) for n in ("w13_q", "w13_s", "w2_q", "w2_s")}
    return d, per_expert


def _draw_q(ss, rows: int, cols: int, return_q: bool):
    rng = np.random.Generator(np.random.PCG64(ss))
    q = rng.integers(-7, 8, size=(rows, cols), dtype=np.int8)
    packed = pack_codes((q + 8).astype(np.uint8))
    return packed, (q if return_q else None)


def _draw_scales(ss, rows: int, ngroups: int):
    rng = np.random.Generator(np.random.PCG64(ss))
    return bf16_bits(np.abs(rng.standard_normal((rows, ngroups))) * 0.02)


def make_expert(shape: LayerShape, seed: int, e: int, return_q: bool = False) -> dict:
    """Regenerate routed expert e of layer `seed` on its own."""
    H, I, G = shape.hidden, shape.inter, shape.group_size
    _, pe = _seeds(seed, shape)
    w13_q, q13 = _draw_q(pe["w13_q"][e], 2 * I, H, return_q)
    w2_q, q2 = _draw_q(pe["w2_q"][e], H, I, return_q)
    out = dict(w13_q=w13_q, w13_s=_draw_scales(pe["w13_s"][e], 2 * I, H // G),
               w2_q=w2_q, w2_s=_draw_scales(pe["w2_s"][e], H, I // G))
    if return_q:
        out.update(q13=q13, q2=q2)
    return out


@dataclasses.dataclass
class Layer:
    shape: LayerShape
    seed: int
    router_w: np.ndarray
    w13_q: np.ndarray
    w13_s: np.ndarray
    w2_q: np.ndarray
    w2_s: np.ndarray
    sh_w13: np.ndarray | None
    sh_w2: np.ndarray | None
    q13: np.ndarray | None = None   # int8 codes before packing (only if asked)
    q2: np.ndarray | None = None


def make_layer(shape: LayerShape, seed: int, return_q: bool = False, threads: int = 8) -> Layer:
    """Generate one whole layer in the plain layout."""
    H, I, E, G = shape.hidden, shape.inter, shape.n_experts, shape.group_size
    d, _ = _seeds(seed, shape)
    router = (np.random.Generator(np.random.PCG64(d["router"])).standard_normal((E, H)) * 0.02).astype(np.float32)
    w13_q = np.empty((E, 2 * I, H // 2), np.uint8)
    w13_s = np.empty((E, 2 * I, H // G), np.uint16)
    w2_q = np.empty((E, H, I // 2), np.uint8)
    w2_s = np.empty((E, H, I // G), np.uint16)
    q13 = np.empty((E, 2 * I, H), np.int8) if return_q else None
    q2 = np.empty((E, H, I), np.int8) if return_q else None

    def one(e):
        x = make_expert(shape, seed, e, return_q)
        w13_q[e], w13_s[e], w2_q[e], w2_s[e] = x["w13_q"], x["w13_s"], x["w2_q"], x["w2_s"]
        if return_q:
            q13[e], q2[e] = x["q13"], x["q2"]

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(E)))
    sh13 = sh2 = None
    if shape.has_shared:
        sh13 = bf16_bits(np.random.Generator(np.random.PCG64(d["sh_w13"])).standard_normal((2 * I, H)) * 0.02)
        sh2 = bf16_bits(np.random.Generator(np.random.PCG64(d["sh_w2"])).standard_normal((H, I)) * 0.02)
    return Layer(shape, seed, router, w13_q, w13_s, w2_q, w2_s, sh13, sh2, q13, q2)


def make_router(shape: LayerShape, seed: int) -> np.ndarray:
    """The router of layer `seed` alone (same values make_layer draws)."""
    d, _ = _seeds(seed, shape)
    rng = np.random.Generator(np.random.PCG64(d["router"]))
    return (rng.standard_normal((shape.n_experts, shape.hidden)) * 0.02).astype(np.float32)


def make_tokens(shape: LayerShape, seed: int, M: int) -> np.ndarray:
    """x: bf16 bit patterns [M][H], bf16(N(0,1))."""
    d, _ = _seeds(seed, shape)
    rng = np.random.Generator(np.random.PCG64(d["x"]))
    return bf16_bits(rng.standard_normal((M, shape.hidden)))


# ---------------------------------------------------------------- other formats
#
# Routed experts in the two other formats the pages serve, for the same
# layer shapes: MXFP4 (bpdata.com article, model section and "Optimalizáció
# 1": the FP4 checkpoint run with MXFP4 MoE kernels) and block FP8 (vLLM
# recipe page, Overview / Prerequisites: the serialized block-FP8
# checkpoint).  The codes are drawn directly in the storage format:
#
#   MXFP4      w13_q uint8 [E][2I][H/2], w2_q [E][H][I/2]: E2M1 nibbles (low
#              nibble = even k), each uniform over the 16 codes;
#              w13_s uint8 [E][2I][H/32], w2_s [E][H][I/32]: E8M0 scales,
#              uniform over 118..124 (2^-9 .. 2^-3);
#   FP8_BLOCK  w13_q uint8 [E][2I][H], w2_q [E][H][I]: E4M3 codes, uniform
#              over the 254 finite codes; w13_s float32
#              [E][ceil(2I/128)][ceil(H/128)], w2_s [E][ceil(H/128)][ceil(I/128)]:
#              |N(0,1)| * 3e-4 + 1e-5 per 128 x 128 block.
#
# The router and the shared expert are those of make_layer(shape, seed).
# Format streams: SeedSequence([seed, fmt]).spawn(4) in the order
# [w13_q, w13_s, w2_q, w2_s], each split per expert (child.spawn(E)).

FMT_INT4_G32, FMT_MXFP4, FMT_FP8_BLOCK = 0, 1, 2


@dataclasses.dataclass
class FmtLayer:
    shape: LayerShape
    seed: int
    fmt: int
    router_w: np.ndarray
    w13_q: np.ndarray
    w13_s: np.ndarray
    w2_q: np.ndarray
    w2_s: np.ndarray
    sh_w13: np.ndarray | None
    sh_w2: np.ndarray | None


def _fp8_codes(rng, shape):
    r = rng.integers(0, 254, size=shape, dtype=np.uint8)
    return np.where(r < 127, r, r + 1).astype(np.uint8)  # skips 0x7F; 0xFF is never reached


def make_layer_fmt(shape: LayerShape, seed: int, fmt: int, threads: int = 8) -> FmtLayer:
    """Layer `seed` with its routed experts in format fmt (MXFP4 or FP8_BLOCK)."""
    if fmt not in (FMT_MXFP4, FMT_FP8_BLOCK):
        raise ValueError("fmt must be FMT_MXFP4 or FMT_FP8_BLOCK")
    H, I, E, G = shape.hidden, shape.inter, shape.n_experts, shape.group_size
    d, _ = _seeds(seed, shape)
    router = (np.random.Generator(np.random.PCG64(d["router"])).standard_normal((E, H)) * 0.02).astype(np.float32)
    kids = [k.spawn(E) for k in np.random.SeedSequence([seed, fmt]).spawn(4)]
    if fmt == FMT_MXFP4:
        w13_q = np.empty((E, 2 * I, H // 2), np.uint8)
        w2_q = np.empty((E, H, I // 2), np.uint8)
        w13_s = np.empty((E, 2 * I, H // G), np.uint8)
        w2_s = np.empty((E, H, I // G), np.uint8)
    else:
        b = lambda n: (n + 127) // 128
        w13_q = np.empty((E, 2 * I, H), np.uint8)
        w2_q = np.empty((E, H, I), np.uint8)
        w13_s = np.empty((E, b(2 * I), b(H)), np.float32)
        w2_s = np.empty((E, b(H), b(I)), np.float32)

    def one(e):
        g = [np.random.Generator(np.random.PCG64(kids[i][e])) for i in range(4)]
        if fmt == FMT_MXFP4:
            w13_q[e] = g[0].integers(0, 256, size=w13_q.shape[1:], dtype=np.uint8)
            w13_s[e] = g[1].integers(118, 125, size=w13_s.shape[1:], dtype=np.uint8)
            w2_q[e] = g[2].integers(0, 256, size=w2_q.shape[1:], dtype=np.uint8)
            w2_s[e] = g[3].integers(118, 125, size=w2_s.shape[1:], dtype=np.uint8)
        else:
            w13_q[e] = _fp8_codes(g[0], w13_q.shape[1:])
            w13_s[e] = (np.abs(g[1].standard_normal(w13_s.shape[1:])) * 3e-4 + 1e-5).astype(np.float32)
            w2_q[e] = _fp8_codes(g[2], w2_q.shape[1:])
            w2_s[e] = (np.abs(g[3].standard_normal(w2_s.shape[1:])) * 3e-4 + 1e-5).astype(np.float32)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(E)))
    sh13 = sh2 = None
    if shape.has_shared:
        sh13 = bf16_bits(np.random.Generator(np.random.PCG64(d["sh_w13"])).standard_normal((2 * I, H)) * 0.02)
        sh2 = bf16_bits(np.random.Generator(np.random.PCG64(d["sh_w2"])).standard_normal((H, I)) * 0.02)
    return FmtLayer(shape, seed, fmt, router, w13_q, w13_s, w2_q, w2_s, sh13, sh2)


# Vocabulary of the LM head (bpdata.com article, model section: the LM head
# projects the 2,560-wide hidden state onto 157,184 tokens).
LM_VOCAB = 157184


def make_lmhead(V: int, H: int, seed: int, threads: int = 8) -> np.ndarray:
    """A BF16 LM head [V][H]: bf16(N(0,1) * 0.02), drawn in blocks of 4096
    rows, block b from SeedSequence([seed, 7, b])."""
    out = np.empty((V, H), np.uint16)
    starts = list(range(0, V, 4096))

    def one(r0):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7, r0 // 4096])))
        r1 = min(V, r0 + 4096)
        out[r0:r1] = bf16_bits(rng.standard_normal((r1 - r0, H), dtype=np.float32) * np.float32(0.02))

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, starts))
    return out
