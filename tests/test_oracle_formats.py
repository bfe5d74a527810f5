"""Pins for the oracle's further weight formats (FP8 E4M3, the online FP8 LM
head, MXFP4, block-FP8 experts) against facts that do not come from the
oracle itself: PyTorch's own float8_e4m3fn conversions (a library routine
the oracle does not use), the values the OCP 8-bit and MX formats define
(largest finite 448, smallest normal 2^-6 and subnormal 2^-9 for E4M3; the
eight E2M1 magnitudes; E8M0 = 2^(c-127)), numpy fp64 matmuls, and special
cases that reduce to the already pinned INT4 and BF16 paths of the oracle.
"""
import numpy as np
import pytest
import torch

from w4a16_grouped_quantized_amd import synth

# The eight E2M1 magnitudes of the OCP MX specification, codes 0..7.
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _torch_e4m3_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_e4m3_encode(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ---------------------------------------------------------------- E4M3

def test_e4m3_decode_matches_torch_for_every_code(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle_mod.e4m3_to_f64(codes)
    ref = _torch_e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(mine[~nan], ref[~nan])


def test_e4m3_format_constants(oracle_mod):
    d = oracle_mod.e4m3_to_f64
    assert d(np.array([0x7E]))[0] == 448.0            # largest finite
    assert d(np.array([0x08]))[0] == 2.0 ** -6         # smallest normal
    assert d(np.array([0x01]))[0] == 2.0 ** -9         # smallest subnormal
    assert d(np.array([0x38]))[0] == 1.0
    assert d(np.array([0xFE]))[0] == -448.0
    # positive finite codes increase strictly; the sign bit only flips the sign
    pos = d(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(d(np.arange(0x80, 0xFF)), -pos)


def test_e4m3_encode_round_trip_and_saturation(oracle_mod):
    d, e = oracle_mod.e4m3_to_f64, oracle_mod.f32_to_e4m3
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(e(d(finite).astype(np.float32)), finite)
    assert list(e(np.array([448 * 4.0, np.inf, -np.inf, -1e30], np.float32))) == [0x7E, 0x7E, 0xFE, 0xFE]
    assert e(np.array([np.nan], np.float32))[0] == 0x7F


def test_e4m3_encode_matches_torch_rounding(oracle_mod):
    rng = np.random.default_rng(7)
    # random values over the whole range, plus every midpoint between
    # neighbouring codes (the ties) and points just off them
    v = (rng.standard_normal(4000) * np.exp2(rng.uniform(-12, 8, 4000))).astype(np.float32)
    pos = oracle_mod.e4m3_to_f64(np.arange(0x7F))
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mid, -mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))])
    v = v[np.abs(v) <= 448.0]
    assert np.array_equal(oracle_mod.f32_to_e4m3(v), _torch_e4m3_encode(v))


# ---------------------------------------------------------------- FP8 LM head

def _head(V, H, seed):
    rng = np.random.default_rng(seed)
    return synth.bf16_bits(rng.standard_normal((V, H)) * 0.02)


def test_lmhead_quantize_matches_torch_and_its_bound(oracle_mod):
    w = _head(37, 256, 1)
    w[3] = 0  # an all-zero row
    q, s = oracle_mod.lmhead_quantize(w)
    wf = synth.bf16_bits_to_f32(w)
    amax = np.abs(wf).max(axis=1)
    assert s[3] == 1.0 and not q[3].any()
    nz = amax > 0
    assert np.array_equal(s[nz], (amax[nz] / np.float32(448.0)).astype(np.float32))
    ref = _torch_e4m3_encode((wf / s[:, None]).astype(np.float32))
    assert np.array_equal(q, ref)
    # the largest element of each row lands on +-448
    r = np.arange(37)[nz]
    top = np.abs(wf[nz]).argmax(axis=1)
    assert set(np.unique(q[r, top] & 0x7F)) == {0x7E}
    # dequantised error within half an E4M3 step (3 mantissa bits) of each value
    deq = _torch_e4m3_decode(q) * s[:, None].astype(np.float64)
    err = np.abs(deq - wf)
    step = np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(wf) / s[:, None], 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(err <= 0.5 * step * s[:, None] * (1 + 1e-6))


def test_lmhead_gemv_matches_numpy(oracle_mod):
    w = _head(53, 512, 2)
    q, s = oracle_mod.lmhead_quantize(w)
    x = synth.bf16_bits(np.random.default_rng(3).standard_normal((3, 512)))
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    got = oracle_mod.lmhead_gemv_fp8(q, s, x)
    ref = (_torch_e4m3_decode(q) * s[:, None].astype(np.float64)) @ xf.T
    np.testing.assert_allclose(got, ref.T, rtol=1e-12, atol=1e-12)
    gotb = oracle_mod.lmhead_gemv_bf16(w, x)
    refb = synth.bf16_bits_to_f32(w).astype(np.float64) @ xf.T
    np.testing.assert_allclose(gotb, refb.T, rtol=1e-12, atol=1e-12)


def test_lmhead_gemv_one_hot_reads_one_column(oracle_mod):
    w = _head(19, 256, 4)
    q, s = oracle_mod.lmhead_quantize(w)
    for h in (0, 1, 31, 32, 255):
        x = np.zeros((1, 256), np.uint16)
        x[0, h] = 0x3F80  # 1.0
        got = oracle_mod.lmhead_gemv_fp8(q, s, x)[0]
        assert np.array_equal(got, _torch_e4m3_decode(q[:, h]) * s.astype(np.float64))


# ---------------------------------------------------------------- MXFP4 / E8M0

def test_e2m1_and_e8m0_values(oracle_mod):
    got = oracle_mod.e2m1_to_f64(np.arange(16))
    assert list(got[:8]) == E2M1_MAGNITUDES
    assert list(-got[8:]) == E2M1_MAGNITUDES
    assert np.signbit(got[8])  # code 8 is -0
    e = oracle_mod.e8m0_to_f64(np.array([127, 126, 128, 0, 254]))
    assert list(e) == [1.0, 0.5, 2.0, 2.0 ** -127, 2.0 ** 127]
    assert np.isnan(oracle_mod.e8m0_to_f64(np.array([255]))[0])


def test_mxfp4_scale_groups_and_nibbles(oracle_mod):
    # every code 1.0 (E2M1 0b0010) with a distinct power-of-two scale per
    # group: the dequantised matrix is the scale map, expanded over 32 columns
    N, K = 3, 128
    codes = np.full((N, K), 2, np.uint8)
    sc = (120 + np.arange(N * K // 32) % 9).astype(np.uint8).reshape(N, K // 32)
    W = oracle_mod.dequant_fmt(oracle_mod.FMT_MXFP4, synth.pack_codes(codes), sc, N, K)
    assert np.array_equal(W, np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=1))
    # even k in the low nibble: codes 6.0 (0b0111) at even k, -0.5 (0b1001) at odd k
    codes = np.tile(np.array([7, 9], np.uint8), (N, K // 2))
    W = oracle_mod.dequant_fmt(oracle_mod.FMT_MXFP4, synth.pack_codes(codes), np.full((N, K // 32), 127, np.uint8), N, K)
    assert np.array_equal(W[:, 0::2], np.full((N, K // 2), 6.0)) and np.array_equal(W[:, 1::2], np.full((N, K // 2), -0.5))


def test_fp8_block_scale_blocks(oracle_mod):
    # every code 1.0 (0x38), a distinct scale per 128 x 128 block, ragged edges
    N, K = 300, 160
    nb, kb = 3, 2
    sc = np.exp2(np.arange(nb * kb, dtype=np.float64) - 3).astype(np.float32).reshape(nb, kb)
    W = oracle_mod.dequant_fmt(oracle_mod.FMT_FP8_BLOCK, np.full((N, K), 0x38, np.uint8), sc, N, K)
    ref = sc.astype(np.float64)[np.arange(N)[:, None] // 128, np.arange(K)[None, :] // 128]
    assert np.array_equal(W, ref)


# ---------------------------------------------------------------- forward in every format

SHAPE = synth.LayerShape(hidden=256, n_experts=6, top_k=2, inter=64, has_shared=True)


def _dense_as_shared(W13, W2):
    """bf16 bit patterns of dense matrices whose values are bf16-exact."""
    b13, b2 = synth.bf16_bits(W13), synth.bf16_bits(W2)
    assert np.array_equal(synth.bf16_bits_to_f32(b13), W13) and np.array_equal(synth.bf16_bits_to_f32(b2), W2)
    return b13, b2


def _one_expert_case(oracle_mod, fmt, q13, s13, q2, s2):
    """forward_fmt with one routed expert (weight 1) and no shared expert must
    equal the oracle's pinned BF16 expert on the same (bf16-exact) values."""
    H, I = SHAPE.hidden, SHAPE.inter
    W13 = oracle_mod.dequant_fmt(fmt, q13, s13, 2 * I, H)
    W2 = oracle_mod.dequant_fmt(fmt, q2, s2, H, I)
    b13, b2 = _dense_as_shared(W13, W2)
    x = synth.bf16_bits(np.random.default_rng(5).standard_normal((1, H)))
    shape = synth.LayerShape(hidden=H, n_experts=1, top_k=1, inter=I, has_shared=False)
    ex = dict(w13_q={0: q13}, w13_s={0: s13}, w2_q={0: q2}, w2_s={0: s2})
    got, bad = oracle_mod.forward_fmt(shape, fmt, ex, x, np.zeros((1, 1), np.int32), np.ones((1, 1)))
    assert bad == 0
    _, ref = oracle_mod.expert_dense(synth.LayerShape(hidden=H, n_experts=1, top_k=1, inter=I), b13, b2,
                                     synth.bf16_bits_to_f32(x[0]).astype(np.float64))
    np.testing.assert_allclose(got[0], ref, rtol=1e-12, atol=1e-15)


def test_forward_mxfp4_reduces_to_the_bf16_expert(oracle_mod):
    rng = np.random.default_rng(11)
    H, I = SHAPE.hidden, SHAPE.inter
    q13 = synth.pack_codes(rng.integers(0, 16, (2 * I, H)).astype(np.uint8))
    q2 = synth.pack_codes(rng.integers(0, 16, (H, I)).astype(np.uint8))
    s13 = rng.integers(118, 125, (2 * I, H // 32)).astype(np.uint8)
    s2 = rng.integers(118, 125, (H, I // 32)).astype(np.uint8)
    _one_expert_case(oracle_mod, oracle_mod.FMT_MXFP4, q13, s13, q2, s2)


def test_forward_fp8_block_reduces_to_the_bf16_expert(oracle_mod):
    rng = np.random.default_rng(12)
    H, I = SHAPE.hidden, SHAPE.inter
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    q13 = rng.choice(finite, (2 * I, H)).astype(np.uint8)
    q2 = rng.choice(finite, (H, I)).astype(np.uint8)
    s13 = np.exp2(rng.integers(-14, -8, (1, 2))).astype(np.float32)
    s2 = np.exp2(rng.integers(-14, -8, (2, 1))).astype(np.float32)
    _one_expert_case(oracle_mod, oracle_mod.FMT_FP8_BLOCK, q13, s13, q2, s2)


def test_forward_fmt_int4_is_the_pinned_forward(oracle_mod):
    layer = synth.make_layer(SHAPE, 13)
    x = synth.make_tokens(SHAPE, 14, 3)
    ids = np.array([[0, 5], [2, 2], [4, 1]], np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.5], [0.9, 0.1]])
    ref, _ = oracle_mod.forward(SHAPE, layer, x, ids, w)
    ex = dict(w13_q=layer.w13_q, w13_s=layer.w13_s, w2_q=layer.w2_q, w2_s=layer.w2_s,
              sh_w13=layer.sh_w13, sh_w2=layer.sh_w2)
    got, bad = oracle_mod.forward_fmt(SHAPE, oracle_mod.FMT_INT4_G32, ex, x, ids, w)
    assert bad == 0
    assert np.array_equal(got, ref)
