"""Pins for the CPU oracle against facts that do not come from the oracle itself.

The pages print no worked example of the layer, so the pins are: a hand-derived
fixture for the storage codes, exhaustive code round-trips, closed forms
(SiLU antisymmetry, softmax identities, RMSNorm of a constant), brute force by
numpy library routines (dense fp64 matmul over the generator's own integer
codes, stable argsort), and structural invariants (token independence, expert
relabelling, exact doubling).  Each would fail on a plausible oracle slip: a
swapped nibble, a wrong offset or scale index, a transposed operand, a gate/up
swap, a sign error in SiLU, a wrong tie-break or a missing shared term.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest

from w4a16_grouped_quantized_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nibble_codes.json")


def _f32(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _dense_expert(q13, s13, q2, s2, G=32):
    """Dense fp64 weights from the generator's integer codes (before packing)."""
    W13 = q13.astype(np.float64) * np.repeat(_f32(s13), G, axis=1)
    W2 = q2.astype(np.float64) * np.repeat(_f32(s2), G, axis=1)
    return W13, W2


def _swiglu_ref(W13, W2, x, I):
    g = W13[:I] @ x
    u = W13[I:] @ x
    h = g / (1.0 + np.exp(-g)) * u
    return W2 @ h


# ---------------------------------------------------------------- storage codes

def test_golden_codes_pin_packer_and_decoder(oracle_mod):
    gold = json.load(open(GOLDEN))
    for ent in gold["bytes"]:
        b = int(ent["byte"], 16)
        codes = np.array([[ent["q_even"] + 8, ent["q_odd"] + 8]], np.uint8)
        assert synth.pack_codes(codes)[0, 0] == b, ent
    for ent in gold["bf16"]:
        v = oracle_mod.bf16_to_f64(np.array([int(ent["bits"], 16)], np.uint16))[0]
        assert v == ent["value"] and math.copysign(1, v) == math.copysign(1, ent["value"])
        assert oracle_mod.f64_to_bf16(np.array([ent["value"]]))[0] == int(ent["bits"], 16)
    row = gold["dequant_row"]
    q = np.array([[int(b, 16) for b in row["bytes"]]], np.uint8)
    s = np.array([[int(v, 16) for v in row["scales"]]], np.uint16)
    W = oracle_mod.dequant(q, s, 32)
    assert W.shape == (1, 64)
    np.testing.assert_array_equal(W[0, :8], row["expected_first8_group0"])
    np.testing.assert_array_equal(W[0, 32:40], row["expected_first8_group1"])
    np.testing.assert_array_equal(W[0, 8:32], 0.0)


def test_dequant_exhaustive_all_code_pairs(oracle_mod):
    # Every (even, odd) code pair = every byte value, in every byte position of
    # a group, with a distinct scale per group.
    pairs = np.array([(a, b) for a in range(16) for b in range(16)], np.uint8)  # 256 pairs
    codes = pairs.reshape(1, 512)
    q = synth.pack_codes(codes)
    assert sorted(set(q.ravel().tolist())) == list(range(256))
    scales = synth.bf16_bits(np.linspace(0.5, 3.0, 16))[None, :]
    W = oracle_mod.dequant(q, scales, 32)
    expect = (codes.astype(np.float64) - 8.0) * np.repeat(_f32(scales), 32, axis=1)
    np.testing.assert_array_equal(W, expect)
    # the round trip of the packer itself is lossless
    np.testing.assert_array_equal(synth.unpack_codes_reference_free(q), codes)


def test_dequant_matches_generator_codes_ling_expert(oracle_mod):
    ex = synth.make_expert(synth.LING, seed=7, e=3, return_q=True)
    W = oracle_mod.dequant(ex["w2_q"], ex["w2_s"], 32)
    expect = ex["q2"].astype(np.float64) * np.repeat(_f32(ex["w2_s"]), 32, axis=1)
    np.testing.assert_array_equal(W, expect)
    assert ex["q13"].min() >= -7 and ex["q13"].max() <= 7


# ---------------------------------------------------------------- bf16 rounding

def test_f64_to_bf16_matches_independent_float32_path(oracle_mod):
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-39).astype(np.float32),  # subnormals
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e38, 0.0], np.float32)])
    # values exactly representable in float32 round the same whether or not
    # they pass through float32 first, so the generator's float32 path is a
    # valid independent reference for them.
    np.testing.assert_array_equal(oracle_mod.f64_to_bf16(v.astype(np.float64)), synth.bf16_bits(v))
    # exact ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert oracle_mod.f64_to_bf16(np.array([1.0 + 2 ** -8]))[0] == 0x3F80
    assert oracle_mod.f64_to_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 0x3F82
    assert oracle_mod.f64_to_bf16(np.array([1e39]))[0] == 0x7F80
    # double-only values: just above a tie must round up
    assert oracle_mod.f64_to_bf16(np.array([1.0 + 2 ** -8 + 2 ** -40]))[0] == 0x3F81


# ---------------------------------------------------------------- routing

@pytest.fixture(scope="module")
def tiny_layer():
    return synth.make_layer(synth.TINY, seed=0, return_q=True)


def test_route_against_numpy_bruteforce(oracle_mod, tiny_layer):
    shape = synth.TINY
    x = synth.make_tokens(shape, 11, 64)
    ids, w, gap, logits = oracle_mod.route(shape, tiny_layer.router_w, x)
    l_ref = _f32(x) @ tiny_layer.router_w.astype(np.float64).T
    np.testing.assert_allclose(logits, l_ref, rtol=0, atol=1e-13)
    for t in range(x.shape[0]):
        order = np.argsort(-l_ref[t], kind="stable")
        if gap[t] > 1e-9:
            assert set(ids[t].tolist()) == set(order[: shape.top_k].tolist())
            np.testing.assert_array_equal(ids[t], order[: shape.top_k])
        p = np.exp(l_ref[t] - l_ref[t].max())
        p /= p.sum()
        w_ref = p[ids[t]] / p[ids[t]].sum()  # full softmax renormalised over the chosen set
        np.testing.assert_allclose(w[t], w_ref, rtol=1e-12, atol=0)
        assert abs(w[t].sum() - 1.0) <= 1e-15 * shape.top_k
        assert np.all(np.diff(w[t]) <= 0)
        srt = np.sort(l_ref[t])[::-1]
        assert gap[t] == pytest.approx(srt[shape.top_k - 1] - srt[shape.top_k], abs=1e-12)


def test_route_k1_weight_is_one_and_ties_prefer_lower_id(oracle_mod, tiny_layer):
    shape = dataclasses.replace(synth.TINY, top_k=1)
    x = synth.make_tokens(shape, 3, 16)
    ids, w, _, _ = oracle_mod.route(shape, tiny_layer.router_w, x)
    assert np.all(w == 1.0)
    # identical router rows give bitwise-identical logits: the lower id must win
    rw = tiny_layer.router_w.copy()
    shape3 = dataclasses.replace(synth.TINY, top_k=3)
    ids0, _, _, l0 = oracle_mod.route(shape3, rw, x)
    for t in range(x.shape[0]):
        top = int(ids0[t, 0])
        dup = (top + 5) % shape.n_experts
        rw2 = rw.copy()
        rw2[dup] = rw[top]
        ids2, w2, gap2, l2 = oracle_mod.route(shape3, rw2, x[t:t + 1])
        lo, hi = min(top, dup), max(top, dup)
        assert l2[0, lo] == l2[0, hi]
        assert ids2[0, 0] == lo and ids2[0, 1] == hi
        assert w2[0, 0] == w2[0, 1]


# ---------------------------------------------------------------- experts + combine

def test_dense_equivalence_all_experts_selected(oracle_mod, tiny_layer):
    shape = dataclasses.replace(synth.TINY, top_k=synth.TINY.n_experts)  # k = E = 16
    L = tiny_layer
    x = synth.make_tokens(shape, 21, 8)
    ids, w, gap, _ = oracle_mod.route(shape, L.router_w, x)
    assert np.all(np.isinf(gap))
    out, bad = oracle_mod.forward(shape, L, x, ids, w)
    assert bad == 0
    I = shape.inter
    dense = [_dense_expert(L.q13[e], L.w13_s[e], L.q2[e], L.w2_s[e]) for e in range(shape.n_experts)]
    for t in range(x.shape[0]):
        xt = _f32(x[t])
        ref = np.zeros(shape.hidden)
        for j in range(shape.top_k):
            W13, W2 = dense[ids[t, j]]
            ref += w[t, j] * _swiglu_ref(W13, W2, xt, I)
        scale = np.abs(ref).max()
        assert np.abs(out[t] - ref).max() <= 1e-12 * scale


def test_ling_expert_matches_numpy_dense(oracle_mod):
    shape = synth.LING
    ex = synth.make_expert(shape, seed=1, e=77, return_q=True)
    x = _f32(synth.make_tokens(shape, 1, 1)[0])
    h, y = oracle_mod.expert_q(shape, ex["w13_q"], ex["w13_s"], ex["w2_q"], ex["w2_s"], x)
    W13, W2 = _dense_expert(ex["q13"], ex["w13_s"], ex["q2"], ex["w2_s"])
    ref = _swiglu_ref(W13, W2, x, shape.inter)
    assert np.abs(y - ref).max() <= 1e-11 * np.abs(ref).max()


def test_shared_only_layer_equals_dense_swiglu(oracle_mod):
    shape = dataclasses.replace(synth.TINY, has_shared=True)
    L = synth.make_layer(shape, seed=4)
    zeroed = dataclasses.replace(L, w13_s=np.zeros_like(L.w13_s), w2_s=np.zeros_like(L.w2_s))
    x = synth.make_tokens(shape, 4, 5)
    ids, w, _, _ = oracle_mod.route(shape, L.router_w, x)
    out, _ = oracle_mod.forward(shape, zeroed, x, ids, w)
    W13 = _f32(L.sh_w13)
    W2 = _f32(L.sh_w2)
    for t in range(x.shape[0]):
        ref = _swiglu_ref(W13, W2, _f32(x[t]), shape.inter)
        assert np.abs(out[t] - ref).max() <= 1e-12 * np.abs(ref).max()


def test_silu_sign_and_gate_up_order(oracle_mod):
    # One-hot x makes every gate/up sum a single exact term, so h is known in
    # closed form: silu(a) - silu(-a) = a for any a, and silu(0) = 0.
    shape = dataclasses.replace(synth.TINY, hidden=64, inter=32)
    H, I = shape.hidden, shape.inter
    k0 = 37
    codes13 = np.full((2 * I, H), 8, np.uint8)
    codes13[0, k0] = 8 + 3      # gate row 0: q = +3
    codes13[1, k0] = 8 - 3      # gate row 1: q = -3
    codes13[2, k0] = 8          # gate row 2: q = 0
    codes13[I:, k0] = 8 + 1     # every up row: q = +1
    s13 = np.full((2 * I, H // 32), 0x3F80, np.uint16)     # 1.0
    s13[I:, :] = 0x4000                                    # up scales 2.0
    codes2 = np.full((H, I), 8, np.uint8)
    s2 = np.full((H, I // 32), 0x3F80, np.uint16)
    x = np.zeros(H)
    x[k0] = 1.0
    h, y = oracle_mod.expert_q(shape, synth.pack_codes(codes13), s13, synth.pack_codes(codes2), s2, x)
    a, u = 3.0, 2.0
    assert h[0] - h[1] == pytest.approx(a * u, rel=1e-15)
    assert h[2] == 0.0
    assert h[0] == pytest.approx(a / (1 + math.exp(-a)) * u, rel=1e-15)
    assert np.all(y == 0.0)


def test_token_independence_and_exact_doubling(oracle_mod, tiny_layer):
    shape = synth.TINY
    L = tiny_layer
    x = synth.make_tokens(shape, 8, 4)
    ids, w, _, _ = oracle_mod.route(shape, L.router_w, x)
    out, _ = oracle_mod.forward(shape, L, x, ids, w)
    for t in range(4):
        one, _ = oracle_mod.forward(shape, L, x[t:t + 1], ids[t:t + 1], w[t:t + 1])
        np.testing.assert_array_equal(one[0], out[t])
    # doubling every down-projection scale (exact in bf16) doubles the routed output exactly
    L2 = dataclasses.replace(L, w2_s=synth.bf16_bits(_f32(L.w2_s) * 2.0))
    out2, _ = oracle_mod.forward(shape, L2, x, ids, w)
    np.testing.assert_array_equal(out2, 2.0 * out)


def test_expert_relabelling_invariance(oracle_mod, tiny_layer):
    shape = synth.TINY
    L = tiny_layer
    pi = np.random.default_rng(9).permutation(shape.n_experts)  # new id of old expert e is pi[e]
    inv = np.argsort(pi)
    P = dataclasses.replace(L, router_w=L.router_w[inv], w13_q=L.w13_q[inv], w13_s=L.w13_s[inv],
                            w2_q=L.w2_q[inv], w2_s=L.w2_s[inv])
    x = synth.make_tokens(shape, 12, 6)
    ids, w, _, _ = oracle_mod.route(shape, L.router_w, x)
    ids_p, w_p, _, _ = oracle_mod.route(shape, P.router_w, x)
    np.testing.assert_array_equal(np.sort(pi[ids], 1), np.sort(ids_p, 1))
    out, _ = oracle_mod.forward(shape, L, x, ids, w)
    out_p, _ = oracle_mod.forward(shape, P, x, ids_p, w_p)
    np.testing.assert_array_equal(out, out_p)


def test_invalid_ids_contribute_zero(oracle_mod, tiny_layer):
    shape = synth.TINY
    x = synth.make_tokens(shape, 2, 2)
    ids, w, _, _ = oracle_mod.route(shape, tiny_layer.router_w, x)
    ids_bad = ids.copy()
    ids_bad[1, 1] = shape.n_experts + 3
    out, bad = oracle_mod.forward(shape, tiny_layer, x, ids_bad, w)
    assert bad == 1
    # token 1 then equals its slot 0 alone, computed through a k=1 view
    k1 = dataclasses.replace(shape, top_k=1)
    only0, _ = oracle_mod.forward(k1, tiny_layer, x[1:], ids[1:, :1], w[1:, :1])
    np.testing.assert_array_equal(out[1], only0[0])


# ---------------------------------------------------------------- permutation

def test_permute_matches_stable_argsort(oracle_mod):
    rng = np.random.default_rng(3)
    E = 64
    ids = rng.integers(0, E, size=(300, 8)).astype(np.int32)
    ids[5, 2] = -1
    ids[7, 0] = E
    counts, offsets, perm, bad = oracle_mod.permute(ids, E)
    assert bad == 2
    flat = ids.ravel()
    valid = np.nonzero((flat >= 0) & (flat < E))[0]
    np.testing.assert_array_equal(counts, np.bincount(flat[valid], minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    order = valid[np.argsort(flat[valid], kind="stable")]
    np.testing.assert_array_equal(perm[: len(valid)], order)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_closed_forms(oracle_mod):
    H = 2560
    c = synth.bf16_bits(np.full((1, H), -0.75))
    out = oracle_mod.rmsnorm(c, 1e-6)
    assert np.all(out == 0xBF80)  # -1.0 exactly after bf16 rounding
    y = synth.bf16_bits(np.random.default_rng(1).standard_normal((4, H)) * 7.0)
    o = _f32(oracle_mod.rmsnorm(y, 1e-6))
    rms = np.sqrt((o ** 2).mean(axis=1))
    assert np.all(np.abs(rms - 1.0) < 2 ** -8)
    # zero input stays zero (eps keeps the denominator positive)
    z = oracle_mod.rmsnorm(np.zeros((1, H), np.uint16), 1e-6)
    assert np.all(z == 0)


def test_rmsnorm_worked_values(oracle_mod):
    # y = (3, 4): mean(y^2) = 12.5, so y / rms = (3, 4) * sqrt(2) / 5
    # = (0.848528..., 1.131370...), which round to bf16 0.84765625 (0x3F59)
    # and 1.1328125 (0x3F91); eps = 1e-6 moves neither.
    y = synth.bf16_bits(np.array([[3.0, 4.0]]))
    np.testing.assert_array_equal(oracle_mod.rmsnorm(y, 1e-6), [[0x3F59, 0x3F91]])
    # four equal entries: the result is 1 / sqrt(1 + 1e-6), i.e. 1.0 in bf16
    y4 = synth.bf16_bits(np.ones((1, 4)))
    np.testing.assert_array_equal(oracle_mod.rmsnorm(y4, 1e-6), [[0x3F80] * 4])


def test_parity_rounding_allowance_is_half_bf16_ulp(oracle_mod):
    # the output check allows the bf16 store of the result on top of the
    # tolerance; that allowance must be exactly the worst rounding error
    from parity import bf16_half_ulp
    rng = np.random.default_rng(12)
    v = rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))
    r = synth.bf16_bits_to_f32(oracle_mod.f64_to_bf16(v)).astype(np.float64)
    q = np.abs(r - v) / bf16_half_ulp(v)
    assert q.max() <= 1.0 and q.max() > 0.999
    # values on a binade edge: 1 has half-ulp 2^-8, just below 1 it is 2^-9
    assert bf16_half_ulp(np.array([1.0, 0.999, -3.0, 0.0])).tolist() == [2.0 ** -8, 2.0 ** -9, 2.0 ** -7, 0.0]
