"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle, on
seeded synthetic inputs (tiny layer, Ling-shape layer at decode M = 1 and at
verify M = 2, 4, ragged M), plus determinism, device error reporting, the
permutation, RMSNorm routing and graph replay."""
import dataclasses
import sys

import numpy as np
import pytest

from w4a16_grouped_quantized_amd import synth
from parity import (DeviceLayer, bf16_f64, bf16_half_ulp, check_ids, check_out, from_dev_bf16,
                    run_and_check, to_dev_bf16)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a16_grouped_quantized_amd import binding as B
    B.lib()  # fails loudly if the library is not built


@pytest.fixture(scope="module")
def tiny():
    return DeviceLayer(synth.make_layer(synth.TINY, 0), max_tokens=64)


@pytest.fixture(scope="module")
def ling_layer(ling_seed1):
    return ling_seed1


@pytest.fixture(scope="module")
def ling(ling_layer):
    return DeviceLayer(ling_layer, max_tokens=64)


@pytest.fixture(scope="module")
def ling_big(ling_layer):
    return DeviceLayer(ling_layer, max_tokens=4096)


# ------------------------------------------------------------------ tiny layer

@pytest.mark.parametrize("M", [1, 2, 8, 33])
def test_tiny_route_forward(tiny, oracle_mod, M):
    _say(f"tiny M={M}")
    x = synth.make_tokens(synth.TINY, 100 + M, M)
    run_and_check(tiny, oracle_mod, x, f"tiny M={M}")


@pytest.mark.parametrize("M", [1, 4])
def test_tiny_all_experts_selected(oracle_mod, M):
    shape = dataclasses.replace(synth.TINY, top_k=16)
    dl = DeviceLayer(synth.make_layer(shape, 5), max_tokens=8)
    x = synth.make_tokens(shape, 7, M)
    run_and_check(dl, oracle_mod, x, f"tiny k=E M={M}")


@pytest.mark.parametrize("M", [1, 3])
def test_tiny_with_shared_expert(oracle_mod, M):
    shape = dataclasses.replace(synth.TINY, has_shared=True)
    dl = DeviceLayer(synth.make_layer(shape, 6), max_tokens=8)
    x = synth.make_tokens(shape, 8, M)
    run_and_check(dl, oracle_mod, x, f"tiny+shared M={M}")


# ------------------------------------------------------------------ Ling shape

def test_ling_decode_m1(ling, oracle_mod):
    # the benchmarked launch configuration: one token per call
    x = synth.make_tokens(synth.LING, 11, 128)
    worst = 0.0
    for t in range(x.shape[0]):
        worst = max(worst, run_and_check(ling, oracle_mod, x[t:t + 1], f"ling M=1 token {t}"))
    _say(f"ling M=1: worst max|err|/rms over 128 tokens = {worst:.3e}")


@pytest.mark.parametrize("M", [2, 4])
def test_ling_verify(ling, oracle_mod, M):
    x = synth.make_tokens(synth.LING, 20 + M, 16 * M)
    worst = 0.0
    for s in range(16):
        worst = max(worst, run_and_check(ling, oracle_mod, x[s * M:(s + 1) * M], f"ling M={M} step {s}"))
    _say(f"ling M={M}: worst ratio {worst:.3e}")


@pytest.mark.parametrize("M", [3, 7, 13])
def test_ling_ragged_m(ling, oracle_mod, M):
    x = synth.make_tokens(synth.LING, 40 + M, M)
    run_and_check(ling, oracle_mod, x, f"ling M={M}")


def test_ling_determinism(ling):
    import torch
    x = to_dev_bf16(synth.make_tokens(synth.LING, 3, 4))
    ref_ids, ref_w = ling.route(x)
    ref = ling.forward(x, ref_ids, ref_w)
    for _ in range(100):
        ids, w = ling.route(x)
        out = ling.forward(x, ids, w)
        assert torch.equal(ids, ref_ids) and torch.equal(w, ref_w)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_ling_caller_ids_duplicates_and_invalid(ling, oracle_mod):
    import torch
    shape = synth.LING
    x = synth.make_tokens(shape, 9, 3)
    ids = np.array([[5, 5, 17, 300, 300, 300, 2, 511],
                    [511, 0, 1, 2, 3, 4, 5, 6],
                    [17, 17, 17, 17, 17, 17, 17, 17]], np.int32)
    w = np.random.default_rng(0).random((3, 8)).astype(np.float32)
    out = ling.forward(to_dev_bf16(x), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    assert ling.device_error() == 0
    ref, bad = oracle_mod.forward(shape, ling.layer, x, ids, w.astype(np.float64))
    assert bad == 0
    check_out(from_dev_bf16(out), ref, "caller ids with duplicates")
    ids_bad = ids.copy()
    ids_bad[1, 3] = 512
    ids_bad[2, 0] = -1
    out = ling.forward(to_dev_bf16(x), torch.from_numpy(ids_bad).cuda(), torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    assert ling.device_error() == 1
    assert ling.device_error() == 0  # cleared by the read
    ref, bad = oracle_mod.forward(shape, ling.layer, x, ids_bad, w.astype(np.float64))
    assert bad == 2
    check_out(from_dev_bf16(out), ref, "invalid ids contribute zero")


def test_permute_bit_exact(oracle_mod):
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    cfg = B.config(shape)
    ws = B.Workspace(cfg, 4096)
    rng = np.random.default_rng(1)
    for M in (1, 4, 257, 300, 4096):
        ids = rng.integers(0, shape.n_experts, size=(M, shape.top_k)).astype(np.int32)
        if M > 4:
            ids[3, 1] = -7
            ids[M - 1, 7] = 4096
        d_ids = torch.from_numpy(ids).cuda()
        counts = torch.empty(shape.n_experts, dtype=torch.int32, device="cuda")
        offsets = torch.empty(shape.n_experts + 1, dtype=torch.int32, device="cuda")
        perm = torch.empty(M * shape.top_k, dtype=torch.int32, device="cuda")
        B.permute(cfg, d_ids, counts, offsets, perm, ws.buf)
        torch.cuda.synchronize()
        c, o, p, bad = oracle_mod.permute(ids, shape.n_experts)
        np.testing.assert_array_equal(counts.cpu().numpy(), c)
        np.testing.assert_array_equal(offsets.cpu().numpy(), o)
        np.testing.assert_array_equal(perm.cpu().numpy(), p)
        assert B.get_device_error(ws.buf) == (1 if bad else 0)


def test_route_with_rmsnorm(ling, oracle_mod):
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    y = synth.bf16_bits(np.random.default_rng(4).standard_normal((4, shape.hidden)) * 9.0)
    y_dev = to_dev_bf16(y)
    x_norm = torch.empty_like(y_dev)
    ids, w = ling.route(y_dev, flags=B.MOE_F_INPUT_RMSNORM, x_norm=x_norm)
    torch.cuda.synchronize()
    xn = from_dev_bf16(x_norm)
    ref = oracle_mod.rmsnorm(y, 1e-6)
    diff = np.abs(xn.astype(np.int32) - ref.astype(np.int32))
    assert diff.max() <= 1, "RMSNorm differs by more than one bf16 step"
    assert (diff == 0).mean() >= 0.999
    # routing is checked on the GPU's normalised input (teacher forcing)
    ids_o, _, gap, logits_o = oracle_mod.route(shape, ling.layer.router_w, xn)
    check_ids(shape, ids.cpu().numpy(), w.cpu().numpy(), ids_o, gap, logits_o)


def test_graph_replay_matches_eager(ling):
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    xs = synth.make_tokens(shape, 77, 6)
    static_x = to_dev_bf16(xs[:1])
    ids = torch.empty((1, shape.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, shape.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((1, shape.hidden), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the stream outside capture
        B.route(ling.cfg, ling.dev.router_w, static_x, ids, w, ling.ws.buf)
        B.forward(ling.cfg, ling.dev.packed, static_x, ids, w, out, ling.ws.buf)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.route(ling.cfg, ling.dev.router_w, static_x, ids, w, ling.ws.buf)
        B.forward(ling.cfg, ling.dev.packed, static_x, ids, w, out, ling.ws.buf)
    for t in range(xs.shape[0]):
        static_x.copy_(to_dev_bf16(xs[t:t + 1]))
        g.replay()
        torch.cuda.synchronize()
        got_ids, got_w, got = ids.clone(), w.clone(), out.clone()
        x_e = to_dev_bf16(xs[t:t + 1])
        e_ids, e_w = ling.route(x_e)
        e_out = ling.forward(x_e, e_ids, e_w)
        torch.cuda.synchronize()
        assert torch.equal(got_ids, e_ids) and torch.equal(got_w, e_w)
        assert torch.equal(got.view(torch.int16), e_out.view(torch.int16)), f"replay {t}"


def test_m0_is_noop(ling):
    import torch
    x = torch.empty((0, synth.LING.hidden), dtype=torch.bfloat16, device="cuda")
    ids, w = ling.route(x)
    out = ling.forward(x, ids, w)
    torch.cuda.synchronize()
    assert out.shape == (0, synth.LING.hidden)


# ------------------------------------------------------------------ many tokens (prefill)

@pytest.mark.parametrize("M", [40, 100, 600])
def test_ling_many_tokens_full_check(ling_big, oracle_mod, M):
    # 40: router as MFMA GEMM, experts on the small-M kernels; 100 and 600:
    # both on the matrix cores (grouped GEMMs with ragged 64-row tiles)
    _say(f"ling M={M}")
    x = synth.make_tokens(synth.LING, 300 + M, M)
    ratio = run_and_check(ling_big, oracle_mod, x, f"ling M={M}")
    _say(f"ling M={M}: max|err|/rms = {ratio:.3e}")


def test_ling_prefill_chunk_4096_sampled(ling_big, oracle_mod):
    import torch
    shape = synth.LING
    M = 4096
    x = synth.make_tokens(shape, 3, M)
    x_dev = to_dev_bf16(x)
    ids, w = ling_big.route(x_dev)
    out = ling_big.forward(x_dev, ids, w)
    out2 = ling_big.forward(x_dev, ids, w)
    torch.cuda.synchronize()
    assert ling_big.device_error() == 0
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "prefill forward not deterministic"
    ids_g, w_g, out_g = ids.cpu().numpy(), w.cpu().numpy(), from_dev_bf16(out)
    rng = np.random.default_rng(4096)
    rows = np.sort(rng.choice(M, size=48, replace=False))
    ids_o, _, gap, logits_o = oracle_mod.route(shape, ling_big.layer.router_w, x[rows])
    w_ref = check_ids(shape, ids_g[rows], w_g[rows], ids_o, gap, logits_o)
    out_ref, bad = oracle_mod.forward(shape, ling_big.layer, x[rows], ids_g[rows], w_ref)
    assert bad == 0
    ratio = check_out(out_g[rows], out_ref, "prefill 4096 sampled rows")
    # every row: finite, and the routing of all 4096 rows is a valid top-k
    assert np.all(np.isfinite(bf16_f64(out_g)))
    assert np.all((ids_g >= 0) & (ids_g < shape.n_experts))
    assert np.all(np.abs(w_g.sum(1) - 1) < 1e-5)
    _say(f"prefill 4096: sampled 48 rows, max|err|/rms = {ratio:.3e}")


# ------------------------------------------------------------------ stacked layers

@pytest.mark.parametrize("M", [1, 3])
def test_stack_three_layers_rmsnorm_teacher_forced(ling, ling_seed23, oracle_mod, M):
    """Three independent Ling-shape layers, each fed the previous layer's
    output through the fused unit-gain RMSNorm (eps 1e-6) of the routing
    call.  Every layer is checked against the oracle on the GPU's own
    normalised input: x_norm within one bf16 step of the oracle's RMSNorm of
    the GPU output before it, routing within the gap band, output within
    tolerance."""
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    stack = [ling] + [DeviceLayer(layer, max_tokens=64) for layer in ling_seed23]
    x = synth.make_tokens(shape, 60 + M, M)
    y_dev = to_dev_bf16(x)
    for li, dl in enumerate(stack):
        if li == 0:
            xin_dev = y_dev
            ids, w = dl.route(xin_dev)
        else:
            xin_dev = torch.empty_like(y_dev)
            ids, w = dl.route(y_dev, flags=B.MOE_F_INPUT_RMSNORM, x_norm=xin_dev)
        out = dl.forward(xin_dev, ids, w)
        torch.cuda.synchronize()
        xin = from_dev_bf16(xin_dev)
        if li > 0:
            ref_norm = oracle_mod.rmsnorm(from_dev_bf16(y_dev), 1e-6)
            diff = np.abs(xin.astype(np.int32) - ref_norm.astype(np.int32))
            assert diff.max() <= 1, f"layer {li}: RMSNorm differs by more than one bf16 step"
        ids_o, _, gap, logits_o = oracle_mod.route(shape, dl.layer.router_w, xin)
        w_ref = check_ids(shape, ids.cpu().numpy(), w.cpu().numpy(), ids_o, gap, logits_o)
        ref, bad = oracle_mod.forward(shape, dl.layer, xin, ids.cpu().numpy(), w_ref)
        assert bad == 0
        ratio = check_out(from_dev_bf16(out), ref, f"stack layer {li} M={M}")
        _say(f"stack layer {li} M={M}: max|err|/rms {ratio:.3e}")
        y_dev = out


def test_ling_many_tokens_caller_ids(ling_big, oracle_mod):
    """The grouped-GEMM path with caller ids: duplicates inside a token, ids
    out of range (error word, zero contribution), one expert taking every
    token (more rows than one work item) and experts with no token at all."""
    import torch
    shape = synth.LING
    M = 200
    x = synth.make_tokens(shape, 91, M)
    rng = np.random.default_rng(91)
    ids = rng.integers(0, 64, size=(M, shape.top_k)).astype(np.int32)   # experts 64.. get no token
    ids[:, 0] = 7                      # expert 7 in every token: 200+ rows, three work items
    ids[5, 1] = ids[5, 2] = 9          # duplicate inside one token
    w = rng.random((M, shape.top_k)).astype(np.float32)
    out = ling_big.forward(to_dev_bf16(x), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    assert ling_big.device_error() == 0
    ref, bad = oracle_mod.forward(shape, ling_big.layer, x, ids, w.astype(np.float64))
    assert bad == 0
    check_out(from_dev_bf16(out), ref, "many tokens, caller ids")
    ids_bad = ids.copy()
    ids_bad[3, 4] = 512
    ids_bad[150, 0] = -2
    out = ling_big.forward(to_dev_bf16(x), torch.from_numpy(ids_bad).cuda(), torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    assert ling_big.device_error() == 1
    ref, bad = oracle_mod.forward(shape, ling_big.layer, x, ids_bad, w.astype(np.float64))
    assert bad == 2
    check_out(from_dev_bf16(out), ref, "many tokens, invalid ids contribute zero")


# ------------------------------------------------------------------ one-hot tokens

def _onehot_tokens(shape, positions):
    x = np.zeros((len(positions), shape.hidden), np.uint16)
    for t, k in enumerate(positions):
        x[t, k] = 0x3F80  # bf16 1.0
    return x


def _check_tight(out_bits, ref, tol, what):
    """|gpu - oracle| - half a bf16 ulp <= tol * rms: with a one-hot token every
    gate and up row of an expert sums exactly one dequantised weight, so a
    wrong nibble, nibble order, scale or row lands as an O(1) error."""
    got = bf16_f64(out_bits)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    excess = float(np.max(np.abs(got - ref) - bf16_half_ulp(ref)))
    assert excess <= tol * rms, f"{what}: excess {excess / rms:.3e} * rms > {tol}"
    _say(f"{what}: max(|err| - half bf16 ulp)/rms = {excess / rms:.3e} (bound {tol})")


# inputs at both nibble positions of a byte, at group and tile edges, first and last
ONEHOT_POS = [0, 1, 7, 8, 31, 32, 33, 255, 1279, 1280, 2527, 2559]


def test_onehot_tokens_every_path(ling_big, oracle_mod):
    """One-hot tokens through each kernel path with caller ids, against the
    oracle at bounds derived from each path's own rounding: the decode and
    verify kernels keep h to about 16 bits (a bf16 hi + lo pair) and sum in
    fp32 (bound 1e-4 * rms); the grouped-GEMM path rounds h to fp16, 2^-12
    relative per element (bound 4e-3 * rms)."""
    import torch
    shape = synth.LING
    xs = _onehot_tokens(shape, ONEHOT_POS)
    n = len(ONEHOT_POS)
    rng = np.random.default_rng(77)
    # decode (M = 1) and a verify-sized call (M = n): separate kernels
    ids = np.stack([rng.choice(shape.n_experts, shape.top_k, replace=False) for _ in range(n)]).astype(np.int32)
    w = rng.random((n, shape.top_k)).astype(np.float32)
    ref, bad = oracle_mod.forward(shape, ling_big.layer, xs, ids, w.astype(np.float64))
    assert bad == 0
    for t in (0, 1, n - 1):
        out = ling_big.forward(to_dev_bf16(xs[t:t + 1]), torch.from_numpy(ids[t:t + 1]).cuda(),
                               torch.from_numpy(w[t:t + 1]).cuda())
        torch.cuda.synchronize()
        _check_tight(from_dev_bf16(out), ref[t:t + 1], 1e-4, f"one-hot decode, input {ONEHOT_POS[t]}")
    out = ling_big.forward(to_dev_bf16(xs), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    _check_tight(from_dev_bf16(out), ref, 1e-4, f"one-hot verify-sized call, M={n}")
    # grouped GEMMs: the same tokens repeated to M = 8n (M k >= 513), new ids per row
    reps = 8
    xb = np.tile(xs, (reps, 1))
    idb = np.stack([rng.choice(shape.n_experts, shape.top_k, replace=False) for _ in range(n * reps)]).astype(np.int32)
    wb = rng.random((n * reps, shape.top_k)).astype(np.float32)
    refb, bad = oracle_mod.forward(shape, ling_big.layer, xb, idb, wb.astype(np.float64))
    assert bad == 0
    out = ling_big.forward(to_dev_bf16(xb), torch.from_numpy(idb).cuda(), torch.from_numpy(wb).cuda())
    torch.cuda.synchronize()
    assert ling_big.device_error() == 0
    _check_tight(from_dev_bf16(out), refb, 4e-3, f"one-hot grouped GEMMs, M={n * reps}")


def test_onehot_token_one_launch_layer(ling_big, oracle_mod):
    """The one-launch layer (routing inside) on one-hot tokens: ids checked as
    in every parity test, the output at the fp16-h bound (4e-3 * rms)."""
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    for k in (0, 33, 2559):
        x = _onehot_tokens(shape, [k])
        ids = torch.empty((1, shape.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((1, shape.top_k), dtype=torch.float32, device="cuda")
        out = torch.empty((1, shape.hidden), dtype=torch.bfloat16, device="cuda")
        B.layer(ling_big.cfg, ling_big.dev.router_w, ling_big.dev.packed, to_dev_bf16(x), ids, w, out,
                ling_big.ws.buf)
        torch.cuda.synchronize()
        assert ling_big.device_error() == 0
        ids_g, w_g = ids.cpu().numpy(), w.cpu().numpy()
        ids_o, _, gap, logits_o = oracle_mod.route(shape, ling_big.layer.router_w, x)
        w_ref = check_ids(shape, ids_g, w_g, ids_o, gap, logits_o)
        ref, bad = oracle_mod.forward(shape, ling_big.layer, x, ids_g, w_ref)
        assert bad == 0
        _check_tight(from_dev_bf16(out), ref, 4e-3, f"one-hot one-launch layer, input {k}")


def _outlier_tokens(shape, seed, M):
    """N(0,1) tokens with a few channels 100-300 times larger, as in the
    hidden states of trained transformers (a handful of massive channels)."""
    x = synth.make_tokens(shape, seed, M)
    rng = np.random.default_rng(seed)
    xf = synth.bf16_bits_to_f32(x).astype(np.float32)
    chans = rng.choice(shape.hidden, 4, replace=False)
    xf[:, chans] = rng.choice([-1.0, 1.0], (M, 4)) * rng.uniform(100.0, 300.0, (M, 4))
    return synth.bf16_bits(xf)


@pytest.mark.parametrize("M", [1, 4, 80])
def test_outlier_channel_tokens(ling_big, oracle_mod, M):
    """Tokens with massive channels through routing and every expert path
    (M = 1 and 4: small-M kernels; M = 80: router GEMM and grouped GEMMs),
    at the parity bound."""
    x = _outlier_tokens(synth.LING, 500 + M, M)
    ratio = run_and_check(ling_big, oracle_mod, x, f"outlier channels M={M}")
    _say(f"outlier channels M={M}: max|err|/rms = {ratio:.3e}")


def test_outlier_channel_token_one_launch_layer(ling_big, oracle_mod):
    """The one-launch layer (routing inside) on tokens with massive channels."""
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    for seed in (601, 602, 603):
        x = _outlier_tokens(shape, seed, 1)
        ids = torch.empty((1, shape.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((1, shape.top_k), dtype=torch.float32, device="cuda")
        out = torch.empty((1, shape.hidden), dtype=torch.bfloat16, device="cuda")
        B.layer(ling_big.cfg, ling_big.dev.router_w, ling_big.dev.packed, to_dev_bf16(x), ids, w, out,
                ling_big.ws.buf)
        torch.cuda.synchronize()
        assert ling_big.device_error() == 0
        ids_g, w_g = ids.cpu().numpy(), w.cpu().numpy()
        ids_o, _, gap, logits_o = oracle_mod.route(shape, ling_big.layer.router_w, x)
        w_ref = check_ids(shape, ids_g, w_g, ids_o, gap, logits_o)
        ref, bad = oracle_mod.forward(shape, ling_big.layer, x, ids_g, w_ref)
        assert bad == 0
        ratio = check_out(from_dev_bf16(out), ref, f"outlier channels, one-launch layer, seed {seed}")
        _say(f"outlier channels one-launch layer seed {seed}: max|err|/rms = {ratio:.3e}, "
             f"beyond the bf16 store {check_out.last_excess:.3e}")


@pytest.mark.parametrize("M", [4, 80, 4096])
def test_graph_replay_matches_eager_many_tokens(ling_big, M):
    """route + forward captured once at M tokens (M = 4: small-M kernels;
    80 and 4096: router GEMM, permutation, grouped GEMMs, combine) and
    replayed on three inputs, eager calls in between; every replay equals the
    eager result bit for bit."""
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    dl = ling_big
    xs = [synth.make_tokens(shape, 880 + M + r, M) for r in range(3)]
    static_x = to_dev_bf16(xs[0])
    ids = torch.empty((M, shape.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((M, shape.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((M, shape.hidden), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.route(dl.cfg, dl.dev.router_w, static_x, ids, w, dl.ws.buf)
        B.forward(dl.cfg, dl.dev.packed, static_x, ids, w, out, dl.ws.buf)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.route(dl.cfg, dl.dev.router_w, static_x, ids, w, dl.ws.buf)
        B.forward(dl.cfg, dl.dev.packed, static_x, ids, w, out, dl.ws.buf)
    for r, x in enumerate(xs):
        static_x.copy_(to_dev_bf16(x))
        g.replay()
        torch.cuda.synchronize()
        got_ids, got_w, got = ids.clone(), w.clone(), out.clone()
        x_e = to_dev_bf16(x)
        e_ids, e_w = dl.route(x_e)
        e_out = dl.forward(x_e, e_ids, e_w)
        torch.cuda.synchronize()
        assert dl.device_error() == 0
        assert torch.equal(got_ids, e_ids) and torch.equal(got_w, e_w), f"M={M} replay {r}: routing"
        assert torch.equal(got.view(torch.int16), e_out.view(torch.int16)), f"M={M} replay {r}: output"
    _say(f"graph replay at M={M}: 3 replays bit-identical to eager")
