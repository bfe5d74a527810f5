"""GPU parity of moe_layer_w4a16, the whole layer in one call: the one-launch
kernel (router, top-k, shared and routed experts and the output as workgroup
roles of one grid; used for M = 1, and for larger M with MOE_F_ONE_LAUNCH)
against the fp64 oracle, and its routing against moe_route bit for bit."""
import dataclasses
import sys

import numpy as np
import pytest

from w4a16_grouped_quantized_amd import synth
from parity import DeviceLayer, check_ids, check_out, from_dev_bf16, to_dev_bf16

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
    B.lib()


@pytest.fixture(scope="module")
def ling(ling_seed1):
    return DeviceLayer(ling_seed1, max_tokens=16)


def _layer(dl, x_dev, flags=None, x_norm=None):
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    M = x_dev.shape[0]
    if flags is None:  # the one-launch kernel at every M it supports
        flags = B.MOE_F_ONE_LAUNCH
    ids = torch.full((M, dl.shape.top_k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((M, dl.shape.top_k), -1.0, dtype=torch.float32, device="cuda")
    out = torch.empty((M, dl.shape.hidden), dtype=torch.bfloat16, device="cuda")
    B.layer(dl.cfg, dl.dev.router_w, dl.dev.packed, x_dev, ids, w, out, dl.ws.buf, flags=flags, x_norm=x_norm)
    return ids, w, out


def _check_layer(dl, oracle, x_bits, what, flags=None):
    import torch
    x_dev = to_dev_bf16(x_bits)
    ids, w, out = _layer(dl, x_dev, flags=flags)
    torch.cuda.synchronize()
    assert dl.device_error() == 0, what
    ids_g, w_g = ids.cpu().numpy(), w.cpu().numpy()
    ids_o, _, gap, logits_o = oracle.route(dl.shape, dl.layer.router_w, x_bits)
    w_ref = check_ids(dl.shape, ids_g, w_g, ids_o, gap, logits_o)
    out_ref, bad = oracle.forward(dl.shape, dl.layer, x_bits, ids_g, w_ref)
    assert bad == 0
    ratio = check_out(from_dev_bf16(out), out_ref, what)
    _say(f"{what}: max|err|/rms {ratio:.3e}, beyond the bf16 store {check_out.last_excess:.3e}")
    return ratio


@pytest.mark.parametrize("M", [1, 2, 4, 8, 9])
def test_layer_ling_matches_oracle(ling, oracle_mod, M):
    # M <= 4: one launch; M = 8, 9: the two-call path
    steps = 24 if M == 1 else 4
    x = synth.make_tokens(synth.LING, 500 + M, steps * M)
    worst = max(_check_layer(ling, oracle_mod, x[s * M:(s + 1) * M], f"layer ling M={M} step {s}") for s in range(steps))
    _say(f"layer ling M={M}: worst ratio {worst:.3e}")


@pytest.mark.parametrize("M", [2, 3, 4])
def test_layer_default_dispatch_matches_oracle(ling, oracle_mod, M):
    """moe_layer_w4a16 with no flags, as a speculative-verify step calls it:
    the library picks the kernels for M tokens itself.  Eight steps of
    seeded Ling tokens, each against the oracle, and the routing equal to
    moe_route's bit for bit."""
    import torch
    x = synth.make_tokens(synth.LING, 700 + M, 8 * M)
    for s in range(8):
        xs = x[s * M:(s + 1) * M]
        _check_layer(ling, oracle_mod, xs, f"default dispatch M={M} step {s}", flags=0)
        x_dev = to_dev_bf16(xs)
        ids, w, _ = _layer(ling, x_dev, flags=0)
        r_ids, r_w = ling.route(x_dev)
        torch.cuda.synchronize()
        assert torch.equal(ids, r_ids) and torch.equal(w, r_w)


def test_layer_after_larger_calls(ling, oracle_mod):
    """Calls of different M share one workspace: the per-call arrays of a
    large call overlap where a small call's arrays live, so the one-launch
    path must keep its flags and counters in the fixed header.  A 9-token
    call (two-call path, fills the arrays with data) and a 4-token one-launch
    call, then single tokens, each checked against the oracle."""
    for M in (9, 4, 1, 9, 1):
        x = synth.make_tokens(synth.LING, 900 + M, M)
        _check_layer(ling, oracle_mod, x, f"layer after larger calls, M={M}")


@pytest.mark.parametrize("M", [1, 3, 8])
def test_layer_equals_route_then_forward(ling, oracle_mod, M):
    """The routing inside the launch is moe_route's bit for bit; both
    outputs (one launch, and the separate calls) meet the oracle."""
    import torch
    x = synth.make_tokens(synth.LING, 600 + M, M)
    x_dev = to_dev_bf16(x)
    ids, w, out = _layer(ling, x_dev)
    r_ids, r_w = ling.route(x_dev)
    r_out = ling.forward(x_dev, r_ids, r_w)
    torch.cuda.synchronize()
    assert ling.device_error() == 0
    assert torch.equal(ids, r_ids) and torch.equal(w, r_w)
    ref, bad = oracle_mod.forward(synth.LING, ling.layer, x, ids.cpu().numpy(), w.cpu().numpy().astype(np.float64))
    assert bad == 0
    check_out(from_dev_bf16(out), ref, f"one launch M={M}")
    check_out(from_dev_bf16(r_out), ref, f"route + forward M={M}")


def test_stages_match_oracle(ling, oracle_mod):
    """moe_gate_up_w4a16 + moe_down_w4a16 (two launches, h kept as a bf16
    pair) and moe_forward_w4a16 (one launch at small M, h of each tile in
    scaled fp16) both against the oracle on the same ids and weights."""
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    for M in (1, 4):
        x = synth.make_tokens(synth.LING, 650 + M, M)
        x_dev = to_dev_bf16(x)
        ids, w = ling.route(x_dev)
        out = ling.forward(x_dev, ids, w)
        out2 = torch.empty_like(out)
        B.gate_up(ling.cfg, ling.dev.packed, x_dev, ids, ling.ws.buf)
        B.down(ling.cfg, ling.dev.packed, ids, w, out2, ling.ws.buf)
        torch.cuda.synchronize()
        assert ling.device_error() == 0
        ref, bad = oracle_mod.forward(synth.LING, ling.layer, x, ids.cpu().numpy(), w.cpu().numpy().astype(np.float64))
        assert bad == 0
        check_out(from_dev_bf16(out), ref, f"forward M={M}")
        check_out(from_dev_bf16(out2), ref, f"stages M={M}")


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("M", [1, 4, 32])
def test_layer_tiny(oracle_mod, shared, M):
    shape = dataclasses.replace(synth.TINY, has_shared=shared)
    dl = DeviceLayer(synth.make_layer(shape, 20 + int(shared)), max_tokens=32)
    x = synth.make_tokens(shape, 700 + M, M)
    _check_layer(dl, oracle_mod, x, f"layer tiny shared={shared} M={M}")


@pytest.mark.parametrize("M", [1, 4])
def test_layer_rmsnorm(ling, oracle_mod, M):
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    y = synth.bf16_bits(np.random.default_rng(40 + M).standard_normal((M, shape.hidden)) * 7.0)
    y_dev = to_dev_bf16(y)
    xn = torch.empty_like(y_dev)
    ids, w, out = _layer(ling, y_dev, flags=B.MOE_F_INPUT_RMSNORM | B.MOE_F_ONE_LAUNCH, x_norm=xn)
    xn2 = torch.empty_like(y_dev)
    r_ids, r_w = ling.route(y_dev, flags=B.MOE_F_INPUT_RMSNORM, x_norm=xn2)
    torch.cuda.synchronize()
    err = ling.device_error()
    assert err == 0, f"device error word {err}"
    assert torch.equal(xn.view(torch.int16), xn2.view(torch.int16))
    assert torch.equal(ids, r_ids) and torch.equal(w, r_w)
    xin = from_dev_bf16(xn)
    ref_norm = oracle_mod.rmsnorm(y, 1e-6)
    assert np.abs(xin.astype(np.int32) - ref_norm.astype(np.int32)).max() <= 1
    ids_o, _, gap, logits_o = oracle_mod.route(shape, ling.layer.router_w, xin)
    w_ref = check_ids(shape, ids.cpu().numpy(), w.cpu().numpy(), ids_o, gap, logits_o)
    ref, bad = oracle_mod.forward(shape, ling.layer, xin, ids.cpu().numpy(), w_ref)
    assert bad == 0
    check_out(from_dev_bf16(out), ref, f"layer rmsnorm M={M}")


def test_layer_graph_replay(ling, oracle_mod):
    """The one-launch layer captured in a graph: every replay (with eager
    work and synchronisations in between) gives the eager bits, and meets
    the oracle."""
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    xs = synth.make_tokens(shape, 808, 8)
    static_x = to_dev_bf16(xs[:1])
    ids = torch.empty((1, shape.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, shape.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((1, shape.hidden), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.layer(ling.cfg, ling.dev.router_w, ling.dev.packed, static_x, ids, w, out, ling.ws.buf)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.layer(ling.cfg, ling.dev.router_w, ling.dev.packed, static_x, ids, w, out, ling.ws.buf)
    for t in range(xs.shape[0]):
        static_x.copy_(to_dev_bf16(xs[t:t + 1]))
        g.replay()
        torch.cuda.synchronize()
        got_ids, got_w, got = ids.clone(), w.clone(), out.clone()
        e_ids, e_w, e_out = _layer(ling, to_dev_bf16(xs[t:t + 1]))
        torch.cuda.synchronize()
        assert torch.equal(got_ids, e_ids) and torch.equal(got_w, e_w), f"replay {t}"
        assert torch.equal(got.view(torch.int16), e_out.view(torch.int16)), f"replay {t}"
        x1 = xs[t:t + 1]
        ids_o, _, gap, logits_o = oracle_mod.route(shape, ling.layer.router_w, x1)
        w_ref = check_ids(shape, got_ids.cpu().numpy(), got_w.cpu().numpy(), ids_o, gap, logits_o)
        ref, bad = oracle_mod.forward(shape, ling.layer, x1, got_ids.cpu().numpy(), w_ref)
        assert bad == 0
        check_out(from_dev_bf16(got), ref, f"graph replay {t}")
    assert ling.device_error() == 0


def test_layer_m0_is_noop(ling):
    import torch
    x = torch.empty((0, synth.LING.hidden), dtype=torch.bfloat16, device="cuda")
    ids, w, out = _layer(ling, x)
    torch.cuda.synchronize()
    assert out.shape == (0, synth.LING.hidden)
