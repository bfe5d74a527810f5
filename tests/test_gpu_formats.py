"""GPU parity of moe_forward_fmt (routed experts in MXFP4 or block FP8, the
shared expert in BF16) against the fp64 oracle's forward in the same format:
tiny layers with and without a shared expert over M = 1..8 (caller ids with
a repeated expert, an out-of-range id), one-hot tokens at
scale-group, chunk and block edges, and the Ling shape routed by moe_route
(decode M = 1 and verify M = 4)."""
import dataclasses
import sys

import numpy as np
import pytest

from w4a16_grouped_quantized_amd import synth
from parity import check_ids, check_out, from_dev_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu

FMTS = [(synth.FMT_MXFP4, "mxfp4"), (synth.FMT_FP8_BLOCK, "fp8_block")]


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


def _experts_dict(layer):
    return dict(w13_q=layer.w13_q, w13_s=layer.w13_s, w2_q=layer.w2_q, w2_s=layer.w2_s,
                sh_w13=layer.sh_w13, sh_w2=layer.sh_w2)


def _run(dl, ws, x_bits, ids, w):
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    M = x_bits.shape[0]
    x = to_dev_bf16(x_bits)
    out = torch.empty((M, dl.shape.hidden), dtype=torch.bfloat16, device="cuda")
    B.forward_fmt(dl, x, torch.from_numpy(ids).cuda(), torch.from_numpy(w.astype(np.float32)).cuda(), out, ws.buf)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("fmt,name", FMTS, ids=[f[1] for f in FMTS])
@pytest.mark.parametrize("shared", [False, True])
def test_tiny_against_oracle(oracle_mod, fmt, name, shared):
    from w4a16_grouped_quantized_amd import binding as B
    shape = dataclasses.replace(synth.TINY, has_shared=shared)
    layer = synth.make_layer_fmt(shape, 31 + int(shared), fmt)
    dl = B.FmtLayerDev(layer)
    ws = B.Workspace(dl.cfg, 8)
    rng = np.random.default_rng(32)
    for M in (1, 2, 4, 7, 8):
        x = synth.make_tokens(shape, 33 + M, M)
        ids = np.stack([rng.choice(shape.n_experts, shape.top_k, replace=False) for _ in range(M)]).astype(np.int32)
        if M >= 2:
            ids[1] = ids[0]                      # a token routed exactly like the previous one
        w = rng.dirichlet(np.ones(shape.top_k), size=M)
        out = _run(dl, ws, x, ids, w)
        assert B.get_device_error(ws.buf) == 0
        ref, bad = oracle_mod.forward_fmt(shape, fmt, _experts_dict(layer), x, ids, w.astype(np.float32))
        assert bad == 0
        ratio = check_out(from_dev_bf16(out), ref, f"{name} tiny shared={shared} M={M}")
        _say(f"{name} tiny shared={shared} M={M}: max|err|/rms {ratio:.3e}")


@pytest.mark.parametrize("fmt,name", FMTS, ids=[f[1] for f in FMTS])
def test_tiny_out_of_range_id(oracle_mod, fmt, name):
    from w4a16_grouped_quantized_amd import binding as B
    shape = dataclasses.replace(synth.TINY, has_shared=True)
    layer = synth.make_layer_fmt(shape, 41, fmt)
    dl = B.FmtLayerDev(layer)
    ws = B.Workspace(dl.cfg, 2)
    x = synth.make_tokens(shape, 42, 2)
    ids = np.array([[3, 99], [5, 6]], np.int32)
    w = np.array([[0.6, 0.4], [0.5, 0.5]])
    out = _run(dl, ws, x, ids, w)
    assert B.get_device_error(ws.buf) == 1
    ref, bad = oracle_mod.forward_fmt(shape, fmt, _experts_dict(layer), x, ids, w.astype(np.float32))
    assert bad == 1
    check_out(from_dev_bf16(out), ref, f"{name} with an out-of-range id")


@pytest.mark.parametrize("fmt,name", FMTS, ids=[f[1] for f in FMTS])
def test_one_hot_tokens_at_group_and_block_edges(oracle_mod, fmt, name):
    """A token with one nonzero input reads one column of each gate/up row:
    the columns at the edges of a 16-byte chunk, a 32-wide MXFP4 scale group
    and a 128-wide FP8 block, odd and even nibbles."""
    from w4a16_grouped_quantized_amd import binding as B
    shape = dataclasses.replace(synth.TINY, has_shared=True)
    layer = synth.make_layer_fmt(shape, 43, fmt)
    dl = B.FmtLayerDev(layer)
    ws = B.Workspace(dl.cfg, 8)
    cols = [0, 1, 15, 16, 31, 32, 127, 128, 255]
    x = np.zeros((len(cols), shape.hidden), np.uint16)
    for i, c in enumerate(cols):
        x[i, c] = 0x4000  # 2.0
    for m0 in range(0, len(cols), 8):
        xs = x[m0:m0 + 8]
        M = xs.shape[0]
        ids = np.tile(np.array([[4, 11]], np.int32), (M, 1))
        w = np.tile(np.array([[0.75, 0.25]]), (M, 1))
        out = _run(dl, ws, xs, ids, w)
        ref, _ = oracle_mod.forward_fmt(shape, fmt, _experts_dict(layer), xs, ids, w.astype(np.float32))
        check_out(from_dev_bf16(out), ref, f"{name} one-hot columns {cols[m0:m0 + 8]}")
    _say(f"{name}: one-hot tokens at chunk, group and block edges pass")


@pytest.mark.parametrize("fmt,name", FMTS, ids=[f[1] for f in FMTS])
def test_ling_routed_decode_and_verify(oracle_mod, fmt, name):
    """The Ling shape routed by moe_route (the same router as the W4A16
    layer of the seed), then moe_forward_fmt: 12 decode tokens and 3 verify
    steps of 4 tokens."""
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    layer = synth.make_layer_fmt(shape, 1, fmt, threads=16)
    dl = B.FmtLayerDev(layer)
    ws = B.Workspace(dl.cfg, 4)
    ex = _experts_dict(layer)
    worst = 0.0
    for M, steps in ((1, 12), (4, 3)):
        for st in range(steps):
            x = synth.make_tokens(shape, 500 + 10 * M + st, M)
            x_dev = to_dev_bf16(x)
            ids = torch.empty((M, shape.top_k), dtype=torch.int32, device="cuda")
            w = torch.empty((M, shape.top_k), dtype=torch.float32, device="cuda")
            B.route(dl.cfg, dl.router_w, x_dev, ids, w, ws.buf)
            out = torch.empty((M, shape.hidden), dtype=torch.bfloat16, device="cuda")
            B.forward_fmt(dl, x_dev, ids, w, out, ws.buf)
            torch.cuda.synchronize()
            assert B.get_device_error(ws.buf) == 0
            ids_g, w_g = ids.cpu().numpy(), w.cpu().numpy()
            ids_o, _, gap, logits_o = oracle_mod.route(shape, layer.router_w, x)
            w_ref = check_ids(shape, ids_g, w_g, ids_o, gap, logits_o)
            used = set(ids_g.ravel().tolist())
            exs = {key: ({e: ex[key][e] for e in used} if key.startswith("w") else ex[key]) for key in ex}
            ref, bad = oracle_mod.forward_fmt(shape, fmt, exs, x, ids_g, w_ref)
            assert bad == 0
            worst = max(worst, check_out(from_dev_bf16(out), ref, f"{name} Ling M={M} step {st}"))
    _say(f"{name} Ling: 12 decode tokens and 3 verify steps of 4, worst max|err|/rms {worst:.3e}")


# ---------------------------------------------------------------- one launch (moe_layer_mxfp4)

def _layer_mx(dl, x_bits, ws, flags=0):
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    M, H, k = x_bits.shape[0], dl.shape.hidden, dl.shape.top_k
    x = to_dev_bf16(x_bits)
    ids = torch.full((M, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((M, k), -1.0, dtype=torch.float32, device="cuda")
    out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    xn = torch.empty((M, H), dtype=torch.bfloat16, device="cuda") if flags else None
    B.layer_mxfp4(dl.cfg, dl.router_w, dl.packed, x, ids, w, out, ws.buf, flags=flags, x_norm=xn)
    torch.cuda.synchronize()
    xn_bits = from_dev_bf16(xn) if xn is not None else None
    return ids.cpu().numpy(), w.cpu().numpy(), from_dev_bf16(out), xn_bits


def _route_dev(dl, x_bits, ws, flags=0):
    """moe_route on the same tokens (the one launch's ids and weights must
    equal these bit for bit)."""
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    M, k = x_bits.shape[0], dl.shape.top_k
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    w = torch.empty((M, k), dtype=torch.float32, device="cuda")
    xn = torch.empty((M, dl.shape.hidden), dtype=torch.bfloat16, device="cuda") if flags else None
    B.route(dl.cfg, dl.router_w, to_dev_bf16(x_bits), ids, w, ws.buf, flags=flags, x_norm=xn)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def _check_mx_step(oracle_mod, shape, layer, ex, x_bits, ids_g, w_g, out_g, what):
    ids_o, _, gap, logits_o = oracle_mod.route(shape, layer.router_w, x_bits)
    w_ref = check_ids(shape, ids_g, w_g, ids_o, gap, logits_o)
    used = set(ids_g.ravel().tolist())
    exs = {key: ({e: ex[key][e] for e in used} if key.startswith("w") else ex[key]) for key in ex}
    ref, bad = oracle_mod.forward_fmt(shape, synth.FMT_MXFP4, exs, x_bits, ids_g, w_ref)
    assert bad == 0
    return check_out(out_g, ref, what)


@pytest.mark.parametrize("shared", [False, True])
def test_mxfp4_one_launch_tiny(oracle_mod, shared):
    from w4a16_grouped_quantized_amd import binding as B
    shape = dataclasses.replace(synth.TINY, has_shared=shared)
    layer = synth.make_layer_fmt(shape, 51 + int(shared), synth.FMT_MXFP4)
    dl = B.MxLayerDev(layer)
    ws = B.Workspace(dl.cfg, 4)
    ex = _experts_dict(layer)
    for M in (1, 2, 3, 4):
        for st in range(3):
            x = synth.make_tokens(shape, 60 + 10 * M + st, M)
            ids_g, w_g, out_g, _ = _layer_mx(dl, x, ws)
            assert B.get_device_error(ws.buf) == 0
            ids_r, w_r = _route_dev(dl, x, ws)
            assert np.array_equal(ids_g, ids_r) and np.array_equal(w_g.view(np.uint32), w_r.view(np.uint32))
            ratio = _check_mx_step(oracle_mod, shape, layer, ex, x, ids_g, w_g, out_g,
                                   f"mxfp4 one launch tiny shared={shared} M={M} step {st}")
    _say(f"mxfp4 one launch tiny shared={shared}: M = 1..4 match the oracle (last max|err|/rms {ratio:.3e})")


def test_mxfp4_one_launch_ling_decode(oracle_mod):
    """The Ling shape at M = 1 over 48 seeded tokens, as bench.py times it."""
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    layer = synth.make_layer_fmt(shape, 1, synth.FMT_MXFP4, threads=16)
    dl = B.MxLayerDev(layer)
    ws = B.Workspace(dl.cfg, 1)
    ex = _experts_dict(layer)
    worst = 0.0
    for t in range(48):
        x = synth.make_tokens(shape, 700 + t, 1)
        ids_g, w_g, out_g, _ = _layer_mx(dl, x, ws)
        assert B.get_device_error(ws.buf) == 0
        if t < 8:
            ids_r, w_r = _route_dev(dl, x, ws)
            assert np.array_equal(ids_g, ids_r) and np.array_equal(w_g.view(np.uint32), w_r.view(np.uint32))
        worst = max(worst, _check_mx_step(oracle_mod, shape, layer, ex, x, ids_g, w_g, out_g,
                                          f"mxfp4 one launch Ling token {t}"))
    _say(f"mxfp4 one launch Ling: 48 decode tokens, worst max|err|/rms {worst:.3e}")


def test_mxfp4_one_launch_rmsnorm_and_onehot(oracle_mod):
    """RMSNorm in the launch (x_norm within one bf16 step of the oracle's, the
    experts on x_norm), and one-hot normalised inputs at chunk, group and
    tile edges, which read a single column of every gate/up row."""
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    layer = synth.make_layer_fmt(shape, 2, synth.FMT_MXFP4, threads=16)
    dl = B.MxLayerDev(layer)
    ws = B.Workspace(dl.cfg, 1)
    ex = _experts_dict(layer)
    cols = [0, 1, 15, 16, 31, 32, 255, 256, 1279, 2559]
    for i in range(len(cols) + 4):
        if i < len(cols):
            x = np.zeros((1, shape.hidden), np.uint16)
            x[0, cols[i]] = 0x4080  # 4.0
            what = f"one-hot column {cols[i]}"
        else:
            x = synth.bf16_bits(np.random.default_rng(800 + i).standard_normal((1, shape.hidden)) * 3.0)
            what = f"token {i}"
        ids_g, w_g, out_g, xn = _layer_mx(dl, x, ws, flags=B.MOE_F_INPUT_RMSNORM)
        assert B.get_device_error(ws.buf) == 0
        ref_norm = oracle_mod.rmsnorm(x, 1e-6)
        assert np.abs(xn.astype(np.int32) - ref_norm.astype(np.int32)).max() <= 1, what
        ids_r, w_r = _route_dev(dl, x, ws, flags=B.MOE_F_INPUT_RMSNORM)
        assert np.array_equal(ids_g, ids_r) and np.array_equal(w_g.view(np.uint32), w_r.view(np.uint32)), what
        _check_mx_step(oracle_mod, shape, layer, ex, xn, ids_g, w_g, out_g, f"mxfp4 one launch RMSNorm, {what}")
    _say("mxfp4 one launch: RMSNorm and one-hot inputs at chunk, group and tile edges pass")


def test_mxfp4_one_launch_graph_replay(oracle_mod):
    """Four decode steps over two resident copies (distinct routers) captured
    in a graph and replayed three times with eager calls in between; every
    replay equals the eager result bit for bit and the oracle."""
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    layer = synth.make_layer_fmt(shape, 3, synth.FMT_MXFP4, threads=16)
    dl = B.MxLayerDev(layer)
    router2 = torch.from_numpy(synth.make_router(shape, 1003)).cuda()
    ws = B.Workspace(dl.cfg, 1)
    ex = _experts_dict(layer)
    X = synth.make_tokens(shape, 900, 4)
    xd = to_dev_bf16(X)
    k, H = shape.top_k, shape.hidden
    ids = torch.empty((4, k), dtype=torch.int32, device="cuda")
    w = torch.empty((4, k), dtype=torch.float32, device="cuda")
    out = torch.empty((4, H), dtype=torch.bfloat16, device="cuda")
    routers = [dl.router_w, router2, dl.router_w, router2]

    def steps():
        for s in range(4):
            B.layer_mxfp4(dl.cfg, routers[s], dl.packed, xd[s:s + 1], ids[s:s + 1], w[s:s + 1], out[s:s + 1],
                          ws.buf)

    steps()
    torch.cuda.synchronize()
    eager = (ids.clone(), w.clone(), out.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps()
    for r in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, eager[0]) and torch.equal(w, eager[1]) and torch.equal(out, eager[2]), f"replay {r}"
        steps()  # eager work between replays
        torch.cuda.synchronize()
    lay2 = dataclasses.replace(layer, router_w=synth.make_router(shape, 1003))
    for s in range(4):
        lay = layer if s % 2 == 0 else lay2
        _check_mx_step(oracle_mod, shape, lay, ex, X[s:s + 1], eager[0][s:s + 1].cpu().numpy(),
                       eager[1][s:s + 1].cpu().numpy(), from_dev_bf16(eager[2][s:s + 1]), f"mxfp4 graph step {s}")
    _say("mxfp4 one launch: graph replays equal eager and the oracle")
