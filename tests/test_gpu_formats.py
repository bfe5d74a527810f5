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
