"""GPU parity of exactly the launch configurations bench.py times, against
the fp64 oracle:

- decode: one moe_layer_w4a16 call (one launch) per token, rotating over
  resident layer copies (cloned packed weights, distinct seeded routers),
  captured in a HIP graph and replayed over 1024 seeded Ling tokens; every
  token's ids, weights and output are checked;
- stacked decode: the one-launch layer with the RMSNorm input flag, one
  x_norm buffer, one workspace, ids/weights shared by the layers of a step
  and outputs alternating between two buffers, eager and replayed from a
  graph, checked layer by layer (teacher-forced);
- prefill: one 4096-token chunk, the routing of every row and the outputs of
  the rows that end an expert's sorted run or a 96-row work item, plus a
  seeded sample (at least 256 rows);
- the one-launch layer's determinism over 100 repeats.
"""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from w4a16_grouped_quantized_amd import synth
from parity import bf16_f64, check_ids, check_out, from_dev_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu

ITEM_ROWS = 96   # rows of one grouped-GEMM work item (an expert's sorted run is cut into these)


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


def _route_rows(oracle, shape, router, x, chunk=256):
    """oracle.route over many rows, chunks in parallel threads (the C call
    releases the interpreter lock); same results as one call."""
    parts = [x[i:i + chunk] for i in range(0, x.shape[0], chunk)]
    with ThreadPoolExecutor(max_workers=16) as ex:
        res = list(ex.map(lambda p: oracle.route(shape, router, p), parts))
    return tuple(np.concatenate([r[i] for r in res]) for i in range(4))


def _check_tokens(shape, oracle, experts, router, x, ids, w, out_bits, what):
    """Per token: ids within the gap band, weights, and the output against
    oracle.forward on the GPU's ids (each token is one call of the bench)."""
    ids_o, _, gap, logits_o = _route_rows(oracle, shape, router, x)
    w_ref = check_ids(shape, ids, w, ids_o, gap, logits_o)
    ref, bad = oracle.forward(shape, experts, x, ids, w_ref)
    assert bad == 0
    worst = 0.0
    for t in range(x.shape[0]):
        worst = max(worst, check_out(out_bits[t:t + 1], ref[t:t + 1], f"{what} token {t}"))
    return worst


COPIES = 4       # resident layer copies the steps rotate over
GRAPH_STEPS = 8  # decode steps captured per graph
REPLAYS = 128    # 1024 tokens


def test_decode_graph_over_rotating_copies_against_oracle(ling_seed1, oracle_mod):
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    H, k = shape.hidden, shape.top_k
    cfg = B.config(shape)
    base = B.MoeLayer(ling_seed1)
    routers = [synth.make_router(shape, 1000 + c) for c in range(COPIES)]
    copies = [(base.packed if c == 0 else base.packed.clone(), torch.from_numpy(routers[c]).cuda())
              for c in range(COPIES)]
    ws = B.Workspace(cfg, 1)
    X = torch.empty((GRAPH_STEPS, 1, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((GRAPH_STEPS, 1, k), dtype=torch.int32, device="cuda")
    w = torch.empty((GRAPH_STEPS, 1, k), dtype=torch.float32, device="cuda")
    out = torch.empty((GRAPH_STEPS, 1, H), dtype=torch.bfloat16, device="cuda")

    def body():
        for i in range(GRAPH_STEPS):
            pk, rt = copies[i % COPIES]
            B.layer(cfg, rt, pk, X[i], ids[i], w[i], out[i], ws.buf)

    n = GRAPH_STEPS * REPLAYS
    xs = synth.make_tokens(shape, 4242, n)
    X.copy_(to_dev_bf16(xs[:GRAPH_STEPS]).view(GRAPH_STEPS, 1, H))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # the first calls outside capture
        body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    got_ids = np.empty((n, k), np.int32)
    got_w = np.empty((n, k), np.float32)
    got_out = np.empty((n, H), np.uint16)
    for r in range(REPLAYS):
        sl = slice(r * GRAPH_STEPS, (r + 1) * GRAPH_STEPS)
        X.copy_(to_dev_bf16(xs[sl]).view(GRAPH_STEPS, 1, H))
        g.replay()
        torch.cuda.synchronize()
        got_ids[sl] = ids.view(GRAPH_STEPS, k).cpu().numpy()
        got_w[sl] = w.view(GRAPH_STEPS, k).cpu().numpy()
        got_out[sl] = from_dev_bf16(out.view(GRAPH_STEPS, H))
    assert B.get_device_error(ws.buf) == 0
    _say(f"decode graph: {n} tokens replayed over {COPIES} copies; checking against the oracle")
    worst = 0.0
    step = np.arange(n) % GRAPH_STEPS
    for c in range(COPIES):
        sel = np.nonzero(step % COPIES == c)[0]
        worst = max(worst, _check_tokens(shape, oracle_mod, ling_seed1, routers[c], xs[sel], got_ids[sel],
                                         got_w[sel], got_out[sel], f"decode graph copy {c}"))
    _say(f"decode graph: {n} tokens, every step checked; worst max|err|/rms {worst:.3e}")


def _stack_chain(B, cfg, layers, x_in, ids, w, bufs, xn, ws, rec):
    """bench.py's stacked step on the one-launch path, plus copies of what
    each layer wrote (the chain itself overwrites them)."""
    for l, (rt, pk) in enumerate(layers):
        if l == 0:
            B.layer(cfg, rt, pk, x_in, ids, w, bufs[0], ws.buf)
        else:
            B.layer(cfg, rt, pk, bufs[(l - 1) % 2], ids, w, bufs[l % 2], ws.buf,
                    flags=B.MOE_F_INPUT_RMSNORM, x_norm=xn)
            rec["xn"][l].copy_(xn)
        rec["out"][l].copy_(bufs[l % 2])
        rec["ids"][l].copy_(ids)
        rec["w"][l].copy_(w)


def test_stack_one_launch_rmsnorm_chain_eager_and_graph(ling_seed1, ling_seed23, oracle_mod):
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    H, k = shape.hidden, shape.top_k
    cfg = B.config(shape)
    np_layers = [ling_seed1] + list(ling_seed23)
    dev = [B.MoeLayer(layer) for layer in np_layers]
    layers = [(d.router_w, d.packed) for d in dev]
    L = len(layers)
    ws = B.Workspace(cfg, 1)
    x_in = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((1, k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, k), dtype=torch.float32, device="cuda")
    bufs = (torch.empty((1, H), dtype=torch.bfloat16, device="cuda"),
            torch.empty((1, H), dtype=torch.bfloat16, device="cuda"))
    xn = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
    rec = {"xn": [torch.zeros_like(xn) for _ in range(L)], "out": [torch.empty_like(xn) for _ in range(L)],
           "ids": [torch.empty_like(ids) for _ in range(L)], "w": [torch.empty_like(w) for _ in range(L)]}
    xs = synth.make_tokens(shape, 777, 12)

    def check(x_bits, what):
        prev = None
        for l in range(L):
            out_b = from_dev_bf16(rec["out"][l])
            if l == 0:
                xin = x_bits
            else:
                xin = from_dev_bf16(rec["xn"][l])
                ref_norm = oracle_mod.rmsnorm(prev, 1e-6)
                d = np.abs(xin.astype(np.int32) - ref_norm.astype(np.int32))
                assert d.max() <= 1, f"{what} layer {l}: RMSNorm differs by more than one bf16 step"
            ids_o, _, gap, logits_o = oracle_mod.route(shape, np_layers[l].router_w, xin)
            w_ref = check_ids(shape, rec["ids"][l].cpu().numpy(), rec["w"][l].cpu().numpy(), ids_o, gap, logits_o)
            ref, bad = oracle_mod.forward(shape, np_layers[l], xin, rec["ids"][l].cpu().numpy(), w_ref)
            assert bad == 0
            check_out(out_b, ref, f"{what} layer {l}")
            prev = out_b

    # eager
    for t in range(4):
        x_in.copy_(to_dev_bf16(xs[t:t + 1]))
        _stack_chain(B, cfg, layers, x_in, ids, w, bufs, xn, ws, rec)
        torch.cuda.synchronize()
        assert B.get_device_error(ws.buf) == 0
        check(xs[t:t + 1], f"stack eager token {t}")
    # the same chain captured once and replayed on new tokens, eager work and
    # synchronisations in between
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _stack_chain(B, cfg, layers, x_in, ids, w, bufs, xn, ws, rec)
    for t in range(4, xs.shape[0]):
        x_in.copy_(to_dev_bf16(xs[t:t + 1]))
        g.replay()
        torch.cuda.synchronize()
        assert B.get_device_error(ws.buf) == 0
        check(xs[t:t + 1], f"stack graph token {t}")
    _say(f"stack chain: {L} one-launch layers with RMSNorm, 4 eager + {xs.shape[0] - 4} replayed tokens checked")


def test_prefill_4096_every_row_routed_and_tail_rows_checked(ling_seed1, oracle_mod):
    import torch
    from parity import DeviceLayer
    shape = synth.LING
    M, k = 4096, shape.top_k
    dl = DeviceLayer(ling_seed1, max_tokens=M)
    x = synth.make_tokens(shape, 3, M)
    x_dev = to_dev_bf16(x)
    ids, w = dl.route(x_dev)
    out = dl.forward(x_dev, ids, w)
    torch.cuda.synchronize()
    assert dl.device_error() == 0
    ids_g, w_g, out_g = ids.cpu().numpy(), w.cpu().numpy(), from_dev_bf16(out)
    assert np.all(np.isfinite(bf16_f64(out_g)))
    # the routing of every row
    ids_o, _, gap, logits_o = _route_rows(oracle_mod, shape, dl.layer.router_w, x)
    w_ref = check_ids(shape, ids_g, w_g, ids_o, gap, logits_o)
    # rows to check: the token of the last pair of every expert's sorted run
    # (ascending pair index inside an expert), of the pairs that end and start
    # a 96-row work item, and a seeded sample
    pairs = ids_g.ravel()
    rows = set()
    for e in np.unique(pairs):
        run = np.nonzero(pairs == e)[0]           # pair indices, ascending = sorted order
        rows.add(int(run[-1] // k))
        for b in range(ITEM_ROWS, run.size, ITEM_ROWS):
            rows.add(int(run[b - 1] // k))
            rows.add(int(run[b] // k))
    rng = np.random.default_rng(4096)
    rows |= set(rng.choice(M, size=256, replace=False).tolist())
    rows = np.array(sorted(rows))
    ref, bad = oracle_mod.forward(shape, ling_seed1, x[rows], ids_g[rows], w_ref[rows])
    assert bad == 0
    ratio = check_out(out_g[rows], ref, "prefill 4096 checked rows")
    _say(f"prefill 4096: routing of all {M} rows checked; outputs of {rows.size} rows "
         f"(every expert's last row, item edges, 256 sampled): max|err|/rms {ratio:.3e}")


def test_one_launch_layer_determinism_100(ling_seed1):
    import torch
    from parity import DeviceLayer
    from w4a16_grouped_quantized_amd import binding as B
    shape = synth.LING
    dl = DeviceLayer(ling_seed1, max_tokens=1)
    x = to_dev_bf16(synth.make_tokens(shape, 31, 1))

    def run():
        ids = torch.empty((1, shape.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((1, shape.top_k), dtype=torch.float32, device="cuda")
        out = torch.empty((1, shape.hidden), dtype=torch.bfloat16, device="cuda")
        B.layer(dl.cfg, dl.dev.router_w, dl.dev.packed, x, ids, w, out, dl.ws.buf)
        return ids, w, out

    r_ids, r_w, r_out = run()
    for i in range(100):
        ids, w, out = run()
        assert torch.equal(ids, r_ids) and torch.equal(w, r_w), f"repeat {i}: routing"
        assert torch.equal(out.view(torch.int16), r_out.view(torch.int16)), f"repeat {i}: output"
    torch.cuda.synchronize()
    assert dl.device_error() == 0
