"""GPU parity of the speculative-decoding round (w4a16_grouped_quantized_amd.mtp):
3 draft steps through a draft layer and a 4-position verify through a stack
of layers, every step of it against the oracle with its inputs taken from
the GPU (teacher-forced), run eagerly and replayed from a captured graph."""
import sys

import numpy as np
import pytest

from w4a16_grouped_quantized_amd import synth
from parity import check_ids, check_out, from_dev_bf16, to_dev_bf16

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


def test_mtp_round_against_oracle(ling_seed1, ling_seed23, oracle_mod):
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    from w4a16_grouped_quantized_amd.mtp import MtpRound
    shape = synth.LING
    cfg = B.config(shape)
    draft_np, stack_np = ling_seed1, list(ling_seed23)
    draft_dev = B.MoeLayer(draft_np)
    stack_dev = [B.MoeLayer(l) for l in stack_np]
    ws = B.Workspace(cfg, 4)
    r = MtpRound(cfg, [(d.router_w, d.packed) for d in stack_dev], (draft_dev.router_w, draft_dev.packed), ws)
    L, nd = len(stack_np), r.n_draft
    rec_d = {"xn": [torch.empty_like(r.d_norm) for _ in range(nd)], "ids": [torch.empty_like(r.d_ids) for _ in range(nd)],
             "w": [torch.empty_like(r.d_w) for _ in range(nd)]}
    rec_v = {"xn": [torch.empty_like(r.v_norm) for _ in range(L)], "ids": [torch.empty_like(r.v_ids) for _ in range(L)],
             "w": [torch.empty_like(r.v_w) for _ in range(L)], "out": [torch.empty_like(r.v_bufs[0]) for _ in range(L)]}

    def keep_d(d, xn, ids, w):
        rec_d["xn"][d].copy_(xn); rec_d["ids"][d].copy_(ids); rec_d["w"][d].copy_(w)

    def keep_v(l, xn, ids, w, out):
        rec_v["xn"][l].copy_(xn); rec_v["ids"][l].copy_(ids); rec_v["w"][l].copy_(w); rec_v["out"][l].copy_(out)

    def layer_check(layer, x_raw, xn_gpu, ids_gpu, w_gpu, out_gpu, what):
        ref_norm = oracle_mod.rmsnorm(x_raw, 1e-6)
        d = np.abs(xn_gpu.astype(np.int32) - ref_norm.astype(np.int32))
        assert d.max() <= 1, f"{what}: RMSNorm differs by more than one bf16 step"
        ids_o, _, gap, logits_o = oracle_mod.route(shape, layer.router_w, xn_gpu)
        w_ref = check_ids(shape, ids_gpu, w_gpu, ids_o, gap, logits_o)
        ref, bad = oracle_mod.forward(shape, layer, xn_gpu, ids_gpu, w_ref)
        assert bad == 0
        check_out(out_gpu, ref, what)

    def check(what):
        rows = from_dev_bf16(r.rows)
        for d in range(nd):
            layer_check(draft_np, rows[d:d + 1], from_dev_bf16(rec_d["xn"][d]), rec_d["ids"][d].cpu().numpy(),
                        rec_d["w"][d].cpu().numpy(), rows[d + 1:d + 2], f"{what} draft {d}")
        prev = rows
        for l in range(L):
            out = from_dev_bf16(rec_v["out"][l])
            layer_check(stack_np[l], prev, from_dev_bf16(rec_v["xn"][l]), rec_v["ids"][l].cpu().numpy(),
                        rec_v["w"][l].cpu().numpy(), out, f"{what} verify layer {l}")
            prev = out

    xs = synth.make_tokens(shape, 4242, 6)
    for t in range(2):
        r.rows[0:1].copy_(to_dev_bf16(xs[t:t + 1]))
        r.round(record_draft=keep_d, record_verify=keep_v)
        torch.cuda.synchronize()
        assert B.get_device_error(ws.buf) == 0
        check(f"round eager {t}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r.round(record_draft=keep_d, record_verify=keep_v)
    for t in range(2, xs.shape[0]):
        r.rows[0:1].copy_(to_dev_bf16(xs[t:t + 1]))
        g.replay()
        torch.cuda.synchronize()
        assert B.get_device_error(ws.buf) == 0
        check(f"round graph {t}")
    _say(f"MTP round: {nd} drafts + {nd + 1}-position verify through {L} layers, 2 eager + 4 replayed rounds checked")
