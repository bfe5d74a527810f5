"""moe_layer_w4a16_noalloc (the layer on the library's static workspace, for
callers that cannot allocate) against moe_layer_w4a16 on a caller workspace:
the same ids and weights, the same output bits, and both within the oracle's
bar; two calls in a row, the second smaller, then an RMSNorm call, then a call
beyond the static workspace, which must be refused before any launch."""
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


def _outputs(dl, M):
    import torch
    k, H = dl.shape.top_k, dl.shape.hidden
    return (torch.full((M, k), -7, dtype=torch.int32, device="cuda"),
            torch.full((M, k), -1.0, dtype=torch.float32, device="cuda"),
            torch.full((M, H), 12345, dtype=torch.int16, device="cuda").view(torch.bfloat16))


def test_noalloc_matches_workspace_entry_point(ling_seed1, oracle_mod):
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    dl = DeviceLayer(ling_seed1, max_tokens=8)
    shape = dl.shape
    cases = [(4, B.MOE_F_ONE_LAUNCH), (1, 0), (2, B.MOE_F_ONE_LAUNCH | B.MOE_F_INPUT_RMSNORM)]
    for i, (M, flags) in enumerate(cases):
        _say(f"no-alloc call {i}: M={M} flags={flags}")
        rms = bool(flags & B.MOE_F_INPUT_RMSNORM)
        if rms:
            x = synth.bf16_bits(np.random.default_rng(1300 + i).standard_normal((M, shape.hidden)) * 5.0)
        else:
            x = synth.make_tokens(shape, 1300 + i, M)
        x_dev = to_dev_bf16(x)
        ids_n, w_n, out_n = _outputs(dl, M)
        ids_r, w_r, out_r = _outputs(dl, M)
        xn_n = torch.empty_like(out_n) if rms else None
        xn_r = torch.empty_like(out_r) if rms else None
        B.layer_noalloc(dl.cfg, dl.dev.router_w, dl.dev.packed, x_dev, ids_n, w_n, out_n, flags=flags, x_norm=xn_n)
        B.layer(dl.cfg, dl.dev.router_w, dl.dev.packed, x_dev, ids_r, w_r, out_r, dl.ws.buf, flags=flags,
                x_norm=xn_r)
        torch.cuda.synchronize()
        assert dl.device_error() == 0
        # the same kernels on the same inputs: identical results
        assert torch.equal(ids_n, ids_r) and torch.equal(w_n, w_r)
        assert torch.equal(out_n.view(torch.int16), out_r.view(torch.int16))
        if rms:
            assert torch.equal(xn_n.view(torch.int16), xn_r.view(torch.int16))
        # and the oracle's bar on the no-alloc results
        x_used = xn_n.view(torch.int16).cpu().numpy().view(np.uint16) if rms else x
        ids_g, w_g = ids_n.cpu().numpy(), w_n.cpu().numpy()
        ids_o, _, gap, logits_o = oracle_mod.route(shape, dl.layer.router_w, x_used)
        w_ref = check_ids(shape, ids_g, w_g, ids_o, gap, logits_o)
        ref, bad = oracle_mod.forward(shape, dl.layer, x_used, ids_g, w_ref)
        assert bad == 0
        ratio = check_out(from_dev_bf16(out_n), ref, f"no-alloc M={M}")
        _say(f"no-alloc call {i}: identical to the workspace call; max|err|/rms {ratio:.3e}")


def test_noalloc_refuses_beyond_its_workspace(ling_seed1):
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    dl = DeviceLayer(ling_seed1, max_tokens=1)
    M = 1
    while B.workspace_size(dl.cfg, M) <= B.MOE_NOALLOC_WS_BYTES:
        M += 1
    _say(f"no-alloc refusal at M={M}")
    x_dev = to_dev_bf16(synth.make_tokens(dl.shape, 1400, M))
    ids, w, out = _outputs(dl, M)
    with pytest.raises(B.MoeError) as e:
        B.layer_noalloc(dl.cfg, dl.dev.router_w, dl.dev.packed, x_dev, ids, w, out)
    assert e.value.status == B.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((ids == -7).all()) and bool((out.view(torch.int16) == 12345).all())
