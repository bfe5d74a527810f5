"""Helpers shared by the GPU parity tests: device marshalling and the parity
rules that compare the HIP path with the CPU oracle.

Parity rules (readings of the pages where they leave the comparison open):
- expert ids: where the oracle's fp64 gap between the k-th and (k+1)-th logit
  is >= 1e-5 the GPU must pick exactly the oracle's set; inside the band every
  GPU id must have an oracle logit >= (k-th logit - 1e-5).  The order within
  the set is checked only up to that band.
- routing weights: within 1e-5 of the softmax over the GPU's ids computed
  from the oracle's fp64 logits.
- outputs: max |gpu - oracle| <= 2e-2 * rms(oracle output of the call) plus
  the rounding of the bf16 output itself (half a bf16 ulp of the oracle
  value), with the oracle fed the GPU's ids and the fp64 weights for them.
"""
from __future__ import annotations

import numpy as np

from w4a16_grouped_quantized_amd import synth

BAND = 1e-5
W_TOL = 1e-5
OUT_TOL = 2e-2


def torch_mod():
    import torch
    return torch


def to_dev_bf16(bits: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def from_dev_bf16(t) -> np.ndarray:
    torch = torch_mod()
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_f64(bits) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def check_ids(shape, ids_gpu, w_gpu, ids_o, gap, logits_o):
    """Returns fp64 weights for the GPU's ids (used as the oracle's input)."""
    M, k = ids_gpu.shape
    w_ref = np.empty((M, k))
    for t in range(M):
        g = ids_gpu[t]
        assert len(set(g.tolist())) == k, f"token {t}: repeated ids {g}"
        assert np.all((g >= 0) & (g < shape.n_experts)), f"token {t}: id out of range {g}"
        l = logits_o[t]
        if gap[t] >= BAND:
            assert set(g.tolist()) == set(ids_o[t].tolist()), (t, g, ids_o[t], gap[t])
        else:
            kth = l[ids_o[t][k - 1]]
            assert np.all(l[g] >= kth - BAND), (t, g, ids_o[t], gap[t])
        assert np.all(np.diff(l[g]) <= BAND), f"token {t}: ids not in descending logit order"
        lg = l[g]
        e = np.exp(lg - lg.max())
        w_ref[t] = e / e.sum()
        assert np.max(np.abs(w_gpu[t] - w_ref[t])) <= W_TOL, (t, w_gpu[t], w_ref[t])
    return w_ref


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place of each value (8 significant bits):
    the largest error of rounding v to bf16 to nearest."""
    _, ex = np.frexp(np.abs(v))            # |v| = m * 2^ex, m in [0.5, 1)
    return np.where(v == 0, 0.0, np.ldexp(1.0, ex - 9))


def check_out(out_gpu_bits, out_ref, what=""):
    """max |gpu - oracle| <= 2e-2 * rms(oracle), read as a bound on the
    computation: the layer output is a bf16 tensor, and its one rounding to
    bf16 (up to half a bf16 ulp of the value, which alone passes 2e-2 * rms
    wherever |out| > 5.1 * rms) is allowed on top.  Returns the plain ratio
    max|err| / rms."""
    got = bf16_f64(out_gpu_bits)
    rms = float(np.sqrt(np.mean(out_ref ** 2)))
    diff = np.abs(got - out_ref)
    err = float(np.max(diff))
    excess = float(np.max(diff - bf16_half_ulp(out_ref)))
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert excess <= OUT_TOL * rms, (
        f"{what}: max(|err| - half bf16 ulp) {excess:.4g} > {OUT_TOL} * rms {rms:.4g} "
        f"(plain max|err|/rms {err / rms:.3g})")
    check_out.last_excess = excess / rms
    return err / rms


class DeviceLayer:
    """A synth layer on the GPU through the C ABI, plus a workspace."""

    def __init__(self, layer, max_tokens: int):
        from w4a16_grouped_quantized_amd import binding as B
        self.B = B
        self.layer = layer
        self.shape = layer.shape
        self.dev = B.MoeLayer(layer)
        self.cfg = self.dev.cfg
        self.ws = B.Workspace(self.cfg, max_tokens)

    def route(self, x_dev, flags=0, x_norm=None):
        torch = torch_mod()
        M = x_dev.shape[0]
        ids = torch.empty((M, self.shape.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((M, self.shape.top_k), dtype=torch.float32, device="cuda")
        self.B.route(self.cfg, self.dev.router_w, x_dev, ids, w, self.ws.buf, flags=flags, x_norm=x_norm)
        return ids, w

    def forward(self, x_dev, ids, w):
        torch = torch_mod()
        out = torch.empty((x_dev.shape[0], self.shape.hidden), dtype=torch.bfloat16, device="cuda")
        self.B.forward(self.cfg, self.dev.packed, x_dev, ids, w, out, self.ws.buf)
        return out

    def device_error(self) -> int:
        return self.B.get_device_error(self.ws.buf)


def run_and_check(dl: DeviceLayer, oracle, x_bits: np.ndarray, what: str = ""):
    """route + forward on the GPU for one call of M = len(x_bits) tokens, and
    the full parity check against the oracle.  Returns the error ratio."""
    torch = torch_mod()
    x_dev = to_dev_bf16(x_bits)
    ids, w = dl.route(x_dev)
    out = dl.forward(x_dev, ids, w)
    torch.cuda.synchronize()
    ids_g, w_g = ids.cpu().numpy(), w.cpu().numpy()
    ids_o, _, gap, logits_o = oracle.route(dl.shape, dl.layer.router_w, x_bits)
    w_ref = check_ids(dl.shape, ids_g, w_g, ids_o, gap, logits_o)
    out_ref, bad = oracle.forward(dl.shape, dl.layer, x_bits, ids_g, w_ref)
    assert bad == 0
    ratio = check_out(from_dev_bf16(out), out_ref, what)
    print(f"{what}: max|err|/rms {ratio:.3e}, beyond the bf16 store {check_out.last_excess:.3e}", flush=True)
    return ratio
