"""GPU parity of the FP8 LM head (moe_lmhead_quantize_fp8, moe_lmhead_fp8,
moe_lmhead_bf16) against the fp64 oracle: the codes and row scales bit for
bit, every E4M3 code through the GEMV's converter, the products within a
bound derived from their fp32 accumulation, on ragged small heads and on
sampled rows of the full 157,184 x 2,560 head in the benchmark's launch."""
import sys

import numpy as np
import pytest

from w4a16_grouped_quantized_amd import synth

pytestmark = pytest.mark.gpu

H_LING = 2560


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


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _quantize_dev(w_bits):
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    V, H = w_bits.shape
    w = _dev(w_bits.view(np.int16))
    q = torch.empty((V, H), dtype=torch.uint8, device="cuda")
    s = torch.empty(V, dtype=torch.float32, device="cuda")
    B.lmhead_quantize_fp8(w, q, s)
    return w, q, s


def _gemv(q_dev, s_dev, x_bits, fp8=True, w_dev=None):
    import torch
    from w4a16_grouped_quantized_amd import binding as B
    x = _dev(x_bits.view(np.int16))
    V = q_dev.shape[0] if fp8 else w_dev.shape[0]
    out = torch.full((x_bits.shape[0], V), float("nan"), dtype=torch.float32, device="cuda")
    if fp8:
        B.lmhead_fp8(q_dev, s_dev, x, out)
    else:
        B.lmhead_bf16(w_dev, x, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _decode(q):
    import torch
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _check_products(got, ref, absterms, what):
    # fp32 accumulation: about 30 roundings per row (dot2 chains of a lane,
    # the 64-lane tree, the scale), each within 2^-24 of the running sum
    bound = 4e-6 * absterms + 1e-30
    err = np.abs(got - ref)
    worst = float(np.max(err / bound))
    _say(f"{what}: worst error / bound {worst:.3f}")
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound), what


def _special_rows(H):
    """Rows with exact ties: amax 1.75 (448 * 2^-8, so the scale is 2^-8) and
    midpoints between neighbouring E4M3 codes (and their bf16 neighbours),
    an all-zero row, a row of tiny values, a row with one huge value."""
    rows = []
    pos = _decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2 * 2.0 ** -8
    r = np.zeros(H)
    r[0] = 1.75
    r[1:1 + mids.size] = mids[: H - 1]
    r[1 + mids.size: 1 + 2 * mids.size] = -mids[: max(0, H - 1 - mids.size)]
    rows.append(synth.bf16_bits(r))
    b = rows[-1].copy()
    b[1:] = np.where(b[1:] != 0, b[1:] + 1, 0)  # the next bf16 above each midpoint's magnitude
    rows.append(b)
    rows.append(np.zeros(H, np.uint16))
    rows.append(synth.bf16_bits(np.random.default_rng(5).standard_normal(H) * 1e-30))
    big = synth.bf16_bits(np.random.default_rng(6).standard_normal(H) * 0.02)
    big[7] = synth.bf16_bits(np.array([3.0e36]))[0]
    rows.append(big)
    return np.stack(rows)


@pytest.mark.parametrize("H", [H_LING, 256])
def test_quantize_bit_exact(oracle_mod, H):
    V = 4133  # several workgroups and a ragged tail
    w = synth.make_lmhead(V, H, 20 + H)
    w[: 5] = _special_rows(H)
    _, q, s = _quantize_dev(w)
    q_o, s_o = oracle_mod.lmhead_quantize(w)
    qg, sg = q.cpu().numpy(), s.cpu().numpy()
    assert np.array_equal(sg.view(np.uint32), s_o.view(np.uint32))
    bad = np.argwhere(qg != q_o)
    assert bad.size == 0, f"{bad.shape[0]} codes differ, first at {bad[:5].tolist()}"
    _say(f"quantize H={H}: {V} rows bit-exact (codes and scales)")


def test_every_e4m3_code_through_the_gemv(oracle_mod):
    """q rows holding every finite code, scale 1: a one-hot token reads one
    column, so each logit is the code's value (one product, exact)."""
    import torch
    H = 256
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    V = finite.size
    q = np.zeros((V, H), np.uint8)
    for j in range(H):
        q[:, j] = np.roll(finite, j)
    q_dev = _dev(q)
    s_dev = torch.ones(V, dtype=torch.float32, device="cuda")
    for h in (0, 1, 15, 16, 17, 127, 128, 255):
        x = np.zeros((1, H), np.uint16)
        x[0, h] = 0x3F80
        got = _gemv(q_dev, s_dev, x)[0]
        ref = oracle_mod.lmhead_gemv_fp8(q, np.ones(V, np.float32), x)[0]
        assert np.array_equal(got, ref.astype(np.float32)), f"column {h}"
    _say("every E4M3 code decodes as the oracle's through the GEMV")


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("H", [H_LING, 256])
def test_gemv_fp8_and_bf16_against_oracle(oracle_mod, M, H):
    V = 4133
    w = synth.make_lmhead(V, H, 30 + H)
    w[: 5] = _special_rows(H)
    w_dev, q, s = _quantize_dev(w)
    x = synth.bf16_bits(np.random.default_rng(40 + M).standard_normal((M, H)))
    q_o, s_o = oracle_mod.lmhead_quantize(w)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    got = _gemv(q, s, x)
    ref = oracle_mod.lmhead_gemv_fp8(q_o, s_o, x)
    absterms = (np.abs(_decode(q_o)) * s_o[:, None].astype(np.float64)) @ np.abs(xf).T
    _check_products(got, ref, absterms.T, f"fp8 GEMV H={H} M={M}")
    gotb = _gemv(None, None, x, fp8=False, w_dev=w_dev)
    refb = oracle_mod.lmhead_gemv_bf16(w, x)
    absb = np.abs(synth.bf16_bits_to_f32(w).astype(np.float64)) @ np.abs(xf).T
    _check_products(gotb, refb, absb.T, f"bf16 GEMV H={H} M={M}")


def test_full_head_sampled_rows(oracle_mod):
    """The 157,184 x 2,560 head as the benchmark runs it: quantised on the
    GPU, then the M = 1 product; 512 rows (first, last, random) against the
    oracle, the codes of those rows bit for bit."""
    V = synth.LM_VOCAB
    w = synth.make_lmhead(V, H_LING, 1, threads=16)
    w_dev, q, s = _quantize_dev(w)
    x = synth.bf16_bits(np.random.default_rng(77).standard_normal((1, H_LING)))
    got = _gemv(q, s, x)[0]
    gotb = _gemv(None, None, x, fp8=False, w_dev=w_dev)[0]
    rows = np.unique(np.concatenate([[0, 1, V - 2, V - 1], np.random.default_rng(78).integers(0, V, 508)]))
    q_o, s_o = oracle_mod.lmhead_quantize(w[rows])
    assert np.array_equal(q.cpu().numpy()[rows], q_o)
    assert np.array_equal(s.cpu().numpy()[rows].view(np.uint32), s_o.view(np.uint32))
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    ref = oracle_mod.lmhead_gemv_fp8(q_o, s_o, x)[0]
    absterms = (np.abs(_decode(q_o)) * s_o[:, None].astype(np.float64)) @ np.abs(xf[0])
    _check_products(got[rows], ref, absterms, "full head fp8, sampled rows")
    refb = oracle_mod.lmhead_gemv_bf16(w[rows], x)[0]
    absb = np.abs(synth.bf16_bits_to_f32(w[rows]).astype(np.float64)) @ np.abs(xf[0])
    _check_products(gotb[rows], refb, absb, "full head bf16, sampled rows")
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(gotb))
