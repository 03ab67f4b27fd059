"""Pins of the oracle's grouped GEMM + dSwiGLU backward ("Grouped GEMM +
dSwiGLU (SM100)", Steps 1 and 2):

  * the epilogue is the gradient of the forward gated SwiGLU
    y = prob * input * gate * sigmoid(gate) with upstream gradient ref:
    torch autograd (fp64, CPU) of that forward gives d/d input = ab / ref,
    d/d gate = dswiglu / ref and d/d prob summed over the row = dprob;
  * ref equals alpha_g times the sReLU operation's C = alpha_g * acc on the
    same operands (the GEMM and routing are shared);
  * the 32-column pairing: ab lands in columns [64b, 64b+32) and dswiglu in
    [64b+32, 64b+64), read from the input / gate blocks at the same places;
  * gate = 0 gives ab = 0 and dswiglu = ref * prob * input / 2.
"""
import numpy as np
import torch

import oracle as O
import workloads as W


def _case(seed=0, n=64, k=128, sizes=(256, 0, 256)):
    off = np.cumsum(sizes).astype(np.int32)
    p = W.grouped_dswiglu_problem(0, len(sizes), n, k, "e4m3", seed=seed, offsets=off)
    s = p.sizes
    r = O.grouped_dswiglu(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], off, p.t["alpha"], p.t["beta"],
                          p.t["prob"], O.bits16(p.t["c"]), s["m"], n, k, len(sizes), "e4m3")
    return p, off, r


def _gather(p, off, n):
    m = p.sizes["m"]
    grp = np.searchsorted(off, np.arange(m), side="right")
    beta = p.t["beta"].double().numpy()[grp]
    c = p.t["c"].double().numpy()
    blocks = np.arange(n) // 32 * 64 + np.arange(n) % 32
    return grp, beta[:, None] * c[:, blocks], beta[:, None] * c[:, blocks + 32], blocks


def test_epilogue_is_the_swiglu_gradient():
    n = 64
    p, off, r = _case(1, n=n)
    grp, x_in, x_gt, cols = _gather(p, off, n)
    ref = torch.from_numpy(r["ref"])
    xi = torch.from_numpy(x_in).requires_grad_(True)
    xg = torch.from_numpy(x_gt).requires_grad_(True)
    pr = p.t["prob"].double().clone().requires_grad_(True)
    y = pr[:, None] * xi * xg * torch.sigmoid(xg)
    y.backward(ref)
    np.testing.assert_allclose(r["d"][:, cols], xi.grad.numpy(), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(r["d"][:, cols + 32], xg.grad.numpy(), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(r["dprob"], pr.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_ref_is_alpha_times_the_srelu_pre_activation():
    n, k = 64, 128
    p, off, r = _case(2, n=n, k=k)
    s = p.sizes
    q = O.grouped_srelu(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], off, p.t["alpha"], p.t["prob"],
                        s["m"], n, k, len(off), "e4m3", 0.0)
    alpha = p.t["alpha"].double().numpy()[q["group"]]
    np.testing.assert_allclose(r["ref"], alpha[:, None] * q["c"], rtol=1e-14, atol=0)


def test_zero_gate_and_column_pairing():
    n = 96
    p, off, r0 = _case(3, n=n)
    c = p.t["c"].clone()
    blocks = np.arange(n) // 32 * 64 + np.arange(n) % 32
    c[:, torch.from_numpy(blocks + 32)] = 0            # gate = 0 everywhere
    p.t["c"] = c
    s = p.sizes
    r = O.grouped_dswiglu(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], off, p.t["alpha"], p.t["beta"],
                          p.t["prob"], O.bits16(p.t["c"]), s["m"], n, s["k"], len(off), "e4m3")
    grp, x_in, _, cols = _gather(p, off, n)
    prob = p.t["prob"].double().numpy()[:, None]
    assert np.all(r["d"][:, cols] == 0.0)
    np.testing.assert_allclose(r["d"][:, cols + 32], r["ref"] * prob * x_in * 0.5, rtol=1e-15, atol=0)
    assert np.all(r["dprob"] == 0.0)
    assert np.array_equal(r["ref"], r0["ref"])         # C does not enter ref
