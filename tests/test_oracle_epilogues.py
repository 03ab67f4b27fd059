"""Pins of the oracle's fused epilogues and MX output quantiser.

  * sReLU / tanh clamp ("Grouped GEMM + sReLU (SM100)", Equations and Tanh
    soft clamp): relu zeroes C <= 0, prob = 0 zeroes D, D <= s^2 prob, the
    unclamped limit, and the closed form tanh(ln(2)/2) = 1/3.
  * BF16 grouped ("Grouped GEMM (SM100 BF16)", Operation): numpy float64
    matmul per expert, and the literal bias / no-bias asymmetry.
  * RoPE ("GEMM + RoPE + MXFP8 Projection (SM100)", Equations): cos=1/sin=0
    is the pure de-interleave, cos=0/sin=1 gives [-b, a], features before the
    rotary part equal the plain projection, both weight layouts agree.
  * Quantiser ("Grouped GEMM + dSwiGLU (SM100)", Step 3): closed forms for
    powers of two, code range [224, 448], norm_const shifts, zero blocks and
    half-step reconstruction.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W


def _srelu_case(m=256, n=64, k=128, s=32.0, seed=0, L=2, sizes=(256, 0)):
    off = np.cumsum(sizes).astype(np.int32)
    p = W.grouped_srelu_problem(0, L, n, k, "e4m3", seed=seed, offsets=off)
    r = O.grouped_srelu(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], p.t["offsets"],
                        p.t["alpha"], p.t["prob"], p.sizes["m"], n, k, L, "e4m3", s)
    return p, r


def test_srelu_relu_and_prob_zeroes():
    p, r = _srelu_case(s=0.0)
    c, d = r["c"], r["d"]
    assert np.all(d[c <= 0] == 0.0)
    prob = p.t["prob"].double().numpy()
    pos = c > 0
    np.testing.assert_allclose(d[pos], (prob[:, None] * c ** 2)[pos], rtol=4e-16, atol=0)
    assert np.all(d[prob == 0.0] == 0.0)


def test_srelu_clamp_bound_and_unclamped_limit():
    p, r = _srelu_case(s=0.5)           # tight clamp: many saturate
    prob = p.t["prob"].double().numpy()[:, None]
    assert np.all(r["d"] <= 0.25 * prob * (1 + 1e-15))
    _, r_big = _srelu_case(s=1e30)
    _, r_none = _srelu_case(s=0.0)
    np.testing.assert_allclose(r_big["d"], r_none["d"], rtol=1e-14, atol=0)


def test_srelu_tanh_closed_form_and_saturation():
    # one-hot A, unit scales, B codes chosen so C = alpha * v; pick alpha so
    # relu(C)/s = ln(2)/2 -> tanh = 1/3 exactly in reals -> D = prob * (s/3)^2.
    n, k, s = 8, 32, 4.0
    A = torch.zeros(256, k, dtype=torch.uint8); A[:, 0] = 0x38          # 1.0
    B = torch.zeros(1, n, k, dtype=torch.uint8); B[0, :, 0] = 0x38
    sfa = torch.full((W.sf_atom_bytes(256, k, 1),), 127, dtype=torch.uint8)
    sfb = torch.full((W.sf_atom_bytes(n, k, 1),), 127, dtype=torch.uint8)
    off = np.array([256], np.int32)
    prob = np.full(256, 0.75, np.float32)
    alpha = np.array([np.float32(s * math.log(2) / 2)], np.float32)
    r = O.grouped_srelu(A, B, sfa, sfb, off, alpha, prob, 256, n, k, 1, "e4m3", s)
    x = float(alpha[0]) / s                       # alpha rounded to fp32
    want = 0.75 * (s * (math.exp(2 * x) - 1) / (math.exp(2 * x) + 1)) ** 2
    np.testing.assert_allclose(r["d"], want, rtol=1e-14)
    np.testing.assert_allclose(want, 0.75 * (s / 3) ** 2, rtol=1e-6)
    # saturation: C >> s gives D == s^2 prob
    alpha = np.array([1e4], np.float32)
    r = O.grouped_srelu(A, B, sfa, sfb, off, alpha, prob, 256, n, k, 1, "e4m3", s)
    assert np.all(r["d"] == 0.75 * s * s)


def test_bf16_grouped_matches_numpy_per_expert_and_bias_branches():
    sizes = np.array([256, 0, 512, 256])
    off = np.cumsum(sizes).astype(np.int32)
    n, k, L = 48, 96, 4
    p = W.grouped_bf16_problem(0, L, n, k, seed=1, offsets=off, extra_rows=32)
    m = p.sizes["m"]
    a_bits, b_bits = O.bits16(p.t["a"]), O.bits16(p.t["b"])
    a = p.t["a"].double().numpy(); b = p.t["b"].double().numpy()
    alpha = p.t["alpha"].numpy(); prob = p.t["prob"].double().numpy()
    bias = p.t["bias"].double().numpy()                     # (L, N)
    rb = O.grouped_bf16(a_bits, b_bits, off, alpha, p.t["prob"], bias, m, n, k, L)
    rn = O.grouped_bf16(a_bits, b_bits, off, alpha, p.t["prob"], None, m, n, k, L)
    rz = O.grouped_bf16(a_bits, b_bits, off, alpha, p.t["prob"], np.zeros_like(bias), m, n, k, L)
    begin = 0
    for g in range(L):
        rows = slice(begin, off[g]); begin = off[g]
        G = float(alpha[g]) * (a[rows] @ b[g].T)
        np.testing.assert_allclose(rn["c"][rows], G, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(rn["d"][rows], prob[rows, None] * G, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(rb["c"][rows], G + prob[rows, None] * bias[g][None, :],
                                   rtol=1e-12, atol=1e-12)
    assert np.array_equal(rb["c"], rb["d"], equal_nan=True)
    # literal asymmetry: zero bias -> D == C == G; no bias -> D == prob * G
    assert np.array_equal(rz["d"], rn["c"], equal_nan=True)
    assert np.all(np.isnan(rn["c"][off[-1]:]))


def _rope_case(cos_val=None, sin_val=None, tokens=8, q_lora=64, heads=3, w_out_in=True):
    p = W.proj_rope_problem(tokens, q_lora, heads, 192, 64, seed=2, w_out_in=w_out_in)
    if cos_val is not None:
        p.t["cos"] = torch.full_like(p.t["cos"], cos_val)
        p.t["sin"] = torch.full_like(p.t["sin"], sin_val)
    y, s = O.proj_rope(O.bits16(p.t["x"]), O.bits16(p.t["w"]), O.bits16(p.t["cos"]),
                       O.bits16(p.t["sin"]), tokens, q_lora, heads, 192, 64, int(w_out_in))
    w = p.t["w"].double().numpy()
    plain = p.t["x"].double().numpy() @ (w.T if w_out_in else w)
    return y, plain


def test_rope_identity_is_deinterleave():
    y, plain = _rope_case(1.0, 0.0)
    y = y.reshape(8, 3, 192); plain = plain.reshape(8, 3, 192)
    np.testing.assert_allclose(y[..., :128], plain[..., :128], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y[..., 128:160], plain[..., 128::2], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y[..., 160:], plain[..., 129::2], rtol=1e-13, atol=1e-13)


def test_rope_quarter_turn():
    y, plain = _rope_case(0.0, 1.0)
    y = y.reshape(8, 3, 192); plain = plain.reshape(8, 3, 192)
    np.testing.assert_allclose(y[..., 128:160], -plain[..., 129::2], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y[..., 160:], plain[..., 128::2], rtol=1e-13, atol=1e-13)


def test_rope_weight_layouts_agree_and_norm_preserved_at_angle0():
    y1, _ = _rope_case(w_out_in=True)
    y0, _ = _rope_case(w_out_in=False)
    assert np.array_equal(y1, y0)
    # position 0 has angle 0 in the generated tables: cos = 1, sin = 0
    cos, sin = W.rope_tables(4)
    assert torch.all(cos[0] == 1) and torch.all(sin[0] == 0)


def test_rope_tables_by_column_and_absolute_row():
    """Every rotary output against the complex product (a_j + i b_j) e^(i theta)
    of the plain projection's pair (2j, 2j+1), with theta from the test's own
    angle array: the real part (output j) takes table column j, the imaginary
    part (output 32 + j) column 32 + j, and rows [t0, t1) read table row t, not
    t - t0.  The angles are independent per column and per row, so reading
    column j where 32 + j is meant, one fixed column, or a row relative to t0
    changes the result."""
    tokens, q_lora, heads, t0 = 12, 64, 2, 5
    p = W.proj_rope_problem(tokens, q_lora, heads, 192, 64, seed=11)
    cos, sin, ang = W.rope_tables_random(tokens, 64, seed=12)
    assert not np.array_equal(ang[:, :32], ang[:, 32:])
    y, _ = O.proj_rope(O.bits16(p.t["x"]), O.bits16(p.t["w"]), O.bits16(cos), O.bits16(sin),
                       tokens, q_lora, heads, 192, 64, 1, t0, tokens)
    plain = p.t["x"].double().numpy() @ p.t["w"].double().numpy().T
    plain = plain.reshape(tokens, heads, 192)[t0:]
    y = y.reshape(tokens - t0, heads, 192)
    # the table entries the kernel sees are the bf16 values of cos/sin theta
    e = (cos.double().numpy() + 1j * sin.double().numpy())[t0:, None, :]   # (rows, 1, 64)
    z = plain[..., 128::2] + 1j * plain[..., 129::2]                        # (rows, heads, 32)
    np.testing.assert_allclose(y[..., 128:160], (z * e[..., :32]).real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[..., 160:], (z * e[..., 32:]).imag, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[..., :128], plain[..., :128], rtol=1e-13, atol=1e-13)
    # the angles themselves: within bf16 rounding of cos/sin, the same products
    ez = np.exp(1j * ang)[t0:, None, :]
    np.testing.assert_allclose(y[..., 128:160], (z * ez[..., :32]).real, atol=2 ** -7 * np.abs(z).max())
    np.testing.assert_allclose(y[..., 160:], (z * ez[..., 32:]).imag, atol=2 ** -7 * np.abs(z).max())


def test_rope_standard_tables_rotate_pairs_by_the_position_angle():
    """With equal halves (the generated tables) each output pair (j, 32 + j) is
    the rotation of (a_j, b_j) by theta = t * 10000^(-j/32): its norm is kept
    to bf16 accuracy of cos/sin, and it matches (a + i b) e^(i theta)."""
    tokens, q_lora, heads = 64, 64, 2
    p = W.proj_rope_problem(tokens, q_lora, heads, 192, 64, seed=13)
    y, _ = O.proj_rope(O.bits16(p.t["x"]), O.bits16(p.t["w"]), O.bits16(p.t["cos"]),
                       O.bits16(p.t["sin"]), tokens, q_lora, heads, 192, 64, 1)
    plain = (p.t["x"].double().numpy() @ p.t["w"].double().numpy().T).reshape(tokens, heads, 192)
    y = y.reshape(tokens, heads, 192)
    theta = np.arange(tokens)[:, None] * 10000.0 ** (-np.arange(32) / 32.0)
    z = plain[..., 128::2] + 1j * plain[..., 129::2]
    rot = z * np.exp(1j * theta)[:, None, :]
    out = y[..., 128:160] + 1j * y[..., 160:]
    tol = 2 ** -7 * np.abs(z)
    assert np.all(np.abs(out - rot) <= tol + 1e-12)
    assert np.all(np.abs(np.abs(out) - np.abs(z)) <= tol + 1e-12)


def test_quantiser_power_of_two_closed_forms():
    # block max exactly 448 * 2^j -> scale byte 127 + j and codes = RNE(D / 2^j)
    rng = np.random.default_rng(5)
    for j in (-20, -3, 0, 4, 30):
        blk = rng.uniform(-1, 1, 32) * 448 * 2.0 ** j
        blk[7] = 448 * 2.0 ** j
        codes, scales = O.mx_quant_rows(blk[None, :])
        assert scales[0, 0] == 127 + j
        assert codes[0, 7] == 0x7E
        for i in range(32):
            v = float(np.float32(blk[i])) / 2.0 ** j
            assert codes[0, i] == O.enc_e4m3(v)
    # one step above a power of two rounds the scale up
    blk = np.full(32, 448.0); blk[0] = 449.0
    _, sc = O.mx_quant_rows(blk[None, :])
    assert sc[0, 0] == 128


def test_quantiser_code_range_norm_const_and_zero_blocks():
    rng = np.random.default_rng(6)
    d = rng.standard_normal((64, 96)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    d[3, 32:64] = 0.0
    codes, scales = O.mx_quant_rows(d)
    vals = np.vectorize(O.dec_e4m3)(codes.astype(np.uint32))
    blkmax = np.abs(vals).reshape(64, 3, 32).max(-1)
    nz = np.abs(d).reshape(64, 3, 32).max(-1) > 0
    assert np.all((blkmax[nz] >= 224) & (blkmax[nz] <= 448))
    assert scales[3, 1] == 0 and np.all(codes[3, 32:64] == 0)
    # half-step reconstruction: |dec(code) * 2^(byte-127) - D| <= half an E4M3 step
    deq = vals * np.exp2(np.repeat(scales.astype(np.float64), 32, axis=1) - 127)
    f = np.abs(vals)
    step = np.where(f < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(f, 1e-300))) - 3))
    step *= np.exp2(np.repeat(scales.astype(np.float64), 32, axis=1) - 127)
    assert np.all(np.abs(deq - d.astype(np.float32)) <= 0.5 * step * (1 + 1e-6) + 1e-300)
    # norm_const = 2^j shifts every nonzero block's byte by j, codes unchanged
    for j in (-3, 5):
        c2, s2 = O.mx_quant_rows(d, norm_const=2.0 ** j)
        assert np.array_equal(c2, codes)
        assert np.array_equal(s2[nz].astype(int), scales[nz].astype(int) + j)


def test_quantiser_columns_equal_rows_of_transpose():
    rng = np.random.default_rng(8)
    d = rng.standard_normal((96, 40)) * 3
    cc, cs = O.mx_quant_cols(d)
    rc, rs = O.mx_quant_rows(np.ascontiguousarray(d.T))
    assert np.array_equal(cc, rc.T) and np.array_equal(cs, rs.T)


def test_quantiser_e5m2_power_of_two_closed_forms():
    # E5M2 codes: block max exactly 57344 * 2^j -> scale byte 127 + j, that
    # element encodes to the top finite code 0x7B, the rest to RNE(D / 2^j).
    rng = np.random.default_rng(15)
    for j in (-30, -2, 0, 3, 20):
        blk = rng.uniform(-1, 1, 32) * 57344 * 2.0 ** j
        blk[11] = 57344 * 2.0 ** j
        codes, scales = O.mx_quant_rows(blk[None, :], fmt="e5m2")
        assert scales[0, 0] == 127 + j
        assert codes[0, 11] == 0x7B
        for i in range(32):
            v = float(np.float32(blk[i])) / 2.0 ** j
            assert codes[0, i] == O.enc_e5m2(v)
    # the same block quantised as E4M3 uses a scale 7 binades larger (448 = 1.75 * 2^8
    # against 57344 = 1.75 * 2^15)
    blk = rng.standard_normal(32) * 10.0
    _, s4 = O.mx_quant_rows(blk[None, :])
    _, s5 = O.mx_quant_rows(blk[None, :], fmt="e5m2")
    assert int(s4[0, 0]) - int(s5[0, 0]) == 7
    # columns agree with rows of the transpose in E5M2 too
    d = rng.standard_normal((64, 40))
    cr, sr = O.mx_quant_cols(d, fmt="e5m2")
    ct, st = O.mx_quant_rows(np.ascontiguousarray(d.T), fmt="e5m2")
    assert np.array_equal(cr, ct.T) and np.array_equal(sr, st.T)


def test_quantiser_e2m1_power_of_two_closed_forms():
    # E2M1 codes (rcp_max 1/6): block max exactly 6 * 2^j -> scale byte 127 + j,
    # that element encodes to the top code 7, the rest to RNE(D / 2^j).
    rng = np.random.default_rng(16)
    for j in (-40, -1, 0, 2, 25):
        blk = rng.uniform(-1, 1, 32) * 6 * 2.0 ** j
        blk[5] = -6 * 2.0 ** j
        codes, scales = O.mx_quant_rows(blk[None, :], fmt="e2m1")
        assert scales[0, 0] == 127 + j
        assert codes[0, 5] == 0xF
        for i in range(32):
            v = float(np.float32(blk[i])) / 2.0 ** j
            assert codes[0, i] == O.enc_e2m1(v)
    # just above 6 * 2^j the scale rounds up and no code saturates
    blk = np.full(32, 6.0); blk[0] = 6.5
    c, sc = O.mx_quant_rows(blk[None, :], fmt="e2m1")
    assert sc[0, 0] == 128 and c[0, 0] == O.enc_e2m1(3.25) and c[0, 1] == O.enc_e2m1(3.0)
    # dequantised codes stay within half a code step of the value: steps are
    # 0.5 below 2, 1 in [2, 4) and 2 in [4, 6] (in units of the block scale)
    d = rng.standard_normal((32, 64)) * np.exp(rng.uniform(-5, 5, (32, 1)))
    c, sc = O.mx_quant_rows(d, fmt="e2m1")
    sf = 2.0 ** (np.repeat(sc.astype(float), 32, 1) - 127)
    y = np.abs(d) / sf
    assert np.all(y <= 6.0)                        # the round-up scale leaves nothing to saturate
    half = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    deq = np.vectorize(O.dec_e2m1)(c.astype(np.uint32)) * sf
    assert np.all(np.abs(deq - d) <= half * sf)
    # columns agree with rows of the transpose
    cr, sr = O.mx_quant_cols(d, fmt="e2m1")
    ct, st = O.mx_quant_rows(np.ascontiguousarray(d.T), fmt="e2m1")
    assert np.array_equal(cr, ct.T) and np.array_equal(sr, st.T)
