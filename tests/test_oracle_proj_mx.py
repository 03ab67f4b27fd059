"""Pins of the oracle's MXFP8-input projection ("GEMM + RoPE + MXFP8
Projection (SM100)", Shapes: x and w as E4M3 codes with row-wise E8M0 block
scales, x_scale (tokens, Q_LORA/32), w_scale (out, Q_LORA/32) for the
[out, in] weight):

  * unit scales (every byte 127) reduce it to the BF16-input projection of
    the decoded codes, which bf16 holds exactly (E4M3 has a 3-bit mantissa and
    a narrower exponent range); the decode here is torch's float8_e4m3fn;
  * a +1 on every scale byte of token t doubles that token's outputs and
    nothing else; a +1 on the scale row of a weight row doubles its feature;
  * a +1 on the single byte x_scale[t, b] adds exactly the contribution of
    x[t, 32b:32b+32], i.e. the byte scales that block of that row only.
"""
import numpy as np
import torch

import oracle as O
import workloads as W

T, Q, H = 32, 256, 2


def _case(seed=0):
    p = W.proj_rope_problem(T, Q, H, 192, 64, seed=seed, in_dtype="e4m3")
    return {k: v.clone() for k, v in p.t.items()}


def _mx(t, t0=0, t1=None):
    return O.proj_rope_mx(t["x"], t["x_scale"], t["w"], t["w_scale"], O.bits16(t["cos"]),
                          O.bits16(t["sin"]), T, Q, H, 192, 64, t0=t0, t1=t1)[0]


def test_unit_scales_equal_bf16_projection_of_decoded_codes():
    t = _case(1)
    t["x_scale"].fill_(127)
    t["w_scale"].fill_(127)
    xb = t["x"].view(torch.float8_e4m3fn).to(torch.bfloat16)
    wb = t["w"].view(torch.float8_e4m3fn).to(torch.bfloat16)
    assert torch.equal(xb.float(), t["x"].view(torch.float8_e4m3fn).float())    # exact widening
    y_bf16, _ = O.proj_rope(O.bits16(xb), O.bits16(wb), O.bits16(t["cos"]), O.bits16(t["sin"]),
                            T, Q, H, 192, 64, 1)
    assert np.array_equal(_mx(t), y_bf16)


def test_token_and_feature_scale_rows_rescale_exactly():
    t = _case(2)
    y = _mx(t)
    t2 = {k: v.clone() for k, v in t.items()}
    t2["x_scale"][5] += 1
    y2 = _mx(t2)
    assert np.array_equal(y2[5], 2 * y[5])
    keep = np.arange(T) != 5
    assert np.array_equal(y2[keep], y[keep])
    # feature 17 of head 1 (pass-through part) is weight row 192 + 17
    t3 = {k: v.clone() for k, v in t.items()}
    t3["w_scale"][192 + 17] += 1
    y3 = _mx(t3)
    assert np.array_equal(y3[:, 192 + 17], 2 * y[:, 192 + 17])
    others = np.ones(H * 192, bool); others[192 + 17] = False
    assert np.array_equal(y3[:, others], y[:, others])


def test_single_scale_byte_scales_one_block_of_one_row():
    t = _case(3)
    tok, blk = 7, 3
    y = _mx(t)
    t2 = {k: v.clone() for k, v in t.items()}
    t2["x_scale"][tok, blk] += 1
    y2 = _mx(t2)
    # contribution of block blk of token tok alone: zero every other code of x
    t3 = {k: v.clone() for k, v in t.items()}
    only = torch.zeros_like(t3["x"])
    only[tok, 32 * blk:32 * blk + 32] = t3["x"][tok, 32 * blk:32 * blk + 32]
    t3["x"] = only
    yb = _mx(t3)
    np.testing.assert_allclose(y2[tok] - y[tok], yb[tok], rtol=1e-12, atol=1e-12)
    nope = np.concatenate([np.arange(h * 192, h * 192 + 128) for h in range(H)])
    assert np.array_equal((y2[tok] - y[tok])[nope], yb[tok][nope])
    keep = np.arange(T) != tok
    assert np.array_equal(y2[keep], y[keep])


def test_row_range_matches_full_run():
    t = _case(4)
    assert np.array_equal(_mx(t, 8, 16), _mx(t)[8:16])
