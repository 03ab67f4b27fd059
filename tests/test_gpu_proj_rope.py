"""GPU parity of gemm_proj_rope_mxfp8 ("GEMM + RoPE + MXFP8 Projection
(SM100)") against the CPU oracle, through the C ABI: BF16 inputs, and MXFP8
inputs (E4M3 codes with row-major E8M0 scales x_scale / w_scale)."""
import numpy as np
import pytest
import torch

import block_scaled_gemm_02_amd as bsg
import oracle as O
import workloads as W
from parity import check_mx_outputs, sum_bound

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def run_proj(p):
    s = p.sizes
    t = {k: v.cuda() for k, v in p.t.items()}
    T, H, D = s["tokens"], s["heads"], s["head_dim"]
    qr = torch.full((T, H, D), 0xEE, dtype=torch.uint8, device="cuda")
    qc = torch.full((T, H, D), 0xEE, dtype=torch.uint8, device="cuda")
    sr = torch.full((T, H, D // 32), 0xEE, dtype=torch.uint8, device="cuda")
    sc = torch.full((T // 32, H, D), 0xEE, dtype=torch.uint8, device="cuda")
    mx = s.get("in_dtype") == "e4m3"
    bsg.gemm_proj_rope_mxfp8(t["x"], t["w"], t.get("x_scale"), t.get("w_scale"), t["cos"], t["sin"],
                             qr, sr, qc, sc, T, s["q_lora"], H, D, s["qk_rope"],
                             in_dtype=bsg.E4M3 if mx else bsg.BF16, w_out_in=s["w_out_in"])
    torch.cuda.synchronize()
    return qr, sr, qc, sc


def w_out_in_view(p):
    """MXFP8 w and w_scale as [out, in] (the oracle's layout): transposed
    back when the problem stores them [in, out]."""
    if p.sizes["w_out_in"]:
        return p.t["w"], p.t["w_scale"]
    return p.t["w"].t().contiguous(), p.t["w_scale"].t().contiguous()


def mx_block_bound(p, t0, t1):
    """Upper bound of Bmax (sum over 32-wide K blocks of the largest |product|)
    for MXFP8 inputs: sum_b max|x^[t,b]| * max|w^[o,b]|, carried through the
    rotary mixing with |cos| and |sin| like the oracle's Sabs."""
    s = p.sizes
    H, D, Q = s["heads"], s["head_dim"], s["q_lora"]

    def dec(codes, scales):
        v = codes.view(torch.float8_e4m3fn).double().numpy()
        v = v.reshape(v.shape[0], Q // 32, 32)
        return np.abs(v).max(-1) * 2.0 ** (scales.numpy().astype(np.float64) - 127)

    w, ws = w_out_in_view(p)
    bx = dec(p.t["x"][t0:t1], p.t["x_scale"][t0:t1])
    bw = dec(w, ws)
    b = (bx @ bw.T).reshape(t1 - t0, H, D)
    cos = np.abs(p.t["cos"][t0:t1].double().numpy())[:, None, :]
    sin = np.abs(p.t["sin"][t0:t1].double().numpy())[:, None, :]
    ev, od = b[..., 128::2].copy(), b[..., 129::2].copy()
    b[..., 128:160] = cos[..., :32] * ev + sin[..., :32] * od
    b[..., 160:] = cos[..., 32:] * od + sin[..., 32:] * ev
    return b.reshape(t1 - t0, H * D)


def oracle_check(p, qr, sr, qc, sc, t0, t1, what):
    s = p.sizes
    T, H, D = s["tokens"], s["heads"], s["head_dim"]
    if s.get("in_dtype") == "e4m3":
        w, ws = w_out_in_view(p)
        y, sab = O.proj_rope_mx(p.t["x"], p.t["x_scale"], w, ws, O.bits16(p.t["cos"]),
                                O.bits16(p.t["sin"]), T, s["q_lora"], H, D, s["qk_rope"], t0, t1)
        bound = sum_bound(sab, s["q_lora"], bmax=mx_block_bound(p, t0, t1)) + 1e-6 * sab
    else:
        y, sab = O.proj_rope(O.bits16(p.t["x"]), O.bits16(p.t["w"]), O.bits16(p.t["cos"]),
                             O.bits16(p.t["sin"]), T, s["q_lora"], H, D, s["qk_rope"],
                             s["w_out_in"], t0, t1)
        bound = sum_bound(sab, s["q_lora"]) + 1e-6 * sab
    N = H * D
    res = check_mx_outputs(y, bound, qr[t0:t1].reshape(t1 - t0, N).cpu().numpy(),
                           sr[t0:t1].reshape(t1 - t0, N // 32).cpu().numpy(),
                           qc[t0:t1].reshape(t1 - t0, N).cpu().numpy(),
                           sc[t0 // 32:t1 // 32].reshape((t1 - t0) // 32, N).cpu().numpy(),
                           1.0, what=what)
    say(f"  {what}: {res}")


@pytest.mark.parametrize("case", [
    dict(tokens=256, q_lora=256, heads=3),
    dict(tokens=384, q_lora=96, heads=2),      # a 128-token tail tile
    dict(tokens=128, q_lora=1536, heads=1),
])
def test_proj_rope_matches_oracle(case):
    say(f"proj_rope parity {case}")
    p = W.proj_rope_problem(case["tokens"], case["q_lora"], case["heads"], seed=5)
    qr, sr, qc, sc = run_proj(p)
    oracle_check(p, qr, sr, qc, sc, 0, case["tokens"], str(case))


@pytest.mark.parametrize("cs", [(1.0, 0.0), (0.0, 1.0)])
def test_proj_rope_special_tables(cs):
    """cos=1/sin=0 is the pure de-interleave; cos=0/sin=1 gives [-b, a]."""
    say(f"proj_rope tables {cs}")
    p = W.proj_rope_problem(256, 128, 2, seed=6)
    p.t["cos"] = torch.full_like(p.t["cos"], cs[0])
    p.t["sin"] = torch.full_like(p.t["sin"], cs[1])
    qr, sr, qc, sc = run_proj(p)
    oracle_check(p, qr, sr, qc, sc, 0, 256, f"tables {cs}")


@pytest.mark.parametrize("in_dtype", ["bf16", "e4m3"])
def test_proj_rope_independent_angle_tables(in_dtype):
    """cos/sin from independent angles per (token, column): the two halves of
    a row differ and every row differs, so a kernel that read column j for
    output 32 + j, one fixed column, or a row relative to the tile would
    disagree with the oracle (whose column and row use is pinned on the CPU)."""
    say(f"proj_rope independent-angle tables ({in_dtype})")
    p = W.proj_rope_problem(384, 256 if in_dtype == "bf16" else 128, 2, seed=9, in_dtype=in_dtype)
    p.t["cos"], p.t["sin"], _ = W.rope_tables_random(384, 64, seed=10)
    qr, sr, qc, sc = run_proj(p)
    oracle_check(p, qr, sr, qc, sc, 0, 384, f"random tables {in_dtype}")


@pytest.mark.parametrize("case", [
    dict(tokens=256, q_lora=256, heads=3),
    dict(tokens=384, q_lora=96, heads=2),      # a 128-token tail tile, K = 96 (a partial pair)
    dict(tokens=128, q_lora=1536, heads=1),
])
def test_proj_rope_w_in_out_matches_oracle(case):
    """w as [in, out] (w_out_in = 0, "GEMM + RoPE + MXFP8 Projection (SM100)",
    Shapes: w is (Q_LORA, NUM_HEADS * HEAD_DIM)): the B tile is staged K-major
    and read with the transposing LDS reads."""
    say(f"proj_rope w [in, out] parity {case}")
    p = W.proj_rope_problem(case["tokens"], case["q_lora"], case["heads"], seed=11, w_out_in=False)
    assert p.t["w"].shape == (case["q_lora"], case["heads"] * 192)
    qr, sr, qc, sc = run_proj(p)
    oracle_check(p, qr, sr, qc, sc, 0, case["tokens"], "w_in_out " + str(case))


def test_proj_rope_w_layouts_agree_bit_for_bit():
    """The same weights as [out, in] and as [in, out] give identical outputs:
    both layouts feed the MFMA the same values in the same order."""
    say("proj_rope w layouts")
    p1 = W.proj_rope_problem(256, 512, 4, seed=12, w_out_in=True)
    p0 = W.proj_rope_problem(256, 512, 4, seed=12, w_out_in=True)
    p0.t["w"] = p1.t["w"].t().contiguous()
    p0.sizes["w_out_in"] = False
    p0.t["cos"], p0.t["sin"], _ = W.rope_tables_random(256, 64, seed=13)
    p1.t["cos"], p1.t["sin"] = p0.t["cos"], p0.t["sin"]
    a = run_proj(p1)
    b = run_proj(p0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    oracle_check(p0, *b, 0, 256, "w [in, out] random tables")


def test_proj_rope_w_in_out_full_size_sampled():
    """x (4096,1536), w (1536, 24576) as [in, out], 128 heads x 192: the first
    and last 128-token panels against the oracle."""
    say("proj_rope w [in, out] full size")
    p = W.proj_rope_problem(4096, 1536, 128, seed=0, device="cuda", w_out_in=False)
    qr, sr, qc, sc = run_proj(p)
    p.t = {k: v.cpu() for k, v in p.t.items()}
    for t0 in (0, 3968):
        say(f"  oracle tokens {t0}..{t0 + 127}")
        oracle_check(p, qr, sr, qc, sc, t0, t0 + 128, f"w_in_out tokens {t0}")


def test_proj_rope_full_size_sampled():
    """x (4096,1536), 128 heads x 192: sampled 128-token panels vs the oracle."""
    say("proj_rope full size")
    p = W.proj_rope_dsv3(device="cuda")
    qr, sr, qc, sc = run_proj(p)
    p.t = {k: v.cpu() for k, v in p.t.items()}
    for t0 in (0, 3968):
        say(f"  oracle tokens {t0}..{t0 + 127}")
        oracle_check(p, qr, sr, qc, sc, t0, t0 + 128, f"tokens {t0}")


@pytest.mark.parametrize("case", [
    dict(tokens=256, q_lora=256, heads=3),
    dict(tokens=384, q_lora=128, heads=2),     # a 128-token tail tile
    dict(tokens=128, q_lora=1536, heads=1),
])
def test_proj_rope_mxfp8_inputs_match_oracle(case):
    say(f"proj_rope MXFP8-input parity {case}")
    p = W.proj_rope_problem(case["tokens"], case["q_lora"], case["heads"], seed=7, in_dtype="e4m3")
    qr, sr, qc, sc = run_proj(p)
    oracle_check(p, qr, sr, qc, sc, 0, case["tokens"], "mx " + str(case))


def test_proj_rope_mxfp8_unit_scales_equal_bf16_path():
    """With every scale byte 127 the MXFP8-input call sees the same values as
    the BF16-input call on the decoded codes (exact in bf16)."""
    say("proj_rope MXFP8 unit scales vs BF16 path")
    p = W.proj_rope_problem(256, 256, 2, seed=8, in_dtype="e4m3")
    p.t["x_scale"].fill_(127)
    p.t["w_scale"].fill_(127)
    mx = run_proj(p)
    pb = W.proj_rope_problem(256, 256, 2, seed=8)
    pb.t["x"] = p.t["x"].view(torch.float8_e4m3fn).to(torch.bfloat16)
    pb.t["w"] = p.t["w"].view(torch.float8_e4m3fn).to(torch.bfloat16)
    pb.t["cos"], pb.t["sin"] = p.t["cos"], p.t["sin"]
    bf = run_proj(pb)
    oracle_check(p, *mx, 0, 256, "mx unit scales")
    oracle_check(pb, *bf, 0, 256, "bf16 of the same values")


def test_proj_rope_mxfp8_full_size_sampled():
    """MXFP8 x (4096,1536), w (24576,1536), 128 heads x 192: sampled panels vs the oracle."""
    say("proj_rope MXFP8 full size")
    p = W.proj_rope_dsv3(device="cuda", in_dtype="e4m3")
    qr, sr, qc, sc = run_proj(p)
    p.t = {k: v.cpu() for k, v in p.t.items()}
    for t0 in (0, 3968):
        say(f"  oracle tokens {t0}..{t0 + 127}")
        oracle_check(p, qr, sr, qc, sc, t0, t0 + 128, f"mx tokens {t0}")


@pytest.mark.parametrize("case", [
    dict(tokens=256, q_lora=256, heads=3),
    dict(tokens=384, q_lora=128, heads=2),     # a 128-token tail tile
    dict(tokens=128, q_lora=2048, heads=2),    # the largest q_lora of this path (64 scale bytes per feature)
])
def test_proj_rope_mxfp8_w_in_out_matches_oracle(case):
    """MXFP8 inputs with w and w_scale as [in, out] (w_out_in = 0, "GEMM +
    RoPE + MXFP8 Projection (SM100)", Shapes: w (Q_LORA, NUM_HEADS*HEAD_DIM),
    w_scale (Q_LORA/32, NUM_HEADS*HEAD_DIM)): codes staged K-major, the head's
    scale columns transposed into LDS."""
    say(f"proj_rope MXFP8 w [in, out] parity {case}")
    p = W.proj_rope_problem(case["tokens"], case["q_lora"], case["heads"], seed=14, in_dtype="e4m3",
                            w_out_in=False)
    assert p.t["w"].shape == (case["q_lora"], case["heads"] * 192)
    assert p.t["w_scale"].shape == (case["q_lora"] // 32, case["heads"] * 192)
    qr, sr, qc, sc = run_proj(p)
    oracle_check(p, qr, sr, qc, sc, 0, case["tokens"], "mx w_in_out " + str(case))


def test_proj_rope_mxfp8_w_layouts_agree_bit_for_bit():
    """The same MXFP8 codes and scales as [out, in] and as [in, out] give
    identical outputs."""
    say("proj_rope MXFP8 w layouts")
    p1 = W.proj_rope_problem(256, 1536, 4, seed=15, in_dtype="e4m3", w_out_in=True)
    p0 = W.proj_rope_problem(256, 1536, 4, seed=15, in_dtype="e4m3", w_out_in=True)
    p0.t["w"] = p1.t["w"].t().contiguous()
    p0.t["w_scale"] = p1.t["w_scale"].t().contiguous()
    p0.sizes["w_out_in"] = 0
    a = run_proj(p1)
    b = run_proj(p0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_proj_rope_mxfp8_w_in_out_full_size_sampled():
    """MXFP8 x (4096,1536), w (1536, 24576) and w_scale (48, 24576) as [in,
    out], 128 heads x 192: the first and last 128-token panels vs the oracle."""
    say("proj_rope MXFP8 w [in, out] full size")
    p = W.proj_rope_dsv3(device="cuda", in_dtype="e4m3", w_out_in=False)
    qr, sr, qc, sc = run_proj(p)
    p.t = {k: v.cpu() for k, v in p.t.items()}
    for t0 in (0, 3968):
        say(f"  oracle tokens {t0}..{t0 + 127}")
        oracle_check(p, qr, sr, qc, sc, t0, t0 + 128, f"mx w_in_out tokens {t0}")
