"""GPU parity of grouped_gemm_dswiglu ("Grouped GEMM + dSwiGLU (SM100)")
against the CPU oracle, through the C ABI: MXFP8 D (row and column
quantisation with their scale atoms) and dprob."""
import numpy as np
import pytest
import torch

import block_scaled_gemm_02_amd as bsg
import oracle as O
import workloads as W
from parity import U, ceil_div, check_float, check_mx_outputs, sum_bound

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def run_dswiglu(p, d_fmt="e4m3", b_major="k"):
    s = p.sizes
    t = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in p.t.items()}
    m, n, k, L = s["m"], s["n"], s["k"], s["l"]
    if b_major == "n":
        # the same codes stored [L][K][N] (stride (1, N, N*K))
        t["b"] = t["b"].reshape(L, n, k).transpose(1, 2).contiguous()
    d = torch.full((m, 2 * n), 0xEE, dtype=torch.uint8, device="cuda")
    d_col = torch.full((m, 2 * n), 0xEE, dtype=torch.uint8, device="cuda")
    sfd_row = torch.full((W.sf_atom_bytes(m, 2 * n, 1),), 0xEE, dtype=torch.uint8, device="cuda")
    sfd_col = torch.full((W.sf_atom_bytes(2 * n, m, 1),), 0xEE, dtype=torch.uint8, device="cuda")
    dprob = torch.zeros(m, device="cuda")
    bsg.grouped_gemm_dswiglu(t["a"], t["b"], t["sfa"], t["sfb"], t["c"], t["offsets"], t["alpha"], t["beta"],
                             t["prob"], t["norm_const"], d, d_col, sfd_row, sfd_col, dprob, m, n, k, L,
                             s["fmt"], d_dtype=d_fmt, b_major=b_major)
    torch.cuda.synchronize()
    return d, d_col, sfd_row, sfd_col, dprob


def gather_scales(sfd_row, sfd_col, r0, r1, m, n2):
    row_idx = O.sf_offset_grid(r0, r1, n2 // 32, 0, m, n2 // 32)
    col_idx = O.sf_offset_grid(0, n2, ceil_div(r1, 32), 0, n2, m // 32)[:, r0 // 32:]
    return sfd_row.cpu().numpy()[row_idx], sfd_col.cpu().numpy()[col_idx].T


def bounds(p, r, r0, r1):
    """Error bounds of D and dprob for rows [r0, r1) (the rows of oracle result
    r) from the bound of ref (fp32 accumulation and the scaled MFMA's per-block
    truncation) and the epilogue's fp32 arithmetic."""
    s = p.sizes
    n, k = s["n"], s["k"]
    off = p.t["offsets"].cpu().numpy()
    grp = np.searchsorted(off, np.arange(r0, r1), side="right")
    beta = p.t["beta"].cpu().double().numpy()[grp][:, None]
    c = p.t["c"][r0:r1].cpu().double().numpy()
    cols = np.arange(n) // 32 * 64 + np.arange(n) % 32
    x_in, x_gt = beta * c[:, cols], beta * c[:, cols + 32]
    sg = 1.0 / (1.0 + np.exp(-x_gt))
    sw = x_gt * sg
    prob = p.t["prob"][r0:r1].cpu().double().numpy()[:, None]
    ref = r["ref"]
    bref = sum_bound(r["sabs"], k, bmax=r["bmax"])
    d = r["d"]
    b_ab = np.abs(prob * sw) * bref + 1e-5 * np.abs(d[:, cols]) + 1e-6 * np.abs(ref * prob) * (1 + np.abs(x_gt))
    g_ds = np.abs(prob * x_in * sg * (1 + x_gt * (1 - sg)))
    b_ds = g_ds * bref + 1e-5 * np.abs(d[:, cols + 32]) + 1e-6 * np.abs(ref * prob * x_in) * (1 + np.abs(x_gt))
    bd = np.empty_like(d)
    bd[:, cols], bd[:, cols + 32] = b_ab, b_ds
    terms = np.abs(sw * x_in)
    b_dp = (terms * bref).sum(1) + (1e-5 + 2 * 2 * n * U) * (terms * np.abs(ref)).sum(1)
    return bd, b_dp


CASES = [
    dict(sizes=[256, 0, 512], n=160, k=256, fmt="e4m3"),       # ragged last n-tile (32 columns)
    dict(sizes=[512, 256], n=256, k=384, fmt="e5m2"),
    dict(sizes=[1024, 512, 0, 768, 256], n=512, k=1024, fmt="e4m3"),
    # E5M2 D codes (rcp_max 1/57344)
    dict(sizes=[256, 0, 512], n=160, k=256, fmt="e4m3", d="e5m2"),
    dict(sizes=[512, 256], n=256, k=384, fmt="e5m2", d="e5m2"),
    # norm_const that is not a power of two (the kernel carries it inside the
    # values and divides by the E8M0 scale alone)
    dict(sizes=[256, 0, 512], n=160, k=256, fmt="e4m3", nc=0.37),
    dict(sizes=[512, 256], n=256, k=384, fmt="e4m3", d="e5m2", nc=3.0),
]


@pytest.mark.parametrize("case", CASES)
def test_grouped_dswiglu_matches_oracle(case):
    say(f"grouped_dswiglu parity {case}")
    off = np.cumsum(case["sizes"]).astype(np.int32)
    L = len(case["sizes"])
    p = W.grouped_dswiglu_problem(0, L, case["n"], case["k"], case["fmt"], seed=6, offsets=off, extra_rows=256)
    nc = case.get("nc", 1.0)
    p.t["norm_const"] = torch.full((1,), nc)
    s = p.sizes
    m, n, k = s["m"], s["n"], s["k"]
    d_fmt = case.get("d", "e4m3")
    d, d_col, sfd_row, sfd_col, dprob = run_dswiglu(p, d_fmt)
    valid = s["valid_m"]
    r = O.grouped_dswiglu(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], off, p.t["alpha"], p.t["beta"],
                          p.t["prob"], O.bits16(p.t["c"]), m, n, k, L, case["fmt"], 0, valid)
    bd, b_dp = bounds(p, r, 0, valid)
    rs, cs = gather_scales(sfd_row, sfd_col, 0, valid, m, 2 * n)
    res = check_mx_outputs(r["d"], bd, d[:valid].cpu().numpy(), rs, d_col[:valid].cpu().numpy(), cs, nc,
                           what="D", fmt=d_fmt)
    say(f"  {res}")
    g = dprob[:valid].cpu().double().numpy()
    err = np.abs(g - r["dprob"])
    assert np.all(err <= b_dp), f"dprob: worst {float((err / np.maximum(b_dp, 1e-300)).max())} of its bound"
    say(f"  dprob: max err / bound {float((err / np.maximum(b_dp, 1e-300)).max()):.3g}")
    # rows at or past valid_m are not written; dprob there stays as the caller left it
    assert torch.all(d[valid:] == 0xEE) and torch.all(d_col[valid:] == 0xEE)
    assert torch.all(dprob[valid:] == 0)


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[4]])
def test_grouped_dswiglu_n_major_b(case):
    """B stored n-major ("Grouped GEMM + dSwiGLU (SM100)", Input/Output
    tensors: B stride (1, N, N*K) for FP8 inputs): D codes and both scale
    arrays equal the k-major call's bit for bit; dprob (atomic adds, whose
    order varies) is checked against the oracle."""
    say(f"grouped_dswiglu n-major B {case}")
    off = np.cumsum(case["sizes"]).astype(np.int32)
    L = len(case["sizes"])
    p = W.grouped_dswiglu_problem(0, L, case["n"], case["k"], case["fmt"], seed=7, offsets=off, extra_rows=256)
    s = p.sizes
    m, n, k = s["m"], s["n"], s["k"]
    d_fmt = case.get("d", "e4m3")
    ref = run_dswiglu(p, d_fmt)
    got = run_dswiglu(p, d_fmt, b_major="n")
    for name, x, y in zip(("d", "d_col", "sfd_row", "sfd_col"), got[:4], ref[:4]):
        assert torch.equal(x, y), name
    valid = s["valid_m"]
    r = O.grouped_dswiglu(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], off, p.t["alpha"], p.t["beta"],
                          p.t["prob"], O.bits16(p.t["c"]), m, n, k, L, case["fmt"], 0, valid)
    _, b_dp = bounds(p, r, 0, valid)
    err = np.abs(got[4][:valid].cpu().double().numpy() - r["dprob"])
    assert np.all(err <= b_dp), f"dprob: worst {float((err / np.maximum(b_dp, 1e-300)).max())} of its bound"
    assert torch.all(got[4][valid:] == 0)


FP4_CASES = [
    dict(sizes=[256, 0, 512], n=160, k=256, d=torch.bfloat16),
    dict(sizes=[512, 256, 256], n=256, k=512, d=torch.float32),
]


@pytest.mark.parametrize("case", FP4_CASES)
def test_grouped_dswiglu_fp4_inputs_bf16_or_f32_d_and_amax(case):
    """FP4 inputs: unquantised D (RNE cast), its optional copy D_col, and the
    per-expert amax (L, 2) of ab and dswiglu, against the oracle."""
    say(f"grouped_dswiglu FP4 inputs {case}")
    off = np.cumsum(case["sizes"]).astype(np.int32)
    L = len(case["sizes"])
    p = W.grouped_dswiglu_problem(0, L, case["n"], case["k"], "e2m1", seed=8, offsets=off, extra_rows=256)
    s = p.sizes
    m, n, k = s["m"], s["n"], s["k"]
    t = {kk: (v.cuda() if isinstance(v, torch.Tensor) else v) for kk, v in p.t.items()}
    sent = float("nan")
    d = torch.full((m, 2 * n), sent, dtype=case["d"], device="cuda")
    d_col = torch.full((m, 2 * n), sent, dtype=case["d"], device="cuda")
    dprob = torch.zeros(m, device="cuda")
    amax = torch.full((L, 2), -1.0, device="cuda")
    bsg.grouped_gemm_dswiglu(t["a"], t["b"], t["sfa"], t["sfb"], t["c"], t["offsets"], t["alpha"], t["beta"],
                             t["prob"], None, d, d_col, None, None, dprob, m, n, k, L, "e2m1",
                             d_dtype=case["d"], amax=amax)
    torch.cuda.synchronize()
    valid = s["valid_m"]
    r = O.grouped_dswiglu(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], off, p.t["alpha"], p.t["beta"],
                          p.t["prob"], O.bits16(p.t["c"]), m, n, k, L, "e2m1", 0, valid)
    bd, b_dp = bounds(p, r, 0, valid)
    res = check_float(d[:valid].cpu(), r["d"], bd, what="D")
    say(f"  D: {res}")
    assert torch.equal(d_col[:valid], d[:valid])
    g = dprob[:valid].cpu().double().numpy()
    assert np.all(np.abs(g - r["dprob"]) <= b_dp)
    # amax (L, 2): max |ab| and max |dswiglu| over each expert's rows, 0 for an empty expert
    grp = np.searchsorted(off, np.arange(valid), side="right")
    cols = np.arange(n) // 32 * 64 + np.arange(n) % 32
    ga = amax.cpu().double().numpy()
    for gi in range(L):
        sel = grp == gi
        for h, cc in ((0, cols), (1, cols + 32)):
            o = float(np.abs(r["d"][sel][:, cc]).max()) if sel.any() else 0.0
            bnd = float(bd[sel][:, cc].max()) if sel.any() else 0.0
            assert abs(ga[gi, h] - o) <= bnd + 1e-6 * o, (gi, h, ga[gi, h], o, bnd)
    assert torch.all(torch.isnan(d[valid:].float())) and torch.all(dprob[valid:] == 0)


@pytest.mark.parametrize("d_fmt", ["e4m3", "e5m2"])
def test_grouped_dswiglu_full_size_sampled(d_fmt):
    """The bench configuration (28672 tokens over 32 experts, Zipf(1.1)
    routing, N = 2048, K = 7168, MXFP8 D with E4M3 or E5M2 codes): the first
    whole 256-row tile (both wave rows) of three experts against the oracle
    computed for those rows alone (D codes and scale atoms in both
    directions, dprob)."""
    say(f"grouped_dswiglu full size, D {d_fmt}")
    p = W.grouped_dswiglu_problem(28672, 32, 2048, 7168, "e4m3", seed=0, device="cuda")
    s = p.sizes
    m, n, k, L = s["m"], s["n"], s["k"], s["l"]
    d, d_col, sfd_row, sfd_col, dprob = run_dswiglu(p, d_fmt)
    t = p.t
    off = t["offsets"].cpu().numpy()
    m_t, n_t, k_t = ceil_div(m, 128), ceil_div(n, 128), ceil_div(k, 128)
    begins = np.concatenate([[0], off[:-1]])
    nonempty = [g for g in range(L) if off[g] > begins[g]]
    for g in (nonempty[0], nonempty[len(nonempty) // 2], nonempty[-1]):
        r0 = int(begins[g])
        assert float(t["prob"][r0].item()) > 0.0           # a routed row
        say(f"  oracle expert {g} rows {r0}..{r0 + 255}")
        sfa = t["sfa"][(r0 // 128) * k_t * 512:(r0 // 128 + 2) * k_t * 512]
        sfb = t["sfb"][g * n_t * k_t * 512:(g + 1) * n_t * k_t * 512]
        r = O.grouped_dswiglu(t["a"][r0:r0 + 256].cpu(), t["b"][g:g + 1].cpu(), sfa.cpu(), sfb.cpu(),
                              np.array([256], np.int32), t["alpha"][g:g + 1].cpu(), t["beta"][g:g + 1].cpu(),
                              t["prob"][r0:r0 + 256].cpu(), O.bits16(t["c"][r0:r0 + 256].cpu()), 256, n, k, 1,
                              "e4m3")
        bd, b_dp = bounds(p, r, r0, r0 + 256)
        rs, cs = gather_scales(sfd_row, sfd_col, r0, r0 + 256, m, 2 * n)
        res = check_mx_outputs(r["d"], bd, d[r0:r0 + 256].cpu().numpy(), rs, d_col[r0:r0 + 256].cpu().numpy(),
                               cs, 1.0, what=f"D e{g}", fmt=d_fmt)
        say(f"  {res}")
        gdp = dprob[r0:r0 + 256].cpu().double().numpy()
        assert np.all(np.abs(gdp - r["dprob"]) <= b_dp)


def test_grouped_dswiglu_n_major_b_full_size():
    """The bench configuration with B stored n-major: D codes and both scale
    arrays equal the k-major call's bit for bit over the whole output."""
    say("grouped_dswiglu full size, n-major B")
    p = W.grouped_dswiglu_problem(28672, 32, 2048, 7168, "e4m3", seed=1, device="cuda")
    ref = run_dswiglu(p)
    got = run_dswiglu(p, b_major="n")
    for name, x, y in zip(("d", "d_col", "sfd_row", "sfd_col"), got[:4], ref[:4]):
        assert torch.equal(x, y), name
    # dprob: the same per-row terms, added in a varying order
    assert torch.allclose(got[4], ref[4], rtol=1e-5, atol=1e-6 * float(ref[4].abs().max()))


def test_grouped_dswiglu_fp4_full_size_sampled():
    """The MXFP4 bench configuration (28672 tokens over 32 experts, N = 2048,
    K = 7168, bf16 D with its D_col copy and the per-expert amax (L, 2)): the
    first whole 256-row tile of three experts against the oracle computed for
    those rows alone; over the whole output, D_col equals D and each amax
    rounded to bf16 equals the largest |D| of its expert and half (RNE is
    monotonic, so the bf16 maximum is the rounded fp32 maximum)."""
    say("grouped_dswiglu FP4 inputs, full size")
    p = W.grouped_dswiglu_problem(28672, 32, 2048, 7168, "e2m1", seed=0, device="cuda")
    s, t = p.sizes, p.t
    m, n, k, L = s["m"], s["n"], s["k"], s["l"]
    d = torch.full((m, 2 * n), float("nan"), dtype=torch.bfloat16, device="cuda")
    d_col = torch.full((m, 2 * n), float("nan"), dtype=torch.bfloat16, device="cuda")
    dprob = torch.zeros(m, device="cuda")
    amax = torch.full((L, 2), -1.0, device="cuda")
    bsg.grouped_gemm_dswiglu(t["a"], t["b"], t["sfa"], t["sfb"], t["c"], t["offsets"], t["alpha"], t["beta"],
                             t["prob"], None, d, d_col, None, None, dprob, m, n, k, L, "e2m1",
                             d_dtype=torch.bfloat16, amax=amax)
    torch.cuda.synchronize()
    valid = s["valid_m"]
    assert torch.equal(d_col[:valid], d[:valid])
    off = t["offsets"].cpu().numpy()
    begins = np.concatenate([[0], off[:-1]])
    cols = torch.arange(n, device="cuda") // 32 * 64 + torch.arange(n, device="cuda") % 32
    for g in range(L):
        for h, cc in ((0, cols), (1, cols + 32)):
            if off[g] > begins[g]:
                want = d[int(begins[g]):int(off[g])][:, cc].float().abs().max()
                got = amax[g, h].to(torch.bfloat16).float()
                assert got.item() == want.item(), (g, h, amax[g, h].item(), want.item())
            else:
                assert amax[g, h].item() == 0.0, (g, h)
    m_t, n_t, k_t = ceil_div(m, 128), ceil_div(n, 128), ceil_div(k, 128)
    nonempty = [g for g in range(L) if off[g] > begins[g]]
    for g in (nonempty[0], nonempty[len(nonempty) // 2], nonempty[-1]):
        r0 = int(begins[g])
        assert float(t["prob"][r0].item()) > 0.0           # a routed row
        say(f"  oracle expert {g} rows {r0}..{r0 + 255}")
        sfa = t["sfa"][(r0 // 128) * k_t * 512:(r0 // 128 + 2) * k_t * 512]
        sfb = t["sfb"][g * n_t * k_t * 512:(g + 1) * n_t * k_t * 512]
        r = O.grouped_dswiglu(t["a"][r0:r0 + 256].cpu(), t["b"][g:g + 1].cpu(), sfa.cpu(), sfb.cpu(),
                              np.array([256], np.int32), t["alpha"][g:g + 1].cpu(), t["beta"][g:g + 1].cpu(),
                              t["prob"][r0:r0 + 256].cpu(), O.bits16(t["c"][r0:r0 + 256].cpu()), 256, n, k, 1,
                              "e2m1")
        bd, b_dp = bounds(p, r, r0, r0 + 256)
        say(f"  D: {check_float(d[r0:r0 + 256].cpu(), r['d'], bd, what=f'D e{g}')}")
        gdp = dprob[r0:r0 + 256].cpu().double().numpy()
        assert np.all(np.abs(gdp - r["dprob"]) <= b_dp)
