"""GPU parity of the discrete-weight forms ("Grouped GEMM (SM100 BF16)",
discrete mode; "Grouped GEMM + sReLU (SM100)", Discrete-weight wrapper):
expert g's B (and SFB) are separate allocations passed as an (L,) int64
device array of addresses.  The math is the dense call's, so the oracle is
called on the stacked tensors, and the discrete outputs must also equal the
dense call's outputs bit for bit."""
import numpy as np
import pytest
import torch

import block_scaled_gemm_02_amd as bsg
import oracle as O
import workloads as W
from parity import check_float, check_mx_outputs, ceil_div, d_bound, gather_scales, sf_slice, sum_bound

pytestmark = pytest.mark.gpu
SENT = -1536.0


def say(msg):
    print(msg, flush=True)


def scattered_copies(parts):
    """Copies of `parts` in separate allocations, made in reverse order with
    spacers in between, so that no address is base + g * stride."""
    out = [None] * len(parts)
    keep = []
    for g in reversed(range(len(parts))):
        keep.append(torch.empty(4096 + 512 * g, dtype=torch.uint8, device="cuda"))
        out[g] = parts[g].clone().cuda()
    return out, keep


def discrete_weights(t, n, k_t, n_t, L, scaled):
    bs, keep_b = scattered_copies([t["b"][g] for g in range(L)])
    b_ptrs = bsg.pointer_array(bs)
    sfbs = sfb_ptrs = keep_s = None
    if scaled:
        sfbs, keep_s = scattered_copies([sf_slice(t["sfb"], g, n_t, k_t, 0, n_t) for g in range(L)])
        sfb_ptrs = bsg.pointer_array(sfbs)
    return b_ptrs, sfb_ptrs, (bs, sfbs, keep_b, keep_s)


def srelu_call(t, s, b_ptrs, sfb_ptrs, c_dtype, d_dtype, fp8):
    m, n, k, L = s["m"], s["n"], s["k"], s["l"]
    c = torch.full((m, n), SENT, dtype=c_dtype, device="cuda")
    if fp8:
        d = torch.full((m, n), 0xEE, dtype=torch.uint8, device="cuda")
        d_col = torch.full((m, n), 0xEE, dtype=torch.uint8, device="cuda")
        sfd_row = torch.full((W.sf_atom_bytes(m, n, 1),), 0xEE, dtype=torch.uint8, device="cuda")
        sfd_col = torch.full((W.sf_atom_bytes(n, m, 1),), 0xEE, dtype=torch.uint8, device="cuda")
        amax, nc, dd = None, torch.ones(1, device="cuda"), "e4m3"
    else:
        d = torch.full((m, n), SENT, dtype=d_dtype, device="cuda")
        d_col = sfd_row = sfd_col = None
        amax, nc, dd = torch.full((L,), -1.0, device="cuda"), None, d_dtype
    args = (c, d, d_col, sfd_row, sfd_col, amax, m, n, k, L, s["fmt"])
    kw = dict(c_dtype=c_dtype, d_dtype=dd, tanh_clamp_scale=s["tanh_clamp"])
    if b_ptrs is None:
        bsg.grouped_gemm_srelu(t["a"], t["b"], t["sfa"], t["sfb"], t["offsets"], t["alpha"], t["prob"],
                               nc, *args, **kw)
    else:
        bsg.grouped_gemm_srelu_discrete(t["a"], b_ptrs, t["sfa"], sfb_ptrs, t["offsets"], t["alpha"],
                                        t["prob"], nc, *args, **kw)
    torch.cuda.synchronize()
    return [x for x in (c, d, d_col, sfd_row, sfd_col, amax) if x is not None]


SRELU_CASES = [
    dict(sizes=[256, 0, 512, 256], n=320, k=192, fmt="e4m3", s=32.0, c=torch.bfloat16, d=torch.bfloat16),
    dict(sizes=[0, 256, 256, 0], n=288, k=256, fmt="e2m1", s=0.0, c=torch.float32, d=torch.float32),
    dict(sizes=[512, 0, 256], n=256, k=512, fmt="e4m3", s=0.5, c=torch.bfloat16, d="e4m3"),
]


@pytest.mark.parametrize("case", SRELU_CASES)
def test_srelu_discrete_matches_oracle_and_dense(case):
    say(f"grouped_srelu discrete {case}")
    off = np.cumsum(case["sizes"]).astype(np.int32)
    L = len(case["sizes"])
    fp8 = case["d"] == "e4m3"
    p = W.grouped_srelu_problem(0, L, case["n"], case["k"], case["fmt"], seed=5, offsets=off,
                                tanh_clamp=case["s"], extra_rows=256, d_dtype="e4m3" if fp8 else "bf16")
    s = p.sizes
    t = {kk: (v.cuda() if isinstance(v, torch.Tensor) else v) for kk, v in p.t.items()}
    m, n, k = s["m"], s["n"], s["k"]
    b_ptrs, sfb_ptrs, keep = discrete_weights(t, n, ceil_div(k, 128), ceil_div(n, 128), L, True)
    got = srelu_call(t, s, b_ptrs, sfb_ptrs, case["c"], None if fp8 else case["d"], fp8)
    ref = srelu_call(t, s, None, None, case["c"], None if fp8 else case["d"], fp8)
    for x, y in zip(got, ref):
        assert torch.equal(x, y)
    # and C and D against the oracle
    r = O.grouped_srelu(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], off, p.t["alpha"], p.t["prob"],
                        m, n, k, L, s["fmt"], s["tanh_clamp"])
    valid = s["valid_m"]
    bc = sum_bound(r["sabs"], k, bmax=r["bmax"])
    say(f"  C {check_float(got[0][:valid].cpu(), r['c'][:valid], bc[:valid], what='C')}")
    bd = d_bound(r["c"], bc, p.t["prob"].double().numpy(), s["tanh_clamp"])[:valid]
    if fp8:
        rs, cs = gather_scales(got[3], got[4], 0, valid, m, n)
        res = check_mx_outputs(r["d"][:valid], bd, got[1][:valid].cpu().numpy(), rs,
                               got[2][:valid].cpu().numpy(), cs, 1.0, what="D")
        say(f"  D {res}")
    else:
        say(f"  D {check_float(got[1][:valid].cpu(), r['d'][:valid], bd, what='D')}")
    del keep


BF16_CASES = [
    dict(sizes=[256, 0, 512, 256], n=264, k=200, bias=torch.bfloat16),
    dict(sizes=[256, 256, 0], n=128, k=64, bias=None),
]


@pytest.mark.parametrize("case", BF16_CASES)
def test_bf16_discrete_matches_oracle_and_dense(case):
    say(f"grouped_gemm discrete {case}")
    off = np.cumsum(case["sizes"]).astype(np.int32)
    L = len(case["sizes"])
    p = W.grouped_bf16_problem(0, L, case["n"], case["k"], seed=6, offsets=off, extra_rows=256,
                               with_bias=case["bias"] is not None)
    s = p.sizes
    m, n, k = s["m"], s["n"], s["k"]
    t = {kk: (v.cuda() if isinstance(v, torch.Tensor) else v) for kk, v in p.t.items()}
    bias = t["bias"].to(case["bias"]) if case["bias"] is not None else None
    b_ptrs, _, keep = discrete_weights(t, n, 0, 0, L, False)
    outs = []
    for discrete in (True, False):
        c = torch.full((m, n), SENT, dtype=torch.bfloat16, device="cuda")
        d = torch.full((m, n), SENT, dtype=torch.bfloat16, device="cuda")
        if discrete:
            bsg.grouped_gemm_discrete(t["a"], b_ptrs, t["offsets"], t["alpha"], t["prob"], bias, c, d,
                                      m, n, k, L, bias_dtype=case["bias"] or torch.bfloat16)
        else:
            bsg.grouped_gemm(t["a"], t["b"], t["offsets"], t["alpha"], t["prob"], bias, c, d, m, n, k, L,
                             bias_dtype=case["bias"] or torch.bfloat16)
        torch.cuda.synchronize()
        outs.append((c, d))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    bias_v = None if bias is None else bias.double().cpu().numpy()
    r = O.grouped_bf16(O.bits16(p.t["a"]), O.bits16(p.t["b"]), off, p.t["alpha"], p.t["prob"],
                       bias_v, m, n, k, L)
    valid = s["valid_m"]
    bnd = sum_bound(r["sabs"], k) + 1e-7 * np.abs(r["c"])
    say(f"  C {check_float(outs[0][0][:valid].cpu(), r['c'][:valid], bnd[:valid], what='C')}")
    dbnd = bnd * (1 if bias is not None else p.t["prob"].double().numpy()[:, None])
    say(f"  D {check_float(outs[0][1][:valid].cpu(), r['d'][:valid], dbnd[:valid], what='D')}")
    del keep


def test_srelu_discrete_full_size_equals_dense():
    """The grouped MXFP8 + sReLU workload (32 experts, N=4096, K=7168) with
    per-expert weight allocations: identical outputs to the dense call, and
    the first 256-row tile of the most popular expert against the oracle."""
    say("grouped_srelu discrete full size")
    p = W.moe_mxfp8_srelu(device="cuda")
    s = p.sizes
    t = p.t
    n, k, L = s["n"], s["k"], s["l"]
    b_ptrs, sfb_ptrs, keep = discrete_weights(t, n, ceil_div(k, 128), ceil_div(n, 128), L, True)
    got = srelu_call(t, s, b_ptrs, sfb_ptrs, torch.bfloat16, torch.bfloat16, False)
    ref = srelu_call(t, s, None, None, torch.bfloat16, torch.bfloat16, False)
    for x, y in zip(got, ref):
        assert torch.equal(x, y)
    m = s["m"]
    m_t, n_t, k_t = ceil_div(m, 128), ceil_div(n, 128), ceil_div(k, 128)
    say("  oracle expert 0 rows 0..255")
    sub = O.grouped_srelu(t["a"][:256].cpu(), t["b"][0:1].cpu(), sf_slice(t["sfa"], 0, m_t, k_t, 0, 2).cpu(),
                          sf_slice(t["sfb"], 0, n_t, k_t, 0, n_t).cpu(), np.array([256], np.int32),
                          t["alpha"][0:1].cpu(), t["prob"][:256].cpu(), 256, n, k, 1, "e4m3", 32.0)
    bc = sum_bound(sub["sabs"], k, bmax=sub["bmax"])
    bd = d_bound(sub["c"], bc, t["prob"][:256].double().cpu().numpy(), 32.0)
    say(f"  C {check_float(got[0][:256].cpu(), sub['c'], bc, what='C')}")
    say(f"  D {check_float(got[1][:256].cpu(), sub['d'], bd, what='D')}")
    del keep
