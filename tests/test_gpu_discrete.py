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
from parity import check_float, ceil_div, sf_slice, sum_bound

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
    # and C against the oracle
    r = O.grouped_srelu(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], off, p.t["alpha"], p.t["prob"],
                        m, n, k, L, s["fmt"], s["tanh_clamp"])
    valid = s["valid_m"]
    bc = sum_bound(r["sabs"], k, bmax=r["bmax"])
    say(f"  C {check_float(got[0][:valid].cpu(), r['c'][:valid], bc[:valid], what='C')}")
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
    del keep


def test_srelu_discrete_full_size_equals_dense():
    """The grouped MXFP8 + sReLU workload (32 experts, N=4096, K=7168) with
    per-expert weight allocations: identical outputs to the dense call, whose
    parity with the oracle the sampled full-size test checks."""
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
    del keep
