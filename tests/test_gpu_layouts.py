"""GPU parity of the operand and output majors of gemm_amax ("GEMM + Amax
(SM100)", Input/Output tensors: A m-major with stride (1, M, M*K), B n-major
with stride (1, N, N*K), C m-major with stride (1, M, M*N); Layouts and
strides: packed FP4 A/B stay k-major).

The majors only move data: the GEMM of the transposed storage is the same
GEMM.  Every case is checked against the CPU oracle (which takes the k-major
operands) and, bit for bit, against the library's own k-major call on the
same values.  All calls go through the C ABI via the thin binding.
"""
import numpy as np
import pytest
import torch

import block_scaled_gemm_02_amd as bsg
import oracle as O
import workloads as W
from parity import check_amax, check_float, sum_bound

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def mn_major(x, l, rows, k):
    """[L][rows][K] codes -> the same codes stored [L][K][rows]."""
    return x.reshape(l, rows, k).transpose(1, 2).contiguous()


def run(t, s, c_dtype, a_major="k", b_major="k", c_major="n"):
    """gemm_amax with the given majors; returns C as (L, M, N) and amax."""
    l, m, n, k = s["l"], s["m"], s["n"], s["k"]
    a = mn_major(t["a"], l, m, k) if a_major == "m" else t["a"]
    b = mn_major(t["b"], l, n, k) if b_major == "n" else t["b"]
    shape = (l, m, n) if c_major == "n" else (l, n, m)
    c = torch.full(shape, 7.0, dtype=c_dtype, device="cuda")
    amax = torch.full((1,), -7.0, device="cuda")
    bsg.gemm_amax(a, b, t["sfa"], t["sfb"], c, amax, m, n, k, l, s["fmt"], c_dtype=c_dtype,
                  a_major=a_major, b_major=b_major, c_major=c_major)
    torch.cuda.synchronize()
    if c_major == "m":
        c = c.transpose(1, 2)
    return c.contiguous(), amax


CASES = [
    dict(m=272, n=400, k=320, l=2, fmt="e4m3", c=torch.float32, maj="mkn"),   # ragged M/N, K tail
    dict(m=272, n=400, k=320, l=2, fmt="e4m3", c=torch.bfloat16, maj="knn"),
    dict(m=528, n=304, k=640, l=1, fmt="e5m2", c=torch.float32, maj="mnn"),
    dict(m=256, n=256, k=256, l=1, fmt="e4m3", c=torch.float32, maj="kkm"),   # m-major C only
    dict(m=272, n=400, k=96, l=2, fmt="e4m3", c=torch.float16, maj="mnm"),
    dict(m=16, n=48, k=32, l=3, fmt="e5m2", c=torch.bfloat16, maj="mnn"),     # one K block, tiny tiles
    dict(m=512, n=768, k=1024, l=1, fmt="e4m3", c=torch.bfloat16, maj="mnn"),  # several whole tiles
    dict(m=260, n=136, k=352, l=2, fmt="e2m1", c=torch.float32, maj="kkm"),   # FP4: C major only
    dict(m=304, n=208, k=256, l=2, fmt="e5m2", c=torch.float16, maj="kkm"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c['fmt']}-{c['maj']}-{c['m']}x{c['n']}x{c['k']}x{c['l']}")
def test_gemm_amax_majors_match_oracle_and_k_major(case):
    say(f"gemm_amax majors {case}")
    p = W.gemm_amax_problem(case["m"], case["n"], case["k"], case["l"], case["fmt"], seed=11)
    s = p.sizes
    t = {k: v.cuda() for k, v in p.t.items()}
    am, bm, cm = case["maj"]
    c, amax = run(t, s, case["c"], am, bm, cm)
    c_ref, amax_ref = run(t, s, case["c"])
    oc, os_, oamax, obm = O.gemm_amax_full(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], s["m"], s["n"],
                                           s["k"], s["l"], s["fmt"], want_bmax=True)
    bound = sum_bound(os_, s["k"], bmax=obm)
    r = check_float(c.cpu(), oc, bound, what=str(case))
    say(f"  oracle: {r}")
    check_amax(float(amax.item()), oamax, float(bound.ravel()[np.argmax(np.abs(oc))]))
    # the same sums as the k-major call, in the same order
    assert torch.equal(c, c_ref), "differs from the k-major result"
    assert amax.item() == amax_ref.item()


def test_gemm_amax_mn_major_writes_only_c():
    """Ragged M/N with m-major A and n-major B: the padding a tile reads past
    M (N) in each K row is the next K row's data, which must not reach C or
    amax; rows of C past the output are never written."""
    say("gemm_amax majors: ragged isolation")
    m, n, k, l = 48, 80, 256, 3
    p = W.gemm_amax_problem(m, n, k, l, "e4m3", seed=12)
    s = p.sizes
    t = {kk: v.cuda() for kk, v in p.t.items()}
    # C inside a larger buffer whose guard band must stay untouched
    buf = torch.full((l * m * n + 4096,), 3.5, device="cuda")
    a = mn_major(t["a"], l, m, k)
    b = mn_major(t["b"], l, n, k)
    amax = torch.zeros(1, device="cuda")
    bsg.gemm_amax(a, b, t["sfa"], t["sfb"], buf, amax, m, n, k, l, "e4m3", c_dtype=torch.float32,
                  a_major="m", b_major="n")
    torch.cuda.synchronize()
    assert torch.all(buf[l * m * n:] == 3.5)
    c = buf[:l * m * n].reshape(l, m, n)
    c_ref, amax_ref = run(t, s, torch.float32)
    assert torch.equal(c, c_ref)
    assert amax.item() == amax_ref.item() == c.abs().max().item()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_gemm_amax_majors_full_size_bit_exact(fmt):
    """M=N=K=8192, L=1 (one batch of the dense benchmark shape): every
    combination of majors gives the k-major result bit for bit; a sampled
    128-row panel of it is checked against the oracle."""
    say(f"gemm_amax majors 8192^3 {fmt}")
    m = n = k = 8192
    l = 1
    p = W.gemm_amax_problem(m, n, k, l, fmt, seed=13, device="cuda")
    s = p.sizes
    t = p.t
    c_ref, amax_ref = run(t, s, torch.bfloat16)
    for maj in ("mkn", "knn", "mnn", "mnm"):
        say(f"  majors {maj}")
        c, amax = run(t, s, torch.bfloat16, *maj)
        assert torch.equal(c, c_ref), maj
        assert amax.item() == amax_ref.item(), maj
        del c
    from parity import ceil_div, sf_slice
    m_t, k_t = ceil_div(m, 128), ceil_div(k, 128)
    mt = 37
    a_sub = t["a"][0, mt * 128:(mt + 1) * 128].cpu()
    oc, os_, obm = O.gemm_amax(a_sub, t["b"][0].cpu(), sf_slice(t["sfa"], 0, m_t, k_t, mt, mt + 1).cpu(),
                               sf_slice(t["sfb"], 0, m_t, k_t, 0, m_t).cpu(), 128, n, k, 1, fmt, want_bmax=True)
    r = check_float(c_ref[0, mt * 128:(mt + 1) * 128].cpu(), oc, sum_bound(os_, k, bmax=obm), what=fmt)
    say(f"  oracle panel: {r}")
