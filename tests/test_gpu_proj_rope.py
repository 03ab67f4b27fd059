"""GPU parity of gemm_proj_rope_mxfp8 ("GEMM + RoPE + MXFP8 Projection
(SM100)") against the CPU oracle, through the C ABI."""
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
    bsg.gemm_proj_rope_mxfp8(t["x"], t["w"], None, None, t["cos"], t["sin"], qr, sr, qc, sc,
                             T, s["q_lora"], H, D, s["qk_rope"], w_out_in=s["w_out_in"])
    torch.cuda.synchronize()
    return qr, sr, qc, sc


def oracle_check(p, qr, sr, qc, sc, t0, t1, what):
    s = p.sizes
    T, H, D = s["tokens"], s["heads"], s["head_dim"]
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


def test_proj_rope_full_size_sampled():
    """x (4096,1536), 128 heads x 192: sampled 128-token panels vs the oracle."""
    say("proj_rope full size")
    p = W.proj_rope_dsv3(device="cuda")
    qr, sr, qc, sc = run_proj(p)
    p.t = {k: v.cpu() for k, v in p.t.items()}
    for t0 in (0, 3968):
        say(f"  oracle tokens {t0}..{t0 + 127}")
        oracle_check(p, qr, sr, qc, sc, t0, t0 + 128, f"tokens {t0}")
