"""Pins of the oracle's block-scaled contraction, amax and expert routing.

"GEMM + Amax (SM100)", Equations: C = sum_k A_hat B_hat, Amax = max |C|.
"Grouped GEMM + sReLU (SM100)" / "Grouped GEMM (SM100 BF16)", Operation:
rows [begin_g, padded_offsets[g]) belong to expert g.

Independent references used here: torch's float8_e4m3fn / float8_e8m0fnu
decoders, the OCP E2M1 table, numpy's float64 matmul and searchsorted,
exact rational arithmetic (fractions.Fraction), and closed forms.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1_TABLE = np.array([float(l.split()[1]) for l in open(os.path.join(GOLDEN, "e2m1_values.txt"))
                       if l.strip() and not l.startswith("#")])


def torch_dec_e4m3(codes: torch.Tensor) -> np.ndarray:
    return codes.contiguous().view(torch.float8_e4m3fn).double().numpy()


def torch_dec_e2m1_packed(codes: torch.Tensor) -> np.ndarray:
    c = codes.numpy()
    lo, hi = E2M1_TABLE[c & 15], E2M1_TABLE[c >> 4]
    return np.stack([lo, hi], axis=-1).reshape(*c.shape[:-1], c.shape[-1] * 2)


def physical_sf_index(mn, k, l):
    """Logical (row, kblock, l) -> byte index via the page's permutation statement."""
    mnt, kbl = -(-mn // 128), -(-k // 32)
    kt = -(-kbl // 4)
    phys = np.arange(l * mnt * kt * 512).reshape(l, mnt, kt, 32, 4, 4)
    lg = phys.transpose(3, 4, 1, 5, 2, 0)
    r = np.arange(mnt * 128)
    kb = np.arange(kt * 4)
    return lg[(r % 32)[:, None, None], ((r % 128) // 32)[:, None, None], (r // 128)[:, None, None],
              (kb % 4)[None, :, None], (kb // 4)[None, :, None], np.arange(l)[None, None, :]]


def unit_scale_problem(m, n, k, l, fmt="e4m3", seed=0):
    p = W.gemm_amax_problem(m, n, k, l, fmt, seed=seed, plain_round=(fmt == "e4m3"))
    p.t["sfa"][:] = 127
    p.t["sfb"][:] = 127
    return p


@pytest.mark.parametrize("m,n,k,l", [(256, 256, 256, 1), (130, 70, 96, 2), (1, 1, 32, 1)])
def test_unit_scales_equal_plain_fp64_gemm(m, n, k, l):
    # The page's own example passes all-ones E8M0 scales; then the op is a plain
    # GEMM of the decoded codes.  E4M3 products have <= 8 significant bits and
    # these sums stay inside fp64's 53, so both sides are exact: bit equality.
    p = unit_scale_problem(m, n, k, l)
    a = torch_dec_e4m3(p.t["a"]); b = torch_dec_e4m3(p.t["b"])
    c, s, amax = O.gemm_amax_full(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], m, n, k, l, "e4m3")
    for li in range(l):
        ref = a[li] @ b[li].T
        assert np.array_equal(c[li], ref)
        assert np.array_equal(s[li], np.abs(a[li]) @ np.abs(b[li]).T)
    assert amax == np.abs(np.stack([a[i] @ b[i].T for i in range(l)])).max()


def test_unit_scales_e5m2_equal_fp64_gemm():
    # E5M2 operands (float8_e5m2 on the page): with unit scales the op is a
    # plain GEMM of the codes decoded by torch; products have <= 6 significant
    # bits, so the fp64 sums agree to rounding of a few units in 2^-53.
    m, n, k, l = 96, 80, 256, 2
    p = W.gemm_amax_problem(m, n, k, l, "e5m2", seed=4)
    p.t["sfa"][:] = 127
    p.t["sfb"][:] = 127
    a = p.t["a"].view(torch.float8_e5m2).double().numpy()
    b = p.t["b"].view(torch.float8_e5m2).double().numpy()
    c, s, amax = O.gemm_amax_full(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], m, n, k, l, "e5m2")
    for li in range(l):
        np.testing.assert_allclose(c[li], a[li] @ b[li].T, rtol=1e-13, atol=0)
        np.testing.assert_allclose(s[li], np.abs(a[li]) @ np.abs(b[li]).T, rtol=1e-13, atol=0)


def test_e5m2_pow2_rescale_is_exact():
    m, n, k, l = 64, 48, 128, 1
    p = W.gemm_amax_problem(m, n, k, l, "e5m2", seed=5)
    c0 = O.gemm_amax_full(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], m, n, k, l, "e5m2")[0]
    p.t["sfb"] = (p.t["sfb"].int() + 3).to(torch.uint8)
    c1 = O.gemm_amax_full(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], m, n, k, l, "e5m2")[0]
    assert np.array_equal(c1, 8.0 * c0)


def test_unit_scales_fp4_and_nibble_order():
    m, n, k = 64, 48, 64
    p = unit_scale_problem(m, n, k, 1, fmt="e2m1", seed=5)
    a = torch_dec_e2m1_packed(p.t["a"][0]); b = torch_dec_e2m1_packed(p.t["b"][0])
    c, _ = O.gemm_amax(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], m, n, k, 1, "e2m1")
    assert np.array_equal(c, a @ b.T)
    # element 2j sits in the low nibble: a one-hot A at K=1 (byte 0, high nibble)
    A = torch.zeros(1, 1, k // 2, dtype=torch.uint8); A[0, 0, 0] = 0x20     # k=1 -> 1.0
    B = torch.zeros(1, 1, k // 2, dtype=torch.uint8); B[0, 0, 0] = 0x40 | 0x07  # k=0 -> 6, k=1 -> 2
    sf = torch.full((W.sf_atom_bytes(1, k, 1),), 127, dtype=torch.uint8)
    c, _ = O.gemm_amax(A, B, sf, sf, 1, 1, k, 1, "e2m1")
    assert c[0, 0] == 2.0


def test_pow2_rescale_is_exact():
    p = W.gemm_amax_problem(160, 96, 128, 2, "e4m3", seed=2)
    base, _, _ = O.gemm_amax_full(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], 160, 96, 128, 2, "e4m3")
    for ja, jb in [(1, 0), (-2, 3), (5, -5)]:
        sfa = (p.t["sfa"].int() + ja).to(torch.uint8)
        sfb = (p.t["sfb"].int() + jb).to(torch.uint8)
        c, _, _ = O.gemm_amax_full(p.t["a"], p.t["b"], sfa, sfb, 160, 96, 128, 2, "e4m3")
        assert np.array_equal(c, base * 2.0 ** (ja + jb))


def test_single_scale_byte_scales_one_row_and_block():
    # Bumping the byte that the page's permutation assigns to (row r, k-block kb)
    # adds exactly that block's contribution once more to row r and nothing else.
    m, n, k, l = 256, 64, 256, 2
    p = W.gemm_amax_problem(m, n, k, l, "e4m3", seed=3)
    p.t["sfb"][:] = 127
    a = torch_dec_e4m3(p.t["a"]); b = torch_dec_e4m3(p.t["b"])
    idx = physical_sf_index(m, k, l)
    base, _, _ = O.gemm_amax_full(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], m, n, k, l, "e4m3")
    rng = np.random.default_rng(0)
    for _ in range(12):
        r, kb, li = int(rng.integers(m)), int(rng.integers(k // 32)), int(rng.integers(l))
        sfa = p.t["sfa"].clone()
        off = int(idx[r, kb, li])
        old = int(sfa[off])
        sfa[off] = old + 1
        c, _, _ = O.gemm_amax_full(p.t["a"], p.t["b"], sfa, p.t["sfb"], m, n, k, l, "e4m3")
        delta = c - base
        blk = slice(32 * kb, 32 * kb + 32)
        want = np.zeros_like(delta)
        want[li, r] = 2.0 ** (old - 127) * (a[li, r, blk] @ b[li, :, blk].T)
        assert np.array_equal(delta, want)


def test_all_code_pairs_one_hot_exact_products():
    # 256 x 256 E4M3 code pairs: one-hot K puts code i of A against code j of B,
    # so C[i, j] = dec(i) dec(j) 2^(sa_i + sb_j - 254), checked in exact rationals.
    k = 32
    A = torch.zeros(1, 256, k, dtype=torch.uint8); A[0, :, 7] = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    B = torch.zeros(1, 256, k, dtype=torch.uint8); B[0, :, 7] = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    g = torch.Generator().manual_seed(9)
    sfa = torch.randint(120, 135, (W.sf_atom_bytes(256, k, 1),), generator=g).to(torch.uint8)
    sfb = torch.randint(120, 135, (W.sf_atom_bytes(256, k, 1),), generator=g).to(torch.uint8)
    c, _ = O.gemm_amax(A, B, sfa, sfb, 256, 256, k, 1, "e4m3")
    idx = physical_sf_index(256, k, 1)
    dec = torch_dec_e4m3(torch.arange(256, dtype=torch.int32).to(torch.uint8))
    for i in range(0, 256, 3):
        for j in range(256):
            if np.isnan(dec[i]) or np.isnan(dec[j]):
                assert np.isnan(c[i, j]); continue
            sa = int(sfa[int(idx[i, 0, 0])]) - 127
            sb = int(sfb[int(idx[j, 0, 0])]) - 127
            want = Fraction(dec[i]) * Fraction(dec[j]) * Fraction(2) ** (sa + sb)
            assert Fraction(c[i, j]) == want


def test_all_fp4_code_pairs():
    k = 64
    codes = torch.arange(16, dtype=torch.int32).to(torch.uint8)
    A = torch.zeros(1, 16, k // 2, dtype=torch.uint8); A[0, :, 3] = codes << 4      # element 7
    B = torch.zeros(1, 16, k // 2, dtype=torch.uint8); B[0, :, 3] = codes << 4
    sf = torch.full((W.sf_atom_bytes(16, k, 1),), 127, dtype=torch.uint8)
    c, _ = O.gemm_amax(A, B, sf, sf, 16, 16, k, 1, "e2m1")
    assert np.array_equal(c, np.outer(E2M1_TABLE, E2M1_TABLE))


def test_cancellation_and_all_ones():
    k = 128
    A = torch.zeros(1, 4, k, dtype=torch.uint8)
    x = torch.randint(0, 0x7E, (k // 2,), generator=torch.Generator().manual_seed(4)).to(torch.uint8)
    A[0, 0, 0::2] = x; A[0, 0, 1::2] = x | 0x80            # pairs (v, -v): C row 0 == 0
    A[0, 1, :] = 0x38                                        # all 1.0
    B = torch.full((1, 4, k), 0x38, dtype=torch.uint8)
    sfa = torch.full((W.sf_atom_bytes(4, k, 1),), 129, dtype=torch.uint8)   # 2^2
    sfb = torch.full((W.sf_atom_bytes(4, k, 1),), 124, dtype=torch.uint8)   # 2^-3
    c, _ = O.gemm_amax(A, B, sfa, sfb, 4, 4, k, 1, "e4m3")
    assert np.all(c[0] == 0.0)
    assert np.all(c[1] == k * 2.0 ** (2 - 3))


def test_routing_matches_searchsorted():
    rng = np.random.default_rng(11)
    for trial in range(20):
        L = int(rng.integers(1, 40))
        sizes = rng.integers(0, 4, L) * 256
        if trial % 3 == 0:
            sizes[rng.integers(L)] = 0
        off = np.cumsum(sizes).astype(np.int32)
        total = int(off[-1])
        for r in range(0, total + 300, 37):
            want = int(np.searchsorted(off, r, side="right"))
            want = want if r < total else -1
            assert O.expert_of_row(off, L, r) == want


def test_grouped_routing_constant_experts():
    # Unit scales, one-hot A, expert g's B codes all equal to the integer g%8+1:
    # C[m, n] = alpha_g * (g(m)%8 + 1), with g(m) from numpy's searchsorted.
    L, n, k = 10, 32, 64
    sizes = np.array([256, 0, 512, 256, 0, 0, 256, 768, 256, 0])
    off = np.cumsum(sizes).astype(np.int32)
    m = int(off[-1]) + 64
    A = torch.zeros(m, k, dtype=torch.uint8); A[:, 5] = 0x38
    ints = torch.tensor([1.0, 2, 3, 4, 5, 6, 7, 8]).to(torch.float8_e4m3fn).view(torch.uint8)
    B = torch.stack([torch.full((n, k), int(ints[g % 8]), dtype=torch.uint8) for g in range(L)])
    sfa = torch.full((W.sf_atom_bytes(m, k, 1),), 127, dtype=torch.uint8)
    sfb = torch.full((W.sf_atom_bytes(n, k, L),), 127, dtype=torch.uint8)
    alpha = np.linspace(0.5, 1.5, L).astype(np.float32)
    prob = np.ones(m, dtype=np.float32)
    r = O.grouped_srelu(A, B, sfa, sfb, off, alpha, prob, m, n, k, L, "e4m3", 0.0)
    g = np.searchsorted(off, np.arange(m), side="right")
    valid = np.arange(m) < off[-1]
    assert np.array_equal(r["group"][valid], g[valid]) and np.all(r["group"][~valid] == -1)
    want = (alpha[g[valid]].astype(np.float64) * (g[valid] % 8 + 1))[:, None]
    assert np.array_equal(r["c"][valid], np.broadcast_to(want, (valid.sum(), n)))
    assert np.all(np.isnan(r["c"][~valid]))
    amax = O.expert_amax(r["d"], r["group"], L)
    for e in range(L):
        assert amax[e] == (0.0 if sizes[e] == 0 else (float(alpha[e]) * (e % 8 + 1)) ** 2)


def test_grouped_single_expert_reduces_to_dense():
    p = W.gemm_amax_problem(256, 64, 96, 1, "e4m3", seed=7)
    dense, sab = O.gemm_amax(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], 256, 64, 96, 1, "e4m3")
    off = np.array([256], dtype=np.int32)
    r = O.grouped_srelu(p.t["a"][0], p.t["b"], p.t["sfa"], p.t["sfb"], off,
                        np.array([1.0], np.float32), np.ones(256, np.float32),
                        256, 64, 96, 1, "e4m3", 0.0)
    assert np.array_equal(r["c"], dense)
    assert np.array_equal(r["d"], np.maximum(dense, 0) ** 2)
    assert np.array_equal(r["sabs"], sab)


def test_block_max_statistic_matches_numpy():
    # Bmax (error-bound statistic) = sum over 32-wide K blocks of max |A_hat B_hat|
    p = unit_scale_problem(64, 40, 96, 1, seed=8)
    a = torch_dec_e4m3(p.t["a"])[0]; b = torch_dec_e4m3(p.t["b"])[0]
    c, s, bm = O.gemm_amax(p.t["a"], p.t["b"], p.t["sfa"], p.t["sfb"], 64, 40, 96, 1, "e4m3",
                           want_bmax=True)
    prod = np.abs(a[:, None, :] * b[None, :, :]).reshape(64, 40, 3, 32)
    assert np.array_equal(bm, prod.max(-1).sum(-1))
