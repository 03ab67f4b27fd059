"""Comparison rules shared by the GPU parity tests.

Tolerances come from the stated targets: fp32 outputs within relative
1e-3, bf16/fp16 outputs within one step of the correctly rounded oracle
value, amax within relative 1e-5, quantised outputs with identical E8M0
scales and FP8 (E4M3 or E5M2) codes within one code step on at most 0.1% of elements.

Cancellation escape: where a sum nearly cancels, a relative test on the
result is meaningless.  An element that misses the relative rule passes if
its error is within the error bound of the GPU's summation (sum_bound), with
S = sum_k |A_hat B_hat| and Bmax from the oracle; escapes are counted and
capped (ESCAPE_CAP: 0.1% for bf16 outputs).  (The CDNA4 scaled MFMA adds
the products of each group of 8 consecutive K elements in a fixed point
whose last bit is 2^-13 of the group's largest product, dropping the bits
below it: measured bit for bit in test_gpu_mfma_precision.py.  A 32-element
scale block therefore loses less than 2^-8 of its largest product, and
near-cancelling outputs carry errors of that order.)

Quantised outputs: a code must lie inside the codes that the oracle value
plus or minus its error bound encodes to (under the same block scale);
codes that differ from the oracle's own code, by one step or more, count
together against the 0.1% budget.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O

U = 2.0 ** -24


def bits_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def ordered16(bits: np.ndarray) -> np.ndarray:
    """Sign-magnitude 16-bit patterns -> integers in value order."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def rne16(o: np.ndarray, kind: str) -> np.ndarray:
    if kind == "bf16":
        return O.rne_bf16_array(o)
    return np.asarray(o, dtype=np.float16).view(np.uint16)   # numpy casts with RNE


def ulp16(o: np.ndarray, kind: str) -> np.ndarray:
    mant = 7 if kind == "bf16" else 10
    e = np.floor(np.log2(np.maximum(np.abs(o), 1e-300)))
    return 2.0 ** (e - mant)


def sum_bound(sabs: np.ndarray, k: int, alpha=1.0, bmax=None) -> np.ndarray:
    """Error bound of the GPU's sum: fp32 accumulation 2*K*2^-24*|alpha|*S,
    plus, for the scaled FP8/FP4 MFMA, 2^-8 * Bmax where Bmax is the sum over
    32-wide K blocks of the block's largest |product| (each of a block's 32
    products loses less than 2^-13 of the block maximum in the instruction's
    fixed-point adder)."""
    b = 2.0 * k * U * np.abs(alpha) * sabs
    if bmax is not None:
        b = b + 2.0 ** -8 * np.abs(alpha) * bmax
    return b


# At most this fraction of a float output may pass by its error bound
# instead of the relative rule: 0.1% for bf16 outputs (one step is 2^-8
# relative).  The fp32 rule (relative 1e-3) and the fp16 rule (one step,
# 2^-11 relative) are 4 to 8 times finer, and on the small mixed-sign cases
# 0.30-0.65% of their elements are sums that cancel to below 1000 times the
# in-group truncation error of the scaled MFMA; every such element still
# lies inside its error bound.  For those outputs the cap is 1%.
ESCAPE_CAP = {torch.bfloat16: 1e-3, torch.float16: 1e-2, torch.float32: 1e-2}


def check_float(gpu: torch.Tensor, o: np.ndarray, bound: np.ndarray, what: str = "",
                max_escape_frac: float | None = None):
    """Elementwise check of a float output against oracle values `o` (fp64);
    `bound` is the per-element cancellation escape bound, which every element
    must meet; the count of elements that use it instead of the relative rule
    is capped (ESCAPE_CAP by output dtype, unless given).

    NaN positions in `o` (rows the oracle did not compute) are skipped."""
    if max_escape_frac is None:
        max_escape_frac = ESCAPE_CAP[gpu.dtype]
    mask = ~np.isnan(o)
    bound = np.where(mask, bound, 0.0)
    o = np.where(mask, o, 0.0)
    if gpu.dtype == torch.float32:
        g = gpu.detach().cpu().double().numpy()
        err = np.abs(g - o)
        strict = err <= 1e-3 * np.abs(o)
        escape = ~strict & (err <= bound)
    else:
        kind = "bf16" if gpu.dtype == torch.bfloat16 else "f16"
        gb = gpu.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        ob = rne16(o, kind)
        strict = np.abs(ordered16(gb) - ordered16(ob)) <= 1
        g = gpu.detach().float().cpu().double().numpy()
        err = np.abs(g - o)
        escape = ~strict & (err <= bound + ulp16(o, kind))
    fail = mask & ~strict & ~escape
    n = int(mask.sum())
    n_esc = int((mask & escape).sum())
    if fail.any():
        idx = np.argwhere(fail)[:5]
        detail = [(tuple(i), float(g[tuple(i)]), float(o[tuple(i)]), float(bound[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(fail.sum())}/{n} elements out of tolerance, e.g. {detail}")
    assert n_esc <= max(1, max_escape_frac * n), f"{what}: {n_esc}/{n} cancellation escapes"
    rel = err / np.maximum(bound, 1e-300)
    return dict(n=n, escapes=n_esc, max_err_over_bound=float(rel[mask].max(initial=0)))


def check_amax(gpu_val: float, o_val: float, bound: float = 0.0, what=""):
    """Relative 1e-5, or within the error bound of the oracle's arg-max element."""
    err = abs(gpu_val - o_val)
    assert err <= 1e-5 * abs(o_val) + 1e-30 or err <= bound, \
        f"{what}: amax {gpu_val} vs {o_val} (bound {bound})"


def e4m3_ordered(codes: np.ndarray) -> np.ndarray:
    c = codes.astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def e2m1_ordered(codes: np.ndarray) -> np.ndarray:
    """E2M1 nibbles (sign in bit 3) -> integers ordered like their values."""
    c = codes.astype(np.int64)
    return np.where(c & 8, -(c & 7), c & 7)


def ordered(codes: np.ndarray, fmt: str) -> np.ndarray:
    return e2m1_ordered(codes) if fmt == "e2m1" else e4m3_ordered(codes)


def unpack_e2m1(raw: np.ndarray) -> np.ndarray:
    """Bytes holding two E2M1 codes (even column in the low nibble) -> one
    nibble per element along the last axis."""
    out = np.empty(raw.shape[:-1] + (2 * raw.shape[-1],), dtype=np.uint8)
    out[..., 0::2], out[..., 1::2] = raw & 15, raw >> 4
    return out


def check_quant(gpu_codes: np.ndarray, gpu_scales: np.ndarray, o_codes: np.ndarray,
                o_scales: np.ndarray, sigma_near_pow2: np.ndarray | None = None, what="",
                max_flip_frac: float = 1e-3, window: tuple | None = None, fmt: str = "e4m3"):
    """Scales identical (except blocks flagged near a power-of-two boundary);
    codes equal to the oracle's, except on at most `max_flip_frac` of the
    elements.  A differing code must be one step off, or (`window` = the
    ordered codes (lo, hi) that the oracle value minus / plus its error
    bound encodes to) lie inside the window: a value that cancels to a small
    fraction of its error bound may legitimately move by more than one step.
    Both kinds count against the same budget."""
    sc_bad = gpu_scales != o_scales
    if sigma_near_pow2 is not None:
        sc_bad &= ~sigma_near_pow2
    assert not sc_bad.any(), f"{what}: {int(sc_bad.sum())} scale bytes differ"
    og = ordered(gpu_codes, fmt)
    d = np.abs(og - ordered(o_codes, fmt))
    far = d > 1
    if window is not None:
        lo, hi = window
        inside = (og >= lo) & (og <= hi)
    else:
        inside = np.zeros_like(far)
    assert not (far & ~inside).any(), \
        f"{what}: code differs by {d[far & ~inside].max()} steps, outside its error-bound window"
    n_esc = int(far.sum())
    flips = int((d == 1).sum())
    assert flips + n_esc <= max(1, max_flip_frac * d.size), \
        f"{what}: {flips} one-step flips + {n_esc} window codes of {d.size}"
    return dict(flips=flips, escapes=n_esc, n=int(d.size))


FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0, "e2m1": 6.0}
_TORCH_FP8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def code_window(d_o: np.ndarray, bound: np.ndarray, scales: np.ndarray, axis: int, norm_const=1.0,
                fmt: str = "e4m3"):
    """Ordered FP8 codes of d_o - bound and d_o + bound under the given E8M0
    block scales (blocks of 32 along `axis`): the codes a value within the
    error bound can take.  The encode is torch's float8_e4m3fn / float8_e5m2
    (RNE) after saturation to the format's largest finite value."""
    inv = norm_const * 2.0 ** (127.0 - np.repeat(scales.astype(np.float64), 32, axis=axis))
    fmax = FP8_MAX[fmt]

    def enc(v):
        v = np.clip(v * inv, -fmax, fmax).astype(np.float32)
        if fmt == "e2m1":   # no torch encode for E2M1: the oracle's (pinned) encoder
            return e2m1_ordered(np.vectorize(lambda x: O.enc_e2m1(float(x)), otypes=[np.uint32])(v))
        return e4m3_ordered(torch.from_numpy(v).to(_TORCH_FP8[fmt]).view(torch.uint8).numpy())

    return enc(d_o - bound), enc(d_o + bound)


def sf_slice(sf: torch.Tensor, l: int, mn_t: int, k_t: int, mt0: int, mt1: int) -> torch.Tensor:
    """Atom row-groups [mt0, mt1) of batch l from a (L, MN', K', 32, 4, 4) buffer."""
    start = ((l * mn_t + mt0) * k_t) * 512
    return sf[start:start + (mt1 - mt0) * k_t * 512]


def ceil_div(a, b):
    return -(-a // b)


def near_pow2_boundary(amax: np.ndarray, bound: np.ndarray, norm_const: float = 1.0,
                       fmax: float = 448.0) -> np.ndarray:
    """True where the E8M0 scale of a block whose true max is `amax` could
    legitimately differ: [amax - bound, amax + bound] straddles a threshold
    fmax * 2^k / norm_const of the quantiser's round-up (fmax = 448 for E4M3
    codes, 57344 for E5M2)."""
    lo = np.maximum(amax - bound, 0.0) * norm_const / fmax
    hi = (amax + bound) * norm_const / fmax
    with np.errstate(divide="ignore"):
        return (np.ceil(np.log2(np.maximum(lo, 1e-300))) != np.ceil(np.log2(np.maximum(hi, 1e-300)))) | (lo == 0)


def check_mx_outputs(d_o: np.ndarray, bound: np.ndarray, gpu_row_codes, gpu_row_scales,
                     gpu_col_codes, gpu_col_scales, norm_const=1.0, what="", fmt="e4m3"):
    """Dual-direction MX quantisation of oracle D (rows x cols, rows % 32 == 0)
    vs the GPU's codes / scales given in logical (row, block) order; fmt is
    the code format ("e4m3", "e5m2" or "e2m1", the last as one nibble per
    element).  Sign-magnitude codes of each format are ordered like their
    values, so one code step is one integer step."""
    rc, rs = O.mx_quant_rows(d_o, norm_const, fmt)
    cc, cs = O.mx_quant_cols(d_o, norm_const, fmt)
    fmax = FP8_MAX[fmt]
    R, C = d_o.shape
    d32 = d_o.astype(np.float32).astype(np.float64)
    rmax = np.abs(d32).reshape(R, C // 32, 32).max(-1)
    rb = bound.reshape(R, C // 32, 32).max(-1)
    cmax = np.abs(d32).reshape(R // 32, 32, C).max(1)
    cb = bound.reshape(R // 32, 32, C).max(1)
    r_near = near_pow2_boundary(rmax, rb, norm_const, fmax)
    c_near = near_pow2_boundary(cmax, cb, norm_const, fmax)
    out = {}
    # row direction: compare codes where the block's scale agrees; a code
    # more than one step off must lie inside its error-bound window
    same_r = np.repeat(gpu_row_scales == rs, 32, axis=1)
    g_r = np.where(same_r, gpu_row_codes, rc)
    out["row"] = check_quant(g_r, gpu_row_scales, rc, rs, r_near, what=what + " row",
                             window=code_window(d_o, bound, rs, 1, norm_const, fmt), fmt=fmt)
    same_c = np.repeat(gpu_col_scales == cs, 32, axis=0)
    g_c = np.where(same_c, gpu_col_codes, cc)
    out["col"] = check_quant(g_c, gpu_col_scales, cc, cs, c_near, what=what + " col",
                             window=code_window(d_o, bound, cs, 0, norm_const, fmt), fmt=fmt)
    out["row_scale_mismatch_near_pow2"] = int((gpu_row_scales != rs).sum())
    out["col_scale_mismatch_near_pow2"] = int((gpu_col_scales != cs).sum())
    return out


def d_bound(o_c, bc, prob, s):
    """Escape bound for D = prob * f(C) given C's bound bc: |f'| <= 2|C| + bc,
    plus the clamp's tanh error (absolute 1e-6 on t, i.e. 2 s^2 1e-6 on f)."""
    b = prob[:, None] * (2 * np.abs(o_c) + bc) * bc
    if s > 0:
        b = b + prob[:, None] * 2 * s * s * 1e-6
    return b


def gather_scales(sfd_row, sfd_col, r0, r1, m, n):
    """Logical (row, N/32) and (rows/32, N) scale arrays for rows [r0, r1)."""
    row_idx = O.sf_offset_grid(r0, r1, n // 32, 0, m, n // 32)
    col_idx = O.sf_offset_grid(0, n, ceil_div(r1, 32), 0, n, m // 32)[:, r0 // 32:]
    rs = sfd_row.cpu().numpy()[row_idx]
    cs = sfd_col.cpu().numpy()[col_idx].T
    return rs, cs
