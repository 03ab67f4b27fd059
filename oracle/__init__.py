"""CPU oracle for the block-scaled GEMM family (fp64, exact decode).

TEST INFRASTRUCTURE.  Only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import this package.  It shares no code
with the HIP path (`block_scaled_gemm_02_amd`) and imports nothing from it.

The arithmetic lives in `oracle.c` (plain loops, fp64); this module only
marshals numpy arrays into it and assembles per-expert / global maxima and
scale-atom placements from the C results.  Citations refer to the cuDNN
frontend "GEMM fusions" documentation pages:
  [GA] "GEMM + Amax (SM100)"          [GS] "Grouped GEMM + sReLU (SM100)"
  [GD] "Grouped GEMM + dSwiGLU (SM100)" [GB] "Grouped GEMM (SM100 BF16)"
  [PR] "GEMM + RoPE + MXFP8 Projection (SM100)"
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

E4M3, E2M1, E5M2 = 0, 1, 2
_FMT = {"e4m3": E4M3, "e2m1": E2M1, "e5m2": E5M2, E4M3: E4M3, E2M1: E2M1, E5M2: E5M2}


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-fno-fast-math", "-ffp-contract=off",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        d, u32, i64, i32, p = (ctypes.c_double, ctypes.c_uint32, ctypes.c_int64,
                               ctypes.c_int, ctypes.c_void_p)
        L.orc_dec_e4m3.restype = d; L.orc_dec_e4m3.argtypes = [u32]
        L.orc_dec_e2m1.restype = d; L.orc_dec_e2m1.argtypes = [u32]
        L.orc_dec_e5m2.restype = d; L.orc_dec_e5m2.argtypes = [u32]
        L.orc_dec_e8m0.restype = d; L.orc_dec_e8m0.argtypes = [u32]
        L.orc_dec_bf16.restype = d; L.orc_dec_bf16.argtypes = [u32]
        L.orc_enc_e4m3.restype = u32; L.orc_enc_e4m3.argtypes = [d]
        L.orc_enc_e5m2.restype = u32; L.orc_enc_e5m2.argtypes = [d]
        L.orc_enc_e2m1.restype = u32; L.orc_enc_e2m1.argtypes = [d]
        L.orc_rne_bf16.restype = u32; L.orc_rne_bf16.argtypes = [d]
        L.orc_e8m0_ceil.restype = u32; L.orc_e8m0_ceil.argtypes = [d]
        L.orc_rne_bf16_array.restype = None; L.orc_rne_bf16_array.argtypes = [p, p, i64]
        L.orc_sf_offset.restype = i64; L.orc_sf_offset.argtypes = [i64] * 5
        L.orc_sf_offset_grid.restype = None; L.orc_sf_offset_grid.argtypes = [i64] * 6 + [p]
        L.orc_expert_of_row.restype = ctypes.c_int32
        L.orc_expert_of_row.argtypes = [p, i64, i64]
        L.orc_gemm_amax.restype = i32
        L.orc_gemm_amax.argtypes = [p, p, p, p, i64, i64, i64, i64, i32, i64, i64, i64, p, p, p]
        L.orc_grouped_srelu.restype = i32
        L.orc_grouped_srelu.argtypes = [p] * 7 + [i64] * 4 + [i32, d, i64, i64, p, p, p, p, p]
        L.orc_grouped_dswiglu.restype = i32
        L.orc_grouped_dswiglu.argtypes = [p] * 9 + [i64] * 4 + [i32, i64, i64] + [p] * 5
        L.orc_grouped_bf16.restype = i32
        L.orc_grouped_bf16.argtypes = [p] * 6 + [i64] * 6 + [p, p, p, p]
        L.orc_proj_rope.restype = i32
        L.orc_proj_rope.argtypes = [p] * 4 + [i64] * 5 + [i32, i64, i64, p, p]
        L.orc_proj_rope_mx.restype = i32
        L.orc_proj_rope_mx.argtypes = [p] * 6 + [i64] * 7 + [p, p]
        L.orc_mx_quant_rows.restype = None
        L.orc_mx_quant_rows.argtypes = [p, i64, i64, i64, ctypes.c_float, i32, p, p]
        L.orc_mx_quant_cols.restype = None
        L.orc_mx_quant_cols.argtypes = [p, i64, i64, i64, ctypes.c_float, i32, p, p]
        L.orc_num_threads.restype = i32
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [i32]
        _lib = L
    return _lib


def _np(x, dtype=None):
    """torch tensor or array -> C-contiguous numpy array on the host."""
    if hasattr(x, "detach"):
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = bits16(x)
        else:
            x = x.detach().cpu().contiguous().numpy()
    x = np.ascontiguousarray(x)
    if dtype is not None:
        x = np.ascontiguousarray(x, dtype=dtype)
    return x


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def bits16(t):
    """bf16/fp16 torch tensor -> uint16 numpy array of its bit patterns."""
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def threads() -> int:
    return lib().orc_num_threads()


def set_threads(n: int) -> None:
    """OpenMP threads for the oracle calls that follow (timing only)."""
    lib().orc_set_threads(int(n))


# ---------------------------------------------------------------------------
# Number formats (scalar access, used by tests that pin the formats)
# ---------------------------------------------------------------------------
def dec_e4m3(code: int) -> float: return lib().orc_dec_e4m3(code)
def dec_e2m1(nib: int) -> float: return lib().orc_dec_e2m1(nib)
def dec_e5m2(code: int) -> float: return lib().orc_dec_e5m2(code)
def dec_e8m0(b: int) -> float: return lib().orc_dec_e8m0(b)
def dec_bf16(h: int) -> float: return lib().orc_dec_bf16(h)
def enc_e4m3(x: float) -> int: return lib().orc_enc_e4m3(float(x))
def enc_e5m2(x: float) -> int: return lib().orc_enc_e5m2(float(x))
def enc_e2m1(x: float) -> int: return lib().orc_enc_e2m1(float(x))
def rne_bf16(x: float) -> int: return lib().orc_rne_bf16(float(x))
def e8m0_ceil(sigma: float) -> int: return lib().orc_e8m0_ceil(float(sigma))


def sf_offset(r: int, kb: int, l: int, mn: int, kblocks: int) -> int:
    """[GA] Shapes: byte offset of the scale of (row r, K-block kb, batch l)."""
    return lib().orc_sf_offset(r, kb, l, mn, kblocks)


def sf_offset_grid(r0: int, r1: int, nkb: int, l: int, mn: int, kblocks: int) -> np.ndarray:
    """Offsets of rows [r0, r1) x k-blocks [0, nkb) of batch l: (r1-r0, nkb) int64."""
    out = np.empty((r1 - r0, nkb), dtype=np.int64)
    lib().orc_sf_offset_grid(r0, r1, nkb, l, mn, kblocks, _ptr(out))
    return out


def rne_bf16_array(x: np.ndarray) -> np.ndarray:
    """Elementwise fp64 -> bf16 bit patterns, one round-to-nearest-even step."""
    flat = np.ascontiguousarray(x, dtype=np.float64).ravel()
    out = np.empty(flat.size, dtype=np.uint16)
    lib().orc_rne_bf16_array(_ptr(flat), _ptr(out), flat.size)
    return out.reshape(np.shape(x))


# ---------------------------------------------------------------------------
# [GA] gemm_amax
# ---------------------------------------------------------------------------
def gemm_amax(a, b, sfa, sfb, m, n, k, l, fmt, batch=0, r0=0, r1=None, want_sabs=True,
              want_bmax=False):
    """Rows [r0, r1) of batch `batch`: C = sum_k A_hat * B_hat in fp64.

    Returns (C, Sabs) where Sabs = sum_k |A_hat * B_hat| (for error bounds),
    plus Bmax = sum over 32-wide K blocks of max |A_hat * B_hat| when
    want_bmax.  Amax over a full problem is `max |C|` over every batch and row.
    """
    L = lib()
    r1 = m if r1 is None else r1
    a, b, sfa, sfb = (_np(x, np.uint8) for x in (a, b, sfa, sfb))
    c = np.empty((r1 - r0, n), dtype=np.float64)
    s = np.empty_like(c) if want_sabs else None
    bm = np.empty_like(c) if want_bmax else None
    rc = L.orc_gemm_amax(_ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb), m, n, k, l, _FMT[fmt],
                         batch, r0, r1, _ptr(c), _ptr(s), _ptr(bm))
    if rc:
        raise ValueError(f"orc_gemm_amax failed ({rc})")
    return (c, s, bm) if want_bmax else (c, s)


def gemm_amax_full(a, b, sfa, sfb, m, n, k, l, fmt, want_bmax=False):
    """Whole problem: C (L, M, N) fp64, Sabs, and Amax = max |C| ([GA] Equations)
    (plus Bmax, see gemm_amax, when want_bmax)."""
    cs, ss, bs = [], [], []
    for bi in range(l):
        r = gemm_amax(a, b, sfa, sfb, m, n, k, l, fmt, batch=bi, want_bmax=want_bmax)
        cs.append(r[0]); ss.append(r[1])
        if want_bmax:
            bs.append(r[2])
    c = np.stack(cs); s = np.stack(ss)
    amax = float(np.abs(c).max()) if c.size else 0.0
    if want_bmax:
        return c, s, amax, np.stack(bs)
    return c, s, amax


# ---------------------------------------------------------------------------
# [GS] grouped_gemm_srelu
# ---------------------------------------------------------------------------
def grouped_srelu(a, b, sfa, sfb, offsets, alpha, prob, m, n, k, L_, fmt, s, r0=0, r1=None):
    """Rows [r0, r1): returns dict(c, d, sabs, group, bmax) in fp64 (bmax and
    sabs include |alpha_g|).

    Rows at or past padded_offsets[L-1] carry group -1 and NaN outputs.
    s <= 0 means no tanh clamp.
    """
    L = lib()
    r1 = m if r1 is None else r1
    a, b, sfa, sfb = (_np(x, np.uint8) for x in (a, b, sfa, sfb))
    off = _np(offsets, np.int32); al = _np(alpha, np.float32); pr = _np(prob, np.float32)
    rows = r1 - r0
    c = np.empty((rows, n)); d = np.empty((rows, n)); sab = np.empty((rows, n))
    bm = np.empty((rows, n))
    grp = np.empty(rows, dtype=np.int32)
    rc = L.orc_grouped_srelu(_ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb), _ptr(off), _ptr(al),
                             _ptr(pr), m, n, k, L_, _FMT[fmt], float(s), r0, r1,
                             _ptr(c), _ptr(d), _ptr(sab), _ptr(grp), _ptr(bm))
    if rc:
        raise ValueError(f"orc_grouped_srelu failed ({rc})")
    return dict(c=c, d=d, sabs=sab, group=grp, bmax=bm)


def grouped_dswiglu(a, b, sfa, sfb, offsets, alpha, beta, prob, c_bits, m, n, k, L_, fmt, r0=0, r1=None):
    """[GD] Steps 1-2, rows [r0, r1): dict(ref (rows,N), d (rows,2N), dprob (rows,),
    sabs, bmax) in fp64; C given as bf16 bits (rows of the full (M, 2N) tensor)."""
    L = lib()
    r1 = m if r1 is None else r1
    a, b, sfa, sfb = (_np(x, np.uint8) for x in (a, b, sfa, sfb))
    off = _np(offsets, np.int32); al = _np(alpha, np.float32); bt = _np(beta, np.float32)
    pr = _np(prob, np.float32); cb = _np(c_bits, np.uint16)
    rows = r1 - r0
    ref = np.empty((rows, n)); d = np.empty((rows, 2 * n)); dp = np.empty(rows)
    sab = np.empty((rows, n)); bm = np.empty((rows, n))
    rc = L.orc_grouped_dswiglu(_ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb), _ptr(off), _ptr(al), _ptr(bt),
                               _ptr(pr), _ptr(cb), m, n, k, L_, _FMT[fmt], r0, r1, _ptr(ref), _ptr(d),
                               _ptr(dp), _ptr(sab), _ptr(bm))
    if rc:
        raise ValueError(f"orc_grouped_dswiglu failed ({rc})")
    return dict(ref=ref, d=d, dprob=dp, sabs=sab, bmax=bm)


def expert_amax(d: np.ndarray, group: np.ndarray, L_: int) -> np.ndarray:
    """[GS] Shapes: Amax (L,1) = max |D| over each expert's rows; 0 when empty."""
    out = np.zeros(L_, dtype=np.float64)
    for g in range(L_):
        sel = group == g
        if sel.any():
            out[g] = float(np.abs(d[sel]).max())
    return out


def expert_of_row(offsets, L_: int, r: int) -> int:
    off = _np(offsets, np.int32)
    return lib().orc_expert_of_row(_ptr(off), L_, r)


# ---------------------------------------------------------------------------
# [GB] grouped_gemm (BF16)
# ---------------------------------------------------------------------------
def grouped_bf16(a_bits, b_bits, offsets, alpha, prob, bias, m, n, k, L_, r0=0, r1=None):
    """a_bits (M,K) / b_bits [L][N][K] are uint16 bf16 patterns; bias is an
    (L, N) array of values (any float dtype) or None.  Returns dict(c, d, sabs, group)."""
    L = lib()
    r1 = m if r1 is None else r1
    a = _np(a_bits, np.uint16); b = _np(b_bits, np.uint16)
    off = _np(offsets, np.int32); al = _np(alpha, np.float32); pr = _np(prob, np.float32)
    bi = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64)
    rows = r1 - r0
    c = np.empty((rows, n)); d = np.empty((rows, n)); sab = np.empty((rows, n))
    grp = np.empty(rows, dtype=np.int32)
    rc = L.orc_grouped_bf16(_ptr(a), _ptr(b), _ptr(off), _ptr(al), _ptr(pr), _ptr(bi),
                            m, n, k, L_, r0, r1, _ptr(c), _ptr(d), _ptr(sab), _ptr(grp))
    if rc:
        raise ValueError(f"orc_grouped_bf16 failed ({rc})")
    return dict(c=c, d=d, sabs=sab, group=grp)


# ---------------------------------------------------------------------------
# [PR] gemm_proj_rope_mxfp8
# ---------------------------------------------------------------------------
def proj_rope(x_bits, w_bits, cos_bits, sin_bits, tokens, q_lora, heads, head_dim, qk_rope,
              w_out_in=1, t0=0, t1=None):
    """Rows [t0, t1) of Y after RoPE, fp64, shape (rows, heads*head_dim), plus Sabs."""
    L = lib()
    t1 = tokens if t1 is None else t1
    x = _np(x_bits, np.uint16); w = _np(w_bits, np.uint16)
    cs = _np(cos_bits, np.uint16); sn = _np(sin_bits, np.uint16)
    y = np.empty((t1 - t0, heads * head_dim)); s = np.empty_like(y)
    rc = L.orc_proj_rope(_ptr(x), _ptr(w), _ptr(cs), _ptr(sn), tokens, q_lora, heads,
                         head_dim, qk_rope, int(w_out_in), t0, t1, _ptr(y), _ptr(s))
    if rc:
        raise ValueError(f"orc_proj_rope failed ({rc})")
    return y, s


def proj_rope_mx(x_codes, x_scale, w_codes, w_scale, cos_bits, sin_bits, tokens, q_lora, heads,
                 head_dim, qk_rope, t0=0, t1=None):
    """MXFP8-input projection ([PR] Shapes: E4M3 codes with row-wise E8M0 scales per
    32 elements; w as [out, in]): rows [t0, t1) of Y after RoPE, fp64, plus Sabs."""
    L = lib()
    t1 = tokens if t1 is None else t1
    x = _np(x_codes, np.uint8); xs = _np(x_scale, np.uint8)
    w = _np(w_codes, np.uint8); ws = _np(w_scale, np.uint8)
    cs = _np(cos_bits, np.uint16); sn = _np(sin_bits, np.uint16)
    y = np.empty((t1 - t0, heads * head_dim)); s = np.empty_like(y)
    rc = L.orc_proj_rope_mx(_ptr(x), _ptr(xs), _ptr(w), _ptr(ws), _ptr(cs), _ptr(sn), tokens, q_lora,
                            heads, head_dim, qk_rope, t0, t1, _ptr(y), _ptr(s))
    if rc:
        raise ValueError(f"orc_proj_rope_mx failed ({rc})")
    return y, s


# ---------------------------------------------------------------------------
# [GD] Step 3: MX output quantiser (row and column direction, blocks of 32)
# ---------------------------------------------------------------------------
def mx_quant_rows(d: np.ndarray, norm_const: float = 1.0, fmt: str = "e4m3"):
    """Blocks of 32 along each row -> (codes uint8 (R,C), scales uint8 (R, ceil(C/32)));
    fmt "e4m3" (rcp_max 1/448), "e5m2" (1/57344) or "e2m1" (1/6; one code
    per byte, unpacked)."""
    d = np.ascontiguousarray(d, dtype=np.float64)
    r, c = d.shape
    codes = np.empty((r, c), dtype=np.uint8)
    scales = np.empty((r, -(-c // 32)), dtype=np.uint8)
    lib().orc_mx_quant_rows(_ptr(d), r, c, c, float(norm_const), _FMT[fmt], _ptr(codes), _ptr(scales))
    return codes, scales


def mx_quant_cols(d: np.ndarray, norm_const: float = 1.0, fmt: str = "e4m3"):
    """Blocks of 32 down each column -> (codes (R,C), scales (ceil(R/32), C))."""
    d = np.ascontiguousarray(d, dtype=np.float64)
    r, c = d.shape
    codes = np.empty((r, c), dtype=np.uint8)
    scales = np.empty((-(-r // 32), c), dtype=np.uint8)
    lib().orc_mx_quant_cols(_ptr(d), r, c, c, float(norm_const), _FMT[fmt], _ptr(codes), _ptr(scales))
    return codes, scales
