"""Python binding of the gfx950 block-scaled GEMM library (libbsg.so).

Argument marshalling only: torch tensors become device pointers, the current
torch stream becomes the hipStream_t, and every step runs inside the HIP
kernels behind the C ABI declared in include/bsg.h.  There is no fallback:
if libbsg.so is missing or a call fails, a RuntimeError is raised.

Entry points keep the C names:
    gemm_amax, grouped_gemm, grouped_gemm_srelu, grouped_gemm_dswiglu,
    gemm_proj_rope_mxfp8, grouped_gemm_discrete, grouped_gemm_srelu_discrete
and validate_only=True calls the host-only check bsg_validate_<name>.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsg.so")

# bsg_dtype
F32, F16, BF16, E4M3, E5M2, E2M1X2, E8M0 = range(7)
_TORCH_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
STATUS = {0: "OK", 1: "NULLPTR", 2: "SHAPE", 3: "DTYPE", 4: "ALIGN", 5: "UNSUPPORTED",
          6: "DEVICE", 7: "LAUNCH"}


class BsgError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load libbsg.so (built by block_scaled_gemm_02_amd/build.py); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m block_scaled_gemm_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        sigs = {
            "gemm_amax": [p] * 6 + [i64] * 4 + [i32] * 3 + [p],
            "grouped_gemm": [p] * 8 + [i64] * 4 + [i32] * 3 + [p],
            "grouped_gemm_srelu": [p] * 14 + [i64] * 4 + [i32] * 4 + [f32, p],
            "gemm_proj_rope_mxfp8": [p] * 10 + [i64] * 5 + [i32, i32, p],
            "grouped_gemm_dswiglu": [p] * 16 + [i64] * 4 + [i32] * 4 + [p],
            "bsg_validate_grouped_gemm_dswiglu": [p] * 16 + [i64] * 4 + [i32] * 4,
            "grouped_gemm_discrete": [p] * 8 + [i64] * 4 + [i32] * 3 + [p],
            "grouped_gemm_srelu_discrete": [p] * 14 + [i64] * 4 + [i32] * 4 + [f32, p],
            "bsg_validate_grouped_gemm_discrete": [p] * 8 + [i64] * 4 + [i32] * 3,
            "bsg_validate_grouped_gemm_srelu_discrete": [p] * 14 + [i64] * 4 + [i32] * 4 + [f32],
            "bsg_validate_gemm_amax": [p] * 6 + [i64] * 4 + [i32] * 3,
            "bsg_validate_grouped_gemm": [p] * 8 + [i64] * 4 + [i32] * 3,
            "bsg_validate_grouped_gemm_srelu": [p] * 14 + [i64] * 4 + [i32] * 4 + [f32],
            "bsg_validate_gemm_proj_rope_mxfp8": [p] * 10 + [i64] * 5 + [i32, i32],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = i32
        L.bsg_status_string.restype = ctypes.c_char_p
        L.bsg_status_string.argtypes = [i32]
        L.bsg_last_error.restype = ctypes.c_char_p
        L.bsg_last_error.argtypes = []
        L.bsg_version.restype = i32
        _lib = L
    return _lib


def symbols():
    """Names of the C entry points this binding expects libbsg.so to export."""
    return ["gemm_amax", "grouped_gemm", "grouped_gemm_srelu", "gemm_proj_rope_mxfp8",
            "grouped_gemm_discrete", "grouped_gemm_srelu_discrete", "grouped_gemm_dswiglu",
            "bsg_validate_gemm_amax", "bsg_validate_grouped_gemm",
            "bsg_validate_grouped_gemm_srelu", "bsg_validate_gemm_proj_rope_mxfp8",
            "bsg_validate_grouped_gemm_dswiglu",
            "bsg_validate_grouped_gemm_discrete", "bsg_validate_grouped_gemm_srelu_discrete",
            "bsg_status_string", "bsg_last_error", "bsg_version"]


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int):
    if rc != 0:
        raise BsgError(rc, lib().bsg_last_error().decode())


def dtype_code(x) -> int:
    """torch dtype or tensor -> bsg_dtype code (float outputs only)."""
    if isinstance(x, int):
        return x
    if isinstance(x, torch.Tensor):
        x = x.dtype
    return _TORCH_DT[x]


def _ab_code(fmt) -> int:
    return {"e4m3": E4M3, "e5m2": E5M2, "e2m1": E2M1X2, E4M3: E4M3, E2M1X2: E2M1X2, E5M2: E5M2}[fmt]


def _d_code(d_dtype, d) -> int:
    """Output dtype code: "e4m3" / "e5m2" (or torch's float8_e4m3fn /
    float8_e5m2) for FP8 outputs, else a torch float dtype (taken from the
    tensor d when d_dtype is None)."""
    x = d_dtype if d_dtype is not None else d
    if isinstance(x, torch.Tensor):
        x = x.dtype
    if x in ("e4m3", E4M3, torch.float8_e4m3fn):
        return E4M3
    if x in ("e5m2", E5M2, torch.float8_e5m2):
        return E5M2
    if x in ("e2m1", E2M1X2):
        return E2M1X2
    return dtype_code(x)


# ---------------------------------------------------------------------------
def gemm_amax(a, b, sfa, sfb, c, amax, m, n, k, l, ab_dtype="e4m3", c_dtype=None,
              sf_vec_size=32, stream=None, validate_only=False):
    """C = sum_k A_hat B_hat per batch and Amax = max |C| (see include/bsg.h).
    c_dtype: a torch float dtype, "e4m3" / "e5m2" (FP8 C) or "e2m1" (packed
    FP4 C, (M, N/2, L) bytes); the last three with FP4 operands only."""
    cd = _d_code(c_dtype, c)
    args = [_ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb), _ptr(c), _ptr(amax), m, n, k, l,
            _ab_code(ab_dtype), cd, sf_vec_size]
    if validate_only:
        return lib().bsg_validate_gemm_amax(*args)
    _check(lib().gemm_amax(*args, _stream(stream)))


def grouped_gemm(a, b, padded_offsets, alpha, prob, bias, c, d, m, n, k, num_experts,
                 bias_dtype=None, c_dtype=None, d_dtype=None, stream=None, validate_only=False):
    """BF16 grouped GEMM with alpha / prob / bias epilogue (see include/bsg.h)."""
    bd = dtype_code(bias_dtype if bias_dtype is not None else (bias if bias is not None else torch.bfloat16))
    cd = dtype_code(c_dtype if c_dtype is not None else (c if c is not None else torch.bfloat16))
    dd = dtype_code(d_dtype if d_dtype is not None else d)
    args = [_ptr(a), _ptr(b), _ptr(padded_offsets), _ptr(alpha), _ptr(prob), _ptr(bias),
            _ptr(c), _ptr(d), m, n, k, num_experts, bd, cd, dd]
    if validate_only:
        return lib().bsg_validate_grouped_gemm(*args)
    _check(lib().grouped_gemm(*args, _stream(stream)))


def grouped_gemm_srelu(a, b, sfa, sfb, padded_offsets, alpha, prob, norm_const, c, d, d_col,
                       sfd_row, sfd_col, amax, m, n, k, num_experts, ab_dtype="e4m3",
                       c_dtype=None, d_dtype=None, sf_vec_size=32, tanh_clamp_scale=0.0,
                       stream=None, validate_only=False):
    """Grouped block-scaled GEMM + prob-gated squared ReLU (see include/bsg.h).

    d_dtype: a torch float dtype, or "e4m3" / "e5m2" for MXFP8 output with SFD_row/col."""
    cd = dtype_code(c_dtype if c_dtype is not None else (c if c is not None else torch.bfloat16))
    dd = _d_code(d_dtype, d)
    s = float(tanh_clamp_scale) if tanh_clamp_scale is not None else 0.0
    args = [_ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb), _ptr(padded_offsets), _ptr(alpha),
            _ptr(prob), _ptr(norm_const), _ptr(c), _ptr(d), _ptr(d_col), _ptr(sfd_row),
            _ptr(sfd_col), _ptr(amax), m, n, k, num_experts, _ab_code(ab_dtype), cd, dd,
            sf_vec_size, s]
    if validate_only:
        return lib().bsg_validate_grouped_gemm_srelu(*args)
    _check(lib().grouped_gemm_srelu(*args, _stream(stream)))


def pointer_array(tensors):
    """(L,) int64 device tensor of the tensors' data pointers, for the
    discrete-weight calls (b_ptrs / sfb_ptrs).  The caller keeps the tensors
    alive until the stream has finished with them."""
    ptrs = [t.data_ptr() for t in tensors]
    return torch.tensor(ptrs, dtype=torch.int64).to(tensors[0].device)


def grouped_gemm_discrete(a, b_ptrs, padded_offsets, alpha, prob, bias, c, d, m, n, k, num_experts,
                          bias_dtype=None, c_dtype=None, d_dtype=None, stream=None, validate_only=False):
    """grouped_gemm with per-expert weight allocations: b_ptrs is an (L,)
    int64 device tensor of (N,K) bf16 matrices (see include/bsg.h)."""
    bd = dtype_code(bias_dtype if bias_dtype is not None else (bias if bias is not None else torch.bfloat16))
    cd = dtype_code(c_dtype if c_dtype is not None else (c if c is not None else torch.bfloat16))
    dd = dtype_code(d_dtype if d_dtype is not None else d)
    args = [_ptr(a), _ptr(b_ptrs), _ptr(padded_offsets), _ptr(alpha), _ptr(prob), _ptr(bias),
            _ptr(c), _ptr(d), m, n, k, num_experts, bd, cd, dd]
    if validate_only:
        return lib().bsg_validate_grouped_gemm_discrete(*args)
    _check(lib().grouped_gemm_discrete(*args, _stream(stream)))


def grouped_gemm_srelu_discrete(a, b_ptrs, sfa, sfb_ptrs, padded_offsets, alpha, prob, norm_const, c, d,
                                d_col, sfd_row, sfd_col, amax, m, n, k, num_experts, ab_dtype="e4m3",
                                c_dtype=None, d_dtype=None, sf_vec_size=32, tanh_clamp_scale=0.0,
                                stream=None, validate_only=False):
    """grouped_gemm_srelu with per-expert weight and scale allocations:
    b_ptrs / sfb_ptrs are (L,) int64 device tensors (see include/bsg.h)."""
    cd = dtype_code(c_dtype if c_dtype is not None else (c if c is not None else torch.bfloat16))
    dd = _d_code(d_dtype, d)
    s = float(tanh_clamp_scale) if tanh_clamp_scale is not None else 0.0
    args = [_ptr(a), _ptr(b_ptrs), _ptr(sfa), _ptr(sfb_ptrs), _ptr(padded_offsets), _ptr(alpha),
            _ptr(prob), _ptr(norm_const), _ptr(c), _ptr(d), _ptr(d_col), _ptr(sfd_row),
            _ptr(sfd_col), _ptr(amax), m, n, k, num_experts, _ab_code(ab_dtype), cd, dd,
            sf_vec_size, s]
    if validate_only:
        return lib().bsg_validate_grouped_gemm_srelu_discrete(*args)
    _check(lib().grouped_gemm_srelu_discrete(*args, _stream(stream)))


def grouped_gemm_dswiglu(a, b, sfa, sfb, c, padded_offsets, alpha, beta, prob, norm_const, d_row, d_col,
                         sfd_row, sfd_col, dprob, m, n, k, num_experts, ab_dtype="e4m3", c_dtype=None,
                         d_dtype="e4m3", sf_vec_size=32, amax=None, stream=None, validate_only=False):
    """Grouped GEMM + dSwiGLU backward (see include/bsg.h): MXFP8 D for FP8
    inputs, bf16/fp32 D with amax (L, 2) for FP4 inputs.  dprob is accumulated:
    zero-fill it first."""
    cd = BF16 if c_dtype is None else (_TORCH_DT[c_dtype] if c_dtype in _TORCH_DT else c_dtype)
    dd = _d_code(d_dtype, d_row)
    args = [_ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb), _ptr(c), _ptr(padded_offsets), _ptr(alpha), _ptr(beta),
            _ptr(prob), _ptr(norm_const), _ptr(d_row), _ptr(d_col), _ptr(sfd_row), _ptr(sfd_col), _ptr(dprob),
            _ptr(amax), m, n, k, num_experts, _ab_code(ab_dtype), cd, dd, sf_vec_size]
    if validate_only:
        return lib().bsg_validate_grouped_gemm_dswiglu(*args)
    _check(lib().grouped_gemm_dswiglu(*args, _stream(stream)))


def gemm_proj_rope_mxfp8(x, w, x_scale, w_scale, cos, sin, out_fp8_row, out_scales_row,
                         out_fp8_col, out_scales_col, tokens, q_lora, num_heads=128,
                         head_dim=192, qk_rope=64, in_dtype=BF16, w_out_in=1, stream=None,
                         validate_only=False):
    """Projection GEMM + per-head RoPE + dual MXFP8 quantisation (see include/bsg.h)."""
    args = [_ptr(x), _ptr(w), _ptr(x_scale), _ptr(w_scale), _ptr(cos), _ptr(sin),
            _ptr(out_fp8_row), _ptr(out_scales_row), _ptr(out_fp8_col), _ptr(out_scales_col),
            tokens, q_lora, num_heads, head_dim, qk_rope, in_dtype, int(w_out_in)]
    if validate_only:
        return lib().bsg_validate_gemm_proj_rope_mxfp8(*args)
    _check(lib().gemm_proj_rope_mxfp8(*args, _stream(stream)))
