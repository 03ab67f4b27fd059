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
            "gemm_amax": [p] * 6 + [i64] * 4 + [i32] * 6 + [p],
            "grouped_gemm": [p] * 8 + [i64] * 4 + [i32] * 3 + [p],
            "grouped_gemm_srelu": [p] * 14 + [i64] * 4 + [i32] * 4 + [f32, p],
            "gemm_proj_rope_mxfp8": [p] * 10 + [i64] * 5 + [i32, i32, p],
            "grouped_gemm_dswiglu": [p] * 16 + [i64] * 4 + [i32] * 5 + [p],
            "bsg_validate_grouped_gemm_dswiglu": [p] * 16 + [i64] * 4 + [i32] * 5,
            "grouped_gemm_discrete": [p] * 8 + [i64] * 4 + [i32] * 3 + [p],
            "grouped_gemm_srelu_discrete": [p] * 14 + [i64] * 4 + [i32] * 4 + [f32, p],
            "bsg_validate_grouped_gemm_discrete": [p] * 8 + [i64] * 4 + [i32] * 3,
            "bsg_validate_grouped_gemm_srelu_discrete": [p] * 14 + [i64] * 4 + [i32] * 4 + [f32],
            "bsg_validate_gemm_amax": [p] * 6 + [i64] * 4 + [i32] * 6,
            "bsg_validate_grouped_gemm": [p] * 8 + [i64] * 4 + [i32] * 3,
            "bsg_validate_grouped_gemm_srelu": [p] * 14 + [i64] * 4 + [i32] * 4 + [f32],
            "bsg_validate_gemm_proj_rope_mxfp8": [p] * 10 + [i64] * 5 + [i32, i32],
            "bsg_check_padded_offsets": [p, i64, i64, p],
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
            "bsg_check_padded_offsets", "bsg_status_string", "bsg_last_error", "bsg_version"]


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


# ---------------------------------------------------------------------------
# Tensor checks.  The C ABI receives bare pointers and cannot see how large a
# buffer is, so the binding checks every torch tensor it is handed against
# what the kernels will read or write for the given sizes: device, dense
# row-major layout, element type and byte count.  Plain integers are device
# addresses; their extent is the caller's contract.
# ---------------------------------------------------------------------------
_OUT_TORCH = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}
_BYTES = {F32: 4.0, F16: 2.0, BF16: 2.0, E4M3: 1.0, E5M2: 1.0, E2M1X2: 0.5}


def _cdiv(a, b):
    return -(-a // b)


def sf_atom_bytes(mn: int, k: int, l: int = 1) -> int:
    """Bytes of a (32, 4, ceil(MN/128), 4, ceil(K/128), L) E8M0 scale-atom buffer."""
    return 512 * _cdiv(mn, 128) * _cdiv(_cdiv(k, 32), 4) * l


def _need(t, name, nbytes, kind=None):
    """Reject a tensor that the kernel cannot use as `name`: kind is a
    bsg_dtype code (a float dtype must match exactly; FP8 / FP4 codes need
    one-byte elements), a torch dtype, or None (any element type)."""
    if t is None or isinstance(t, int):
        return
    if not t.is_cuda or t.device.index != torch.cuda.current_device():
        raise BsgError(6, f"{name} must be on the current CUDA device (got {t.device})")
    if not t.is_contiguous():
        raise BsgError(4, f"{name} must be contiguous")
    if isinstance(kind, torch.dtype):
        if t.dtype != kind:
            raise BsgError(3, f"{name} must be {kind} (got {t.dtype})")
    elif kind in _OUT_TORCH:
        if t.dtype != _OUT_TORCH[kind]:
            raise BsgError(3, f"{name} must be {_OUT_TORCH[kind]} for dtype code {kind} (got {t.dtype})")
    elif kind is not None and t.element_size() != 1:
        raise BsgError(3, f"{name} holds one-byte codes (got {t.dtype})")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise BsgError(2, f"{name} holds {have} bytes; these sizes need {int(nbytes)}")


def _out_bytes(code, count):
    return int(_BYTES.get(code, 1.0) * count)


def _ab_row_bytes(ab, k):
    return k // 2 if ab == E2M1X2 else k


def _grouped_common_need(padded_offsets, alpha, prob, m, num_experts):
    _need(padded_offsets, "padded_offsets", 4 * num_experts, torch.int32)
    _need(alpha, "alpha", 4 * num_experts, torch.float32)
    _need(prob, "prob", 4 * m, torch.float32)


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
def _major(x, allowed, name):
    """A major argument as the character code the C ABI takes."""
    if not isinstance(x, str) or len(x) != 1:
        raise ValueError(f"{name} must be one of {allowed!r}, got {x!r}")
    return ord(x)


def gemm_amax(a, b, sfa, sfb, c, amax, m, n, k, l, ab_dtype="e4m3", c_dtype=None,
              sf_vec_size=32, a_major="k", b_major="k", c_major="n", stream=None, validate_only=False):
    """C = sum_k A_hat B_hat per batch and Amax = max |C| (see include/bsg.h).
    c_dtype: a torch float dtype, "e4m3" / "e5m2" (FP8 C) or "e2m1" (packed
    FP4 C, (M, N/2, L) bytes); the last three with FP4 operands only.
    a_major "k" (memory [L][M][K]) or "m" ([L][K][M]); b_major "k" or "n"
    ([L][K][N]); c_major "n" ([L][M][N]) or "m" ([L][N][M])."""
    cd = _d_code(c_dtype, c)
    ab = _ab_code(ab_dtype)
    if m * n * l > 0:
        rb = _ab_row_bytes(ab, k)
        _need(a, "a", l * m * rb, ab); _need(b, "b", l * n * rb, ab)
        _need(sfa, "sfa", sf_atom_bytes(m, k, l), E8M0); _need(sfb, "sfb", sf_atom_bytes(n, k, l), E8M0)
        _need(c, "c", _out_bytes(cd, l * m * n), cd)
    _need(amax, "amax", 4, torch.float32)
    args = [_ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb), _ptr(c), _ptr(amax), m, n, k, l,
            ab, cd, sf_vec_size, _major(a_major, "km", "a_major"), _major(b_major, "kn", "b_major"),
            _major(c_major, "nm", "c_major")]
    if validate_only:
        return lib().bsg_validate_gemm_amax(*args)
    _check(lib().gemm_amax(*args, _stream(stream)))


def check_padded_offsets(padded_offsets, m, num_experts=None, stream=None):
    """Opt-in debug check of the routing offsets' values on the device
    (bsg_check_padded_offsets: multiples of 256 in [0, m], nondecreasing);
    waits for the stream.  Raises BsgError naming the first violation."""
    if num_experts is None:
        num_experts = padded_offsets.numel()
    _need(padded_offsets, "padded_offsets", 4 * num_experts, torch.int32)
    _check(lib().bsg_check_padded_offsets(_ptr(padded_offsets), num_experts, m, _stream(stream)))


def grouped_gemm(a, b, padded_offsets, alpha, prob, bias, c, d, m, n, k, num_experts,
                 bias_dtype=None, c_dtype=None, d_dtype=None, stream=None, validate_only=False):
    """BF16 grouped GEMM with alpha / prob / bias epilogue (see include/bsg.h)."""
    bd = dtype_code(bias_dtype if bias_dtype is not None else (bias if bias is not None else torch.bfloat16))
    cd = dtype_code(c_dtype if c_dtype is not None else (c if c is not None else torch.bfloat16))
    dd = dtype_code(d_dtype if d_dtype is not None else d)
    _grouped_common_need(padded_offsets, alpha, prob, m, num_experts)
    if m * n > 0:
        _need(a, "a", 2 * m * k, torch.bfloat16); _need(b, "b", 2 * num_experts * n * k, torch.bfloat16)
        _need(bias, "bias", _out_bytes(bd, n * num_experts), bd)
        _need(c, "c", _out_bytes(cd, m * n), cd); _need(d, "d", _out_bytes(dd, m * n), dd)
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

    d_dtype: a torch float dtype, or "e4m3" / "e5m2" / "e2m1" for MX-quantised
    output with SFD_row/col.  c_dtype: a torch float dtype, or "e4m3" /
    "e5m2" / "e2m1" for an unscaled saturating cast of C (E2M1 packed two
    per byte)."""
    cd = _d_code(c_dtype if c_dtype is not None else (c if c is not None else torch.bfloat16), None)
    dd = _d_code(d_dtype, d)
    s = float(tanh_clamp_scale) if tanh_clamp_scale is not None else 0.0
    ab = _ab_code(ab_dtype)
    _grouped_common_need(padded_offsets, alpha, prob, m, num_experts)
    _need(amax, "amax", 4 * num_experts, torch.float32)
    if m * n > 0:
        rb = _ab_row_bytes(ab, k)
        _need(a, "a", m * rb, ab); _need(sfa, "sfa", sf_atom_bytes(m, k, 1), E8M0)
        _need(b, "b", num_experts * n * rb, ab)
        _need(sfb, "sfb", sf_atom_bytes(n, k, num_experts), E8M0)
        _need(c, "c", _out_bytes(cd, m * n), cd)
        _need(d, "d", _out_bytes(dd, m * n), dd); _need(d_col, "d_col", _out_bytes(dd, m * n), dd)
        _need(norm_const, "norm_const", 4, torch.float32)
        _need(sfd_row, "sfd_row", sf_atom_bytes(m, n, 1), E8M0)
        _need(sfd_col, "sfd_col", sf_atom_bytes(n, m, 1), E8M0)
    args = [_ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb), _ptr(padded_offsets), _ptr(alpha),
            _ptr(prob), _ptr(norm_const), _ptr(c), _ptr(d), _ptr(d_col), _ptr(sfd_row),
            _ptr(sfd_col), _ptr(amax), m, n, k, num_experts, ab, cd, dd,
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
    _grouped_common_need(padded_offsets, alpha, prob, m, num_experts)
    if m * n > 0:
        _need(a, "a", 2 * m * k, torch.bfloat16); _need(b_ptrs, "b_ptrs", 8 * num_experts, torch.int64)
        _need(bias, "bias", _out_bytes(bd, n * num_experts), bd)
        _need(c, "c", _out_bytes(cd, m * n), cd); _need(d, "d", _out_bytes(dd, m * n), dd)
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
    cd = _d_code(c_dtype if c_dtype is not None else (c if c is not None else torch.bfloat16), None)
    dd = _d_code(d_dtype, d)
    s = float(tanh_clamp_scale) if tanh_clamp_scale is not None else 0.0
    ab = _ab_code(ab_dtype)
    _grouped_common_need(padded_offsets, alpha, prob, m, num_experts)
    _need(amax, "amax", 4 * num_experts, torch.float32)
    if m * n > 0:
        rb = _ab_row_bytes(ab, k)
        _need(a, "a", m * rb, ab); _need(sfa, "sfa", sf_atom_bytes(m, k, 1), E8M0)
        _need(b_ptrs, "b_ptrs", 8 * num_experts, torch.int64)
        _need(sfb_ptrs, "sfb_ptrs", 8 * num_experts, torch.int64)
        _need(c, "c", _out_bytes(cd, m * n), cd)
        _need(d, "d", _out_bytes(dd, m * n), dd); _need(d_col, "d_col", _out_bytes(dd, m * n), dd)
        _need(norm_const, "norm_const", 4, torch.float32)
        _need(sfd_row, "sfd_row", sf_atom_bytes(m, n, 1), E8M0)
        _need(sfd_col, "sfd_col", sf_atom_bytes(n, m, 1), E8M0)
    args = [_ptr(a), _ptr(b_ptrs), _ptr(sfa), _ptr(sfb_ptrs), _ptr(padded_offsets), _ptr(alpha),
            _ptr(prob), _ptr(norm_const), _ptr(c), _ptr(d), _ptr(d_col), _ptr(sfd_row),
            _ptr(sfd_col), _ptr(amax), m, n, k, num_experts, ab, cd, dd,
            sf_vec_size, s]
    if validate_only:
        return lib().bsg_validate_grouped_gemm_srelu_discrete(*args)
    _check(lib().grouped_gemm_srelu_discrete(*args, _stream(stream)))


def grouped_gemm_dswiglu(a, b, sfa, sfb, c, padded_offsets, alpha, beta, prob, norm_const, d_row, d_col,
                         sfd_row, sfd_col, dprob, m, n, k, num_experts, ab_dtype="e4m3", c_dtype=None,
                         d_dtype="e4m3", sf_vec_size=32, amax=None, b_major="k", stream=None,
                         validate_only=False):
    """Grouped GEMM + dSwiGLU backward (see include/bsg.h): MXFP8 D for FP8
    inputs, bf16/fp32 D with amax (L, 2) for FP4 inputs.  dprob is accumulated:
    zero-fill it first.  b_major "k" (B memory [L][N][K]) or "n" ([L][K][N],
    FP8 only)."""
    cd = BF16 if c_dtype is None else (_TORCH_DT[c_dtype] if c_dtype in _TORCH_DT else c_dtype)
    dd = _d_code(d_dtype, d_row)
    ab = _ab_code(ab_dtype)
    _grouped_common_need(padded_offsets, alpha, prob, m, num_experts)
    _need(beta, "beta", 4 * num_experts, torch.float32)
    _need(amax, "amax", 8 * num_experts, torch.float32)
    if m * n > 0:
        rb = _ab_row_bytes(ab, k)
        _need(a, "a", m * rb, ab); _need(b, "b", num_experts * n * rb, ab)
        _need(sfa, "sfa", sf_atom_bytes(m, k, 1), E8M0); _need(sfb, "sfb", sf_atom_bytes(n, k, num_experts), E8M0)
        _need(c, "c", 2 * m * 2 * n, torch.bfloat16)
        _need(d_row, "d_row", _out_bytes(dd, m * 2 * n), dd); _need(d_col, "d_col", _out_bytes(dd, m * 2 * n), dd)
        _need(norm_const, "norm_const", 4, torch.float32)
        _need(sfd_row, "sfd_row", sf_atom_bytes(m, 2 * n, 1), E8M0)
        _need(sfd_col, "sfd_col", sf_atom_bytes(2 * n, m, 1), E8M0)
        _need(dprob, "dprob", 4 * m, torch.float32)
    args = [_ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb), _ptr(c), _ptr(padded_offsets), _ptr(alpha), _ptr(beta),
            _ptr(prob), _ptr(norm_const), _ptr(d_row), _ptr(d_col), _ptr(sfd_row), _ptr(sfd_col), _ptr(dprob),
            _ptr(amax), m, n, k, num_experts, ab, cd, dd, sf_vec_size, _major(b_major, "kn", "b_major")]
    if validate_only:
        return lib().bsg_validate_grouped_gemm_dswiglu(*args)
    _check(lib().grouped_gemm_dswiglu(*args, _stream(stream)))


def gemm_proj_rope_mxfp8(x, w, x_scale, w_scale, cos, sin, out_fp8_row, out_scales_row,
                         out_fp8_col, out_scales_col, tokens, q_lora, num_heads=128,
                         head_dim=192, qk_rope=64, in_dtype=BF16, w_out_in=1, stream=None,
                         validate_only=False):
    """Projection GEMM + per-head RoPE + dual MXFP8 quantisation (see include/bsg.h)."""
    if tokens * num_heads > 0:
        nout = num_heads * head_dim
        es = 1 if in_dtype == E4M3 else 2
        kind = E4M3 if in_dtype == E4M3 else torch.bfloat16
        _need(x, "x", es * tokens * q_lora, kind); _need(w, "w", es * nout * q_lora, kind)
        _need(x_scale, "x_scale", tokens * (q_lora // 32), E8M0)
        _need(w_scale, "w_scale", nout * (q_lora // 32), E8M0)
        _need(cos, "cos", 2 * tokens * qk_rope, torch.bfloat16); _need(sin, "sin", 2 * tokens * qk_rope, torch.bfloat16)
        _need(out_fp8_row, "out_fp8_row", tokens * nout, E4M3); _need(out_fp8_col, "out_fp8_col", tokens * nout, E4M3)
        _need(out_scales_row, "out_scales_row", tokens * nout // 32, E8M0)
        _need(out_scales_col, "out_scales_col", (tokens // 32) * nout, E8M0)
    args = [_ptr(x), _ptr(w), _ptr(x_scale), _ptr(w_scale), _ptr(cos), _ptr(sin),
            _ptr(out_fp8_row), _ptr(out_scales_row), _ptr(out_fp8_col), _ptr(out_scales_col),
            tokens, q_lora, num_heads, head_dim, qk_rope, in_dtype, int(w_out_in)]
    if validate_only:
        return lib().bsg_validate_gemm_proj_rope_mxfp8(*args)
    _check(lib().gemm_proj_rope_mxfp8(*args, _stream(stream)))
