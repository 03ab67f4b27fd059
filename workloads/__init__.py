"""Seeded synthetic inputs for the block-scaled GEMM family.

This module only *draws* inputs: operand codes, scale-factor bytes, expert
row ranges, per-expert alpha, per-row prob, bias and RoPE tables.  It holds
none of the arithmetic the GEMM path computes (no decode of a scale factor,
no contraction, no epilogue, no output quantiser, no scale-atom addressing):
both the CPU oracle and the HIP path consume what it returns.

Shapes and layouts follow the problem statements of the cuDNN frontend
"GEMM fusions" pages:
  * "GEMM + Amax (SM100)", Shapes / Parameters: A (M,K,L) and B (N,K,L)
    k-major, i.e. memory order [L][rows][K]; SFA/SFB scale-atom buffers of
    32*4*ceil(MN/128)*4*ceil(K/128)*L bytes.
  * "Grouped GEMM + sReLU (SM100)", Shapes: A (valid_m,K), B (N,K,L),
    padded_offsets int32 cumulative padded ends, alpha (L,), prob (valid_m,).
  * "Grouped GEMM (SM100 BF16)", Tensors and layouts: bias (N,L) with stride
    (1,N), i.e. memory order [L][N].
  * "GEMM + RoPE + MXFP8 Projection (SM100)", Shapes: x (tokens,Q_LORA),
    w [out,in], cos/sin (tokens,64) bf16.

Scale-factor bytes are drawn directly as bytes over the whole atom buffer
(padding bytes included), so no atom addressing is needed here.  Operand
codes are drawn in code space: each 32-element K block of a normal draw is
stretched so its largest magnitude lands on the format's largest finite
value, then rounded to the format by torch's own float8 conversion (E4M3) or
by nearest-magnitude bucketing (E2M1).  The drawn scale byte of that block is
independent of the block's content, so dequantised operands are normal-like
with a per-block magnitude jitter of a factor of two either way.

Every generator takes a seed and a device; the same seed on the same device
type gives the same bytes.  Large configurations are drawn on the GPU with a
seeded torch.Generator; small ones on the CPU.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

E4M3 = "e4m3"
E2M1 = "e2m1"
E5M2 = "e5m2"

# Largest finite magnitude of each operand format (OCP MX formats).
_FMT_MAX = {E4M3: 448.0, E2M1: 6.0, E5M2: 57344.0}
# scale byte that puts a block-stretched N(0,1) draw back near unit size
_SF_CENTRE = {E4M3: 120, E2M1: 126, E5M2: 113}
# Decision points between adjacent E2M1 magnitudes {0,.5,1,1.5,2,3,4,6}.
_E2M1_EDGES = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def sf_atom_bytes(mn: int, k: int, l: int, sf_vec: int = 32) -> int:
    """Byte count of a (32,4,ceil(MN/128),4,ceil(ceil(K/sf)/4),L) atom buffer."""
    return 32 * 4 * ceil_div(mn, 128) * 4 * ceil_div(ceil_div(k, sf_vec), 4) * l


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _codes_from_normal(x: torch.Tensor, fmt: str) -> torch.Tensor:
    """Normal draws (..., K) -> uint8 code bytes, block-stretched to the format max.

    E4M3 and E5M2 return one byte per element; E2M1 returns two elements per
    byte, element 2j in the low nibble and 2j+1 in the high nibble.
    """
    *lead, k = x.shape
    blk = x.reshape(*lead, k // 32, 32)
    amax = blk.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    y = (blk / amax * _FMT_MAX[fmt]).reshape(*lead, k)
    if fmt == E4M3:
        y = y.clamp(-448.0, 448.0)
        return y.to(torch.float8_e4m3fn).view(torch.uint8)
    if fmt == E5M2:
        y = y.clamp(-57344.0, 57344.0)
        return y.to(torch.float8_e5m2).view(torch.uint8)
    edges = torch.tensor(_E2M1_EDGES, device=y.device, dtype=y.dtype)
    mag = torch.bucketize(y.abs(), edges).to(torch.uint8)          # 0..7
    code = mag | ((y < 0).to(torch.uint8) << 3)
    code = torch.where(mag == 0, torch.zeros_like(code), code)     # no -0
    pairs = code.reshape(*lead, k // 2, 2)
    return pairs[..., 0] | (pairs[..., 1] << 4)


def _sf_bytes(n: int, centre: int, spread: int, g: torch.Generator, device) -> torch.Tensor:
    return torch.randint(centre - spread, centre + spread + 1, (n,), generator=g,
                         device=device, dtype=torch.int32).to(torch.uint8)


def zipf_padded_offsets(tokens: int, experts: int, exponent: float, align: int,
                        seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Expert row ranges of a Zipf-popularity top-k routing.

    Row counts are one multinomial draw of `tokens` over experts with
    p_g proportional to (g+1)^-exponent; each count is padded up to a multiple
    of `align`.  Returns the int32 cumulative padded ends and the int64 counts.
    """
    rng = np.random.default_rng(seed)
    p = (np.arange(1, experts + 1, dtype=np.float64)) ** (-exponent)
    p /= p.sum()
    counts = rng.multinomial(tokens, p)
    padded = ((counts + align - 1) // align) * align
    return np.cumsum(padded).astype(np.int32), counts.astype(np.int64)


@dataclass
class Problem:
    """A bag of named tensors plus scalar sizes for one call of one entry point."""
    op: str
    sizes: dict
    t: dict = field(default_factory=dict)

    def to(self, device):
        self.t = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in self.t.items()}
        return self


def row_valid_mask(offsets: np.ndarray, counts: np.ndarray, m: int) -> np.ndarray:
    """True for routed rows, False for padding rows of each expert range."""
    mask = np.zeros(m, dtype=bool)
    begin = 0
    for end, c in zip(offsets.tolist(), counts.tolist()):
        mask[begin:begin + c] = True
        begin = end
    return mask


# ---------------------------------------------------------------------------
# Dense block-scaled GEMM + amax
# ---------------------------------------------------------------------------
def gemm_amax_problem(m: int, n: int, k: int, l: int, fmt: str = E4M3, *, seed: int = 0,
                      device="cpu", sf_centre: int | None = None, sf_spread: int = 3,
                      plain_round: bool = False, c_dtype: str = "f32") -> Problem:
    """A (M,K,L), B (N,K,L) codes in memory order [L][rows][K] plus SF atom buffers.

    plain_round=True rounds N(0,1) straight to E4M3 (small 256^3 workload);
    otherwise each 32-block is stretched to the format max (MX-style data).
    sf_centre defaults to the byte that puts block maxima near N(0,1) scale.
    """
    g = _gen(seed, device)
    if sf_centre is None:
        sf_centre = 127 if plain_round else _SF_CENTRE[fmt]
    xa = torch.randn(l, m, k, generator=g, device=device)
    xb = torch.randn(l, n, k, generator=g, device=device)
    if plain_round:
        assert fmt == E4M3
        a = xa.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        b = xb.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    else:
        a = _codes_from_normal(xa, fmt)
        b = _codes_from_normal(xb, fmt)
    del xa, xb
    sfa = _sf_bytes(sf_atom_bytes(m, k, l), sf_centre, sf_spread, g, device)
    sfb = _sf_bytes(sf_atom_bytes(n, k, l), sf_centre, sf_spread, g, device)
    return Problem("gemm_amax", dict(m=m, n=n, k=k, l=l, fmt=fmt, c_dtype=c_dtype),
                   dict(a=a.contiguous(), b=b.contiguous(), sfa=sfa, sfb=sfb))


# ---------------------------------------------------------------------------
# Grouped block-scaled GEMM + sReLU
# ---------------------------------------------------------------------------
def grouped_srelu_problem(tokens: int, experts: int, n: int, k: int, fmt: str = E4M3, *,
                          seed: int = 0, device="cpu", tanh_clamp: float = 32.0,
                          d_dtype: str = "bf16", zipf: float = 1.1, align: int = 256,
                          offsets: np.ndarray | None = None, extra_rows: int = 0) -> Problem:
    """Grouped MXFP8/MXFP4 operands over Zipf-routed expert ranges.

    A (M,K) codes with zero codes on padding rows; B (N,K,L) codes stored
    [L][N][K]; SFA (atoms over M), SFB (atoms over N, per expert); alpha
    U(0.5,1.5); prob U(0,1) with 0 on padding rows.  B is drawn from
    N(0,0.02): its scale bytes sit 6 binades below A's.
    """
    if offsets is None:
        offsets, counts = zipf_padded_offsets(tokens, experts, zipf, align, seed)
    else:
        offsets = np.asarray(offsets, dtype=np.int32)
        counts = np.diff(np.concatenate([[0], offsets])).astype(np.int64)
    valid_m = int(offsets[-1]) if len(offsets) else 0
    m = valid_m + extra_rows
    g = _gen(seed + 1, device)
    xa = torch.randn(m, k, generator=g, device=device)
    a = _codes_from_normal(xa, fmt)
    del xa
    mask = torch.from_numpy(row_valid_mask(offsets, counts, m)).to(device)
    a = torch.where(mask[:, None], a, torch.zeros_like(a))
    xb = torch.randn(experts, n, k, generator=g, device=device)
    b = _codes_from_normal(xb, fmt)
    del xb
    centre_a = _SF_CENTRE[fmt]
    sfa = _sf_bytes(sf_atom_bytes(max(m, 1), k, 1), centre_a, 1, g, device)
    sfb = _sf_bytes(sf_atom_bytes(n, k, experts), centre_a - 6, 1, g, device)
    alpha = torch.rand(experts, generator=g, device=device) + 0.5
    prob = torch.rand(m, generator=g, device=device) * mask.float()
    return Problem("grouped_gemm_srelu",
                   dict(m=m, n=n, k=k, l=experts, fmt=fmt, valid_m=valid_m,
                        tanh_clamp=tanh_clamp, d_dtype=d_dtype, norm_const=1.0),
                   dict(a=a.contiguous(), b=b.contiguous(), sfa=sfa, sfb=sfb,
                        offsets=torch.from_numpy(offsets.copy()).to(device),
                        alpha=alpha, prob=prob,
                        norm_const=torch.ones(1, device=device)))


def grouped_dswiglu_problem(tokens: int, experts: int, n: int, k: int, fmt: str = E4M3, *,
                            seed: int = 0, device="cpu", offsets: np.ndarray | None = None,
                            extra_rows: int = 0) -> Problem:
    """Grouped GEMM + dSwiGLU backward operands: the grouped sReLU problem's
    A, B, scales, routing, alpha and prob, plus beta U(0.5,1.5) per expert and
    the forward tensor C (M, 2N) bf16 N(0,1) (input and gate in 32-column
    blocks), zero on padding rows; MXFP8 output with norm_const 1."""
    p = grouped_srelu_problem(tokens, experts, n, k, fmt, seed=seed, device=device, offsets=offsets,
                              extra_rows=extra_rows, d_dtype="e4m3")
    m = p.sizes["m"]
    g = _gen(seed + 5, device)
    beta = torch.rand(experts, generator=g, device=device) + 0.5
    c = torch.randn(m, 2 * n, generator=g, device=device)
    routed = p.t["prob"] > 0                      # prob is 0 exactly on padding rows
    c = torch.where(routed[:, None], c, torch.zeros_like(c)).to(torch.bfloat16)
    p.op = "grouped_gemm_dswiglu"
    p.t["beta"] = beta
    p.t["c"] = c.contiguous()
    return p


# ---------------------------------------------------------------------------
# Unfused BF16 grouped GEMM
# ---------------------------------------------------------------------------
def grouped_bf16_problem(tokens: int, experts: int, n: int, k: int, *, seed: int = 0,
                         device="cpu", with_bias: bool = True, zipf: float = 1.1,
                         align: int = 256, offsets: np.ndarray | None = None,
                         extra_rows: int = 0) -> Problem:
    """A (M,K) bf16 N(0,1), zero padding rows; B (N,K,L) bf16 N(0,0.02) stored
    [L][N][K]; alpha U(0.5,1.5); prob U(0,1) zero on padding; bias (N,L) bf16
    N(0,0.1) stored [L][N]."""
    if offsets is None:
        offsets, counts = zipf_padded_offsets(tokens, experts, zipf, align, seed)
    else:
        offsets = np.asarray(offsets, dtype=np.int32)
        counts = np.diff(np.concatenate([[0], offsets])).astype(np.int64)
    valid_m = int(offsets[-1]) if len(offsets) else 0
    m = valid_m + extra_rows
    g = _gen(seed + 2, device)
    mask = torch.from_numpy(row_valid_mask(offsets, counts, m)).to(device)
    a = torch.randn(m, k, generator=g, device=device).to(torch.bfloat16)
    a = torch.where(mask[:, None], a, torch.zeros_like(a))
    b = (torch.randn(experts, n, k, generator=g, device=device) * 0.02).to(torch.bfloat16)
    alpha = torch.rand(experts, generator=g, device=device) + 0.5
    prob = torch.rand(m, generator=g, device=device) * mask.float()
    bias = (torch.randn(experts, n, generator=g, device=device) * 0.1).to(torch.bfloat16)
    t = dict(a=a.contiguous(), b=b.contiguous(),
             offsets=torch.from_numpy(offsets.copy()).to(device),
             alpha=alpha, prob=prob, bias=bias.contiguous() if with_bias else None)
    return Problem("grouped_gemm", dict(m=m, n=n, k=k, l=experts, valid_m=valid_m), t)


# ---------------------------------------------------------------------------
# Projection GEMM + RoPE + dual MXFP8
# ---------------------------------------------------------------------------
def rope_tables(tokens: int, rope_dim: int = 64, base: float = 10000.0, device="cpu"):
    """bf16 cos/sin (tokens, rope_dim) for positions 0..tokens-1.

    Frequencies inv_f_j = base^(-j/(rope_dim/2)) for j < rope_dim/2; angle
    t*inv_f_j evaluated in float64; the table repeats the half-width row
    (column j and j+rope_dim/2 hold the same angle), rounded to bf16.
    """
    half = rope_dim // 2
    j = np.arange(half, dtype=np.float64)
    inv_f = base ** (-j / half)
    ang = np.arange(tokens, dtype=np.float64)[:, None] * inv_f[None, :]
    ang = np.concatenate([ang, ang], axis=1)
    cos = torch.from_numpy(np.cos(ang)).to(torch.bfloat16)
    sin = torch.from_numpy(np.sin(ang)).to(torch.bfloat16)
    return cos.to(device).contiguous(), sin.to(device).contiguous()


def rope_tables_random(tokens: int, rope_dim: int = 64, seed: int = 0, device="cpu"):
    """bf16 cos/sin (tokens, rope_dim) of independent angles U(-pi, pi) per
    (token, column), returned with the fp64 angles: unlike rope_tables, the
    two halves of a row differ and every row differs, so a table read from
    the wrong column or the wrong row gives different values."""
    rng = np.random.default_rng(seed)
    ang = rng.uniform(-np.pi, np.pi, size=(tokens, rope_dim))
    cos = torch.from_numpy(np.cos(ang)).to(torch.bfloat16)
    sin = torch.from_numpy(np.sin(ang)).to(torch.bfloat16)
    return cos.to(device).contiguous(), sin.to(device).contiguous(), ang


def proj_rope_problem(tokens: int, q_lora: int, heads: int = 128, head_dim: int = 192,
                      qk_rope: int = 64, *, seed: int = 0, device="cpu",
                      w_out_in: bool = True, in_dtype: str = "bf16") -> Problem:
    """x (tokens,Q_LORA) bf16 N(0,1); w bf16 N(0,0.02), [out,in] when w_out_in
    else [in,out]; bf16 cos/sin (tokens,qk_rope) from positions, base 10000.

    in_dtype "e4m3" (MXFP8 inputs): x and w are E4M3 codes of block-stretched
    normal draws with row-major E8M0 scale bytes x_scale (tokens, Q_LORA/32)
    and w_scale (out, Q_LORA/32), drawn around the bytes that give N(0,1) and
    N(0,0.02) magnitudes (w six binades below x); with w [in,out] both w and
    w_scale are stored transposed, (Q_LORA, out) and (Q_LORA/32, out)."""
    g = _gen(seed + 3, device)
    extra = {}
    if in_dtype == E4M3:
        x = _codes_from_normal(torch.randn(tokens, q_lora, generator=g, device=device), E4M3)
        w = _codes_from_normal(torch.randn(heads * head_dim, q_lora, generator=g, device=device), E4M3)
        extra["x_scale"] = _sf_bytes(tokens * (q_lora // 32), 120, 1, g, device).reshape(tokens, q_lora // 32)
        extra["w_scale"] = _sf_bytes(heads * head_dim * (q_lora // 32), 114, 1, g, device).reshape(
            heads * head_dim, q_lora // 32)
        if not w_out_in:
            w = w.t().contiguous()
            extra["w_scale"] = extra["w_scale"].t().contiguous()
    else:
        x = torch.randn(tokens, q_lora, generator=g, device=device).to(torch.bfloat16)
        w = (torch.randn(heads * head_dim, q_lora, generator=g, device=device) * 0.02).to(torch.bfloat16)
        if not w_out_in:
            w = w.t().contiguous()
    cos, sin = rope_tables(tokens, qk_rope, device=device)
    return Problem("gemm_proj_rope_mxfp8",
                   dict(tokens=tokens, q_lora=q_lora, heads=heads, head_dim=head_dim,
                        qk_rope=qk_rope, w_out_in=int(w_out_in), in_dtype=in_dtype),
                   dict(x=x.contiguous(), w=w.contiguous(), cos=cos, sin=sin, **extra))


# ---------------------------------------------------------------------------
# The five named workloads (full size) and their reduced parity variants.
# ---------------------------------------------------------------------------
def dense_256(device="cpu", seed=0):
    """Dense E4M3 GEMM + amax, L=1, M=N=K=256, plain-rounded N(0,1), SF 127+U{-3..3}, C fp32."""
    return gemm_amax_problem(256, 256, 256, 1, E4M3, seed=seed, device=device,
                             plain_round=True, sf_centre=127, sf_spread=3, c_dtype="f32")


def dense_8192(fmt=E4M3, device="cuda", seed=0, size=8192, batch=4):
    """Batched dense MXFP8/MXFP4 GEMM + amax, M=N=K=8192, L=4, C bf16."""
    return gemm_amax_problem(size, size, size, batch, fmt, seed=seed, device=device,
                             sf_spread=1, c_dtype="bf16")


def moe_bf16(device="cuda", seed=0, tokens=16384 * 8, experts=64, n=2048, k=7168, **kw):
    """BF16 MoE grouped GEMM: 16384 tokens x top-8 over 64 experts, N=2048, K=7168."""
    return grouped_bf16_problem(tokens, experts, n, k, seed=seed, device=device, **kw)


def moe_mxfp8_srelu(device="cuda", seed=0, tokens=28672, experts=32, n=4096, k=7168,
                    d_dtype="bf16", fmt=E4M3, **kw):
    """Grouped MXFP8 + sReLU: 32 experts, N=4096, K=7168, valid_m ~ 32768, s=32
    (fmt E2M1: the same problem with MXFP4 operands)."""
    return grouped_srelu_problem(tokens, experts, n, k, fmt, seed=seed, device=device,
                                 tanh_clamp=32.0, d_dtype=d_dtype, **kw)


def proj_rope_dsv3(device="cuda", seed=0, tokens=4096, in_dtype="bf16", w_out_in=True):
    """DeepSeek-V3 Q up-projection: x (4096,1536), 128 heads x 192, rope on trailing 64;
    w as [out, in] (w_out_in) or [in, out]."""
    return proj_rope_problem(tokens, 1536, 128, 192, 64, seed=seed, device=device, in_dtype=in_dtype,
                             w_out_in=w_out_in)
