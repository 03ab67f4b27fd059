"""The binding's tensor checks on the GPU: a tensor whose dtype, layout or
size disagrees with what the kernel would read or write for the given sizes
is refused before anything is enqueued (the C ABI sees only pointers)."""
import pytest
import torch

import block_scaled_gemm_02_amd as bsg
import workloads as W

pytestmark = pytest.mark.gpu
SHAPE, DTYPE, ALIGN = 2, 3, 4


def grouped_bf16_args(m=512, n=256, k=256, L=2):
    dev = "cuda"
    return dict(a=torch.zeros(m, k, dtype=torch.bfloat16, device=dev),
                b=torch.zeros(L, n, k, dtype=torch.bfloat16, device=dev),
                padded_offsets=torch.tensor([256, 512], dtype=torch.int32, device=dev),
                alpha=torch.ones(L, device=dev), prob=torch.ones(m, device=dev), bias=None,
                c=torch.empty(m, n, dtype=torch.bfloat16, device=dev),
                d=torch.empty(m, n, dtype=torch.bfloat16, device=dev), m=m, n=n, k=k, num_experts=L)


def status_of(fn, **kw):
    with pytest.raises(bsg.BsgError) as e:
        fn(**kw)
    return e.value.status


def test_binding_refuses_mismatched_tensors():
    print("binding tensor checks", flush=True)
    kw = grouped_bf16_args()
    bsg.grouped_gemm(**kw)                       # the well-formed call runs
    torch.cuda.synchronize()
    # a bf16 C declared as fp32 would receive 4 bytes per element: refused
    assert status_of(bsg.grouped_gemm, **kw, c_dtype=torch.float32) == DTYPE
    # too small for M x N
    assert status_of(bsg.grouped_gemm, **{**kw, "d": kw["d"][:256]}) == SHAPE
    # not dense row-major
    assert status_of(bsg.grouped_gemm, **{**kw, "c": torch.empty(256, 512, dtype=torch.bfloat16,
                                                                 device="cuda").t()}) == ALIGN
    # prob must be fp32 with one value per row
    assert status_of(bsg.grouped_gemm, **{**kw, "prob": kw["prob"].double()}) == DTYPE
    assert status_of(bsg.grouped_gemm, **{**kw, "prob": kw["prob"][:100]}) == SHAPE
    # gemm_amax: scale atoms sized for the operands
    m = n = k = 256
    a = torch.zeros(m, k, dtype=torch.uint8, device="cuda")
    sf = torch.full((W.sf_atom_bytes(m, k, 1),), 127, dtype=torch.uint8, device="cuda")
    c = torch.empty(m, n, device="cuda")
    amax = torch.empty(1, device="cuda")
    assert status_of(bsg.gemm_amax, a=a, b=a, sfa=sf[:100], sfb=sf, c=c, amax=amax, m=m, n=n, k=k,
                     l=1) == SHAPE
    assert status_of(bsg.gemm_amax, a=a, b=a, sfa=sf, sfb=sf, c=c.half(), amax=amax, m=m, n=n, k=k,
                     l=1, c_dtype=torch.float32) == DTYPE


@pytest.mark.parametrize("offsets,m,status,words", [
    ([256, 256, 768, 1024], 1024, 0, ""),
    ([0, 0], 0, 0, ""),
    ([256, 300, 512], 512, SHAPE, "not a multiple of 256"),
    ([512, 256, 768], 768, SHAPE, "is below"),
    ([256, 768], 512, SHAPE, "exceeds m"),
    ([-256, 256], 512, SHAPE, "negative"),
])
def test_check_padded_offsets(offsets, m, status, words):
    """The opt-in offsets check reads the device values and names the first
    value that breaks the kernels' contract (multiples of 256 in [0, m],
    nondecreasing)."""
    print(f"check_padded_offsets {offsets} m={m}", flush=True)
    t = torch.tensor(offsets, dtype=torch.int32, device="cuda")
    if status == 0:
        bsg.check_padded_offsets(t, m)
    else:
        with pytest.raises(bsg.BsgError) as e:
            bsg.check_padded_offsets(t, m)
        assert e.value.status == status and words in str(e.value), str(e.value)
