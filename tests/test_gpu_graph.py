"""The entry points inside a captured HIP graph.  Each call enqueues kernels
only (the amax zero fill is a kernel of the library, not a memset; dprob is
cleared by the caller with torch's fill kernel), so a graph can capture it.
Every replay is checked against the eager result of the same call, with
eager work of the same op and a synchronisation between replays, and the
graph's outputs are reset to sentinels before each replay so that a replay
that wrote nothing would show."""
import numpy as np
import pytest
import torch

import block_scaled_gemm_02_amd as bsg
import workloads as W

pytestmark = pytest.mark.gpu
REPLAYS = 3


def say(msg):
    print(msg, flush=True)


def capture(enqueue):
    """Capture enqueue() (which launches into fixed buffers) in a graph, after
    one warm-up call on a side stream, as torch requires."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        enqueue()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enqueue()
    torch.cuda.synchronize()
    return g


def replay_and_compare(g, outs, sentinels, eager_outs, eager_again, exact=None, close=None):
    """Replay g REPLAYS times; before each, reset outs to their sentinels;
    after each, run eager_again() (the same op into other buffers) and
    compare.  exact: indices compared bit for bit; close: (index, rtol)."""
    exact = range(len(outs)) if exact is None else exact
    for r in range(REPLAYS):
        for o, s in zip(outs, sentinels):
            o.fill_(s)
        torch.cuda.synchronize()
        g.replay()
        eager_again()
        torch.cuda.synchronize()
        for i in exact:
            assert torch.equal(outs[i].view(torch.uint8), eager_outs[i].view(torch.uint8)), (r, i)
        for i, rtol in close or ():
            torch.testing.assert_close(outs[i], eager_outs[i], rtol=rtol, atol=rtol * float(eager_outs[i].abs().max()))
        say(f"  replay {r}: equal to the eager call")


def test_graph_gemm_amax():
    say("graph: gemm_amax MXFP8, bf16 C, 2 x 512 x 384 x 512")
    p = W.gemm_amax_problem(512, 384, 512, 2, "e4m3", seed=11, device="cuda")
    t, s = p.t, p.sizes
    m, n, k, L = s["m"], s["n"], s["k"], s["l"]

    def call(c, amax):
        bsg.gemm_amax(t["a"], t["b"], t["sfa"], t["sfb"], c, amax, m, n, k, L, "e4m3")

    ce = torch.empty(L, m, n, dtype=torch.bfloat16, device="cuda")
    ae = torch.empty(1, device="cuda")
    call(ce, ae)
    cg = torch.empty_like(ce)
    ag = torch.empty_like(ae)
    g = capture(lambda: call(cg, ag))
    cx, ax = torch.empty_like(ce), torch.empty_like(ae)
    replay_and_compare(g, [cg, ag], [float("nan"), -1.0], [ce, ae], lambda: call(cx, ax))


def test_graph_grouped_srelu():
    say("graph: grouped_gemm_srelu MXFP8, bf16 C/D, per-expert amax")
    off = np.cumsum([256, 0, 512, 256]).astype(np.int32)
    p = W.grouped_srelu_problem(0, 4, 320, 256, "e4m3", seed=12, device="cuda", offsets=off, extra_rows=256)
    t, s = p.t, p.sizes
    m, n, k, L = s["m"], s["n"], s["k"], s["l"]

    def call(c, d, amax):
        bsg.grouped_gemm_srelu(t["a"], t["b"], t["sfa"], t["sfb"], t["offsets"], t["alpha"], t["prob"],
                               None, c, d, None, None, None, amax, m, n, k, L, "e4m3",
                               c_dtype=torch.bfloat16, d_dtype=torch.bfloat16, tanh_clamp_scale=32.0)

    bufs = lambda: (torch.full((m, n), 7.0, dtype=torch.bfloat16, device="cuda"),
                    torch.full((m, n), 7.0, dtype=torch.bfloat16, device="cuda"),
                    torch.empty(L, device="cuda"))
    e = bufs()
    call(*e)
    gb = bufs()
    g = capture(lambda: call(*gb))
    x = bufs()
    # rows past valid_m are never written: their sentinel must equal the eager buffers' 7.0
    replay_and_compare(g, list(gb), [7.0, 7.0, -1.0], list(e), lambda: call(*x))


def test_graph_grouped_dswiglu():
    say("graph: grouped_gemm_dswiglu MXFP8, MXFP8 D, dprob cleared inside the graph")
    off = np.cumsum([512, 256]).astype(np.int32)
    p = W.grouped_dswiglu_problem(0, 2, 256, 384, "e4m3", seed=13, device="cuda", offsets=off)
    t, s = p.t, p.sizes
    m, n, k, L = s["m"], s["n"], s["k"], s["l"]

    def bufs():
        return (torch.zeros(m, 2 * n, dtype=torch.uint8, device="cuda"),
                torch.zeros(m, 2 * n, dtype=torch.uint8, device="cuda"),
                torch.zeros(W.sf_atom_bytes(m, 2 * n, 1), dtype=torch.uint8, device="cuda"),
                torch.zeros(W.sf_atom_bytes(2 * n, m, 1), dtype=torch.uint8, device="cuda"),
                torch.zeros(m, device="cuda"))

    def call(d, dc, sr, sc, dprob):
        dprob.zero_()                       # a fill kernel: capturable, unlike a memset node
        bsg.grouped_gemm_dswiglu(t["a"], t["b"], t["sfa"], t["sfb"], t["c"], t["offsets"], t["alpha"],
                                 t["beta"], t["prob"], t["norm_const"], d, dc, sr, sc, dprob, m, n, k, L,
                                 "e4m3", d_dtype="e4m3")

    e = bufs()
    call(*e)
    gb = bufs()
    g = capture(lambda: call(*gb))
    x = bufs()
    # dprob adds two half-rows with atomics: compared to a relative 1e-6
    replay_and_compare(g, list(gb), [0xEE, 0xEE, 0xEE, 0xEE, float("nan")], list(e), lambda: call(*x),
                       exact=range(4), close=[(4, 1e-6)])


def test_graph_proj_rope():
    say("graph: gemm_proj_rope_mxfp8, BF16 inputs, 256 tokens x 8 heads, q_lora 512")
    p = W.proj_rope_problem(256, 512, heads=8, seed=14, device="cuda")
    t, s = p.t, p.sizes
    T, H, D = s["tokens"], s["heads"], s["head_dim"]

    def bufs():
        return (torch.zeros(T, H, D, dtype=torch.uint8, device="cuda"),
                torch.zeros(T, H, D // 32, dtype=torch.uint8, device="cuda"),
                torch.zeros(T, H, D, dtype=torch.uint8, device="cuda"),
                torch.zeros(T // 32, H, D, dtype=torch.uint8, device="cuda"))

    def call(qr, sr, qc, sc):
        bsg.gemm_proj_rope_mxfp8(t["x"], t["w"], None, None, t["cos"], t["sin"], qr, sr, qc, sc, T,
                                 s["q_lora"], H, D, s["qk_rope"], in_dtype=bsg.BF16, w_out_in=1)

    e = bufs()
    call(*e)
    gb = bufs()
    g = capture(lambda: call(*gb))
    x = bufs()
    replay_and_compare(g, list(gb), [0xEE] * 4, list(e), lambda: call(*x))
