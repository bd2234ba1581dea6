"""Decode steps captured in a HIP graph (torch.cuda.graph) and replayed: the
inner loop of generation is a few short launches per token, so one graph
launch per token takes the host's launch cost out of it. Every replay must
equal, bit for bit, the same calls made eagerly (same kernels, same inputs).
Between replays the test does its own eager work (copying the next token's
inputs into the graph's buffers, a synchronisation) and checks each replay;
nothing in these calls allocates, clears memory or synchronises."""
import pytest
import torch

from selective_state_space_48_amd import selscan

pytestmark = pytest.mark.gpu


def case(msg):
    print(f"[case] {msg}", flush=True)


def _replay_all(graph, buf, toks, outs, expect):
    for t, k in enumerate(toks):
        for n in buf:
            buf[n].copy_(k[n])
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, expect[t]):
            assert torch.equal(o, e), f"replay {t}"


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_block_decode_step_graph(dtype, fused):
    """The Mamba block's decode step: the convolution's step, then the scan's
    (or the scan's step with the convolution fused in front)."""
    batch, dim, N, T = 4, 320, 16, 6
    case(f"graph: block decode step b{batch} d{dim} {dtype} fused={fused}")
    g = torch.Generator(device="cuda").manual_seed(11)
    rn = lambda *s: torch.randn(s, device="cuda", generator=g)
    A = -torch.exp(0.5 * rn(dim, N))
    D, cw, cb = rn(dim), 0.5 * rn(dim, 4), 0.1 * rn(dim)
    toks = [dict(x=rn(batch, dim).to(dtype), delta=(rn(batch, dim) - 1).to(dtype),
                 z=rn(batch, dim).to(dtype), B=rn(batch, N).to(dtype), C=rn(batch, N).to(dtype))
            for _ in range(T)]
    cst0, st0 = rn(batch, dim, 3), 0.1 * rn(batch, dim, N)

    cst, st = cst0.clone(), st0.clone()
    expect = []
    def token(k, cst, st, xa=None, y=None):
        if fused:
            y = selscan.step(st, k["x"], k["delta"], A, k["B"], k["C"], D=D, z=k["z"], y=y,
                             conv_w=cw, conv_b=cb, conv_state=cst)
            return y, y
        xa = selscan.conv1d_step(cst, k["x"], cw, cb, out=xa)
        return xa, selscan.step(st, xa, k["delta"], A, k["B"], k["C"], D=D, z=k["z"], y=y)

    for k in toks:
        xa, y = token(k, cst, st)
        expect.append((xa.clone(), y.clone()))
    torch.cuda.synchronize()
    cst_e, st_e = cst.clone(), st.clone()

    buf = {n: torch.empty_like(v) for n, v in toks[0].items()}
    cst, st = cst0.clone(), st0.clone()
    xa, y = torch.empty_like(toks[0]["x"]), torch.empty_like(toks[0]["x"])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        token(buf, cst, st, xa, y)
    assert torch.equal(st, st0) and torch.equal(cst, cst0)  # capture runs nothing
    _replay_all(graph, buf, toks, (y, y) if fused else (xa, y), expect)
    assert torch.equal(st, st_e) and torch.equal(cst, cst_e)


def test_ssd_decode_step_graph():
    batch, H, N, P, T = 3, 8, 128, 64, 5
    case(f"graph: SSD decode step b{batch} h{H} n{N}")
    g = torch.Generator(device="cuda").manual_seed(12)
    rn = lambda *s: torch.randn(s, device="cuda", generator=g)
    bf = torch.bfloat16
    A, D, dtb = -1.0 - 15.0 * torch.rand(H, device="cuda", generator=g), rn(H), rn(H) - 3.0
    toks = [dict(x=rn(batch, H, P).to(bf), delta=rn(batch, H).to(bf), B=rn(batch, N).to(bf),
                 C=rn(batch, N).to(bf)) for _ in range(T)]
    st0 = 0.1 * rn(batch, H, N, P)

    st = st0.clone()
    expect = []
    for k in toks:
        y = selscan.ssd_step(st, k["x"], k["delta"], A, k["B"], k["C"], D=D, dt_bias=dtb)
        expect.append((y.clone(),))
    torch.cuda.synchronize()
    st_e = st.clone()

    buf = {n: torch.empty_like(v) for n, v in toks[0].items()}
    st = st0.clone()
    y = torch.empty_like(toks[0]["x"])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        selscan.ssd_step(st, buf["x"], buf["delta"], A, buf["B"], buf["C"], D=D, dt_bias=dtb, y=y)
    assert torch.equal(st, st0)
    _replay_all(graph, buf, toks, (y,), expect)
    assert torch.equal(st, st_e)
