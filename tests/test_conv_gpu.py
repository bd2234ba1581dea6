"""GPU parity of the causal depthwise convolution (width 4) + SiLU and its
decode step against the fp64 oracle on the same seeded inputs: small and
ragged shapes on both code paths (16-byte rows and element rows), carried-in
inputs, streaming splits, in-place state, steps against one call, and the
full headline-shaped tensor. Error measure as for the scan: |gpu - ref| over
the oracle's magnitude sum of the pre-activation terms."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import TDT, TOL, dev, to_np
from selective_state_space_48_amd import selscan
from selective_state_space_48_amd import workloads as W

pytestmark = pytest.mark.gpu


def case(msg):
    print(f"[case] {msg}", flush=True)


def _inputs(batch, L, dim, dtype, seed=0):
    w = W.scaled(W.get(W.HEADLINE if dtype == "bf16" else "m130m_f32_b8_l2048_d1536"),
                 batch=batch, seqlen=L, dim=dim, seed=seed)
    return W.conv_inputs(w)


def _gpu(p, dtype, with_bias=True, with_prev=True, **kw):
    td = TDT[dtype]
    out, last = selscan.conv1d(dev(p["x"], td), dev(p["w"]), dev(p["bias"]) if with_bias else None,
                               dev(p["x_prev"]) if with_prev else None, **kw)
    torch.cuda.synchronize()
    return out, last


def _ref(p, with_bias=True, with_prev=True):
    return oracle.conv1d(p["x"], p["w"], p["bias"] if with_bias else None,
                         p["x_prev"] if with_prev else None)


def _check(out, last, ref, dtype, what):
    err = oracle.scaled_error(to_np(out), ref["out"], ref["out_scale"])
    print(f"[parity] {what}: err={err:.3e} tol={TOL[dtype]:.0e}", flush=True)
    assert err <= TOL[dtype], f"{what}: err {err:.3e}"
    if last is not None:
        assert np.array_equal(to_np(last), ref["x_last"]), f"{what}: x_last differs"


SHAPES = [
    # (batch, L, dim, dtype)
    (1, 1, 1, "f32"),
    (1, 2, 3, "bf16"),       # shorter than the window: x_last reaches into x_prev
    (2, 3, 5, "f32"),
    (2, 64, 7, "bf16"),      # 16-byte rows
    (3, 37, 70, "f32"),      # rows off a 16-byte boundary: aligned blocks shifted
    (2, 45, 66, "bf16"),     # rows off a 16-byte boundary
    (1, 1000, 130, "bf16"),  # many waves per row
    (2, 516, 33, "f32"),
    (3, 2047, 96, "bf16"),   # every byte offset of a row start, blocks across wave edges
    (2, 1001, 70, "f32"),
    (4, 7, 50, "bf16"),      # rows shorter than a vector
]


@pytest.mark.parametrize("batch,L,dim,dtype", SHAPES)
def test_conv_shapes(batch, L, dim, dtype):
    p = _inputs(batch, L, dim, dtype, seed=L)
    for with_bias, with_prev in ((True, True), (False, False), (True, False)):
        case(f"conv b{batch} L{L} d{dim} {dtype} bias={with_bias} prev={with_prev}")
        out, last = _gpu(p, dtype, with_bias, with_prev)
        _check(out, last, _ref(p, with_bias, with_prev), dtype,
               f"b{batch} L{L} d{dim} bias={with_bias} prev={with_prev}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_streaming_split(dtype):
    """[0, t) then [t, L) with x_prev = the first call's x_last gives the same
    bits as one call (the carried inputs are exact fp32 copies)."""
    p = _inputs(2, 200, 48, dtype, seed=3)
    td = TDT[dtype]
    whole, wlast = _gpu(p, dtype)
    x = dev(p["x"], td)
    for t in (1, 2, 8, 77):
        case(f"conv split at {t} {dtype}")
        a, alast = selscan.conv1d(x[..., :t].contiguous(), dev(p["w"]), dev(p["bias"]),
                                  dev(p["x_prev"]))
        b, blast = selscan.conv1d(x[..., t:].contiguous(), dev(p["w"]), dev(p["bias"]), alast)
        torch.cuda.synchronize()
        assert torch.equal(torch.cat([a, b], -1), whole) and torch.equal(blast, wlast)


def test_conv_state_in_place_and_empty():
    p = _inputs(2, 50, 32, "f32", seed=4)
    case("conv x_last is x_prev")
    st = dev(p["x_prev"])
    out, last = selscan.conv1d(dev(p["x"]), dev(p["w"]), dev(p["bias"]), st, x_last=st)
    torch.cuda.synchronize()
    _check(out, last, _ref(p), "f32", "in place")
    case("conv L = 0")
    st = dev(p["x_prev"])
    out, last = selscan.conv1d(torch.empty((2, 32, 0), device="cuda"), dev(p["w"]), None, st)
    torch.cuda.synchronize()
    assert out.shape == (2, 32, 0) and torch.equal(last, st)
    out, last = selscan.conv1d(torch.empty((0, 32, 9), device="cuda"), dev(p["w"]))
    torch.cuda.synchronize()
    assert out.shape == (0, 32, 9)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_steps(dtype):
    """Decode steps against the oracle's step, and L steps against one call
    (same arithmetic in the same order: equal bits)."""
    w = W.scaled(W.get(W.DECODE), batch=8, dim=256) if dtype == "bf16" else \
        W.scaled(W.get(W.DECODE), batch=8, dim=256, dtype="f32")
    p = W.conv_inputs(W.scaled(w, seqlen=12, kind="fwd"))
    td = TDT[dtype]
    st = dev(p["x_prev"])
    ref_state = p["x_prev"].astype(np.float64)
    whole, wlast = _gpu(p, dtype)
    for t in range(12):
        case(f"conv step {t} {dtype}")
        xt = dev(np.ascontiguousarray(p["x"][..., t]), td)
        out = selscan.conv1d_step(st, xt, dev(p["w"]), dev(p["bias"]))
        torch.cuda.synchronize()
        r = oracle.conv1d_step(ref_state, p["x"][..., t], p["w"], p["bias"])
        err = oracle.scaled_error(to_np(out), r["out"], r["out_scale"])
        assert err <= TOL[dtype], f"step {t}: {err:.3e}"
        assert np.array_equal(to_np(st), r["conv_state"])
        assert torch.equal(out, whole[..., t])
        ref_state = r["conv_state"]
    assert torch.equal(st, wlast)


def test_conv_headline_shape_full():
    """The whole headline-shaped tensor (batch 8, L 2048, d_inner 4096, bf16)
    against the oracle, every element."""
    w = W.get(W.HEADLINE)
    p = W.conv_inputs(w)
    case("conv full b8 L2048 d4096 bf16")
    out, last = _gpu(p, "bf16")
    _check(out, last, _ref(p), "bf16", "headline shape")


def test_conv_decode_shape_steps():
    """The decode shape (batch 256, d_inner 5120, bf16): 4 steps, every row."""
    w = W.get(W.DECODE)
    p = W.conv_inputs(W.scaled(w, seqlen=1, kind="fwd"))
    st = dev(p["x_prev"])
    ref_state = p["x_prev"]
    for s in range(4):
        case(f"conv decode step {s} b256 d5120 bf16")
        x = W.conv_step_inputs(w, s)
        out = selscan.conv1d_step(st, dev(x, torch.bfloat16), dev(p["w"]), dev(p["bias"]))
        torch.cuda.synchronize()
        r = oracle.conv1d_step(ref_state, x, p["w"], p["bias"])
        assert oracle.scaled_error(to_np(out), r["out"], r["out_scale"]) <= TOL["bf16"]
        assert np.array_equal(to_np(st), r["conv_state"])
        ref_state = r["conv_state"]


CONV_BWD_SHAPES = [
    # (batch, L, dim, dtype)
    (1, 1, 1, "f32"),
    (1, 2, 64, "f32"),       # fewer tokens than the window
    (2, 17, 65, "bf16"),     # element rows
    (2, 64, 40, "f32"),      # 16-byte rows
    (3, 100, 130, "bf16"),
    (2, 2048, 64, "bf16"),   # several 256-vector trips
    (1, 40000, 8, "f32"),    # long rows split into pieces
    (5, 700, 24, "bf16"),    # element rows, batch entries in two uneven groups
    (8, 4096, 16, "bf16"),   # four batch groups of two rows, two pieces per row
    (1, 40001, 8, "bf16"),   # rows off a 16-byte boundary split into pieces, several trips
    (3, 2047, 96, "f32"),    # rows off a 16-byte boundary, blocks across wave edges
]


@pytest.mark.parametrize("batch,L,dim,dtype", CONV_BWD_SHAPES)
@pytest.mark.parametrize("with_bias,with_prev", [(True, True), (False, False)])
def test_conv1d_bwd(batch, L, dim, dtype, with_bias, with_prev):
    """selscan_conv1d_bwd against the oracle's gradients of the convolution."""
    p = _inputs(batch, L, dim, dtype, seed=L + dim)
    dout = np.random.default_rng([L, dim, 3]).standard_normal((batch, dim, L)).astype(np.float32)
    if dtype == "bf16":
        dout = W._maybe_bf16(W.get(W.HEADLINE), dout)
    case(f"conv bwd b{batch} L{L} d{dim} {dtype} bias={with_bias} prev={with_prev}")
    td = TDT[dtype]
    g = selscan.conv1d_bwd(dev(p["x"], td), dev(p["w"]), dev(p["bias"]) if with_bias else None,
                           dev(p["x_prev"]) if with_prev else None, dout=dev(dout, td))
    torch.cuda.synchronize()
    ref = oracle.conv1d_bwd(p["x"], p["w"], p["bias"] if with_bias else None,
                            p["x_prev"] if with_prev else None, dout=dout)
    errs = {k: oracle.scaled_error(to_np(g[k]), ref[k], ref[k + "_scale"])
            for k in ("dx", "dw", "dbias", "dx_prev")}
    print(f"[parity] conv bwd b{batch} L{L} d{dim} {dtype}: " +
          " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= TOL[dtype] for v in errs.values()), errs


def test_conv1d_bwd_deterministic_and_empty():
    p = _inputs(2, 500, 96, "bf16", seed=4)
    dout = dev(np.random.default_rng(5).standard_normal((2, 96, 500)), TDT["bf16"])
    args = (dev(p["x"], TDT["bf16"]), dev(p["w"]), dev(p["bias"]), dev(p["x_prev"]))
    case("conv bwd determinism")
    g1 = selscan.conv1d_bwd(*args, dout=dout)
    g2 = selscan.conv1d_bwd(*args, dout=dout)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k
    case("conv bwd L = 0")
    x = torch.empty((2, 8, 0), device="cuda")
    g = selscan.conv1d_bwd(x, torch.ones((8, 4), device="cuda"), dout=x.clone())
    torch.cuda.synchronize()
    assert torch.all(g["dw"] == 0) and torch.all(g["dbias"] == 0) and torch.all(g["dx_prev"] == 0)
