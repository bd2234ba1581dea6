"""GPU parity of the forward with the block's causal convolution (width 4) +
SiLU fused in front (selscan_fwd_ex's conv_w): the scan's input is the
convolution of x, formed in the per-token phase and never stored.

The reference composes two separately pinned oracle functions: the
convolution (conv1d) of x, then the scan (fwd) of its fp64 output. Cases:
ragged lengths and rows, both dtypes, with and without bias, carried-in
inputs, gate and D; segmented runs (the convolution's history crosses
segment boundaries); the last-inputs output; and the fused call against the
two separate calls. Error measure as for the scan, with the scales of the
composition (see _ref)."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import TDT, TOL, dev, to_np
from selective_state_space_48_amd import selscan
from selective_state_space_48_amd import workloads as W

pytestmark = pytest.mark.gpu
M14 = W.HEADLINE
M130 = "m130m_f32_b8_l2048_d1536"


def case(msg):
    print(f"[case] {msg}", flush=True)


def _inputs(batch, L, dim, dtype):
    w = W.scaled(W.get(M14 if dtype == "bf16" else M130), batch=batch, seqlen=L, dim=dim)
    p = W.fwd_inputs(w)
    c = W.conv_inputs(w)
    p.update(cw=c["w"], cb=c["bias"], x_prev=c["x_prev"], x=c["x"])
    return p


def _gpu(p, dtype, with_bias=True, with_prev=True, segments=0, x_last=False):
    td = TDT[dtype]
    last = torch.full((p["x"].shape[0], p["x"].shape[1], 3), float("nan"), device="cuda") if x_last else None
    y, hs = selscan.fwd(dev(p["x"], td), dev(p["delta"], td), dev(p["A"]), dev(p["B"], td),
                        dev(p["C"], td), D=dev(p["D"]),
                        z=dev(p["z"], td) if p.get("z") is not None else None,
                        dt_bias=dev(p["dt_bias"]), segments=segments, conv_w=dev(p["cw"]),
                        conv_b=dev(p["cb"]) if with_bias else None,
                        conv_x_prev=dev(p["x_prev"]) if with_prev else None, conv_x_last=last)
    torch.cuda.synchronize()
    return y, hs, last


def _ref(p, with_bias=True, with_prev=True):
    """The oracle's convolution, then its scan. The error scales compose: an
    error in the scan's input of up to its magnitude sum (the convolution's
    out_scale: the pre-activation terms, SiLU's slope being at most 1.1)
    moves y by at most the scan's scale with that magnitude as input, and
    the scan's scales are linear in |x|, so the scale of the composition is
    the scan's scale with |x| + out_scale as input."""
    c = oracle.conv1d(p["x"], p["cw"], p["cb"] if with_bias else None,
                      p["x_prev"] if with_prev else None)
    args = (p["delta"], p["A"], p["B"], p["C"], p["D"], p.get("z"), p["dt_bias"])
    r = oracle.fwd(c["out"], *args)
    mag = oracle.fwd(np.abs(c["out"]) + 1.1 * c["out_scale"], *args)
    r["y_scale"], r["state_scale"] = mag["y_scale"], mag["state_scale"]
    r["x_last"] = c["x_last"]
    return r


def _check(y, hs, ref, dtype, what):
    ey = oracle.scaled_error(to_np(y), ref["y"], ref["y_scale"])
    es = oracle.scaled_error(to_np(hs), ref["last_state"], ref["state_scale"])
    print(f"[parity] fused conv {what}: err_y={ey:.3e} err_state={es:.3e} tol={TOL[dtype]:.0e}", flush=True)
    assert ey <= TOL[dtype] and es <= TOL[dtype], what


CASES = [
    # (batch, L, dim, dtype, bias, prev, segments)
    (1, 1, 1, "f32", True, True, 0),
    (1, 2, 64, "f32", True, True, 0),        # fewer tokens than the window
    (2, 17, 65, "bf16", True, True, 0),
    (2, 100, 130, "bf16", False, False, 0),
    (1, 300, 64, "f32", True, False, 0),
    (2, 64, 40, "f32", True, True, 0),       # element rows (L*4 % 16 == 0, dim ragged)
    (2, 63, 66, "f32", True, True, 0),       # element loads (ragged L)
    (1, 2000, 64, "f32", True, True, 0),     # automatic segments
    (2, 700, 65, "bf16", True, True, 5),     # forced segments: history across boundaries
    (1, 1000, 128, "bf16", False, True, 7),
]


@pytest.mark.parametrize("batch,L,dim,dtype,bias,prev,segments", CASES)
def test_fused_conv_forward(batch, L, dim, dtype, bias, prev, segments):
    p = _inputs(batch, L, dim, dtype)
    case(f"fused conv b{batch} L{L} d{dim} {dtype} bias={bias} prev={prev} segments={segments}")
    y, hs, last = _gpu(p, dtype, bias, prev, segments, x_last=True)
    ref = _ref(p, bias, prev)
    _check(y, hs, ref, dtype, f"b{batch} L{L} d{dim} {dtype} segments={segments}")
    assert np.array_equal(to_np(last), ref["x_last"])


def test_fused_conv_matches_separate_calls():
    """conv1d then fwd (the convolution's output rounded to bf16 in between)
    against the fused call (not rounded): close, and the fused one at least
    as close to the oracle."""
    p = _inputs(2, 500, 192, "bf16")
    case("fused conv vs conv1d + fwd")
    td = TDT["bf16"]
    xc, _ = selscan.conv1d(dev(p["x"], td), dev(p["cw"]), dev(p["cb"]), dev(p["x_prev"]))
    y_sep, _ = selscan.fwd(xc, dev(p["delta"], td), dev(p["A"]), dev(p["B"], td), dev(p["C"], td),
                           D=dev(p["D"]), z=dev(p["z"], td), dt_bias=dev(p["dt_bias"]))
    y_fused, _, _ = _gpu(p, "bf16")
    ref = _ref(p)
    e_sep = oracle.scaled_error(to_np(y_sep), ref["y"], ref["y_scale"])
    e_fused = oracle.scaled_error(to_np(y_fused), ref["y"], ref["y_scale"])
    print(f"[parity] separate {e_sep:.3e} fused {e_fused:.3e}", flush=True)
    assert e_fused <= TOL["bf16"] and e_sep <= TOL["bf16"]


def test_fused_conv_streaming_split():
    """A sequence in two calls, the second from the first's last state and
    last inputs (in place), against the unsplit oracle."""
    p = _inputs(2, 300, 64, "f32")
    case("fused conv split at 131")
    cut = 131
    part = lambda a, lo, hi: np.ascontiguousarray(a[..., lo:hi])
    kw = lambda lo, hi: dict(D=dev(p["D"]), z=dev(part(p["z"], lo, hi)), dt_bias=dev(p["dt_bias"]),
                             conv_w=dev(p["cw"]), conv_b=dev(p["cb"]))
    args = lambda lo, hi: (dev(part(p["x"], lo, hi)), dev(part(p["delta"], lo, hi)), dev(p["A"]),
                           dev(part(p["B"], lo, hi)), dev(part(p["C"], lo, hi)))
    cst = dev(p["x_prev"])
    y1, st = selscan.fwd(*args(0, cut), **kw(0, cut), conv_x_prev=cst, conv_x_last=cst)
    y2, st2 = selscan.fwd(*args(cut, 300), **kw(cut, 300), h0=st, last_state=st, conv_x_prev=cst,
                          conv_x_last=cst)
    torch.cuda.synchronize()
    ref = _ref(p)
    y = np.concatenate([to_np(y1), to_np(y2)], axis=-1)
    _check(torch.from_numpy(y), st2, ref, "f32", "split")
    assert np.array_equal(to_np(cst), ref["x_last"])


def test_fused_conv_empty_sequence():
    case("fused conv L = 0")
    x = torch.empty((2, 64, 0), device="cuda")
    prev = torch.randn((2, 64, 3), device="cuda")
    last = torch.empty_like(prev)
    selscan.fwd(x, x.clone(), -torch.ones((64, 16), device="cuda"), torch.empty((2, 16, 0), device="cuda"),
                torch.empty((2, 16, 0), device="cuda"), conv_w=torch.ones((64, 4), device="cuda"),
                conv_x_prev=prev, conv_x_last=last)
    torch.cuda.synchronize()
    assert torch.equal(last, prev)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_prefill_then_decode(dtype, fused):
    """The block's inference path end to end: a prefill with the convolution
    fused (its last inputs and the scan's last state out), then decode steps
    from those, either the convolution's step then the scan's step, or the
    scan's step with the convolution fused in front (selscan_step_ex); the
    decoded outputs against the oracle's convolution then scan over the whole
    sequence (the decode step takes the step size with the channel bias
    already added)."""
    batch, L, T, dim = 2, 150, 6, 128
    p = _inputs(batch, L + T, dim, dtype)
    td = TDT[dtype]
    case(f"block prefill {L} then {T} decode steps {dtype} fused={fused}")
    cut = lambda a: np.ascontiguousarray(a[..., :L])
    cst = torch.empty((batch, dim, 3), device="cuda")
    _, st = selscan.fwd(dev(cut(p["x"]), td), dev(cut(p["delta"]), td), dev(p["A"]), dev(cut(p["B"]), td),
                        dev(cut(p["C"]), td), D=dev(p["D"]), z=dev(cut(p["z"]), td), dt_bias=dev(p["dt_bias"]),
                        conv_w=dev(p["cw"]), conv_b=dev(p["cb"]), conv_x_prev=dev(p["x_prev"]),
                        conv_x_last=cst)
    ys = []
    for t in range(L, L + T):
        dl = (p["delta"][..., t] + p["dt_bias"][None]).astype(np.float32)
        tok = (dev(dl, td), dev(p["A"]), dev(p["B"][..., t], td), dev(p["C"][..., t], td))
        if fused:
            y = selscan.step(st, dev(p["x"][..., t], td), *tok, D=dev(p["D"]), z=dev(p["z"][..., t], td),
                             conv_w=dev(p["cw"]), conv_b=dev(p["cb"]), conv_state=cst)
        else:
            xa = selscan.conv1d_step(cst, dev(p["x"][..., t], td), dev(p["cw"]), dev(p["cb"]))
            y = selscan.step(st, xa, *tok, D=dev(p["D"]), z=dev(p["z"][..., t], td))
        ys.append(to_np(y))
    torch.cuda.synchronize()
    ref = _ref(p)
    ey = oracle.scaled_error(np.stack(ys, -1), ref["y"][..., L:], ref["y_scale"][..., L:])
    es = oracle.scaled_error(to_np(st), ref["last_state"], ref["state_scale"])
    print(f"[parity] block prefill+decode {dtype} fused={fused}: err_y={ey:.3e} err_state={es:.3e}", flush=True)
    assert ey <= TOL[dtype] and es <= TOL[dtype]
    assert np.array_equal(to_np(cst), ref["x_last"])


@pytest.mark.parametrize("batch,dim", [(1, 1), (3, 77), (2, 256), (5, 1000)])
def test_fused_conv_step_equals_two_calls(batch, dim):
    """In fp32 the fused step's arithmetic is that of conv1d_step then step
    (same operations in the same order; the convolved input is not rounded in
    either), so y, the state and the convolution's state are equal bit for
    bit over a few steps; ragged rows (not a multiple of the kernel's
    2 x 256 quads) included, with and without bias and gate."""
    N = 16
    g = torch.Generator(device="cuda").manual_seed(batch * 1000 + dim)
    rn = lambda *s: torch.randn(s, device="cuda", generator=g)
    A, D, cw, cb = -torch.exp(0.5 * rn(dim, N)), rn(dim), 0.5 * rn(dim, 4), 0.1 * rn(dim)
    for bias, gate in ((True, True), (False, False)):
        case(f"fused conv step b{batch} d{dim} bias={bias} gate={gate}")
        st1, cs1 = 0.1 * rn(batch, dim, N), rn(batch, dim, 3)
        st2, cs2 = st1.clone(), cs1.clone()
        for _ in range(3):
            x, dl, z = rn(batch, dim), rn(batch, dim) - 1.0, rn(batch, dim) if gate else None
            Bt, Ct = rn(batch, N), rn(batch, N)
            xa = selscan.conv1d_step(cs1, x, cw, cb if bias else None)
            y1 = selscan.step(st1, xa, dl, A, Bt, Ct, D=D, z=z)
            y2 = selscan.step(st2, x, dl, A, Bt, Ct, D=D, z=z, conv_w=cw, conv_b=cb if bias else None,
                              conv_state=cs2)
            torch.cuda.synchronize()
            assert torch.equal(y1, y2) and torch.equal(st1, st2) and torch.equal(cs1, cs2)
