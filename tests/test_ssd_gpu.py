"""GPU parity of the Mamba-2 SSD layer (selscan_ssd_fwd, bf16, matrix cores)
against the fp64 oracle on the same seeded inputs: ragged lengths around the
64-token chunks, both state sizes, optional D and dt_bias, determinism, an
empty sequence, and the full 1.3B-shaped layer. Error measure: |gpu - ref|
over the oracle's magnitude-sum scale; limit 2e-2 (bf16 inputs)."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import TOL, dev, to_np
from selective_state_space_48_amd import selscan
from selective_state_space_48_amd import workloads as W

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def case(msg):
    print(f"[case] {msg}", flush=True)


def _gpu(p, use_D=True, use_bias=True):
    y, hs = selscan.ssd_fwd(dev(p["x"], BF), dev(p["delta"], BF), dev(p["A"]), dev(p["B"], BF),
                            dev(p["C"], BF), D=dev(p["D"]) if use_D else None,
                            dt_bias=dev(p["dt_bias"]) if use_bias else None)
    torch.cuda.synchronize()
    return y, hs


def _check(y, hs, p, what, use_D=True, use_bias=True):
    r = oracle.ssd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"] if use_D else None,
                   p["dt_bias"] if use_bias else None)
    ey = oracle.scaled_error(to_np(y), r["y"], r["y_scale"])
    es = oracle.scaled_error(to_np(hs), r["last_state"], r["state_scale"])
    print(f"[parity] ssd {what}: err_y={ey:.3e} err_state={es:.3e}", flush=True)
    assert ey <= TOL["bf16"] and es <= TOL["bf16"], f"{what}: {ey:.3e} {es:.3e}"


SHAPES = [
    # (batch, L, heads, dstate)
    (1, 1, 1, 64),
    (1, 64, 2, 64),
    (2, 65, 3, 128),     # one token into a second chunk
    (2, 130, 2, 64),
    (1, 300, 4, 128),
    (3, 63, 1, 128),
]


@pytest.mark.parametrize("batch,L,heads,N", SHAPES)
def test_ssd_shapes(batch, L, heads, N):
    p = W.ssd_inputs(batch, L, heads, 64, N, seed=L)
    case(f"ssd b{batch} L{L} H{heads} N{N}")
    y, hs = _gpu(p)
    _check(y, hs, p, f"b{batch} L{L} H{heads} N{N}")


def test_ssd_optional_inputs_absent():
    p = W.ssd_inputs(2, 200, 3, 64, 128, seed=9)
    case("ssd without D and dt_bias")
    y, hs = _gpu(p, use_D=False, use_bias=False)
    _check(y, hs, p, "no D, no dt_bias", use_D=False, use_bias=False)


def test_ssd_long_sequence():
    p = W.ssd_inputs(1, 4096, 2, 64, 128, seed=10)
    case("ssd L4096")
    y, hs = _gpu(p)
    _check(y, hs, p, "L4096")


def test_ssd_deterministic_and_empty():
    p = W.ssd_inputs(2, 150, 2, 64, 64, seed=11)
    case("ssd determinism")
    y1, h1 = _gpu(p)
    y2, h2 = _gpu(p)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    case("ssd L = 0")
    x = torch.empty((2, 0, 3, 64), dtype=BF, device="cuda")
    hs = torch.full((2, 3, 64, 64), 5.0, device="cuda")
    y, hs = selscan.ssd_fwd(x, torch.empty((2, 0, 3), dtype=BF, device="cuda"),
                            -torch.ones(3, device="cuda"), torch.empty((2, 0, 64), dtype=BF, device="cuda"),
                            torch.empty((2, 0, 64), dtype=BF, device="cuda"), last_state=hs)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 3, 64) and torch.all(hs == 0)


def test_ssd_headline_shape():
    """batch 8, L 2048, 64 heads of 64, state 128 (a 1.3B-shaped Mamba-2 layer)."""
    s = W.SSD_HEADLINE
    p = W.ssd_inputs(s["batch"], s["seqlen"], s["heads"], s["headdim"], s["dstate"], s["seed"])
    case("ssd full b8 L2048 H64 P64 N128")
    y, hs = _gpu(p)
    _check(y, hs, p, "headline shape")


def _state(batch, H, N, seed, scale=0.5):
    return (np.random.default_rng(seed).standard_normal((batch, H, N, 64)) * scale).astype(np.float32)


@pytest.mark.parametrize("batch,L,heads,N", [(2, 65, 3, 128), (1, 130, 2, 64), (2, 7, 1, 128)])
def test_ssd_from_initial_state(batch, L, heads, N):
    """selscan_ssd_fwd_ex: the recurrence starts from h0."""
    p = W.ssd_inputs(batch, L, heads, 64, N, seed=L + 100)
    h0 = _state(batch, heads, N, L)
    case(f"ssd from h0 b{batch} L{L} H{heads} N{N}")
    y, hs = selscan.ssd_fwd(dev(p["x"], BF), dev(p["delta"], BF), dev(p["A"]), dev(p["B"], BF),
                            dev(p["C"], BF), D=dev(p["D"]), dt_bias=dev(p["dt_bias"]), h0=dev(h0))
    torch.cuda.synchronize()
    r = oracle.ssd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["dt_bias"], h0=h0)
    ey = oracle.scaled_error(to_np(y), r["y"], r["y_scale"])
    es = oracle.scaled_error(to_np(hs), r["last_state"], r["state_scale"])
    print(f"[parity] ssd h0 b{batch} L{L} H{heads} N{N}: err_y={ey:.3e} err_state={es:.3e}", flush=True)
    assert ey <= TOL["bf16"] and es <= TOL["bf16"]


def test_ssd_split_sequence_matches_unsplit():
    """A sequence in two pieces, the second from the first's last state (in
    place: h0 is last_state), against the unsplit oracle."""
    batch, L, H, N, cut = 2, 300, 3, 128, 137
    p = W.ssd_inputs(batch, L, H, 64, N, seed=77)
    case(f"ssd split at {cut} of {L}")
    part = lambda a, lo, hi: np.ascontiguousarray(a[:, lo:hi])
    run = lambda lo, hi, **kw: selscan.ssd_fwd(
        dev(part(p["x"], lo, hi), BF), dev(part(p["delta"], lo, hi), BF), dev(p["A"]),
        dev(part(p["B"], lo, hi), BF), dev(part(p["C"], lo, hi), BF), D=dev(p["D"]),
        dt_bias=dev(p["dt_bias"]), **kw)
    y1, st = run(0, cut)
    y2, st2 = run(cut, L, h0=st, last_state=st)
    torch.cuda.synchronize()
    assert st2.data_ptr() == st.data_ptr()
    r = oracle.ssd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["dt_bias"])
    y = np.concatenate([to_np(y1), to_np(y2)], axis=1)
    ey = oracle.scaled_error(y, r["y"], r["y_scale"])
    es = oracle.scaled_error(to_np(st), r["last_state"], r["state_scale"])
    print(f"[parity] ssd split: err_y={ey:.3e} err_state={es:.3e}", flush=True)
    assert ey <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("N", [64, 128])
def test_ssd_decode_steps(N):
    """selscan_ssd_step: several tokens one at a time from a given state. Each
    step against the oracle's step from the same state (the GPU's previous
    one), and the chain against the oracle's layer over those tokens from the
    first state (whose error scales carry the whole history)."""
    batch, H, T = 3, 5, 6
    p = W.ssd_inputs(batch, T, H, 64, N, seed=N + 7)
    st0 = _state(batch, H, N, N)
    st = dev(st0)
    case(f"ssd decode N{N}: {T} steps")
    worst_y = worst_s = 0.0
    ys = []
    for t in range(T):
        xt, dt = np.ascontiguousarray(p["x"][:, t]), np.ascontiguousarray(p["delta"][:, t])
        Bt, Ct = np.ascontiguousarray(p["B"][:, t]), np.ascontiguousarray(p["C"][:, t])
        prev = to_np(st)
        y = selscan.ssd_step(st, dev(xt, BF), dev(dt, BF), dev(p["A"]), dev(Bt, BF), dev(Ct, BF),
                             D=dev(p["D"]), dt_bias=dev(p["dt_bias"]))
        torch.cuda.synchronize()
        r = oracle.ssd_step(prev, xt, dt, p["A"], Bt, Ct, p["D"], p["dt_bias"])
        ys.append(to_np(y))
        worst_y = max(worst_y, oracle.scaled_error(ys[-1], r["y"], r["y_scale"]))
        worst_s = max(worst_s, oracle.scaled_error(to_np(st), r["state"], r["state_scale"]))
    full = oracle.ssd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["dt_bias"], h0=st0)
    ey = oracle.scaled_error(np.stack(ys, 1), full["y"], full["y_scale"])
    es = oracle.scaled_error(to_np(st), full["last_state"], full["state_scale"])
    print(f"[parity] ssd decode N{N}: per step err_y={worst_y:.3e} err_state={worst_s:.3e}; "
          f"chain err_y={ey:.3e} err_state={es:.3e}", flush=True)
    # y is bf16; the state is fp32 arithmetic throughout: held to the fp32 limit
    assert worst_y <= TOL["bf16"] and ey <= TOL["bf16"]
    assert worst_s <= TOL["f32"] and es <= TOL["f32"]


def test_ssd_decode_continues_prefill():
    """Prefill with selscan_ssd_fwd, then decode with selscan_ssd_step from its
    last state: the decoded tokens match the oracle over the whole sequence."""
    batch, L, H, N, T = 2, 100, 3, 128, 4
    p = W.ssd_inputs(batch, L + T, H, 64, N, seed=5)
    case("ssd prefill then decode")
    part = lambda a, lo, hi: np.ascontiguousarray(a[:, lo:hi])
    _, st = selscan.ssd_fwd(dev(part(p["x"], 0, L), BF), dev(part(p["delta"], 0, L), BF),
                            dev(p["A"]), dev(part(p["B"], 0, L), BF), dev(part(p["C"], 0, L), BF),
                            D=dev(p["D"]), dt_bias=dev(p["dt_bias"]))
    ys = []
    for t in range(L, L + T):
        ys.append(to_np(selscan.ssd_step(st, dev(p["x"][:, t], BF), dev(p["delta"][:, t], BF),
                                         dev(p["A"]), dev(p["B"][:, t], BF), dev(p["C"][:, t], BF),
                                         D=dev(p["D"]), dt_bias=dev(p["dt_bias"]))))
    torch.cuda.synchronize()
    r = oracle.ssd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["dt_bias"])
    ey = oracle.scaled_error(np.stack(ys, 1), r["y"][:, L:], r["y_scale"][:, L:])
    es = oracle.scaled_error(to_np(st), r["last_state"], r["state_scale"])
    print(f"[parity] ssd prefill+decode: err_y={ey:.3e} err_state={es:.3e}", flush=True)
    assert ey <= TOL["bf16"] and es <= TOL["bf16"]


def test_ssd_empty_from_initial_state():
    case("ssd L = 0 from h0")
    x = torch.empty((2, 0, 3, 64), dtype=BF, device="cuda")
    h0 = torch.randn((2, 3, 64, 64), device="cuda")
    _, hs = selscan.ssd_fwd(x, torch.empty((2, 0, 3), dtype=BF, device="cuda"),
                            -torch.ones(3, device="cuda"), torch.empty((2, 0, 64), dtype=BF, device="cuda"),
                            torch.empty((2, 0, 64), dtype=BF, device="cuda"), h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(hs, h0)
