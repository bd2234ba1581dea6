"""GPU parity of the forward pass from a given initial state (selscan_fwd_ex
with h0), the caller-workspace path, and the kernel-timing hook.

A state is all the layer keeps between tokens ("State Space Models and
Mamba", multigrid.ai, sections "It is a linear recurrence" and "The state, in
bytes, against a KV cache"), so a sequence fed in two pieces, the second
starting from the first's last state, must give the unsplit result. The
oracle takes h0 directly; the split is checked against the unsplit oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import TDT, TOL, assert_close, dev, errors, small, to_np
from selective_state_space_48_amd import selscan
from selective_state_space_48_amd import workloads as W

pytestmark = pytest.mark.gpu

M14 = W.HEADLINE
M130 = "m130m_f32_b8_l2048_d1536"


def case(msg):
    print(f"[case] {msg}", flush=True)


def _state(batch, dim, seed, scale=0.5):
    return (np.random.default_rng(seed).standard_normal((batch, dim, 16)) * scale).astype(np.float32)


def _run(inp, dtype, h0=None, **kw):
    td = TDT[dtype]
    y, hs = selscan.fwd(dev(inp["x"], td), dev(inp["delta"], td), dev(inp["A"]),
                        dev(inp["B"], td), dev(inp["C"], td), D=dev(inp["D"]),
                        z=dev(inp["z"], td) if inp.get("z") is not None else None,
                        dt_bias=dev(inp["dt_bias"]), h0=None if h0 is None else dev(h0), **kw)
    torch.cuda.synchronize()
    return y, hs


def _oracle(inp, h0):
    return oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                      z=inp.get("z"), dt_bias=inp["dt_bias"], h0=h0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("segments", [1, 3, 0])
def test_fwd_from_h0(dtype, segments):
    """y and last_state from a random initial state, one-pass and split
    launches (the carry pass then starts from h0)."""
    inp = small(M14 if dtype == "bf16" else M130, batch=2, seqlen=700, dim=130)
    h0 = _state(2, 130, 11)
    case(f"h0 {dtype} segments={segments}")
    y, hs = _run(inp, dtype, h0, segments=segments)
    assert_close(y, hs, _oracle(inp, h0), dtype, f"h0 segments={segments}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_sequence_equals_whole(dtype):
    """Feeding [0, t) then [t, L) from the carried state equals one call over
    [0, L), at a split inside a tile and at a tile boundary."""
    L = 520
    inp = small(M14 if dtype == "bf16" else M130, batch=2, seqlen=L, dim=96)
    ref = _oracle(inp, None)
    for t in (77, 256):
        first = {k: (v[..., :t] if isinstance(v, np.ndarray) and v.ndim == 3 and v.shape[-1] == L
                     else v) for k, v in inp.items()}
        second = {k: (v[..., t:] if isinstance(v, np.ndarray) and v.ndim == 3 and v.shape[-1] == L
                      else v) for k, v in inp.items()}
        case(f"split at {t} {dtype}")
        y1, h1 = _run(first, dtype)
        y2, h2 = _run(second, dtype, to_np(h1).astype(np.float32))
        y = torch.cat([y1, y2], dim=-1)
        # the carried state goes through fp32 once more than in one call: same bar
        assert_close(y, h2, ref, dtype, f"split at {t}")


def test_h0_in_place():
    """h0 may be the last_state tensor itself."""
    inp = small(M130, batch=2, seqlen=300, dim=64)
    h0 = _state(2, 64, 12)
    case("h0 is last_state (one pass)")
    st = dev(h0)
    y, hs = selscan.fwd(dev(inp["x"]), dev(inp["delta"]), dev(inp["A"]), dev(inp["B"]),
                        dev(inp["C"]), D=dev(inp["D"]), z=dev(inp["z"]),
                        dt_bias=dev(inp["dt_bias"]), h0=st, last_state=st, segments=1)
    torch.cuda.synchronize()
    assert hs.data_ptr() == st.data_ptr()
    ref = _oracle(inp, h0)
    assert_close(y, hs, ref, "f32", "in place, one pass")
    case("h0 is last_state (4 segments)")
    st = dev(h0)
    y, hs = selscan.fwd(dev(inp["x"]), dev(inp["delta"]), dev(inp["A"]), dev(inp["B"]),
                        dev(inp["C"]), D=dev(inp["D"]), z=dev(inp["z"]),
                        dt_bias=dev(inp["dt_bias"]), h0=st, last_state=st, segments=4)
    torch.cuda.synchronize()
    assert_close(y, hs, ref, "f32", "in place, 4 segments")


def test_empty_sequence_returns_h0():
    case("L = 0 with h0")
    x = torch.empty((2, 64, 0), device="cuda")
    A = -torch.ones((64, 16), device="cuda")
    B = torch.empty((2, 16, 0), device="cuda")
    h0 = torch.randn((2, 64, 16), device="cuda")
    hs = torch.full((2, 64, 16), 7.0, device="cuda")
    y, hs = selscan.fwd(x, x.clone(), A, B, B.clone(), last_state=hs, h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(hs, h0)


@pytest.mark.parametrize("segments", [1, 5])
def test_caller_workspace(segments):
    """A caller-owned workspace (larger than needed, dirty) gives the same
    bits as the library's own."""
    inp = small(M14, batch=2, seqlen=640, dim=128)
    case(f"caller workspace segments={segments}")
    y0, h0 = _run(inp, "bf16", segments=segments)
    need = selscan.workspace_size(2, 640, 128, torch.bfloat16, segments=segments)
    ws = torch.full((need + 4096,), 0xAB, dtype=torch.uint8, device="cuda")
    y1, h1 = _run(inp, "bf16", segments=segments, workspace=ws)
    assert torch.equal(y0, y1) and torch.equal(h0, h1)
    with pytest.raises(selscan.SelscanError):
        _run(inp, "bf16", segments=segments, workspace=ws[: need - 256])


def test_timing_hook_counts_launches():
    inp = small(M14, batch=2, seqlen=256, dim=128)
    td = torch.bfloat16
    args = [dev(inp[k], td) for k in ("x", "delta")] + [dev(inp["A"])] + \
        [dev(inp[k], td) for k in ("B", "C")]
    case("timing hook")
    selscan.timing_start(2)
    for _ in range(3):   # the third launch is beyond capacity and not recorded
        selscan.fwd(*args)
    ms, n = selscan.timing_stop()
    assert n == 2 and ms > 0.0
    with pytest.raises(selscan.SelscanError):
        selscan.timing_stop()
    state = torch.zeros((2, 128, 16), device="cuda")
    xs = torch.zeros((2, 128), dtype=td, device="cuda")
    Bs = torch.zeros((2, 16), dtype=td, device="cuda")
    selscan.timing_start(8)
    selscan.step(state, xs, xs.clone(), args[2], Bs, Bs.clone())
    ms, n = selscan.timing_stop()
    assert n == 1 and ms > 0.0
