"""The no-allocation forward (selscan_fwd_noalloc), called through the C ABI,
against the allocating one (selscan_fwd) and the oracle: two calls in a row,
the second with a smaller input, then a third at the 130m-shaped size. Both
entry points run the same kernels and launch plan, so their outputs must be
bit-identical; the oracle bounds both to the usual tolerance. The scratch
keeps the previous call's contents, so the smaller second call also checks
that nothing left there leaks into a result. pytest -m gpu."""
import numpy as np
import pytest
import torch

from parity_util import TDT, assert_close, dev, oracle_fwd, small
from selective_state_space_48_amd import selscan
from selective_state_space_48_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = [
    # (workload recipe, batch, L, dim, gate): a segmented launch, then a
    # smaller one-pass launch, then the 8-wave one-pass plan at full size
    (W.HEADLINE, 2, 3000, 200, True),
    ("m130m_f32_b8_l2048_d1536", 1, 500, 64, False),
]


def _run_both(inp, dtype, gate):
    td = TDT[dtype]
    args = (dev(inp["x"], td), dev(inp["delta"], td), dev(inp["A"]), dev(inp["B"], td), dev(inp["C"], td))
    kw = dict(D=dev(inp["D"]), z=dev(inp["z"], td) if gate else None, dt_bias=dev(inp["dt_bias"]))
    batch, dim, L = inp["x"].shape
    y_na = torch.full((batch, dim, L), float("nan"), device="cuda").to(td)
    s_na = torch.full((batch, dim, 16), float("nan"), device="cuda")
    selscan.fwd_noalloc(*args, **kw, y=y_na, last_state=s_na)
    y_ref, s_ref = selscan.fwd(*args, **kw)
    torch.cuda.synchronize()
    return y_na, s_na, y_ref, s_ref


def test_noalloc_two_calls_second_smaller():
    for name, batch, L, dim, gate in CASES:
        w = W.get(name)
        print(f"[case] noalloc {name} b{batch} L{L} d{dim} gate={gate}", flush=True)
        inp = small(name, batch=batch, seqlen=L, dim=dim)
        y_na, s_na, y_ref, s_ref = _run_both(inp, w.dtype, gate)
        assert torch.equal(y_na, y_ref) and torch.equal(s_na, s_ref), "noalloc differs from selscan_fwd"
        ref = oracle_fwd(inp, use_z=gate)
        assert_close(y_na, s_na, ref, w.dtype, f"noalloc {name} b{batch} L{L} d{dim}")


def test_noalloc_full_130m_shape():
    name = "m130m_f32_b8_l2048_d1536"
    w = W.get(name)
    print(f"[case] noalloc full {name}", flush=True)
    inp = W.fwd_inputs(w)
    y_na, s_na, y_ref, s_ref = _run_both(inp, w.dtype, True)
    assert torch.equal(y_na, y_ref) and torch.equal(s_na, s_ref), "noalloc differs from selscan_fwd"
    rows = np.unique(np.concatenate([np.arange(0, w.rows, 997), [w.rows - 1]])).astype(np.int64)
    ref = oracle_fwd(inp, use_z=True, rows=rows)
    assert_close(y_na, s_na, ref, w.dtype, f"noalloc full {name} sampled", rows=rows)


def test_noalloc_rejects_oversize_without_touching_outputs():
    """A problem beyond the scratch is refused before anything is enqueued:
    the outputs keep their contents."""
    batch, dim, L = 1, 16, selscan.NOALLOC_SCRATCH_BYTES // 128 + 32
    f = lambda *s: torch.zeros(*s, device="cuda")
    x = f(batch, dim, L)
    y = torch.full((batch, dim, L), 7.0, device="cuda")
    with pytest.raises(selscan.SelscanError, match="-10"):
        selscan.fwd_noalloc(x, f(batch, dim, L), -torch.ones(dim, 16, device="cuda"), f(batch, 16, L),
                            f(batch, 16, L), y=y)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
