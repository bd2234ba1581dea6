"""Randomised invariants of the fp64 oracle (hypothesis). CPU only."""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle
from oracle_pins import _rand_problem, _brute, _close


shapes = st.tuples(st.integers(1, 3), st.integers(1, 4), st.integers(1, 16), st.integers(1, 40))


@settings(max_examples=40, deadline=None)
@given(shapes, st.integers(0, 2**31 - 1), st.booleans(), st.booleans())
def test_split_invariance_random(shape, seed, gate, with_bias):
    batch, dim, N, L = shape
    p = _rand_problem(seed, batch, dim, N, L, gate=gate, with_bias=with_bias)
    O = oracle.default()
    full = O.fwd(**p)
    L1 = np.random.default_rng(seed).integers(0, L + 1)
    seq = ("x", "delta", "z", "B", "C")
    a = {k: (v[..., :L1] if k in seq else v) for k, v in p.items()}
    b = {k: (v[..., L1:] if k in seq else v) for k, v in p.items()}
    h0 = np.zeros((batch, dim, N)); hs0 = np.zeros_like(h0)
    ys = []
    if L1 > 0:
        ra = O.fwd(**a)
        h0, hs0 = ra["last_state"], ra["state_scale"]
        ys.append(ra["y"])
    if L1 < L:
        rb = O.fwd(**b, h0=h0, h0_scale=hs0)
        ys.append(rb["y"])
        h0 = rb["last_state"]
    _close(np.concatenate(ys, -1), full["y"], 1e-13, full["y_scale"], what="split y")
    _close(h0, full["last_state"], 1e-13, full["state_scale"], what="split state")


@settings(max_examples=25, deadline=None)
@given(st.tuples(st.integers(1, 2), st.integers(1, 3), st.integers(1, 6), st.integers(1, 6)),
       st.integers(0, 2**31 - 1))
def test_bruteforce_random(shape, seed):
    batch, dim, N, L = shape
    p = _rand_problem(seed, batch, dim, N, L)
    r = oracle.default().fwd(**p)
    y, ys, hL, hsL = _brute(p)
    _close(r["y"], y, 1e-12, ys, what="brute y")
    _close(r["last_state"], hL, 1e-12, hsL, what="brute state")
