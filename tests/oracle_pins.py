"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
if the oracle disagrees with:

* values the pages print for their worked examples (``tests/golden/``);
* closed forms (the unrolled convolution of a time-invariant SSM, Theorem 1's
  gated RNN);
* brute-force unrolling on tiny inputs, written as sums of products rather
  than as a recurrence;
* library routines (numpy/scipy/torch softplus, sigmoid, silu, FFT
  convolution);
* exact invariants (linearity, zero input, split invariance, forward equals
  repeated decode steps, N-embedding).

They are collected by ``test_oracle_pins.py`` against the built oracle and by
``test_oracle_mutants.py`` against copies of the oracle with planted mistakes,
which must each fail at least one pin.
"""
from __future__ import annotations

import math
import os

import numpy as np
import scipy.signal
import scipy.special
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = [float(t) for t in v.split()]
    return out


def softplus_lib(u):
    """softplus via numpy's logaddexp: log(e^0 + e^u)."""
    return np.logaddexp(0.0, np.asarray(u, np.float64))


def silu_lib(z):
    return torch.nn.functional.silu(torch.from_numpy(np.asarray(z, np.float64))).numpy()


def inv_softplus(v):
    """The u with softplus(u) = v (input construction only)."""
    return np.log(np.expm1(np.asarray(v, np.float64)))


def _close(got, want, tol, scale=None, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    s = np.ones_like(want) if scale is None else np.maximum(np.asarray(scale, np.float64), 1e-300)
    err = np.max(np.abs(got - want) / s) if want.size else 0.0
    assert err <= tol, f"{what}: scaled error {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------------------
# Worked examples printed on the pages
# ----------------------------------------------------------------------------

def pin_run_ssm_printed(O):
    """Fixed-decay scalar example (mernstackdev.com, "A tiny example you can run").

    Through S6 with one state: A = ln a, step size exactly 1 (delta_raw =
    softplus^-1(1), no bias), B = C = 1, no D, no gate. Checked against the
    printed 3-decimal values and the hand closed form y_t = a^t + 5 a^(t-4).
    Also run with N = 16 where states 1..15 get B = 0 (they must not leak).
    """
    g = golden("run_ssm.txt")
    sig = np.array(g["signal"])
    L = sig.size
    for N in (1, 16):
        for key, a in (("a=0.9", 0.9), ("a=0.3", 0.3)):
            rng = np.random.default_rng(7)
            A = -rng.uniform(0.1, 3.0, (1, N))
            A[0, 0] = math.log(a)
            B = np.zeros((1, N, L)); B[0, 0] = 1.0
            C = rng.standard_normal((1, N, L)); C[0, 0] = 1.0
            x = sig.reshape(1, 1, L)
            delta = np.full((1, 1, L), inv_softplus(1.0))
            r = O.fwd(x, delta, A, B, C)
            y = r["y"][0, 0]
            t = np.arange(L)
            closed = a ** t + 5.0 * np.where(t >= 4, a ** np.maximum(t - 4, 0), 0.0)
            _close(y, closed, 1e-12, what=f"run_ssm {key} N={N} closed form")
            _close(np.round(y, 3), np.array(g[key]), 1e-9, what=f"run_ssm {key} N={N} printed")
            _close(r["last_state"][0, 0, 0], closed[-1], 1e-12, what="run_ssm last state")


def pin_run_selective_printed(O):
    """Input-dependent keep/write example (mernstackdev.com, "Selectivity, shown in code").

    Through S6 with A = -1: keep = exp(-delta) so delta = -ln(keep); the write
    factor is delta * B, so B = write / delta. C = 1, no D, no gate.
    """
    g = golden("run_selective.txt")
    vals = np.array(g["values"])
    imp = np.array(g["important"]) > 0
    keep = np.where(imp, g["keep_important"][0], g["keep_other"][0])
    write = np.where(imp, g["write_important"][0], g["write_other"][0])
    L = vals.size
    dl = -np.log(keep)
    delta = inv_softplus(dl).reshape(1, 1, L)
    B = (write / dl).reshape(1, 1, L)
    C = np.ones((1, 1, L))
    r = O.fwd(vals.reshape(1, 1, L), delta, -np.ones((1, 1)), B, C)
    y = r["y"][0, 0]
    _close(y, np.array(g["exact"]), 1e-12, what="run_selective exact")
    _close(np.round(y, 2), np.array(g["printed"]), 1e-9, what="run_selective printed")


# ----------------------------------------------------------------------------
# Closed forms
# ----------------------------------------------------------------------------

def pin_theorem1_gated_rnn(O):
    """Theorem 1 ("Mamba: Linear-Time Sequence Modeling with Selective State
    Spaces", azimuth.plus): with one state, A = -1 and the step size
    delta = softplus(u), exp(-delta) = 1 - sigmoid(u), so the S6 recurrence is
    the gated RNN h = (1 - g) h + g x with g = sigmoid(u), provided the input
    term delta*B equals g, i.e. B = sigmoid(u) / softplus(u).
    The RNN below is computed independently with scipy's expit.
    """
    rng = np.random.default_rng(11)
    batch, L = 4, 64
    dt_bias = np.array([0.3])
    delta = rng.standard_normal((batch, 1, L)) * 2.0
    u = delta + dt_bias[0]
    x = rng.standard_normal((batch, 1, L))
    gte = scipy.special.expit(u)
    B = (gte / softplus_lib(u)).reshape(batch, 1, L)
    C = np.ones((batch, 1, L))
    r = O.fwd(x, delta, -np.ones((1, 1)), B, C, dt_bias=dt_bias)
    h = np.zeros(batch)
    want = np.empty((batch, L))
    for t in range(L):
        h = (1.0 - gte[:, 0, t]) * h + gte[:, 0, t] * x[:, 0, t]
        want[:, t] = h
    _close(r["y"][:, 0], want, 1e-12, what="theorem 1")


def _lti_problem(seed, batch, dim, N, L):
    rng = np.random.default_rng(seed)
    A = -rng.uniform(0.05, 2.0, (dim, N))
    c = rng.standard_normal((batch, dim, 1))
    delta = np.broadcast_to(c, (batch, dim, L)).copy()
    dt_bias = rng.standard_normal(dim) * 0.5
    beta = rng.standard_normal((batch, N, 1))
    gamma = rng.standard_normal((batch, N, 1))
    B = np.broadcast_to(beta, (batch, N, L)).copy()
    C = np.broadcast_to(gamma, (batch, N, L)).copy()
    D = rng.standard_normal(dim)
    x = rng.standard_normal((batch, dim, L))
    dl = softplus_lib(c[..., 0] + dt_bias[None, :])  # [batch, dim]
    k = np.arange(L)
    # K[b, d, k] = sum_n gamma_bn * exp(k * dl_bd * A_dn) * dl_bd * beta_bn
    K = np.einsum("bn,bdkn->bdk", gamma[..., 0],
                  np.exp(k[None, None, :, None] * dl[:, :, None, None] * A[None, :, None, :])
                  * dl[:, :, None, None] * beta[:, None, None, :, 0])
    return dict(x=x, delta=delta, A=A, B=B, C=C, D=D, dt_bias=dt_bias), K, dl


def pin_lti_convolution_direct(O):
    """Time-invariant case ("State Space Models and Mamba", multigrid.ai,
    "Why a linear recurrence can be trained in parallel"): with step size, B
    and C constant in time the output is a causal convolution of x with the
    kernel K_k = sum_n C_n exp(k delta A_n) delta B_n, plus D x.
    Direct O(L^2) sum with numpy.convolve; also the last state in closed form.
    """
    batch, dim, N, L = 2, 3, 16, 200
    p, K, dl = _lti_problem(21, batch, dim, N, L)
    r = O.fwd(**p)
    for b in range(batch):
        for d in range(dim):
            x = p["x"][b, d]
            want = np.convolve(x, K[b, d])[:L] + p["D"][d] * x
            scale = np.convolve(np.abs(x), np.abs(K[b, d]))[:L] + np.abs(p["D"][d] * x)
            _close(r["y"][b, d], want, 1e-11, scale, what=f"LTI direct b={b} d={d}")
            # last state: h_n = sum_k exp(k dl A_n) dl B_n x_{L-1-k}
            k = np.arange(L)
            hn = np.array([np.sum(np.exp(k * dl[b, d] * p["A"][d, n]) * dl[b, d]
                                  * p["B"][b, n, 0] * x[::-1]) for n in range(N)])
            hs = np.array([np.sum(np.exp(k * dl[b, d] * p["A"][d, n]) * dl[b, d]
                                  * abs(p["B"][b, n, 0]) * np.abs(x[::-1])) for n in range(N)])
            _close(r["last_state"][b, d], hn, 1e-11, hs, what="LTI last state")


def pin_lti_convolution_fft(O):
    """Same time-invariant closed form at L = 4096 through an FFT convolution
    (scipy.signal.fftconvolve), the S4 route the same page describes."""
    batch, dim, N, L = 1, 2, 16, 4096
    p, K, _ = _lti_problem(22, batch, dim, N, L)
    r = O.fwd(**p)
    for d in range(dim):
        x = p["x"][0, d]
        want = scipy.signal.fftconvolve(x, K[0, d])[:L] + p["D"][d] * x
        scale = np.max(np.convolve(np.abs(x), np.abs(K[0, d]))[:L] + np.abs(p["D"][d] * x))
        _close(r["y"][0, d], want, 1e-9, scale, what=f"LTI fft d={d}")


# ----------------------------------------------------------------------------
# Brute force on tiny inputs
# ----------------------------------------------------------------------------

def _brute(p, h0=None):
    """Unrolled sums: h_t = prod_{j<=t} Abar_j h0 + sum_{s<=t} exp(A sum_{s<j<=t} delta_j) delta_s B_s x_s,
    with the products formed from the summed step sizes, from scratch per (s, t)."""
    x, delta, A, B, C = p["x"], p["delta"], p["A"], p["B"], p["C"]
    batch, dim, L = x.shape
    N = A.shape[1]
    bias = p.get("dt_bias")
    u = delta + (0.0 if bias is None else bias[None, :, None])
    dl = softplus_lib(u)
    y = np.zeros((batch, dim, L)); ys = np.zeros((batch, dim, L))
    hL = np.zeros((batch, dim, N)); hsL = np.zeros((batch, dim, N))
    for b in range(batch):
        for d in range(dim):
            for t in range(L):
                h = np.zeros(N); hs = np.zeros(N)
                for n in range(N):
                    if h0 is not None:
                        f = math.exp(A[d, n] * sum(dl[b, d, j] for j in range(0, t + 1)))
                        h[n] += f * h0[b, d, n]
                        hs[n] += f * abs(h0[b, d, n])
                    for s in range(t + 1):
                        f = math.exp(A[d, n] * sum(dl[b, d, j] for j in range(s + 1, t + 1)))
                        term = f * dl[b, d, s] * B[b, n, s] * x[b, d, s]
                        h[n] += term
                        hs[n] += abs(term)
                Dd = 0.0 if p.get("D") is None else p["D"][d]
                v = sum(C[b, n, t] * h[n] for n in range(N)) + Dd * x[b, d, t]
                sv = sum(abs(C[b, n, t]) * hs[n] for n in range(N)) + abs(Dd * x[b, d, t])
                if p.get("z") is not None:
                    gz = silu_lib(np.array([p["z"][b, d, t]]))[0]
                    v *= gz
                    sv *= abs(gz)
                y[b, d, t] = v; ys[b, d, t] = sv
                if t == L - 1:
                    hL[b, d] = h; hsL[b, d] = hs
    return y, ys, hL, hsL


def _rand_problem(seed, batch, dim, N, L, gate=True, with_D=True, with_bias=True):
    rng = np.random.default_rng(seed)
    p = dict(
        x=rng.standard_normal((batch, dim, L)),
        delta=rng.standard_normal((batch, dim, L)),
        A=-rng.uniform(0.1, 4.0, (dim, N)),
        B=rng.standard_normal((batch, N, L)),
        C=rng.standard_normal((batch, N, L)),
    )
    if with_D:
        p["D"] = rng.uniform(0.5, 1.5, dim)
    if gate:
        p["z"] = rng.standard_normal((batch, dim, L)) * 2.0
    if with_bias:
        p["dt_bias"] = rng.standard_normal(dim) - 1.0
    return p


def pin_bruteforce_unrolled(O):
    """Everything time-varying, L <= 8: oracle vs the unrolled sums of
    "State Space Models and Mamba" (multigrid.ai, "Why a linear recurrence can be
    trained in parallel"), generalised to per-step decays; outputs and scales."""
    cases = [(1, 1, 1), (1, 8, 2), (5, 7, 3), (16, 8, 4), (16, 3, 5), (3, 6, 6)]
    for N, L, seed in cases:
        p = _rand_problem(100 + seed, 2, 3, N, L)
        r = O.fwd(**p)
        y, ys, hL, hsL = _brute(p)
        _close(r["y"], y, 1e-12, ys, what=f"brute y N={N} L={L}")
        _close(r["last_state"], hL, 1e-12, hsL, what=f"brute state N={N} L={L}")
        _close(r["y_scale"], ys, 1e-12, ys, what=f"brute y scale N={N} L={L}")
        _close(r["state_scale"], hsL, 1e-12, hsL, what=f"brute state scale N={N} L={L}")


def pin_bruteforce_initial_state(O):
    """Same brute force with a nonzero state before the first token."""
    for N, L, seed in [(4, 5, 1), (16, 6, 2)]:
        p = _rand_problem(200 + seed, 2, 3, N, L)
        h0 = np.random.default_rng(300 + seed).standard_normal((2, 3, N))
        r = O.fwd(**p, h0=h0)
        y, ys, hL, hsL = _brute(p, h0=h0)
        _close(r["y"], y, 1e-12, ys, what=f"brute h0 y N={N}")
        _close(r["last_state"], hL, 1e-12, hsL, what=f"brute h0 state N={N}")


def pin_decode_step_bruteforce(O):
    """One decode step against the single-token unrolled form
    h' = exp(delta A) h + delta B x, y = (C h' + D x) silu(z), delta = softplus(delta_in)."""
    rng = np.random.default_rng(31)
    batch, dim, N = 3, 5, 16
    h = rng.standard_normal((batch, dim, N))
    x = rng.standard_normal((batch, dim)); din = rng.standard_normal((batch, dim))
    z = rng.standard_normal((batch, dim)); D = rng.uniform(0.5, 1.5, dim)
    A = -rng.uniform(0.1, 4.0, (dim, N))
    B = rng.standard_normal((batch, N)); C = rng.standard_normal((batch, N))
    r = O.step(h, x, din, A, B, C, D=D, z=z)
    dl = softplus_lib(din)
    hn = np.exp(dl[..., None] * A[None]) * h + dl[..., None] * B[:, None, :] * x[..., None]
    y = (np.einsum("bdn,bn->bd", hn, C) + D[None] * x) * silu_lib(z)
    hs = np.exp(dl[..., None] * A[None]) * np.abs(h) + np.abs(dl[..., None] * B[:, None, :] * x[..., None])
    ys = (np.einsum("bdn,bn->bd", hs, np.abs(C)) + np.abs(D[None] * x)) * np.abs(silu_lib(z))
    _close(r["state"], hn, 1e-13, hs, what="step state")
    _close(r["y"], y, 1e-13, ys, what="step y")
    _close(r["y_scale"], ys, 1e-13, ys, what="step y scale")


# ----------------------------------------------------------------------------
# Library routines through the public entry
# ----------------------------------------------------------------------------

def pin_softplus_library(O):
    """One token, one state, A = 0, B = C = x = 1: y equals the step size
    softplus(delta_raw + dt_bias), compared with numpy's logaddexp over
    [-40, 40]."""
    dim = 801
    u = np.linspace(-40, 40, dim)
    bias = np.linspace(-1.0, 1.0, dim)
    delta = (u - bias).reshape(1, dim, 1)
    ones = np.ones((1, 1, 1))
    r = O.fwd(np.ones((1, dim, 1)), delta, np.zeros((dim, 1)), ones, ones, dt_bias=bias)
    want = softplus_lib(delta[0, :, 0] + bias)
    _close(r["y"][0, :, 0], want, 1e-14, np.abs(want), what="softplus")


def pin_silu_library(O):
    """One token, B = 0 so the state stays 0, D = x = 1: y equals silu(z),
    compared with torch.nn.functional.silu in float64."""
    dim = 401
    z = np.linspace(-30, 30, dim).reshape(1, dim, 1)
    zero = np.zeros((1, 1, 1))
    r = O.fwd(np.ones((1, dim, 1)), np.zeros((1, dim, 1)), -np.ones((dim, 1)), zero, zero,
              D=np.ones(dim), z=z)
    want = silu_lib(z[0, :, 0])
    _close(r["y"][0, :, 0], want, 1e-14, np.abs(want) + 1e-300, what="silu")


# ----------------------------------------------------------------------------
# Exact invariants
# ----------------------------------------------------------------------------

def pin_scale_equals_value_for_positive_terms(O):
    """When every term is nonnegative (x, B, C > 0, D >= 0, z > 0 so silu > 0)
    the error scales equal the values themselves."""
    p = _rand_problem(41, 2, 3, 16, 50)
    for k in ("x", "B", "C", "z"):
        p[k] = np.abs(p[k]) + 0.01
    r = O.fwd(**p)
    _close(r["y_scale"], r["y"], 1e-13, np.abs(r["y"]), what="positive y scale")
    _close(r["state_scale"], r["last_state"], 1e-13, np.abs(r["last_state"]), what="positive state scale")


def pin_split_invariance(O):
    """Running tokens [0, L1) then [L1, L) from the carried state equals one pass."""
    p = _rand_problem(51, 2, 3, 16, 97)
    full = O.fwd(**p)
    for L1 in (1, 40, 96):
        a = {k: (v[..., :L1] if k in ("x", "delta", "z", "B", "C") else v) for k, v in p.items()}
        b = {k: (v[..., L1:] if k in ("x", "delta", "z", "B", "C") else v) for k, v in p.items()}
        ra = O.fwd(**a)
        rb = O.fwd(**b, h0=ra["last_state"], h0_scale=ra["state_scale"])
        _close(np.concatenate([ra["y"], rb["y"]], -1), full["y"], 1e-13, full["y_scale"],
               what=f"split y L1={L1}")
        _close(rb["last_state"], full["last_state"], 1e-13, full["state_scale"], what="split state")


def pin_forward_equals_steps(O):
    """Forward over L tokens equals L decode steps fed delta_raw + dt_bias
    (the two execution modes of the same layer)."""
    p = _rand_problem(61, 2, 3, 16, 20)
    full = O.fwd(**p)
    h = np.zeros((2, 3, 16))
    hs = np.zeros_like(h)
    for t in range(20):
        r = O.step(h, p["x"][..., t], p["delta"][..., t] + p["dt_bias"][None, :], p["A"],
                   p["B"][..., t], p["C"][..., t], D=p["D"], z=p["z"][..., t], state_scale=hs)
        h, hs = r["state"], r["state_scale"]
        _close(r["y"], full["y"][..., t], 1e-14, full["y_scale"][..., t], what=f"steps y t={t}")
        _close(r["y_scale"], full["y_scale"][..., t], 1e-14, full["y_scale"][..., t], what="steps y scale")
    _close(h, full["last_state"], 1e-14, full["state_scale"], what="steps state")


def pin_linearity_and_zero(O):
    """Without the gate the output is linear in x for fixed delta, B, C; zero
    input gives exactly zero output and state."""
    p1 = _rand_problem(71, 2, 3, 16, 30, gate=False)
    x2 = np.random.default_rng(72).standard_normal(p1["x"].shape)
    p2 = dict(p1, x=x2)
    p12 = dict(p1, x=2.5 * p1["x"] - 0.75 * x2)
    r1, r2, r12 = O.fwd(**p1), O.fwd(**p2), O.fwd(**p12)
    want = 2.5 * r1["y"] - 0.75 * r2["y"]
    scale = 2.5 * r1["y_scale"] + 0.75 * r2["y_scale"]
    _close(r12["y"], want, 1e-13, scale, what="linearity y")
    r0 = O.fwd(**dict(p1, x=np.zeros_like(x2)))
    assert np.all(r0["y"] == 0.0) and np.all(r0["last_state"] == 0.0), "zero in, zero out"


def pin_state_embedding(O):
    """N = 16 with B[n >= 1] = 0 gives the N = 1 result (states 1..15 stay 0)."""
    p = _rand_problem(81, 2, 3, 16, 25)
    p1 = dict(p, A=p["A"][:, :1], B=p["B"][:, :1], C=p["C"][:, :1])
    pe = dict(p, B=np.concatenate([p["B"][:, :1], np.zeros_like(p["B"][:, 1:])], 1))
    r1, re = O.fwd(**p1), O.fwd(**pe)
    _close(re["y"], r1["y"], 0.0, what="embedding y")
    assert np.all(re["last_state"][..., 1:] == 0.0)


def pin_row_subset_and_threads(O):
    """Computing a subset of rows, or with any thread count, gives the same bits."""
    p = _rand_problem(91, 3, 5, 16, 33)
    full = O.fwd(**p, nthreads=1)
    rows = [14, 0, 7, 7, 3]
    sub = O.fwd(**p, rows=rows, nthreads=3)
    flat = full["y"].reshape(15, -1)
    assert np.array_equal(sub["y"], flat[rows]), "row subset"
    many = O.fwd(**p, nthreads=8)
    assert np.array_equal(many["y"], full["y"]), "thread count"


def pin_nan_propagation(O):
    """A NaN input at (b, d, t0) makes that row's outputs from t0 on NaN and
    leaves every other row finite."""
    p = _rand_problem(95, 2, 3, 16, 12)
    p["x"][1, 2, 5] = np.nan
    r = O.fwd(**p)
    assert np.all(np.isnan(r["y"][1, 2, 5:])) and np.all(np.isfinite(r["y"][1, 2, :5]))
    mask = np.ones((2, 3), bool); mask[1, 2] = False
    assert np.all(np.isfinite(r["y"][mask]))
    assert np.all(np.isnan(r["last_state"][1, 2]))


# ----------------------------------------------------------------------------
# The short causal convolution (depthwise, width K) + SiLU, and its step
# ----------------------------------------------------------------------------

def _conv_problem(seed, batch, dim, L, K=4, with_bias=True, with_prev=True):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((batch, dim, L)),
                w=rng.standard_normal((dim, K)) * 0.7,
                bias=rng.standard_normal(dim) * 0.3 if with_bias else None,
                x_prev=rng.standard_normal((batch, dim, K - 1)) if with_prev else None)


def pin_conv1d_library_filter(O):
    """Each row against scipy's FIR filter (lfilter with the taps reversed is
    the causal sum over the last K inputs), then torch's silu; the inputs
    before token 0 are prepended explicitly (or zeros)."""
    for with_prev in (False, True):
        p = _conv_problem(31, 2, 5, 23, with_prev=with_prev)
        r = O.conv1d(p["x"], p["w"], p["bias"], p["x_prev"])
        K = p["w"].shape[1]
        for b in range(2):
            for d in range(5):
                prev = p["x_prev"][b, d] if with_prev else np.zeros(K - 1)
                seq = np.concatenate([prev, p["x"][b, d]])
                pre = scipy.signal.lfilter(p["w"][d, ::-1], [1.0], seq)[K - 1:] + p["bias"][d]
                _close(r["out"][b, d], silu_lib(pre), 1e-12, what=f"conv lfilter prev={with_prev}")
                _close(r["x_last"][b, d], seq[-(K - 1):], 0.0, what="conv x_last")


def pin_conv1d_torch_grouped(O):
    """Against torch's grouped conv1d in fp64 (groups = channels, left padding
    K-1, first L outputs): the layer the pages name, from a library."""
    p = _conv_problem(32, 3, 7, 40, with_prev=False)
    K = p["w"].shape[1]
    xt = torch.from_numpy(p["x"])
    ref = torch.nn.functional.conv1d(xt, torch.from_numpy(p["w"])[:, None, :],
                                     torch.from_numpy(p["bias"]), padding=K - 1, groups=7)
    ref = torch.nn.functional.silu(ref[..., :40]).numpy()
    _close(O.conv1d(p["x"], p["w"], p["bias"])["out"], ref, 1e-12, what="conv torch grouped")


def pin_conv1d_bwd_torch_autograd(O):
    """Every gradient of the convolution (x, the inputs before token 0, taps,
    bias) against torch autograd in fp64 of the grouped conv1d (the
    library's chain rule) over the previous inputs prepended, then silu."""
    for with_bias in (True, False):
        p = _conv_problem(35, 2, 5, 19, with_bias=with_bias)
        dout = np.random.default_rng(36).standard_normal((2, 5, 19))
        r = O.conv1d_bwd(p["x"], p["w"], p["bias"], p["x_prev"], dout=dout)
        K = p["w"].shape[1]
        T = {k: torch.tensor(p[k], requires_grad=True) for k in ("x", "w", "x_prev")}
        bias = torch.tensor(p["bias"], requires_grad=True) if with_bias else None
        seq = torch.cat([T["x_prev"], T["x"]], dim=-1)
        pre = torch.nn.functional.conv1d(seq, T["w"][:, None, :], bias, groups=5)
        (torch.nn.functional.silu(pre) * torch.from_numpy(dout)).sum().backward()
        for k, g in (("x", "dx"), ("w", "dw"), ("x_prev", "dx_prev")):
            _close(r[g], T[k].grad.numpy(), 1e-12, scale=r[g + "_scale"] + 1e-300,
                   what=f"conv bwd autograd {g} bias={with_bias}")
        if with_bias:
            _close(r["dbias"], bias.grad.numpy(), 1e-12, scale=r["dbias_scale"] + 1e-300,
                   what="conv bwd autograd dbias")
        assert np.all(r["dx_scale"] >= np.abs(r["dx"]) * (1 - 1e-12))


def pin_conv1d_bwd_finite_differences(O):
    """Central differences of sum(dout * out) through the oracle's own
    convolution, every element of every input, on a tiny problem."""
    p = _conv_problem(37, 2, 2, 6)
    dout = np.random.default_rng(38).standard_normal((2, 2, 6))
    r = O.conv1d_bwd(p["x"], p["w"], p["bias"], p["x_prev"], dout=dout)

    def loss(q):
        return float(np.sum(dout * O.conv1d(q["x"], q["w"], q["bias"], q["x_prev"])["out"]))

    for name, gname in (("x", "dx"), ("w", "dw"), ("bias", "dbias"), ("x_prev", "dx_prev")):
        base = p[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            eps = 1e-6 * max(1.0, abs(base[idx]))
            q = dict(p); arr = base.copy(); arr[idx] += eps; q[name] = arr
            lp = loss(q)
            arr = base.copy(); arr[idx] -= eps; q[name] = arr
            fd[idx] = (lp - loss(q)) / (2 * eps)
        _close(r[gname], fd, 1e-6, scale=np.maximum(np.abs(fd), 1.0), what=f"conv bwd finite diff {gname}")


def pin_conv1d_one_hot_taps(O):
    """A single tap k = K-1-j gives out[t] = silu(x[t-j]) (zero before the
    start): fixes the causal direction and the tap order."""
    rng = np.random.default_rng(33)
    x = rng.standard_normal((1, 4, 12))
    for j in range(4):
        w = np.zeros((4, 4)); w[:, 3 - j] = 1.0
        out = O.conv1d(x, w)["out"]
        shifted = np.concatenate([np.zeros((1, 4, j)), x[..., :12 - j]], axis=-1)
        _close(out, silu_lib(shifted), 1e-14, what=f"conv one-hot shift {j}")


def pin_conv1d_streaming(O):
    """Feeding [0, t) then [t, L) with x_prev = the first call's x_last equals
    one call, for splits shorter and longer than the window."""
    p = _conv_problem(34, 2, 3, 30)
    whole = O.conv1d(p["x"], p["w"], p["bias"], p["x_prev"])
    for t in (1, 2, 3, 11):
        a = O.conv1d(p["x"][..., :t], p["w"], p["bias"], p["x_prev"])
        b = O.conv1d(p["x"][..., t:], p["w"], p["bias"], a["x_last"])
        _close(np.concatenate([a["out"], b["out"]], -1), whole["out"], 0.0, what=f"conv split {t}")
        _close(b["x_last"], whole["x_last"], 0.0, what="conv split x_last")


def pin_conv1d_steps_equal_call(O):
    """L decode steps from conv_state = x_prev give the call's outputs, and
    the final conv_state is its x_last."""
    p = _conv_problem(35, 2, 3, 9)
    whole = O.conv1d(p["x"], p["w"], p["bias"], p["x_prev"])
    st = p["x_prev"]
    for t in range(9):
        r = O.conv1d_step(st, p["x"][..., t], p["w"], p["bias"])
        _close(r["out"], whole["out"][..., t], 0.0, what=f"conv step {t}")
        _close(r["out_scale"], whole["out_scale"][..., t], 0.0, what=f"conv step scale {t}")
        st = r["conv_state"]
    _close(st, whole["x_last"], 0.0, what="conv step final state")


def pin_conv1d_scale(O):
    """With every term nonnegative the scale is the pre-activation itself
    (and out = silu(scale)); with mixed signs it is the sum of |terms|,
    brute-forced here."""
    rng = np.random.default_rng(36)
    x = rng.uniform(0.1, 1.0, (1, 3, 10)); w = rng.uniform(0.1, 1.0, (3, 4))
    bias = rng.uniform(0.0, 0.5, 3); prev = rng.uniform(0.1, 1.0, (1, 3, 3))
    r = O.conv1d(x, w, bias, prev)
    _close(r["out"], silu_lib(r["out_scale"]), 1e-14, what="conv positive scale")
    p = _conv_problem(37, 1, 2, 6)
    r = O.conv1d(p["x"], p["w"], p["bias"], p["x_prev"])
    seq = np.concatenate([p["x_prev"], p["x"]], -1)
    for d in range(2):
        for t in range(6):
            want = abs(p["bias"][d]) + sum(abs(p["w"][d, k] * seq[0, d, t + k]) for k in range(4))
            _close(r["out_scale"][0, d, t], want, 1e-14, what="conv mixed scale")


# ----------------------------------------------------------------------------
# Backward pass
# ----------------------------------------------------------------------------

def _bwd_problem(seed, batch, dim, N, L, gate=True, with_D=True, with_bias=True):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((batch, dim, L)), delta=rng.standard_normal((batch, dim, L)),
                A=-rng.uniform(0.3, 2.0, (dim, N)), B=rng.standard_normal((batch, N, L)),
                C=rng.standard_normal((batch, N, L)),
                D=rng.standard_normal(dim) if with_D else None,
                z=rng.standard_normal((batch, dim, L)) if gate else None,
                dt_bias=rng.standard_normal(dim) * 0.5 if with_bias else None,
                dy=rng.standard_normal((batch, dim, L)))


_GRAD_OF = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
            "dt_bias": "ddt_bias", "h0": "dh0"}


def _torch_grads(p):
    """Gradients from torch autograd (fp64) of the forward written with torch
    ops: a library's chain rule, not the oracle's. With ``h0`` in p the
    recurrence starts there; with ``dlast`` the loss adds sum(dlast * h_L)."""
    T = {k: (torch.tensor(v, dtype=torch.float64, requires_grad=True) if v is not None else None)
         for k, v in p.items() if k not in ("dy", "dlast")}
    x, dl, A, B, C = T["x"], T["delta"], T["A"], T["B"], T["C"]
    batch, dim, L = x.shape
    N = A.shape[1]
    u = dl + (T["dt_bias"][None, :, None] if T["dt_bias"] is not None else 0.0)
    delta = torch.nn.functional.softplus(u)
    h = T["h0"] if T.get("h0") is not None else torch.zeros((batch, dim, N), dtype=torch.float64)
    ys = []
    for t in range(L):
        abar = torch.exp(delta[:, :, t, None] * A[None])
        h = abar * h + delta[:, :, t, None] * B[:, None, :, t] * x[:, :, t, None]
        yt = (h * C[:, None, :, t]).sum(-1)
        if T["D"] is not None:
            yt = yt + T["D"][None] * x[:, :, t]
        ys.append(yt)
    y = torch.stack(ys, -1)
    if T["z"] is not None:
        y = y * torch.nn.functional.silu(T["z"])
    loss = (y * torch.tensor(p["dy"])).sum()
    if p.get("dlast") is not None:
        loss = loss + (h * torch.tensor(p["dlast"])).sum()
    loss.backward()
    return {_GRAD_OF[k]: v.grad.numpy() for k, v in T.items() if v is not None}


def pin_bwd_torch_autograd(O):
    """Every gradient against torch autograd of the same forward in fp64, with
    and without the optional inputs."""
    for kw in (dict(), dict(gate=False, with_D=False, with_bias=False)):
        p = _bwd_problem(41, 2, 3, 4, 17, **kw)
        r = O.bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["dt_bias"],
                  dy=p["dy"])
        ref = _torch_grads(p)
        for k, v in ref.items():
            _close(r[k], v, 1e-10, scale=r[k + "_scale"] + 1e-300, what=f"bwd autograd {k} {kw}")
        for k in ("dD", "dz", "ddt_bias"):
            assert (k in r) == (k in ref), k


def pin_bwd_initial_and_final_state_autograd(O):
    """With an initial state h0 and a gradient flowing into the final state:
    every gradient and dh0 against torch autograd (fp64) of the same forward,
    the loss being sum(dy * y) + sum(dlast * h_L)."""
    for kw in (dict(), dict(gate=False, with_D=False, with_bias=False)):
        p = _bwd_problem(44, 2, 3, 4, 13, **kw)
        rng = np.random.default_rng(45)
        p["h0"] = rng.standard_normal((2, 3, 4))
        p["dlast"] = rng.standard_normal((2, 3, 4))
        r = O.bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["dt_bias"],
                  dy=p["dy"], h0=p["h0"], dlast_state=p["dlast"], want_dh0=True)
        ref = _torch_grads(p)
        assert "dh0" in ref
        for k, v in ref.items():
            _close(r[k], v, 1e-10, scale=r[k + "_scale"] + 1e-300, what=f"bwd h0/dlast autograd {k} {kw}")
    # No tokens: last_state = h0, so dh0 = dlast and every other gradient is zero.
    p = _bwd_problem(46, 1, 2, 3, 0)
    h0 = np.random.default_rng(47).standard_normal((1, 2, 3))
    dl = np.random.default_rng(48).standard_normal((1, 2, 3))
    r = O.bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["dt_bias"],
              dy=p["dy"], h0=h0, dlast_state=dl, want_dh0=True)
    assert np.array_equal(r["dh0"], dl)
    assert not np.any(r["dA"]) and not np.any(r["dD"]) and not np.any(r["ddt_bias"])


def pin_bwd_finite_differences(O):
    """Central differences of the loss sum(dy * y) through the oracle's own
    forward pass, every element of every input, on a tiny problem."""
    p = _bwd_problem(42, 2, 2, 3, 5)
    rng = np.random.default_rng(49)
    p["h0"] = rng.standard_normal((2, 2, 3))
    dlast = rng.standard_normal((2, 2, 3))
    r = O.bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["dt_bias"], dy=p["dy"],
              h0=p["h0"], dlast_state=dlast, want_dh0=True)

    def loss(q):
        o = O.fwd(q["x"], q["delta"], q["A"], q["B"], q["C"], q["D"], q["z"], q["dt_bias"], h0=q["h0"])
        return float(np.sum(p["dy"] * o["y"]) + np.sum(dlast * o["last_state"]))

    for name, gname in _GRAD_OF.items():
        base = p[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            eps = 1e-6 * max(1.0, abs(base[idx]))
            q = dict(p); arr = base.copy(); arr[idx] += eps; q[name] = arr
            lp = loss(q)
            arr = base.copy(); arr[idx] -= eps; q[name] = arr
            lm = loss(q)
            fd[idx] = (lp - lm) / (2 * eps)
        _close(r[gname], fd, 1e-6, scale=np.maximum(np.abs(fd), 1.0), what=f"bwd finite diff {gname}")


def pin_bwd_scales_bound_values(O):
    """Each error scale is at least the magnitude of its value, and the
    gradients are linear in dy (doubling dy doubles every gradient exactly)."""
    p = _bwd_problem(43, 2, 3, 5, 11)
    args = (p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["dt_bias"])
    r = O.bwd(*args, dy=p["dy"])
    r2 = O.bwd(*args, dy=2.0 * p["dy"])
    for k in ("dx", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddt_bias"):
        assert np.all(r[k + "_scale"] >= np.abs(r[k]) * (1 - 1e-12)), k
        _close(r2[k], 2.0 * r[k], 0.0, what=f"bwd linear in dy {k}")


# ----------------------------------------------------------------------------
# Mamba-2 SSD layer
# ----------------------------------------------------------------------------

def _ssd_problem(seed, batch, L, H, P, N, with_D=True, with_bias=True):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((batch, L, H, P)), delta=rng.standard_normal((batch, L, H)),
                A=-rng.uniform(0.2, 2.0, H), B=rng.standard_normal((batch, L, N)),
                C=rng.standard_normal((batch, L, N)),
                D=rng.standard_normal(H) if with_D else None,
                dt_bias=rng.standard_normal(H) * 0.5 if with_bias else None)


def pin_ssd_equals_restricted_selective_scan(O):
    """SSD is the selective scan with A[d, n] = A_h for every state n, one step
    size per head and B, C shared: run the (separately pinned) selective-scan
    definition on the channels of every head and compare y and the state."""
    p = _ssd_problem(51, 2, 23, 3, 4, 5)
    r = O.ssd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["dt_bias"])
    batch, L, H, P = p["x"].shape
    N = p["B"].shape[2]
    x = p["x"].transpose(0, 2, 3, 1).reshape(batch, H * P, L)          # channel d = h*P + p
    delta = np.repeat(p["delta"].transpose(0, 2, 1), P, axis=1)
    A = np.repeat(p["A"], P)[:, None] * np.ones((1, N))
    s6 = O.fwd(x, delta, A, p["B"].transpose(0, 2, 1), p["C"].transpose(0, 2, 1),
               D=np.repeat(p["D"], P), dt_bias=np.repeat(p["dt_bias"], P))
    _close(r["y"], s6["y"].reshape(batch, H, P, L).transpose(0, 3, 1, 2), 1e-12, what="ssd vs S6 y")
    _close(r["last_state"], s6["last_state"].reshape(batch, H, P, N).transpose(0, 1, 3, 2), 1e-12,
           what="ssd vs S6 state")
    _close(r["y_scale"], s6["y_scale"].reshape(batch, H, P, L).transpose(0, 3, 1, 2), 1e-12,
           what="ssd vs S6 scale")


def pin_ssd_initial_state_and_step(O):
    """From an initial state: SSD equals the (separately pinned) selective scan
    started from the same state laid out per channel (d = h*P + p, state
    [d, n]); and one decode step is the layer over one token from the state,
    so L steps give the L-token call."""
    p = _ssd_problem(53, 2, 19, 3, 4, 5)
    batch, L, H, P = p["x"].shape
    N = p["B"].shape[2]
    h0 = np.random.default_rng(54).standard_normal((batch, H, N, P))
    r = O.ssd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["dt_bias"], h0=h0)
    x = p["x"].transpose(0, 2, 3, 1).reshape(batch, H * P, L)
    delta = np.repeat(p["delta"].transpose(0, 2, 1), P, axis=1)
    A = np.repeat(p["A"], P)[:, None] * np.ones((1, N))
    s6 = O.fwd(x, delta, A, p["B"].transpose(0, 2, 1), p["C"].transpose(0, 2, 1),
               D=np.repeat(p["D"], P), dt_bias=np.repeat(p["dt_bias"], P),
               h0=h0.transpose(0, 1, 3, 2).reshape(batch, H * P, N))
    _close(r["y"], s6["y"].reshape(batch, H, P, L).transpose(0, 3, 1, 2), 1e-12, what="ssd h0 vs S6 y")
    _close(r["last_state"], s6["last_state"].reshape(batch, H, P, N).transpose(0, 1, 3, 2), 1e-12,
           what="ssd h0 vs S6 state")
    st = h0
    for t in range(L):
        o = O.ssd_step(st, p["x"][:, t], p["delta"][:, t], p["A"], p["B"][:, t], p["C"][:, t],
                       p["D"], p["dt_bias"])
        _close(o["y"], r["y"][:, t], 1e-12, what=f"ssd step {t} y")
        st = o["state"]
    _close(st, r["last_state"], 1e-12, what="ssd steps final state")


def pin_ssd_dual_quadratic_form(O):
    """The attention-like dual: y = (Lmask o C B^T)(delta x) + D x with
    Lmask[t,s] = exp(A_h sum_{s<k<=t} delta_k) (s <= t), by numpy matrix
    products; and the last state sum_s exp(A_h sum_{k>s} delta_k) delta_s
    B_s x_s^T."""
    for kw in (dict(), dict(with_D=False, with_bias=False)):
        p = _ssd_problem(52, 2, 31, 2, 3, 4, **kw)
        r = O.ssd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["dt_bias"])
        batch, L, H, P = p["x"].shape
        bias = p["dt_bias"] if p["dt_bias"] is not None else np.zeros(H)
        for b in range(batch):
            CBt = p["C"][b] @ p["B"][b].T                                  # [L, L]
            for h in range(H):
                dl = softplus_lib(p["delta"][b, :, h] + bias[h])
                cum = np.cumsum(dl)
                seg = cum[:, None] - cum[None, :]                            # sum_{s<k<=t}
                Lmask = np.where(np.tril(np.ones((L, L))) > 0, np.exp(p["A"][h] * seg), 0.0)
                xs = p["x"][b, :, h, :]
                y = (Lmask * CBt) @ (dl[:, None] * xs)
                if p["D"] is not None:
                    y = y + p["D"][h] * xs
                _close(r["y"][b, :, h, :], y, 1e-11, scale=r["y_scale"][b, :, h, :] + 1e-300,
                       what=f"ssd dual form {kw}")
                w = np.exp(p["A"][h] * (cum[-1] - cum)) * dl
                S = p["B"][b].T @ (w[:, None] * xs)                          # [N, P]
                _close(r["last_state"][b, h], S, 1e-11, scale=r["state_scale"][b, h] + 1e-300,
                       what="ssd dual last state")


PINS = {name: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}
