"""Python entry to the fp64 CPU oracle of the selective scan (S6).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the CPU-baseline leg of the benchmark. The GPU library never imports or links
it, and it imports nothing from the GPU library.

The arithmetic lives in ``selscan_ref.c`` (plain C, IEEE double, libm); this
module only converts arrays to float64 and calls it. The definition it
follows, with its citations of the pages, is in the header of that file.

Every array argument is converted exactly to float64 (float32 and bfloat16
values are exactly representable). Layouts:

* ``x, delta, z``: ``[batch, dim, seqlen]``
* ``B, C``: ``[batch, dstate, seqlen]``
* ``A``: ``[dim, dstate]``; ``D, dt_bias``: ``[dim]``
* states: ``[batch, dim, dstate]``
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "selscan_ref.c")
_LIB_PATH = os.path.join(_HERE, "libselscan_ref.so")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, strict IEEE: no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
               "-shared", "-pthread", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor (any dtype, any device)
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


class Oracle:
    """The oracle library loaded from ``path`` (default: the built one)."""

    def __init__(self, path: Optional[str] = None):
        path = path or _LIB_PATH
        if path == _LIB_PATH and not os.path.exists(path):
            build(force=False)
        lib = ctypes.CDLL(path)
        lib.ssm_ref_fwd.restype = ctypes.c_int
        lib.ssm_ref_fwd.argtypes = [_dp] * 10 + [ctypes.c_int64] * 4 + [_ip, ctypes.c_int64] + \
            [_dp] * 4 + [ctypes.c_int]
        lib.ssm_ref_step.restype = ctypes.c_int
        lib.ssm_ref_step.argtypes = [_dp] * 9 + [ctypes.c_int64] * 3 + [_dp] * 2
        lib.ssm_ref_bwd.restype = ctypes.c_int
        lib.ssm_ref_bwd.argtypes = [_dp] * 11 + [ctypes.c_int64] * 4 + [_dp] * 18 + [ctypes.c_int]
        lib.ssm_ref_ssd.restype = ctypes.c_int
        lib.ssm_ref_ssd.argtypes = [_dp] * 8 + [ctypes.c_int64] * 5 + [_dp] * 4 + [ctypes.c_int]
        lib.ssm_ref_conv1d.restype = ctypes.c_int
        lib.ssm_ref_conv1d.argtypes = [_dp] * 4 + [ctypes.c_int64] * 4 + [_dp] * 3
        lib.ssm_ref_conv1d_bwd.restype = ctypes.c_int
        lib.ssm_ref_conv1d_bwd.argtypes = [_dp] * 5 + [ctypes.c_int64] * 4 + [_dp] * 8
        lib.ssm_ref_conv1d_step.restype = ctypes.c_int
        lib.ssm_ref_conv1d_step.argtypes = [_dp] * 4 + [ctypes.c_int64] * 3 + [_dp] * 2
        self.lib = lib
        self.path = path

    def bwd(self, x, delta, A, B, C, D=None, z=None, dt_bias=None, *, dy, h0=None,
            dlast_state=None, want_dh0: bool = False, nthreads: Optional[int] = None):
        """Gradients of the forward pass for an output gradient ``dy``
        ``[batch, dim, seqlen]``: the forward starts from ``h0`` (``[batch,
        dim, dstate]``, zero when None) and ``dlast_state`` (same shape) is the
        gradient flowing into the final state (zero when None).

        Returns a dict with ``dx, ddelta, dA, dB, dC`` and, when the matching
        input is given, ``dD``, ``dz``, ``ddt_bias``, and ``dh0`` when wanted;
        each with a ``<name>_scale`` (the same computation on magnitudes).
        Shapes follow the inputs; dA is ``[dim, dstate]``, dD and ddt_bias
        ``[dim]``. All float64.
        """
        x, delta, A, B, C, dy = map(_f64, (x, delta, A, B, C, dy))
        D, z, dt_bias, h0, dlast_state = map(_f64, (D, z, dt_bias, h0, dlast_state))
        batch, dim, L = x.shape
        N = A.shape[1]
        assert delta.shape == x.shape and dy.shape == x.shape and A.shape == (dim, N)
        assert B.shape == (batch, N, L) and C.shape == (batch, N, L)
        e = lambda *shape: np.zeros(shape, np.float64)
        out = {k: e(batch, dim, L) for k in ("dx", "ddelta", "dx_scale", "ddelta_scale")}
        out.update({k: e(batch, N, L) for k in ("dB", "dC", "dB_scale", "dC_scale")})
        out.update({"dA": e(dim, N), "dA_scale": e(dim, N)})
        if D is not None:
            out.update({"dD": e(dim), "dD_scale": e(dim)})
        if z is not None:
            out.update({"dz": e(batch, dim, L), "dz_scale": e(batch, dim, L)})
        if dt_bias is not None:
            out.update({"ddt_bias": e(dim), "ddt_bias_scale": e(dim)})
        for st in (h0, dlast_state):
            assert st is None or st.shape == (batch, dim, N)
        if want_dh0:
            out.update({"dh0": e(batch, dim, N), "dh0_scale": e(batch, dim, N)})
        g = lambda k: _ptr(out.get(k))
        rc = self.lib.ssm_ref_bwd(
            _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
            _ptr(dy), _ptr(h0), _ptr(dlast_state), batch, L, dim, N,
            g("dx"), g("ddelta"), g("dA"), g("dB"), g("dC"), g("dD"), g("dz"), g("ddt_bias"),
            g("dh0"),
            g("dx_scale"), g("ddelta_scale"), g("dA_scale"), g("dB_scale"), g("dC_scale"),
            g("dD_scale"), g("dz_scale"), g("ddt_bias_scale"), g("dh0_scale"),
            nthreads or default_threads())
        if rc != 0:
            raise RuntimeError(f"ssm_ref_bwd failed with code {rc}")
        return out

    def ssd(self, x, delta, A, B, C, D=None, dt_bias=None, h0=None,
            nthreads: Optional[int] = None):
        """Mamba-2's SSD layer (scalar decay per head), from the state ``h0``
        (``[batch, heads, dstate, headdim]``; zeros when None).

        ``x``: ``[batch, seqlen, heads, headdim]``; ``delta`` (raw):
        ``[batch, seqlen, heads]``; ``A, D, dt_bias``: ``[heads]``; ``B, C``:
        ``[batch, seqlen, dstate]``. Returns ``y``, ``y_scale`` (like x) and
        ``last_state``, ``state_scale`` (``[batch, heads, dstate, headdim]``).
        """
        x, delta, A, B, C, D, dt_bias, h0 = map(_f64, (x, delta, A, B, C, D, dt_bias, h0))
        batch, L, H, P = x.shape
        N = B.shape[2]
        assert delta.shape == (batch, L, H) and A.shape == (H,)
        assert B.shape == (batch, L, N) and C.shape == (batch, L, N)
        assert h0 is None or h0.shape == (batch, H, N, P)
        y = np.empty_like(x)
        ys = np.empty_like(x)
        hs = np.empty((batch, H, N, P), np.float64)
        hss = np.empty((batch, H, N, P), np.float64)
        rc = self.lib.ssm_ref_ssd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                  _ptr(dt_bias), _ptr(h0), batch, L, H, P, N, _ptr(y), _ptr(ys), _ptr(hs),
                                  _ptr(hss), nthreads or default_threads())
        if rc != 0:
            raise RuntimeError(f"ssm_ref_ssd failed with code {rc}")
        return {"y": y, "y_scale": ys, "last_state": hs, "state_scale": hss}

    def ssd_step(self, state, x, delta, A, B, C, D=None, dt_bias=None):
        """One decode step of the SSD layer: the layer over a single token
        from ``state`` ``[batch, heads, dstate, headdim]``. ``x``: ``[batch,
        heads, headdim]``; ``delta`` (raw): ``[batch, heads]``; ``B, C``:
        ``[batch, dstate]``. Returns ``y`` ``[batch, heads, headdim]``,
        ``y_scale``, ``state`` (the new state) and ``state_scale``."""
        x, delta, B, C = (np.asarray(v, np.float64) for v in (x, delta, B, C))
        r = self.ssd(x[:, None], delta[:, None], A, B[:, None], C[:, None], D, dt_bias, h0=state)
        return {"y": r["y"][:, 0], "y_scale": r["y_scale"][:, 0], "state": r["last_state"],
                "state_scale": r["state_scale"]}

    def conv1d(self, x, w, bias=None, x_prev=None):
        """Causal depthwise convolution of width K = w.shape[1], then SiLU.

        ``x``: ``[batch, dim, seqlen]``; ``w``: ``[dim, K]``; ``bias``: ``[dim]``;
        ``x_prev``: ``[batch, dim, K-1]``, the inputs before token 0 (zeros if
        None). Returns a dict with ``out`` and ``out_scale`` (``[batch, dim,
        seqlen]``) and ``x_last`` (``[batch, dim, K-1]``), all float64.
        """
        x, w, bias, x_prev = map(_f64, (x, w, bias, x_prev))
        batch, dim, L = x.shape
        K = w.shape[1]
        assert w.shape == (dim, K)
        if bias is not None:
            assert bias.shape == (dim,)
        if x_prev is not None:
            assert x_prev.shape == (batch, dim, K - 1)
        out = np.empty((batch, dim, L), np.float64)
        sc = np.empty((batch, dim, L), np.float64)
        last = np.empty((batch, dim, K - 1), np.float64)
        rc = self.lib.ssm_ref_conv1d(_ptr(x), _ptr(w), _ptr(bias), _ptr(x_prev), batch, L, dim, K,
                                     _ptr(out), _ptr(sc), _ptr(last))
        if rc != 0:
            raise RuntimeError(f"ssm_ref_conv1d failed with code {rc}")
        return {"out": out, "out_scale": sc, "x_last": last}

    def conv1d_bwd(self, x, w, bias=None, x_prev=None, *, dout):
        """Gradients of ``conv1d`` for an output gradient ``dout`` ``[batch, dim,
        seqlen]``. Returns a dict with ``dx`` (like x), ``dx_prev`` (``[batch,
        dim, K-1]``), ``dw`` (``[dim, K]``) and ``dbias`` (``[dim]``), each with a
        ``<name>_scale``, all float64."""
        x, w, bias, x_prev, dout = map(_f64, (x, w, bias, x_prev, dout))
        batch, dim, L = x.shape
        K = w.shape[1]
        assert w.shape == (dim, K) and dout.shape == x.shape
        e = lambda *shape: np.zeros(shape, np.float64)
        out = {"dx": e(batch, dim, L), "dx_scale": e(batch, dim, L), "dx_prev": e(batch, dim, K - 1),
               "dx_prev_scale": e(batch, dim, K - 1), "dw": e(dim, K), "dw_scale": e(dim, K),
               "dbias": e(dim), "dbias_scale": e(dim)}
        g = lambda k: _ptr(out[k])
        rc = self.lib.ssm_ref_conv1d_bwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(x_prev), _ptr(dout),
                                         batch, L, dim, K, g("dx"), g("dx_prev"), g("dw"), g("dbias"),
                                         g("dx_scale"), g("dx_prev_scale"), g("dw_scale"),
                                         g("dbias_scale"))
        if rc != 0:
            raise RuntimeError(f"ssm_ref_conv1d_bwd failed with code {rc}")
        return out

    def conv1d_step(self, conv_state, x, w, bias=None):
        """One decode step of the convolution from ``conv_state`` ``[batch, dim,
        K-1]`` (oldest first) and ``x`` ``[batch, dim]``. Returns a dict with
        ``out``, ``out_scale`` and the new ``conv_state`` (float64); the inputs
        are not modified."""
        st = _f64(conv_state).copy()
        x, w, bias = map(_f64, (x, w, bias))
        batch, dim = x.shape
        K = w.shape[1]
        assert st.shape == (batch, dim, K - 1) and w.shape == (dim, K)
        out = np.empty((batch, dim), np.float64)
        sc = np.empty((batch, dim), np.float64)
        rc = self.lib.ssm_ref_conv1d_step(_ptr(st), _ptr(x), _ptr(w), _ptr(bias), batch, dim, K,
                                          _ptr(out), _ptr(sc))
        if rc != 0:
            raise RuntimeError(f"ssm_ref_conv1d_step failed with code {rc}")
        return {"out": out, "out_scale": sc, "conv_state": st}

    def fwd(self, x, delta, A, B, C, D=None, z=None, dt_bias=None, h0=None, h0_scale=None,
            rows: Optional[Sequence[int]] = None, nthreads: Optional[int] = None):
        """Selective-scan forward over whole rows.

        ``rows`` (optional) lists flat row indices ``b*dim + d`` to compute; the
        outputs then have a leading axis of ``len(rows)`` instead of
        ``[batch, dim]``. ``h0`` (optional, ``[batch, dim, dstate]``) is the state
        before the first token; ``h0_scale`` its error scale (default ``|h0|``).

        Returns a dict with ``y`` and ``y_scale`` (``[..., seqlen]``) and
        ``last_state`` and ``state_scale`` (``[..., dstate]``), all float64.
        """
        x, delta, A, B, C = map(_f64, (x, delta, A, B, C))
        D, z, dt_bias, h0, h0_scale = map(_f64, (D, z, dt_bias, h0, h0_scale))
        batch, dim, L = x.shape
        N = A.shape[1]
        assert delta.shape == x.shape and A.shape == (dim, N)
        assert B.shape == (batch, N, L) and C.shape == (batch, N, L)
        if z is not None:
            assert z.shape == x.shape
        if D is not None:
            assert D.shape == (dim,)
        if dt_bias is not None:
            assert dt_bias.shape == (dim,)
        if h0 is not None:
            assert h0.shape == (batch, dim, N)
        if h0_scale is not None:
            assert h0 is not None and h0_scale.shape == h0.shape
        if rows is None:
            rows_arr = None
            lead = (batch, dim)
            nrows = batch * dim
        else:
            rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
            lead = (rows_arr.shape[0],)
            nrows = rows_arr.shape[0]
        y = np.empty(lead + (L,), np.float64)
        ys = np.empty(lead + (L,), np.float64)
        hs = np.empty(lead + (N,), np.float64)
        hss = np.empty(lead + (N,), np.float64)
        nt = nthreads or default_threads()
        rc = self.lib.ssm_ref_fwd(
            _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
            _ptr(h0), _ptr(h0_scale), batch, L, dim, N,
            None if rows_arr is None else rows_arr.ctypes.data_as(_ip), nrows,
            _ptr(y), _ptr(hs), _ptr(ys), _ptr(hss), nt)
        if rc != 0:
            raise RuntimeError(f"ssm_ref_fwd failed with code {rc}")
        return {"y": y, "y_scale": ys, "last_state": hs, "state_scale": hss}

    def step(self, state, x, delta, A, B, C, D=None, z=None, state_scale=None):
        """One decode step from ``state`` (``[batch, dim, dstate]``).

        ``delta`` is the pre-activation with any bias already added; the step
        applies softplus to it. ``x, delta, z``: ``[batch, dim]``; ``B, C``:
        ``[batch, dstate]``. Returns a dict with the new ``state`` and
        ``state_scale`` and the output ``y`` and ``y_scale`` (float64). The inputs
        are not modified.
        """
        h = _f64(state).copy()
        hs = _f64(state_scale).copy() if state_scale is not None else np.abs(h)
        x, delta, A, B, C, D, z = map(_f64, (x, delta, A, B, C, D, z))
        batch, dim, N = h.shape
        assert x.shape == (batch, dim) and delta.shape == (batch, dim)
        assert A.shape == (dim, N) and B.shape == (batch, N) and C.shape == (batch, N)
        y = np.empty((batch, dim), np.float64)
        ys = np.empty((batch, dim), np.float64)
        rc = self.lib.ssm_ref_step(_ptr(h), _ptr(hs), _ptr(x), _ptr(delta), _ptr(A), _ptr(B),
                                  _ptr(C), _ptr(D), _ptr(z), batch, dim, N, _ptr(y), _ptr(ys))
        if rc != 0:
            raise RuntimeError(f"ssm_ref_step failed with code {rc}")
        return {"y": y, "y_scale": ys, "state": h, "state_scale": hs}


_default: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle library: the built one, or the one named by the environment
    variable SELSCAN_ORACLE_LIB (the sanitizer test loads an instrumented
    build of the same source this way)."""
    global _default
    if _default is None:
        _default = Oracle(os.environ.get("SELSCAN_ORACLE_LIB") or None)
    return _default


def fwd(*args, **kw):
    """Forward through the built oracle; see ``Oracle.fwd``."""
    return default().fwd(*args, **kw)


def step(*args, **kw):
    """One decode step through the built oracle; see ``Oracle.step``."""
    return default().step(*args, **kw)


def bwd(*args, **kw):
    """Backward pass through the built oracle; see ``Oracle.bwd``."""
    return default().bwd(*args, **kw)


def ssd(*args, **kw):
    """Mamba-2 SSD layer through the built oracle; see ``Oracle.ssd``."""
    return default().ssd(*args, **kw)


def ssd_step(*args, **kw):
    return default().ssd_step(*args, **kw)


def conv1d(*args, **kw):
    """Causal depthwise conv + SiLU through the built oracle; see ``Oracle.conv1d``."""
    return default().conv1d(*args, **kw)


def conv1d_bwd(*args, **kw):
    """Gradients of the convolution; see ``Oracle.conv1d_bwd``."""
    return default().conv1d_bwd(*args, **kw)


def conv1d_step(*args, **kw):
    """One convolution decode step; see ``Oracle.conv1d_step``."""
    return default().conv1d_step(*args, **kw)


def scaled_error(got, ref, scale, floor: float = 1e-30) -> float:
    """max_i |got_i - ref_i| / max(scale_i, floor), NaN-aware.

    Positions where ``ref`` is NaN must be NaN in ``got`` too (else the error
    is infinite); they are excluded from the maximum. Infinite references must
    be matched exactly. The three arrays must have one shape: a comparison
    that broadcast a smaller result over a larger reference would check less
    than it claims.
    """
    got = _f64(got)
    ref = _f64(ref)
    scale = _f64(scale)
    if got.shape != ref.shape or scale.shape != ref.shape:
        raise ValueError(f"shape mismatch: got {got.shape}, ref {ref.shape}, scale {scale.shape}")
    nan_ref = np.isnan(ref)
    if np.any(np.isnan(got) != nan_ref):
        return float("inf")
    inf_ref = np.isinf(ref)
    if np.any(inf_ref):
        if np.any(got[inf_ref] != ref[inf_ref]):
            return float("inf")
    ok = ~(nan_ref | inf_ref)
    if not np.any(ok):
        return 0.0
    err = np.abs(got[ok] - ref[ok]) / np.maximum(np.abs(scale[ok]), floor)
    return float(np.max(err)) if err.size else 0.0
