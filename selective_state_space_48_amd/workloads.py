"""Seeded synthetic inputs for the selective scan, shared by the tests and the benchmark.

This module only draws random numbers and lays them out; it holds none of the
scan's arithmetic. Each tensor is drawn from its own counter-addressed stream
``numpy.random.default_rng([seed, tensor_id, batch_index])``, so any batch
slice can be regenerated on its own and every consumer sees identical values.

Value recipe (the workloads below are model-layer shapes from the pages'
discussion; no dataset is involved):

* ``x``, ``z``, ``B``, ``C`` ~ N(0, 1); ``delta_raw`` ~ N(0, 1).
* ``A[d, n] = -(n + 1)``: negative reals, one decay per (channel, state).
* ``dt_bias[d]`` is chosen so that softplus(dt_bias) is log-uniform in
  ``[delta_lo, delta_hi]``: the inverse map ``log(expm1(v))`` is part of this
  input recipe only.
* ``D`` is 1, or U[0.5, 1.5] where the workload says so.
* The short convolution in front of the scan: taps ``w[d, k]`` ~ N(0, 0.5^2),
  ``bias[d]`` ~ N(0, 0.1^2); its input is the workload's ``x``; the carried-in
  inputs ``x_prev`` [batch, dim, 3] ~ N(0, 1).
* For bfloat16 workloads every float input is rounded to bfloat16
  (round-to-nearest-even, by torch) before either side sees it; the arrays
  returned here hold those rounded values in float32, which represents them
  exactly.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Sequence

import numpy as np

# Stream ids, fixed so that every consumer draws the same values.
TID_X, TID_DELTA, TID_Z, TID_B, TID_C, TID_DT_BIAS, TID_D = 0, 1, 2, 3, 4, 5, 6
TID_PRE_X, TID_PRE_DELTA, TID_PRE_B = 7, 8, 9
TID_STEP0 = 10  # decode step s uses ids TID_STEP0 + s (sub-stream k = tensor)
TID_CONV_W, TID_CONV_BIAS, TID_CONV_PREV = 200, 201, 202
TID_CONV_STEP0 = 300  # convolution decode step s uses id TID_CONV_STEP0 + s
TID_SSD = 400          # SSD layer: ids TID_SSD + 0..6


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int  # tokens per forward call; 1 for decode steps
    dim: int  # d_inner, the number of channels
    dstate: int  # N
    dtype: str  # "f32" or "bf16": x, delta, z, B, C and y
    gate: bool  # y * silu(z)
    d_uniform: bool  # D ~ U[0.5, 1.5] instead of 1
    delta_lo: float
    delta_hi: float
    seed: int
    kind: str = "fwd"  # "fwd" or "step"
    steps: int = 0  # decode steps
    prefill: int = 0  # tokens run through a forward pass to build the decode state
    notes: str = field(default="", compare=False)

    @property
    def elements(self) -> int:
        """E = batch * seqlen * dim: the element count throughput is quoted in."""
        return self.batch * self.seqlen * self.dim

    @property
    def rows(self) -> int:
        return self.batch * self.dim


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_f32_b1_l256_d16", 1, 256, 16, 16, "f32", gate=False, d_uniform=False,
                 delta_lo=1e-3, delta_hi=1e-1, seed=0,
                 notes="small fp32 forward; z drawn but the gate is off"),
        Workload("m130m_f32_b8_l2048_d1536", 8, 2048, 1536, 16, "f32", gate=True,
                 d_uniform=False, delta_lo=1e-3, delta_hi=1e-1, seed=1,
                 notes="Mamba-130m-shaped layer, fp32, gate and D skip, last state"),
        Workload("m1p4b_bf16_b8_l2048_d4096", 8, 2048, 4096, 16, "bf16", gate=True,
                 d_uniform=True, delta_lo=1e-3, delta_hi=1e-1, seed=2,
                 notes="Mamba-1.4B-shaped layer, bf16 inputs/outputs, fp32 state"),
        Workload("long_f32_b1_l1048576_d128", 1, 1 << 20, 128, 16, "f32", gate=False,
                 d_uniform=False, delta_lo=1e-4, delta_hi=1e-2, seed=3,
                 notes="million-token sequence; step sizes small so the state carries far"),
        Workload("decode_bf16_b256_d5120", 256, 1, 5120, 16, "bf16", gate=True,
                 d_uniform=True, delta_lo=1e-3, delta_hi=1e-1, seed=4, kind="step",
                 steps=64, prefill=512,
                 notes="2.8B-shaped decode: 64 one-token steps from a 512-token prefill state"),
    ]
}

# The forward configuration the throughput figure is quoted on.
HEADLINE = "m1p4b_bf16_b8_l2048_d4096"
DECODE = "decode_bf16_b256_d5120"


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(w: Workload, **kw) -> Workload:
    """A copy with some sizes changed (same value recipe and seed)."""
    return replace(w, **kw)


def _rng(seed: int, tid: int, sub: int) -> np.random.Generator:
    return np.random.default_rng([seed, tid, sub])


def _round_bf16(a: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _maybe_bf16(w: Workload, a: np.ndarray) -> np.ndarray:
    return _round_bf16(a) if w.dtype == "bf16" else a


def params(w: Workload) -> Dict[str, np.ndarray]:
    """Per-channel parameters: A [dim, N], D [dim], dt_bias [dim] (float32)."""
    A = -np.broadcast_to(np.arange(1, w.dstate + 1, dtype=np.float32), (w.dim, w.dstate)).copy()
    lo, hi = np.log(w.delta_lo), np.log(w.delta_hi)
    v = np.exp(_rng(w.seed, TID_DT_BIAS, 0).uniform(lo, hi, size=w.dim))
    dt_bias = np.log(np.expm1(v)).astype(np.float32)
    if w.d_uniform:
        D = _rng(w.seed, TID_D, 0).uniform(0.5, 1.5, size=w.dim).astype(np.float32)
    else:
        D = np.ones(w.dim, np.float32)
    return {"A": A, "D": D, "dt_bias": dt_bias}


def fwd_inputs(w: Workload, batches: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Forward-pass inputs as float32 arrays (bf16-rounded values for bf16 workloads).

    ``batches`` selects batch indices (default all); the arrays then have that
    many leading entries. ``z`` is None when the workload's gate is off.
    """
    bs = list(range(w.batch)) if batches is None else list(batches)
    L, d, N = w.seqlen, w.dim, w.dstate

    def draw(tid, shape):
        out = np.empty((len(bs),) + shape, np.float32)
        for i, b in enumerate(bs):
            out[i] = _rng(w.seed, tid, b).standard_normal(shape, dtype=np.float32)
        return _maybe_bf16(w, out)

    out = {
        "x": draw(TID_X, (d, L)),
        "delta": draw(TID_DELTA, (d, L)),
        "z": draw(TID_Z, (d, L)) if w.gate else None,
        "B": draw(TID_B, (N, L)),
        "C": draw(TID_C, (N, L)),
    }
    out.update(params(w))
    return out


def prefill_inputs(w: Workload, b: int) -> Dict[str, np.ndarray]:
    """Inputs of the prefill that builds batch entry ``b`` of a decode state.

    ``w.prefill`` tokens of x, delta_raw and B for one batch entry, drawn like
    the forward workloads (bf16-rounded for bf16 workloads). Shapes:
    x, delta [1, dim, prefill]; B [1, N, prefill].
    """
    P, d, N = w.prefill, w.dim, w.dstate
    x = _rng(w.seed, TID_PRE_X, b).standard_normal((1, d, P), dtype=np.float32)
    dl = _rng(w.seed, TID_PRE_DELTA, b).standard_normal((1, d, P), dtype=np.float32)
    B = _rng(w.seed, TID_PRE_B, b).standard_normal((1, N, P), dtype=np.float32)
    return {"x": _maybe_bf16(w, x), "delta": _maybe_bf16(w, dl), "B": _maybe_bf16(w, B)}


def step_inputs(w: Workload, s: int) -> Dict[str, np.ndarray]:
    """Inputs of decode step ``s``: x, delta (pre-activation, bias included), z
    as [batch, dim]; B, C as [batch, N].

    The step takes delta with the channel bias already added, so delta here is
    delta_raw + dt_bias in float32, then rounded for bf16 workloads.
    """
    bt, d, N = w.batch, w.dim, w.dstate
    tid = TID_STEP0 + s
    x = _rng(w.seed, tid, 0).standard_normal((bt, d), dtype=np.float32)
    draw_delta = _rng(w.seed, tid, 1).standard_normal((bt, d), dtype=np.float32)
    z = _rng(w.seed, tid, 2).standard_normal((bt, d), dtype=np.float32)
    B = _rng(w.seed, tid, 3).standard_normal((bt, N), dtype=np.float32)
    C = _rng(w.seed, tid, 4).standard_normal((bt, N), dtype=np.float32)
    delta = draw_delta + params(w)["dt_bias"][None, :]
    return {
        "x": _maybe_bf16(w, x),
        "delta": _maybe_bf16(w, delta.astype(np.float32)),
        "z": _maybe_bf16(w, z) if w.gate else None,
        "B": _maybe_bf16(w, B),
        "C": _maybe_bf16(w, C),
    }


def random_state(w: Workload, scale: float = 0.1) -> np.ndarray:
    """A synthetic decode state [batch, dim, N] ~ N(0, scale^2) (for timing only)."""
    out = np.empty((w.batch, w.dim, w.dstate), np.float32)
    for b in range(w.batch):
        out[b] = _rng(w.seed, TID_PRE_X + 100, b).standard_normal(
            (w.dim, w.dstate), dtype=np.float32) * np.float32(scale)
    return out


def conv_inputs(w: Workload, batches: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Inputs of the causal convolution over the workload's sequence: x [b, dim, L]
    (the forward's x stream), taps w [dim, 4], bias [dim] and x_prev [b, dim, 3]
    (bf16-rounded values for bf16 workloads; taps and bias are fp32)."""
    bs = list(range(w.batch)) if batches is None else list(batches)
    d, L = w.dim, w.seqlen
    x = np.empty((len(bs), d, L), np.float32)
    prev = np.empty((len(bs), d, 3), np.float32)
    for i, b in enumerate(bs):
        x[i] = _rng(w.seed, TID_X, b).standard_normal((d, L), dtype=np.float32)
        prev[i] = _rng(w.seed, TID_CONV_PREV, b).standard_normal((d, 3), dtype=np.float32)
    out = {"x": _maybe_bf16(w, x), "x_prev": _maybe_bf16(w, prev)}
    out.update(conv_params(w))
    return out


def conv_params(w: Workload) -> Dict[str, np.ndarray]:
    """The convolution's taps w [dim, 4] ~ N(0, 0.5^2) and bias [dim] ~ N(0, 0.1^2)
    (float32; the streams ``conv_inputs`` uses)."""
    return {
        "w": (_rng(w.seed, TID_CONV_W, 0).standard_normal((w.dim, 4), dtype=np.float32) * 0.5),
        "bias": (_rng(w.seed, TID_CONV_BIAS, 0).standard_normal(w.dim, dtype=np.float32) * 0.1),
    }


def conv_step_inputs(w: Workload, s: int) -> np.ndarray:
    """The input token of convolution decode step ``s``: x [batch, dim]."""
    x = _rng(w.seed, TID_CONV_STEP0 + s, 0).standard_normal((w.batch, w.dim), dtype=np.float32)
    return _maybe_bf16(w, x)


# Mamba-2 SSD layer: a 1.3B-shaped layer (d_inner 4096 = 64 heads of 64
# channels, state 128, one B/C group), bf16.
SSD_HEADLINE = dict(batch=8, seqlen=2048, heads=64, headdim=64, dstate=128, seed=5)
# Decode of a Mamba-2-2.7B-shaped layer (d_inner 5120: 80 heads of 64, state
# 128), 256 sequences at once: an fp32 state of 671 MB read and written per step.
SSD_DECODE = dict(batch=256, heads=80, headdim=64, dstate=128, seed=6)


def ssd_inputs(batch: int, seqlen: int, heads: int, headdim: int, dstate: int, seed: int,
               batches: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Inputs of the SSD layer (bf16-rounded values as float32): x [b, L, H, P],
    delta_raw [b, L, H], B, C [b, L, N] ~ N(0, 1); per head A = -U[1, 16],
    dt_bias with softplus(dt_bias) log-uniform in [1e-3, 1e-1], D ~ U[0.5, 1.5]."""
    bs = list(range(batch)) if batches is None else list(batches)

    def draw(k, shape):
        out = np.empty((len(bs),) + shape, np.float32)
        for i, b in enumerate(bs):
            out[i] = _rng(seed, TID_SSD + k, b).standard_normal(shape, dtype=np.float32)
        return _round_bf16(out)

    out = {
        "x": draw(0, (seqlen, heads, headdim)),
        "delta": draw(1, (seqlen, heads)),
        "B": draw(2, (seqlen, dstate)),
        "C": draw(3, (seqlen, dstate)),
    }
    out.update(ssd_params(heads, seed))
    return out


def ssd_params(heads: int, seed: int) -> Dict[str, np.ndarray]:
    """Per-head parameters of the SSD layer (the streams ``ssd_inputs`` uses):
    A = -U[1, 16], dt_bias with softplus(dt_bias) log-uniform in [1e-3, 1e-1],
    D ~ U[0.5, 1.5] (float32)."""
    v = np.exp(_rng(seed, TID_SSD + 5, 0).uniform(np.log(1e-3), np.log(1e-1), size=heads))
    return {
        "A": -_rng(seed, TID_SSD + 4, 0).uniform(1.0, 16.0, size=heads).astype(np.float32),
        "dt_bias": np.log(np.expm1(v)).astype(np.float32),
        "D": _rng(seed, TID_SSD + 6, 0).uniform(0.5, 1.5, size=heads).astype(np.float32),
    }


def device_normal(shape, seed: int, tid: int, device, dtype):
    """N(0, 1) values drawn directly on the device by torch's generator, seeded
    from (seed, tid), then rounded to ``dtype``: for tensors too large to draw
    on the host (billions of elements). These values are not those of the
    host streams above; a comparison reads both sides' inputs from the device
    tensor."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(tid))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return t if dtype == torch.float32 else t.to(dtype)
