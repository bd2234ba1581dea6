"""Throughput of the selective scan on one MI355X.

A step is one selscan_fwd call on the Mamba-1.4B-shaped layer (batch 8,
L 2048, d_inner 4096, N 16; bf16 x/delta/z/B/C/y, fp32 state and arithmetic)
with inputs resident in HBM. The line also reports the decode step on the
2.8B-shaped state (batch 256, d_inner 5120, N 16) in microseconds, the other
forward workloads, and the fp64 CPU oracle timed on a bounded sample of the
same workload.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-extras]
                       [--no-cpu-baseline]
                       [--only fwd|decode|long|m130m|conv|bwd|ssd|ragged|copy]
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X published HBM3E bandwidth
# VALU issue-slot peak: 256 CUs x 64 lanes (4 SIMDs x 16) x 2.4 GHz, one
# non-packed fp32 VALU instruction per lane-slot. (The published fp32 vector
# rate, 157.3 TFLOP/s, is this times 4: a packed FMA is 4 flops per slot.)
SLOT_PEAK = 256 * 64 * 2.4e9
TRANS_SLOTS = 2            # v_exp/v_log/v_rcp occupy a wave twice as long as an FMA (measured)


# HBM traffic of one output-pass launch on the headline workload: rocprofv3
# --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what the
# same counter reads for a plain copy kernel of known size (torch's copy of
# 1 GiB: FETCH_SIZE reads half the bytes moved, WRITE_SIZE all of them; the
# profiles/ summary also lists the factors of copies with the scan's row
# access pattern, for comparison). It is valid only for the device code it
# was taken on, identified by the sha256 of the forward kernel's sources: the
# part of fwd.hip before the B/C pack (the kernels and everything they use;
# the host launch code comes after it) and common.hpp.
TRAFFIC = {"sources_sha256": "61fd7310dfb1d22dd75437b492ba3641f84e99afa98e4c9a4961287ffb5116c2",
           "fetch_kib": 205776.4, "fetch_factor": 2.0, "write_kib": 157736.9, "write_factor": 1.0}


def kernel_sources_sha256():
    import hashlib

    h = hashlib.sha256()
    for f in ("fwd.hip", "common.hpp"):
        with open(os.path.join(ROOT, "selective_state_space_48_amd", "csrc", f), "rb") as fh:
            text = fh.read()
        if f == "fwd.hip":
            text = text[:text.index(b"// Pack B and C")]
        h.update(text)
    return h.hexdigest()


def measured_traffic():
    """Counted HBM bytes per launch, or None when the counters were taken on
    other device code (or never)."""
    if TRAFFIC is None or TRAFFIC["sources_sha256"] != kernel_sources_sha256():
        return None
    return int(TRAFFIC["fetch_kib"] * 1024 * TRAFFIC["fetch_factor"]
               + TRAFFIC["write_kib"] * 1024 * TRAFFIC["write_factor"])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w):
    """HBM bytes one forward call must move: every input read once, y and the
    final state written once (B and C re-reads by other row blocks hit cache)."""
    es = 2 if w.dtype == "bf16" else 4
    E = w.batch * w.seqlen * w.dim
    n_seq = 4 if w.gate else 3                      # x, delta, (z), y
    bc = 2 * w.batch * w.dstate * w.seqlen * es      # B, C
    params = w.dim * w.dstate * 4 + 2 * w.dim * 4    # A, D, dt_bias
    state = w.batch * w.dim * w.dstate * 4           # last_state
    return n_seq * E * es + bc + params + state


def step_bytes(w):
    """HBM bytes of one decode step: the fp32 state read and written, the
    per-row x, delta, z read and y written, B, C, A, D read."""
    es = 2 if w.dtype == "bf16" else 4
    rows = w.batch * w.dim
    return 2 * rows * w.dstate * 4 + 4 * rows * es + 2 * w.batch * w.dstate * es \
        + w.dim * w.dstate * 4 + w.dim * 4


def method_slots(w):
    """VALU issue slots (lane-instructions, a transcendental = TRANS_SLOTS) the
    method needs per forward call, at its minimum:
    per (token, state): l*A, w*B, state FMA, readout FMA + one exp;
    per token: softplus (add bias, exp, add, log), delta*x, D*x FMA,
    silu (exp, add, reciprocal, multiply), gate multiply."""
    E = w.batch * w.seqlen * w.dim
    per_tn = 4 + TRANS_SLOTS
    per_tok = 6 + 4 * TRANS_SLOTS
    return E * (per_tn * w.dstate + per_tok)


def device_inputs(w, torch, dev, inp=None):
    from selective_state_space_48_amd import workloads as W

    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    inp = W.fwd_inputs(w) if inp is None else inp

    def t(a, dt=torch.float32):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)

    return dict(x=t(inp["x"], td), delta=t(inp["delta"], td), z=t(inp["z"], td), A=t(inp["A"]),
                B=t(inp["B"], td), C=t(inp["C"], td), D=t(inp["D"]), dt_bias=t(inp["dt_bias"]))


def time_fwd(w, steps, warmup, torch, dev, inp=None, distribution=False):
    from selective_state_space_48_amd import selscan

    d = device_inputs(w, torch, dev, inp)
    y = torch.empty_like(d["x"])
    hs = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)

    def run():
        selscan.fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                    dt_bias=d["dt_bias"], y=y, last_state=hs)

    for _ in range(warmup):
        run()
    stream = torch.cuda.current_stream(dev)   # the stream selscan launches on
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # The library records its own HIP events on the same stream around each
    # output-pass kernel (the kernel that writes y), for the per-kernel time.
    selscan.timing_start(steps)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    k_ms, k_n = selscan.timing_stop()
    assert k_n == steps, (k_n, steps)
    ms = e0.elapsed_time(e1) / steps
    dist = per_call_distribution(run, torch, dev) if distribution else None
    del d, y, hs
    return ms, wall, k_ms / k_n, dist


def _pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]


def per_call_distribution(run, torch, dev, n=20, scratch_mb=512):
    """Per-call times (µs) of ``n`` calls, each bracketed by its own events:
    warm (right after an untimed call); ``cold``: with the caches flushed,
    i.e. a 512 MB scratch buffer written and then a second 512 MB buffer read,
    so that the 256 MB last-level cache and the L2s hold neither the call's
    data nor dirty lines waiting to be written back (the write-back of the
    first sweep happens during the second, before the call); and
    ``cold_dirty``: right after the write sweep alone, where the call's misses
    also evict the sweep's dirty lines and pay for writing them back."""
    stream = torch.cuda.current_stream(dev)
    scratch = torch.empty(scratch_mb << 18, dtype=torch.float32, device=dev)
    scratch_r = torch.ones(scratch_mb << 18, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    out = {}
    for mode in ("warm", "cold", "cold_dirty"):
        ts = []
        for i in range(n):
            torch.cuda.synchronize(dev)
            # The timed call is queued behind other work (a call, or the
            # sweeps), so the events measure its execution, not the launch
            # latency of an idle GPU.
            if mode == "warm":
                run()
            else:
                scratch.fill_(float(i))
                if mode == "cold":
                    torch.sum(scratch_r, dim=0, out=sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run()
            b.record(stream)
            torch.cuda.synchronize(dev)
            ts.append(a.elapsed_time(b) * 1e3)
        out[mode] = {"p10_us": round(_pct(ts, 0.1), 2), "p50_us": round(_pct(ts, 0.5), 2),
                     "p90_us": round(_pct(ts, 0.9), 2)}
    del scratch, scratch_r, sink
    return out


def time_decode(w, steps, warmup, torch, dev):
    from selective_state_space_48_amd import selscan
    from selective_state_space_48_amd import workloads as W

    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    p = W.params(w)

    def t(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)

    state = t(W.random_state(w))
    A, D = t(p["A"]), t(p["D"])
    ins = []
    for s in range(w.steps):
        si = W.step_inputs(w, s)
        ins.append((t(si["x"], td), t(si["delta"], td), t(si["B"], td), t(si["C"], td),
                    t(si["z"], td)))
    y = torch.empty((w.batch, w.dim), dtype=td, device=dev)
    for i in range(warmup):
        x, dl, B, C, z = ins[i % len(ins)]
        selscan.step(state, x, dl, A, B, C, D=D, z=z, y=y)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        x, dl, B, C, z = ins[i % len(ins)]
        selscan.step(state, x, dl, A, B, C, D=D, z=z, y=y)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    back_to_back = e0.elapsed_time(e1) / steps
    # again with the library's events around each step kernel
    selscan.timing_start(steps)
    for i in range(steps):
        x, dl, B, C, z = ins[i % len(ins)]
        selscan.step(state, x, dl, A, B, C, D=D, z=z, y=y)
    k_ms, k_n = selscan.timing_stop()
    assert k_n == steps, (k_n, steps)
    # each of the 64 distinct steps alone, warm and after evicting the caches
    it = iter(range(10 ** 9))

    def one():
        i = next(it)
        x, dl, B, C, z = ins[i % len(ins)]
        selscan.step(state, x, dl, A, B, C, D=D, z=z, y=y)

    dist = per_call_distribution(one, torch, dev, n=len(ins))
    return back_to_back, k_ms / k_n, dist


def time_block_decode(w, torch, dev, per_graph=16, replays=16):
    """The Mamba block's decode step on the decode shape, two ways: the
    convolution's step then the scan's (two launches per token), and the
    scan's step with the convolution fused in front (one). Each back to back
    from Python, and captured as a HIP graph of ``per_graph`` consecutive
    tokens (distinct inputs, the states updated in place) replayed ``replays``
    times; the gap between the two is the host's cost of the launches."""
    from selective_state_space_48_amd import selscan
    from selective_state_space_48_amd import workloads as W

    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    p = W.params(w)

    def t(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)

    state = t(W.random_state(w))
    A, D = t(p["A"]), t(p["D"])
    c = W.conv_inputs(W.scaled(w, seqlen=1))
    cst, cw, cb = t(c["x_prev"]), t(c["w"]), t(c["bias"])
    ins = []
    for s in range(per_graph):
        si = W.step_inputs(w, s)
        ins.append((t(si["x"], td), t(si["delta"], td), t(si["B"], td), t(si["C"], td),
                    t(si["z"], td)))
    xa = torch.empty((w.batch, w.dim), dtype=td, device=dev)
    ys = [torch.empty_like(xa) for _ in range(per_graph)]

    def two_calls():
        for i, (x, dl, B, C, z) in enumerate(ins):
            selscan.conv1d_step(cst, x, cw, cb, out=xa)
            selscan.step(state, xa, dl, A, B, C, D=D, z=z, y=ys[i])

    def fused():
        for i, (x, dl, B, C, z) in enumerate(ins):
            selscan.step(state, x, dl, A, B, C, D=D, z=z, y=ys[i], conv_w=cw, conv_b=cb, conv_state=cst)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def per_token(run):
        for _ in range(2):
            run()
        torch.cuda.synchronize(dev)
        e0.record()
        for _ in range(replays):
            run()
        e1.record()
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) * 1e3 / (replays * per_graph)

    res = {"workload": f"block decode step on {w.name}", "tokens_per_graph": per_graph}
    for name, run in (("two_calls", two_calls), ("fused", fused)):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        res[f"us_per_token_{name}_eager"] = round(per_token(run), 2)
        res[f"us_per_token_{name}_graph"] = round(per_token(graph.replay), 2)
    # fused: the scan's step bytes with the raw input in place of the convolved
    # one, plus the convolution's state (read, written), taps and bias
    nbytes = step_bytes(w) + w.rows * 24 + w.dim * 20
    us = res["us_per_token_fused_graph"]
    res.update({"achieved_GBps_fused_graph": round(nbytes / (us * 1e-6) / 1e9, 1),
                "frac_hbm_fused_graph": round(nbytes / (us * 1e-6) / HBM_PEAK, 4),
                "bytes_per_token_fused": nbytes})
    return res


def time_ragged(torch, dev, reps=5):
    """Rows whose length is not a multiple of the 16-byte vector: the headline
    shape at L 2047 against L 2048 (bf16; synthetic N(0, 1) inputs, the step
    size centred at -1), for the forward (plain and with the convolution
    fused), the backward, and the convolution and its gradients."""
    from selective_state_space_48_amd import selscan

    g = torch.Generator(device=dev)
    g.manual_seed(7)
    out = {}
    b, d, dt = 8, 4096, torch.bfloat16
    A = -torch.arange(1, 17, device=dev, dtype=torch.float32).repeat(d, 1).contiguous()
    D = torch.ones(d, device=dev)
    bias = torch.full((d,), -4.0, device=dev)
    cw = 0.5 * torch.randn((d, 4), device=dev, generator=g)
    cb = 0.1 * torch.randn((d,), device=dev, generator=g)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def per_call(f):
        for _ in range(2):
            f()
        torch.cuda.synchronize(dev)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize(dev)
        return round(e0.elapsed_time(e1) * 1e3 / reps, 1)

    for L in (2048, 2047):
        r = lambda *sh: torch.randn(*sh, device=dev, generator=g)
        x, z, dy = r(b, d, L).to(dt), r(b, d, L).to(dt), r(b, d, L).to(dt)
        dl = (0.5 * r(b, d, L) - 1.0).to(dt)
        B, C = r(b, 16, L).to(dt), r(b, 16, L).to(dt)
        y = torch.empty_like(x)
        res = {
            "fwd_us": per_call(lambda: selscan.fwd(x, dl, A, B, C, D=D, z=z, dt_bias=bias, y=y)),
            "fwd_fused_conv_us": per_call(lambda: selscan.fwd(x, dl, A, B, C, D=D, z=z, dt_bias=bias, y=y,
                                                              conv_w=cw, conv_b=cb)),
            "bwd_us": per_call(lambda: selscan.bwd(x, dl, A, B, C, D=D, z=z, dt_bias=bias, dy=dy)),
            "conv1d_us": per_call(lambda: selscan.conv1d(x, cw, cb, None, out=y)),
            "conv1d_bwd_us": per_call(lambda: selscan.conv1d_bwd(x, cw, cb, None, dout=dy)),
        }
        out[f"L{L}"] = res
        del x, z, dy, dl, B, C, y
    out["workload"] = "m1p4b_bf16_b8_d4096 at L 2048 and 2047 (rows off a 16-byte boundary)"
    return out


def time_bwd(torch, dev, reps=5):
    """The backward pass on the headline shape (bf16, gate, D, dt_bias): all
    eight gradients for a synthetic dy, whole call (checkpoint pass, reverse
    pass, fixed-order reductions, workspace on the stream). Also timed: the
    forward that stores checkpoints and the backward that takes them (no
    checkpoint pass), i.e. a training step's two calls each way."""
    from selective_state_space_48_amd import selscan
    from selective_state_space_48_amd import workloads as W

    w = W.get(W.HEADLINE)
    d = device_inputs(w, torch, dev)
    dy = torch.randn(d["x"].shape, generator=torch.Generator().manual_seed(8)).to(dev).to(torch.bfloat16)
    y = torch.empty_like(d["x"])
    ck = torch.empty(selscan.ckpt_shape(w.batch, w.dim, w.seqlen), dtype=torch.float32, device=dev)
    args = (d["x"], d["delta"], d["A"], d["B"], d["C"])
    kw = dict(D=d["D"], z=d["z"], dt_bias=d["dt_bias"])

    def timed(run):
        for _ in range(2):
            run()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / reps

    ms = timed(lambda: selscan.bwd(*args, **kw, dy=dy))
    fwd_ms = timed(lambda: selscan.fwd(*args, **kw, y=y))
    fwd_ck_ms = timed(lambda: selscan.fwd(*args, **kw, y=y, ckpt=ck))
    bwd_ck_ms = timed(lambda: selscan.bwd(*args, **kw, dy=dy, ckpt=ck))
    # algorithmic bytes: read x, delta, z, dy, B, C; write dx, ddelta, dz, dB, dC
    nbytes = 7 * w.elements * 2 + 4 * w.batch * w.dstate * w.seqlen * 2
    del d, dy, y, ck
    return {"workload": f"backward on {w.name}", "ms_per_call": round(ms, 4),
            "Gelem_per_s": round(w.elements / (ms * 1e-3) / 1e9, 2),
            "ratio_to_forward": round(ms / fwd_ms, 2), "algorithmic_bytes": nbytes,
            "frac_hbm": round(nbytes / (ms * 1e-3) / HBM_PEAK, 4),
            "forward_ms": round(fwd_ms, 4),
            "forward_storing_checkpoints_ms": round(fwd_ck_ms, 4),
            "backward_from_checkpoints_ms": round(bwd_ck_ms, 4),
            "training_step_ms": {"recompute": round(fwd_ms + ms, 4),
                                 "checkpoints": round(fwd_ck_ms + bwd_ck_ms, 4)}}


def time_bwd_long(torch, dev, reps=3):
    """The backward pass on the long-memory workload (fp32, batch 1, L 2^20,
    d_inner 128, no gate): two 64-row blocks, so the sweep is cut into
    sequence segments (automatic choice); whole call."""
    from selective_state_space_48_amd import selscan
    from selective_state_space_48_amd import workloads as W

    w = W.get("long_f32_b1_l1048576_d128")
    d = device_inputs(w, torch, dev)
    dy = torch.randn(d["x"].shape, generator=torch.Generator().manual_seed(9)).to(dev)
    run = lambda: selscan.bwd(d["x"], d["delta"], d["A"], d["B"], d["C"], D=d["D"], z=d.get("z"),
                              dt_bias=d["dt_bias"], dy=dy)
    run()
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / reps
    # read x, delta, dy, B, C; write dx, ddelta, dB, dC (fp32)
    nbytes = 4 * w.elements * 4 + 4 * w.batch * w.dstate * w.seqlen * 4
    del d, dy
    return {"workload": f"backward on {w.name}", "ms_per_call": round(ms, 4),
            "Gelem_per_s": round(w.elements / (ms * 1e-3) / 1e9, 2),
            "algorithmic_bytes": nbytes, "frac_hbm": round(nbytes / (ms * 1e-3) / HBM_PEAK, 4)}


def time_ssd(torch, dev, reps=10):
    """Mamba-2 SSD layer, batch 8, L 2048, 64 heads of 64, state 128, bf16:
    whole call (one fused kernel: per (batch, head) the 64-token chunks in
    order, state on chip). Roofline terms: the chunked algorithm's
    matrix-product flops (64-token chunks) against the 2.5 PFLOP/s bf16 peak,
    and the algorithmic bytes (inputs once, y and the final state once)
    against 8 TB/s."""
    from selective_state_space_48_amd import selscan
    from selective_state_space_48_amd import workloads as W

    s = W.SSD_HEADLINE
    p = W.ssd_inputs(s["batch"], s["seqlen"], s["heads"], s["headdim"], s["dstate"], s["seed"])

    def t(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)

    bf = torch.bfloat16
    x, dl, B, C = t(p["x"], bf), t(p["delta"], bf), t(p["B"], bf), t(p["C"], bf)
    A, D, bias = t(p["A"]), t(p["D"]), t(p["dt_bias"])
    y = torch.empty_like(x)
    hs = torch.empty((s["batch"], s["heads"], s["dstate"], s["headdim"]), device=dev)
    run = lambda: selscan.ssd_fwd(x, dl, A, B, C, D=D, dt_bias=bias, y=y, last_state=hs)
    for _ in range(3):
        run()
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize(dev)
    us = e0.elapsed_time(e1) / reps * 1e3
    Bb, L, H, P, N = s["batch"], s["seqlen"], s["heads"], s["headdim"], s["dstate"]
    Q = 64
    chunks = Bb * H * ((L + Q - 1) // Q)
    flops = chunks * 2 * Q * (P * N + Q * N + Q * P + N * P)
    nbytes = 2 * (2 * Bb * L * H * P) + 2 * Bb * L * H + 2 * 2 * Bb * L * N + 4 * Bb * H * N * P
    E = Bb * L * H * P
    return {"workload": f"ssd_bf16_b{Bb}_l{L}_h{H}_p{P}_n{N}", "us_per_call": round(us, 2),
            "Gelem_per_s": round(E / (us * 1e-6) / 1e9, 1),
            "mfma_TFLOPs": round(flops / (us * 1e-6) / 1e12, 2), "frac_mfma_peak": round(flops / (us * 1e-6) / 2.5e15, 4),
            "algorithmic_bytes": nbytes, "frac_hbm": round(nbytes / (us * 1e-6) / HBM_PEAK, 4)}


def time_ssd_decode(torch, dev, steps=8):
    """One decode step of the SSD layer, 256 sequences, 80 heads of 64, state
    128 (bf16 x/B/C/y, fp32 state in place): per step the state is read and
    written once. Steps over distinct tokens, back to back."""
    from selective_state_space_48_amd import selscan
    from selective_state_space_48_amd import workloads as W

    s = W.SSD_DECODE
    Bb, H, P, N = s["batch"], s["heads"], s["headdim"], s["dstate"]
    p = W.ssd_inputs(Bb, steps, H, P, N, s["seed"])

    def t(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)

    bf = torch.bfloat16
    toks = [(t(p["x"][:, i], bf), t(p["delta"][:, i], bf), t(p["B"][:, i], bf), t(p["C"][:, i], bf))
            for i in range(steps)]
    A, D, bias = t(p["A"]), t(p["D"]), t(p["dt_bias"])
    state = torch.zeros((Bb, H, N, P), dtype=torch.float32, device=dev)
    y = torch.empty((Bb, H, P), dtype=bf, device=dev)
    run = lambda i: selscan.ssd_step(state, *toks[i][:2], A, *toks[i][2:], D=D, dt_bias=bias, y=y)
    for i in range(steps):
        run(i)
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(4):
        for i in range(steps):
            run(i)
    e1.record()
    torch.cuda.synchronize(dev)
    us = e0.elapsed_time(e1) / (4 * steps) * 1e3
    nbytes = 2 * 4 * Bb * H * N * P + 2 * 2 * Bb * H * P + 2 * Bb * H + 2 * 2 * Bb * N
    del toks, state
    return {"workload": f"ssd_decode_bf16_b{Bb}_h{H}_p{P}_n{N}", "us_per_step": round(us, 2),
            "bytes_per_step": nbytes, "achieved_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(nbytes / (us * 1e-6) / HBM_PEAK, 4)}


def time_fused_conv(torch, dev, reps=10):
    """The block's convolution + SiLU and the scan on the headline shape, as two
    calls (conv1d writes its output, the scan reads it) and as one (the
    convolution formed in the scan's per-token phase)."""
    from selective_state_space_48_amd import selscan
    from selective_state_space_48_amd import workloads as W

    w = W.get(W.HEADLINE)
    d = device_inputs(w, torch, dev)
    c = W.conv_inputs(w)
    cw = torch.from_numpy(c["w"]).to(dev)
    cb = torch.from_numpy(c["bias"]).to(dev)
    y = torch.empty_like(d["x"])
    xc = torch.empty_like(d["x"])
    kw = dict(D=d["D"], z=d["z"], dt_bias=d["dt_bias"], y=y)

    def timed(run):
        for _ in range(2):
            run()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / reps * 1e3

    def separate():
        selscan.conv1d(d["x"], cw, cb, out=xc, return_x_last=False)
        selscan.fwd(xc, d["delta"], d["A"], d["B"], d["C"], **kw)

    sep = timed(separate)
    fused = timed(lambda: selscan.fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], **kw,
                                      conv_w=cw, conv_b=cb))
    scan = timed(lambda: selscan.fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], **kw))
    del d, y, xc
    return {"workload": f"conv1d + scan on {w.name}", "separate_us": round(sep, 2),
            "fused_us": round(fused, 2), "scan_alone_us": round(scan, 2),
            "speedup": round(sep / fused, 3),
            "fused_Gelem_per_s": round(w.elements / (fused * 1e-6) / 1e9, 1)}


def time_conv(torch, dev, reps=20):
    """The causal conv1d (width 4) + SiLU over the headline-shaped input
    (bf16, x_last returned), and its decode step on the decode shape. Kernel
    times from the library's own events are not taken here: the whole call is
    one kernel (plus a one-thread-per-row x_last kernel)."""
    from selective_state_space_48_amd import selscan
    from selective_state_space_48_amd import workloads as W

    def t(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)

    out = {}
    w = W.get(W.HEADLINE)
    p = W.conv_inputs(w)
    x, cw, cb = t(p["x"], torch.bfloat16), t(p["w"]), t(p["bias"])
    y = torch.empty_like(x)
    last = torch.empty((w.batch, w.dim, 3), dtype=torch.float32, device=dev)
    run = lambda: selscan.conv1d(x, cw, cb, None, out=y, x_last=last)
    for _ in range(3):
        run()
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize(dev)
    us = e0.elapsed_time(e1) / reps * 1e3
    nbytes = 2 * w.elements * 2 + w.rows * 12 + w.dim * 20
    out["conv1d"] = {"workload": f"conv1d on {w.name}", "us_per_call": round(us, 2),
                     "Gelem_per_s": round(w.elements / (us * 1e-6) / 1e9, 1),
                     "achieved_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "frac_hbm": round(nbytes / (us * 1e-6) / HBM_PEAK, 4), "bytes_per_call": nbytes}
    # the gradients of the same convolution: read x and dout, write dx
    dout = torch.randn(x.shape, generator=torch.Generator().manual_seed(3)).to(dev).to(torch.bfloat16)
    runb = lambda: selscan.conv1d_bwd(x, cw, cb, None, dout=dout)
    for _ in range(3):
        runb()
    torch.cuda.synchronize(dev)
    e0.record()
    for _ in range(reps):
        runb()
    e1.record()
    torch.cuda.synchronize(dev)
    us = e0.elapsed_time(e1) / reps * 1e3
    nbytes = 3 * w.elements * 2 + w.rows * 12 + w.dim * 40
    out["conv1d_bwd"] = {"workload": f"conv1d gradients on {w.name}", "us_per_call": round(us, 2),
                         "achieved_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                         "frac_hbm": round(nbytes / (us * 1e-6) / HBM_PEAK, 4), "bytes_per_call": nbytes}
    del x, y, last, dout
    wd = W.get(W.DECODE)
    pd = W.conv_inputs(W.scaled(wd, seqlen=1))
    st = t(pd["x_prev"])
    cw, cb = t(pd["w"]), t(pd["bias"])
    xs = [t(W.conv_step_inputs(wd, s), torch.bfloat16) for s in range(16)]
    yo = torch.empty_like(xs[0])
    for i in range(4):
        selscan.conv1d_step(st, xs[i], cw, cb, out=yo)
    torch.cuda.synchronize(dev)
    e0.record()
    for i in range(256):
        selscan.conv1d_step(st, xs[i % 16], cw, cb, out=yo)
    e1.record()
    torch.cuda.synchronize(dev)
    us = e0.elapsed_time(e1) / 256 * 1e3
    nbytes = wd.rows * (12 + 12 + 2 + 2) + wd.dim * 20
    out["conv1d_step"] = {"workload": f"conv1d step on {wd.name}", "us_per_step": round(us, 2),
                          "achieved_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                          "frac_hbm": round(nbytes / (us * 1e-6) / HBM_PEAK, 4),
                          "bytes_per_step": nbytes}
    log(f"[bench] conv1d: {out['conv1d']}; gradients: {out['conv1d_bwd']}; step: {out['conv1d_step']}")
    return out


def measured_ceilings(torch, dev):
    """Measured ceilings on this GPU: the device-copy rate (torch copy of
    1 GiB each way, bytes read + written per second) and the rate of the
    forward kernel's inner-loop instruction mix alone (VALU slots per second,
    8 waves per SIMD, from the calibration library)."""
    import ctypes

    from selective_state_space_48_amd import build as Bld

    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize(dev)
    copy_bps = 2 * n * 4 * 5 / (e0.elapsed_time(e1) * 1e-3)
    del src, dst
    lib = ctypes.CDLL(Bld.CALIB_LIB)
    lib.selscan_calib_scan_mix.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_void_p]
    blocks, nsub = 256 * 8, 512
    rec = torch.zeros(8192, dtype=torch.float32, device=dev)
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    best = None
    for _ in range(4):
        e0.record()
        assert lib.selscan_calib_scan_mix(rec.data_ptr(), out.data_ptr(), blocks, nsub, stream) == 0
        e1.record()
        torch.cuda.synchronize(dev)
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    slots = blocks * 256 * nsub * 16 * (4 + TRANS_SLOTS)
    return {"copy_GBps": round(copy_bps / 1e9, 1), "scan_mix_T_slot_per_s": round(slots / (best * 1e-3) / 1e12, 3)}


def cpu_baseline(w, inp, reps=3):
    """The oracle as it stands, on the whole headline workload (every row,
    every token; about 1e9 (token, state) updates in float64), all host
    threads, repeated ``reps`` times; plus one thread on one batch entry."""
    import oracle

    nt = oracle.default_threads()
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                   dt_bias=inp["dt_bias"], nthreads=nt)
    dt = (time.perf_counter() - t0) / reps
    # one thread, on the first 1/8 of the rows
    nrows = w.rows // 8
    t0 = time.perf_counter()
    sl = slice(0, max(1, nrows // w.dim))
    oracle.fwd(inp["x"][sl], inp["delta"][sl], inp["A"], inp["B"][sl], inp["C"][sl], D=inp["D"],
               z=inp["z"][sl], dt_bias=inp["dt_bias"], nthreads=1)
    dt1 = time.perf_counter() - t0
    e1 = (sl.stop - sl.start) * w.dim * w.seqlen
    return {"value": round(w.elements / dt / 1e9, 6), "unit": "Gelem/s", "cores": nt,
            "kind": "oracle",
            "sample": f"the whole {w.name} workload ({w.rows} rows x {w.seqlen} tokens), fp64, "
                      f"{reps} runs, {dt:.2f} s wall each on {nt} threads",
            "single_thread": {"value": round(e1 / dt1 / 1e9, 6), "unit": "Gelem/s",
                              "sample": f"{sl.stop - sl.start} batch entries ({e1:,} elements), "
                                        f"{dt1:.2f} s on 1 thread"}}


def cpu_baseline_per_config():
    """The oracle timed on every workload of the benchmark's configuration
    list, all host threads and one: the forward workloads over all their
    rows (Gelem/s), the decode workload as the 512-token prefill of all 256
    sequences (timed on its own) and one step over every row (us per step).
    Some 20-40 s of host time in all."""
    import oracle
    from selective_state_space_48_amd import workloads as W

    nt = oracle.default_threads()
    res = {"cores": nt, "kind": "oracle"}
    for name in ("tiny_f32_b1_l256_d16", "m130m_f32_b8_l2048_d1536", W.HEADLINE, "long_f32_b1_l1048576_d128"):
        w = W.get(name)
        inp = W.fwd_inputs(w)
        kw = dict(D=inp["D"], z=inp["z"] if w.gate else None, dt_bias=inp["dt_bias"])
        t0 = time.perf_counter()
        oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], nthreads=nt, **kw)
        dt = time.perf_counter() - t0
        # one thread on a bounded slice: one batch entry, at most 32 rows
        nr = min(w.dim, 32)
        sl = (slice(0, 1), slice(0, nr))
        t0 = time.perf_counter()
        oracle.fwd(inp["x"][sl], inp["delta"][sl], inp["A"][:nr], inp["B"][:1], inp["C"][:1],
                   D=inp["D"][:nr], z=None if kw["z"] is None else inp["z"][sl],
                   dt_bias=inp["dt_bias"][:nr], nthreads=1)
        dt1 = time.perf_counter() - t0
        res[name] = {"Gelem_per_s": round(w.elements / dt / 1e9, 6), "s_wall": round(dt, 4),
                     "Gelem_per_s_1_thread": round(nr * w.seqlen / dt1 / 1e9, 6),
                     "sample": f"all {w.rows} rows x {w.seqlen} tokens on {nt} threads; "
                               f"1 thread: {nr} rows"}
        del inp
    wd = W.get(W.DECODE)
    p = W.params(wd)
    t0 = time.perf_counter()
    h = np.empty((wd.batch, wd.dim, wd.dstate))
    gen = 0.0
    for b in range(wd.batch):
        g0 = time.perf_counter()
        pre = W.prefill_inputs(wd, b)
        gen += time.perf_counter() - g0
        r = oracle.fwd(pre["x"], pre["delta"], p["A"], pre["B"], np.zeros_like(pre["B"]), D=p["D"],
                       dt_bias=p["dt_bias"], nthreads=nt)
        h[b] = r["last_state"][0]
    prefill = time.perf_counter() - t0 - gen
    si = W.step_inputs(wd, 0)
    t0 = time.perf_counter()
    oracle.step(h, si["x"], si["delta"], p["A"], si["B"], si["C"], D=p["D"], z=si["z"])
    step = time.perf_counter() - t0
    res[W.DECODE] = {"us_per_step": round(step * 1e6, 1), "prefill_s": round(prefill, 3),
                     "sample": f"one step over all {wd.rows} rows (the step oracle is one "
                               f"thread); prefill: {wd.prefill} tokens of all {wd.batch} "
                               f"sequences on {nt} threads, input generation excluded"}
    return res


def copy_calibration(torch, dev, gib=1, reps=3):
    """Device copies of known size, run under rocprofv3 --pmc FETCH_SIZE /
    WRITE_SIZE to turn those counters into bytes: torch's copy kernel, and the
    calibration library's plain, non-temporal and row-pattern copies (the
    access patterns of the scan kernels)."""
    import ctypes

    from selective_state_space_48_amd import build as B

    n = (gib << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    lib = ctypes.CDLL(B.CALIB_LIB)
    lib.selscan_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    for mode in (0, 1, 2):
        for _ in range(reps):
            rc = lib.selscan_calib_copy(src.data_ptr(), dst.data_ptr(), n * 4, mode, stream)
            assert rc == 0, rc
    torch.cuda.synchronize(dev)
    return {"copy_bytes_each_way": n * 4, "reps": reps,
            "kernels": ["torch copy", "calib mode 0 plain", "calib mode 1 non-temporal",
                        "calib mode 2 non-temporal row pattern"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extras", action="store_true", help="headline forward only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["fwd", "decode", "long", "m130m", "conv", "bwd", "ssd", "ragged",
                                       "copy"],
                    default=None,
                    help="run just one workload (for profiling); copy = counter calibration")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}). Across GPUs the rows "
              "would be split, or a long sequence's segments, each GPU passing on its segments' "
              "end states and summed step sizes for the carries; that is not measured here.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_48_amd import workloads as W

    dev = torch.device("cuda:0")
    out = {}
    w = W.get(W.HEADLINE)
    if args.only == "copy":
        print(json.dumps(copy_calibration(torch, dev)), flush=True)
        return

    inp = None
    if args.only in (None, "fwd"):
        inp = W.fwd_inputs(w)
        log(f"[bench] {w.name}: {args.warmup} warmup + {args.steps} timed forward calls")
        ceil = measured_ceilings(torch, dev)
        log(f"[bench] measured ceilings: {ceil}")
        ms, wall, k_ms, dist = time_fwd(w, args.steps, args.warmup, torch, dev, inp, distribution=True)
        E = w.elements
        gelem = E / (ms * 1e-3) / 1e9
        bytes_ = algorithmic_bytes(w)
        slots = method_slots(w)
        hbm = bytes_ / (k_ms * 1e-3)
        alu = slots / (k_ms * 1e-3)
        log(f"[bench] {w.name}: {ms * 1e3:.1f} us/call ({k_ms * 1e3:.1f} us output-pass kernel), "
            f"{gelem:.1f} Gelem/s, kernel at {hbm / 1e12:.2f} TB/s algorithmic, "
            f"{alu / 1e12:.1f} T VALU-slot/s method")
        traffic = measured_traffic()
        out.update({
            "metric": "selective-scan fwd Gelem/s (B*L*d_inner), Mamba-1.4B-shaped layer",
            "value": round(gelem, 3),
            "unit": "Gelem/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms, 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16 in/out, f32 state+math",
            "data": "synthetic (seeded; see selective_state_space_48_amd/workloads.py)",
            "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen,
                       "d_inner": w.dim, "d_state": w.dstate, "gate": w.gate,
                       "parallelism": "single GPU"},
            "roofline": {"bound": "alu", "achieved": round(alu / 1e12, 3),
                         "peak": round(SLOT_PEAK / 1e12, 3), "unit": "T VALU-slot/s",
                         "frac": round(alu / SLOT_PEAK, 4), "traffic": traffic,
                         "kernel": "fwd_kernel<bf16, 4 waves, gate, 16-byte rows, output pass>",
                         "kernel_us": round(k_ms * 1e3, 2), "slots_per_launch": slots,
                         "measured_peak": ceil["scan_mix_T_slot_per_s"],
                         "frac_of_measured_peak": round(alu / 1e12 / ceil["scan_mix_T_slot_per_s"], 4)},
            "hbm": {"achieved": round(hbm / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                    "frac": round(hbm / HBM_PEAK, 4), "bytes_per_launch": bytes_,
                    "traffic_over_algorithmic": None if traffic is None else round(traffic / bytes_, 3),
                    "copy_GBps": ceil["copy_GBps"],
                    "frac_of_copy": round(hbm / 1e9 / ceil["copy_GBps"], 4),
                    # the aim of 70% of the HBM peak on this workload, and why it
                    # is out of reach for this method without packed fp32
                    "target_frac": 0.70, "target_met": bool(hbm / HBM_PEAK >= 0.70),
                    "bound_by": "VALU issue: one exp (2 slots) and four fp32 operations per "
                                "(token, state) make 6 slots, 96 per element, plus the per-token "
                                "softplus/silu; the method's 110 slots per element take "
                                f"{slots / SLOT_PEAK * 1e6:.0f} us at the 2.4 GHz slot peak, "
                                f"above the {bytes_ / (0.7 * HBM_PEAK) * 1e6:.0f} us that 70% of "
                                "8 TB/s allows"},
            "per_call": dist,
            "wall_s_timed": round(wall, 4),
        })

    extras = {}
    if not args.no_extras and args.only in (None, "decode"):
        wd = W.get(W.DECODE)
        log(f"[bench] {wd.name}: decode steps")
        ms_step, k_ms, ddist = time_decode(wd, 256, 16, torch, dev)
        us, kus = ms_step * 1e3, k_ms * 1e3
        gbs = step_bytes(wd) / (kus * 1e-6) / 1e9
        cold = ddist["cold"]["p50_us"]
        log(f"[bench] decode: {us:.2f} us/step back to back ({kus:.2f} us kernel, {gbs:.0f} GB/s); "
            f"cold median {cold:.2f} us")
        # Primary: the median of the 64 distinct steps each run with the
        # caches flushed (a 512 MB write sweep, then a 512 MB read sweep of
        # another buffer: the 84 MB state would otherwise stay in the 256 MB
        # last-level cache between back-to-back steps; in a model the other
        # layers run in between). Beside it: right after the write sweep
        # alone (the step also writes back the sweep's dirty lines), and back
        # to back.
        cold_gbs = step_bytes(wd) / (cold * 1e-6) / 1e9
        extras["decode"] = {"workload": wd.name, "us_per_step": round(cold, 3),
                            "us_per_step_is": "cold p50 (caches flushed before each step: write sweep, then read sweep)",
                            "cold_dirty_us_per_step": ddist["cold_dirty"]["p50_us"],
                            "achieved_GBps": round(cold_gbs, 1),
                            "frac_hbm": round(cold_gbs * 1e9 / HBM_PEAK, 4),
                            "back_to_back_us_per_step": round(us, 3),
                            "back_to_back_kernel_us": round(kus, 3),
                            "back_to_back_kernel_GBps": round(gbs, 1),
                            "back_to_back_kernel_frac_hbm": round(gbs * 1e9 / HBM_PEAK, 4),
                            "bytes_per_step": step_bytes(wd), "per_step": ddist}
        # the same at one sequence, where the launches rather than the bytes set the rate
        extras["block_decode"] = [time_block_decode(wd, torch, dev),
                                  time_block_decode(W.scaled(wd, batch=1, name=wd.name.replace("b256", "b1")),
                                                    torch, dev)]
        log(f"[bench] block decode step: {extras['block_decode']}")
    if not args.no_extras and args.only in (None, "bwd"):
        log("[bench] backward: headline shape")
        extras["bwd"] = time_bwd(torch, dev)
        log(f"[bench] backward: {extras['bwd']}")
        log("[bench] backward: long-memory workload")
        extras["bwd_long"] = time_bwd_long(torch, dev)
        log(f"[bench] backward long: {extras['bwd_long']}")
    if not args.no_extras and args.only in (None, "ssd"):
        log("[bench] SSD layer")
        extras["ssd"] = time_ssd(torch, dev)
        log(f"[bench] ssd: {extras['ssd']}")
        log("[bench] SSD decode step")
        extras["ssd_decode"] = time_ssd_decode(torch, dev)
        log(f"[bench] ssd decode: {extras['ssd_decode']}")
    if not args.no_extras and args.only in (None, "conv"):
        log("[bench] conv1d: headline shape and decode steps")
        extras.update(time_conv(torch, dev))
        log("[bench] conv1d fused into the scan")
        extras["conv_fused"] = time_fused_conv(torch, dev)
        log(f"[bench] conv fused: {extras['conv_fused']}")
    if not args.no_extras and args.only in (None, "ragged"):
        log("[bench] ragged rows (L 2047 against 2048)")
        extras["ragged"] = time_ragged(torch, dev)
        log(f"[bench] ragged: {extras['ragged']}")
    for key, name in (("long", "long_f32_b1_l1048576_d128"), ("m130m", "m130m_f32_b8_l2048_d1536")):
        if args.no_extras or args.only not in (None, key):
            continue
        wx = W.get(name)
        log(f"[bench] {name}: forward")
        ms, _, k_ms, _ = time_fwd(wx, 10, 2, torch, dev)
        extras[key] = {"workload": name, "ms_per_call": round(ms, 4),
                       "output_pass_ms": round(k_ms, 4),
                       "Gelem_per_s": round(wx.elements / (ms * 1e-3) / 1e9, 2),
                       "frac_hbm": round(algorithmic_bytes(wx) / (ms * 1e-3) / HBM_PEAK, 4),
                       # the method's slots (one pass) against the slot peak: over the
                       # output pass alone, and over the whole call (which adds the
                       # state pass of a segmented plan)
                       "output_pass_frac_alu": round(method_slots(wx) / (k_ms * 1e-3) / SLOT_PEAK, 4),
                       "call_frac_alu": round(method_slots(wx) / (ms * 1e-3) / SLOT_PEAK, 4)}
    if extras:
        out["extras"] = extras

    if args.only in (None, "fwd") and not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(w, inp)
        log(f"[bench] cpu baseline: {out['cpu_baseline']}")
        if not args.no_extras:
            log("[bench] cpu baseline per configuration (oracle)")
            out["cpu_baseline_per_config"] = cpu_baseline_per_config()
            log(f"[bench] cpu baseline per configuration: {out['cpu_baseline_per_config']}")

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
