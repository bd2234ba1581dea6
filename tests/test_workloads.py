"""The seeded input generator: determinism, batch-sliceability, value recipe. CPU only."""
import numpy as np
import torch

from selective_state_space_48_amd import workloads as W


def test_deterministic_and_sliceable():
    w = W.scaled(W.get(W.HEADLINE), seqlen=64, dim=32, batch=3)
    a = W.fwd_inputs(w)
    b = W.fwd_inputs(w)
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k])
    part = W.fwd_inputs(w, batches=[2])
    for k in ("x", "delta", "z", "B", "C"):
        assert np.array_equal(part[k][0], a[k][2])


def test_bf16_values_are_torch_rounded():
    w = W.scaled(W.get(W.HEADLINE), seqlen=16, dim=8, batch=1)
    a = W.fwd_inputs(w)
    for k in ("x", "delta", "z", "B", "C"):
        t = torch.from_numpy(a[k])
        assert torch.equal(t.to(torch.bfloat16).float(), t)


def test_value_recipe():
    w = W.get(W.HEADLINE)
    p = W.params(w)
    assert p["A"].shape == (4096, 16)
    assert np.array_equal(p["A"][7], -np.arange(1, 17, dtype=np.float32))
    sp = np.logaddexp(0.0, p["dt_bias"].astype(np.float64))
    assert sp.min() >= 1e-3 * 0.999 and sp.max() <= 1e-1 * 1.001
    assert p["D"].min() >= 0.5 and p["D"].max() <= 1.5
    lw = W.get("long_f32_b1_l1048576_d128")
    sp = np.logaddexp(0.0, W.params(lw)["dt_bias"].astype(np.float64))
    assert sp.min() >= 1e-4 * 0.999 and sp.max() <= 1e-2 * 1.001
    tiny = W.get("tiny_f32_b1_l256_d16")
    assert np.all(W.params(tiny)["D"] == 1.0) and W.fwd_inputs(tiny)["z"] is None


def test_state_size_arithmetic():
    """The per-layer decode state of a d_inner 4096, N 16 layer holds 65,536
    values, 131,072 bytes at 16 bits ("State Space Models and Mamba",
    multigrid.ai, "The state, in bytes, against a KV cache")."""
    w = W.get(W.HEADLINE)
    assert w.dim * w.dstate == 65536
    assert w.dim * w.dstate * 2 == 131072


def test_step_inputs_shapes():
    w = W.scaled(W.get(W.DECODE), batch=4, dim=64)
    s = W.step_inputs(w, 0)
    assert s["x"].shape == (4, 64) and s["B"].shape == (4, 16)
    s2 = W.step_inputs(w, 1)
    assert not np.array_equal(s["x"], s2["x"])
    pre = W.prefill_inputs(w, 2)
    assert pre["x"].shape == (1, 64, 512) and pre["B"].shape == (1, 16, 512)


def test_conv_inputs():
    w = W.scaled(W.get(W.HEADLINE), seqlen=40, dim=16, batch=3)
    a = W.conv_inputs(w)
    assert a["x"].shape == (3, 16, 40) and a["x_prev"].shape == (3, 16, 3)
    assert a["w"].shape == (16, 4) and a["bias"].shape == (16,)
    assert np.array_equal(a["x"], W.fwd_inputs(w)["x"])      # the forward's x stream
    part = W.conv_inputs(w, batches=[1])
    assert np.array_equal(part["x_prev"][0], a["x_prev"][1])
    t = torch.from_numpy(a["x_prev"])
    assert torch.equal(t.to(torch.bfloat16).float(), t)
    assert W.conv_step_inputs(W.get(W.DECODE), 3).shape == (256, 5120)
