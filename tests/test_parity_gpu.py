"""GPU parity: libselscan's forward pass against the fp64 oracle on the same
seeded inputs, element by element, at small sizes (several tiles, ragged
tails) and on every launch variant; plus edge cases and the pages' worked
examples through the GPU kernels. Run on an MI355X: pytest -m gpu."""
import math

import numpy as np
import pytest
import torch

from parity_util import TOL, TDT, assert_close, dev, errors, gpu_fwd, oracle_fwd, small, to_np
from selective_state_space_48_amd import selscan
from selective_state_space_48_amd import workloads as W

pytestmark = pytest.mark.gpu

TINY = "tiny_f32_b1_l256_d16"
M14 = W.HEADLINE


def case(msg):
    print(f"[case] {msg}", flush=True)


def test_tiny_workload():
    case("tiny fp32 b1 l256 d16")
    inp = W.fwd_inputs(W.get(TINY))
    y, hs = gpu_fwd(inp, "f32")
    assert_close(y, hs, oracle_fwd(inp), "f32", "tiny")


SHAPES = [
    # (batch, L, dim, dtype, gate)
    (1, 1, 1, "f32", False),
    (1, 1, 1, "bf16", True),
    (2, 31, 65, "f32", True),      # L below one tile, ragged rows
    (2, 33, 64, "bf16", True),     # one full tile plus one token
    (3, 100, 130, "bf16", True),   # several tiles, ragged tail, 3 row blocks
    (1, 257, 7, "f32", False),
    (2, 64, 128, "f32", True),
    (1, 37, 70, "bf16", True),     # rows not 16-byte aligned (element path)
    (2, 45, 66, "f32", True),      # rows not 16-byte aligned (element path)
    (1, 600, 64, "bf16", False),   # long enough for automatic segmenting
]


@pytest.mark.parametrize("batch,L,dim,dtype,gate", SHAPES)
def test_shapes(batch, L, dim, dtype, gate):
    case(f"shape b{batch} L{L} d{dim} {dtype} gate={gate}")
    name = M14 if dtype == "bf16" else "m130m_f32_b8_l2048_d1536"
    inp = small(name, batch=batch, seqlen=L, dim=dim)
    if not gate:
        inp["z"] = None
    y, hs = gpu_fwd(inp, dtype)
    assert_close(y, hs, oracle_fwd(inp), dtype, f"b{batch} L{L} d{dim} {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_launch_variant(dtype):
    """Every wave split and several segment counts give the oracle's result;
    the segmented (chunk state + carry + rescan) path is thereby checked
    against the same definition as the one-pass path."""
    inp = small(M14 if dtype == "bf16" else "m130m_f32_b8_l2048_d1536", batch=2, seqlen=1100,
                dim=130)
    ref = oracle_fwd(inp)
    ys = {}
    for groups in (1, 2, 4, 8):
        for segments in (1, 2, 5, 34):
            case(f"variant {dtype} groups={groups} segments={segments}")
            y, hs = gpu_fwd(inp, dtype, groups=groups, segments=segments)
            assert_close(y, hs, ref, dtype, f"groups={groups} segments={segments}")
            ys[(groups, segments)] = to_np(y)
    # the split over waves only reorders the readout sum: one-pass variants agree closely
    a, b = ys[(1, 1)], ys[(4, 1)]
    assert np.max(np.abs(a - b) / (np.abs(ref["y_scale"]) + 1e-30)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("segments", [65, 200])
def test_many_segments_few_rows(dtype, segments):
    """Many segments over few rows, as in the long-sequence plans: the carries
    are composed in runs of segments per wave, chained through LDS, instead of
    one sequential chain per (row, state)."""
    inp = small(M14 if dtype == "bf16" else "m130m_f32_b8_l2048_d1536", batch=1, seqlen=6400, dim=40)
    case(f"{segments} segments {dtype} b1 L6400 d40")
    y, hs = gpu_fwd(inp, dtype, segments=segments)
    assert_close(y, hs, oracle_fwd(inp), dtype, f"{segments} segments {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L,dim,segments", [(1101, 130, 1), (1101, 130, 3), (37, 64, 1), (2048, 64, 0)])
def test_eight_waves(dtype, L, dim, segments):
    """8 waves of 2 states per row block (bf16: 8-byte token slices): element
    rows (L * element size not a multiple of 16), a segmented run (the
    8-wave state pass), a short sequence, and a shape whose automatic plan
    picks 8 waves (blocks of 64 rows: 160 fp32 or 224 bf16 batch entries of
    one block each)."""
    batch = (160 if dtype == "f32" else 224) if segments == 0 else 2
    case(f"8 waves {dtype} b{batch} L{L} d{dim} segments={segments}")
    inp = small(M14 if dtype == "bf16" else "m130m_f32_b8_l2048_d1536", batch=batch, seqlen=L, dim=dim)
    y, hs = gpu_fwd(inp, dtype, groups=8 if segments else 0, segments=segments)
    assert_close(y, hs, oracle_fwd(inp), dtype, f"8 waves {dtype} L{L} d{dim} segments={segments}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_optional_inputs_absent(dtype):
    case(f"no D, no dt_bias, no gate {dtype}")
    inp = small(M14, batch=2, seqlen=96, dim=64)
    y, hs = gpu_fwd(inp, dtype, use_D=False, use_bias=False, use_z=False)
    assert_close(y, hs, oracle_fwd(inp, use_D=False, use_bias=False, use_z=False), dtype,
                 "no optional inputs")
    case(f"no last_state {dtype}")
    y2, none = gpu_fwd(inp, dtype, use_D=False, use_bias=False, use_z=False, last_state=False)
    assert none is None
    assert torch.equal(y, y2)


def test_deterministic():
    inp = small(M14, batch=2, seqlen=700, dim=100)
    for seg in (1, 4):
        case(f"determinism segments={seg}")
        y1, h1 = gpu_fwd(inp, "bf16", segments=seg)
        y2, h2 = gpu_fwd(inp, "bf16", segments=seg)
        assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_extreme_values():
    """softplus far beyond +-20, decays that underflow to 0, large gates."""
    rng = np.random.default_rng(5)
    inp = small("m130m_f32_b8_l2048_d1536", batch=1, seqlen=300, dim=64)
    inp["delta"] = (rng.uniform(-80, 80, inp["delta"].shape)).astype(np.float32)
    inp["A"][:8] = -1e4        # decay exp(delta*A) underflows to 0 for these channels
    inp["z"] = (rng.uniform(-60, 60, inp["z"].shape)).astype(np.float32)
    inp["dt_bias"][:] = 0.0
    case("extreme values fp32")
    y, hs = gpu_fwd(inp, "f32")
    assert_close(y, hs, oracle_fwd(inp), "f32", "extremes")


def test_small_step_sizes_long_memory():
    """Step sizes ~1e-4 (the long-sequence recipe) over 4096 tokens: the
    decays sit just below 1 and errors would accumulate."""
    inp = small("long_f32_b1_l1048576_d128", seqlen=4096, dim=64)
    case("long-memory fp32 L=4096")
    y, hs = gpu_fwd(inp, "f32")
    assert_close(y, hs, oracle_fwd(inp), "f32", "long memory one pass")
    y, hs = gpu_fwd(inp, "f32", segments=16)
    assert_close(y, hs, oracle_fwd(inp), "f32", "long memory 16 segments")


def test_nan_propagates():
    inp = small("m130m_f32_b8_l2048_d1536", batch=2, seqlen=80, dim=64)
    inp["x"][1, 3, 50] = np.nan
    case("NaN input fp32")
    y, hs = gpu_fwd(inp, "f32")
    assert_close(y, hs, oracle_fwd(inp), "f32", "NaN propagation")
    yn = to_np(y)
    assert np.all(np.isnan(yn[1, 3, 50:])) and np.all(np.isfinite(yn[1, 3, :50]))
    assert np.isfinite(yn[0]).all()


def test_empty_inputs():
    case("L = 0")
    x = torch.empty((2, 64, 0), device="cuda")
    A = -torch.ones((64, 16), device="cuda")
    B = torch.empty((2, 16, 0), device="cuda")
    hs = torch.full((2, 64, 16), 7.0, device="cuda")
    y, hs = selscan.fwd(x, x.clone(), A, B, B.clone(), last_state=hs)
    torch.cuda.synchronize()
    assert y.shape == (2, 64, 0) and torch.all(hs == 0)
    case("batch = 0")
    x = torch.empty((0, 64, 10), device="cuda")
    B = torch.empty((0, 16, 10), device="cuda")
    y, hs = selscan.fwd(x, x.clone(), A, B, B.clone())
    torch.cuda.synchronize()
    assert y.shape == (0, 64, 10)


def _embed_scalar(A1, B1, C1, dl_raw, x, dtype):
    """One-state problems placed in state 0 of the 16-state kernel (B = 0 elsewhere)."""
    dim, L = x.shape
    A = -np.ones((dim, 16), np.float32) * 2.0
    A[:, 0] = A1
    B = np.zeros((1, 16, L), np.float32)
    B[0, 0] = B1
    C = np.random.default_rng(0).standard_normal((1, 16, L)).astype(np.float32)
    C[0, 0] = C1
    td = TDT[dtype]
    y, hs = selscan.fwd(dev(x[None], td), dev(dl_raw[None], td), dev(A), dev(B, td), dev(C, td))
    torch.cuda.synchronize()
    return to_np(y)[0], to_np(hs)[0]


def test_worked_example_run_ssm_on_gpu():
    """The fixed-decay example ("A tiny example you can run", mernstackdev.com)
    through the GPU kernel: a = 0.9 and 0.3 as two channels."""
    from oracle_pins import golden
    g = golden("run_ssm.txt")
    sig = np.array(g["signal"], np.float32)
    L = sig.size
    x = np.stack([sig, sig])
    A1 = np.array([math.log(0.9), math.log(0.3)], np.float32)
    dl = np.full((2, L), math.log(math.e - 1.0), np.float32)   # softplus = 1
    case("run_ssm fp32 on GPU")
    y, _ = _embed_scalar(A1, np.ones(L, np.float32), np.ones(L, np.float32), dl, x, "f32")
    t = np.arange(L)
    for i, (key, a) in enumerate((("a=0.9", 0.9), ("a=0.3", 0.3))):
        closed = a ** t + 5.0 * np.where(t >= 4, a ** np.maximum(t - 4, 0), 0.0)
        assert np.max(np.abs(y[i] - closed)) < 2e-5
        assert np.array_equal(np.round(y[i], 3), np.array(g[key]))


def test_worked_example_run_selective_on_gpu():
    from oracle_pins import golden
    g = golden("run_selective.txt")
    vals = np.array(g["values"], np.float32)
    imp = np.array(g["important"]) > 0
    keep = np.where(imp, g["keep_important"][0], g["keep_other"][0])
    write = np.where(imp, g["write_important"][0], g["write_other"][0])
    dl = -np.log(keep)
    case("run_selective fp32 on GPU")
    y, _ = _embed_scalar(np.array([-1.0], np.float32), (write / dl).astype(np.float32),
                         np.ones(vals.size, np.float32),
                         np.log(np.expm1(dl)).astype(np.float32)[None], vals[None], "f32")
    assert np.max(np.abs(y[0] - np.array(g["exact"]))) < 5e-5
    assert np.array_equal(np.round(y[0], 2), np.array(g["printed"]))


def test_forward_equals_steps_on_gpu():
    """The two execution modes agree on the GPU: a forward pass over L tokens
    and L decode steps fed delta_raw + dt_bias (formed in fp32, as the forward
    kernel forms it), both against the oracle."""
    import oracle
    inp = small("m130m_f32_b8_l2048_d1536", batch=2, seqlen=40, dim=96)
    case("fwd vs steps fp32")
    y, hs = gpu_fwd(inp, "f32")
    state = torch.zeros((2, 96, 16), device="cuda")
    ys = []
    for t in range(40):
        dsum = (inp["delta"][..., t] + inp["dt_bias"][None]).astype(np.float32)
        ys.append(selscan.step(state, dev(inp["x"][..., t]), dev(dsum), dev(inp["A"]),
                               dev(inp["B"][..., t]), dev(inp["C"][..., t]), D=dev(inp["D"]),
                               z=dev(inp["z"][..., t])))
    torch.cuda.synchronize()
    ref = oracle_fwd(inp)
    ystep = np.stack([to_np(v) for v in ys], -1)
    assert oracle.scaled_error(ystep, ref["y"], ref["y_scale"]) <= TOL["f32"]
    assert oracle.scaled_error(to_np(state), ref["last_state"], ref["state_scale"]) <= TOL["f32"]
    assert np.max(np.abs(ystep - to_np(y)) / (ref["y_scale"] + 1e-30)) <= TOL["f32"]
