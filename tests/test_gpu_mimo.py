"""GPU parity of the bias-free linear layers (MIMO head mixer, out_proj)
against the float64 oracle: bf16 matrix products with fp32 accumulation, so
the bf16 tolerance (2e-2, normwise per (batch, head) slice for MIMO, per row
for plain layers), plus exact structural cases: the identity mixer returns y
rounded to bf16, a head permutation permutes heads bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_09_amd as ssd
from selective_state_space_09_amd import inputs
from _metrics import report
import _gpu

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


def _rand(shape, std, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(std)


LINEAR_CASES = [
    # M, K, Nout, x dtype, z dtype
    (1, 64, 128, "f32", "bf16"),
    (300, 128, 256, "f32", "f32"),
    (257, 192, 128, "bf16", "bf16"),
    (1000, 1024, 1024, "bf16", "f32"),
    (130, 512, 384, "f32", "bf16"),
]


@pytest.mark.parametrize("case", LINEAR_CASES, ids=lambda c: "M%dK%dN%d_%s_%s" % c)
def test_linear_small(case):
    M, K, Nout, xd, zd = case
    print("case:", case, flush=True)
    x = _rand((M, K), 1.0, 1)
    W = inputs.f32_to_bf16_bits(_rand((Nout, K), 1.0 / np.sqrt(K), 2))
    xin = inputs.f32_to_bf16_bits(x) if xd == "bf16" else x
    z = ssd.ssd_linear_fwd(_gpu.to_dev(xin), _gpu.to_dev(W),
                           out_dtype=torch.bfloat16 if zd == "bf16" else torch.float32)
    torch.cuda.synchronize()
    zr = oracle.linear(xin, W)
    # normwise per row (a wrong row or a wrong output tile shows in its rows)
    zg = _gpu.to_host64(z)
    assert report("z per row", zg[:, None, :], zr[:, None, :], "state") < TOL_BF16


def test_linear_empty_and_bad_shapes():
    W = torch.zeros((128, 64), dtype=torch.bfloat16, device="cuda")
    z = ssd.ssd_linear_fwd(torch.zeros((0, 64), device="cuda"), W)
    assert z.shape == (0, 128)
    with pytest.raises(ssd.SSDError) as e:
        ssd.ssd_linear_fwd(torch.zeros((4, 64), device="cuda"),
                           torch.zeros((100, 64), dtype=torch.bfloat16, device="cuda"))
    assert e.value.code == ssd.SSD_EUNSUPPORTED


@pytest.mark.parametrize("ydtype", ["f32", "bf16"])
def test_mimo_identity_returns_y_rounded(ydtype):
    """W = I: each output is one product 1 * y in fp32, so z is y rounded to
    bf16 (nearest even) bit for bit."""
    inp = inputs.make_mimo(2, 100, 4, 32, seed=3, identity=True)
    y = inp["y"] if ydtype == "f32" else inputs.f32_to_bf16_bits(inp["y"])
    z = ssd.ssd_mimo_fwd(_gpu.to_dev(y), _gpu.to_dev(inp["W"]))
    torch.cuda.synchronize()
    expect = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(inp["y"])).astype(np.float64)
    np.testing.assert_array_equal(_gpu.to_host64(z), expect)


def test_mimo_head_permutation_is_exact():
    """W = (head permutation) x I_P moves head perm[h] to head h exactly."""
    H, P = 8, 16
    perm = [5, 2, 7, 0, 1, 6, 3, 4]
    W = np.zeros((H * P, H * P), np.float32)
    for h in range(H):
        for p in range(P):
            W[h * P + p, perm[h] * P + p] = 1.0
    y = inputs.f32_to_bf16_bits(_rand((3, 77, H, P), 1.0, 4))
    z = ssd.ssd_mimo_fwd(_gpu.to_dev(y), _gpu.to_dev(inputs.f32_to_bf16_bits(W)),
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    zg = _gpu.to_host64(z)
    yg = inputs.bf16_bits_to_f32(y).astype(np.float64)
    for h in range(H):
        np.testing.assert_array_equal(zg[:, :, h, :], yg[:, :, perm[h], :])


def test_mimo_workload_sampled_rows():
    """The MIMO mixer at the Mamba-3-Lite block shape (B8 T2048 H16 P64, fp32
    scan output in, random bf16 weight, bf16 out), in the launch configuration
    the benchmark times, compared on sampled token rows computed by the
    oracle one by one."""
    print("case: mimo_bf16 workload", flush=True)
    inp = inputs.make_workload("mimo_bf16")
    y, W = inp["y"], inp["W"]
    z = ssd.ssd_mimo_fwd(_gpu.to_dev(y), _gpu.to_dev(W))
    torch.cuda.synchronize()
    Bsz, T = y.shape[:2]
    rows = [(0, 0), (0, 1), (1, 127), (3, 128), (5, 1000), (7, 2046), (7, 2047), (2, 513)]
    zs = np.stack([_gpu.to_host64(z[b, t]) for b, t in rows])[None]       # (1, R, H, P)
    zr = np.stack([oracle.mimo(y[b:b + 1, t:t + 1], W)[0, 0] for b, t in rows])[None]
    assert report("z (8 rows)", zs, zr) < TOL_BF16
