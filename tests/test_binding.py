"""Host-only checks of the Python binding: every tensor argument's shape is
checked against x (or h, xbc, proj) before anything reaches the library, so a
mismatched tensor raises instead of sending the kernels outside an
allocation.  CPU tensors are used: shape errors must come first, ahead of the
device check (a correctly shaped CPU tensor fails on the device check)."""
import pytest
import torch

import selective_state_space_09_amd as ssd

f32 = torch.float32


def real_args(Bsz=2, T=10, H=4, P=16, G=2, N=16):
    return dict(x=torch.zeros(Bsz, T, H, P), dt=torch.zeros(Bsz, T, H), A=torch.zeros(H),
                B=torch.zeros(Bsz, T, G, N), C=torch.zeros(Bsz, T, G, N), D=torch.zeros(H),
                dt_bias=torch.zeros(H), h0=torch.zeros(Bsz, H, P, N))


def _raises_shape(fn, name, **kw):
    with pytest.raises(ValueError) as e:
        fn(**kw)
    assert name in str(e.value) and "shape" in str(e.value) or "dimensions" in str(e.value), \
        str(e.value)


def test_real_forward_good_shapes_reach_device_check():
    with pytest.raises(ValueError, match="GPU tensor"):
        ssd.ssd_chunk_fwd(**real_args())


@pytest.mark.parametrize("name,bad", [
    ("dt", torch.zeros(2, 10, 3)), ("A", torch.zeros(5)), ("B", torch.zeros(2, 9, 2, 16)),
    ("C", torch.zeros(2, 10, 2, 8)), ("D", torch.zeros(3)), ("dt_bias", torch.zeros(1)),
    ("h0", torch.zeros(2, 4, 16, 8)), ("y", torch.zeros(2, 10, 4, 8)),
    ("h_final", torch.zeros(1, 4, 16, 16)),
])
def test_real_forward_rejects_mismatched_shapes(name, bad):
    kw = real_args()
    kw[name] = bad
    _raises_shape(ssd.ssd_chunk_fwd, name, **kw)


def test_real_forward_rejects_wrong_rank():
    kw = real_args()
    kw["x"] = torch.zeros(2, 10, 64)
    with pytest.raises(ValueError, match="dimensions"):
        ssd.ssd_chunk_fwd(**kw)


def cplx_args(Bsz=1, T=8, H=2, P=16, G=2, N=16):
    return dict(x=torch.zeros(Bsz, T, H, P), dt=torch.zeros(Bsz, T, H), A=torch.zeros(H, 2),
                B=torch.zeros(Bsz, T, G, N, 2), C=torch.zeros(Bsz, T, G, N, 2),
                dt_bias=torch.zeros(H), h0=torch.zeros(Bsz, H, P, N, 2))


@pytest.mark.parametrize("name,bad", [
    ("A", torch.zeros(2)), ("C", torch.zeros(1, 8, 2, 16)), ("C", torch.zeros(1, 8, 1, 16, 2)),
    ("dt", torch.zeros(1, 7, 2)), ("h0", torch.zeros(1, 2, 16, 16)),
    ("y", torch.zeros(1, 8, 2, 15)), ("h_final", torch.zeros(1, 2, 16, 15, 2)),
])
def test_complex_forward_rejects_mismatched_shapes(name, bad):
    kw = cplx_args()
    kw[name] = bad
    _raises_shape(ssd.ssd_complex_chunk_fwd, name, **kw)


def test_complex_forward_accepts_complex64_views():
    kw = cplx_args()
    kw["B"] = torch.zeros(1, 8, 2, 16, dtype=torch.complex64)
    kw["C"] = torch.zeros(1, 8, 2, 16, dtype=torch.complex64)
    kw["A"] = torch.zeros(2, dtype=torch.complex64)
    with pytest.raises(ValueError, match="GPU tensor"):
        ssd.ssd_complex_chunk_fwd(**kw)


def decode_args(Bsz=3, H=4, P=8, G=2, N=16):
    return dict(h=torch.zeros(Bsz, H, P, N), x=torch.zeros(Bsz, H, P), dt=torch.zeros(Bsz, H),
                A=torch.zeros(H), B=torch.zeros(Bsz, G, N), C=torch.zeros(Bsz, G, N),
                D=torch.zeros(H), dt_bias=torch.zeros(H))


@pytest.mark.parametrize("name,bad", [
    ("x", torch.zeros(3, 4, 7)), ("dt", torch.zeros(2, 4)), ("A", torch.zeros(8)),
    ("C", torch.zeros(3, 2, 8)), ("D", torch.zeros(2)), ("y", torch.zeros(3, 4, 9)),
])
def test_decode_rejects_mismatched_shapes(name, bad):
    kw = decode_args()
    kw[name] = bad
    _raises_shape(ssd.ssd_step_decode, name, **kw)


@pytest.mark.parametrize("name,bad", [
    ("x", torch.zeros(3, 4, 7)), ("A", torch.zeros(4)), ("B", torch.zeros(3, 2, 16)),
    ("y", torch.zeros(3, 4, 9)),
])
def test_complex_decode_rejects_mismatched_shapes(name, bad):
    kw = decode_args()
    kw["h"] = torch.zeros(3, 4, 8, 16, 2)
    kw["A"] = torch.zeros(4, 2)
    kw["B"] = torch.zeros(3, 2, 16, 2)
    kw["C"] = torch.zeros(3, 2, 16, 2)
    kw.pop("D")
    kw[name] = bad
    _raises_shape(ssd.ssd_complex_step_decode, name, **kw)


def test_conv_rejects_mismatched_shapes():
    xbc = torch.zeros(2, 5, 64 + 2 * 16)
    w = torch.zeros(96, 4)
    with pytest.raises(ValueError, match="GPU tensor"):
        ssd.ssd_conv1d_fwd(xbc, w, 64, 16)
    for name, bad in (("w", torch.zeros(95, 4)), ("bias", torch.zeros(64)),
                      ("state_in", torch.zeros(2, 3, 95)), ("x", torch.zeros(2, 5, 63)),
                      ("B", torch.zeros(2, 4, 16)), ("state_out", torch.zeros(1, 3, 96))):
        kw = dict(xbc=xbc, w=w, HP=64, GN=16)
        kw[name] = bad
        _raises_shape(ssd.ssd_conv1d_fwd, name, **kw)
    with pytest.raises(ValueError, match="channels"):
        ssd.ssd_conv1d_fwd(xbc, w, 64, 8)


def test_conv_step_rejects_mismatched_shapes():
    xt = torch.zeros(2, 96)
    w = torch.zeros(96, 4)
    st = torch.zeros(2, 3, 96)
    for name, bad in (("state", torch.zeros(2, 3, 95)), ("w", torch.zeros(95, 4)),
                      ("x", torch.zeros(2, 63)), ("C", torch.zeros(1, 16))):
        kw = dict(state=st, xt=xt, w=w, HP=64, GN=16)
        kw[name] = bad
        _raises_shape(ssd.ssd_conv1d_step, name, **kw)


@pytest.mark.parametrize("name,bad", [
    ("dy", torch.zeros(2, 10, 4, 8)), ("B", torch.zeros(2, 9, 2, 16)),
    ("dh_final", torch.zeros(2, 4, 16, 8)), ("dt", torch.zeros(10, 4)),
])
def test_backward_rejects_mismatched_shapes(name, bad):
    kw = real_args()
    kw["dy"] = torch.zeros(2, 10, 4, 16)
    kw["dh_final"] = torch.zeros(2, 4, 16, 16)
    kw[name] = bad
    _raises_shape(ssd.ssd_chunk_bwd, name, **kw)


def test_packed_rejects_mismatched_shapes():
    H, P, N = 2, 16, 16
    proj = torch.zeros(1, 8, H * (P + 4 * N + 1))
    for name, bad in (("A", torch.zeros(2)), ("h0", torch.zeros(1, 2, 16, 16)),
                      ("y", torch.zeros(1, 8, 2, 8)), ("dt_bias", torch.zeros(3))):
        kw = dict(proj=proj, A=torch.zeros(H, 2), H=H, P=P, N=N)
        kw[name] = bad
        _raises_shape(ssd.ssd_complex_chunk_fwd_packed, name, **kw)
    with pytest.raises(ValueError, match="columns"):
        ssd.ssd_complex_chunk_fwd_packed(proj[..., :-1], torch.zeros(H, 2), H, P, N)


def test_complex_backward_rejects_mismatched_shapes():
    kw = cplx_args()
    kw["dy"] = torch.zeros(1, 8, 2, 16)
    kw["dh_final"] = torch.zeros(1, 2, 16, 16, 2)
    with pytest.raises(ValueError, match="GPU tensor"):
        ssd.ssd_complex_chunk_bwd(**kw)
    for name, bad in (("dy", torch.zeros(1, 8, 2, 8)), ("dh_final", torch.zeros(1, 2, 16, 16)),
                      ("A", torch.zeros(2)), ("C", torch.zeros(1, 8, 2, 15, 2))):
        k2 = dict(kw)
        k2[name] = bad
        _raises_shape(ssd.ssd_complex_chunk_bwd, name, **k2)


def test_varlen_binding_checks_shapes_before_the_call():
    """cu_seqlens must be host memory and agree with x's token rows; the
    per-sequence states must have nseq rows."""
    import numpy as np
    x = torch.zeros((9, 4, 64), dtype=torch.bfloat16)
    B = torch.zeros((9, 1, 128), dtype=torch.bfloat16)
    dt = torch.zeros((9, 4))
    A = torch.zeros(4)
    with pytest.raises(ValueError, match="cu_seqlens"):
        ssd.ssd_chunk_fwd_varlen(x, dt, A, B, B, [0, 5, 8])
    with pytest.raises(ValueError, match="h0"):
        ssd.ssd_chunk_fwd_varlen(x, dt, A, B, B, np.array([0, 5, 9]),
                                 h0=torch.zeros((3, 4, 64, 128)))
    with pytest.raises(ValueError, match="at least 2"):
        ssd.ssd_chunk_fwd_varlen(x, dt, A, B, B, [9])
