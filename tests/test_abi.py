"""CPU checks of the C-ABI library: it loads, exports every function that
include/ssd.h declares, and rejects bad arguments before any HIP call (these
tests pass host pointers that are never dereferenced, on a machine with or
without a GPU)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import selective_state_space_09_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("ssd_chunk_fwd", "ssd_complex_chunk_fwd", "ssd_step_decode",
              "ssd_complex_step_decode", "ssd_workspace_size", "ssd_last_error",
              "ssd_abi_version", "ssd_conv1d_fwd", "ssd_conv1d_step", "ssd_chunk_bwd",
              "ssd_bwd_workspace_size", "ssd_complex_chunk_fwd_packed"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ssd.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_abi_version():
    assert ssd.lib().ssd_abi_version() == 1


# a 256-byte aligned host buffer stands in for device memory: validation
# rejects the call before anything touches it
_buf = np.zeros(1 << 16, np.uint8)
_base = (_buf.ctypes.data + 255) // 256 * 256
GOOD = ctypes.c_void_p(_base)
MISALIGNED = ctypes.c_void_p(_base + 4)


def _real_call(**over):
    a = dict(x=GOOD, dt=GOOD, A=GOOD, B=GOOD, C=GOOD, D=None, dt_bias=None, dt_min=0.0,
             dt_max=math.inf, h0=None, y=GOOD, h_final=None, Bsz=1, T=64, H=2, P=16, G=1,
             N=16, chunk=64, dtype=0, ws=GOOD, wsb=1 << 30, stream=None)
    a.update(over)
    L = ssd.lib()
    rc = L.ssd_chunk_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["dt_bias"],
                         a["dt_min"], a["dt_max"], a["h0"], a["y"], a["h_final"], a["Bsz"],
                         a["T"], a["H"], a["P"], a["G"], a["N"], a["chunk"], a["dtype"],
                         a["ws"], a["wsb"], a["stream"])
    return rc, L.ssd_last_error().decode()


@pytest.mark.parametrize("over,code,needle", [
    (dict(x=None), ssd.SSD_EINVAL, "x is NULL"),
    (dict(y=None), ssd.SSD_EINVAL, "y is NULL"),
    (dict(B=MISALIGNED), ssd.SSD_EINVAL, "aligned"),
    (dict(H=3, G=2), ssd.SSD_EINVAL, "multiple"),
    (dict(Bsz=0), ssd.SSD_EINVAL, "positive"),
    (dict(T=-1), ssd.SSD_EINVAL, "positive"),
    (dict(P=24), ssd.SSD_EUNSUPPORTED, "P=24"),
    (dict(N=256), ssd.SSD_EUNSUPPORTED, "N=256"),
    (dict(chunk=48), ssd.SSD_EUNSUPPORTED, "chunk=48"),
    (dict(dtype=7), ssd.SSD_EUNSUPPORTED, "dtype"),
    (dict(dt_min=0.5, dt_max=0.1), ssd.SSD_EINVAL, "dt_min"),
    (dict(dt_min=float("nan")), ssd.SSD_EINVAL, "dt_min"),
    (dict(ws=None), ssd.SSD_EINVAL, "workspace"),
    (dict(wsb=16), ssd.SSD_EWORKSPACE, "workspace"),
])
def test_real_forward_rejects(over, code, needle):
    rc, msg = _real_call(**over)
    assert rc == code
    assert needle in msg


def test_complex_forward_rejects():
    L = ssd.lib()
    rc = L.ssd_complex_chunk_fwd(GOOD, GOOD, GOOD, GOOD, GOOD, None, 0.0, 1.0, None, GOOD, None,
                                 1, 64, 2, 16, 2, 128, 64, GOOD, 1 << 30, None)
    assert rc == ssd.SSD_EUNSUPPORTED and "N=128" in L.ssd_last_error().decode()
    rc = L.ssd_complex_chunk_fwd(GOOD, GOOD, MISALIGNED, GOOD, GOOD, None, 0.0, 1.0, None, GOOD,
                                 None, 1, 64, 2, 16, 2, 64, 64, GOOD, 1 << 30, None)
    assert rc == ssd.SSD_EINVAL and "A" in L.ssd_last_error().decode()


def test_decode_rejects():
    L = ssd.lib()
    rc = L.ssd_step_decode(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, None, 0.0, 1.0, GOOD,
                           2, 4, 16, 3, 128, None)
    assert rc == ssd.SSD_EINVAL and "multiple" in L.ssd_last_error().decode()
    rc = L.ssd_step_decode(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, None, 0.0, 1.0, GOOD,
                           2, 4, 16, 1, 100, None)
    assert rc == ssd.SSD_EUNSUPPORTED
    rc = L.ssd_step_decode(None, GOOD, GOOD, GOOD, GOOD, GOOD, None, None, 0.0, 1.0, GOOD,
                           2, 4, 16, 1, 128, None)
    assert rc == ssd.SSD_EINVAL and "h is NULL" in L.ssd_last_error().decode()


def test_complex_decode_rejects():
    """Argument checks of the complex decode step run before any HIP call."""
    L = ssd.lib()
    rc = L.ssd_complex_step_decode(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, 0.0, 1.0, GOOD,
                                   2, 4, 16, 3, 64, None)
    assert rc == ssd.SSD_EINVAL and "multiple" in L.ssd_last_error().decode()
    rc = L.ssd_complex_step_decode(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, 0.0, 1.0, GOOD,
                                   2, 4, 16, 1, 256, None)
    assert rc == ssd.SSD_EUNSUPPORTED and "N=256" in L.ssd_last_error().decode()
    rc = L.ssd_complex_step_decode(None, GOOD, GOOD, GOOD, GOOD, GOOD, None, 0.0, 1.0, GOOD,
                                   2, 4, 16, 1, 64, None)
    assert rc == ssd.SSD_EINVAL and "h is NULL" in L.ssd_last_error().decode()
    rc = L.ssd_complex_step_decode(GOOD, GOOD, GOOD, GOOD, ctypes.c_void_p(_base + 8), GOOD, None, 0.0, 1.0, GOOD,
                                   2, 4, 16, 1, 64, None)
    assert rc == ssd.SSD_EINVAL and "B is not 16-byte aligned" in L.ssd_last_error().decode()
    rc = L.ssd_complex_step_decode(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, 1.0, 0.5, GOOD,
                                   2, 4, 16, 1, 64, None)
    assert rc == ssd.SSD_EINVAL
    rc = L.ssd_complex_step_decode(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, 0.0, 1.0, GOOD,
                                   0, 4, 16, 1, 64, None)
    assert rc == ssd.SSD_EINVAL and "positive" in L.ssd_last_error().decode()


def _conv(**over):
    a = dict(xbc=GOOD, ld=48, w=GOOD, bias=None, si=None, act=1, x=GOOD, B=GOOD, C=GOOD,
             so=None, Bsz=2, T=40, HP=32, GN=8, K=4, dtype=1)
    a.update(over)
    L = ssd.lib()
    rc = L.ssd_conv1d_fwd(a["xbc"], a["ld"], a["w"], a["bias"], a["si"], a["act"], a["x"],
                          a["B"], a["C"], a["so"], a["Bsz"], a["T"], a["HP"], a["GN"], a["K"],
                          a["dtype"], None)
    return rc, L.ssd_last_error().decode()


def test_conv_rejects():
    """Argument checks of the convolution run before any HIP call."""
    assert _conv(K=3) == (ssd.SSD_EUNSUPPORTED, "K=3: only kernel size 4 is built")
    rc, msg = _conv(HP=36)  # not a multiple of 8 for bf16
    assert rc == ssd.SSD_EUNSUPPORTED and "multiples of 8" in msg
    rc, msg = _conv(ld=40)  # ld < HP + 2*GN = 48
    assert rc == ssd.SSD_EINVAL and "smaller" in msg
    rc, msg = _conv(ld=52)
    assert rc == ssd.SSD_EINVAL and "multiple of 8" in msg
    rc, msg = _conv(act=2)
    assert rc == ssd.SSD_EINVAL and "act" in msg
    rc, msg = _conv(dtype=5)
    assert rc == ssd.SSD_EUNSUPPORTED
    rc, msg = _conv(T=-1)
    assert rc == ssd.SSD_EINVAL
    rc, msg = _conv(x=MISALIGNED)
    assert rc == ssd.SSD_EINVAL and "x is not 16-byte aligned" in msg
    rc, msg = _conv(w=None)
    assert rc == ssd.SSD_EINVAL and "w is NULL" in msg
    # the two states may not overlap (here: same buffer)
    rc, msg = _conv(si=GOOD, so=ctypes.c_void_p(_base + 256))
    assert rc == ssd.SSD_EINVAL and "overlap" in msg
    # rows of one batch entry past 4 GiB
    rc, msg = _conv(T=1 << 26, ld=64)
    assert rc == ssd.SSD_EUNSUPPORTED
    L = ssd.lib()
    rc = L.ssd_conv1d_step(GOOD, GOOD, 48, GOOD, None, 1, GOOD, GOOD, GOOD, 2, 30, 9, 4, None)
    assert rc == ssd.SSD_EUNSUPPORTED and "multiples of 4" in L.ssd_last_error().decode()
    rc = L.ssd_conv1d_step(None, GOOD, 48, GOOD, None, 1, GOOD, GOOD, GOOD, 2, 32, 8, 4, None)
    assert rc == ssd.SSD_EINVAL and "state is NULL" in L.ssd_last_error().decode()


def test_workspace_size():
    L = ssd.lib()
    # BitMamba layer shape: states (2, 8, 64, 64, 128) fp32 + decays + the
    # per-token (exponent, step) pairs (2, 8, 64, 256) of the real form
    n = ssd.ssd_workspace_size(2, 2048, 64, 64, 1, 128, 256, False)
    assert n >= 2 * 8 * 64 * 64 * 128 * 4 + 2 * 64 * 8 * 8 + 2 * 8 * 64 * 256 * 8
    assert n % 256 == 0
    # complex doubles the state width
    nc = ssd.ssd_workspace_size(8, 2048, 16, 64, 16, 64, 256, True)
    assert nc >= 8 * 8 * 16 * 64 * 128 * 4
    assert ssd.ssd_workspace_size(1, 10, 2, 16, 1, 16, 48, False) == 0
    assert L.ssd_workspace_size(1, 0, 2, 16, 1, 16, 64, 0) > 0


def test_python_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 16)
    with pytest.raises(ValueError, match="GPU"):
        ssd.ssd_chunk_fwd(x, torch.zeros(1, 4, 2), torch.zeros(2), torch.zeros(1, 4, 1, 16),
                          torch.zeros(1, 4, 1, 16))


def test_complex_packed_rejects():
    """Argument checks of the packed-row complex forward (H=2, P=16, N=16:
    rows need H*(P+4N+1) = 162 floats)."""
    L = ssd.lib()

    def call(ld=164, proj=GOOD, H=2, P=16, N=16, chunk=64):
        rc = L.ssd_complex_chunk_fwd_packed(proj, ld, GOOD, None, 0.0, 1.0, None, GOOD, None,
                                            1, 64, H, P, N, chunk, GOOD, 1 << 30, None)
        return rc, L.ssd_last_error().decode()
    rc, msg = call(ld=160)
    assert rc == ssd.SSD_EINVAL and "smaller" in msg
    rc, msg = call(ld=162)
    assert rc == ssd.SSD_EINVAL and "multiple of 4" in msg
    rc, msg = call(proj=MISALIGNED)
    assert rc == ssd.SSD_EINVAL and "proj is not 16-byte aligned" in msg
    rc, msg = call(N=128)
    assert rc == ssd.SSD_EUNSUPPORTED


def test_noalloc_rejects_shapes_beyond_its_scratch_without_device_use():
    """The allocation-free forward refuses a shape whose workspace exceeds its
    64 MiB scratch array, before any HIP call (this host has no GPU), and
    names the limit."""
    L = ssd.lib()
    # B1 T65536 H64 P64 N128 (the long workload): ~540 MB of chunk states
    rc = L.ssd_chunk_fwd_noalloc(GOOD, GOOD, GOOD, GOOD, GOOD, None, None, 0.0, 1.0, None, GOOD,
                                 None, 1, 65536, 64, 64, 1, 128, 256, ssd.SSD_BF16, None)
    msg = L.ssd_last_error().decode()
    assert rc == ssd.SSD_EWORKSPACE, (rc, msg)
    assert str(64 << 20) in msg and "scratch" in msg
    assert ssd.ssd_workspace_size(1, 65536, 64, 64, 1, 128, 256) > ssd.NOALLOC_SCRATCH_BYTES
    # the same argument checks as ssd_chunk_fwd run first
    rc = L.ssd_chunk_fwd_noalloc(GOOD, GOOD, GOOD, GOOD, GOOD, None, None, 0.0, 1.0, None, GOOD,
                                 None, 1, 64, 2, 16, 1, 16, 48, ssd.SSD_BF16, None)
    assert rc == ssd.SSD_EUNSUPPORTED
    rc = L.ssd_chunk_fwd_noalloc(GOOD, GOOD, GOOD, MISALIGNED, GOOD, None, None, 0.0, 1.0, None,
                                 GOOD, None, 1, 64, 2, 16, 1, 16, 64, ssd.SSD_BF16, None)
    assert rc == ssd.SSD_EINVAL and "B is not 16-byte aligned" in L.ssd_last_error().decode()


def test_noalloc_scratch_covers_the_bitmamba_shape():
    """The BitMamba layer shape (B2 T2048 H64 P64 N128, chunk 256) fits the
    allocation-free forward's scratch array."""
    assert ssd.ssd_workspace_size(2, 2048, 64, 64, 1, 128, 256) <= ssd.NOALLOC_SCRATCH_BYTES


def test_f32_and_complex_backward_rejects_without_device_use():
    """Argument checks of the float32 and complex backward run before any HIP
    call (this host has no GPU): chunk must be 64, the (P, N) sets are
    enforced, the workspace size is checked, pointers must be aligned."""
    L = ssd.lib()

    def f32(chunk=64, P=64, N=128, ws=1 << 40, B=GOOD):
        rc = L.ssd_chunk_bwd(GOOD, GOOD, GOOD, B, GOOD, None, None, 0.0, 1.0, None, GOOD, None,
                             GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None,
                             1, 64, 2, P, 1, N, chunk, ssd.SSD_F32, GOOD, ws, None)
        return rc, L.ssd_last_error().decode()
    rc, msg = f32(chunk=256)
    assert rc == ssd.SSD_EUNSUPPORTED and "chunk=256" in msg
    rc, msg = f32(N=16)
    assert rc == ssd.SSD_EUNSUPPORTED and "fp32 backward" in msg
    rc, msg = f32(ws=16)
    assert rc == ssd.SSD_EWORKSPACE
    rc, msg = f32(B=MISALIGNED)
    assert rc == ssd.SSD_EINVAL and "B is not 16-byte aligned" in msg
    assert ssd.ssd_bwd_workspace_size_f32(1, 64, 2, 64, 1, 128) > 0

    def cplx(chunk=64, P=64, N=64, ws=1 << 40, A=GOOD):
        rc = L.ssd_complex_chunk_bwd(GOOD, GOOD, A, GOOD, GOOD, None, 0.0, 1.0, None, GOOD, None,
                                     GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None,
                                     1, 64, 2, P, 2, N, chunk, GOOD, ws, None)
        return rc, L.ssd_last_error().decode()
    rc, msg = cplx(chunk=128)
    assert rc == ssd.SSD_EUNSUPPORTED and "chunk=128" in msg
    rc, msg = cplx(P=128)
    assert rc == ssd.SSD_EUNSUPPORTED and "complex backward" in msg
    rc, msg = cplx(N=128)
    assert rc == ssd.SSD_EUNSUPPORTED
    rc, msg = cplx(ws=16)
    assert rc == ssd.SSD_EWORKSPACE
    assert ssd.ssd_complex_bwd_workspace_size(1, 64, 2, 64, 2, 64) > 0


def test_varlen_rejects_without_device_use():
    """The variable-length forward checks cu_seqlens (a host array) and the
    other arguments before any HIP call (this host has no GPU)."""
    import numpy as np
    L = ssd.lib()

    def call(cu, dtype=ssd.SSD_BF16, ws=1 << 40, chunk=256, x=GOOD):
        cu = np.ascontiguousarray(cu, np.int32)
        rc = L.ssd_chunk_fwd_varlen(x, GOOD, GOOD, GOOD, GOOD, None, None, 0.0, 1.0, None, GOOD, None,
                                    cu.ctypes.data_as(ctypes.c_void_p), cu.size - 1, 4, 64, 1, 128,
                                    chunk, dtype, GOOD, ws, None)
        return rc, L.ssd_last_error().decode()
    rc, msg = call([1, 5, 9])
    assert rc == ssd.SSD_EINVAL and "cu_seqlens[0]" in msg
    rc, msg = call([0, 5, 3])
    assert rc == ssd.SSD_EINVAL and "non-decreasing" in msg
    rc, msg = call([0, 5, 9], dtype=ssd.SSD_F32)
    assert rc == ssd.SSD_EUNSUPPORTED and "bfloat16" in msg
    rc, msg = call([0, 5, 9], ws=16)
    assert rc == ssd.SSD_EWORKSPACE
    rc, msg = call([0, 5, 9], chunk=48)
    assert rc == ssd.SSD_EUNSUPPORTED and "chunk=48" in msg
    rc, msg = call([0, 5, 9], x=MISALIGNED)
    assert rc == ssd.SSD_EINVAL and "x is not 16-byte aligned" in msg
    rc = L.ssd_chunk_fwd_varlen(GOOD, GOOD, GOOD, GOOD, GOOD, None, None, 0.0, 1.0, None, GOOD, None,
                                None, 2, 4, 64, 1, 128, 256, ssd.SSD_BF16, GOOD, 1 << 40, None)
    assert rc == ssd.SSD_EINVAL and "cu_seqlens is NULL" in L.ssd_last_error().decode()
    assert ssd.ssd_varlen_workspace_size([0, 5, 9], 4, 64, 1, 128, 256) > 0
    assert ssd.ssd_varlen_workspace_size([0, 5, 3], 4, 64, 1, 128, 256) == 0
    # the segment table grows with the number of sequences, not only with Ttot
    one = ssd.ssd_varlen_workspace_size([0, 512], 4, 64, 1, 128, 256)
    many = ssd.ssd_varlen_workspace_size([0] + list(range(1, 513)), 4, 64, 1, 128, 256)
    assert many > one


def test_conv_varlen_rejects_without_device_use():
    import numpy as np
    L = ssd.lib()

    def call(cu, ws=1 << 20, K=4, x=GOOD):
        cu = np.ascontiguousarray(cu, np.int32)
        rc = L.ssd_conv1d_fwd_varlen(x, 384, GOOD, None, None, 1, GOOD, GOOD, GOOD, None,
                                     cu.ctypes.data_as(ctypes.c_void_p), cu.size - 1, 256, 64, K,
                                     ssd.SSD_BF16, GOOD, ws, None)
        return rc, L.ssd_last_error().decode()
    rc, msg = call([2, 5])
    assert rc == ssd.SSD_EINVAL and "cu_seqlens[0]" in msg
    rc, msg = call([0, 5, 4])
    assert rc == ssd.SSD_EINVAL and "non-decreasing" in msg
    rc, msg = call([0, 5, 9], ws=0)
    assert rc == ssd.SSD_EWORKSPACE
    rc, msg = call([0, 5, 9], K=3)
    assert rc == ssd.SSD_EUNSUPPORTED
    rc, msg = call([0, 5, 9], x=MISALIGNED)
    assert rc == ssd.SSD_EINVAL and "xbc" in msg
    assert ssd.lib().ssd_conv1d_varlen_workspace_size(3) >= 16
    assert ssd.lib().ssd_conv1d_varlen_workspace_size(0) == 0
