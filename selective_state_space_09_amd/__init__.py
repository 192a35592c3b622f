"""MI355X (gfx950) chunked selective state-space (SSD) scan.

Python binding of the C ABI in ``include/ssd.h`` (library ``libssd.so`` in
this package).  The functions keep the C names and only marshal arguments:
tensors must already live on the GPU; PyTorch provides device memory and the
current stream, every step of the scan runs in the library's HIP kernels.
There is no CPU path: without the built library every call raises.
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd.so")

SSD_OK, SSD_EINVAL, SSD_EUNSUPPORTED, SSD_EWORKSPACE, SSD_EHIP = 0, 1, 2, 3, 4
SSD_F32, SSD_BF16 = 0, 1

_lib = None


class SSDError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"ssd error {code}: {msg}")
        self.code = code


def lib():
    """The loaded C library (ctypes), with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.ssd_abi_version.restype = I
    L.ssd_abi_version.argtypes = []
    L.ssd_last_error.restype = ctypes.c_char_p
    L.ssd_last_error.argtypes = []
    L.ssd_workspace_size.restype = S
    L.ssd_workspace_size.argtypes = [I] * 8
    L.ssd_chunk_fwd.restype = I
    L.ssd_chunk_fwd.argtypes = [P, P, P, P, P, P, P, F, F, P, P, P,
                                I, I, I, I, I, I, I, I, P, S, P]
    L.ssd_complex_chunk_fwd.restype = I
    L.ssd_complex_chunk_fwd.argtypes = [P, P, P, P, P, P, F, F, P, P, P,
                                        I, I, I, I, I, I, I, P, S, P]
    L.ssd_chunk_fwd_noalloc.restype = I
    L.ssd_chunk_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, F, F, P, P, P,
                                        I, I, I, I, I, I, I, I, P]
    L.ssd_chunk_fwd_ev.restype = I
    L.ssd_chunk_fwd_ev.argtypes = L.ssd_chunk_fwd.argtypes + [P]
    L.ssd_varlen_workspace_size.restype = S
    L.ssd_varlen_workspace_size.argtypes = [P, I, I, I, I, I, I]
    L.ssd_chunk_fwd_varlen.restype = I
    L.ssd_chunk_fwd_varlen.argtypes = [P, P, P, P, P, P, P, F, F, P, P, P,
                                       P, I, I, I, I, I, I, I, P, S, P]
    L.ssd_chunk_fwd_varlen_ev.restype = I
    L.ssd_chunk_fwd_varlen_ev.argtypes = L.ssd_chunk_fwd_varlen.argtypes + [P]
    L.ssd_complex_chunk_fwd_ev.restype = I
    L.ssd_complex_chunk_fwd_ev.argtypes = L.ssd_complex_chunk_fwd.argtypes + [P]
    L.ssd_step_decode.restype = I
    L.ssd_step_decode.argtypes = [P, P, P, P, P, P, P, P, F, F, P, I, I, I, I, I, P]
    L.ssd_step_decode_ev.restype = I
    L.ssd_step_decode_ev.argtypes = L.ssd_step_decode.argtypes + [P]
    L.ssd_complex_step_decode.restype = I
    L.ssd_complex_step_decode.argtypes = [P, P, P, P, P, P, P, F, F, P, I, I, I, I, I, P]
    L.ssd_complex_step_decode_ev.restype = I
    L.ssd_complex_step_decode_ev.argtypes = L.ssd_complex_step_decode.argtypes + [P]
    LL = ctypes.c_longlong
    L.ssd_complex_chunk_fwd_packed.restype = I
    L.ssd_complex_chunk_fwd_packed.argtypes = [P, LL, P, P, F, F, P, P, P, I, I, I, I, I, I, P, S, P]
    L.ssd_complex_chunk_fwd_packed_ev.restype = I
    L.ssd_complex_chunk_fwd_packed_ev.argtypes = L.ssd_complex_chunk_fwd_packed.argtypes + [P]
    L.ssd_bwd_workspace_size.restype = S
    L.ssd_bwd_workspace_size.argtypes = [I] * 7
    L.ssd_chunk_bwd.restype = I
    L.ssd_chunk_bwd.argtypes = [P, P, P, P, P, P, P, F, F, P, P, P,
                                P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P, S, P]
    L.ssd_chunk_bwd_ev.restype = I
    L.ssd_chunk_bwd_ev.argtypes = L.ssd_chunk_bwd.argtypes + [P]
    L.ssd_bwd_workspace_size_f32.restype = S
    L.ssd_bwd_workspace_size_f32.argtypes = [I] * 6
    L.ssd_complex_bwd_workspace_size.restype = S
    L.ssd_complex_bwd_workspace_size.argtypes = [I] * 6
    L.ssd_complex_chunk_bwd.restype = I
    L.ssd_complex_chunk_bwd.argtypes = [P, P, P, P, P, P, F, F, P, P, P, P, P, P, P, P, P, P,
                                        I, I, I, I, I, I, I, P, S, P]
    L.ssd_complex_chunk_bwd_ev.restype = I
    L.ssd_complex_chunk_bwd_ev.argtypes = L.ssd_complex_chunk_bwd.argtypes + [P]
    L.ssd_conv1d_fwd.restype = I
    L.ssd_conv1d_fwd.argtypes = [P, LL, P, P, P, I, P, P, P, P, I, I, I, I, I, I, P]
    L.ssd_conv1d_varlen_workspace_size.restype = S
    L.ssd_conv1d_varlen_workspace_size.argtypes = [I]
    L.ssd_conv1d_fwd_varlen.restype = I
    L.ssd_conv1d_fwd_varlen.argtypes = [P, LL, P, P, P, I, P, P, P, P, P, I, I, I, I, I, P, S, P]
    L.ssd_conv1d_fwd_varlen_ev.restype = I
    L.ssd_conv1d_fwd_varlen_ev.argtypes = L.ssd_conv1d_fwd_varlen.argtypes + [P]
    L.ssd_conv1d_fwd_ev.restype = I
    L.ssd_conv1d_fwd_ev.argtypes = L.ssd_conv1d_fwd.argtypes + [P]
    L.ssd_linear_fwd.restype = I
    L.ssd_linear_fwd.argtypes = [P, I, P, P, I, I, I, I, P]
    L.ssd_linear_fwd_ev.restype = I
    L.ssd_linear_fwd_ev.argtypes = L.ssd_linear_fwd.argtypes + [P]
    L.ssd_mimo_fwd.restype = I
    L.ssd_mimo_fwd.argtypes = [P, I, P, P, I, I, I, I, I, P]
    L.ssd_conv1d_step.restype = I
    L.ssd_conv1d_step.argtypes = [P, P, LL, P, P, I, P, P, P, I, I, I, I, P]
    L.ssd_conv1d_step_ev.restype = I
    L.ssd_conv1d_step_ev.argtypes = L.ssd_conv1d_step.argtypes + [P]
    _lib = L
    return L


def _check(rc):
    if rc != SSD_OK:
        raise SSDError(rc, lib().ssd_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _expect(t, name, shape, ref=None):
    """Shape (and, given a reference tensor, device) check of an optional
    argument, done before anything reaches the library: a tensor of the wrong
    shape would make the kernels read or write outside its allocation."""
    if t is None:
        return
    shape = tuple(int(s) for s in shape)
    if tuple(t.shape) != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    if ref is not None and t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _ndim(t, name, n):
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _pairs(t):
    return torch.view_as_real(t) if t is not None and t.is_complex() else t


def ssd_abi_version():
    return lib().ssd_abi_version()


def ssd_workspace_size(Bsz, T, H, P, G, N, chunk, is_complex=False):
    return int(lib().ssd_workspace_size(Bsz, T, H, P, G, N, chunk, int(bool(is_complex))))


def _workspace(nbytes, device, workspace):
    if workspace is None:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    return _dev(workspace, "workspace")


def ssd_chunk_fwd(x, dt, A, B, C, D=None, dt_bias=None, dt_min=0.0, dt_max=math.inf,
                  h0=None, chunk=256, y=None, h_final=None, return_final_state=False,
                  workspace=None, stream=None):
    """Real chunked forward.  x (Bsz,T,H,P) and B, C (Bsz,T,G,N) in float32 or
    bfloat16; dt (Bsz,T,H), A/D/dt_bias (H), h0 (Bsz,H,P,N) float32.
    Returns y (and h_final when asked or given)."""
    _ndim(x, "x", 4)
    _ndim(B, "B", 4)
    Bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _expect(B, "B", (Bsz, T, G, N), x)
    _expect(C, "C", (Bsz, T, G, N), x)
    _expect(dt, "dt", (Bsz, T, H), x)
    _expect(A, "A", (H,), x)
    _expect(D, "D", (H,), x)
    _expect(dt_bias, "dt_bias", (H,), x)
    _expect(h0, "h0", (Bsz, H, P, N), x)
    _expect(y, "y", (Bsz, T, H, P), x)
    _expect(h_final, "h_final", (Bsz, H, P, N), x)
    if x.dtype == torch.bfloat16:
        dtype = SSD_BF16
    elif x.dtype == torch.float32:
        dtype = SSD_F32
    else:
        raise TypeError("x must be float32 or bfloat16")
    _dev(x, "x")
    _dev(B, "B", x.dtype)
    _dev(C, "C", x.dtype)
    _dev(dt, "dt", torch.float32)
    _dev(A, "A", torch.float32)
    _dev(D, "D", torch.float32)
    _dev(dt_bias, "dt_bias", torch.float32)
    _dev(h0, "h0", torch.float32)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype)
    if h_final is None and return_final_state:
        h_final = torch.empty((Bsz, H, P, N), dtype=torch.float32, device=x.device)
    _dev(h_final, "h_final", torch.float32)
    nbytes = ssd_workspace_size(Bsz, T, H, P, G, N, chunk, False)
    ws = _workspace(nbytes, x.device, workspace)
    _check(lib().ssd_chunk_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                               _ptr(dt_bias), float(dt_min), float(dt_max), _ptr(h0),
                               _ptr(y), _ptr(h_final), Bsz, T, H, P, G, N, chunk, dtype,
                               _ptr(ws), ws.numel(), _stream(stream)))
    return (y, h_final) if h_final is not None else y


def _cu_host(cu_seqlens):
    """cu_seqlens as a contiguous host int32 array (the library reads it on
    the host)."""
    import numpy as np
    if isinstance(cu_seqlens, torch.Tensor):
        if cu_seqlens.is_cuda:
            raise ValueError("cu_seqlens must be host memory (a list, numpy array or CPU tensor)")
        cu_seqlens = cu_seqlens.numpy()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int32)
    if cu.ndim != 1 or cu.size < 2:
        raise ValueError(f"cu_seqlens must be 1-D with at least 2 entries, got shape {cu.shape}")
    return cu


def ssd_varlen_workspace_size(cu_seqlens, H, P, G, N, chunk):
    cu = _cu_host(cu_seqlens)
    return int(lib().ssd_varlen_workspace_size(cu.ctypes.data_as(ctypes.c_void_p), cu.size - 1,
                                               H, P, G, N, chunk))


def ssd_chunk_fwd_varlen(x, dt, A, B, C, cu_seqlens, D=None, dt_bias=None, dt_min=0.0,
                         dt_max=math.inf, h0=None, chunk=256, y=None, h_final=None,
                         return_final_state=False, workspace=None, stream=None, events=None):
    """Variable-length batch of the real forward: x (Ttot,H,P) and B, C
    (Ttot,G,N) bfloat16, dt (Ttot,H), sequence b on the rows cu_seqlens[b] ..
    cu_seqlens[b+1]-1 (cu_seqlens a host array of nseq+1 ints), h0 and
    h_final (nseq,H,P,N) float32.  Returns y (and h_final when asked or
    given)."""
    cu = _cu_host(cu_seqlens)
    nseq = cu.size - 1
    _ndim(x, "x", 3)
    _ndim(B, "B", 3)
    Ttot, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    if int(cu[-1]) != Ttot:
        raise ValueError(f"cu_seqlens[-1] = {int(cu[-1])} but x has {Ttot} token rows")
    _expect(B, "B", (Ttot, G, N), x)
    _expect(C, "C", (Ttot, G, N), x)
    _expect(dt, "dt", (Ttot, H), x)
    _expect(A, "A", (H,), x)
    _expect(D, "D", (H,), x)
    _expect(dt_bias, "dt_bias", (H,), x)
    _expect(h0, "h0", (nseq, H, P, N), x)
    _expect(y, "y", (Ttot, H, P), x)
    _expect(h_final, "h_final", (nseq, H, P, N), x)
    _dev(x, "x", torch.bfloat16)
    _dev(B, "B", torch.bfloat16)
    _dev(C, "C", torch.bfloat16)
    _dev(dt, "dt", torch.float32)
    _dev(A, "A", torch.float32)
    _dev(D, "D", torch.float32)
    _dev(dt_bias, "dt_bias", torch.float32)
    _dev(h0, "h0", torch.float32)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", torch.bfloat16)
    if h_final is None and return_final_state:
        h_final = torch.empty((nseq, H, P, N), dtype=torch.float32, device=x.device)
    _dev(h_final, "h_final", torch.float32)
    cup = cu.ctypes.data_as(ctypes.c_void_p)
    nbytes = int(lib().ssd_varlen_workspace_size(cup, nseq, H, P, G, N, chunk))
    if nbytes == 0:
        _check(lib().ssd_chunk_fwd_varlen(None, None, None, None, None, None, None, float(dt_min),
                                          float(dt_max), None, None, None, cup, nseq, H, P, G, N,
                                          chunk, SSD_BF16, None, 0, None))
    ws = _workspace(nbytes, x.device, workspace)
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias), float(dt_min),
            float(dt_max), _ptr(h0), _ptr(y), _ptr(h_final), cup, nseq, H, P, G, N, chunk, SSD_BF16,
            _ptr(ws), ws.numel(), _stream(stream))
    if events is None:
        _check(lib().ssd_chunk_fwd_varlen(*args))
    else:
        _check(lib().ssd_chunk_fwd_varlen_ev(*args, events))
    return (y, h_final) if h_final is not None else y


NOALLOC_SCRATCH_BYTES = 64 << 20


def ssd_chunk_fwd_noalloc(x, dt, A, B, C, y, D=None, dt_bias=None, dt_min=0.0,
                          dt_max=math.inf, h0=None, h_final=None, chunk=256, stream=None):
    """ssd_chunk_fwd without a workspace: the library's per-GPU scratch array
    holds the chunk states (shapes whose workspace exceeds 64 MiB are
    rejected).  The caller passes y (and h_final when wanted); nothing is
    allocated.  Calls that overlap on one GPU race on the scratch array."""
    _ndim(x, "x", 4)
    _ndim(B, "B", 4)
    Bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _expect(B, "B", (Bsz, T, G, N), x)
    _expect(C, "C", (Bsz, T, G, N), x)
    _expect(dt, "dt", (Bsz, T, H), x)
    _expect(A, "A", (H,), x)
    _expect(D, "D", (H,), x)
    _expect(dt_bias, "dt_bias", (H,), x)
    _expect(h0, "h0", (Bsz, H, P, N), x)
    _expect(y, "y", (Bsz, T, H, P), x)
    _expect(h_final, "h_final", (Bsz, H, P, N), x)
    if x.dtype == torch.bfloat16:
        dtype = SSD_BF16
    elif x.dtype == torch.float32:
        dtype = SSD_F32
    else:
        raise TypeError("x must be float32 or bfloat16")
    for t, n in ((x, "x"), (B, "B"), (C, "C"), (y, "y")):
        _dev(t, n, x.dtype)
    for t, n in ((dt, "dt"), (A, "A"), (D, "D"), (dt_bias, "dt_bias"), (h0, "h0"),
                 (h_final, "h_final")):
        _dev(t, n, torch.float32)
    _check(lib().ssd_chunk_fwd_noalloc(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                       _ptr(dt_bias), float(dt_min), float(dt_max), _ptr(h0),
                                       _ptr(y), _ptr(h_final), Bsz, T, H, P, G, N, chunk, dtype,
                                       _stream(stream)))
    return (y, h_final) if h_final is not None else y


def ssd_complex_chunk_fwd(x, dt, A, B, C, dt_bias=None, dt_min=0.0, dt_max=math.inf,
                          h0=None, chunk=256, y=None, h_final=None,
                          return_final_state=False, workspace=None, stream=None):
    """Complex chunked forward.  x (Bsz,T,H,P) float32; A (H) complex64 or
    (H,2) float32; B, C (Bsz,T,G,N) complex64 or (...,N,2) float32; h0
    likewise.  Returns y = Re(h C) (and h_final as (Bsz,H,P,N,2) float32)."""
    A, B, C, h0 = _pairs(A), _pairs(B), _pairs(C), _pairs(h0)
    y, h_final = _pairs(y), _pairs(h_final)
    _ndim(x, "x", 4)
    _ndim(B, "B", 5)
    Bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _expect(B, "B", (Bsz, T, G, N, 2), x)
    _expect(C, "C", (Bsz, T, G, N, 2), x)
    _expect(dt, "dt", (Bsz, T, H), x)
    _expect(A, "A", (H, 2), x)
    _expect(dt_bias, "dt_bias", (H,), x)
    _expect(h0, "h0", (Bsz, H, P, N, 2), x)
    _expect(y, "y", (Bsz, T, H, P), x)
    _expect(h_final, "h_final", (Bsz, H, P, N, 2), x)
    _dev(x, "x", torch.float32)
    _dev(dt, "dt", torch.float32)
    _dev(A, "A", torch.float32)
    _dev(B, "B", torch.float32)
    _dev(C, "C", torch.float32)
    _dev(dt_bias, "dt_bias", torch.float32)
    _dev(h0, "h0", torch.float32)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", torch.float32)
    if h_final is None and return_final_state:
        h_final = torch.empty((Bsz, H, P, N, 2), dtype=torch.float32, device=x.device)
    h_final = _pairs(h_final)
    _dev(h_final, "h_final", torch.float32)
    nbytes = ssd_workspace_size(Bsz, T, H, P, G, N, chunk, True)
    ws = _workspace(nbytes, x.device, workspace)
    _check(lib().ssd_complex_chunk_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                       _ptr(dt_bias), float(dt_min), float(dt_max),
                                       _ptr(h0), _ptr(y), _ptr(h_final), Bsz, T, H, P, G,
                                       N, chunk, _ptr(ws), ws.numel(), _stream(stream)))
    return (y, h_final) if h_final is not None else y


def ssd_step_decode(h, x, dt, A, B, C, D=None, dt_bias=None, dt_min=0.0, dt_max=math.inf,
                    y=None, stream=None):
    """One decode step, state h (Bsz,H,P,N) float32 updated in place; x
    (Bsz,H,P), dt (Bsz,H), B/C (Bsz,G,N).  Returns y (Bsz,H,P)."""
    _ndim(h, "h", 4)
    _ndim(B, "B", 3)
    Bsz, H, P, N = h.shape
    G = B.shape[1]
    _expect(x, "x", (Bsz, H, P), h)
    _expect(dt, "dt", (Bsz, H), h)
    _expect(A, "A", (H,), h)
    _expect(B, "B", (Bsz, G, N), h)
    _expect(C, "C", (Bsz, G, N), h)
    _expect(D, "D", (H,), h)
    _expect(dt_bias, "dt_bias", (H,), h)
    _expect(y, "y", (Bsz, H, P), h)
    for t, n in ((h, "h"), (x, "x"), (dt, "dt"), (A, "A"), (B, "B"), (C, "C")):
        _dev(t, n, torch.float32)
    _dev(D, "D", torch.float32)
    _dev(dt_bias, "dt_bias", torch.float32)
    if y is None:
        y = torch.empty((Bsz, H, P), dtype=torch.float32, device=h.device)
    _dev(y, "y", torch.float32)
    _check(lib().ssd_step_decode(_ptr(h), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                 _ptr(D), _ptr(dt_bias), float(dt_min), float(dt_max),
                                 _ptr(y), Bsz, H, P, G, N, _stream(stream)))
    return y


def ssd_complex_step_decode(h, x, dt, A, B, C, dt_bias=None, dt_min=0.0, dt_max=math.inf,
                            y=None, stream=None):
    """One complex decode step, state h (Bsz,H,P,N,2) float32 (re, im) updated
    in place; x (Bsz,H,P), dt (Bsz,H), A (H,2), B/C (Bsz,G,N,2).  Returns
    y = Re(C . h) (Bsz,H,P)."""
    h, A, B, C = _pairs(h), _pairs(A), _pairs(B), _pairs(C)
    _ndim(h, "h", 5)
    _ndim(B, "B", 4)
    Bsz, H, P, N, _ = h.shape
    G = B.shape[1]
    _expect(h, "h", (Bsz, H, P, N, 2))
    _expect(x, "x", (Bsz, H, P), h)
    _expect(dt, "dt", (Bsz, H), h)
    _expect(A, "A", (H, 2), h)
    _expect(B, "B", (Bsz, G, N, 2), h)
    _expect(C, "C", (Bsz, G, N, 2), h)
    _expect(dt_bias, "dt_bias", (H,), h)
    _expect(y, "y", (Bsz, H, P), h)
    for t, n in ((h, "h"), (x, "x"), (dt, "dt"), (A, "A"), (B, "B"), (C, "C")):
        _dev(t, n, torch.float32)
    _dev(dt_bias, "dt_bias", torch.float32)
    if y is None:
        y = torch.empty((Bsz, H, P), dtype=torch.float32, device=h.device)
    _dev(y, "y", torch.float32)
    _check(lib().ssd_complex_step_decode(_ptr(h), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                         _ptr(dt_bias), float(dt_min), float(dt_max), _ptr(y),
                                         Bsz, H, P, G, N, _stream(stream)))
    return y


def _rows(t, name, ndim):
    """A GPU tensor whose last dimension is contiguous and whose rows are
    evenly spaced (a column slice of a wider row-major tensor is accepted).
    Returns the row stride in elements."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() == ndim and t.numel() == 0:
        return t.shape[-1]  # nothing is read
    if t.dim() != ndim or t.stride(-1) != 1:
        raise ValueError(f"{name} must have {ndim} dims with a contiguous last dim")
    ld = t.stride(-2)
    if ndim == 3 and t.shape[0] > 1 and t.shape[1] > 0 and t.stride(0) != t.shape[1] * ld:
        raise ValueError(f"{name}: batch entries must follow each other (stride T*ld)")
    return ld


def ssd_conv1d_fwd_varlen(xbc, w, HP, GN, cu_seqlens, bias=None, state_in=None, act=1, x=None,
                          B=None, C=None, state_out=None, workspace=None, stream=None):
    """The convolution over a variable-length batch: xbc (Ttot,Ch) rows (or a
    column slice of wider rows) of nseq packed sequences, sequence b on rows
    cu_seqlens[b] .. cu_seqlens[b+1]-1 (cu_seqlens a host array of nseq+1
    ints); state_in/state_out (nseq,3,Ch).  Returns (x, B, C, state_out)."""
    cu = _cu_host(cu_seqlens)
    nseq = cu.size - 1
    _ndim(xbc, "xbc", 2)
    Ttot, Ch = xbc.shape
    if int(cu[-1]) != Ttot:
        raise ValueError(f"cu_seqlens[-1] = {int(cu[-1])} but xbc has {Ttot} token rows")
    if Ch != HP + 2 * GN:
        raise ValueError(f"xbc has {Ch} channels, HP + 2*GN = {HP + 2 * GN}")
    _ndim(w, "w", 2)
    K = w.shape[1]
    _expect(w, "w", (Ch, K), xbc)
    _expect(bias, "bias", (Ch,), xbc)
    _expect(state_in, "state_in", (nseq, K - 1, Ch), xbc)
    _expect(state_out, "state_out", (nseq, K - 1, Ch), xbc)
    _expect(x, "x", (Ttot, HP), xbc)
    _expect(B, "B", (Ttot, GN), xbc)
    _expect(C, "C", (Ttot, GN), xbc)
    ld = _rows(xbc, "xbc", 2)
    if xbc.dtype == torch.bfloat16:
        dtype = SSD_BF16
    elif xbc.dtype == torch.float32:
        dtype = SSD_F32
    else:
        raise TypeError("xbc must be float32 or bfloat16")
    _dev(w, "w", torch.float32)
    _dev(bias, "bias", torch.float32)
    _dev(state_in, "state_in", torch.float32)
    dev = xbc.device
    x = torch.empty((Ttot, HP), dtype=xbc.dtype, device=dev) if x is None else x
    B = torch.empty((Ttot, GN), dtype=xbc.dtype, device=dev) if B is None else B
    C = torch.empty((Ttot, GN), dtype=xbc.dtype, device=dev) if C is None else C
    if state_out is None:
        state_out = torch.empty((nseq, K - 1, Ch), dtype=torch.float32, device=dev)
    for t, n in ((x, "x"), (B, "B"), (C, "C")):
        _dev(t, n, xbc.dtype)
    _dev(state_out, "state_out", torch.float32)
    ws = _workspace(int(lib().ssd_conv1d_varlen_workspace_size(nseq)), dev, workspace)
    _check(lib().ssd_conv1d_fwd_varlen(_ptr(xbc), ld, _ptr(w), _ptr(bias), _ptr(state_in), int(act),
                                       _ptr(x), _ptr(B), _ptr(C), _ptr(state_out),
                                       cu.ctypes.data_as(ctypes.c_void_p), nseq, HP, GN, K, dtype,
                                       _ptr(ws), ws.numel(), _stream(stream)))
    return x, B, C, state_out


def ssd_conv1d_fwd(xbc, w, HP, GN, bias=None, state_in=None, act=1, x=None, B=None, C=None,
                   state_out=None, stream=None):
    """Depthwise causal convolution (kernel 4) over the Ch = HP + 2*GN
    channels of xbc (Bsz,T,Ch) -- contiguous or a column slice of wider rows,
    float32 or bfloat16 -- split into x (Bsz,T,HP), B and C (Bsz,T,GN).
    w (Ch,4), bias (Ch), state_in/state_out (Bsz,3,Ch) float32.  act 1 = SiLU.
    Returns (x, B, C, state_out); state_out is allocated when not given."""
    _ndim(xbc, "xbc", 3)
    Bsz, T, Ch = xbc.shape
    if Ch != HP + 2 * GN:
        raise ValueError(f"xbc has {Ch} channels, HP + 2*GN = {HP + 2 * GN}")
    _ndim(w, "w", 2)
    K = w.shape[1]
    _expect(w, "w", (Ch, K), xbc)
    _expect(bias, "bias", (Ch,), xbc)
    _expect(state_in, "state_in", (Bsz, K - 1, Ch), xbc)
    _expect(state_out, "state_out", (Bsz, K - 1, Ch), xbc)
    _expect(x, "x", (Bsz, T, HP), xbc)
    _expect(B, "B", (Bsz, T, GN), xbc)
    _expect(C, "C", (Bsz, T, GN), xbc)
    ld = _rows(xbc, "xbc", 3)
    if xbc.dtype == torch.bfloat16:
        dtype = SSD_BF16
    elif xbc.dtype == torch.float32:
        dtype = SSD_F32
    else:
        raise TypeError("xbc must be float32 or bfloat16")
    _dev(w, "w", torch.float32)
    _dev(bias, "bias", torch.float32)
    _dev(state_in, "state_in", torch.float32)
    dev = xbc.device
    if x is None:
        x = torch.empty((Bsz, T, HP), dtype=xbc.dtype, device=dev)
    if B is None:
        B = torch.empty((Bsz, T, GN), dtype=xbc.dtype, device=dev)
    if C is None:
        C = torch.empty((Bsz, T, GN), dtype=xbc.dtype, device=dev)
    if state_out is None:
        state_out = torch.empty((Bsz, 3, Ch), dtype=torch.float32, device=dev)
    for t, n in ((x, "x"), (B, "B"), (C, "C")):
        _dev(t, n, xbc.dtype)
    _dev(state_out, "state_out", torch.float32)
    _check(lib().ssd_conv1d_fwd(_ptr(xbc), ld, _ptr(w), _ptr(bias), _ptr(state_in), int(act),
                                _ptr(x), _ptr(B), _ptr(C), _ptr(state_out), Bsz, T, HP, GN,
                                w.shape[1], dtype, _stream(stream)))
    return x, B, C, state_out


def ssd_conv1d_step(state, xt, w, HP, GN, bias=None, act=1, x=None, B=None, C=None,
                    stream=None):
    """One decode step of the convolution on the float32 state (Bsz,3,Ch),
    updated in place; xt (Bsz,Ch) float32, contiguous or a column slice.
    Returns x (Bsz,HP), B, C (Bsz,GN) float32."""
    _ndim(xt, "xt", 2)
    _ndim(w, "w", 2)
    Bsz, Ch = xt.shape
    if Ch != HP + 2 * GN:
        raise ValueError(f"xt has {Ch} channels, HP + 2*GN = {HP + 2 * GN}")
    K = w.shape[1]
    _expect(w, "w", (Ch, K), xt)
    _expect(bias, "bias", (Ch,), xt)
    _expect(state, "state", (Bsz, K - 1, Ch), xt)
    _expect(x, "x", (Bsz, HP), xt)
    _expect(B, "B", (Bsz, GN), xt)
    _expect(C, "C", (Bsz, GN), xt)
    _dev(state, "state", torch.float32)
    ld = _rows(xt, "xt", 2)
    if xt.dtype != torch.float32:
        raise TypeError("xt must be float32")
    _dev(w, "w", torch.float32)
    _dev(bias, "bias", torch.float32)
    Bsz = xt.shape[0]
    dev = xt.device
    if x is None:
        x = torch.empty((Bsz, HP), dtype=torch.float32, device=dev)
    if B is None:
        B = torch.empty((Bsz, GN), dtype=torch.float32, device=dev)
    if C is None:
        C = torch.empty((Bsz, GN), dtype=torch.float32, device=dev)
    for t, n in ((x, "x"), (B, "B"), (C, "C")):
        _dev(t, n, torch.float32)
    _check(lib().ssd_conv1d_step(_ptr(state), _ptr(xt), ld, _ptr(w), _ptr(bias), int(act),
                                 _ptr(x), _ptr(B), _ptr(C), Bsz, HP, GN, w.shape[1],
                                 _stream(stream)))
    return x, B, C


def ssd_bwd_workspace_size(Bsz, T, H, P, G, N, chunk):
    return int(lib().ssd_bwd_workspace_size(Bsz, T, H, P, G, N, chunk))


def ssd_bwd_workspace_size_f32(Bsz, T, H, P, G, N):
    return int(lib().ssd_bwd_workspace_size_f32(Bsz, T, H, P, G, N))


def ssd_complex_bwd_workspace_size(Bsz, T, H, P, G, N):
    return int(lib().ssd_complex_bwd_workspace_size(Bsz, T, H, P, G, N))


def ssd_chunk_bwd(x, dt, A, B, C, dy, D=None, dt_bias=None, dt_min=0.0, dt_max=math.inf,
                  h0=None, dh_final=None, chunk=256, want_dh0=True, workspace=None, stream=None):
    """Gradient of sum(dy * y) + <dh_final, h_final> of ssd_chunk_fwd (real
    form; x/B/C/dy all bfloat16, or all float32 with chunk 64).  Returns a
    dict: dx (x's dtype), ddt, dA, dB, dC, dD, ddt_bias and dh0 (float32; dh0
    None unless want_dh0)."""
    _ndim(x, "x", 4)
    _ndim(B, "B", 4)
    Bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _expect(B, "B", (Bsz, T, G, N), x)
    _expect(C, "C", (Bsz, T, G, N), x)
    _expect(dy, "dy", (Bsz, T, H, P), x)
    _expect(dt, "dt", (Bsz, T, H), x)
    _expect(A, "A", (H,), x)
    _expect(D, "D", (H,), x)
    _expect(dt_bias, "dt_bias", (H,), x)
    _expect(h0, "h0", (Bsz, H, P, N), x)
    _expect(dh_final, "dh_final", (Bsz, H, P, N), x)
    xdt = _dcode(x.dtype, "x")
    for t, n in ((x, "x"), (B, "B"), (C, "C"), (dy, "dy")):
        _dev(t, n, torch.bfloat16 if xdt == SSD_BF16 else torch.float32)
    for t, n in ((dt, "dt"), (A, "A")):
        _dev(t, n, torch.float32)
    for t, n in ((D, "D"), (dt_bias, "dt_bias"), (h0, "h0"), (dh_final, "dh_final")):
        _dev(t, n, torch.float32)
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dx=torch.empty_like(x), ddt=torch.empty((Bsz, T, H), **f32),
               dA=torch.empty(H, **f32), dB=torch.empty((Bsz, T, G, N), **f32),
               dC=torch.empty((Bsz, T, G, N), **f32), dD=torch.empty(H, **f32),
               ddt_bias=torch.empty(H, **f32),
               dh0=torch.empty((Bsz, H, P, N), **f32) if want_dh0 else None)
    nbytes = (ssd_bwd_workspace_size(Bsz, T, H, P, G, N, chunk) if xdt == SSD_BF16
              else ssd_bwd_workspace_size_f32(Bsz, T, H, P, G, N))
    ws = _workspace(nbytes, dev, workspace)
    _check(lib().ssd_chunk_bwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                               _ptr(dt_bias), float(dt_min), float(dt_max), _ptr(h0), _ptr(dy),
                               _ptr(dh_final), _ptr(out["dx"]), _ptr(out["ddt"]),
                               _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]),
                               _ptr(out["dD"]), _ptr(out["ddt_bias"]), _ptr(out["dh0"]),
                               Bsz, T, H, P, G, N, chunk, xdt, _ptr(ws), ws.numel(),
                               _stream(stream)))
    return out


def ssd_complex_chunk_bwd(x, dt, A, B, C, dy, dt_bias=None, dt_min=0.0, dt_max=math.inf,
                          h0=None, dh_final=None, chunk=64, want_dh0=True, workspace=None,
                          stream=None):
    """Gradient of sum(dy * y) + <dh_final, h_final> of ssd_complex_chunk_fwd
    (float32 x and dy, complex64 A/B/C/h0/dh_final as (re, im) pairs, chunk
    64).  Complex gradients come as (d/d re, d/d im) pairs.  Returns a dict:
    dx, ddt, dA (H,2), dB, dC (Bsz,T,G,N,2), ddt_bias, dh0 (Bsz,H,P,N,2; None
    unless want_dh0), all float32."""
    A, B, C, h0, dh_final = _pairs(A), _pairs(B), _pairs(C), _pairs(h0), _pairs(dh_final)
    _ndim(x, "x", 4)
    _ndim(B, "B", 5)
    Bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _expect(B, "B", (Bsz, T, G, N, 2), x)
    _expect(C, "C", (Bsz, T, G, N, 2), x)
    _expect(dy, "dy", (Bsz, T, H, P), x)
    _expect(dt, "dt", (Bsz, T, H), x)
    _expect(A, "A", (H, 2), x)
    _expect(dt_bias, "dt_bias", (H,), x)
    _expect(h0, "h0", (Bsz, H, P, N, 2), x)
    _expect(dh_final, "dh_final", (Bsz, H, P, N, 2), x)
    for t, n in ((x, "x"), (dt, "dt"), (A, "A"), (B, "B"), (C, "C"), (dy, "dy"),
                 (dt_bias, "dt_bias"), (h0, "h0"), (dh_final, "dh_final")):
        _dev(t, n, torch.float32)
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dx=torch.empty((Bsz, T, H, P), **f32), ddt=torch.empty((Bsz, T, H), **f32),
               dA=torch.empty((H, 2), **f32), dB=torch.empty((Bsz, T, G, N, 2), **f32),
               dC=torch.empty((Bsz, T, G, N, 2), **f32), ddt_bias=torch.empty(H, **f32),
               dh0=torch.empty((Bsz, H, P, N, 2), **f32) if want_dh0 else None)
    ws = _workspace(ssd_complex_bwd_workspace_size(Bsz, T, H, P, G, N), dev, workspace)
    _check(lib().ssd_complex_chunk_bwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                       _ptr(dt_bias), float(dt_min), float(dt_max), _ptr(h0),
                                       _ptr(dy), _ptr(dh_final), _ptr(out["dx"]),
                                       _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dB"]),
                                       _ptr(out["dC"]), _ptr(out["ddt_bias"]), _ptr(out["dh0"]),
                                       Bsz, T, H, P, G, N, chunk, _ptr(ws), ws.numel(),
                                       _stream(stream)))
    return out


def ssd_complex_chunk_fwd_packed(proj, A, H, P, N, dt_bias=None, dt_min=0.0, dt_max=math.inf,
                                 h0=None, chunk=256, return_final_state=False, y=None,
                                 workspace=None, stream=None):
    """Complex chunked forward reading x, B, C and dt in place from the
    in_proj output rows proj (Bsz, T, W) float32, W >= H*(P + 4N + 1): slices
    [x | B_re | B_im | C_re | C_im | dt], head-major, per-head B/C.  proj may
    be a column slice of wider rows (its row stride is passed).  Returns y
    (Bsz,T,H,P) float32 (and h_final (Bsz,H,P,N,2) if return_final_state)."""
    _ndim(proj, "proj", 3)
    Bsz, T, W = proj.shape
    if W < H * (P + 4 * N + 1):
        raise ValueError(f"proj rows have {W} columns, need {H * (P + 4 * N + 1)}")
    A, h0, y = _pairs(A), _pairs(h0), _pairs(y)
    _expect(A, "A", (H, 2), proj)
    _expect(dt_bias, "dt_bias", (H,), proj)
    _expect(h0, "h0", (Bsz, H, P, N, 2), proj)
    _expect(y, "y", (Bsz, T, H, P), proj)
    ld = _rows(proj, "proj", 3)
    if proj.dtype != torch.float32:
        raise TypeError("proj must be float32")
    _dev(A, "A", torch.float32)
    _dev(dt_bias, "dt_bias", torch.float32)
    _dev(h0, "h0", torch.float32)
    dev = proj.device
    if y is None:
        y = torch.empty((Bsz, T, H, P), dtype=torch.float32, device=dev)
    _dev(y, "y", torch.float32)
    hf = torch.empty((Bsz, H, P, N, 2), dtype=torch.float32, device=dev) if return_final_state else None
    nbytes = ssd_workspace_size(Bsz, T, H, P, H, N, chunk, True)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib().ssd_complex_chunk_fwd_packed(_ptr(proj), ld, _ptr(A), _ptr(dt_bias),
                                              float(dt_min), float(dt_max), _ptr(h0), _ptr(y),
                                              _ptr(hf), Bsz, T, H, P, N, chunk, _ptr(ws),
                                              ws.numel(), _stream(stream)))
    return (y, hf) if return_final_state else y


def _dcode(dtype, name):
    if dtype == torch.bfloat16:
        return SSD_BF16
    if dtype == torch.float32:
        return SSD_F32
    raise TypeError(f"{name} must be float32 or bfloat16, got {dtype}")


def ssd_linear_fwd(x, W, z=None, out_dtype=torch.bfloat16, stream=None):
    """Bias-free linear layer z = x W^T on the last axis: x (..., K) float32 or
    bfloat16, W (Nout, K) bfloat16, z (..., Nout) in out_dtype (bf16 matrix
    products, fp32 accumulation).  K % 64 == 0, Nout % 128 == 0."""
    _ndim(W, "W", 2)
    Nout, K = W.shape
    if x.dim() < 1 or x.shape[-1] != K:
        raise ValueError(f"x has shape {tuple(x.shape)}, its last axis must be K={K}")
    if z is not None:
        _expect(z, "z", tuple(x.shape[:-1]) + (Nout,), x)
    xd = _dcode(x.dtype, "x")
    _dev(x, "x")
    _dev(W, "W", torch.bfloat16)
    if z is None:
        z = torch.empty(tuple(x.shape[:-1]) + (Nout,), dtype=out_dtype, device=x.device)
    zd = _dcode(z.dtype, "z")
    _dev(z, "z")
    M = x.numel() // K
    _check(lib().ssd_linear_fwd(_ptr(x), xd, _ptr(W), _ptr(z), zd, M, K, Nout, _stream(stream)))
    return z


def ssd_mimo_fwd(y, W, z=None, out_dtype=torch.bfloat16, stream=None):
    """MIMO head mixer: y (Bsz, T, H, P) float32 or bfloat16, read per token as
    H*P features head-major; W (H*P, H*P) bfloat16; returns z (Bsz, T, H, P)
    in out_dtype.  H*P % 128 == 0."""
    _ndim(y, "y", 4)
    Bsz, T, H, P = y.shape
    _expect(W, "W", (H * P, H * P), y)
    _expect(z, "z", (Bsz, T, H, P), y)
    yd = _dcode(y.dtype, "y")
    _dev(y, "y")
    _dev(W, "W", torch.bfloat16)
    if z is None:
        z = torch.empty((Bsz, T, H, P), dtype=out_dtype, device=y.device)
    zd = _dcode(z.dtype, "z")
    _dev(z, "z")
    _check(lib().ssd_mimo_fwd(_ptr(y), yd, _ptr(W), _ptr(z), zd, Bsz, T, H, P, _stream(stream)))
    return z
