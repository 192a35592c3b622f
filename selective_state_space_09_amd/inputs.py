"""Seeded synthetic inputs for the SSD scan and the decode step.

Shared by the tests, the smoke check and the benchmark, on both sides of every
parity comparison.  This module holds none of the scan's arithmetic: only
random draws, the float32 -> bfloat16 encoding of inputs, and the named
workloads.  Each generator uses one ``numpy.random.default_rng(seed)`` stream
and draws in a fixed order (x, dt, dt_bias, A, B, C, D, h0; decode: dt_bias,
A, D, h0, then x, dt, B, C per step), so a seed fixes every bit.

Large normal tensors are drawn directly in float32
(``Generator.standard_normal(dtype=float32)``); bfloat16 inputs are the
round-to-nearest-even encodings of those float32 values, so the oracle and the
GPU read identical bits.

The backward workload adds dy ~ N(0,1) (bfloat16), drawn from a second
stream (seed + 1) after the forward inputs.

Workloads (shapes of the BitMamba-1B Mamba-2 layer -- d_inner 4096, 64 heads,
d_state 128 -- and of the Mamba-3-Lite layer -- 16 heads, head_dim 64, 64
complex states):
"""
import math

import numpy as np

WORKLOADS = {
    # small fp32 case the oracle finishes in well under a second
    "tiny_f32": dict(kind="real", Bsz=1, T=256, H=2, P=16, N=16, G=1, chunk=64,
                     dtype="f32"),
    # BitMamba-1B layer shape, bf16 x/B/C, fp32 dt/A/state
    "bitmamba_bf16": dict(kind="real", Bsz=2, T=2048, H=64, P=64, N=128, G=1,
                          chunk=256, dtype="bf16"),
    # Mamba-3-Lite layer shape, complex64 state, per-head B/C
    "mamba3lite_complex": dict(kind="complex", Bsz=8, T=2048, H=16, P=64, N=64,
                               G=16, chunk=256),
    # long sequence at the BitMamba shape: 256 chunks of 256
    "long_bf16": dict(kind="real", Bsz=1, T=65536, H=64, P=64, N=128, G=1,
                      chunk=256, dtype="bf16"),
    # single-token recurrent decode at the BitMamba shape, 64 steps in place
    "decode_f32": dict(kind="decode", Bsz=256, H=64, P=64, N=128, G=1, steps=64),
    # complex decode at the Mamba-3-Lite head shape; 1024 sequences so that the
    # complex64 state (537 MB) exceeds the 256 MB Infinity Cache like the real one
    "decode_complex": dict(kind="complex_decode", Bsz=1024, H=16, P=64, N=64, G=16, steps=64),
    # the Mamba-3-Lite layer read in place from its in_proj output rows (width
    # H(D + 4N + 1) = 16 * 321 = 5136: x, B_re, B_im, C_re, C_im, dt)
    "mamba3lite_packed": dict(kind="complex_packed", Bsz=8, T=2048, H=16, P=64, N=64,
                              chunk=256),
    # backward of the chunked scan at the BitMamba layer shape (gradient of a
    # loss through y: seeded dy, no h0, no dh_final)
    "bwd_bf16": dict(kind="bwd", Bsz=2, T=2048, H=64, P=64, N=128, G=1, chunk=256,
                     dtype="bf16"),
    # backward of the complex scan at the Mamba-3-Lite layer shape (loss
    # through y: seeded dy, no h0, no dh_final), chunk 64
    # a batch of six prompts of mixed lengths (4096 tokens in all) through the
    # BitMamba layer shape: the variable-length prefill
    "varlen_bf16": dict(kind="varlen", lengths=(1024, 517, 2048, 3, 64, 440), H=64, P=64, N=128, G=1,
                        chunk=256, dtype="bf16"),
    "bwd_complex": dict(kind="bwd_complex", Bsz=8, T=2048, H=16, P=64, N=64, G=16, chunk=64),
    # depthwise causal conv (K = 4, SiLU) of the BitMamba layer over its x|B|C
    # channels (4096 + 128 + 128), read from the in_proj output row (width
    # 2*4096 + 2*128 + 64 = 8512: z, x, B, C, dt) and split into the scan's inputs
    "conv_bf16": dict(kind="conv", Bsz=2, T=2048, HP=4096, GN=128, ld=8512, K=4,
                      dtype="bf16"),
    # its single-token step at the decode batch of decode_f32, 64 steps in place
    "conv_decode_f32": dict(kind="conv_decode", Bsz=256, HP=4096, GN=128, ld=8512, K=4,
                            steps=64),
    # the MIMO head mixer after the Mamba-3-Lite scan: its fp32 output y (B8 T2048,
    # H16 P64 -> 1024 features per token) times a bf16 (1024, 1024) weight, bf16 out
    "mimo_bf16": dict(kind="mimo", Bsz=8, T=2048, H=16, P=64),
}

DT_MIN = 1e-3
DT_MAX = 1e-1


def f32_to_bf16_bits(a):
    """Round float32 values to bfloat16 (nearest, ties to even); returns the
    16-bit patterns as uint16.  Inputs here are finite."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    """Widen bfloat16 bit patterns (uint16) to float32, exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng, shape, std=1.0):
    z = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        z *= np.float32(std)
    return z


def _dt_bias(rng, H, lo=DT_MIN, hi=DT_MAX):
    # bias b with softplus(b) = u, u log-uniform in [lo, hi]:  b = log(expm1(u))
    u = np.exp(rng.uniform(math.log(lo), math.log(hi), size=H))
    return np.log(np.expm1(u)).astype(np.float32)


def make_real(Bsz, T, H, P, N, G=1, dtype="f32", seed=0, with_h0=False,
              with_D=True, with_bias=True, a_range=(1.0, 16.0), **_ignored):
    """Inputs of the real Mamba-2 form.

    x, B, C ~ N(0,1); dt_raw ~ N(0,1); dt_bias such that softplus(dt_bias) is
    log-uniform in [1e-3, 1e-1]; A_h = -exp(U(log a0, log a1)); D_h ~ N(0,1);
    clamp [1e-3, 1e-1]; optional h0 ~ N(0,1).  x/B/C are float32 or bfloat16
    bit patterns (uint16) according to ``dtype``.
    """
    rng = np.random.default_rng(seed)
    x = _normal(rng, (Bsz, T, H, P))
    dt = _normal(rng, (Bsz, T, H))
    dt_bias = _dt_bias(rng, H) if with_bias else None
    A = (-np.exp(rng.uniform(math.log(a_range[0]), math.log(a_range[1]), size=H))
         ).astype(np.float32)
    B = _normal(rng, (Bsz, T, G, N))
    C = _normal(rng, (Bsz, T, G, N))
    D = rng.standard_normal(H).astype(np.float32) if with_D else None
    h0 = _normal(rng, (Bsz, H, P, N)) if with_h0 else None
    if dtype == "bf16":
        x, B, C = f32_to_bf16_bits(x), f32_to_bf16_bits(B), f32_to_bf16_bits(C)
    elif dtype != "f32":
        raise ValueError(dtype)
    return dict(kind="real", x=x, dt=dt, A=A, B=B, C=C, D=D, dt_bias=dt_bias,
                dt_min=DT_MIN, dt_max=DT_MAX, h0=h0, dtype=dtype,
                dims=dict(Bsz=Bsz, T=T, H=H, P=P, G=G, N=N))


def make_varlen(lengths, H, P, N, G=1, dtype="bf16", seed=0, with_h0=False, **kw):
    """A variable-length batch of the real form: the sequences of ``lengths``
    packed along the token axis (x (Ttot,H,P), dt (Ttot,H), B/C (Ttot,G,N),
    cu_seqlens (nseq+1) int32), drawn as ``make_real`` draws one sequence of
    Ttot tokens; h0 (nseq,H,P,N) when asked."""
    lengths = [int(t) for t in lengths]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    Ttot = int(cu[-1])
    inp = make_real(1, Ttot, H, P, N, G=G, dtype=dtype, seed=seed, with_h0=False, **kw)
    for k in ("x", "dt", "B", "C"):
        inp[k] = np.ascontiguousarray(inp[k][0])
    rng = np.random.default_rng(seed + 7919)
    inp["h0"] = _normal(rng, (len(lengths), H, P, N)) if with_h0 else None
    inp["cu_seqlens"] = cu
    inp["kind"] = "varlen"
    inp["dims"] = dict(nseq=len(lengths), Ttot=Ttot, H=H, P=P, G=G, N=N)
    return inp


def make_complex(Bsz, T, H, P, N, G=None, seed=0, with_h0=False, **_ignored):
    """Inputs of the complex Mamba-3-Lite form.

    x ~ N(0,1) float32; dt_raw ~ N(0,1) with no bias and clamp [1e-3, 1e-1];
    A_re = -exp(U(log 0.5, log 4)), A_im ~ U(-pi, pi); B, C complex with real
    and imaginary parts each ~ N(0, 1/2) (variance 1/2), stored as (re, im)
    float32 pairs; optional h0 with parts ~ N(0, 1/2).
    """
    if G is None:
        G = H
    rng = np.random.default_rng(seed)
    x = _normal(rng, (Bsz, T, H, P))
    dt = _normal(rng, (Bsz, T, H))
    a_re = -np.exp(rng.uniform(math.log(0.5), math.log(4.0), size=H))
    a_im = rng.uniform(-math.pi, math.pi, size=H)
    A = np.stack([a_re, a_im], axis=-1).astype(np.float32)
    s = math.sqrt(0.5)
    B = _normal(rng, (Bsz, T, G, N, 2), s)
    C = _normal(rng, (Bsz, T, G, N, 2), s)
    h0 = _normal(rng, (Bsz, H, P, N, 2), s) if with_h0 else None
    return dict(kind="complex", x=x, dt=dt, A=A, B=B, C=C, D=None, dt_bias=None,
                dt_min=DT_MIN, dt_max=DT_MAX, h0=h0, dtype="f32",
                dims=dict(Bsz=Bsz, T=T, H=H, P=P, G=G, N=N))


def pack_complex_rows(inp, ld=None):
    """The inputs of ``make_complex`` (per-head B/C) laid out as in_proj
    output rows (Bsz, T, ld) float32: head-major slices x (H*P), B_re, B_im,
    C_re, C_im (H*N each), dt (H); columns past them are zero.  Layout only."""
    d = inp["dims"]
    Bsz, T, H, P, N = d["Bsz"], d["T"], d["H"], d["P"], d["N"]
    if d["G"] != H:
        raise ValueError("packed rows carry per-head B and C (G = H)")
    W = H * (P + 4 * N + 1)
    ld = W if ld is None else ld
    proj = np.zeros((Bsz, T, ld), np.float32)
    HP, HN = H * P, H * N
    proj[:, :, :HP] = inp["x"].reshape(Bsz, T, HP)
    proj[:, :, HP:HP + HN] = inp["B"][..., 0].reshape(Bsz, T, HN)
    proj[:, :, HP + HN:HP + 2 * HN] = inp["B"][..., 1].reshape(Bsz, T, HN)
    proj[:, :, HP + 2 * HN:HP + 3 * HN] = inp["C"][..., 0].reshape(Bsz, T, HN)
    proj[:, :, HP + 3 * HN:HP + 4 * HN] = inp["C"][..., 1].reshape(Bsz, T, HN)
    proj[:, :, HP + 4 * HN:W] = inp["dt"]
    return proj


def make_decode(Bsz, H, P, N, G=1, steps=1, seed=0, **_ignored):
    """Inputs of the single-token decode workload.

    State h ~ N(0,1) float32 (Bsz,H,P,N); A, D, dt_bias as in ``make_real``;
    then per step x (Bsz,H,P), dt_raw (Bsz,H), B, C (Bsz,G,N), all N(0,1)
    float32.  Clamp [1e-3, 1e-1].
    """
    rng = np.random.default_rng(seed)
    dt_bias = _dt_bias(rng, H)
    A = (-np.exp(rng.uniform(0.0, math.log(16.0), size=H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    h0 = _normal(rng, (Bsz, H, P, N))
    per_step = []
    for _ in range(steps):
        per_step.append(dict(x=_normal(rng, (Bsz, H, P)), dt=_normal(rng, (Bsz, H)),
                             B=_normal(rng, (Bsz, G, N)), C=_normal(rng, (Bsz, G, N))))
    return dict(kind="decode", h0=h0, A=A, D=D, dt_bias=dt_bias, dt_min=DT_MIN,
                dt_max=DT_MAX, steps=per_step,
                dims=dict(Bsz=Bsz, H=H, P=P, G=G, N=N))


def make_complex_decode(Bsz, H, P, N, G=None, steps=1, seed=0, **_ignored):
    """Inputs of the complex single-token decode workload.

    State h (Bsz,H,P,N,2) with real and imaginary parts ~ N(0, 1/2) float32;
    A as in ``make_complex``; then per step x (Bsz,H,P) ~ N(0,1), dt_raw
    (Bsz,H) ~ N(0,1) with no bias and clamp [1e-3, 1e-1], B, C (Bsz,G,N,2)
    with parts ~ N(0, 1/2).
    """
    if G is None:
        G = H
    rng = np.random.default_rng(seed)
    a_re = -np.exp(rng.uniform(math.log(0.5), math.log(4.0), size=H))
    a_im = rng.uniform(-math.pi, math.pi, size=H)
    A = np.stack([a_re, a_im], axis=-1).astype(np.float32)
    s = math.sqrt(0.5)
    h0 = _normal(rng, (Bsz, H, P, N, 2), s)
    per_step = []
    for _ in range(steps):
        per_step.append(dict(x=_normal(rng, (Bsz, H, P)), dt=_normal(rng, (Bsz, H)),
                             B=_normal(rng, (Bsz, G, N, 2), s),
                             C=_normal(rng, (Bsz, G, N, 2), s)))
    return dict(kind="complex_decode", h0=h0, A=A, D=None, dt_bias=None, dt_min=DT_MIN,
                dt_max=DT_MAX, steps=per_step, dims=dict(Bsz=Bsz, H=H, P=P, G=G, N=N))


def make_conv(Bsz, T, HP, GN, ld=None, K=4, dtype="f32", seed=0, with_state=True,
              with_bias=True, **_ignored):
    """Inputs of the depthwise causal convolution over the x|B|C channels
    (Ch = HP + 2*GN).

    xbc (Bsz,T,ld) ~ N(0,1) (channels Ch..ld-1 of each row belong to other
    slices of the projection and are never read); w (Ch,K) and bias (Ch)
    ~ U(-1/sqrt(K), 1/sqrt(K)) (the usual fan-in bound of a depthwise conv);
    state_in (Bsz,K-1,Ch) ~ N(0,1) float32.  xbc is float32 or bfloat16 bits.
    """
    Ch = HP + 2 * GN
    ld = Ch if ld is None else ld
    rng = np.random.default_rng(seed)
    xbc = _normal(rng, (Bsz, T, ld))
    bound = 1.0 / math.sqrt(K)
    w = rng.uniform(-bound, bound, size=(Ch, K)).astype(np.float32)
    bias = rng.uniform(-bound, bound, size=Ch).astype(np.float32) if with_bias else None
    state_in = _normal(rng, (Bsz, K - 1, Ch)) if with_state else None
    if dtype == "bf16":
        xbc = f32_to_bf16_bits(xbc)
    elif dtype != "f32":
        raise ValueError(dtype)
    return dict(kind="conv", xbc=xbc, w=w, bias=bias, state_in=state_in, dtype=dtype,
                dims=dict(Bsz=Bsz, T=T, HP=HP, GN=GN, ld=ld, K=K))


def make_conv_decode(Bsz, HP, GN, ld=None, K=4, steps=1, seed=0, **_ignored):
    """Inputs of the convolution's single-token step: w, bias and the state
    (Bsz,K-1,Ch) as in ``make_conv``, then per step a row xt (Bsz,ld) ~ N(0,1)
    float32."""
    Ch = HP + 2 * GN
    ld = Ch if ld is None else ld
    rng = np.random.default_rng(seed)
    bound = 1.0 / math.sqrt(K)
    w = rng.uniform(-bound, bound, size=(Ch, K)).astype(np.float32)
    bias = rng.uniform(-bound, bound, size=Ch).astype(np.float32)
    state0 = _normal(rng, (Bsz, K - 1, Ch))
    per_step = [_normal(rng, (Bsz, ld)) for _ in range(steps)]
    return dict(kind="conv_decode", w=w, bias=bias, state0=state0, steps=per_step,
                dims=dict(Bsz=Bsz, HP=HP, GN=GN, ld=ld, K=K))


def make_workload(name, seed=0, **overrides):
    """Inputs for a named workload (see WORKLOADS), with optional overrides."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    kind = cfg["kind"]
    if kind == "real":
        return make_real(seed=seed, **cfg)
    if kind == "complex":
        return make_complex(seed=seed, **cfg)
    if kind == "varlen":
        c = dict(cfg)
        return make_varlen(c.pop("lengths"), c.pop("H"), c.pop("P"), c.pop("N"), seed=seed,
                           **{k: v for k, v in c.items() if k not in ("kind", "chunk")})
    if kind == "complex_packed":
        inp = make_complex(seed=seed, **cfg)
        inp["proj"] = pack_complex_rows(inp, cfg.get("ld"))
        inp["kind"] = "complex_packed"
        return inp
    if kind == "complex_decode":
        return make_complex_decode(seed=seed, **cfg)
    if kind == "conv":
        return make_conv(seed=seed, **cfg)
    if kind == "bwd":
        inp = make_real(seed=seed, **cfg)
        rng = np.random.default_rng(seed + 1)
        d = inp["dims"]
        dy = _normal(rng, (d["Bsz"], d["T"], d["H"], d["P"]))
        inp["dy"] = f32_to_bf16_bits(dy) if cfg.get("dtype") == "bf16" else dy
        inp["kind"] = "bwd"
        return inp
    if kind == "bwd_complex":
        inp = make_complex(seed=seed, **cfg)
        rng = np.random.default_rng(seed + 1)
        d = inp["dims"]
        inp["dy"] = _normal(rng, (d["Bsz"], d["T"], d["H"], d["P"]))
        inp["kind"] = "bwd_complex"
        return inp
    if kind == "conv_decode":
        return make_conv_decode(seed=seed, **cfg)
    if kind == "mimo":
        return make_mimo(seed=seed, **cfg)
    return make_decode(seed=seed, **cfg)


def make_mimo(Bsz, T, H, P, seed=0, identity=False, **_ignored):
    """MIMO inputs: y (Bsz, T, H, P) ~ N(0, 1) float32 (the scan output) and W
    (H*P, H*P) as bfloat16 bits, N(0, 1/(H*P)) (a mixed, trained-like weight;
    the block initialises it to the identity, identity=True)."""
    rng = np.random.default_rng(seed)
    y = _normal(rng, (Bsz, T, H, P))
    HP = H * P
    if identity:
        W = np.eye(HP, dtype=np.float32)
    else:
        W = _normal(rng, (HP, HP), 1.0 / math.sqrt(HP))
    return {"kind": "mimo", "y": y, "W": f32_to_bf16_bits(W),
            "dims": dict(Bsz=Bsz, T=T, H=H, P=P)}
