"""Independent re-statements of the scan used to pin the oracle.

Nothing here is imported by the product or by the oracle.  Each function
computes the same quantity as the oracle by a different route:

* ``chunked_real`` / ``chunked_complex``: the chunkwise form -- intra-chunk
  decay matrix L[l,s] = exp(cs_l - cs_s) 1[l >= s] and inter-chunk carry
  through the cumulative chunk log-decays CD (Numerical Stability in
  Mamba-3-Lite, section 4), evaluated with numpy matrix products in float64.
* ``dual_real_mp`` / ``dual_complex_mp``: the quadratic (attention-like,
  state-space-duality) form y_t = sum_{s<=t} (C_t . B_s) prod_{r in (s,t]}
  a_r dt_s x_s + D x_t + C_t (prod_{r<=t} a_r) h0, in mpmath at 50 digits.
* ``seq_complex_np``: the complex recurrence on numpy complex128 scalars.
"""
import math

import mpmath
import numpy as np


def softplus_np(z):
    return np.logaddexp(0.0, z)


def deltas(dt, dt_bias, dt_min, dt_max):
    z = dt.astype(np.float64)
    if dt_bias is not None:
        z = z + dt_bias.astype(np.float64)
    return np.clip(softplus_np(z), dt_min, dt_max)


def widen(a):
    """float32 or bfloat16-bits (uint16) array -> float64."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _causal_decay(cs):
    diff = cs[:, None] - cs[None, :]
    mask = np.tril(np.ones_like(diff, dtype=bool))
    return np.where(mask, np.exp(np.where(mask, diff, 0.0)), 0.0)


def chunked_real(inp, Q):
    x, B, C = widen(inp["x"]), widen(inp["B"]), widen(inp["C"])
    Bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    dlt = deltas(inp["dt"], inp["dt_bias"], inp["dt_min"], inp["dt_max"])
    A = inp["A"].astype(np.float64)
    D = np.zeros(H) if inp["D"] is None else inp["D"].astype(np.float64)
    h0 = inp["h0"]
    y = np.zeros((Bsz, T, H, P))
    hf = np.zeros((Bsz, H, P, N))
    nc = -(-T // Q)
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            a = A[h] * dlt[b, :, h]
            start = np.zeros((P, N)) if h0 is None else h0[b, h].astype(np.float64)
            lam, states, parts = [], [], []
            for c in range(nc):
                sl = slice(c * Q, min(T, (c + 1) * Q))
                cs = np.cumsum(a[sl])
                Xc, Bc, Cc, dc = x[b, sl, h], B[b, sl, g], C[b, sl, g], dlt[b, sl, h]
                ydiag = ((Cc @ Bc.T) * _causal_decay(cs)) @ (dc[:, None] * Xc)
                w = np.exp(cs[-1] - cs) * dc
                states.append((w[:, None] * Xc).T @ Bc)
                lam.append(cs[-1])
                parts.append((sl, cs, Cc, ydiag))
            CD = np.cumsum(lam)
            for z in range(nc + 1):
                # state entering chunk z: chunk c < z decays by exp(CD[z-1]-CD[c]),
                # the initial state by exp(CD[z-1])
                if z == 0:
                    hin = start.copy()
                else:
                    hin = math.exp(CD[z - 1]) * start
                    for c in range(z):
                        hin = hin + math.exp(CD[z - 1] - CD[c]) * states[c]
                if z == nc:
                    hf[b, h] = hin
                    break
                sl, cs, Cc, ydiag = parts[z]
                yoff = np.exp(cs)[:, None] * (Cc @ hin.T)
                y[b, sl, h] = ydiag + yoff + D[h] * x[b, sl, h]
    return y, hf


def chunked_complex(inp, Q):
    x = inp["x"].astype(np.float64)
    Bc_ = inp["B"].astype(np.float64)
    Cc_ = inp["C"].astype(np.float64)
    B = Bc_[..., 0] + 1j * Bc_[..., 1]
    C = Cc_[..., 0] + 1j * Cc_[..., 1]
    Bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    dlt = deltas(inp["dt"], inp["dt_bias"], inp["dt_min"], inp["dt_max"])
    A = inp["A"][:, 0].astype(np.float64) + 1j * inp["A"][:, 1].astype(np.float64)
    h0 = inp["h0"]
    y = np.zeros((Bsz, T, H, P))
    hf = np.zeros((Bsz, H, P, N), np.complex128)
    nc = -(-T // Q)
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            a = A[h] * dlt[b, :, h]
            start = np.zeros((P, N), np.complex128) if h0 is None else (
                h0[b, h, ..., 0].astype(np.float64) + 1j * h0[b, h, ..., 1].astype(np.float64))
            lam, states, parts = [], [], []
            for c in range(nc):
                sl = slice(c * Q, min(T, (c + 1) * Q))
                cs = np.cumsum(a[sl])
                Xc, Bk, Ck = x[b, sl, h], B[b, sl, g], C[b, sl, g]
                diff = cs[:, None] - cs[None, :]
                mask = np.tril(np.ones(diff.shape, bool))
                L = np.where(mask, np.exp(np.where(mask, diff, 0.0)), 0.0)
                ydiag = (((Ck @ Bk.T) * L) @ Xc).real
                w = np.exp(cs[-1] - cs)
                states.append(Xc.T @ (w[:, None] * Bk))
                lam.append(cs[-1])
                parts.append((sl, cs, Ck, ydiag))
            CD = np.cumsum(lam)
            for z in range(nc + 1):
                if z == 0:
                    hin = start.copy()
                else:
                    hin = np.exp(CD[z - 1]) * start
                    for c in range(z):
                        hin = hin + np.exp(CD[z - 1] - CD[c]) * states[c]
                if z == nc:
                    hf[b, h] = hin
                    break
                sl, cs, Ck, ydiag = parts[z]
                yoff = (np.exp(cs)[:, None] * (Ck @ hin.T)).real
                y[b, sl, h] = ydiag + yoff
    return y, np.stack([hf.real, hf.imag], axis=-1)


def seq_complex_np(inp):
    """Complex recurrence with numpy complex128 arithmetic (no hand expansion)."""
    x = inp["x"].astype(np.float64)
    B = inp["B"][..., 0].astype(np.float64) + 1j * inp["B"][..., 1].astype(np.float64)
    C = inp["C"][..., 0].astype(np.float64) + 1j * inp["C"][..., 1].astype(np.float64)
    Bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    dlt = deltas(inp["dt"], inp["dt_bias"], inp["dt_min"], inp["dt_max"])
    A = inp["A"][:, 0].astype(np.float64) + 1j * inp["A"][:, 1].astype(np.float64)
    y = np.zeros((Bsz, T, H, P))
    hf = np.zeros((Bsz, H, P, N), np.complex128)
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            S = np.zeros((P, N), np.complex128)
            if inp["h0"] is not None:
                S = (inp["h0"][b, h, ..., 0].astype(np.float64)
                     + 1j * inp["h0"][b, h, ..., 1].astype(np.float64))
            for t in range(T):
                S = np.exp(A[h] * dlt[b, t, h]) * S + np.outer(x[b, t, h], B[b, t, g])
                y[b, t, h] = (S @ C[b, t, g]).real
            hf[b, h] = S
    return y, np.stack([hf.real, hf.imag], axis=-1)


def dual_real_mp(inp, dps=50):
    """Quadratic dual form of the real scan, in mpmath (small T only)."""
    mpmath.mp.dps = dps
    x, B, C = widen(inp["x"]), widen(inp["B"]), widen(inp["C"])
    Bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    D = inp["D"]
    h0 = inp["h0"]
    out = np.zeros((Bsz, T, H, P))
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            bias = mpmath.mpf(float(inp["dt_bias"][h])) if inp["dt_bias"] is not None else 0
            dl = []
            for t in range(T):
                z = mpmath.mpf(float(inp["dt"][b, t, h])) + bias
                d = mpmath.log(1 + mpmath.exp(z))
                d = min(max(d, mpmath.mpf(inp["dt_min"])), mpmath.mpf(inp["dt_max"]))
                dl.append(d)
            Ah = mpmath.mpf(float(inp["A"][h]))
            for t in range(T):
                for p in range(P):
                    acc = mpmath.mpf(0)
                    for s in range(t + 1):
                        cb = mpmath.fsum(mpmath.mpf(C[b, t, g, n]) * mpmath.mpf(B[b, s, g, n])
                                         for n in range(N))
                        dec = mpmath.exp(Ah * mpmath.fsum(dl[s + 1:t + 1]))
                        acc += cb * dec * dl[s] * mpmath.mpf(x[b, s, h, p])
                    if h0 is not None:
                        dec0 = mpmath.exp(Ah * mpmath.fsum(dl[:t + 1]))
                        acc += dec0 * mpmath.fsum(mpmath.mpf(C[b, t, g, n]) *
                                                  mpmath.mpf(float(h0[b, h, p, n]))
                                                  for n in range(N))
                    if D is not None:
                        acc += mpmath.mpf(float(D[h])) * mpmath.mpf(x[b, t, h, p])
                    out[b, t, h, p] = float(acc)
    return out


def dual_complex_mp(inp, dps=50):
    """Quadratic dual form of the complex scan, in mpmath (small T only)."""
    mpmath.mp.dps = dps
    x = inp["x"].astype(np.float64)
    Bsz, T, H, P = x.shape
    G, N = inp["B"].shape[2], inp["B"].shape[3]
    hpg = H // G

    def cplx(a):
        return mpmath.mpc(float(a[0]), float(a[1]))

    out = np.zeros((Bsz, T, H, P))
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            dl = []
            for t in range(T):
                z = mpmath.mpf(float(inp["dt"][b, t, h]))
                d = mpmath.log(1 + mpmath.exp(z))
                d = min(max(d, mpmath.mpf(inp["dt_min"])), mpmath.mpf(inp["dt_max"]))
                dl.append(d)
            Ah = cplx(inp["A"][h])
            for t in range(T):
                for p in range(P):
                    acc = mpmath.mpc(0)
                    for s in range(t + 1):
                        cb = mpmath.fsum(cplx(inp["C"][b, t, g, n]) * cplx(inp["B"][b, s, g, n])
                                         for n in range(N))
                        dec = mpmath.exp(Ah * mpmath.fsum(dl[s + 1:t + 1]))
                        acc += cb * dec * mpmath.mpf(x[b, s, h, p])
                    if inp["h0"] is not None:
                        dec0 = mpmath.exp(Ah * mpmath.fsum(dl[:t + 1]))
                        acc += dec0 * mpmath.fsum(cplx(inp["C"][b, t, g, n]) *
                                                  cplx(inp["h0"][b, h, p, n])
                                                  for n in range(N))
                    out[b, t, h, p] = float(acc.real)
    return out
