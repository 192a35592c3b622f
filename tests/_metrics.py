"""Parity metrics shared by the tests (comparison only, no scan arithmetic).

The error of a result against the oracle is normwise per (batch, head) slice:
max over slices of ||got - ref||_inf / ||ref||_inf.  A wrong head or a wrong
chunk shows up in its own slice, and near-zero elements cannot inflate it.
Any non-finite value fails outright.
"""
import numpy as np


def _slices_y(a):
    # (Bsz, T, H, P) -> (Bsz*H, T*P)
    a = np.asarray(a, np.float64)
    Bsz, T, H, P = a.shape
    return a.transpose(0, 2, 1, 3).reshape(Bsz * H, T * P)


def _slices_state(a):
    # (Bsz, H, ...) -> (Bsz*H, rest)
    a = np.asarray(a, np.float64)
    return a.reshape(a.shape[0] * a.shape[1], -1)


def _err(g, r):
    if not np.all(np.isfinite(g)):
        return float("inf")
    num = np.max(np.abs(g - r), axis=1)
    den = np.maximum(np.max(np.abs(r), axis=1), 1e-300)
    return float(np.max(num / den))


def y_err(got, ref):
    """Normwise error of an output (Bsz, T, H, P) per (b, h)."""
    return _err(_slices_y(got), _slices_y(ref))


def state_err(got, ref):
    """Normwise error of a state (Bsz, H, ...) per (b, h)."""
    return _err(_slices_state(got), _slices_state(ref))


def y_err_bh(got, ref):
    """Per-(b,h) errors of a (Bsz, H, P)-shaped decode output."""
    return _err(_slices_state(got), _slices_state(ref))


def global_err(got, ref):
    """Global normwise error ||got - ref||_inf / ||ref||_inf over the whole
    array."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    if not np.all(np.isfinite(g)):
        return float("inf")
    return float(np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-300))


def p999_err(got, ref):
    """99.9th percentile of the elementwise relative error |got - ref| /
    max(|ref|, 1e-6 ||ref||_inf)."""
    g = np.asarray(got, np.float64).ravel()
    r = np.asarray(ref, np.float64).ravel()
    if not np.all(np.isfinite(g)):
        return float("inf")
    if r.size == 0:
        return 0.0
    floor = 1e-6 * max(np.max(np.abs(r)), 1e-300)
    return float(np.percentile(np.abs(g - r) / np.maximum(np.abs(r), floor), 99.9))


def report(label, got, ref, kind="y"):
    """The three figures of a comparison, printed on one line: per-slice
    normwise (the asserted one), global normwise, 99.9th-percentile
    elementwise.  Returns the per-slice figure."""
    e = y_err(got, ref) if kind == "y" else state_err(got, ref)
    print("%s: normwise %.3g  global %.3g  p99.9 %.3g"
          % (label, e, global_err(got, ref), p999_err(got, ref)), flush=True)
    return e
