"""Pins of the oracle's variable-length batch (oracle.fwd_varlen), CPU only.

Its definition: every packed sequence is one recurrence from its own initial
state.  The pins check the slicing against the pinned batched recurrence
(oracle.fwd) and against the properties that definition fixes: equal lengths
reduce to the batched form, sequences do not interact, an empty sequence
returns its h0, and a sequence cut in two and chained through the state
equals the uncut one.  A shifted or overlapping slice fails one of them.
"""
import numpy as np

import oracle
from selective_state_space_09_amd import inputs


def _run(inp, **over):
    d = dict(inp, **over)
    return oracle.fwd_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["cu_seqlens"], d["D"],
                             d["dt_bias"], d["dt_min"], d["dt_max"], d["h0"])


def test_equal_lengths_reduce_to_the_batched_form():
    L, nseq = 37, 3
    inp = inputs.make_varlen([L] * nseq, H=2, P=8, N=8, G=1, dtype="bf16", seed=3, with_h0=True)
    y, hf = _run(inp)
    rs = lambda a: a.reshape((nseq, L) + a.shape[1:])
    yb, hb = oracle.fwd(rs(inp["x"]), rs(inp["dt"]), inp["A"], rs(inp["B"]), rs(inp["C"]), inp["D"],
                        inp["dt_bias"], inp["dt_min"], inp["dt_max"], inp["h0"])
    np.testing.assert_array_equal(y, yb.reshape(y.shape))
    np.testing.assert_array_equal(hf, hb)


def test_sequences_do_not_interact():
    lengths = [9, 14, 6]
    inp = inputs.make_varlen(lengths, H=2, P=4, N=8, G=2, dtype="f32", seed=5, with_h0=True)
    y, hf = _run(inp)
    cu = inp["cu_seqlens"]
    x2 = inp["x"].copy()
    x2[cu[1]:cu[2]] += 1.0  # change the middle sequence only
    y2, hf2 = _run(inp, x=x2)
    np.testing.assert_array_equal(y2[:cu[1]], y[:cu[1]])
    np.testing.assert_array_equal(y2[cu[2]:], y[cu[2]:])
    np.testing.assert_array_equal(hf2[[0, 2]], hf[[0, 2]])
    assert np.abs(y2[cu[1]:cu[2]] - y[cu[1]:cu[2]]).max() > 1e-3
    assert np.abs(hf2[1] - hf[1]).max() > 1e-3


def test_empty_sequence_returns_its_initial_state():
    inp = inputs.make_varlen([4, 0, 3], H=2, P=4, N=4, dtype="f32", seed=7, with_h0=True)
    y, hf = _run(inp)
    assert y.shape[0] == 7
    np.testing.assert_array_equal(hf[1], inp["h0"][1].astype(np.float64))


def test_cut_and_chained_sequence_equals_the_uncut_one():
    """Sequence of 23 tokens vs. the same tokens as sequences of 10 and 13,
    the second starting from the first's final state (rounded to float32, as
    h0 is passed): equal to that rounding."""
    inp = inputs.make_varlen([23], H=2, P=4, N=8, dtype="f32", seed=11, with_h0=True)
    y, hf = _run(inp)
    cut = dict(inp, cu_seqlens=np.array([0, 10], np.int32))
    first = {k: (v[:10] if k in ("x", "dt", "B", "C") else v) for k, v in cut.items()}
    y1, h1 = _run(first)
    second = {k: (v[10:] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    second["cu_seqlens"] = np.array([0, 13], np.int32)
    second["h0"] = h1.astype(np.float32)
    y2, h2 = _run(second)
    np.testing.assert_array_equal(y1, y[:10])
    scale = np.abs(y).max()
    assert np.abs(y2 - y[10:]).max() <= 1e-6 * scale
    assert np.abs(h2 - hf).max() <= 1e-6 * np.abs(hf).max()


# ---- the convolution over a variable-length batch (oracle.conv1d_varlen) ----

def _conv_inputs(lengths, Ch=24, seed=0):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    xbc = rng.standard_normal((int(cu[-1]), Ch)).astype(np.float32)
    w = rng.uniform(-0.5, 0.5, size=(Ch, 4)).astype(np.float32)
    bias = rng.uniform(-0.5, 0.5, size=Ch).astype(np.float32)
    st = rng.standard_normal((len(lengths), 3, Ch)).astype(np.float32)
    return xbc, w, bias, st, cu


def test_conv_varlen_equal_lengths_reduce_to_the_batched_form():
    L, nseq = 11, 3
    xbc, w, bias, st, cu = _conv_inputs([L] * nseq, seed=1)
    out, so = oracle.conv1d_varlen(xbc, w, cu, bias, st)
    ob, sb = oracle.conv1d(xbc.reshape(nseq, L, -1), w, bias, st)
    np.testing.assert_array_equal(out, ob.reshape(out.shape))
    np.testing.assert_array_equal(so, sb)


def test_conv_varlen_sequences_do_not_interact_and_empty_keeps_state():
    xbc, w, bias, st, cu = _conv_inputs([5, 0, 2, 7], seed=2)
    out, so = oracle.conv1d_varlen(xbc, w, cu, bias, st)
    np.testing.assert_array_equal(so[1], st[1].astype(np.float64))
    x2 = xbc.copy()
    x2[cu[2]:cu[3]] += 1.0  # the third sequence only
    out2, so2 = oracle.conv1d_varlen(x2, w, cu, bias, st)
    np.testing.assert_array_equal(out2[:cu[2]], out[:cu[2]])
    np.testing.assert_array_equal(out2[cu[3]:], out[cu[3]:])
    np.testing.assert_array_equal(so2[[0, 1, 3]], so[[0, 1, 3]])
    assert np.abs(out2[cu[2]:cu[3]] - out[cu[2]:cu[3]]).max() > 1e-3


def test_conv_varlen_cut_and_chained_equals_uncut():
    """a sequence of 9 rows vs. its first 4 and last 5 as two calls chained
    through the carried state (raw inputs, so exactly)"""
    xbc, w, bias, st, cu = _conv_inputs([9], seed=3)
    out, so = oracle.conv1d_varlen(xbc, w, cu, bias, st)
    o1, s1 = oracle.conv1d_varlen(xbc[:4], w, [0, 4], bias, st)
    o2, s2 = oracle.conv1d_varlen(xbc[4:], w, [0, 5], bias, s1.astype(np.float32))
    np.testing.assert_array_equal(np.concatenate([o1, o2]), out)
    np.testing.assert_array_equal(s2, so)
