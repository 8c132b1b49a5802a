"""Pins of the oracle's causal depthwise conv1d against facts that do not come from it: a
worked example by hand, numpy's full convolution and scipy's FIR filter (zero initial
state), the split invariance a carried conv state must give, the state shift of short
sequences, and decode = a one-token prefill.  A reversed kernel, an off-by-one in the
window, a state taken from the wrong end or a dropped bias fails at least one of them.
"""
import numpy as np
import pytest
import scipy.signal
import scipy.special

from oracle import conv1d_prefill, conv1d_update


def test_hand_example():
    # W = 4, one channel, weights w0..w3 = 1, 10, 100, 1000 (w3 multiplies the newest input)
    w = np.array([[1.0, 10.0, 100.0, 1000.0]])
    x = np.array([[1.0], [2.0], [3.0]])
    out, st = conv1d_prefill(x, w, np.array([0.5]), [0, 3])
    np.testing.assert_array_equal(out[:, 0], [1000.5, 2100.5, 3210.5])
    np.testing.assert_array_equal(st[0, :, 0], [1.0, 2.0, 3.0])
    # with a carried state 7, 8, 9 (oldest first): 7*1 + 8*10 + 9*100 + 1*1000
    out, st = conv1d_prefill(x[:1], w, None, [0, 1],
                             conv_states=[np.array([[7.0], [8.0], [9.0]])])
    assert out[0, 0] == 1987.0
    np.testing.assert_array_equal(st[0, :, 0], [8.0, 9.0, 1.0])


@pytest.mark.parametrize("W", [2, 3, 4])
def test_zero_state_is_numpy_convolution_and_fir(W):
    rng = np.random.default_rng(71 + W)
    T, D = 37, 5
    x = rng.standard_normal((T, D))
    w = rng.standard_normal((D, W))
    b = rng.standard_normal(D)
    out, _ = conv1d_prefill(x, w, b, [0, T])
    for c in range(D):
        # out[n] = sum_j w[c, W-1-j] x[n-j]: a full convolution with the reversed kernel
        np.testing.assert_allclose(out[:, c], np.convolve(x[:, c], w[c, ::-1])[:T] + b[c],
                                   rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(out[:, c], scipy.signal.lfilter(w[c, ::-1], [1.0], x[:, c]) + b[c],
                                   rtol=1e-12, atol=1e-12)


def test_silu_activation():
    rng = np.random.default_rng(75)
    x = rng.standard_normal((9, 3))
    w = rng.standard_normal((3, 4))
    lin, _ = conv1d_prefill(x, w, None, [0, 9])
    act, _ = conv1d_prefill(x, w, None, [0, 9], activation=True)
    np.testing.assert_allclose(act, lin * scipy.special.expit(lin), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("cut", [1, 2, 3, 4, 10])
def test_split_invariance_through_the_carried_state(cut):
    """Prefilling a sequence in two calls, the second starting from the state the first
    left, gives the one-shot outputs and final state; sequences in one batch stay
    independent."""
    rng = np.random.default_rng(76)
    T, D, W = 23, 6, 4
    x = rng.standard_normal((T, D))
    w = rng.standard_normal((D, W))
    b = rng.standard_normal(D)
    s0 = rng.standard_normal((W - 1, D))
    whole, st = conv1d_prefill(x, w, b, [0, T], conv_states=[s0])
    a, st_a = conv1d_prefill(x[:cut], w, b, [0, cut], conv_states=[s0])
    c, st_c = conv1d_prefill(x[cut:], w, b, [0, T - cut], conv_states=[st_a[0]])
    np.testing.assert_allclose(np.concatenate([a, c]), whole, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(st_c, st)
    # the same two pieces as two sequences of one batch, each with its own state
    both, st2 = conv1d_prefill(x, w, b, [0, cut, T], conv_states=[s0, st_a[0]])
    np.testing.assert_allclose(both, whole, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(st2[1], st[0])


def test_short_sequence_shifts_the_state():
    """Fewer new inputs than W - 1: the new state is the old one shifted left by L with the
    inputs appended."""
    rng = np.random.default_rng(77)
    D, W = 4, 4
    s0 = rng.standard_normal((W - 1, D))
    x = rng.standard_normal((2, D))
    _, st = conv1d_prefill(x, rng.standard_normal((D, W)), None, [0, 1, 2],
                           conv_states=[s0, None])
    np.testing.assert_array_equal(st[0], np.concatenate([s0[1:], x[:1]]))
    np.testing.assert_array_equal(st[1], np.concatenate([np.zeros((2, D)), x[1:2]]))


def test_update_is_a_prefill_of_the_row_tokens():
    rng = np.random.default_rng(78)
    slots, D, W, B_pad, ntok = 9, 5, 4, 4, 3
    pool = rng.standard_normal((slots, W - 1, D))
    idx = np.array([3, 0, 7, 1])                  # row 1 is padding (null 0)
    x = rng.standard_normal((B_pad, ntok, D))
    w = rng.standard_normal((D, W))
    b = rng.standard_normal(D)
    out, writes = conv1d_update(pool, idx, x, w, b, null_block_id=0, activation=True)
    assert set(out) == {0, 2, 3} and set(writes) == {3, 7, 1}
    for r in (0, 2, 3):
        ref, st = conv1d_prefill(x[r], w, b, [0, ntok], conv_states=[pool[idx[r]]],
                                 activation=True)
        np.testing.assert_allclose(out[r], ref, rtol=1e-14, atol=1e-14)
        np.testing.assert_array_equal(writes[int(idx[r])], st[0])
