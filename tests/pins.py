"""Independent numpy/scipy evaluations used to pin the oracle.

None of these shares code with the oracle: they take the mixer's definition
through different formulas or library routines, so that a plausible slip in the
oracle (a dropped term, a flipped sign or index, a transposed operand, an
unstable softplus) disagrees with at least one of them.

* ``brute_force_sequence``: the state written as the materialised sum over all
  earlier tokens of (product of the decays since then) x (that token's input),
  plus the decayed initial state -- the unrolled "checkpoint plus buffer of
  recent inputs" view of the recurrence described on the ReplaySSM page.  The
  conv stage is ``np.convolve`` with the reversed taps, softplus is
  ``np.logaddexp(0, v)``, the logistic is ``scipy.special.expit``.
* ``geometric_closed_form``: constant inputs give a geometric series per state
  index.
* ``lfilter_scan``: with one state index, constant delta and B = C = 1 the scan
  is a first-order IIR filter (``scipy.signal.lfilter``).
* ``conv_silu`` and ``matmul_loops``: the conv activation by ``np.convolve`` and
  ``expit``, and a matrix product written as Python loops, for the projections.
"""
from __future__ import annotations

import numpy as np
from scipy.signal import lfilter
from scipy.special import expit


def to64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return a.astype(np.float64)


def brute_force_sequence(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, conv0, h0):
    """One sequence.  x, z, dt [L, d]; B, C [L, N]; conv0 [d, K-1]; h0 [d, N].

    Returns (out [L, d], final conv state [d, K-1], final ssm state [d, N]).
    """
    x, z, dt, B, C = (to64(a) for a in (x, z, dt, B, C))
    A_log, D, dt_bias, conv_w, conv_b = (to64(a) for a in (A_log, D, dt_bias, conv_w, conv_b))
    conv0, h0 = to64(conv0), to64(h0)
    L, d = x.shape
    K = conv_w.shape[1]
    X = np.concatenate([conv0.T, x], axis=0)  # [K-1+L, d], time ascending
    xc = np.empty((L, d))
    for c in range(d):
        xc[:, c] = np.convolve(X[:, c], conv_w[c, ::-1], mode="valid") + conv_b[c]
    u = xc * expit(xc)
    delta = np.logaddexp(0.0, dt + dt_bias[None, :])
    A = -np.exp(A_log)  # [d, N]
    abar = np.exp(delta[:, :, None] * A[None, :, :])  # [L, d, N]
    inp = delta[:, :, None] * B[:, None, :] * u[:, :, None]  # [L, d, N]
    h = np.empty_like(abar)
    for t in range(L):
        acc = np.prod(abar[: t + 1], axis=0) * h0
        for j in range(t + 1):
            acc = acc + np.prod(abar[j + 1: t + 1], axis=0) * inp[j]
        h[t] = acc
    y = np.einsum("tdn,tn->td", h, C) + D[None, :] * u
    out = y * (z * expit(z))
    conv_final = X[L: L + K - 1].T.copy()
    ssm_final = h[L - 1].copy() if L > 0 else h0.copy()
    return out, conv_final, ssm_final


def geometric_closed_form(L, x0, z0, dt0, Bv, Cv, A_log_c, D_c, dt_bias_c, w_c, b_c, h0_c):
    """Constant inputs on one channel (conv state pre-filled with x0): closed-form outputs and state.

    h_t[n] = a^(t+1) h0[n] + beta[n] (1 - a^(t+1)) / (1 - a),  a = exp(delta A[n]), beta = delta B[n] u.
    """
    K = len(w_c)
    xc = b_c + x0 * float(np.sum(w_c))
    u = xc * expit(xc)
    delta = float(np.logaddexp(0.0, dt0 + dt_bias_c))
    A = -np.exp(np.asarray(A_log_c, dtype=np.float64))
    a = np.exp(delta * A)
    beta = delta * np.asarray(Bv, dtype=np.float64) * u
    t = np.arange(L)[:, None]
    at = a[None, :] ** (t + 1)
    h = at * np.asarray(h0_c, dtype=np.float64)[None, :] + beta[None, :] * (1.0 - at) / (1.0 - a[None, :])
    y = h @ np.asarray(Cv, dtype=np.float64) + D_c * u
    out = y * (z0 * expit(z0))
    del K
    return out, h[-1]


def lfilter_scan(u, delta, A, h0):
    """h_t = a h_{t-1} + delta u_t with a = exp(delta A), via scipy's IIR filter."""
    a = np.exp(delta * A)
    h, _ = lfilter([1.0], [1.0, -a], delta * np.asarray(u, dtype=np.float64), zi=[a * h0])
    return h


def conv_silu(x, conv_w, conv_b, conv0):
    """SiLU of the causal conv of one sequence by np.convolve: x [L, d], conv0 [d, K-1] (older
    first); returns u [L, d]."""
    x, conv_w, conv_b, conv0 = (to64(a) for a in (x, conv_w, conv_b, conv0))
    L, d = x.shape
    X = np.concatenate([conv0.T, x], axis=0)
    u = np.empty((L, d))
    for c in range(d):
        xc = np.convolve(X[:, c], conv_w[c, ::-1], mode="valid") + conv_b[c]
        u[:, c] = xc * expit(xc)
    return u


def matmul_loops(a, b):
    """a @ b by explicit loops (tiny sizes only)."""
    a, b = to64(a), to64(b)
    m, k = a.shape
    k2, n = b.shape
    assert k == k2
    out = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for q in range(k):
                acc += float(a[i, q]) * float(b[q, j])
            out[i, j] = acc
    return out
