"""CPU oracle of the selective-SSM mixer core (fp64, sequential, slow, plain).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke entry point and the
benchmark's CPU-baseline leg may use this package; the HIP library and its
binding never import it, and it never imports them.

``prefill`` and ``decode`` wrap the plain C routines in ``mamba_oracle.c``
(one token at a time, double precision; see that file for the passages each
step follows).  ``project`` is plain numpy (the projections ahead of the scan).  ``check`` holds the independent numpy pins (brute-force
materialised sums, closed forms, library routines) the oracle is tested
against.

Every function here is pinned by tests that run without a GPU, except where
"parity unpinned" is stated (none at present).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mamba_oracle.c")
_LIB = os.path.join(_HERE, "libmamba_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-std=c99", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.oracle_prefill.argtypes = [i64, i32, i32, i32, i32] + [P] * 14 + [ctypes.c_int]
        lib.oracle_prefill.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [i32, i32, i32, i32] + [P] * 13 + [ctypes.c_int]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_prefill_backward.argtypes = [i64, i32, i32, i32, i32] + [P] * 26
        lib.oracle_prefill_backward.restype = ctypes.c_int
        lib.oracle_threads.argtypes = [ctypes.c_int]
        lib.oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads(n: int = 0) -> int:
    """Set (n > 0) and return the OpenMP thread count the oracle uses."""
    return _load().oracle_threads(int(n))


def as_f64(a: np.ndarray, io: str | None = None) -> np.ndarray:
    """float64 copy of an input; bf16 inputs arrive as uint16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def prefill(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state, ssm_state,
            nthreads: int = 0):
    """Run the mixer over packed sequences.  Returns (y, conv_state_out, ssm_state_out), all float64.

    x, z, dt: [T, d]; B, C: [T, N]; A_log: [d, N]; D, dt_bias, conv_b: [d]; conv_w: [d, K];
    cu_seqlens: [S+1]; conv_state: [S, d, K-1]; ssm_state: [S, d, N] (inputs are not modified).
    """
    x, z, dt, B, C = (as_f64(a) for a in (x, z, dt, B, C))
    A_log, D, dt_bias, conv_w, conv_b = (as_f64(a) for a in (A_log, D, dt_bias, conv_w, conv_b))
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, d = x.shape
    N = B.shape[1]
    K = conv_w.shape[1]
    S = cu.shape[0] - 1
    cs = as_f64(conv_state).reshape(S, d, K - 1).copy()
    ss = as_f64(ssm_state).reshape(S, d, N).copy()
    y = np.zeros((T, d), dtype=np.float64)
    rc = _load().oracle_prefill(T, S, d, N, K, _p(x), _p(z), _p(dt), _p(B), _p(C), _p(A_log), _p(D),
                                _p(dt_bias), _p(conv_w), _p(conv_b), _p(cu), _p(cs), _p(ss), _p(y),
                                int(nthreads))
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments (cu_seqlens or dims)")
    return y, cs, ss


def prefill_backward(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state, ssm_state, dy):
    """Gradients of a loss with dL/dy = dy (and no dependence on the final states) with respect to
    every prefill input and the initial states (reverse mode of ``prefill``; see
    ``oracle_prefill_backward`` in mamba_oracle.c).  Returns a dict of float64 arrays: dx, dz, ddt
    [T, d]; dB, dC [T, N]; dA_log [d, N]; dD, ddt_bias, dconv_b [d]; dconv_w [d, K];
    dconv_state [S, d, K-1]; dssm_state [S, d, N]."""
    x, z, dt, B, C, dy = (as_f64(a) for a in (x, z, dt, B, C, dy))
    A_log, D, dt_bias, conv_w, conv_b = (as_f64(a) for a in (A_log, D, dt_bias, conv_w, conv_b))
    T, d = x.shape
    N = B.shape[1]
    K = conv_w.shape[1]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    S = cu.shape[0] - 1
    cs = as_f64(conv_state).reshape(S, d, K - 1).copy()
    ss = as_f64(ssm_state).reshape(S, d, N).copy()
    out = dict(dx=np.zeros((T, d)), dz=np.zeros((T, d)), ddt=np.zeros((T, d)), dB=np.zeros((T, N)),
               dC=np.zeros((T, N)), dA_log=np.zeros((d, N)), dD=np.zeros(d), ddt_bias=np.zeros(d),
               dconv_w=np.zeros((d, K)), dconv_b=np.zeros(d), dconv_state=np.zeros((S, d, K - 1)),
               dssm_state=np.zeros((S, d, N)))
    rc = _load().oracle_prefill_backward(
        T, S, d, N, K, _p(x), _p(z), _p(dt), _p(B), _p(C), _p(A_log), _p(D), _p(dt_bias), _p(conv_w), _p(conv_b),
        cu.ctypes.data_as(ctypes.c_void_p), _p(cs), _p(ss), _p(dy),
        *[_p(out[k]) for k in ("dx", "dz", "ddt", "dB", "dC", "dA_log", "dD", "ddt_bias", "dconv_w", "dconv_b",
                               "dconv_state", "dssm_state")])
    if rc != 0:
        raise ValueError("oracle_prefill_backward rejected its arguments")
    return out


def decode(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state, nthreads: int = 0):
    """One decode step for Bs rows.  Returns (y, conv_state_out, ssm_state_out), all float64."""
    x, z, dt, B, C = (as_f64(a) for a in (x, z, dt, B, C))
    A_log, D, dt_bias, conv_w, conv_b = (as_f64(a) for a in (A_log, D, dt_bias, conv_w, conv_b))
    Bs, d = x.shape
    N = B.shape[1]
    K = conv_w.shape[1]
    cs = as_f64(conv_state).reshape(Bs, d, K - 1).copy()
    ss = as_f64(ssm_state).reshape(Bs, d, N).copy()
    y = np.zeros((Bs, d), dtype=np.float64)
    rc = _load().oracle_decode(Bs, d, N, K, _p(x), _p(z), _p(dt), _p(B), _p(C), _p(A_log), _p(D),
                               _p(dt_bias), _p(conv_w), _p(conv_b), _p(cs), _p(ss), _p(y), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return y, cs, ss


def decode_replay(x_ring, dt_ring, B_ring, k, z, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state,
                  nthreads: int = 0):
    """Decode step k of a replay window ("ReplaySSM: Cache SSM Inputs, Not State", abstract).

    The recurrent state is kept as a checkpoint (``conv_state``, ``ssm_state``: the state before
    window step 0) plus a buffer of the recent steps' inputs (``x_ring``, ``dt_ring`` [W, Bs, d]
    and ``B_ring`` [W, Bs, N]; slot s holds window step s).  The output of step k comes from
    replaying the buffered steps 0..k-1 from the checkpoint and then taking step k with its own
    z and C: the plain sequential definition, one ``decode`` step after another.  The outputs of
    the replayed steps were emitted by earlier calls; only their effect on the state matters here.

    Returns (y_k, conv_state, ssm_state) with the states after step k (float64).
    """
    Bs, d = np.asarray(z).shape
    N = np.asarray(C).shape[1]
    cs, ss = conv_state, ssm_state
    zero_z = np.zeros((Bs, d))
    zero_c = np.zeros((Bs, N))
    for s in range(k):
        _, cs, ss = decode(x_ring[s], zero_z, dt_ring[s], B_ring[s], zero_c, A_log, D, dt_bias, conv_w, conv_b,
                           cs, ss, nthreads)
    return decode(x_ring[k], z, dt_ring[k], B_ring[k], C, A_log, D, dt_bias, conv_w, conv_b, cs, ss, nthreads)


def bf16_round(a):
    """Values rounded to the nearest bfloat16 (8 significant bits), ties to even, as float64.
    With a = m 2^e, 0.5 <= |m| < 1 (frexp), the bf16 value is round(256 m) / 256 * 2^e, where
    round takes halves to the even neighbour (numpy's round); a carry to 256 gives 2^e exactly."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def decode_replay_lo(x_ring, dt_ring, B_ring, k, z, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state,
                     nthreads: int = 0):
    """Output of window step k with the dual-precision checkpoint ("ReplaySSM: Cache SSM Inputs,
    Not State", abstract: a low-precision checkpoint serves the output computation of most steps,
    a higher-precision one the recurrent updates): ``decode_replay`` from the checkpoint (conv and
    SSM state) rounded to bfloat16.  Returns (y_k, conv_state, ssm_state) as decode_replay does
    (the states after step k from the rounded checkpoint; a committing step uses the full one)."""
    return decode_replay(x_ring, dt_ring, B_ring, k, z, C, A_log, D, dt_bias, conv_w, conv_b,
                         bf16_round(conv_state), bf16_round(ssm_state), nthreads)


def project(x, conv_w, conv_b, cu_seqlens, conv_state, w_x, w_dt, R: int, N: int):
    """The input-dependent projections ahead of the scan, as the TensorRT Mamba tensor-parallel
    builder (_add_mamba_tp_layer) lays them out: the conv activation u (window = the state's K-1
    older raw inputs, then x; weighted sum with conv_w, plus conv_b, SiLU) is multiplied by the
    three input-major weights w_dt_in [d, R], w_B [d, N] and w_C [d, N] -- here the columns of
    w_x [d, R + 2N] in that order -- and dt_in is multiplied by w_dt_out [R, d] (w_dt here).  The
    builder then adds dt_proj_bias and takes softplus, which the mixer core does with dt_bias.

    x [T, d]; conv_w [d, K]; conv_b [d]; cu_seqlens [S+1]; conv_state [S, d, K-1] (the initial
    state, read only).  Returns a dict of float64 arrays u [T, d], dt_in [T, R], B [T, N],
    C [T, N], dt [T, d].  Sequences never see one another's tokens (PackMamba).
    """
    x = as_f64(x)
    conv_w, conv_b, w_x, w_dt = (as_f64(a) for a in (conv_w, conv_b, w_x, w_dt))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    S = cu.shape[0] - 1
    T, d = x.shape
    K = conv_w.shape[1]
    cs = as_f64(conv_state).reshape(S, d, K - 1)
    u = np.zeros((T, d))
    for s in range(S):
        a, b = int(cu[s]), int(cu[s + 1])
        window = np.concatenate([cs[s].T, x[a:b]], axis=0)  # rows oldest first: K-1 state columns, then tokens
        for t in range(b - a):
            xc = conv_b.copy()
            for k in range(K):
                xc += conv_w[:, k] * window[t + k]
            u[a + t] = xc / (1.0 + np.exp(-xc))
    xdbl = u @ w_x
    dt_in = xdbl[:, :R]
    return dict(u=u, dt_in=dt_in, B=xdbl[:, R:R + N], C=xdbl[:, R + N:R + 2 * N], dt=dt_in @ w_dt)
