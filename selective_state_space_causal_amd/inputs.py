"""Seeded synthetic inputs for the selective-SSM mixer core.

This module only draws random numbers and packs them into arrays; it holds none
of the mixer's arithmetic. Both the HIP path's tests/bench and the CPU oracle
take their inputs from here, so that the two sides see the same bytes.

Recipe (all draws from numpy's PCG64 via ``SeedSequence(seed, spawn_key=...)``):

* Token tensors ``x, z, dt`` (shape [T, d]) are drawn N(0, 1) in float32, in
  independent sub-streams per (tensor, row block of 4096 tokens, column block
  of 64 channels).  Any row/column window can therefore be regenerated without
  drawing the rest, which lets the oracle check channel or token subsets of the
  very large workloads.
* ``B, C`` (shape [T, N], one group shared by all channels) are N(0, 1), one
  sub-stream per (tensor, row block).
* Parameters, per channel: ``A_log[c, n] = ln(n + 1)`` (so A = -(n + 1)),
  ``D = 1``, ``dt_bias = softplus^-1(dt0)`` with ``dt0 = exp(U[ln 1e-3, ln 0.1])``,
  ``conv_w[c, k], conv_b[c] ~ U(-0.5, 0.5)``.  This is the recipe of the measured
  workloads.  ``params_per_channel`` draws parameters that differ in every channel
  as a trained layer's do: ``A_log[c, n] = ln U[0.5, 16]`` independently per (c, n)
  and ``D[c] ~ N(0, 1)``, the rest as above (parity tests only).
* bf16 tensors are the float32 draws rounded to nearest-even bf16, stored as
  raw ``uint16`` bit patterns.
* Packed variable lengths: integers uniform on [lo, hi] drawn until the running
  total reaches the token budget; the last one is cut so the total is exact.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

ROW_BLOCK = 4096
COL_BLOCK = 64

# sub-stream tags
TAG_X, TAG_Z, TAG_DT, TAG_B, TAG_C, TAG_PARAMS, TAG_LENS = 1, 2, 3, 4, 5, 6, 7
TAG_DY = 8
TAG_PARAMS_VAR = 9
TAG_STEP = 100  # decode step k uses tags TAG_STEP * (k + 1) + {TAG_X, ...}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(int(seed), spawn_key=tuple(int(k) for k in key)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to nearest-even bf16; returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def token_tensor(seed: int, tag: int, rows: tuple[int, int], cols: tuple[int, int], io: str,
                 threads: int | None = None) -> np.ndarray:
    """N(0,1) draws for rows [r0, r1) and columns [c0, c1) of a [T, d] token tensor.

    Returns float32 for io == "f32" and uint16 bf16 bit patterns for io == "bf16".
    """
    r0, r1 = rows
    c0, c1 = cols
    out_dtype = np.float32 if io == "f32" else np.uint16
    out = np.empty((r1 - r0, c1 - c0), dtype=out_dtype)
    if r1 <= r0 or c1 <= c0:
        return out
    jobs = []
    for rb in range(r0 // ROW_BLOCK, (r1 - 1) // ROW_BLOCK + 1):
        for cb in range(c0 // COL_BLOCK, (c1 - 1) // COL_BLOCK + 1):
            jobs.append((rb, cb))

    def work(job):
        rb, cb = job
        block = _rng(seed, tag, rb, cb).standard_normal((ROW_BLOCK, COL_BLOCK), dtype=np.float32)
        br0, bc0 = rb * ROW_BLOCK, cb * COL_BLOCK
        lr0, lr1 = max(r0, br0), min(r1, br0 + ROW_BLOCK)
        lc0, lc1 = max(c0, bc0), min(c1, bc0 + COL_BLOCK)
        piece = block[lr0 - br0:lr1 - br0, lc0 - bc0:lc1 - bc0]
        out[lr0 - r0:lr1 - r0, lc0 - c0:lc1 - c0] = piece if io == "f32" else f32_to_bf16_bits(piece)

    n = threads or _workers()
    if n == 1 or len(jobs) < 4:
        for j in jobs:
            work(j)
    else:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(work, jobs))
    return out


def shared_tensor(seed: int, tag: int, rows: tuple[int, int], N: int, io: str) -> np.ndarray:
    """N(0,1) draws for rows [r0, r1) of a [T, N] tensor shared by all channels."""
    r0, r1 = rows
    out_dtype = np.float32 if io == "f32" else np.uint16
    out = np.empty((r1 - r0, N), dtype=out_dtype)
    if r1 <= r0:
        return out
    for rb in range(r0 // ROW_BLOCK, (r1 - 1) // ROW_BLOCK + 1):
        block = _rng(seed, tag, rb, N).standard_normal((ROW_BLOCK, N), dtype=np.float32)
        br0 = rb * ROW_BLOCK
        lr0, lr1 = max(r0, br0), min(r1, br0 + ROW_BLOCK)
        piece = block[lr0 - br0:lr1 - br0]
        out[lr0 - r0:lr1 - r0] = piece if io == "f32" else f32_to_bf16_bits(piece)
    return out


def params(seed: int, d: int, N: int, K: int) -> dict[str, np.ndarray]:
    """Per-channel parameters (float32): A_log [d,N], D [d], dt_bias [d], conv_w [d,K], conv_b [d]."""
    rng = _rng(seed, TAG_PARAMS, d, N, K)
    dt0 = np.exp(rng.uniform(np.log(1e-3), np.log(0.1), size=d))
    dt_bias = (dt0 + np.log(-np.expm1(-dt0))).astype(np.float32)  # inverse of softplus at dt0
    conv_w = rng.uniform(-0.5, 0.5, size=(d, K)).astype(np.float32)
    conv_b = rng.uniform(-0.5, 0.5, size=d).astype(np.float32)
    A_log = np.tile(np.log(np.arange(1, N + 1, dtype=np.float64)), (d, 1)).astype(np.float32)
    D = np.ones(d, dtype=np.float32)
    return dict(A_log=A_log, D=D, dt_bias=dt_bias, conv_w=conv_w, conv_b=conv_b)


def params_per_channel(seed: int, d: int, N: int, K: int) -> dict[str, np.ndarray]:
    """Parameters that vary in every channel (and A_log in every state entry): A_log[c, n] =
    ln U[0.5, 16] drawn independently per (c, n), D[c] ~ N(0, 1); dt_bias, conv_w, conv_b as in
    ``params``.  A kernel that took A_log or D of the wrong channel or state entry would not
    match the oracle on these."""
    p = params(seed, d, N, K)
    rng = _rng(seed, TAG_PARAMS_VAR, d, N, K)
    p["A_log"] = np.log(rng.uniform(0.5, 16.0, size=(d, N))).astype(np.float32)
    p["D"] = rng.standard_normal(d).astype(np.float32)
    return p


def packed_lengths(seed: int, total: int, lo: int, hi: int) -> np.ndarray:
    """Lengths uniform on [lo, hi] drawn until they sum to ``total`` (last one cut)."""
    rng = _rng(seed, TAG_LENS, total, lo, hi)
    lens = []
    acc = 0
    while acc < total:
        v = int(rng.integers(lo, hi + 1))
        v = min(v, total - acc)
        lens.append(v)
        acc += v
    return np.asarray(lens, dtype=np.int64)


def cu_from_lengths(lens) -> np.ndarray:
    lens = np.asarray(lens, dtype=np.int64)
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    np.cumsum(lens, out=cu[1:])
    return cu.astype(np.int32)


def prefill_inputs(seed: int, T: int, d: int, N: int, io: str, rows: tuple[int, int] | None = None,
                   cols: tuple[int, int] | None = None, tag_base: int = 0) -> dict[str, np.ndarray]:
    """Token inputs x, z, dt [rows, cols] and B, C [rows, N] of a T-token stream."""
    rows = rows or (0, T)
    cols = cols or (0, d)
    return dict(
        x=token_tensor(seed, tag_base + TAG_X, rows, cols, io),
        z=token_tensor(seed, tag_base + TAG_Z, rows, cols, io),
        dt=token_tensor(seed, tag_base + TAG_DT, rows, cols, io),
        B=shared_tensor(seed, tag_base + TAG_B, rows, N, io),
        C=shared_tensor(seed, tag_base + TAG_C, rows, N, io),
    )


def grad_output(seed: int, T: int, d: int, io: str, rows: tuple[int, int] | None = None,
                cols: tuple[int, int] | None = None) -> np.ndarray:
    """dL/dy [rows, cols] of a T-token stream for the backward: N(0,1) draws."""
    return token_tensor(seed, TAG_DY, rows or (0, T), cols or (0, d), io)


def decode_inputs(seed: int, step: int, Bs: int, d: int, N: int, io: str,
                  cols: tuple[int, int] | None = None) -> dict[str, np.ndarray]:
    """Inputs of decode step ``step``: x, z, dt [Bs, cols] and B, C [Bs, N]."""
    return prefill_inputs(seed, Bs, d, N, io, rows=(0, Bs), cols=cols, tag_base=TAG_STEP * (step + 1))


def zero_states(S: int, d: int, N: int, K: int) -> tuple[np.ndarray, np.ndarray]:
    return (np.zeros((S, d, K - 1), dtype=np.float32), np.zeros((S, d, N), dtype=np.float32))


# The workloads: shapes and structure of the configurations the method is measured on.
WORKLOADS = {
    "tiny_f32": dict(S=1, L=64, d=16, N=4, K=4, io="f32"),
    "m130_prefill": dict(S=8, L=2048, d=1536, N=16, K=4, io="bf16"),
    "m1p4b_packed": dict(T=16384, lens=(128, 4096), d=4096, N=16, K=4, io="bf16"),
    "m7b_decode": dict(Bs=256, L_init=512, steps=128, d=8192, N=16, K=4, io="bf16"),
    "m2p8b_long": dict(S=1, L=131072, chunk=8192, decode_steps=64, d=5120, N=16, K=4, io="bf16"),
}
