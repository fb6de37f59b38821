"""Helpers for the GPU tests: move seeded numpy inputs to the device, read results
back, and the tolerance rules the HIP path is held to.

Tolerances (floating point, against the fp64 oracle):
  * bf16 io (fp32 state):  |g - r| <= 1e-2 + 2e-2 |r|            (abs 1e-2, rel 2e-2)
  * fp32 io:               |g - r| <= 1e-4 (|r| + rms(r))          ("rel 1e-4", made
    well defined where r crosses zero by adding the array's rms to |r|)
  * conv_state is a copy of inputs and must match bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import torch


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, io: str | None = None) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    if a.dtype == np.int32:
        return torch.from_numpy(a).cuda()
    return torch.from_numpy(a.astype(np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> float64 numpy (bf16 widened exactly)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def within(g: np.ndarray, r: np.ndarray, io: str) -> tuple[bool, str]:
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if g.shape != r.shape:
        return False, f"shape {g.shape} vs {r.shape}"
    if not np.all(np.isfinite(g)):
        return False, "non-finite values in GPU result"
    err = np.abs(g - r)
    if io == "bf16":
        bound = 1e-2 + 2e-2 * np.abs(r)
    else:
        rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
        bound = 1e-4 * (np.abs(r) + rms)
    ok = bool(np.all(err <= bound))
    big = np.abs(r) >= (np.sqrt(np.mean(r * r)) if r.size else 0)
    mrel = float(np.max(err[big] / np.abs(r[big]))) if np.any(big) else 0.0
    norm = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    worst = float(np.max(err / bound)) if err.size else 0.0
    return ok, f"max err/bound {worst:.3g}, max rel (|r|>=rms) {mrel:.3g}, normwise {norm:.3g}"


def assert_within(g, r, io, what):
    ok, msg = within(g, r, io)
    assert ok, f"{what}: {msg}"
    return msg


def make_prefill(seed, lens, d, N, io, nonzero_state=True, extra_slots=0, varied=False):
    """Seeded inputs for a packed prefill (numpy).  Returns dict with cu, tokens, params, states.
    varied=True draws parameters that differ in every channel (inputs.params_per_channel)."""
    from selective_state_space_causal_amd import inputs

    T = int(np.sum(lens))
    tok = inputs.prefill_inputs(seed, T, d, N, io)
    p = (inputs.params_per_channel if varied else inputs.params)(seed, d, N, 4)
    S = len(lens)
    rng = np.random.default_rng(seed + 1000)
    if nonzero_state:
        cs = rng.standard_normal((S + extra_slots, d, 3)).astype(np.float32)
        if io == "bf16":  # the conv state holds raw inputs; keep them bf16-representable
            cs = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(cs)).reshape(cs.shape)
        ss = (0.5 * rng.standard_normal((S + extra_slots, d, N))).astype(np.float32)
    else:
        cs = np.zeros((S + extra_slots, d, 3), np.float32)
        ss = np.zeros((S + extra_slots, d, N), np.float32)
    return dict(cu=inputs.cu_from_lengths(lens), T=T, S=S, d=d, N=N, io=io, cs=cs, ss=ss, **tok, **p)


def run_gpu_prefill(case, chunk_len=0, slots=None, engine=0):
    """Run the HIP prefill on a case; returns (y, conv_state, ssm_state) as float64 numpy."""
    import selective_state_space_causal_amd as mm

    S = case["S"]
    cs = dev(case["cs"][:S] if slots is None else case["cs"])
    ss = dev(case["ss"][:S] if slots is None else case["ss"])
    y = mm.prefill(dev(case["x"]), dev(case["z"]), dev(case["dt"]), dev(case["B"]), dev(case["C"]),
                   dev(case["A_log"]), dev(case["D"]), dev(case["dt_bias"]), dev(case["conv_w"]),
                   dev(case["conv_b"]), dev(case["cu"]), cs, ss, chunk_len=chunk_len, engine=engine)
    torch.cuda.synchronize()
    return host(y), host(cs), host(ss)


def run_oracle_prefill(case, cols=None):
    import oracle

    S = case["S"]
    if cols is None:
        cols = np.arange(case["d"])
    return oracle.prefill(case["x"][:, cols], case["z"][:, cols], case["dt"][:, cols], case["B"], case["C"],
                          case["A_log"][cols], case["D"][cols], case["dt_bias"][cols], case["conv_w"][cols],
                          case["conv_b"][cols], case["cu"], case["cs"][:S][:, cols], case["ss"][:S][:, cols])
