"""The dt/B/C projections on the matrix cores against the oracle's fp64 products.

Tolerance: |g - r| <= 4e-3 |r| + 2e-4 rms(r) per output.  The products run with fp32-quality
operands (u and dt_in split into bf16 high and low parts) and fp32 accumulation, so the error is
the rounding of the outputs to bf16 (at most half an ulp, 2^-8 = 3.9e-3 relative) plus fp32
rounding of the sums.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_causal_amd as mm
from selective_state_space_causal_amd import inputs
from tests.gpu_util import dev, host, log

pytestmark = pytest.mark.gpu


def _case(seed, lens, d, N, R):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    x = inputs.token_tensor(seed, 1, (0, T), (0, d), "bf16")
    p = inputs.params(seed, d, N, 4)
    cs = rng.standard_normal((len(lens), d, 3)).astype(np.float32)
    cs = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(cs)).reshape(cs.shape)
    w_x = inputs.f32_to_bf16_bits((rng.standard_normal((d, R + 2 * N)) / np.sqrt(d)).astype(np.float32))
    w_dt = inputs.f32_to_bf16_bits((rng.standard_normal((R, d)) / np.sqrt(R)).astype(np.float32))
    return dict(x=x, conv_w=p["conv_w"], conv_b=p["conv_b"], cu=inputs.cu_from_lengths(lens), cs=cs, w_x=w_x,
                w_dt=w_dt, T=T, d=d, N=N, R=R)


def _close(g, r, what):
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    err = np.abs(g - r)
    bound = 4e-3 * np.abs(r) + 2e-4 * rms
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if r.size else 0.0
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    assert np.all(err <= bound), f"{what}: max err/bound {worst:.3g}"
    return worst


def _run(f):
    dt, B, C = mm.project(dev(f["x"]), dev(f["conv_w"]), dev(f["conv_b"]), dev(f["cu"]), dev(f["cs"]),
                          dev(f["w_x"]), dev(f["w_dt"]))
    torch.cuda.synchronize()
    return host(dt), host(B), host(C)


CASES = [
    ([37, 1, 0, 64, 2, 3, 90, 17], 48, 16, 3),   # short and empty sequences, d not a multiple of 32
    ([300, 200], 1536, 16, 48),                   # the 130m layer's d_inner and dt_rank
    ([100], 256, 8, 256),                         # the largest dt_rank, N < 16
    ([70, 5], 64, 16, 33),                        # dt_rank padded to 64, 65 output columns
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_project_vs_oracle(ci):
    lens, d, N, R = CASES[ci]
    f = _case(60 + ci, lens, d, N, R)
    log(f"[proj] case {ci}: lens={lens} d={d} N={N} R={R}")
    dt, B, C = _run(f)
    o = oracle.project(f["x"], f["conv_w"], f["conv_b"], f["cu"], f["cs"], f["w_x"], f["w_dt"], R, N)
    w = [_close(dt, o["dt"], "dt"), _close(B, o["B"], "B"), _close(C, o["C"], "C")]
    log(f"[proj] case {ci}: worst err/bound dt {w[0]:.3g} B {w[1]:.3g} C {w[2]:.3g}")


def test_project_m130_shape():
    """8 x 2048 tokens, d_inner 1536, dt_rank 48, N 16: every output against the oracle."""
    lens, d, N, R = [2048] * 8, 1536, 16, 48
    f = _case(130, lens, d, N, R)
    dt, B, C = _run(f)
    o = oracle.project(f["x"], f["conv_w"], f["conv_b"], f["cu"], f["cs"], f["w_x"], f["w_dt"], R, N)
    w = [_close(dt, o["dt"], "dt"), _close(B, o["B"], "B"), _close(C, o["C"], "C")]
    log(f"[proj] m130 shape: worst err/bound dt {w[0]:.3g} B {w[1]:.3g} C {w[2]:.3g}")


def test_project_feeds_prefill():
    """The projection's outputs are the prefill's dt, B, C: a packed call on them equals separate
    calls (the projections, like the scan, keep sequences apart) bit for bit."""
    lens, d, N, R = [50, 77], 64, 16, 8
    f = _case(7, lens, d, N, R)
    dt, B, C = mm.project(dev(f["x"]), dev(f["conv_w"]), dev(f["conv_b"]), dev(f["cu"]), dev(f["cs"]),
                          dev(f["w_x"]), dev(f["w_dt"]))
    for s in range(2):
        a, b = int(f["cu"][s]), int(f["cu"][s + 1])
        dts, Bs, Cs = mm.project(dev(f["x"][a:b]), dev(f["conv_w"]), dev(f["conv_b"]),
                                 torch.tensor([0, b - a], dtype=torch.int32, device="cuda"), dev(f["cs"][s:s + 1]),
                                 dev(f["w_x"]), dev(f["w_dt"]))
        torch.cuda.synchronize()
        assert torch.equal(dts, dt[a:b]) and torch.equal(Bs, B[a:b]) and torch.equal(Cs, C[a:b]), s


def _sweep_shape(nt):
    """N and R whose R + 2N needs exactly nt 16-column output tiles (one short of a full tile), so
    that every kernel instance (1..18 column tiles; dt_rank in 1..8 K steps of 32) runs once."""
    N = 4 if nt == 1 else (8 if nt == 2 else 16)
    return N, 16 * nt - 2 * N - 3


@pytest.mark.parametrize("nt", range(1, 19))
def test_project_every_instance(nt):
    N, R = _sweep_shape(nt)
    d = (48, 80, 144)[nt % 3]
    lens = [1, 2, 0, 57, 3, 40 + nt]
    f = _case(200 + nt, lens, d, N, R)
    log(f"[proj] instance nt={nt}: lens={lens} d={d} N={N} R={R} (K steps of dt_rank {(R + 31) // 32})")
    dt, B, C = _run(f)
    o = oracle.project(f["x"], f["conv_w"], f["conv_b"], f["cu"], f["cs"], f["w_x"], f["w_dt"], R, N)
    w = [_close(dt, o["dt"], "dt"), _close(B, o["B"], "B"), _close(C, o["C"], "C")]
    log(f"[proj] instance nt={nt}: worst err/bound dt {w[0]:.3g} B {w[1]:.3g} C {w[2]:.3g}")


def test_project_m1p4b_width():
    """The 1.4B layer's d_inner 4096 and dt_rank 128 (10 column tiles, 4 K steps of dt_rank) on
    ragged sequences: every output against the oracle."""
    lens, d, N, R = [5, 130, 2, 200], 4096, 16, 128
    f = _case(14, lens, d, N, R)
    dt, B, C = _run(f)
    o = oracle.project(f["x"], f["conv_w"], f["conv_b"], f["cu"], f["cs"], f["w_x"], f["w_dt"], R, N)
    w = [_close(dt, o["dt"], "dt"), _close(B, o["B"], "B"), _close(C, o["C"], "C")]
    log(f"[proj] 1.4B width: worst err/bound dt {w[0]:.3g} B {w[1]:.3g} C {w[2]:.3g}")


@pytest.mark.parametrize("offset", [0, 1])
def test_project_conv_state_paths(offset):
    """Sequences that start inside a 64-token tile read their initial conv state either from the
    workgroup's staged copy (up to three sequences per tile, conv_state 16-byte aligned) or from
    global memory (more sequences in the tile, or conv_state only 4-byte aligned: offset 1 float).
    Tiles here hold 1, 3 and 5 sequence starts; every output against the oracle."""
    lens, d, N, R = [64, 20, 30, 14, 9, 7, 5, 40, 3, 2, 90], 4096, 16, 128
    f = _case(300 + offset, lens, d, N, R)
    S = len(lens)
    flat = torch.zeros(S * d * 3 + 4, dtype=torch.float32, device="cuda")
    cs = flat[offset:offset + S * d * 3].view(S, d, 3)
    cs.copy_(dev(f["cs"]))
    log(f"[proj] conv state paths: lens={lens} offset={offset} (ptr % 16 = {cs.data_ptr() % 16})")
    dt, B, C = mm.project(dev(f["x"]), dev(f["conv_w"]), dev(f["conv_b"]), dev(f["cu"]), cs, dev(f["w_x"]),
                          dev(f["w_dt"]))
    torch.cuda.synchronize()
    o = oracle.project(f["x"], f["conv_w"], f["conv_b"], f["cu"], f["cs"], f["w_x"], f["w_dt"], R, N)
    w = [_close(host(dt), o["dt"], "dt"), _close(host(B), o["B"], "B"), _close(host(C), o["C"], "C")]
    log(f"[proj] conv state paths offset {offset}: worst err/bound dt {w[0]:.3g} B {w[1]:.3g} C {w[2]:.3g}")
