"""Parity of every HIP path with the fp64 oracle on parameters that differ in every channel
and state entry, on dt + dt_bias spread over [-40, 40], and through the plain C entry points.

* Parameters as a trained layer has them (the builder page holds A as a [d_inner, d_state]
  constant and D as [1, d_inner]): A_log[c, n] = ln U[0.5, 16] per (channel, state entry) and
  D[c] ~ N(0, 1) (inputs.params_per_channel).  A kernel that read A_log or D of the wrong channel
  or state entry, or dropped D, fails these.
* softplus(dt + dt_bias) over v in [-40, 40]: the kernels return v itself past v = 20 and use a
  series for e^v < 1/64 (v < -4.16); the measured workloads keep v in about [-11, 2].
* mamba_mixer_prefill and mamba_mixer_prefill_workspace_bytes called through ctypes as a C
  caller would, for plans that need no workspace, a chunked row plan and a lane plan.

Tolerances are those of every GPU test (bf16: |g - r| <= 1e-2 + 2e-2 |r|; fp32:
|g - r| <= 1e-4 (|r| + rms r); conv_state bit-exact).  Needs an MI355X.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_causal_amd as mm
from selective_state_space_causal_amd import inputs
from tests import test_gpu_backward as tb
from tests.gpu_util import assert_within, dev, host, log, make_prefill, run_gpu_prefill, run_oracle_prefill

pytestmark = pytest.mark.gpu

PRM = ("A_log", "D", "dt_bias", "conv_w", "conv_b")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mm.load()
    oracle.build(force=False)


def _check_prefill(case, chunk_len, what, engine=0):
    log(f"[params] {what}: T={case['T']} S={case['S']} d={case['d']} N={case['N']} io={case['io']} "
        f"chunk={chunk_len} engine={engine}")
    y, cs, ss = run_gpu_prefill(case, chunk_len, engine=engine)
    yr, csr, ssr = run_oracle_prefill(case)
    assert_within(y, yr, case["io"], f"{what} y")
    assert_within(ss, ssr, case["io"], f"{what} ssm_state")
    assert np.array_equal(cs, csr), f"{what}: conv_state not bit-exact"


def test_varied_parameters_really_vary():
    p = inputs.params_per_channel(0, 64, 16, 4)
    assert np.unique(p["A_log"]).size == 64 * 16
    assert np.unique(p["D"]).size == 64 and np.any(p["D"] < 0)
    A = np.exp(p["A_log"].astype(np.float64))
    assert A.min() >= 0.5 and A.max() <= 16.0


# ---------------------------------------------------------------- prefill, both engines


@pytest.mark.parametrize("engine", [mm.ENGINE_LANE, mm.ENGINE_ROW])
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("chunk", [0, 64, 100])
def test_prefill_varied(engine, io, chunk):
    """Ragged packing (empty and < K-1 sequences), a ragged channel block (d = 200), nonzero slots,
    whole sequences (chunk 0) and two chunk lengths (pass 1, carries, pass 2)."""
    case = make_prefill(501, [300, 1, 0, 2, 517, 64, 3], 200, 16, io, varied=True)
    _check_prefill(case, chunk, f"varied io={io}", engine)


@pytest.mark.parametrize("engine", [mm.ENGINE_LANE, mm.ENGINE_ROW])
@pytest.mark.parametrize("N", [1, 5, 8, 12])
def test_prefill_varied_state_sizes(engine, N):
    """N < 16: the lane engine's 4- and 8-entry variants and the row engine's masked lanes."""
    case = make_prefill(510 + N, [70, 130, 33], 72, N, "f32", varied=True)
    _check_prefill(case, 48, f"varied N={N}", engine)


def test_prefill_varied_element_staging():
    """The row engine's element staging (d not a multiple of 4)."""
    case = make_prefill(520, [300, 17, 0, 211, 5, 64], 70, 16, "bf16", varied=True)
    for chunk in (0, 64):
        _check_prefill(case, chunk, "varied d=70", mm.ENGINE_ROW)


# ---------------------------------------------------------------- decode


def _decode_stream(seed, steps, Bs, d, N, io):
    toks = [inputs.decode_inputs(seed, s, Bs, d, N, io) for s in range(steps)]
    p = inputs.params_per_channel(seed, d, N, 4)
    rng = np.random.default_rng(seed)
    cs = rng.standard_normal((Bs, d, 3)).astype(np.float32)
    if io == "bf16":  # the conv state holds raw inputs; keep them bf16-representable
        cs = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(cs)).reshape(cs.shape)
    ss = (0.5 * rng.standard_normal((Bs, d, N))).astype(np.float32)
    return toks, p, cs, ss


def _offset(t: torch.Tensor) -> torch.Tensor:
    """t copied to one element past an aligned allocation (defeats 4-element vector loads)."""
    buf = torch.zeros(t.numel() + 1, dtype=t.dtype, device="cuda")
    v = buf[1:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("path", ["vec", "generic_N12", "generic_unaligned"])
def test_decode_varied(io, path):
    """Six steps from nonzero states, y of every step and the final states against the oracle.
    N = 16 with aligned B/C runs the streaming kernel (four lanes per channel, A_log read as
    float4 per lane); N = 12 or B/C one element off alignment run the generic kernel."""
    N = 12 if path == "generic_N12" else 16
    Bs, d, steps = 9, 264, 6
    toks, p, cs, ss = _decode_stream(530 + N, steps, Bs, d, N, io)
    prm = [dev(p[k]) for k in PRM]
    csd, ssd = dev(cs), dev(ss)
    cs_o, ss_o = cs, ss
    log(f"[params] decode {path} io={io} Bs={Bs} d={d} N={N}")
    for s, t in enumerate(toks):
        tk = [dev(t[k]) for k in ("x", "z", "dt", "B", "C")]
        if path == "generic_unaligned":
            tk[3], tk[4] = _offset(tk[3]), _offset(tk[4])
        y = mm.decode(*tk, *prm, csd, ssd)
        yr, cs_o, ss_o = oracle.decode(t["x"], t["z"], t["dt"], t["B"], t["C"], *[p[k] for k in PRM], cs_o, ss_o)
        assert_within(host(y), yr, io, f"decode {path} step {s} y")
    assert_within(host(ssd), ss_o, io, f"decode {path} ssm_state")
    assert np.array_equal(host(csd), cs_o)


def test_decode_varied_7b_shape():
    """Batch 256, d_inner 8192 (the streaming kernel at its measured shape): every step's y on
    sampled channels, the final states on the same channels."""
    Bs, d, N, steps = 256, 8192, 16, 4
    toks, p, cs, ss = _decode_stream(540, steps, Bs, d, N, "bf16")
    ch = np.unique(np.concatenate([[0, 1, 2, 3, 4095, 4096, d - 1],
                                   np.random.default_rng(540).choice(d, 40, replace=False)]))
    idx = torch.from_numpy(ch.astype(np.int64)).cuda()
    prm = [dev(p[k]) for k in PRM]
    csd, ssd = dev(cs), dev(ss)
    cs_o, ss_o = cs[:, ch], ss[:, ch]
    for s, t in enumerate(toks):
        y = mm.decode(*[dev(t[k]) for k in ("x", "z", "dt", "B", "C")], *prm, csd, ssd)
        yr, cs_o, ss_o = oracle.decode(t["x"][:, ch], t["z"][:, ch], t["dt"][:, ch], t["B"], t["C"],
                                       *[p[k][ch] for k in PRM], cs_o, ss_o)
        assert_within(host(y.index_select(1, idx)), yr, "bf16", f"7b decode step {s} y")
    assert_within(host(ssd)[:, ch], ss_o, "bf16", "7b decode ssm_state")
    assert np.array_equal(host(csd)[:, ch], cs_o)


# ---------------------------------------------------------------- replay decode


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_replay_varied(io):
    """Replay steps equal the eager decode bit for bit and the oracle's replay within tolerance;
    the multi-step call emits the same outputs and commits the same state."""
    W, Bs, d, N = 4, 6, 328, 16
    toks, p, cs, ss = _decode_stream(550, W, Bs, d, N, io)
    prm = [dev(p[k]) for k in PRM]
    dt_ = torch.bfloat16 if io == "bf16" else torch.float32
    ring = {k: np.stack([t[k] for t in toks]) for k in ("x", "dt", "B", "z", "C")}
    R = {k: dev(v) for k, v in ring.items()}
    # eager reference
    cse, sse = dev(cs), dev(ss)
    ye = []
    for t in toks:
        ye.append(host(mm.decode(*[dev(t[k]) for k in ("x", "z", "dt", "B", "C")], *prm, cse, sse)))
    # single-step replay calls
    csd, ssd = dev(cs), dev(ss)
    for k in range(W):
        y = mm.decode_replay(R["x"], R["dt"], R["B"], R["z"][k], R["C"][k], *prm, csd, ssd, k)
        yh = host(y)
        assert np.array_equal(yh, ye[k]), f"replay step {k} != eager"
        yo, cso, sso = oracle.decode_replay(ring["x"], ring["dt"], ring["B"], k, toks[k]["z"], toks[k]["C"],
                                            *[p[q] for q in PRM], cs, ss)
        assert_within(yh, yo, io, f"replay step {k} vs oracle")
    assert np.array_equal(host(csd), host(cse)) and np.array_equal(host(ssd), host(sse))
    assert_within(host(ssd), sso, io, "replay checkpoint vs oracle")
    assert np.array_equal(host(csd), cso)
    # one multi-step call, committing after step 2
    csm, ssm = dev(cs), dev(ss)
    ym = torch.full((W, Bs, d), float("nan"), dtype=dt_, device="cuda")
    mm.decode_replay_multi(R["x"], R["dt"], R["B"], R["z"], R["C"], *prm, csm, ssm, 0, 3, 2, y_ring=ym)
    for k in range(W):
        assert np.array_equal(host(ym[k]), ye[k]), f"multi step {k} != eager"
    _, cs2, ss2 = oracle.decode_replay(ring["x"], ring["dt"], ring["B"], 2, toks[2]["z"], toks[2]["C"],
                                       *[p[q] for q in PRM], cs, ss)
    assert_within(host(ssm), ss2, io, "multi commit after step 2 vs oracle")
    assert np.array_equal(host(csm), cs2)


# ---------------------------------------------------------------- backward and training forward


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("ci", [0, 1])
def test_backward_varied(io, ci):
    """All twelve gradients against the oracle's reverse mode, with the standalone backward and
    with the training forward's checkpoints (whole sequences and 32-token chunks)."""
    lens, d, N = [([37, 1, 0, 64, 2, 3, 90, 17], 40, 16), ([200, 5, 111], 24, 5)][ci]
    case = make_prefill(560 + ci, lens, d, N, io, varied=True)
    dy = inputs.grad_output(560 + ci, case["T"], d, io)
    log(f"[params] backward case {ci} io={io} lens={lens} d={d} N={N}")
    r = tb.oracle_backward(case, dy)
    tb.check_all(tb.gpu_backward(case, dy), r, io, f"varied case {ci} {io}")
    S = case["S"]
    for chunk_len in (0, 32):
        y, ck, cs, ss = tb._train(case, chunk_len)
        yr, csr, ssr = run_oracle_prefill(case)
        assert_within(host(y), yr, io, f"train forward chunk {chunk_len} y")
        assert_within(host(ss), ssr, io, f"train forward chunk {chunk_len} ssm_state")
        assert np.array_equal(host(cs), csr)
        g = mm.prefill_backward(*[dev(case[k]) for k in ("x", "z", "dt", "B", "C")], *[dev(case[k]) for k in PRM],
                                dev(case["cu"]), dev(case["cs"][:S]), None, dev(dy), ckpt=ck)
        torch.cuda.synchronize()
        tb.check_all({k: host(v) for k, v in g.items()}, r, io, f"varied from checkpoints chunk {chunk_len}")


# ---------------------------------------------------------------- full size, sampled channels


def test_m1p4b_packed_varied_sampled():
    """The 1.4B-shaped packed stream (lengths U[128, 4096] to 16384 tokens, d_inner 4096, bf16)
    with per-channel parameters, in the plan bench.py times and in two chunked plans (row and
    lane engines): sampled channels against the oracle."""
    d, N = 4096, 16
    lens = inputs.packed_lengths(0, 16384, 128, 4096)
    T, S = int(lens.sum()), len(lens)
    tok = inputs.prefill_inputs(0, T, d, N, "bf16")
    p = inputs.params_per_channel(0, d, N, 4)
    cu = inputs.cu_from_lengths(lens)
    rng = np.random.default_rng(570)
    cs = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(rng.standard_normal((S, d, 3)).astype(np.float32)))
    cs = cs.reshape(S, d, 3)
    ss = (0.5 * rng.standard_normal((S, d, N))).astype(np.float32)
    ch = np.unique(np.concatenate([[0, 15, 16, 2047, 2048, d - 1], rng.choice(d, 40, replace=False)]))
    idx = torch.from_numpy(ch.astype(np.int64)).cuda()
    yr, csr, ssr = oracle.prefill(*[tok[k][:, ch] for k in ("x", "z", "dt")], tok["B"], tok["C"],
                                  *[p[k][ch] for k in PRM], cu, cs[:, ch], ss[:, ch])
    for chunk, engine in ((0, 0), (1024, mm.ENGINE_ROW), (1024, mm.ENGINE_LANE)):
        log(f"[params] m1p4b varied S={S} chunk={chunk} engine={engine}")
        csd, ssd = dev(cs), dev(ss)
        y = mm.prefill(*[dev(tok[k]) for k in ("x", "z", "dt", "B", "C")], *[dev(p[k]) for k in PRM], dev(cu),
                       csd, ssd, chunk_len=chunk, engine=engine)
        assert_within(host(y.index_select(1, idx)), yr, "bf16", f"m1p4b varied chunk {chunk} engine {engine} y")
        assert_within(host(ssd)[:, ch], ssr, "bf16", f"m1p4b varied chunk {chunk} ssm_state")
        assert np.array_equal(host(csd)[:, ch], csr)
        del y


# ---------------------------------------------------------------- softplus extremes


def _sweep_case(seed, lens, d, N, io):
    """dt + dt_bias spread over about [-41, 41]: dt ~ U[-40, 40] (io-rounded), dt_bias ~ U[-1, 1]."""
    case = make_prefill(seed, lens, d, N, io, varied=True)
    rng = np.random.default_rng(seed)
    dt = rng.uniform(-40.0, 40.0, size=(case["T"], d)).astype(np.float32)
    case["dt"] = inputs.f32_to_bf16_bits(dt) if io == "bf16" else dt
    case["dt_bias"] = rng.uniform(-1.0, 1.0, size=d).astype(np.float32)
    v = oracle.as_f64(case["dt"]) + case["dt_bias"][None, :].astype(np.float64)
    # the case reaches the clamp (v > 20), the series (e^v < 1/64) and the log form between
    assert (v > 20).mean() > 0.2 and (v < -4.2).mean() > 0.3 and ((v > -4) & (v < 20)).mean() > 0.2
    return case


@pytest.mark.parametrize("engine", [mm.ENGINE_LANE, mm.ENGINE_ROW])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_softplus_sweep_prefill(engine, io):
    case = _sweep_case(580, [200, 3, 0, 333, 40], 96, 16, io)
    for chunk in (0, 64):
        _check_prefill(case, chunk, f"softplus sweep io={io}", engine)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("N", [16, 12])
def test_softplus_sweep_decode_and_replay(io, N):
    """Decode (streaming kernel for N = 16, generic for N = 12) and, for N = 16, the replay decode,
    on dt + dt_bias over [-41, 41]."""
    Bs, d, W = 64, 96, 4
    toks, p, cs, ss = _decode_stream(590 + N, W, Bs, d, N, io)
    rng = np.random.default_rng(590)
    p["dt_bias"] = rng.uniform(-1.0, 1.0, size=d).astype(np.float32)
    for t in toks:
        dt = rng.uniform(-40.0, 40.0, size=(Bs, d)).astype(np.float32)
        t["dt"] = inputs.f32_to_bf16_bits(dt) if io == "bf16" else dt
    prm = [dev(p[k]) for k in PRM]
    csd, ssd = dev(cs), dev(ss)
    cs_o, ss_o = cs, ss
    ye = []
    for s, t in enumerate(toks):
        y = mm.decode(*[dev(t[k]) for k in ("x", "z", "dt", "B", "C")], *prm, csd, ssd)
        yr, cs_o, ss_o = oracle.decode(t["x"], t["z"], t["dt"], t["B"], t["C"], *[p[k] for k in PRM], cs_o, ss_o)
        ye.append(host(y))
        assert_within(ye[-1], yr, io, f"sweep decode N={N} step {s} y")
    assert_within(host(ssd), ss_o, io, f"sweep decode N={N} ssm_state")
    assert np.array_equal(host(csd), cs_o)
    if N != 16:
        return
    R = {k: dev(np.stack([t[k] for t in toks])) for k in ("x", "dt", "B", "z", "C")}
    csr, ssr = dev(cs), dev(ss)
    for k in range(W):
        y = mm.decode_replay(R["x"], R["dt"], R["B"], R["z"][k], R["C"][k], *prm, csr, ssr, k)
        assert np.array_equal(host(y), ye[k]), f"sweep replay step {k} != eager"
    assert np.array_equal(host(ssr), host(ssd)) and np.array_equal(host(csr), host(csd))


def test_softplus_sweep_backward():
    """The backward's softplus derivative over the same range (fp32 io)."""
    case = _sweep_case(600, [90, 2, 0, 61], 32, 16, "f32")
    dy = inputs.grad_output(600, case["T"], 32, "f32")
    tb.check_all(tb.gpu_backward(case, dy), tb.oracle_backward(case, dy), "f32", "softplus sweep backward")


# ---------------------------------------------------------------- the plain C entry points


def _c_prefill(case, workspace, wbytes):
    lib = mm.load()
    S, T, d, N = case["S"], case["T"], case["d"], case["N"]
    t = {k: dev(case[k]) for k in ("x", "z", "dt", "B", "C", *PRM, "cu")}
    cs, ss = dev(case["cs"][:S]), dev(case["ss"][:S])
    y = torch.full((T, d), float("nan"), dtype=t["x"].dtype, device="cuda")
    ptr = lambda a: ctypes.c_void_p(a.data_ptr())
    io = mm.MM_IO_BF16 if case["io"] == "bf16" else mm.MM_IO_F32
    rc = lib.mamba_mixer_prefill(*[ptr(t[k]) for k in ("x", "z", "dt", "B", "C", *PRM, "cu")], ptr(cs), ptr(ss),
                                 ptr(y), S, T, d, N, 4, io, workspace, wbytes,
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return rc, y, cs, ss


@pytest.mark.parametrize("shape", ["whole", "row_chunked", "lane"])
def test_plain_c_prefill_entry_point(shape):
    """mamba_mixer_prefill with the workspace mamba_mixer_prefill_workspace_bytes reports, called
    through ctypes: matches the oracle; a workspace one byte short is refused before any launch."""
    lens, d = {"whole": ([300, 1, 0, 217], 80), "row_chunked": ([3000], 64),
               "lane": ([3, 1, 0, 2] * 2048 + [5], 64)}[shape]
    case = make_prefill(610, lens, d, 16, "bf16", varied=True)
    S, T = case["S"], case["T"]
    lib = mm.load()
    need = int(lib.mamba_mixer_prefill_workspace_bytes(S, T, d, 16, 4))
    plan = mm.plan(S, T, d, 16)
    log(f"[params] plain C prefill {shape}: S={S} T={T} d={d} plan={plan['kernels']} workspace={need}")
    assert need == plan["workspace_bytes"]
    assert (need == 0) == (shape == "whole")
    assert plan["engine_name"] == ("lane" if shape == "lane" else "row")
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    if need > 0:
        rc, _, _, _ = _c_prefill(case, ctypes.c_void_p(ws.data_ptr()), need - 1)
        assert rc == -5, f"short workspace: status {rc}"  # MM_ERR_WORKSPACE
    rc, y, cs, ss = _c_prefill(case, ctypes.c_void_p(ws.data_ptr()) if need > 0 else None, need)
    assert rc == 0, mm.status_string(rc)
    yr, csr, ssr = run_oracle_prefill(case)
    assert_within(host(y), yr, "bf16", f"plain C {shape} y")
    assert_within(host(ss), ssr, "bf16", f"plain C {shape} ssm_state")
    assert np.array_equal(host(cs), csr)


def test_check_cu_seqlens_before_calls():
    """With the binding's cu_seqlens check on, a call whose cu_seqlens does not end at T raises
    before anything is launched (the array used here stays inside the buffers, so the call would
    be harmless even unchecked), and a valid one runs as usual."""
    lens, d, N = [5, 7], 32, 16
    T = sum(lens)
    tok = inputs.prefill_inputs(4, T, d, N, "f32")
    p = inputs.params_per_channel(4, d, N, 4)
    cs, ss = inputs.zero_states(len(lens), d, N, 4)
    args = [dev(tok[k]) for k in ("x", "z", "dt", "B", "C")] + [dev(p[k]) for k in PRM]
    saved = mm.CHECK_CU
    mm.CHECK_CU = True
    try:
        bad = dev(np.array([0, 5, T - 1], dtype=np.int32))
        with pytest.raises(mm.MambaMixError):
            mm.prefill(*args, bad, dev(cs), dev(ss))
        y = mm.prefill(*args, dev(inputs.cu_from_lengths(lens)), dev(cs), dev(ss))
        torch.cuda.synchronize()
        assert np.all(np.isfinite(host(y)))
    finally:
        mm.CHECK_CU = saved
