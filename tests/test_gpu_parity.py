"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle on small and
ragged problems, plus the invariants: packed == separate, chunked == one-shot,
decode == scan, isolation, guards.  Needs an MI355X."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_causal_amd as mm
from selective_state_space_causal_amd import inputs
from tests.gpu_util import (assert_within, dev, host, log, make_prefill, run_gpu_prefill, run_oracle_prefill)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mm.load()
    oracle.build(force=False)


ENGINES = [mm.ENGINE_LANE, mm.ENGINE_ROW]


def _check_prefill(case, chunk_len, what, engine=0):
    log(f"[prefill] {what}: T={case['T']} S={case['S']} d={case['d']} N={case['N']} io={case['io']} "
        f"chunk={chunk_len} engine={engine}")
    y, cs, ss = run_gpu_prefill(case, chunk_len, engine=engine)
    yr, csr, ssr = run_oracle_prefill(case)
    assert_within(y, yr, case["io"], f"{what} y")
    assert_within(ss, ssr, case["io"], f"{what} ssm_state")
    assert np.array_equal(cs, csr), f"{what}: conv_state not bit-exact"


@pytest.mark.parametrize("engine", [0] + ENGINES)
def test_tiny_f32_workload(engine):
    """B=1, L=64, d=16, N=4, fp32 io, seed 0, zero initial states (the small workload)."""
    case = make_prefill(0, [64], 16, 4, "f32", nonzero_state=False)
    for ch in (0, 64, 16, 7):
        _check_prefill(case, ch, "tiny_f32", engine)


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("chunk", [0, 64, 100, 1000])
def test_ragged_packed(io, chunk, engine):
    """Several tiles, ragged channel block (d=200), empty and < K-1 sequences, nonzero slots."""
    case = make_prefill(3, [300, 1, 0, 2, 517, 64, 3], 200, 16, io)
    _check_prefill(case, chunk, f"ragged io={io}", engine)


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("N", [1, 3, 4, 5, 8, 9, 16])
def test_state_sizes(N, engine):
    case = make_prefill(10 + N, [70, 130, 33], 72, N, "f32")
    _check_prefill(case, 48, f"N={N}", engine)


def _offset_copy(a: np.ndarray) -> torch.Tensor:
    """a on the device, starting one element past an aligned allocation."""
    t = dev(a)
    buf = torch.zeros(t.numel() + 1, dtype=t.dtype, device="cuda")
    v = buf[1:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("chunk", [0, 64])
def test_row_staging_paths_agree(io, chunk):
    """The row engine stages a block with one 4-element load per lane when N = 16, d % 4 == 0 and
    the io tensors are aligned to 4 elements, and element by element otherwise.  The staging does
    no arithmetic, so the same inputs placed one element past an aligned address (element path)
    give bit-identical outputs; with d = 70 (not a multiple of 4) the element path matches the
    oracle."""
    row = mm.ENGINE_ROW
    lens = [300, 17, 0, 211, 5, 64]
    case = make_prefill(29, lens, 64, 16, io)
    log(f"[staging] io={io} chunk={chunk} d=64 aligned vs offset by one element")
    y, cs, ss = run_gpu_prefill(case, chunk, engine=row)
    S = case["S"]
    cs2, ss2 = dev(case["cs"][:S]), dev(case["ss"][:S])
    y2 = _offset_copy(np.zeros_like(case["x"]))
    mm.prefill(*(_offset_copy(case[k]) for k in ("x", "z", "dt", "B", "C")),
               *(dev(case[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b", "cu")), cs2, ss2,
               y=y2, chunk_len=chunk, engine=row)
    torch.cuda.synchronize()
    assert np.array_equal(host(y2), y), "element staging != vector staging (y)"
    assert np.array_equal(host(ss2), ss) and np.array_equal(host(cs2), cs), "element staging != vector (states)"
    case70 = make_prefill(31, lens, 70, 16, io)
    _check_prefill(case70, chunk, f"d=70 io={io}", row)


@pytest.mark.parametrize("engine", [0] + ENGINES)
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_many_short_sequences(io, engine):
    """Hundreds of short sequences (lengths 0..20, so many shorter than the conv window) with a
    ragged channel count: every sequence starts from its own slot, and empty ones stay untouched."""
    rng = np.random.default_rng(17)
    lens = rng.integers(0, 21, size=300).tolist()
    case = make_prefill(17, lens, 48, 16, io)
    _check_prefill(case, 0, f"300 short sequences io={io}", engine)


def test_auto_plan_picks_lane_engine_for_many_sequences():
    """8192 sequences x 64 channels reach the lane engine's wave threshold: the automatic plan
    uses it, and the result matches the oracle."""
    rng = np.random.default_rng(23)
    lens = rng.integers(1, 9, size=8192).tolist()
    case = make_prefill(23, lens, 64, 16, "bf16")
    assert mm.plan(case["S"], case["T"], 64, 16)["engine_name"] == "lane"
    _check_prefill(case, 0, "8192 sequences (auto -> lane)", 0)


@pytest.mark.parametrize("engine", ENGINES)
def test_sequences_ending_on_chunk_boundaries(engine):
    lens = [64, 64, 128, 1, 63, 64, 1, 16, 17, 15]
    case = make_prefill(5, lens, 64, 16, "bf16")
    for ch in (64, 32, 16, 65):
        _check_prefill(case, ch, "boundaries", engine)


@pytest.mark.parametrize("engine", ENGINES)
def test_packed_equals_separate_gpu(engine):
    """Chunks never cross a sequence boundary, so with the same chunk length and engine a packed run
    and per-sequence runs do the same arithmetic: bit-identical."""
    lens = [257, 3, 0, 900, 128, 2]
    case = make_prefill(7, lens, 128, 16, "bf16")
    T = case["T"]
    y, cs, ss = run_gpu_prefill(case, chunk_len=T, engine=engine)
    yc, csc, ssc = run_gpu_prefill(case, chunk_len=96, engine=engine)
    cu = case["cu"]
    for s in range(len(lens)):
        g0, g1 = int(cu[s]), int(cu[s + 1])
        sub = make_prefill(7, lens, 128, 16, "bf16")
        for k in ("x", "z", "dt", "B", "C"):
            sub[k] = case[k][g0:g1]
        sub.update(T=g1 - g0, S=1, cu=np.array([0, g1 - g0], np.int32), cs=case["cs"][s:s + 1],
                   ss=case["ss"][s:s + 1])
        if g1 == g0:
            continue
        ys, css, sss = run_gpu_prefill(sub, chunk_len=T, engine=engine)
        assert np.array_equal(ys, y[g0:g1]), f"seq {s}: packed != separate (single chunk)"
        assert np.array_equal(sss[0], ss[s]) and np.array_equal(css[0], cs[s])
        ysc, cssc, sssc = run_gpu_prefill(sub, chunk_len=96, engine=engine)
        assert np.array_equal(ysc, yc[g0:g1]), f"seq {s}: packed != separate (96-token chunks)"
        assert np.array_equal(sssc[0], ssc[s]) and np.array_equal(cssc[0], csc[s])
        assert_within(yc[g0:g1], ys, "bf16", f"seq {s} multi-chunk vs single chunk")
    # the empty sequence's slot is unchanged
    assert np.array_equal(cs[2], case["cs"][2]) and np.array_equal(ss[2], case["ss"][2])


def test_chunked_calls_equal_one_shot():
    """State carried across prefill calls continues the sequence (the state cache)."""
    L, d, N = 1000, 96, 16
    case = make_prefill(11, [L], d, N, "bf16")
    y1, cs1, ss1 = run_gpu_prefill(case)
    yr, csr, ssr = run_oracle_prefill(case)
    cs = dev(case["cs"])
    ss = dev(case["ss"])
    parts = []
    for a, b in ((0, 1), (1, 2), (2, 250), (250, 700), (700, 1000)):
        y = mm.prefill(dev(case["x"][a:b]), dev(case["z"][a:b]), dev(case["dt"][a:b]), dev(case["B"][a:b]),
                       dev(case["C"][a:b]), dev(case["A_log"]), dev(case["D"]), dev(case["dt_bias"]),
                       dev(case["conv_w"]), dev(case["conv_b"]), dev(np.array([0, b - a], np.int32)), cs, ss)
        parts.append(host(y))
    yk = np.concatenate(parts)
    assert np.array_equal(host(cs), csr)
    assert_within(yk, yr, "bf16", "chunked calls vs oracle")
    assert_within(host(ss), ssr, "bf16", "chunked calls state")
    assert_within(yk, y1, "bf16", "chunked calls vs one-shot")


def _decode_case(seed, Bs, d, N, io):
    tok = inputs.decode_inputs(seed, 0, Bs, d, N, io)
    p = inputs.params(seed, d, N, 4)
    rng = np.random.default_rng(seed)
    cs = rng.standard_normal((Bs, d, 3)).astype(np.float32)
    ss = (0.5 * rng.standard_normal((Bs, d, N))).astype(np.float32)
    return tok, p, cs, ss


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("Bs,d,N", [(1, 16, 4), (5, 200, 16), (3, 64, 7), (256, 512, 16), (9, 136, 8), (2, 72, 12)])
def test_decode_vs_oracle(io, Bs, d, N):
    log(f"[decode] Bs={Bs} d={d} N={N} io={io}")
    tok, p, cs, ss = _decode_case(Bs + d + N, Bs, d, N, io)
    csd, ssd = dev(cs), dev(ss)
    y = mm.decode(dev(tok["x"]), dev(tok["z"]), dev(tok["dt"]), dev(tok["B"]), dev(tok["C"]), dev(p["A_log"]),
                  dev(p["D"]), dev(p["dt_bias"]), dev(p["conv_w"]), dev(p["conv_b"]), csd, ssd)
    yr, csr, ssr = oracle.decode(tok["x"], tok["z"], tok["dt"], tok["B"], tok["C"], p["A_log"], p["D"],
                                 p["dt_bias"], p["conv_w"], p["conv_b"], cs, ss)
    assert_within(host(y), yr, io, "decode y")
    assert_within(host(ssd), ssr, io, "decode ssm_state")
    assert np.array_equal(host(csd), csr)


def test_decode_equals_prefill_one_token_sequences():
    """Decode equals a prefill of Bs one-token sequences: the states bit for bit (same per-element
    arithmetic); y within tolerance (the decode kernel sums the readout over four lane groups)."""
    Bs, d, N = 37, 130, 16
    tok, p, cs, ss = _decode_case(99, Bs, d, N, "bf16")
    args = [dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    cs1, ss1 = dev(cs), dev(ss)
    yd = mm.decode(dev(tok["x"]), dev(tok["z"]), dev(tok["dt"]), dev(tok["B"]), dev(tok["C"]), *args, cs1, ss1)
    cs2, ss2 = dev(cs), dev(ss)
    yp = mm.prefill(dev(tok["x"]), dev(tok["z"]), dev(tok["dt"]), dev(tok["B"]), dev(tok["C"]), *args,
                    dev(np.arange(Bs + 1, dtype=np.int32)), cs2, ss2)
    assert_within(host(yd), host(yp), "bf16", "decode vs one-token prefill")
    assert np.array_equal(host(ss1), host(ss2)) and np.array_equal(host(cs1), host(cs2))


def test_decode_steps_equal_scan():
    Bs, L, d, N = 4, 40, 64, 16
    case = make_prefill(21, [L] * Bs, d, N, "bf16")
    yp, csp, ssp = run_gpu_prefill(case)
    args = [dev(case[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    cs, ss = dev(case["cs"]), dev(case["ss"])
    for t in range(L):
        rows = [r * L + t for r in range(Bs)]
        yd = mm.decode(dev(case["x"][rows]), dev(case["z"][rows]), dev(case["dt"][rows]), dev(case["B"][rows]),
                       dev(case["C"][rows]), *args, cs, ss)
        assert_within(host(yd), yp[rows], "bf16", f"decode step {t}")
    assert np.array_equal(host(cs), csp)
    assert_within(host(ss), ssp, "bf16", "decode final state")


def test_isolation_and_guards():
    """Perturbing one sequence leaves the others bit-identical; nothing outside the
    outputs is written; slots past S are untouched; every y row is written."""
    lens = [50, 200, 7, 0, 90]
    d, N = 80, 16
    case = make_prefill(31, lens, d, N, "bf16", extra_slots=2)
    S, T = case["S"], case["T"]
    G = 64  # guard elements
    args = [dev(case[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]

    def run(xarr, chunk, engine):
        csf = dev(case["cs"])  # S + 2 slots
        ssf = dev(case["ss"])
        ybuf = torch.full((T * d + 2 * G,), float("nan"), dtype=torch.bfloat16, device="cuda")
        y = ybuf[G:G + T * d].view(T, d)
        mm.prefill(dev(xarr), dev(case["z"]), dev(case["dt"]), dev(case["B"]), dev(case["C"]), *args,
                   dev(case["cu"]), csf[:S], ssf[:S], y=y, chunk_len=chunk, engine=engine)
        torch.cuda.synchronize()
        return host(ybuf), host(csf), host(ssf)

    for chunk, engine in ((0, 0), (40, mm.ENGINE_LANE), (40, mm.ENGINE_ROW), (24, mm.ENGINE_ROW)):
        yb, csf, ssf = run(case["x"], chunk, engine)
        assert np.all(np.isnan(yb[:G])) and np.all(np.isnan(yb[G + T * d:])), "guard region written"
        assert np.all(np.isfinite(yb[G:G + T * d])), "a y element was not written"
        assert np.array_equal(csf[S:], case["cs"][S:]) and np.array_equal(ssf[S:], case["ss"][S:])
        x2 = case["x"].copy()
        cu = case["cu"]
        x2[cu[1]:cu[2]] ^= np.uint16(0x0040)  # perturb sequence 1 only
        yb2, csf2, ssf2 = run(x2, chunk, engine)
        y1 = yb[G:G + T * d].reshape(T, d)
        y2 = yb2[G:G + T * d].reshape(T, d)
        for s in (0, 2, 4):
            sl = slice(cu[s], cu[s + 1])
            assert np.array_equal(y1[sl], y2[sl]), f"sequence {s} changed"
            assert np.array_equal(csf[s], csf2[s]) and np.array_equal(ssf[s], ssf2[s])
        assert not np.array_equal(y1[cu[1]:cu[2]], y2[cu[1]:cu[2]])


def test_empty_inputs_are_noops():
    d, N = 64, 16
    p = inputs.params(0, d, N, 4)
    cs = torch.zeros((2, d, 3), device="cuda")
    ss = torch.ones((2, d, N), device="cuda")
    e = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    eb = torch.empty((0, N), dtype=torch.bfloat16, device="cuda")
    y = mm.prefill(e, e, e, eb, eb, dev(p["A_log"]), dev(p["D"]), dev(p["dt_bias"]), dev(p["conv_w"]),
                   dev(p["conv_b"]), dev(np.zeros(3, np.int32)), cs, ss)
    torch.cuda.synchronize()
    assert y.shape == (0, d)
    assert torch.all(ss == 1) and torch.all(cs == 0)


def test_decode_graph_capture_replays():
    """Decode steps captured in a HIP graph replay identically to eager launches."""
    Bs, d, N = 8, 256, 16
    tok, p, cs, ss = _decode_case(5, Bs, d, N, "bf16")
    args = [dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    xin = [dev(tok[k]) for k in ("x", "z", "dt", "B", "C")]
    cse, sse = dev(cs), dev(ss)
    eager = []
    for _ in range(3):
        eager.append(host(mm.decode(*xin, *args, cse, sse)))
    csg, ssg = dev(cs), dev(ss)
    yg = torch.empty((Bs, d), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mm.decode(*xin, *args, csg, ssg, y=yg, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(yg), eager[i]), f"replay {i}"
    assert np.array_equal(host(ssg), host(sse)) and np.array_equal(host(csg), host(cse))
