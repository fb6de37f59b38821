"""Replay decode (checkpoint + buffered inputs) on the GPU: bit-identical to the eager decode
step by step, and within tolerance of the oracle's replay."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_causal_amd as mm
from selective_state_space_causal_amd import inputs
from tests.gpu_util import assert_within, dev, host, log

pytestmark = pytest.mark.gpu


def _stream(seed, steps, Bs, d, N, io):
    toks = [inputs.decode_inputs(seed, s, Bs, d, N, io) for s in range(steps)]
    p = inputs.params(seed, d, N, 4)
    rng = np.random.default_rng(seed)
    cs = rng.standard_normal((Bs, d, 3)).astype(np.float32)
    if io == "bf16":  # the conv state holds raw inputs; keep them bf16-representable
        cs = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(cs)).reshape(cs.shape)
    ss = (0.5 * rng.standard_normal((Bs, d, N))).astype(np.float32)
    return toks, p, cs, ss


def _run_replay(toks, p, cs, ss, W, commit_at=()):
    """Feed the steps through the replay path; returns per-step y and the checkpoint after each
    committing step."""
    steps = len(toks)
    Bs, d = toks[0]["x"].shape
    N = toks[0]["B"].shape[1]
    io = torch.bfloat16 if toks[0]["x"].dtype == np.uint16 else torch.float32
    prm = [dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    csd, ssd = dev(cs), dev(ss)
    xr = torch.zeros((W, Bs, d), dtype=io, device="cuda")
    dr = torch.zeros((W, Bs, d), dtype=io, device="cuda")
    br = torch.zeros((W, Bs, N), dtype=io, device="cuda")
    ys, ckpts = [], {}
    k = 0
    for s in range(steps):
        xr[k].copy_(dev(toks[s]["x"]))
        dr[k].copy_(dev(toks[s]["dt"]))
        br[k].copy_(dev(toks[s]["B"]))
        commit = s in commit_at
        y = mm.decode_replay(xr, dr, br, dev(toks[s]["z"]), dev(toks[s]["C"]), *prm, csd, ssd, k, commit=commit)
        ys.append(host(y))
        if commit or k == W - 1:
            ckpts[s] = (host(csd), host(ssd))
            k = 0
        else:
            k += 1
    return ys, ckpts


def _run_eager(toks, p, cs, ss, keep):
    """Eager decode of the same steps; returns per-step y and the states after the steps in keep."""
    prm = [dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    csd, ssd = dev(cs), dev(ss)
    ys, states = [], {}
    for s, t in enumerate(toks):
        y = mm.decode(dev(t["x"]), dev(t["z"]), dev(t["dt"]), dev(t["B"]), dev(t["C"]), *prm, csd, ssd)
        ys.append(host(y))
        if s in keep:
            states[s] = (host(csd), host(ssd))
    return ys, states


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_replay_equals_eager_decode(io, W):
    """Every step's y and every committed checkpoint equal the eager decode bit for bit (the replay
    performs the eager step's operations in the same order), including an early commit."""
    Bs, d, N = 5, 200, 16
    steps = 3 * W + 2
    log(f"[replay] W={W} io={io} Bs={Bs} d={d} steps={steps}")
    toks, p, cs, ss = _stream(70 + W, steps, Bs, d, N, io)
    commit_at = {W + 1} if W > 2 else set()  # an explicit commit in the middle of the second window
    yr, ck = _run_replay(toks, p, cs, ss, W, commit_at)
    ye, st = _run_eager(toks, p, cs, ss, set(ck))
    for s in range(steps):
        assert np.array_equal(yr[s], ye[s]), f"step {s}: y differs from the eager decode"
    assert ck, "no checkpoint was committed"
    for s, (c1, s1) in ck.items():
        assert np.array_equal(c1, st[s][0]) and np.array_equal(s1, st[s][1]), f"checkpoint after step {s}"


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_replay_vs_oracle(io):
    W, Bs, d, N = 4, 7, 136, 16
    toks, p, cs, ss = _stream(91, W, Bs, d, N, io)
    yr, ck = _run_replay(toks, p, cs, ss, W)
    ring = {k: np.stack([t[k] for t in toks]) for k in ("x", "dt", "B")}
    for k in range(W):
        y, csr, ssr = oracle.decode_replay(ring["x"], ring["dt"], ring["B"], k, toks[k]["z"], toks[k]["C"],
                                           p["A_log"], p["D"], p["dt_bias"], p["conv_w"], p["conv_b"], cs, ss)
        assert_within(yr[k], y, io, f"replay step {k} y")
    c1, s1 = ck[W - 1]
    assert np.array_equal(c1, csr)
    assert_within(s1, ssr, io, "replay checkpoint")


def test_replay_7b_shape_window():
    """The 7B-shaped decode (batch 256, d 8192) over one full window and a bit more."""
    W, Bs, d, N = 4, 256, 8192, 16
    steps = W + 1
    toks, p, cs, ss = _stream(5, steps, Bs, d, N, "bf16")
    yr, ck = _run_replay(toks, p, cs, ss, W)
    ye, st = _run_eager(toks, p, cs, ss, {W - 1})
    for s in range(steps):
        assert np.array_equal(yr[s], ye[s]), s
    assert np.array_equal(ck[W - 1][1], st[W - 1][1])


def _rings(toks, W, io):
    def stack(key):
        return dev(np.stack([t[key] for t in toks[:W]]))
    return {k: stack(k) for k in ("x", "dt", "B", "z", "C")}


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_replay_multi_equals_eager_steps(io):
    """One call emitting window steps k0..k1 equals the eager decode step by step, bit for bit,
    with no state written unless a commit step is given (then the state after that step)."""
    W, Bs, d, N = 4, 3, 300, 16
    toks, p, cs, ss = _stream(33, W, Bs, d, N, io)
    prm = [dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    ye, st = _run_eager(toks, p, cs, ss, set(range(W)))
    R = _rings(toks, W, io)
    for k0, k1, cstep in ((0, 3, -1), (1, 2, -1), (2, 2, 2), (0, 3, 1), (3, 3, 0), (0, 1, 1)):
        csd, ssd = dev(cs), dev(ss)
        y = torch.full((W, Bs, d), float("nan"), dtype=R["x"].dtype, device="cuda")
        mm.decode_replay_multi(R["x"], R["dt"], R["B"], R["z"], R["C"], *prm, csd, ssd, k0, k1, cstep, y_ring=y)
        yh = host(y)
        for t in range(W):
            if k0 <= t <= k1:
                assert np.array_equal(yh[t], ye[t]), (k0, k1, cstep, t)
            else:
                assert np.all(np.isnan(yh[t])), f"slot {t} written outside {k0}..{k1}"
        if (k0, k1) == (0, 3):  # and against the oracle's replay of each step
            ring = {k: np.stack([t[k] for t in toks]) for k in ("x", "dt", "B")}
            for t in range(W):
                yo, _, _ = oracle.decode_replay(ring["x"], ring["dt"], ring["B"], t, toks[t]["z"], toks[t]["C"],
                                                p["A_log"], p["D"], p["dt_bias"], p["conv_w"], p["conv_b"], cs, ss)
                assert_within(yh[t], yo, io, f"multi step {t} vs oracle")
        if cstep < 0:
            assert np.array_equal(host(csd), cs) and np.array_equal(host(ssd), ss), "state written without commit"
        else:
            assert np.array_equal(host(csd), st[cstep][0]) and np.array_equal(host(ssd), st[cstep][1]), (k0, k1, cstep)


def test_speculative_accept_prefix_and_continue():
    """Draft four tokens, verify all four outputs in one call without writing state, accept two
    (commit after step 1), then continue from the accepted prefix with two new tokens: every
    output equals the eager decode that took exactly the accepted tokens."""
    W, Bs, d, N = 4, 4, 256, 16
    toks, p, cs, ss = _stream(44, 6, Bs, d, N, "bf16")
    prm = [dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    draft = toks[:4]
    R = _rings(draft, W, "bf16")
    csd, ssd = dev(cs), dev(ss)
    y = mm.decode_replay_multi(R["x"], R["dt"], R["B"], R["z"], R["C"], *prm, csd, ssd, 0, 3, -1)
    ye, _ = _run_eager(draft, p, cs, ss, set())
    for t in range(4):
        assert np.array_equal(host(y[t]), ye[t]), t
    # accept tokens 0 and 1: commit after window step 1 (a second call, outputs of step 1 again)
    mm.decode_replay_multi(R["x"], R["dt"], R["B"], R["z"], R["C"], *prm, csd, ssd, 1, 1, 1)
    # continue with two new tokens (toks 4 and 5) in a fresh window
    accepted = toks[:2] + toks[4:6]
    ye2, _ = _run_eager(accepted, p, cs, ss, set())
    R2 = _rings(toks[4:6] + toks[4:6], W, "bf16")  # slots 0, 1 hold the new tokens
    y2 = mm.decode_replay_multi(R2["x"], R2["dt"], R2["B"], R2["z"], R2["C"], *prm, csd, ssd, 0, 1, -1)
    assert np.array_equal(host(y2[0]), ye2[2]) and np.array_equal(host(y2[1]), ye2[3])


# ---------------------------------------------------------------- dual-precision checkpoint


def _run_dual(toks, p, cs, ss, W):
    """Feed the steps through the dual-precision replay; returns per-step y, the fp32 and bf16
    checkpoints after every committing step, and the checkpoint each window started from."""
    Bs, d = toks[0]["x"].shape
    N = toks[0]["B"].shape[1]
    prm = [dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    csd, ssd = dev(cs), dev(ss)
    clo, slo = mm.replay_checkpoint_lo(csd, ssd)
    xr = torch.zeros((W, Bs, d), dtype=torch.bfloat16, device="cuda")
    dr = torch.zeros_like(xr)
    br = torch.zeros((W, Bs, N), dtype=torch.bfloat16, device="cuda")
    ys, ckpts, starts = [], {}, {0: (cs, ss)}
    k = 0
    for s, t in enumerate(toks):
        xr[k].copy_(dev(t["x"]))
        dr[k].copy_(dev(t["dt"]))
        br[k].copy_(dev(t["B"]))
        y = mm.decode_replay_dual(xr, dr, br, dev(t["z"]), dev(t["C"]), *prm, csd, ssd, clo, slo, k)
        ys.append(host(y))
        if k == W - 1:
            ckpts[s] = (host(csd), host(ssd), host(clo), host(slo))
            starts[s + 1] = (host(csd), host(ssd))
            k = 0
        else:
            k += 1
    return ys, ckpts, starts


@pytest.mark.parametrize("W", [2, 4])
def test_replay_dual_precision(W):
    """Steps that do not commit give the oracle's outputs from the bf16-rounded checkpoint (within
    the bf16 tolerance); committing steps equal the eager decode bit for bit, output and state;
    the bf16 copy written at a commit is the fp32 checkpoint rounded to nearest even (bit for
    bit), with conv entry 3 zero."""
    Bs, d, N = 6, 200, 16
    steps = 2 * W + 1
    toks, p, cs, ss = _stream(80 + W, steps, Bs, d, N, "bf16")
    log(f"[replay-dual] W={W} Bs={Bs} d={d} steps={steps}")
    yd, ck, starts = _run_dual(toks, p, cs, ss, W)
    ye, st = _run_eager(toks, p, cs, ss, set(ck))
    prm = [p[k] for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    for s in range(steps):
        w0 = (s // W) * W
        k = s - w0
        if k == W - 1:
            assert np.array_equal(yd[s], ye[s]), f"committing step {s}: y differs from the eager decode"
            continue
        cs0, ss0 = starts[w0]
        ring = {q: np.stack([toks[w0 + i][q] for i in range(W) if w0 + i < steps]) for q in ("x", "dt", "B")}
        yo, _, _ = oracle.decode_replay_lo(ring["x"], ring["dt"], ring["B"], k, toks[s]["z"], toks[s]["C"], *prm,
                                           cs0, ss0)
        assert_within(yd[s], yo, "bf16", f"dual step {s} (window step {k}) vs oracle from the rounded checkpoint")
    for s, (c32, s32, clo, slo) in ck.items():
        assert np.array_equal(c32, st[s][0]) and np.array_equal(s32, st[s][1]), f"checkpoint after step {s}"
        want_s = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(s32.astype(np.float32))).reshape(s32.shape)
        want_c = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(c32.astype(np.float32))).reshape(c32.shape)
        assert np.array_equal(slo, want_s), "bf16 copy of the SSM state is not the rounded fp32 state"
        assert np.array_equal(clo[..., :3], want_c) and np.all(clo[..., 3] == 0), "bf16 copy of the conv state"


def test_replay_checkpoint_lo_rounds_to_nearest_even():
    Bs, d, N = 5, 136, 16
    rng = np.random.default_rng(3)
    cs = rng.standard_normal((Bs, d, 3)).astype(np.float32)
    ss = (rng.standard_normal((Bs, d, N)) * np.exp2(rng.integers(-10, 10, (Bs, d, N)))).astype(np.float32)
    clo, slo = mm.replay_checkpoint_lo(dev(cs), dev(ss))
    torch.cuda.synchronize()
    assert np.array_equal(host(slo), oracle.bf16_round(ss))
    assert np.array_equal(host(clo)[..., :3], oracle.bf16_round(cs)) and np.all(host(clo)[..., 3] == 0)


def test_replay_dual_7b_shape():
    """Batch 256, d_inner 8192, one window of 4 and a step of the next: the committing step and its
    state equal the eager decode; the other steps give the oracle's outputs from the bf16-rounded
    checkpoint on sampled rows (within the bf16 tolerance), and stay within a normwise 1e-2 of the
    exact replay on every row (the effect of rounding the state to 8 significant bits)."""
    W, Bs, d, N = 4, 256, 8192, 16
    steps = W + 1
    toks, p, cs, ss = _stream(6, steps, Bs, d, N, "bf16")
    log(f"[replay-dual] W={W} Bs={Bs} d={d} steps={steps}")
    yd, ck, starts = _run_dual(toks, p, cs, ss, W)
    ye, st = _run_eager(toks, p, cs, ss, {W - 1})
    prm = [p[k] for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    rows = np.array([0, 1, 77, 128, 200, 255])
    for s in range(steps):
        if s == W - 1:
            assert np.array_equal(yd[s], ye[s])
            continue
        w0 = (s // W) * W
        k = s - w0
        cs0, ss0 = starts[w0]
        ring = {q: np.stack([toks[w0 + i][q][rows] for i in range(k + 1)]) for q in ("x", "dt", "B")}
        yo, _, _ = oracle.decode_replay_lo(ring["x"], ring["dt"], ring["B"], k, toks[s]["z"][rows],
                                           toks[s]["C"][rows], *prm, cs0[rows], ss0[rows])
        assert_within(yd[s][rows], yo, "bf16", f"dual step {s} vs oracle from the rounded checkpoint")
        norm = np.linalg.norm(yd[s].astype(np.float64) - ye[s]) / np.linalg.norm(ye[s].astype(np.float64))
        assert norm < 1e-2, f"dual step {s}: normwise {norm:.3g} from the exact replay"
    assert np.array_equal(ck[W - 1][1], st[W - 1][1]) and np.array_equal(ck[W - 1][0], st[W - 1][0])
