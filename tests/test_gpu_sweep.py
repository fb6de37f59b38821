"""Seeded random sweep of the HIP path against the fp64 oracle: prefill (both engines and the
automatic plan, explicit and automatic chunk lengths), the training forward with checkpoints,
the backward, and decode, over shapes drawn at random -- sequence counts and lengths (empty
ones and ones shorter than the conv window included), channel counts that are not multiples
of 16 or 64, every state size 1..16, both io types.  Every case is printed before it runs, so
a failure names its seed and shape.  Needs an MI355X."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_causal_amd as mm
from selective_state_space_causal_amd import inputs
from tests.gpu_util import assert_within, dev, host, log, make_prefill, run_gpu_prefill, run_oracle_prefill
from tests.test_gpu_backward import check_all, gpu_backward, oracle_backward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mm.load()
    oracle.build(force=False)


def _draw(seed: int, max_len: int):
    rng = np.random.default_rng(7000 + seed)
    S = int(rng.integers(1, 7))
    kind = rng.random(S)
    # a mix of empty, sub-window, short and longer sequences
    lens = [0 if k < 0.1 else (int(rng.integers(1, 4)) if k < 0.25 else int(rng.integers(4, max_len + 1)))
            for k in kind]
    d = int(rng.choice([1, 3, 15, 16, 17, 33, 64, 70, 96, 130]))
    N = int(rng.integers(1, 17))
    io = "bf16" if rng.random() < 0.5 else "f32"
    chunk = int(rng.choice([0, 0, 16, 17, 48, 64, 100, 256]))
    engine = int(rng.choice([mm.ENGINE_AUTO, mm.ENGINE_LANE, mm.ENGINE_ROW]))
    return rng, lens, d, N, io, chunk, engine


@pytest.mark.parametrize("seed", range(96))
def test_prefill_sweep(seed):
    _, lens, d, N, io, chunk, engine = _draw(seed, 400)
    log(f"[sweep prefill] seed={seed} lens={lens} d={d} N={N} io={io} chunk={chunk} engine={engine}")
    case = make_prefill(9000 + seed, lens, d, N, io)
    y, cs, ss = run_gpu_prefill(case, chunk, engine=engine)
    yr, csr, ssr = run_oracle_prefill(case)
    assert_within(y, yr, io, f"seed {seed} y")
    assert_within(ss, ssr, io, f"seed {seed} ssm_state")
    assert np.array_equal(cs, csr), f"seed {seed}: conv_state not bit-exact"


@pytest.mark.parametrize("seed", range(24))
def test_train_and_backward_sweep(seed):
    """The training forward (checkpoints) matches the plain prefill's outputs; the backward from
    those checkpoints and the standalone backward both match the oracle's reverse mode."""
    _, lens, d, N, io, chunk, _ = _draw(100 + seed, 160)
    log(f"[sweep backward] seed={seed} lens={lens} d={d} N={N} io={io} chunk={chunk}")
    case = make_prefill(9500 + seed, lens, d, N, io)
    S, T = case["S"], case["T"]
    dy = inputs.grad_output(9500 + seed, T, d, io)
    args = [dev(case[k]) for k in ("x", "z", "dt", "B", "C", "A_log", "D", "dt_bias", "conv_w", "conv_b", "cu")]
    cs, ss = dev(case["cs"][:S]), dev(case["ss"][:S])
    y, ck = mm.prefill_train(*args, cs, ss, chunk_len=chunk)
    torch.cuda.synchronize()
    yr, csr, ssr = run_oracle_prefill(case)
    assert_within(host(y), yr, io, f"seed {seed} train y")
    assert_within(host(ss), ssr, io, f"seed {seed} train ssm_state")
    assert np.array_equal(host(cs), csr), f"seed {seed}: train conv_state not bit-exact"
    r = oracle_backward(case, dy)
    g = mm.prefill_backward(*args, dev(case["cs"][:S]), None, dev(dy), ckpt=ck)
    torch.cuda.synchronize()
    check_all({k: host(v) for k, v in g.items()}, r, io, f"sweep seed {seed} from checkpoints")
    check_all(gpu_backward(case, dy), r, io, f"sweep seed {seed} standalone")


@pytest.mark.parametrize("seed", range(12))
def test_decode_sweep(seed):
    """Several decode steps in a row on random batch rows, states carried between them."""
    rng, _, d, N, io, _, _ = _draw(200 + seed, 8)
    Bs = int(rng.integers(1, 300))
    steps = 3
    log(f"[sweep decode] seed={seed} Bs={Bs} d={d} N={N} io={io} steps={steps}")
    p = inputs.params(9800 + seed, d, N, 4)
    cs = rng.standard_normal((Bs, d, 3)).astype(np.float32)
    if io == "bf16":
        cs = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(cs)).reshape(cs.shape)
    ss = (0.5 * rng.standard_normal((Bs, d, N))).astype(np.float32)
    prm = [p[k] for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    csd, ssd = dev(cs), dev(ss)
    for s in range(steps):
        tok = inputs.prefill_inputs(9800 + 17 * seed + s, Bs, d, N, io)
        tk = [tok[k] for k in ("x", "z", "dt", "B", "C")]
        y = mm.decode(*[dev(a) for a in tk], *[dev(a) for a in prm], csd, ssd)
        yr, cs, ss = oracle.decode(*tk, *prm, cs, ss)
        assert_within(host(y), yr, io, f"seed {seed} step {s} y")
        assert_within(host(ssd), ss, io, f"seed {seed} step {s} ssm_state")
        assert np.array_equal(host(csd), cs), f"seed {seed} step {s}: conv_state not bit-exact"
