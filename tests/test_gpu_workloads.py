"""The HIP path at the full sizes of the measured workloads, in the launch configuration
bench.py times (default chunk length), checked against the fp64 oracle on sampled
channels (channels are independent, so a channel subset of the oracle run is exact
for those channels).  Needs an MI355X."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_causal_amd as mm
from selective_state_space_causal_amd import inputs
from tests.gpu_util import assert_within, dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mm.load()
    oracle.build(force=False)


def _sample_channels(seed, d, k):
    rng = np.random.default_rng(seed)
    ch = np.sort(rng.choice(d, size=k, replace=False))
    # always include both edges of the channel range
    return np.unique(np.concatenate([[0, d - 1], ch]))


def _gpu_prefill(tok, p, cu, cs, ss, chunk_len=0):
    csd, ssd = dev(cs), dev(ss)
    y = mm.prefill(dev(tok["x"]), dev(tok["z"]), dev(tok["dt"]), dev(tok["B"]), dev(tok["C"]), dev(p["A_log"]),
                   dev(p["D"]), dev(p["dt_bias"]), dev(p["conv_w"]), dev(p["conv_b"]), dev(cu), csd, ssd,
                   chunk_len=chunk_len)
    return y, csd, ssd


def _oracle_cols(tok, p, cu, cs, ss, ch):
    return oracle.prefill(tok["x"][:, ch], tok["z"][:, ch], tok["dt"][:, ch], tok["B"], tok["C"], p["A_log"][ch],
                          p["D"][ch], p["dt_bias"][ch], p["conv_w"][ch], p["conv_b"][ch], cu, cs[:, ch], ss[:, ch])


def _y_cols(y, ch):
    """Sampled columns of a device y without copying the whole array to the host."""
    idx = torch.from_numpy(ch.astype(np.int64)).cuda()
    return host(y.index_select(1, idx))


def test_m130_prefill_full_size():
    """8 x 2048 tokens, d_inner 1536, N 16, bf16: the bench step."""
    S, L, d, N = 8, 2048, 1536, 16
    T = S * L
    log(f"[workload] m130 prefill T={T} d={d} chunk={mm.chunk_len(S, T, d, N)}")
    tok = inputs.prefill_inputs(0, T, d, N, "bf16")
    p = inputs.params(0, d, N, 4)
    cs, ss = inputs.zero_states(S, d, N, 4)
    cu = inputs.cu_from_lengths([L] * S)
    y, csd, ssd = _gpu_prefill(tok, p, cu, cs, ss)
    ch = _sample_channels(1, d, 62)
    yr, csr, ssr = _oracle_cols(tok, p, cu, cs, ss, ch)
    assert_within(_y_cols(y, ch), yr, "bf16", "m130 y")
    assert_within(host(ssd)[:, ch], ssr, "bf16", "m130 ssm_state")
    assert np.array_equal(host(csd)[:, ch], csr)
    assert np.all(np.isfinite(host(y)))


def test_m1p4b_packed_full_size():
    """PackMamba-style packing: lengths U[128, 4096] up to 16384 tokens, d_inner 4096; packed
    equals per-sequence runs, and both match the oracle."""
    d, N = 4096, 16
    lens = inputs.packed_lengths(0, 16384, 128, 4096)
    T = int(lens.sum())
    S = len(lens)
    log(f"[workload] m1p4b packed S={S} lens={lens.tolist()} d={d} chunk={mm.chunk_len(S, T, d, N)}")
    tok = inputs.prefill_inputs(0, T, d, N, "bf16")
    p = inputs.params(0, d, N, 4)
    cs, ss = inputs.zero_states(S, d, N, 4)
    cu = inputs.cu_from_lengths(lens)
    y, csd, ssd = _gpu_prefill(tok, p, cu, cs, ss)
    ch = _sample_channels(2, d, 46)
    yr, csr, ssr = _oracle_cols(tok, p, cu, cs, ss, ch)
    assert_within(_y_cols(y, ch), yr, "bf16", "m1p4b y")
    assert_within(host(ssd)[:, ch], ssr, "bf16", "m1p4b ssm_state")
    assert np.array_equal(host(csd)[:, ch], csr)
    yh = host(y)
    for s in range(S):
        g0, g1 = int(cu[s]), int(cu[s + 1])
        sub = {k: tok[k][g0:g1] for k in ("x", "z", "dt", "B", "C")}
        ys, css, sss = _gpu_prefill(sub, p, np.array([0, g1 - g0], np.int32), cs[s:s + 1], ss[s:s + 1])
        assert_within(host(ys), yh[g0:g1], "bf16", f"m1p4b seq {s} separate vs packed")
        assert_within(host(sss)[0], host(ssd)[s], "bf16", f"m1p4b seq {s} state")
        assert np.array_equal(host(css)[0], host(csd)[s])


def test_m7b_decode_full_size():
    """256 rows, d_inner 8192: states from a 512-token prefill, then 128 decode steps, y of every
    step checked on the sampled channels."""
    Bs, L, d, N, steps = 256, 512, 8192, 16, 128
    T = Bs * L
    log(f"[workload] m7b init prefill T={T} d={d} chunk={mm.chunk_len(Bs, T, d, N)}")
    tok = inputs.prefill_inputs(0, T, d, N, "bf16")
    p = inputs.params(0, d, N, 4)
    cs, ss = inputs.zero_states(Bs, d, N, 4)
    cu = inputs.cu_from_lengths([L] * Bs)
    y, csd, ssd = _gpu_prefill(tok, p, cu, cs, ss)
    ch = _sample_channels(3, d, 14)
    yr, csr, ssr = _oracle_cols(tok, p, cu, cs, ss, ch)
    assert_within(_y_cols(y, ch), yr, "bf16", "m7b init y")
    assert_within(host(ssd)[:, ch], ssr, "bf16", "m7b init ssm_state")
    assert np.array_equal(host(csd)[:, ch], csr)
    del y, tok
    torch.cuda.empty_cache()
    prm = [dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    cs_o, ss_o = csr, ssr
    log(f"[workload] m7b decode {steps} steps Bs={Bs}")
    for s in range(steps):
        dt_ = inputs.decode_inputs(0, s, Bs, d, N, "bf16")
        yd = mm.decode(*[dev(dt_[k]) for k in ("x", "z", "dt", "B", "C")], *prm, csd, ssd)
        ydr, cs_o, ss_o = oracle.decode(dt_["x"][:, ch], dt_["z"][:, ch], dt_["dt"][:, ch], dt_["B"], dt_["C"],
                                        p["A_log"][ch], p["D"][ch], p["dt_bias"][ch], p["conv_w"][ch],
                                        p["conv_b"][ch], cs_o, ss_o)
        assert_within(_y_cols(yd, ch), ydr, "bf16", f"m7b decode step {s} y")
    assert_within(host(ssd)[:, ch], ss_o, "bf16", "m7b decode final ssm_state")
    assert np.array_equal(host(csd)[:, ch], cs_o)


def test_m2p8b_long_chunked_full_size():
    """One 131072-token sequence, d_inner 5120: 16 prefill calls of 8192 tokens carrying the
    state equal the one-shot call and the oracle; then 64 decode steps at batch 1."""
    L, chunk, d, N = 131072, 8192, 5120, 16
    log(f"[workload] m2p8b long L={L} d={d} chunk_len(one-shot)={mm.chunk_len(1, L, d, N)}")
    tok = inputs.prefill_inputs(0, L, d, N, "bf16")
    p = inputs.params(0, d, N, 4)
    cs, ss = inputs.zero_states(1, d, N, 4)
    y1, cs1, ss1 = _gpu_prefill(tok, p, np.array([0, L], np.int32), cs, ss)
    ch = _sample_channels(4, d, 14)
    y1c = _y_cols(y1, ch)
    del y1
    csd, ssd = dev(cs), dev(ss)
    prm = [dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    parts = []
    cu1 = dev(np.array([0, chunk], np.int32))
    for k in range(L // chunk):
        sl = slice(k * chunk, (k + 1) * chunk)
        yk = mm.prefill(*[dev(tok[n][sl]) for n in ("x", "z", "dt", "B", "C")], *prm, cu1, csd, ssd)
        parts.append(_y_cols(yk, ch))
    yk = np.concatenate(parts)
    yr, csr, ssr = _oracle_cols(tok, p, np.array([0, L], np.int32), cs, ss, ch)
    assert_within(y1c, yr, "bf16", "m2p8b one-shot y")
    assert_within(yk, yr, "bf16", "m2p8b chunked y")
    assert_within(yk, y1c, "bf16", "m2p8b chunked vs one-shot")
    assert_within(host(ssd)[:, ch], ssr, "bf16", "m2p8b chunked state")
    assert_within(host(ss1)[:, ch], ssr, "bf16", "m2p8b one-shot state")
    assert np.array_equal(host(csd), host(cs1))
    assert np.array_equal(host(csd)[:, ch], csr)
    cs_o, ss_o = csr, ssr
    for s in range(64):
        dt_ = inputs.decode_inputs(0, s, 1, d, N, "bf16")
        yd = mm.decode(*[dev(dt_[k]) for k in ("x", "z", "dt", "B", "C")], *prm, csd, ssd)
        ydr, cs_o, ss_o = oracle.decode(dt_["x"][:, ch], dt_["z"][:, ch], dt_["dt"][:, ch], dt_["B"], dt_["C"],
                                        p["A_log"][ch], p["D"][ch], p["dt_bias"][ch], p["conv_w"][ch],
                                        p["conv_b"][ch], cs_o, ss_o)
        assert_within(_y_cols(yd, ch), ydr, "bf16", f"m2p8b decode step {s}")
    assert_within(host(ssd)[:, ch], ss_o, "bf16", "m2p8b decode final state")
