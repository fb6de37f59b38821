"""mamba_mixer_prefill_noalloc, the prefill for callers that cannot allocate (its carries live in the
library's fixed per-GPU scratch), through the C ABI: three calls in a row, each smaller than the one
before (a lane-engine plan with about 1.9 MB of carries and packed B/C, a chunked row-engine plan
with about 0.1 MB, a whole-sequence plan with none), each equal bit for bit to mamba_mixer_prefill with a
caller-allocated workspace on the same inputs (the same plan and kernels) and within the bf16
tolerance of the oracle.  Needs an MI355X."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import selective_state_space_causal_amd as mm
from tests.gpu_util import assert_within, dev, host, log, make_prefill, run_oracle_prefill

pytestmark = pytest.mark.gpu

PRM = ("A_log", "D", "dt_bias", "conv_w", "conv_b")


def _run(case, noalloc):
    lib = mm.load()
    S, T, d, N = case["S"], case["T"], case["d"], case["N"]
    t = {k: dev(case[k]) for k in ("x", "z", "dt", "B", "C", *PRM, "cu")}
    cs, ss = dev(case["cs"][:S]), dev(case["ss"][:S])
    y = torch.full((T, d), float("nan"), dtype=t["x"].dtype, device="cuda")
    ptr = lambda a: ctypes.c_void_p(a.data_ptr())
    args = [ptr(t[k]) for k in ("x", "z", "dt", "B", "C", *PRM, "cu")] + [ptr(cs), ptr(ss), ptr(y)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        rc = lib.mamba_mixer_prefill_noalloc(*args, S, T, d, N, 4, mm.MM_IO_BF16, stream)
    else:
        need = int(lib.mamba_mixer_prefill_workspace_bytes(S, T, d, N, 4))
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        rc = lib.mamba_mixer_prefill(*args, S, T, d, N, 4, mm.MM_IO_BF16, ctypes.c_void_p(ws.data_ptr()), need,
                                     stream)
    torch.cuda.synchronize()
    assert rc == 0, mm.status_string(rc)
    return host(y), host(cs), host(ss)


CASES = [  # (lengths, d, expected engine): workspace from the plan query, falling from call to call
    ([3, 1, 0, 2] * 2048 + [5], 64, "lane"),
    ([3000], 64, "row"),
    ([300, 1, 0, 499], 80, "row"),
]


def test_noalloc_prefill_equals_workspace_prefill():
    assert torch.cuda.is_available(), "needs a GPU"
    prev = None
    for i, (lens, d, engine) in enumerate(CASES):
        case = make_prefill(700 + i, lens, d, 16, "bf16", varied=True)
        p = mm.plan(case["S"], case["T"], d, 16)
        need = p["workspace_bytes"]
        log(f"[noalloc] call {i}: S={case['S']} T={case['T']} d={d} plan {p['kernels']} workspace {need}")
        assert p["engine_name"] == engine
        assert (need == 0) == (i == len(CASES) - 1), "the last call needs no workspace, the others do"
        assert need <= mm.NOALLOC_SCRATCH_BYTES
        if prev is not None:
            assert need < prev, "each call needs less scratch than the one before"
        prev = need
        yn, csn, ssn = _run(case, noalloc=True)
        yw, csw, ssw = _run(case, noalloc=False)
        assert np.array_equal(yn, yw), f"call {i}: y differs from mamba_mixer_prefill"
        assert np.array_equal(csn, csw) and np.array_equal(ssn, ssw), f"call {i}: states differ"
        yr, csr, ssr = run_oracle_prefill(case)
        assert_within(yn, yr, "bf16", f"noalloc call {i} y")
        assert_within(ssn, ssr, "bf16", f"noalloc call {i} ssm_state")
        assert np.array_equal(csn, csr)
