"""The library loaded before torch has been imported.

Loaded first, the library used to bring in the system HIP runtime and torch then its own, so
that every launch on a torch stream failed (MM_ERR_HIP).  The binding now imports torch before
it loads the library; this runs a small prefill in a fresh interpreter that calls load() before
anything else and checks it against the same call made here.
"""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import selective_state_space_causal_amd as mm
from selective_state_space_causal_amd import inputs
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import selective_state_space_causal_amd as mm   # no torch import before this line
lib = mm.load()
import numpy as np, torch
from selective_state_space_causal_amd import inputs
lens, d, N = [37, 90], 64, 16
T = sum(lens)
tok = inputs.prefill_inputs(3, T, d, N, "f32")
p = inputs.params_per_channel(3, d, N, 4)
cs, ss = inputs.zero_states(len(lens), d, N, 4)
f = lambda a: torch.from_numpy(np.ascontiguousarray(a if a.dtype == np.int32 else a.astype(np.float32))).cuda()
y = mm.prefill(*[f(tok[k]) for k in ("x", "z", "dt", "B", "C")], *[f(p[k]) for k in ("A_log", "D", "dt_bias",
               "conv_w", "conv_b")], f(inputs.cu_from_lengths(lens)), f(cs), f(ss))
torch.cuda.synchronize()
np.save(sys.argv[2], y.cpu().numpy())
print("child ok", flush=True)
"""


def test_library_loaded_before_torch(tmp_path):
    out = tmp_path / "y.npy"
    res = subprocess.run([sys.executable, "-c", CHILD, ROOT, str(out)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and "child ok" in res.stdout, res.stdout[-2000:] + res.stderr[-2000:]
    lens, d, N = [37, 90], 64, 16
    T = sum(lens)
    tok = inputs.prefill_inputs(3, T, d, N, "f32")
    p = inputs.params_per_channel(3, d, N, 4)
    cs, ss = inputs.zero_states(len(lens), d, N, 4)
    y = mm.prefill(*[dev(tok[k]) for k in ("x", "z", "dt", "B", "C")],
                   *[dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")],
                   dev(inputs.cu_from_lengths(lens)), dev(cs), dev(ss))
    torch.cuda.synchronize()
    assert np.array_equal(np.load(out), host(y).astype(np.float32))
