"""Benchmark of the selective-SSM mixer core on one MI355X.

One step = one prefill call over the 1.4B-shaped packed workload (PackMamba-style packing:
sequence lengths uniform on [128, 4096] drawn until 16384 tokens, d_inner 4096, N 16, bf16 io,
fp32 state): conv + SiLU, softplus, discretisation, the segmented selective scan, readout and
gate, and the final-state write-back.  `value` is prefill tokens/s with all inputs resident in
HBM.  The same JSON line also carries:
  * the 130m-shaped prefill (8 x 2048 tokens, d_inner 1536) and the 2.8B-shaped long prefill
    (131072 tokens in 16 state-carrying calls of 8192, d_inner 5120), each with its own roofline;
  * packed vs one call per sequence on the 1.4B-shaped stream (PackMamba's comparison, context);
  * the batch-256 decode (Falcon-Mamba-7B-shaped: d_inner 8192, N 16, state initialised by a
    512-token prefill, then 128 single-token steps) and its replay variant;
  * the prefill backward and the dt/B/C projections;
  * per-kernel times measured with HIP events on the launch stream inside the timed steps, the
    roofline of each dominant kernel (algorithmic FLOP and bytes per launch over its time, HBM
    traffic and VALU issue fraction from the committed rocprofv3 summaries under profiles/);
  * the fp64 CPU oracle timed on this host as a baseline.

Every timed measurement follows an untimed settle phase (--settle-ms, default 100 ms of
back-to-back calls of the measured workload): under sustained load the GPU raises its clocks
over the first ~20 ms, so that steps timed right after a short warm-up run slower than the same
steps in a continuous workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s + decode steps/s (B=256); achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
# FP32 vector peak (AMD's published figure): 157.3 TFLOP/s = 256 CUs x 4 SIMDs x 2.4 GHz x 32 fp32
# FMA per clock x 2 FLOP.  A SIMD retires one wave64 instruction per 4 clocks (16 lanes per clock);
# the factor 2 on top is packed fp32 (two fp32 operations per lane and instruction), which this build
# does not generate, so its own ceiling is half the peak.  The rooflines count algorithmic FLOP
# against the published peak.
ALU_PEAK_TFLOPS = 157.3


def log(msg):
    print(msg, file=sys.stderr, flush=True)


SETTLE_MS = 100.0  # set from --settle-ms


def settle(fn, ms=None):
    """Call fn(i) back to back, untimed, for about ms milliseconds; returns the number of calls.

    The GPU raises its clocks over the first ~20 ms of sustained load.  On the 130m prefill step a
    kernel trace of 600 back-to-back calls shows 177 us per call over the first 25 calls and 153 us
    from about the 125th call on; calls 2 ms apart stay at 166 us.  Timing after this phase
    measures the steady state of a continuous workload (a serving or training loop)."""
    import torch

    ms = SETTLE_MS if ms is None else ms
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


class HipEvents:
    """hipEvent_t handles created through libamdhip64 (recorded by the library on its launch stream)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.ev.append(h.value)

    def ms(self, a, b):
        f = ctypes.c_float()
        self.hip.hipEventSynchronize(ctypes.c_void_p(self.ev[b]))
        rc = self.hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(self.ev[a]), ctypes.c_void_p(self.ev[b]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(f.value)

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


KERNEL_DIR = os.path.join(ROOT, "selective_state_space_causal_amd", "csrc")


def kernel_source_sha256():
    """sha256 over the HIP sources (every file of csrc/, in name order), to tie a counter summary to them."""
    import hashlib

    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_DIR)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(KERNEL_DIR, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()

PROFILE_DECODE = os.path.join(ROOT, "profiles", "k_decode_vec__m7b_decode_b256_d8192_N16_bf16.txt")
PROFILE_REPLAY = os.path.join(ROOT, "profiles", "k_decode_replay__m7b_decode_b256_d8192_N16_W4_bf16.txt")
PROFILE_DUAL = os.path.join(ROOT, "profiles", "k_decode_replay_dual__m7b_decode_b256_d8192_N16_W4_bf16.txt")
PROFILE_BACKWARD = os.path.join(ROOT, "profiles", "k_row_bwd__m130_backward_8x2048_d1536_N16_bf16.txt")
PROFILE_PROJECT = {(k, sh): os.path.join(ROOT, "profiles", f"{k}__{sh}_project_8x2048_d{d}_R{r}_N16_bf16.txt")
                   for k in ("k_proj_in", "k_proj_dt") for sh, d, r in (("m130", 1536, 48), ("m1p4b", 4096, 128))}


def counted_traffic(profile_path):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None when the summary is
    missing or was taken on a different kernel source than the one built now."""
    try:
        text = open(profile_path).read()
        src = kernel_source_sha256()
    except OSError:
        return None
    sha = traffic = None
    for line in text.splitlines():
        if line.startswith("kernel source sha256:"):
            sha = line.split(":", 1)[1].strip()
        if line.startswith("traffic_bytes_per_launch:"):
            traffic = int(float(line.split(":", 1)[1]))
    return traffic if sha == src else None


def dev(a):
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    if a.dtype == np.int32:
        return torch.from_numpy(a).cuda()
    return torch.from_numpy(a.astype(np.float32)).cuda()


def prefill_alg_bytes(T, S, d, N, K, s_io):
    """Bytes the method must move for one prefill: token io, shared B/C, parameters, cu_seqlens, states in+out."""
    return T * d * 4 * s_io + 2 * T * N * s_io + d * (N + K + 3) * 4 + (S + 1) * 4 + 2 * S * d * (N + K - 1) * 4


def decode_alg_bytes(Bs, d, N, K, s_io):
    return Bs * d * 4 * s_io + 2 * Bs * N * s_io + d * (N + K + 3) * 4 + 2 * Bs * d * (N + K - 1) * 4


def replay_alg_bytes(Bs, d, N, K, s_io, W):
    """Mean bytes per replay-decode step over a window of W steps: every step reads the checkpoint
    (ssm + conv state), the buffered x, dt of steps 0..k and B of steps 0..k, this step's z and C,
    the parameters, and writes y; the last step of the window also writes the checkpoint."""
    total = 0
    for k in range(W):
        b = Bs * d * (N + K - 1) * 4                      # checkpoint read
        b += Bs * d * 2 * (k + 1) * s_io + Bs * N * (k + 1) * s_io  # buffered x, dt and B
        b += Bs * d * 2 * s_io + Bs * N * s_io            # z in, y out; C
        b += d * (N + K + 3) * 4                          # parameters
        if k == W - 1:
            b += Bs * d * (N + K - 1) * 4                 # checkpoint write
        total += b
    return total / W


def alg_flop_per_token_channel(N):
    """Algorithmic FLOP of the method per (token, channel): an FMA counts 2, an add or multiply 1,
    a transcendental (exp, log, reciprocal) 1.

    conv: 4 FMA (8); SiLU(xc) = xc / (1 + e^-xc): add, multiply + exp, rcp (2 + 2); softplus(v) =
    log(1 + e^v), v = dt + dt_bias: 2 adds + exp, log (2 + 2); delta * u (1); per state entry:
    delta * A (1) + exp, (delta u) * B (1), the state FMA (2), the readout FMA (2) -- 6 + 1 each;
    + D u (2); SiLU(z): add, multiply + exp, rcp (2 + 2); the gate multiply (1).
    At N = 16: 114 + 22 = 136.
    """
    plain = 8 + 2 + 2 + 1 + 6 * N + 2 + 2 + 1
    trans = 2 + 2 + N + 2
    return plain + trans


def alg_flop_backward(N):
    """Algorithmic FLOP of the backward per (token, channel), counted as alg_flop_per_token_channel:
    the forward's (the states and per-token quantities are recomputed, not stored) plus the
    adjoint's.  Per state entry: the lambda FMA (2), the dC and dB terms (2), the S1 term and its
    sum (2), lambda a h_prev (2) times A and its sum (2), the dA FMA (2) -- 12 each.  Per token:
    dp 1, dz 4, du 2, d(delta) 2, d(dt) = d(delta) sigmoid(v) 3 + 2 transcendentals, d(xc) 4 + 2
    transcendentals, dconv_w 4 FMA (8), dconv_b 1, dx 4 FMA (8), dD FMA (2), ddt_bias 1 -- 36 + 4."""
    return alg_flop_per_token_channel(N) + 12 * N + 36 + 4


def make_prefill_set(seed, lens, d, N, io):
    from selective_state_space_causal_amd import inputs

    T = int(sum(lens))
    tok = inputs.prefill_inputs(seed, T, d, N, io)
    p = inputs.params(seed, d, N, 4)
    cs, ss = inputs.zero_states(len(lens), d, N, 4)
    cu = inputs.cu_from_lengths(lens)
    return tok, p, cs, ss, cu


def prefill_workloads():
    """The prefill workloads: packed lengths and d_inner of each (N 16, conv 4, bf16 io, fp32 state).

    m1p4b_packed -- the headline: PackMamba-style packing of sequences with lengths uniform on
                    [128, 4096] until 16384 tokens, d_inner 4096 (1.4B-shaped layer); one call.
    m130_prefill -- 8 sequences x 2048 tokens, d_inner 1536 (130m-shaped layer); one call.
    m2p8b_long   -- one 131072-token sequence, d_inner 5120 (2.8B-shaped layer), in 16 calls of
                    8192 tokens that carry the conv/SSM state from call to call (the state cache).
    """
    from selective_state_space_causal_amd import inputs

    lens = [int(v) for v in inputs.packed_lengths(0, 16384, 128, 4096)]
    return {
        "m1p4b_packed": dict(lens=lens, d=4096, calls=1,
                             workload=f"1.4B-shaped packed prefill: {len(lens)} sequences, lengths U[128,4096] to "
                                      f"T=16384 ({lens}), d_inner 4096, d_state 16, conv 4, bf16 io, fp32 state"),
        "m130_prefill": dict(lens=[2048] * 8, d=1536, calls=1,
                             workload="mamba-130m-shaped layer prefill: 8 packed sequences x 2048 tokens, "
                                      "d_inner 1536, d_state 16, conv 4, bf16 io, fp32 state"),
        "m2p8b_long": dict(lens=[131072], d=5120, calls=16,
                           workload="2.8B-shaped long prefill: 1 sequence of 131072 tokens in 16 calls of 8192 "
                                    "tokens carrying the conv/SSM state, d_inner 5120, d_state 16, conv 4, bf16 io, "
                                    "fp32 state"),
    }


def profile_path(kernel, name):
    """profiles/<kernel>__<workload>.txt: the committed rocprofv3 summary of one kernel on one workload."""
    tags = {"m1p4b_packed": "m1p4b_packed_T16384_d4096_N16_bf16", "m130_prefill": "m130_prefill_8x2048_d1536_N16_bf16",
            "m2p8b_long": "m2p8b_long_16x8192_d5120_N16_bf16"}
    return os.path.join(ROOT, "profiles", f"{kernel}__{tags[name]}.txt")


def profile_field(path, field):
    """A numeric field of a committed profile summary ("<field>: <value>"), or None when the summary
    is missing or was taken on a different kernel source than the one built now."""
    try:
        text = open(path).read()
        src = kernel_source_sha256()
    except OSError:
        return None
    sha = val = None
    for line in text.splitlines():
        if line.startswith("kernel source sha256:"):
            sha = line.split(":", 1)[1].strip()
        if line.startswith(field + ":"):
            val = float(line.split(":", 1)[1].split()[0])
    return val if sha == src else None


def bench_prefill_workload(name, steps, warmup):
    """Time `steps` steps of one prefill workload (a step = all its calls) on resident inputs.

    Inputs, workspaces, plans and the HIP events are set up before anything is timed.  Calls-1
    workloads alternate between two resident input sets (seeds 0 and 1), so that the 256 MB
    Infinity Cache cannot hold a step's inputs.  The 16-call workload runs over the 131072 tokens
    of one resident set; its state slots are not reset between steps (a step continues the state
    of the step before: the same work on nonzero initial states).  After the warm-up steps an
    untimed settle phase of back-to-back steps lets the clocks ramp.  The timed steps run back to
    back, and the per-kernel times come from HIP events the library records on its launch stream
    inside them (see below)."""
    import torch

    import selective_state_space_causal_amd as mm

    wl = prefill_workloads()[name]
    lens, d, calls = wl["lens"], wl["d"], wl["calls"]
    N, K = 16, 4
    T = int(sum(lens))
    S = len(lens)
    Tc, cl = (T // calls, [T // calls]) if calls > 1 else (T, lens)  # tokens and lengths of one call
    Sc = len(cl)
    plan = mm.plan(Sc, Tc, d, N, K)
    names = plan["kernels"]
    nk = len(names)
    sets = []
    t0 = time.perf_counter()
    for seed in ((0,) if calls > 1 else (0, 1)):
        tok, p, cs, ss, cu = make_prefill_set(seed, lens, d, N, "bf16")
        st = {k: dev(v) for k, v in tok.items()}
        del tok
        st.update({k: dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")})
        st.update(cu=dev(inputs_cu(cl)), cs=dev(cs), ss=dev(ss))
        st["y"] = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
        # at least 256 bytes: with a workspace given, the binding makes no plan query of its own
        st["ws"] = torch.empty(max(plan["workspace_bytes"], 256), dtype=torch.uint8, device="cuda")
        sets.append(st)
    torch.cuda.synchronize()
    log(f"[bench] {name}: inputs resident ({time.perf_counter() - t0:.1f} s), plan {names}, "
        f"chunk {plan['chunk_len']}, workspace {plan['workspace_bytes']} B")
    views = []  # per call: the io slices of each set
    for st in sets:
        vs = []
        for c in range(calls):
            sl = slice(c * Tc, (c + 1) * Tc)
            vs.append([st[k][sl] for k in ("x", "z", "dt", "B", "C")] + [st["y"][sl]])
        views.append(vs)

    def step(i, ev=None):
        st = sets[i % len(sets)]
        for c, v in enumerate(views[i % len(sets)]):
            e = None if ev is None else ev[c * (nk + 1):(c + 1) * (nk + 1)]
            mm.prefill(*v[:5], st["A_log"], st["D"], st["dt_bias"], st["conv_w"], st["conv_b"], st["cu"], st["cs"],
                       st["ss"], y=v[5], workspace=st["ws"], events=e)

    # One kernel per step: one event before the first timed step's kernel and one after the last
    # step's (the library records them on its launch stream), so the steps run unperturbed and the
    # kernel's mean launch time is the span over the steps (launch gaps included).  Several kernels
    # per call: an event before each kernel and after the last, in every call of the first and the
    # last timed step (events between kernels cost several microseconds each, so the steps between
    # run uninstrumented).
    span = calls == 1 and nk == 1
    per_step_ev = calls * (nk + 1)
    inst = sorted({0, steps - 1})  # the instrumented steps
    hev = HipEvents(4 if span else len(inst) * per_step_ev)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    n_settle = settle(step)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if span:
            first, last = i == 0, i == steps - 1
            step(i, [hev.ev[0], hev.ev[1]] if first and last else
                 ([hev.ev[0], hev.ev[2]] if first else ([hev.ev[3], hev.ev[1]] if last else None)))
        else:
            step(i, hev.ev[inst.index(i) * per_step_ev:(inst.index(i) + 1) * per_step_ev] if i in inst else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = {n: [] for n in names}
    inst_ms = []  # each instrumented step: first event of its first call to the last of its last call
    if span:
        kern[names[0]].append(hev.ms(0, 1) / steps)
    else:
        for q in range(len(inst)):
            inst_ms.append(hev.ms(q * per_step_ev, (q + 1) * per_step_ev - 1))
            for c in range(calls):
                b = q * per_step_ev + c * (nk + 1)
                for k, n in enumerate(names):
                    kern[n].append(hev.ms(b + k, b + k + 1))
    hev.close()
    del sets, views
    torch.cuda.empty_cache()
    return dict(name=name, workload=wl["workload"], S=S, T=T, d=d, N=N, K=K, calls=calls, call_T=Tc, call_S=Sc,
                wall_s=wall, steps=steps, settle_steps=n_settle, names=names, chunk_len=plan["chunk_len"],
                kernel_timing="span of the timed steps / steps" if span else
                "events around every kernel of the first and the last timed step",
                engine=plan["engine_name"], kern_ms={n: float(np.mean(v)) for n, v in kern.items()},
                inst_step_ms=float(np.mean(inst_ms)) if inst_ms else None)


def inputs_cu(lens):
    from selective_state_space_causal_amd import inputs

    return inputs.cu_from_lengths(lens)


def prefill_line(pf):
    """Throughput, per-kernel times and the roofline of one timed prefill workload."""
    T, d, N, K, calls = pf["T"], pf["d"], pf["N"], pf["K"], pf["calls"]
    ms_per_step = pf["wall_s"] / pf["steps"] * 1e3
    kern = pf["kern_ms"]
    # the final pass runs every token of a call through the whole method: the dominant kernel
    dom = pf["names"][-1]
    dom_ms = kern[dom]
    Tc, Sc = pf["call_T"], pf["call_S"]
    flop = alg_flop_per_token_channel(N)
    alg_flop = flop * Tc * d
    alg_bytes = prefill_alg_bytes(Tc, Sc, d, N, K, 2)
    tflops = alg_flop / (dom_ms * 1e-3) / 1e12
    gbs = alg_bytes / (dom_ms * 1e-3) / 1e9
    prof = profile_path(dom, pf["name"])
    issue = profile_field(prof, "valu_issue_frac")
    roof = dict(bound="alu", achieved=round(tflops, 2), peak=ALU_PEAK_TFLOPS, unit="TFLOP/s",
                frac=round(tflops / ALU_PEAK_TFLOPS, 4), traffic=_int_or_none(profile_field(prof, "traffic_bytes_per_launch")),
                kernel=dom, kernel_ms=round(dom_ms, 4), alg_flop_per_launch=alg_flop,
                per_unit=f"{flop} algorithmic FLOP per (token, channel) at N={N} (an FMA 2, an add or multiply 1, "
                         f"a transcendental 1); {Tc} tokens x {d} channels per launch",
                hbm_view=dict(alg_bytes_per_launch=alg_bytes, achieved_GBs=round(gbs, 1), peak_GBs=HBM_PEAK_GBS,
                              frac=round(gbs / HBM_PEAK_GBS, 4)),
                issue_view=dict(valu_issue_frac=issue,
                                source=os.path.relpath(prof, ROOT),
                                note="fraction of the SIMDs' VALU issue cycles the kernel kept busy, from the "
                                     "committed rocprofv3 counters of this kernel (null when the summary is missing "
                                     "or stale); without packed fp32 the 157.3 TFLOP/s peak is out of reach, so "
                                     "this is the kernel's headroom against its own instruction stream"))
    call_ms = sum(kern.values())
    return dict(workload=pf["workload"], tokens_per_s=round(T * pf["steps"] / pf["wall_s"], 1),
                ms_per_step=round(ms_per_step, 4), steps=pf["steps"], settle_steps=pf["settle_steps"],
                kernel_timing=pf["kernel_timing"],
                calls_per_step=calls, engine=pf["engine"], chunk_len=pf["chunk_len"],
                kernels_ms={k: round(v, 4) for k, v in kern.items()},
                kernels_ms_per_step=round(call_ms * calls, 4),
                **({} if pf["inst_step_ms"] is None else dict(
                    instrumented_step_ms=round(pf["inst_step_ms"], 4),
                    instrumented_step_note="the kernel times come from the instrumented steps, which the event "
                                           "records between kernels slow down: their kernels fit inside "
                                           "instrumented_step_ms, which ms_per_step (the mean over all timed "
                                           "steps, most of them uninstrumented) can undercut")),
                hbm_view_step=dict(alg_bytes_per_step=prefill_alg_bytes(Tc, Sc, d, N, K, 2) * calls,
                                   achieved_GBs=round(prefill_alg_bytes(Tc, Sc, d, N, K, 2) * calls
                                                      / (ms_per_step * 1e-3) / 1e9, 1)),
                roofline=roof)


def _int_or_none(v):
    return None if v is None else int(v)


def bench_packed_vs_separate():
    """Context for PackMamba's comparison: the 1.4B-shaped packed stream in one call against one call
    per sequence on the same resident inputs (each call timed with events after a settle phase;
    workspaces preallocated)."""
    import torch

    import selective_state_space_causal_amd as mm

    wl = prefill_workloads()["m1p4b_packed"]
    lens, d, N = wl["lens"], wl["d"], 16
    tok, p, cs, ss, cu = make_prefill_set(0, lens, d, N, "bf16")
    st = {k: dev(v) for k, v in tok.items()}
    prm = [dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    T = int(sum(lens))
    y = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(mm.workspace_bytes(len(lens), T, d, N), 256), dtype=torch.uint8, device="cuda")
    css, sss = dev(cs), dev(ss)
    calls = [([st[k] for k in ("x", "z", "dt", "B", "C")], dev(cu), css, sss, y)]
    sep = []
    off = 0
    for L in lens:
        sl = slice(off, off + L)
        sep.append(([st[k][sl] for k in ("x", "z", "dt", "B", "C")], dev(np.array([0, L], np.int32)),
                    css[:1].clone(), sss[:1].clone(), y[sl]))
        off += L
    wss = [torch.empty(max(mm.workspace_bytes(1, L, d, N), 256), dtype=torch.uint8, device="cuda") for L in lens]

    def run(cs_, ws_):
        for (io, cu_, c_, s_, y_), w in zip(cs_, ws_):
            mm.prefill(*io, *prm, cu_, c_, s_, y=y_, workspace=w)

    out = {}
    for key, cs_, ws_ in (("packed", calls, [ws]), ("separate", sep, wss)):
        settle(lambda i: run(cs_, ws_))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(5):
            e0.record()
            run(cs_, ws_)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        out[key] = float(np.mean(times))
    del st, y, ws, wss, calls, sep
    torch.cuda.empty_cache()
    return dict(what="the 1.4B-shaped packed stream in one call vs one call per sequence (PackMamba's comparison; "
                     "context only)", packed_ms=round(out["packed"], 4), separate_ms=round(out["separate"], 4),
                packed_speedup=round(out["separate"] / out["packed"], 3))


def _time_calls(fn, n_kernels, names, reps=10):
    """Mean whole-call time (torch events) and per-kernel times (HIP events the library records
    around each of its kernels) of fn(events) over reps calls after one warm-up call."""
    import torch

    hev = HipEvents(n_kernels + 1)
    kern = {n: [] for n in names}
    whole = []
    settle(lambda i: fn(None))
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn(hev.ev)
        e1.record()
        torch.cuda.synchronize()
        if r > 0:
            whole.append(e0.elapsed_time(e1))
            for i, n in enumerate(names):
                kern[n].append(hev.ms(i, i + 1))
    hev.close()
    return float(np.mean(whole)), {n: float(np.mean(v)) for n, v in kern.items()}


def bench_backward(args):
    """Prefill backward of the 130M training shape (8 x 2048 tokens, d 1536, bf16 io) on resident
    inputs: the standalone backward (it runs its own checkpoint pass), and a training step =
    the forward that stores checkpoints + the backward that uses them."""
    import torch

    import selective_state_space_causal_amd as mm
    from selective_state_space_causal_amd import inputs

    S, L, d, N = 8, 2048, 1536, 16
    T = S * L
    tok, p, cs, ss, cu = make_prefill_set(0, [L] * S, d, N, "bf16")
    st = {k: dev(v) for k, v in tok.items()}
    st.update({k: dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")})
    st.update(cu=dev(cu), cs=dev(cs), ss=dev(ss), dy=dev(inputs.grad_output(0, T, d, "bf16")))
    prm = [st[k] for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    tk = [st[k] for k in ("x", "z", "dt", "B", "C")]
    cs0 = st["cs"].clone()  # the initial states (the forward overwrites its copies)
    ss0 = st["ss"].clone()
    # standalone backward
    plan = mm.backward_plan(S, T, d, N)
    ws = torch.empty(plan["workspace"], dtype=torch.uint8, device="cuda")
    out = mm.prefill_backward(*tk, *prm, st["cu"], cs0, ss0, st["dy"], workspace=ws)
    names = ["k_row_ckpt", "k_row_bwd", "k_bwd_sum_bc", "k_bwd_sum_params"]
    ms_b, k_b = _time_calls(lambda ev: mm.prefill_backward(*tk, *prm, st["cu"], cs0, ss0, st["dy"], out=out,
                                                           workspace=ws, events=ev), plan["kernels"], names)
    del ws
    # training step: forward with checkpoints, backward from them
    fplan = mm.plan(S, T, d, N, engine=mm.ENGINE_ROW)
    fws = torch.empty(max(fplan["workspace_bytes"], 1), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    ck = torch.empty((mm.checkpoint_bytes(S, T, d) // 4,), dtype=torch.float32, device="cuda").view(-1, d, 16)
    cs1, ss1 = st["cs"], st["ss"]

    def fwd(ev):
        cs1.copy_(cs0)
        ss1.copy_(ss0)
        mm.prefill_train(*tk, *prm, st["cu"], cs1, ss1, y=y, ckpt=ck, workspace=fws, events=ev)
    fnames = [f"fwd_{k}" for k in fplan["kernels"]]
    ms_f, k_f = _time_calls(fwd, len(fnames), fnames)
    bplan = mm.backward_plan(S, T, d, N, has_ckpt=True)
    bws = torch.empty(bplan["workspace"], dtype=torch.uint8, device="cuda")
    bnames = ["k_row_bwd", "k_bwd_sum_bc", "k_bwd_sum_params"]
    ms_bc, k_bc = _time_calls(lambda ev: mm.prefill_backward(*tk, *prm, st["cu"], cs0, None, st["dy"], ckpt=ck,
                                                             out=out, workspace=bws, events=ev),
                              bplan["kernels"], bnames)
    io_bytes = T * d * 2 * 4 + T * d * 2 * 3 + 2 * T * N * 2 * 2  # x, z, dt, dy in; dx, dz, ddt out; B, C in, dB, dC out
    del st, bws, fws, out, ck, y
    torch.cuda.empty_cache()
    step_ms = ms_f + ms_bc
    flop = alg_flop_backward(N)
    kb = k_bc["k_row_bwd"]
    ach = T * d * flop / (kb * 1e-3) / 1e12
    return dict(
        workload=f"mamba-130m-shaped layer backward: {S} packed sequences x {L} tokens, d_inner {d}, d_state {N}, "
                 "conv 4, bf16 io, fp32 state; gradients of all inputs, parameters and initial states",
        standalone=dict(tokens_per_s=round(T / (ms_b * 1e-3), 1), ms=round(ms_b, 4),
                        kernels_ms={n: round(v, 4) for n, v in k_b.items()}, workspace_bytes=plan["workspace"],
                        note="own checkpoint pass (the forward's states before every 16-token block), reverse "
                             "pass, fixed-order partial sums"),
        train_step=dict(tokens_per_s=round(T / (step_ms * 1e-3), 1), ms=round(step_ms, 4),
                        forward_ms=round(ms_f, 4), backward_ms=round(ms_bc, 4),
                        kernels_ms={**{n: round(v, 4) for n, v in k_f.items()},
                                    **{n: round(v, 4) for n, v in k_bc.items()}},
                        note="forward storing checkpoints (row engine, state copies included in forward_ms) + "
                             "backward from them"),
        roofline=dict(bound="alu", achieved=round(ach, 2), peak=ALU_PEAK_TFLOPS, unit="TFLOP/s",
                      frac=round(ach / ALU_PEAK_TFLOPS, 4), traffic=counted_traffic(PROFILE_BACKWARD),
                      kernel="k_row_bwd", kernel_ms=round(kb, 4),
                      per_unit=f"{flop} algorithmic FLOP per (token, channel) (the forward's, recomputed, and the "
                               "adjoint's; an FMA 2, an add or multiply 1, a transcendental 1)",
                      issue_view=dict(valu_issue_frac=profile_field(PROFILE_BACKWARD, "valu_issue_frac"),
                                      source=os.path.relpath(PROFILE_BACKWARD, ROOT)),
                      note="the reverse kernel of the training step's backward"),
        io_bytes=io_bytes, io_GBs_standalone=round(io_bytes / (ms_b * 1e-3) / 1e9, 1))


def project_alg_bytes(T, S, d, N, R):
    """HBM bytes of the two projection kernels, each counted as its own launch.

    k_proj_in: x in (bf16), B and C out, dt_in out as bf16 high and low parts [T][Rp], the re-laid
    w_x, the conv parameters, the initial conv state and cu_seqlens.  k_proj_dt: dt out (bf16),
    dt_in in, the re-laid w_dt.  "call" is the projection as one operation: x in, dt, B, C out,
    the weights and conv parameters (dt_in stays between the kernels)."""
    P = R + 2 * N
    Pp = -(-P // 16) * 16
    dk = -(-d // 32) * 32
    Rp = -(-R // 32) * 32
    params = d * 5 * 4 + S * d * 3 * 4 + (S + 1) * 4
    dtin = 2 * T * Rp * 2
    return dict(k_proj_in=T * d * 2 + 2 * T * N * 2 + dtin + Pp * dk * 2 + params,
                k_proj_dt=T * d * 2 + dtin + d * Rp * 2,
                call=2 * T * d * 2 + 2 * T * N * 2 + (d * P + R * d) * 2 + params)


def bench_project(args, only_m130=False):
    """The dt/B/C projections (conv activation x w_x, dt_in x w_dt on the matrix cores) at the 130m
    layer shape (T 16384, d 1536, dt_rank 48, N 16) and the 1.4B one (d 4096, dt_rank 128)."""
    import torch

    import selective_state_space_causal_amd as mm
    from selective_state_space_causal_amd import inputs

    out = {}
    names = ["k_proj_pack", "k_proj_in", "k_proj_dt"]
    shapes = (("m130", 8, 2048, 1536, 48), ("m1p4b", 8, 2048, 4096, 128))
    for name, S, L, d, R in shapes[:1] if only_m130 else shapes:
        N = 16
        T = S * L
        rng = np.random.default_rng(3)
        x = dev(inputs.token_tensor(0, 1, (0, T), (0, d), "bf16"))
        p = inputs.params(0, d, N, 4)
        w_x = dev(inputs.f32_to_bf16_bits((rng.standard_normal((d, R + 2 * N)) / np.sqrt(d)).astype(np.float32)))
        w_dt = dev(inputs.f32_to_bf16_bits((rng.standard_normal((R, d)) / np.sqrt(R)).astype(np.float32)))
        cu = dev(inputs.cu_from_lengths([L] * S))
        cs = torch.zeros((S, d, 3), device="cuda")
        cw, cb = dev(p["conv_w"]), dev(p["conv_b"])
        dt = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
        Bo = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        Co = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(int(mm.load().mamba_mixer_project_workspace_bytes(T, d, N, R)), 1), dtype=torch.uint8,
                         device="cuda")
        ms, kern = _time_calls(lambda ev: mm.project(x, cw, cb, cu, cs, w_x, w_dt, dt=dt, B=Bo, C=Co, workspace=ws,
                                                     events=ev), len(names), names, reps=20)
        alg = project_alg_bytes(T, S, d, N, R)
        roofs = {}
        for k in ("k_proj_in", "k_proj_dt"):
            gbs = alg[k] / (kern[k] * 1e-3) / 1e9
            prof = PROFILE_PROJECT.get((k, name))
            roofs[k] = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                            frac=round(gbs / HBM_PEAK_GBS, 4),
                            traffic=counted_traffic(prof) if prof else None,
                            kernel=k, kernel_ms=round(kern[k], 4), alg_bytes_per_launch=alg[k])
        dom = max(("k_proj_in", "k_proj_dt"), key=lambda k: kern[k])
        flops = 2.0 * T * d * (R + 2 * N) + 2.0 * T * R * d
        kms = kern["k_proj_in"] + kern["k_proj_dt"]
        out[name] = dict(
            workload=f"dt/B/C projections: {S} x {L} tokens, d_inner {d}, dt_rank {R}, d_state {N}, bf16",
            ms=round(ms, 4), kernels_ms={k: round(v, 4) for k, v in kern.items()},
            tokens_per_s=round(T / (ms * 1e-3), 1),
            roofline=roofs[dom], kernel_rooflines=roofs,
            call_hbm_view=dict(alg_bytes=alg["call"], achieved_GBs=round(alg["call"] / (kms * 1e-3) / 1e9, 1),
                               note="the projection as one operation over the two projection kernels' time "
                                    "(the weight re-layout excluded: it depends on the weights only)"),
            mfma_view=dict(achieved_TFLOPs=round(flops / (kms * 1e-3) / 1e12, 2), peak_TFLOPs=2500.0,
                           note="algorithmic bf16 FLOP (2 T d (R+2N) + 2 T R d) over both kernels' time; the "
                                "kernels issue twice that (high and low operand parts)"))
        del x, dt, Bo, Co, ws, w_x, w_dt
    torch.cuda.empty_cache()
    return out


def bench_decode(args):
    """Batch-256 decode: a 512-token prefill initialises the states, then 128 decode steps.

    Measurements of the same 128 steps:
      * per-kernel time with the 256 MB Infinity Cache flushed before every step (a 1 GiB
        buffer is read; the kernel is timed alone with HIP events on the launch stream):
        this is the HBM-roofline number;
      * the 128 steps captured in one HIP graph and replayed back to back (the serving loop
        without host launch overhead; the fp32 state may stay cache-resident between steps);
      * the same steps launched eagerly from Python;
      * the replay decode (checkpoint + ring of the window's inputs) over the same steps,
        flushed per kernel and as a HIP graph; its last output must equal the eager one.
    Every measurement starts from the prefilled states.
    """
    import torch

    import selective_state_space_causal_amd as mm
    from selective_state_space_causal_amd import inputs

    Bs, Linit, steps, d, N, K, io = 256, 512, 128, 8192, 16, 4, "bf16"
    T = Bs * Linit
    t0 = time.perf_counter()
    tok, p, cs, ss, cu = make_prefill_set(0, [Linit] * Bs, d, N, io)
    log(f"[bench] decode init inputs generated in {time.perf_counter() - t0:.1f}s")
    prm = [dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")]
    csd, ssd = dev(cs), dev(ss)
    xin = [dev(tok[k]) for k in ("x", "z", "dt", "B", "C")]
    del tok
    names = mm.kernel_names(Bs, T, d, N, K)
    ev = HipEvents(len(names) + 1)
    cud = dev(cu)
    # a first call on copies of the states loads the code object; the second is the one timed
    mm.prefill(*xin, *prm, cud, csd.clone(), ssd.clone())
    mm.prefill(*xin, *prm, cud, csd, ssd, events=ev.ev)
    init_kern = {n: ev.ms(k, k + 1) for k, n in enumerate(names)}
    init_ms = ev.ms(0, len(names))
    ev.close()
    del xin
    torch.cuda.empty_cache()
    cs0, ss0 = csd.clone(), ssd.clone()
    t0 = time.perf_counter()
    # the steps' inputs stacked [steps, Bs, ...]: four consecutive steps are also a replay window's ring
    stk = {k: [] for k in ("x", "z", "dt", "B", "C")}
    for s in range(steps):
        dt_ = inputs.decode_inputs(0, s, Bs, d, N, io)
        for k in stk:
            stk[k].append(dev(dt_[k]))
    stk = {k: torch.stack(v) for k, v in stk.items()}
    dins = [[stk[k][s] for k in ("x", "z", "dt", "B", "C")] for s in range(steps)]
    log(f"[bench] decode step inputs generated in {time.perf_counter() - t0:.1f}s")
    y = torch.empty((Bs, d), dtype=torch.bfloat16, device="cuda")

    def restore():
        csd.copy_(cs0)
        ssd.copy_(ss0)

    # warm-up (then the states are restored)
    for s in range(min(args.warmup, steps)):
        mm.decode(*dins[s], *prm, csd, ssd, y=y)
    torch.cuda.synchronize()

    # (1) flushed, per kernel: before each step a 1 GiB buffer is read (not written), so the
    # Infinity Cache holds clean lines of that buffer and no write-back of earlier steps'
    # dirty lines lands inside the timed kernel
    restore()
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s in range(steps):
        flush.sum()
        evs[s][0].record()
        mm.decode(*dins[s], *prm, csd, ssd, y=y)
        evs[s][1].record()
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    del flush
    y_flushed_last = y.clone()

    # (1b) replay decode over the same steps: windows of W steps, each window's ring is a
    # view of four consecutive stacked steps; flushed per-kernel timing (graph below)
    W = 4

    def replay(s, stream=None):
        w0 = (s // W) * W
        return mm.decode_replay(stk["x"][w0:w0 + W], stk["dt"][w0:w0 + W], stk["B"][w0:w0 + W], stk["z"][s],
                                stk["C"][s], *prm, csd, ssd, s - w0, y=y, stream=stream)

    restore()
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s in range(steps):
        flush.sum()
        rev[s][0].record()
        replay(s)
        rev[s][1].record()
    torch.cuda.synchronize()
    rkern = [a.elapsed_time(b) for a, b in rev]
    del flush
    y_replay_flushed_last = y.clone()

    # (1c) dual-precision replay (bf16 copy of the checkpoint read by the steps that do not
    # commit), flushed per kernel; the copy is made from the restored fp32 state first
    restore()
    clo, slo = mm.replay_checkpoint_lo(csd, ssd)

    def replay_dual(s, stream=None):
        w0 = (s // W) * W
        return mm.decode_replay_dual(stk["x"][w0:w0 + W], stk["dt"][w0:w0 + W], stk["B"][w0:w0 + W], stk["z"][s],
                                     stk["C"][s], *prm, csd, ssd, clo, slo, s - w0, y=y, stream=stream)

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dev_ = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s in range(steps):
        flush.sum()
        dev_[s][0].record()
        replay_dual(s)
        dev_[s][1].record()
    torch.cuda.synchronize()
    dkern = [a.elapsed_time(b) for a, b in dev_]
    del flush
    y_dual_flushed_last = y.clone()  # the last step commits: equal to the eager step
    if args.decode_flushed_only:  # profiling runs: only the flushed dispatches
        return dict(Bs=Bs, d=d, N=N, K=K, steps=steps, kern_ms=float(np.mean(kern_ms)),
                    replay_kern_ms=float(np.mean(rkern)), dual_kern_ms=float(np.mean(dkern)))

    # (2) HIP graph of the 128 steps, replayed back to back
    restore()
    gstream = torch.cuda.Stream()
    gstream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gstream):
        with torch.cuda.graph(g, stream=gstream):
            for s in range(steps):
                mm.decode(*dins[s], *prm, csd, ssd, y=y, stream=gstream)
    torch.cuda.current_stream().wait_stream(gstream)
    torch.cuda.synchronize()
    g.replay()  # warm-up replay
    torch.cuda.synchronize()
    restore()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1)
    same = bool(torch.equal(y, y_flushed_last))

    # (3) eager Python loop
    restore()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        mm.decode(*dins[s], *prm, csd, ssd, y=y)
    torch.cuda.synchronize()
    eager_s = time.perf_counter() - t0
    y_eager_last = y.clone()

    replay_matches = bool(torch.equal(y_replay_flushed_last, y_eager_last))
    restore()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gstream):
        with torch.cuda.graph(g2, stream=gstream):
            for s in range(steps):
                replay(s, stream=gstream)
    torch.cuda.current_stream().wait_stream(gstream)
    torch.cuda.synchronize()
    g2.replay()
    torch.cuda.synchronize()
    restore()
    torch.cuda.synchronize()
    e0.record()
    g2.replay()
    e1.record()
    torch.cuda.synchronize()
    rgraph_ms = e0.elapsed_time(e1)
    replay_graph_matches = bool(torch.equal(y, y_eager_last))
    # dual-precision replay as a HIP graph (the bf16 copy refreshed from the restored state first)
    restore()
    mm.replay_checkpoint_lo(csd, ssd, clo, slo)
    torch.cuda.synchronize()
    g3 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gstream):
        with torch.cuda.graph(g3, stream=gstream):
            for s in range(steps):
                replay_dual(s, stream=gstream)
    torch.cuda.current_stream().wait_stream(gstream)
    torch.cuda.synchronize()
    g3.replay()
    torch.cuda.synchronize()
    restore()
    mm.replay_checkpoint_lo(csd, ssd, clo, slo)
    torch.cuda.synchronize()
    e0.record()
    g3.replay()
    e1.record()
    torch.cuda.synchronize()
    dgraph_ms = e0.elapsed_time(e1)
    dual_matches = bool(torch.equal(y, y_eager_last)) and bool(torch.equal(y_dual_flushed_last, y_eager_last))
    return dict(Bs=Bs, d=d, N=N, K=K, steps=steps, kern_ms=float(np.mean(kern_ms)),
                kern_ms_min=float(np.min(kern_ms)), graph_ms=graph_ms, eager_s=eager_s,
                graph_matches_eager=same, init_T=T, init_ms=init_ms, init_kern=init_kern,
                replay=dict(W=W, kern_ms=float(np.mean(rkern)), kern_ms_min=float(np.min(rkern)),
                            kern_ms_by_k=[float(np.mean(rkern[k::W])) for k in range(W)], graph_ms=rgraph_ms,
                            matches_eager=replay_matches and replay_graph_matches),
                dual=dict(W=W, kern_ms=float(np.mean(dkern)), kern_ms_min=float(np.min(dkern)),
                          kern_ms_by_k=[float(np.mean(dkern[k::W])) for k in range(W)], graph_ms=dgraph_ms,
                          last_step_matches_eager=dual_matches))


def cpu_baseline(lens, d, N, io):
    """The fp64 oracle on this host's cores: full prefills of the headline workload (all tokens, all
    channels), repeated until about 12 s of CPU time have been spent (at most 8 runs), and one
    thread on its first sequence."""
    import oracle

    oracle.build(force=False)
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    threads = oracle.threads(min(ncpu, 64))
    tok, p, cs, ss, cu = make_prefill_set(0, lens, d, N, io)
    T = int(sum(lens))
    runs, c0, t0 = 0, time.process_time(), time.perf_counter()
    while runs < 8 and (runs == 0 or time.process_time() - c0 < 12.0):
        oracle.prefill(tok["x"], tok["z"], tok["dt"], tok["B"], tok["C"], p["A_log"], p["D"], p["dt_bias"],
                       p["conv_w"], p["conv_b"], cu, cs, ss)
        runs += 1
    el = time.perf_counter() - t0
    cpu = time.process_time() - c0
    # one thread, on one sequence of the workload (the oracle's cost is linear in tokens x channels)
    oracle.threads(1)
    t1 = time.perf_counter()
    L0 = lens[0]
    oracle.prefill(tok["x"][:L0], tok["z"][:L0], tok["dt"][:L0], tok["B"][:L0], tok["C"][:L0], p["A_log"], p["D"],
                   p["dt_bias"], p["conv_w"], p["conv_b"], np.array([0, L0], dtype=np.int32), cs[:1], ss[:1])
    el1 = time.perf_counter() - t1
    oracle.threads(threads)
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return dict(value=round(runs * T / el, 1), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{runs} full prefills of the headline workload ({len(lens)} packed sequences, T={T}, d={d}, "
                       f"N={N}), fp64, {el:.2f} s wall, {cpu:.1f} s CPU on {threads} threads (input widening to "
                       "fp64 included)",
                single_thread=dict(value=round(L0 / el1, 1), unit="tokens/s",
                                   sample=f"one sequence of {L0} tokens, d={d}, N={N}, {el1:.2f} s"),
                cpu_model=model)


def copy_calibration():
    """A plain copy of a known size: 1 GiB read + 1 GiB written per launch (torch's copy kernel)."""
    import torch

    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps(dict(copy_calibration=True, bytes_read_per_launch=1 << 30, bytes_written_per_launch=1 << 30,
                          launches=3)), flush=True)


def hbm_probe():
    """Plain streams of known size on this GPU with torch's own kernels: write-only (fill) and
    read+write (copy), each timed alone with events after a 1 GiB read that leaves the Infinity
    Cache holding clean lines of another buffer.  Context for the HBM rooflines: what a simple
    stream reaches here against the 8 TB/s peak."""
    import torch

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    res = []
    for mib in (64, 256, 1024):
        n = (mib << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        ops = (("write", n * 4, lambda: a.fill_(2.0)), ("copy", n * 8, lambda: b.copy_(a)))
        for name, nbytes, fn in ops:
            for _ in range(3):
                fn()
            ts = []
            for _ in range(10):
                flush.sum()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ms = float(np.median(ts))
            res.append(dict(op=name, MiB=mib, bytes=nbytes, us=round(ms * 1e3, 2),
                            GBs=round(nbytes / (ms * 1e-3) / 1e9, 1)))
            log(f"[hbm-probe] {name:5s} {mib:5d} MiB  {ms * 1e3:9.2f} us  {res[-1]['GBs']:8.1f} GB/s")
        del a, b
    print(json.dumps(dict(hbm_probe=res, peak_GBs=HBM_PEAK_GBS,
                          note="median of 10 launches, each after a 1 GiB read")), flush=True)


def _short_kernel_name(name):
    return name.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0]


def summarize_rocprof(path):
    import csv

    rows = list(csv.DictReader(open(path)))
    if rows and "Counter_Name" in rows[0]:
        agg = {}
        for r in rows:
            key = (_short_kernel_name(r["Kernel_Name"]), r["Counter_Name"])
            agg.setdefault(key, []).append(float(r["Counter_Value"]))
        print(f"{'kernel':46s} {'counter':12s} {'dispatches':>10s} {'avg_per_dispatch':>18s} {'min':>14s} {'max':>14s}")
        for (k, c), v in sorted(agg.items()):
            print(f"{k[:46]:46s} {c:12s} {len(v):10d} {np.mean(v):18.1f} {np.min(v):14.1f} {np.max(v):14.1f}")
        return
    print(f"{'kernel':42s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'total%':>7s}")
    for r in rows:
        name = _short_kernel_name(r["Name"])
        print(f"{name[:42]:42s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
              f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):7.2f}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed back-to-back calls before each timed measurement (the clocks' ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-other-prefills", action="store_true",
                    help="skip the other prefill workloads (130m-shaped, 2.8B-shaped long) and packed vs separate")
    ap.add_argument("--no-backward", action="store_true", help="skip the prefill backward timing")
    ap.add_argument("--no-project", action="store_true", help="skip the projection timing")
    ap.add_argument("--only-prefill", metavar="WORKLOAD",
                    help="only this prefill workload (m1p4b_packed, m130_prefill, m2p8b_long): the kernel-trace "
                         "and counter runs of its profile")
    ap.add_argument("--only-project", action="store_true",
                    help="only the projection timing at the 130m shape (the kernel-trace and counter runs of its "
                         "profile)")
    ap.add_argument("--only-backward", action="store_true",
                    help="only the backward timing (the kernel-trace and counter runs of its profile)")
    ap.add_argument("--only-decode", action="store_true", help="only the decode measurements")
    ap.add_argument("--decode-flushed-only", action="store_true",
                    help="with --only-decode: only the flushed-cache eager and replay decode dispatches "
                         "(the kernel-trace and counter runs of the profiles)")
    ap.add_argument("--summarize-rocprof", metavar="CSV",
                    help="print a per-kernel table of a rocprofv3 kernel_stats.csv or counter_collection.csv "
                         "and exit")
    ap.add_argument("--source-sha", action="store_true", help="print the HIP source hash and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy three times (to scale HBM byte counters)")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="time plain write and copy streams of 64 MiB to 1 GiB and exit")
    args = ap.parse_args()
    global SETTLE_MS
    SETTLE_MS = args.settle_ms
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof)
        return
    if args.source_sha:
        print(kernel_source_sha256())
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the mixer core shards by channel or sequence with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.hbm_probe:
        hbm_probe()
        return

    import torch

    import selective_state_space_causal_amd as mm

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mm.load()
    log(f"[bench] {mm.version()} on {torch.cuda.get_device_name(0)}")
    diag = dict(metric=METRIC, note="diagnostic run (profiling); no headline value")
    if args.only_prefill:
        pf = bench_prefill_workload(args.only_prefill, args.steps, args.warmup)
        print(json.dumps(dict(diag, prefill={args.only_prefill: prefill_line(pf)})), flush=True)
        return
    if args.only_project:
        print(json.dumps(dict(diag, project=bench_project(args))), flush=True)
        return
    if args.only_backward:
        print(json.dumps(dict(diag, backward=bench_backward(args))), flush=True)
        return
    if args.only_decode:
        out = decode_result(args) if not args.decode_flushed_only else bench_decode(args)
        print(json.dumps(dict(diag, decode=out)), flush=True)
        return

    head = prefill_line(bench_prefill_workload("m1p4b_packed", args.steps, args.warmup))
    out = dict(metric=METRIC, value=head["tokens_per_s"], unit="tokens/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup,
               settle=dict(ms=args.settle_ms, steps=head["settle_steps"],
                           note="untimed back-to-back steps after the warmup, before the timed ones (the GPU's "
                                "clocks ramp over ~20 ms of load)"),
               ms_per_step=head["ms_per_step"], higher_is_better=True, scaling="weak", vs_baseline=None,
               dtype="f32", io_dtype="bf16", data="synthetic",
               config=dict(workload=head["workload"], T=16384, S=len(prefill_workloads()["m1p4b_packed"]["lens"]),
                           d_inner=4096, d_state=16, d_conv=4, chunk_len=head["chunk_len"], engine=head["engine"]),
               roofline=head["roofline"], kernels_ms=head["kernels_ms"],
               dtype_note="the path computes in fp32 (fp32 state); x, z, dt, B, C and y are bf16 in HBM")
    if not args.no_other_prefills:
        out["other_prefills"] = {n: prefill_line(bench_prefill_workload(n, args.steps, args.warmup))
                                 for n in ("m130_prefill", "m2p8b_long")}
        out["packed_vs_separate"] = bench_packed_vs_separate()
    if not args.no_backward:
        out["backward"] = bench_backward(args)
    if not args.no_project:
        out["project"] = bench_project(args)
    if not args.no_decode:
        out["decode"] = decode_result(args)
    if not args.no_cpu_baseline:
        wl = prefill_workloads()["m1p4b_packed"]
        out["cpu_baseline"] = cpu_baseline(wl["lens"], wl["d"], 16, "bf16")
    print(json.dumps(out), flush=True)


def replay_result(dc):
    rp = dc["replay"]
    rb = replay_alg_bytes(dc["Bs"], dc["d"], dc["N"], dc["K"], 2, rp["W"])
    gbs = rb / (rp["kern_ms"] * 1e-3) / 1e9
    return dict(
        what="replay decode (checkpoint + ring of the last W steps' x, dt, B; the state is written once "
             "per window), same 128 steps",
        W=rp["W"],
        steps_per_s=round(dc["steps"] / (rp["graph_ms"] * 1e-3), 1),
        steps_per_s_note="128 steps captured in one HIP graph and replayed back to back",
        steps_per_s_kernel_flushed=round(1e3 / rp["kern_ms"], 1),
        kernel_ms_by_window_step=[round(v, 4) for v in rp["kern_ms_by_k"]],
        roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(gbs / HBM_PEAK_GBS, 4), traffic=counted_traffic(PROFILE_REPLAY),
                      kernel="k_decode_replay",
                      kernel_ms=round(rp["kern_ms"], 4), alg_bytes_per_launch_mean=round(rb),
                      note="mean over the window; kernel timed alone, Infinity Cache flushed before each step"),
        y_matches_eager_decode=rp["matches_eager"])


def dual_alg_bytes(Bs, d, N, K, s_io, W):
    """Mean bytes per dual-precision replay step over a window of W steps: the steps that do not
    commit read the bf16 copy of the checkpoint (N + 4 bf16 per (row, channel)); the committing
    step reads the fp32 checkpoint and writes it and its copy; every step reads the buffered x,
    dt, B of steps 0..k, its z and C, the parameters, and writes y."""
    total = 0
    for k in range(W):
        b = Bs * d * 2 * (k + 1) * s_io + Bs * N * (k + 1) * s_io  # buffered x, dt and B
        b += Bs * d * 2 * s_io + Bs * N * s_io                      # z in, y out; C
        b += d * (N + K + 3) * 4                                    # parameters
        if k == W - 1:
            b += 2 * Bs * d * (N + K - 1) * 4 + Bs * d * (N + 4) * 2  # fp32 checkpoint in and out, bf16 copy out
        else:
            b += Bs * d * (N + 4) * 2                                 # bf16 copy in
        total += b
    return total / W


def dual_result(dc):
    rp = dc["dual"]
    rb = dual_alg_bytes(dc["Bs"], dc["d"], dc["N"], dc["K"], 2, rp["W"])
    gbs = rb / (rp["kern_ms"] * 1e-3) / 1e9
    return dict(
        what="replay decode with the dual-precision checkpoint (the steps that do not commit read a bf16 copy of "
             "the checkpoint; the committing step reads the fp32 one and rewrites both), same 128 steps",
        W=rp["W"],
        steps_per_s=round(dc["steps"] / (rp["graph_ms"] * 1e-3), 1),
        steps_per_s_note="128 steps captured in one HIP graph and replayed back to back",
        steps_per_s_kernel_flushed=round(1e3 / rp["kern_ms"], 1),
        kernel_ms_by_window_step=[round(v, 4) for v in rp["kern_ms_by_k"]],
        roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(gbs / HBM_PEAK_GBS, 4), traffic=counted_traffic(PROFILE_DUAL),
                      kernel="k_decode_replay (dual)", kernel_ms=round(rp["kern_ms"], 4),
                      alg_bytes_per_launch_mean=round(rb),
                      note="mean over the window; kernel timed alone, Infinity Cache flushed before each step"),
        committing_step_matches_eager_decode=rp["last_step_matches_eager"])


def decode_result(args):
    dc = bench_decode(args)
    db = decode_alg_bytes(dc["Bs"], dc["d"], dc["N"], dc["K"], 2)
    gbs = db / (dc["kern_ms"] * 1e-3) / 1e9
    ib = prefill_alg_bytes(dc["init_T"], dc["Bs"], dc["d"], dc["N"], dc["K"], 2)
    return dict(
        workload="falcon-mamba-7b-shaped decode: batch 256, d_inner 8192, d_state 16, conv 4, bf16 io, "
                 "states from a 512-token prefill, 128 single-token steps",
        steps_per_s=round(dc["steps"] / (dc["graph_ms"] * 1e-3), 1),
        steps_per_s_note="128 steps captured in one HIP graph and replayed back to back",
        tokens_per_s=round(dc["Bs"] * dc["steps"] / (dc["graph_ms"] * 1e-3), 1),
        steps_per_s_eager_python=round(dc["steps"] / dc["eager_s"], 1),
        steps_per_s_kernel_flushed=round(1e3 / dc["kern_ms"], 1),
        roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(gbs / HBM_PEAK_GBS, 4), traffic=counted_traffic(PROFILE_DECODE),
                      kernel="k_decode_vec",
                      kernel_ms=round(dc["kern_ms"], 4), kernel_ms_min=round(dc["kern_ms_min"], 4),
                      alg_bytes_per_launch=db,
                      note="kernel timed alone with HIP events, Infinity Cache flushed before each step",
                      steady_state=dict(
                          kernel_ms=round(dc["graph_ms"] / dc["steps"], 4),
                          achieved_GBs=round(db / (dc["graph_ms"] / dc["steps"] * 1e-3) / 1e9, 1),
                          frac=round(db / (dc["graph_ms"] / dc["steps"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          note="the graph's back-to-back steps (one kernel each, no gaps between them): here "
                               "every step also writes back the previous step's state from the Infinity "
                               "Cache, which after a read flush the timed kernel can leave dirty in the cache")),
        graph_replay_matches_flushed_run=dc["graph_matches_eager"],
        replay=replay_result(dc),
        replay_dual=dual_result(dc),
        init_prefill=dict(T=dc["init_T"], ms=round(dc["init_ms"], 3),
                          tokens_per_s=round(dc["init_T"] / (dc["init_ms"] * 1e-3), 1),
                          kernels_ms={k: round(v, 4) for k, v in dc["init_kern"].items()},
                          hbm_GBs=round(ib / (dc["init_ms"] * 1e-3) / 1e9, 1)))


if __name__ == "__main__":
    main()
