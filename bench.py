"""Benchmark of the selective-SSM mixer core on one MI355X.

One step = one prefill call over the Mamba-130m-shaped layer workload (8 packed
sequences of 2048 tokens, d_inner 1536, N 16, bf16 io, fp32 state): conv + SiLU,
softplus, discretisation, the segmented selective scan, readout and gate, and the
final-state write-back.  `value` is prefill tokens/s with all inputs resident in
HBM.  The same JSON line also carries the batch-256 decode measurement (Falcon-
Mamba-7B-shaped: d_inner 8192, N 16, state initialised by a 512-token prefill,
then 128 single-token steps), the per-kernel times measured with HIP events on
the launch stream, the roofline of the dominant kernel, and the fp64 CPU oracle
timed on this host as a baseline.

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
# FP32 vector peak 157.3 TFLOP/s = 256 CUs x 2.4 GHz x 128 FMA lanes/clk x 2; one issue slot = one
# plain fp32 op (an FMA counts 2 flops), a transcendental (exp2/log2/rcp) issues at a quarter of the
# rate and counts 4 slots.
ALU_PEAK_TFLOPS = 157.3
TRANS_SLOTS = 4


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

PREFILL_PROFILE_SUFFIX = "__m130_prefill_8x2048_d1536_N16_bf16.txt"  # profiles/<final kernel><suffix>
PROFILE_DECODE = os.path.join(ROOT, "profiles", "k_decode_vec__m7b_decode_b256_d8192_N16_bf16.txt")
PROFILE_REPLAY = os.path.join(ROOT, "profiles", "k_decode_replay__m7b_decode_b256_d8192_N16_W4_bf16.txt")
PROFILE_BACKWARD = os.path.join(ROOT, "profiles", "k_row_bwd__m130_backward_8x2048_d1536_N16_bf16.txt")
PROFILE_PROJECT = os.path.join(ROOT, "profiles", "k_project__m130_project_8x2048_d1536_R48_N16_bf16.txt")


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


def alu_slots_per_token_channel(N):
    """Issue slots of the method's fp32 arithmetic per (token, channel), transcendentals weighted x4.

    conv 4 FMA; SiLU(xc) = xc / (1 + exp(-xc)): add, mul + exp, rcp; softplus = log(1 + exp(v)):
    2 adds + exp, log; delta*u 1; per state index: delta*A, delta*u*B, the state FMA, the readout FMA
    (4) + 1 exp; D*u 1; SiLU(z) 2 + exp, rcp; gating multiply 1.
    """
    plain = 4 + 2 + 2 + 1 + 4 * N + 1 + 2 + 1
    trans = 2 + 2 + N + 2
    return plain + TRANS_SLOTS * trans, plain, trans


def alu_slots_backward(N):
    """Issue slots of the backward's fp32 arithmetic per (token, channel): the forward's (its
    per-token quantities and states are recomputed, not stored) plus the adjoint's.  Adjoint per
    state index: the lambda update 2, the dC term 1, the dB term 1, the S1 term and sum 2, the S2
    term lambda h a A and sum 4, the dA term 1 (11); per token: dp 1, dz 3, du 2, d(delta) 2,
    d(dt) 1 + sigmoid (add + exp, rcp), d(xc) 4 + sigmoid (add + exp, rcp), dconv_w 4, dconv_b 1,
    dx 4, dD 1, ddt_bias 1, dt + dt_bias and masks 3 (29 plain + 4 transcendentals)."""
    f_slots, f_plain, f_trans = alu_slots_per_token_channel(N)
    plain = f_plain + 11 * N + 29
    trans = f_trans + 4
    return plain + TRANS_SLOTS * trans, plain, trans


def make_prefill_set(seed, lens, d, N, io):
    from selective_state_space_causal_amd import inputs

    T = int(sum(lens))
    tok = inputs.prefill_inputs(seed, T, d, N, io)
    p = inputs.params(seed, d, N, 4)
    cs, ss = inputs.zero_states(len(lens), d, N, 4)
    cu = inputs.cu_from_lengths(lens)
    return tok, p, cs, ss, cu


def bench_prefill(args):
    import torch

    import selective_state_space_causal_amd as mm

    S, L, d, N, K, io = 8, 2048, 1536, 16, 4, "bf16"
    T = S * L
    lens = [L] * S
    names = mm.kernel_names(S, T, d, N, K)
    nk = len(names)
    # two resident input sets, used alternately, so the 256 MB Infinity Cache cannot hold a whole step
    sets = []
    for seed in (0, 1):
        tok, p, cs, ss, cu = make_prefill_set(seed, lens, d, N, io)
        st = dict(x=dev(tok["x"]), z=dev(tok["z"]), dt=dev(tok["dt"]), B=dev(tok["B"]), C=dev(tok["C"]),
                  A_log=dev(p["A_log"]), D=dev(p["D"]), dt_bias=dev(p["dt_bias"]), conv_w=dev(p["conv_w"]),
                  conv_b=dev(p["conv_b"]), cu=dev(cu), cs=dev(cs), ss=dev(ss))
        st["y"] = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
        st["ws"] = torch.empty(mm.workspace_bytes(S, T, d, N), dtype=torch.uint8, device="cuda")
        sets.append(st)
    torch.cuda.synchronize()

    def step(i, events=None):
        st = sets[i % 2]
        mm.prefill(st["x"], st["z"], st["dt"], st["B"], st["C"], st["A_log"], st["D"], st["dt_bias"],
                   st["conv_w"], st["conv_b"], st["cu"], st["cs"], st["ss"], y=st["y"], workspace=st["ws"],
                   events=events)

    ev = HipEvents(args.steps * (nk + 1))  # created before the timed steps: no idle time between them
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    n_settle = settle(step)
    # the timed steps, back to back, without instrumentation
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same steps again with HIP events around each kernel, for the per-kernel times
    for i in range(args.steps):
        step(i, ev.ev[i * (nk + 1):(i + 1) * (nk + 1)])
    torch.cuda.synchronize()
    per_kernel = {n: [] for n in names}
    for i in range(args.steps):
        b = i * (nk + 1)
        for k, n in enumerate(names):
            per_kernel[n].append(ev.ms(b + k, b + k + 1))
    ev.close()
    kern_ms = {n: float(np.mean(v)) for n, v in per_kernel.items()}
    plan = mm.plan(S, T, d, N, K)
    return dict(S=S, L=L, T=T, d=d, N=N, K=K, wall_s=wall, kern_ms=kern_ms, names=names,
                chunk_len=plan["chunk_len"], engine=plan["engine_name"], settle_steps=n_settle)


def _time_prefill_call(mm, st, lens, d, N, reps, chunk_len=0, events=True):
    """Mean event time (ms) of whole prefill calls on resident inputs (the library launches on torch's
    current stream), states zeroed before each call; the first call is a warm-up."""
    import torch

    times = []

    def call(i):
        mm.prefill(st["x"], st["z"], st["dt"], st["B"], st["C"], st["A_log"], st["D"], st["dt_bias"],
                   st["conv_w"], st["conv_b"], st["cu"], st["cs"], st["ss"], y=st["y"], chunk_len=chunk_len)

    settle(call)
    for r in range(reps + 1):
        st["cs"].zero_()
        st["ss"].zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        mm.prefill(st["x"], st["z"], st["dt"], st["B"], st["C"], st["A_log"], st["D"], st["dt_bias"],
                   st["conv_w"], st["conv_b"], st["cu"], st["cs"], st["ss"], y=st["y"], chunk_len=chunk_len)
        e1.record()
        torch.cuda.synchronize()
        if r > 0:
            times.append(e0.elapsed_time(e1))
    return float(np.mean(times))


def bench_other_prefills(args):
    """Prefill rates of the other configurations (context; the headline is the 130m step):
    the packed 1.4B-shaped stream, the same sequences one call each (PackMamba's comparison),
    one 8192-token chunk of the 2.8B-shaped long sequence, and that sequence's 16 chunk calls."""
    import torch

    import selective_state_space_causal_amd as mm
    from selective_state_space_causal_amd import inputs

    out = {}

    def resident(lens, d, N, seed=0):
        tok, p, cs, ss, cu = make_prefill_set(seed, lens, d, N, "bf16")
        st = {k: dev(v) for k, v in tok.items()}
        st.update({k: dev(p[k]) for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")})
        st.update(cu=dev(cu), cs=dev(cs), ss=dev(ss))
        st["y"] = torch.empty((int(sum(lens)), d), dtype=torch.bfloat16, device="cuda")
        return st

    # 1.4B-shaped packed stream, and the same sequences one call each
    lens = inputs.packed_lengths(0, 16384, 128, 4096).tolist()
    d = 4096
    st = resident(lens, d, 16)
    T = int(sum(lens))
    ms = _time_prefill_call(mm, st, lens, d, 16, reps=5)
    plan = mm.plan(len(lens), T, d, 16)
    sep_ms = 0.0
    off = 0
    for L in lens:  # one call per sequence, each on its own slice of the same inputs
        sub = dict(st)
        for k in ("x", "z", "dt", "B", "C", "y"):
            sub[k] = st[k][off:off + L]
        sub["cu"] = torch.tensor([0, L], dtype=torch.int32, device="cuda")
        sub["cs"], sub["ss"] = st["cs"][:1].clone(), st["ss"][:1].clone()
        sep_ms += _time_prefill_call(mm, sub, [L], d, 16, reps=3)
        off += L
    out["m1p4b_packed"] = dict(
        workload=f"1.4B-shaped packed prefill: {len(lens)} sequences, lengths U[128,4096] to T={T}, d_inner {d}",
        tokens_per_s=round(T / (ms * 1e-3), 1), ms=round(ms, 4), engine=plan["engine_name"],
        chunk_len=plan["chunk_len"], kernels=plan["kernels"],
        separate_calls_ms=round(sep_ms, 4), packed_speedup_over_separate=round(sep_ms / ms, 3))
    del st
    # 2.8B-shaped long sequence: 16 chunk calls of 8192 tokens carrying the state (for timing,
    # every call takes the same 8192 resident input tokens; the parity tests use distinct ones)
    d, L, nch = 5120, 8192, 16
    st = resident([L], d, 16)
    plan = mm.plan(1, L, d, 16)
    times = []
    st["cs"].zero_()
    st["ss"].zero_()
    for k in range(nch + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        mm.prefill(st["x"], st["z"], st["dt"], st["B"], st["C"], st["A_log"], st["D"], st["dt_bias"],
                   st["conv_w"], st["conv_b"], st["cu"], st["cs"], st["ss"], y=st["y"])
        e1.record()
        torch.cuda.synchronize()
        if k > 0:  # the first call is a warm-up
            times.append(e0.elapsed_time(e1))
    tot = float(np.sum(times))
    out["m2p8b_long_chunked"] = dict(
        workload=f"2.8B-shaped long prefill: 1 sequence of {L * nch} tokens in {nch} calls of {L}, d_inner {d}, "
                 "state carried between calls",
        tokens_per_s=round(L * nch / (tot * 1e-3), 1), ms_total=round(tot, 3),
        ms_per_chunk_call=round(tot / nch, 4), engine=plan["engine_name"], chunk_len=plan["chunk_len"],
        kernels=plan["kernels"])
    del st
    torch.cuda.empty_cache()
    return out


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
    slots, plain, trans = alu_slots_backward(N)
    kb = k_bc["k_row_bwd"]
    ach = T * d * slots * 2 / (kb * 1e-3) / 1e12
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
                      per_unit=f"{slots} issue slots per (token, channel) = {plain} plain fp32 ops + {trans} "
                               f"transcendentals x {TRANS_SLOTS} (the forward's, recomputed, and the adjoint's); "
                               "FLOP = 2 x slots", note="the reverse kernel of the training step's backward"),
        io_bytes=io_bytes, io_GBs_standalone=round(io_bytes / (ms_b * 1e-3) / 1e9, 1))


def project_alg_bytes(T, S, d, N, R):
    """HBM bytes one k_project launch must move: x in, dt, B, C out (bf16), the re-laid weights,
    the conv parameters, the initial conv state and cu_seqlens."""
    P = R + 2 * N
    Pp = -(-P // 16) * 16
    dk = -(-d // 32) * 32
    Rp = -(-R // 32) * 32
    return T * d * 2 * 2 + 2 * T * N * 2 + (Pp * dk + d * Rp) * 2 + d * 5 * 4 + S * d * 3 * 4 + (S + 1) * 4


def bench_project(args, only_m130=False):
    """The dt/B/C projections (conv activation x w_x, dt_in x w_dt on the matrix cores) at the 130m
    layer shape (T 16384, d 1536, dt_rank 48, N 16) and the 1.4B one (d 4096, dt_rank 128)."""
    import torch

    import selective_state_space_causal_amd as mm
    from selective_state_space_causal_amd import inputs

    out = {}
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
        ws = torch.empty(max(int(mm.load().mamba_mixer_project_workspace_bytes(d, N, R)), 1), dtype=torch.uint8,
                         device="cuda")
        ms, kern = _time_calls(lambda ev: mm.project(x, cw, cb, cu, cs, w_x, w_dt, dt=dt, B=Bo, C=Co, workspace=ws,
                                                     events=ev), 2, ["k_proj_pack", "k_project"], reps=20)
        kp = kern["k_project"]
        alg = project_alg_bytes(T, S, d, N, R)
        gbs = alg / (kp * 1e-3) / 1e9
        flops = 2.0 * T * d * (R + 2 * N) + 2.0 * T * R * d
        out[name] = dict(
            workload=f"dt/B/C projections: {S} x {L} tokens, d_inner {d}, dt_rank {R}, d_state {N}, bf16",
            ms=round(ms, 4), kernels_ms={k: round(v, 4) for k, v in kern.items()},
            tokens_per_s=round(T / (ms * 1e-3), 1),
            roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                          frac=round(gbs / HBM_PEAK_GBS, 4),
                          traffic=counted_traffic(PROFILE_PROJECT) if name == "m130" else None,
                          kernel="k_project", kernel_ms=round(kp, 4), alg_bytes_per_launch=alg,
                          mfma_view=dict(achieved_TFLOPs=round(flops / (kp * 1e-3) / 1e12, 2), peak_TFLOPs=2500.0,
                                         note="algorithmic bf16 FLOP (2 T d (R+2N) + 2 T R d); the kernel issues "
                                              "twice that (high and low operand parts)")))
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
    mm.prefill(*xin, *prm, dev(cu), csd, ssd, events=ev.ev)
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
    if args.decode_flushed_only:  # profiling runs: only the flushed dispatches
        return dict(Bs=Bs, d=d, N=N, K=K, steps=steps, kern_ms=float(np.mean(kern_ms)),
                    replay_kern_ms=float(np.mean(rkern)))

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
    return dict(Bs=Bs, d=d, N=N, K=K, steps=steps, kern_ms=float(np.mean(kern_ms)),
                kern_ms_min=float(np.min(kern_ms)), graph_ms=graph_ms, eager_s=eager_s,
                graph_matches_eager=same, init_T=T, init_ms=init_ms, init_kern=init_kern,
                replay=dict(W=W, kern_ms=float(np.mean(rkern)), kern_ms_min=float(np.min(rkern)),
                            kern_ms_by_k=[float(np.mean(rkern[k::W])) for k in range(W)], graph_ms=rgraph_ms,
                            matches_eager=replay_matches and replay_graph_matches))


def cpu_baseline(lens, d, N, io):
    """The fp64 oracle on this host's cores: full prefills of the bench workload (all tokens, all
    channels), repeated until about 12 s of CPU time have been spent (at most 8 runs)."""
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
                sample=f"{runs} full prefills of the bench workload ({len(lens)} x {lens[0]} tokens, d={d}, N={N}), "
                       f"fp64, {el:.2f} s wall, {cpu:.1f} s CPU on {threads} threads (input widening to fp64 included)",
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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed back-to-back calls before each timed measurement (the clocks' ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="decode measurement only (for profiling)")
    ap.add_argument("--no-other-prefills", action="store_true",
                    help="skip the context prefill rates of the other configurations")
    ap.add_argument("--no-backward", action="store_true", help="skip the prefill backward timing")
    ap.add_argument("--no-project", action="store_true", help="skip the projection timing")
    ap.add_argument("--only-project", action="store_true",
                    help="only the projection timing at the 130m shape (the kernel-trace and counter runs of its "
                         "profile)")
    ap.add_argument("--only-backward", action="store_true",
                    help="only the backward timing (the kernel-trace and counter runs of its profile)")
    ap.add_argument("--decode-flushed-only", action="store_true",
                    help="with --no-prefill: only the flushed-cache eager and replay decode dispatches "
                         "(the kernel-trace and counter runs of the profiles)")
    ap.add_argument("--summarize-rocprof", metavar="CSV",
                    help="print a per-kernel table of a rocprofv3 kernel_stats.csv or counter_collection.csv "
                         "and exit")
    ap.add_argument("--source-sha", action="store_true", help="print the HIP source hash and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy three times (to scale HBM byte counters)")
    args = ap.parse_args()
    global SETTLE_MS
    SETTLE_MS = args.settle_ms
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.source_sha:
        print(kernel_source_sha256())
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the mixer core shards by channel or sequence with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import selective_state_space_causal_amd as mm

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mm.load()
    log(f"[bench] {mm.version()} on {torch.cuda.get_device_name(0)}")
    if args.only_project:
        print(json.dumps(dict(metric=METRIC, note="projection-only diagnostic run (--only-project); no headline value",
                              project=bench_project(args, only_m130=True))), flush=True)
        return
    if args.only_backward:
        print(json.dumps(dict(metric=METRIC, note="backward-only diagnostic run (--only-backward); no headline value",
                              backward=bench_backward(args))), flush=True)
        return

    if args.no_prefill:
        args.no_cpu_baseline = True
        out = dict(metric=METRIC, note="decode-only diagnostic run (--no-prefill); no headline value")
    else:
        out = prefill_result(args)
    if not args.no_prefill and not args.no_other_prefills:
        out["other_prefills"] = bench_other_prefills(args)
    if not args.no_prefill and not args.no_backward:
        out["backward"] = bench_backward(args)
    if not args.no_prefill and not args.no_project:
        out["project"] = bench_project(args)
    if not args.no_decode:
        out["decode"] = decode_result(args) if not args.decode_flushed_only else bench_decode(args)
    if not args.no_cpu_baseline:
        c = out["config"]
        out["cpu_baseline"] = cpu_baseline([c["L"]] * c["S"], c["d_inner"], c["d_state"], "bf16")
    print(json.dumps(out), flush=True)


def prefill_result(args):
    pf = bench_prefill(args)
    T, d, N, K = pf["T"], pf["d"], pf["N"], pf["K"]
    ms_per_step = pf["wall_s"] / args.steps * 1e3
    tokens_per_s = T * args.steps / pf["wall_s"]
    step_bytes = prefill_alg_bytes(T, pf["S"], d, N, K, 2)
    dom = pf["names"][-1]  # the final pass: the dominant kernel
    dom_ms = pf["kern_ms"][dom]
    slots, plain, trans = alu_slots_per_token_channel(N)
    achieved_tflops = T * d * slots * 2 / (dom_ms * 1e-3) / 1e12
    roofline = dict(bound="alu", achieved=round(achieved_tflops, 2), peak=ALU_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved_tflops / ALU_PEAK_TFLOPS, 4), traffic=counted_traffic(os.path.join(ROOT, "profiles", dom + PREFILL_PROFILE_SUFFIX)),
                    kernel=dom, kernel_ms=round(dom_ms, 4),
                    per_unit=f"{slots} issue slots per (token, channel) = {plain} plain fp32 ops + "
                             f"{trans} transcendentals x {TRANS_SLOTS}; FLOP = 2 x slots")
    out = dict(metric=METRIC, value=round(tokens_per_s, 1), unit="tokens/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, settle=dict(ms=args.settle_ms, steps=pf["settle_steps"],
                                               note="untimed back-to-back steps after the warmup, before the "
                                                    "timed ones (the GPU's clocks ramp over ~20 ms of load)"),
               ms_per_step=round(ms_per_step, 4), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="f32", io_dtype="bf16", data="synthetic",
               config=dict(workload="mamba-130m-shaped layer prefill: 8 packed sequences x 2048 tokens, "
                                    "d_inner 1536, d_state 16, conv 4, bf16 io, fp32 state",
                           S=pf["S"], L=pf["L"], T=T, d_inner=d, d_state=N, d_conv=K,
                           chunk_len=pf["chunk_len"], engine=pf["engine"]),
               roofline=roofline,
               kernels_ms={k: round(v, 4) for k, v in pf["kern_ms"].items()},
               hbm_view=dict(alg_bytes_per_step=step_bytes,
                             achieved_GBs=round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                             peak_GBs=HBM_PEAK_GBS,
                             frac=round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)))
    return out


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
                      note="kernel timed alone with HIP events, Infinity Cache flushed before each step"),
        graph_replay_matches_flushed_run=dc["graph_matches_eager"],
        replay=replay_result(dc),
        init_prefill=dict(T=dc["init_T"], ms=round(dc["init_ms"], 3),
                          tokens_per_s=round(dc["init_T"] / (dc["init_ms"] * 1e-3), 1),
                          kernels_ms={k: round(v, 4) for k, v in dc["init_kern"].items()},
                          hbm_GBs=round(ib / (dc["init_ms"] * 1e-3) / 1e9, 1)))


if __name__ == "__main__":
    main()
