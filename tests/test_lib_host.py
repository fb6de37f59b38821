"""The C-ABI library without a GPU: it loads, exports every declared entry point,
and rejects bad arguments on the host before anything is enqueued."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import selective_state_space_causal_amd as mm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MM_ERR_NULL, MM_ERR_DIM, MM_ERR_UNSUPPORTED, MM_ERR_ALIGN, MM_ERR_WORKSPACE, MM_ERR_ALIAS = -1, -2, -3, -4, -5, -6


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"\b(mamba_mixer_\w+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return mm.load()


def test_library_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert mm.version().startswith("libmambamix")
    for code in (0, -1, -2, -3, -4, -5, -6, -7, 42):
        s = mm.status_string(code)
        assert isinstance(s, str) and s


# fake, well-aligned device addresses: the calls below must fail validation before touching them
A = 0x10000000
STEP = 0x01000000


def _ptrs(n, start=A):
    return [ctypes.c_void_p(start + i * STEP) for i in range(n)]


def _prefill(lib, ptrs, S=2, T=100, d=64, N=16, K=4, io=1, ws=None, wsb=0, chunk=32):
    # 32-token chunks: a plan that needs workspace (whole sequences need none)
    return lib.mamba_mixer_prefill_chunked(*ptrs, S, T, d, N, K, io, chunk, ws, wsb, None)


def _decode(lib, ptrs, Bs=2, d=64, N=16, K=4, io=1):
    return lib.mamba_mixer_decode(*ptrs, Bs, d, N, K, io, None)


def test_prefill_validation(lib):
    p = _ptrs(14)
    ws_need = mm.workspace_bytes(2, 100, 64, 16, chunk_len=32)
    assert ws_need > 0 and mm.workspace_bytes(2, 100, 64, 16) == 0
    ws = ctypes.c_void_p(0x70000000)
    assert _prefill(lib, p, K=3, ws=ws, wsb=ws_need) == MM_ERR_UNSUPPORTED
    assert _prefill(lib, p, N=17, ws=ws, wsb=ws_need) == MM_ERR_UNSUPPORTED
    assert _prefill(lib, p, N=0, ws=ws, wsb=ws_need) == MM_ERR_UNSUPPORTED
    assert _prefill(lib, p, io=7, ws=ws, wsb=ws_need) == MM_ERR_UNSUPPORTED
    assert _prefill(lib, p, T=-1, ws=ws, wsb=ws_need) == MM_ERR_DIM
    assert _prefill(lib, p, S=-1, ws=ws, wsb=ws_need) == MM_ERR_DIM
    assert _prefill(lib, p, d=-5, ws=ws, wsb=ws_need) == MM_ERR_DIM
    assert _prefill(lib, p, S=0, T=10, ws=ws, wsb=ws_need) == MM_ERR_DIM
    assert _prefill(lib, p, T=2 ** 31, ws=ws, wsb=ws_need) == MM_ERR_DIM
    for i in range(14):
        q = list(p)
        q[i] = ctypes.c_void_p(0)
        assert _prefill(lib, q, ws=ws, wsb=ws_need) == MM_ERR_NULL, i
    # misaligned bf16 x and misaligned fp32 parameter
    q = list(p)
    q[0] = ctypes.c_void_p(A + 1)
    assert _prefill(lib, q, ws=ws, wsb=ws_need) == MM_ERR_ALIGN
    q = list(p)
    q[6] = ctypes.c_void_p(p[6].value + 2)
    assert _prefill(lib, q, ws=ws, wsb=ws_need) == MM_ERR_ALIGN
    # bf16 io only needs 2-byte alignment
    q = list(p)
    q[0] = ctypes.c_void_p(A + 2)
    assert _prefill(lib, q, ws=None, wsb=0) == MM_ERR_WORKSPACE
    # workspace too small / missing / misaligned
    assert _prefill(lib, p, ws=ws, wsb=ws_need - 1) == MM_ERR_WORKSPACE
    assert _prefill(lib, p, ws=None, wsb=ws_need) == MM_ERR_WORKSPACE
    assert _prefill(lib, p, ws=ctypes.c_void_p(0x70000010), wsb=ws_need) == MM_ERR_ALIGN
    # y aliasing x, and conv_state overlapping ssm_state
    q = list(p)
    q[13] = q[0]
    assert _prefill(lib, q, ws=ws, wsb=ws_need) == MM_ERR_ALIAS
    q = list(p)
    q[12] = ctypes.c_void_p(q[11].value + 64)
    assert _prefill(lib, q, ws=ws, wsb=ws_need) == MM_ERR_ALIAS
    # empty problems succeed without touching anything (null pointers allowed then)
    z = [ctypes.c_void_p(0)] * 14
    assert _prefill(lib, z, S=0, T=0) == 0
    assert _prefill(lib, z, S=3, T=0) == 0
    assert _prefill(lib, z, S=3, T=5, d=0) == 0


def test_decode_validation(lib):
    p = _ptrs(13)
    assert _decode(lib, p, K=5) == MM_ERR_UNSUPPORTED
    assert _decode(lib, p, N=32) == MM_ERR_UNSUPPORTED
    assert _decode(lib, p, io=2) == MM_ERR_UNSUPPORTED
    assert _decode(lib, p, Bs=-1) == MM_ERR_DIM
    for i in range(13):
        q = list(p)
        q[i] = ctypes.c_void_p(0)
        assert _decode(lib, q) == MM_ERR_NULL, i
    q = list(p)
    q[3] = ctypes.c_void_p(A + 1)
    assert _decode(lib, q) == MM_ERR_ALIGN
    q = list(p)
    q[12] = q[2]
    assert _decode(lib, q) == MM_ERR_ALIAS
    assert _decode(lib, [ctypes.c_void_p(0)] * 13, Bs=0) == 0


def test_workspace_query_and_plan(lib):
    assert mm.workspace_bytes(0, 0, 64, 16) == 0
    assert mm.workspace_bytes(1, 64, 16, 4) == 0  # one sequence, one chunk: the row engine needs none
    assert mm.workspace_bytes(1, 64, 16, 4, engine=mm.ENGINE_LANE) > 0
    # the size is a pure function of the arguments, and grows with the number of carry slots
    w1 = mm.workspace_bytes(8, 16384, 1536, 16, chunk_len=16384)
    w2 = mm.workspace_bytes(8, 16384, 1536, 16, chunk_len=256)
    assert w2 > w1
    assert mm.workspace_bytes(8, 16384, 1536, 16, chunk_len=256) == w2
    p = mm.plan(8, 16384, 1536, 16)
    assert mm.workspace_bytes(8, 16384, 1536, 16) == p["workspace_bytes"]
    # few (sequence, channel-block) pairs -> the row engine, whole sequences per chunk
    assert p["engine_name"] == "row" and p["chunk_len"] > 16384
    assert p["kernels"] == ["k_row_final"] and p["workspace_bytes"] == 0
    # many sequences -> the lane engine; sequences of the mean length are not split
    q = mm.plan(256, 131072, 8192, 16)
    assert q["engine_name"] == "lane" and q["chunk_len"] >= 512 and q["kernels"][-1] == "k_lane_final"
    # a single long sequence is split into chunks to fill the GPU: pass 1 over the pieces of the
    # non-last chunks, then the final pass, which folds the carries itself; with few sequences
    # the kernels compute the chunk plan themselves
    r = mm.plan(1, 131072, 5120, 16)
    assert r["engine_name"] == "row" and r["chunk_len"] < 131072
    assert r["kernels"] == ["k_row_agg", "k_row_final"]
    r2 = mm.plan(300, 300 * 2048, 64, 16, chunk_len=512, engine=2)
    assert r2["kernels"] == ["k_chunk_plan", "k_row_agg", "k_row_final"]
    # pass-1 pieces have their own carry slots: one sequence of 8192 tokens in 2048-token
    # chunks (3 non-last chunks) with 320 channel blocks takes 4 pieces per chunk to give
    # pass 1 about 8 workgroups per CU.  Workspace: the chunk offsets, then sum(delta) and the
    # end state per slot (slots for the 4-chunk bound x 4 pieces), the stash per chunk
    d = 5120
    assert mm.workspace_bytes(1, 8192, d, 16, chunk_len=2048, engine=2) == \
        2 * 256 + 4 * 4 * d * 4 + 4 * 4 * d * 16 * 4 + 4 * d * 19 * 4
    # explicit engines and chunk lengths are honoured (chunk lengths round up to 16)
    for e, name in ((1, "lane"), (2, "row")):
        pe = mm.plan(3, 500, 100, 16, chunk_len=40, engine=e)
        assert pe["engine_name"] == name and pe["chunk_len"] == 48
    # unknown engine
    with pytest.raises(mm.MambaMixError):
        mm.plan(3, 500, 100, 16, engine=3)
    p = _ptrs(14)
    ws = ctypes.c_void_p(0x70000000)
    rc = lib.mamba_mixer_prefill_ex(*p, 2, 100, 64, 16, 4, 1, 0, 9, ws, 1 << 30, None, None, 0)
    assert rc == MM_ERR_UNSUPPORTED
    # too few events for the kernels of the call
    evs = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    rc = lib.mamba_mixer_prefill_ex(*p, 2, 100, 64, 16, 4, 1, 32, 0, ws, 1 << 30, None, evs, 2)
    assert rc == MM_ERR_DIM


def _replay(lib, ptrs, Bs=2, d=64, N=16, K=4, io=1, W=4, k=0, commit=0):
    return lib.mamba_mixer_decode_replay(*ptrs, Bs, d, N, K, io, W, k, commit, None)


def test_decode_replay_validation(lib):
    p = _ptrs(13)
    assert _replay(lib, p, N=8) == MM_ERR_UNSUPPORTED  # 4 lanes x 4 state entries per channel: N must be 16
    assert _replay(lib, p, K=3) == MM_ERR_UNSUPPORTED
    assert _replay(lib, p, W=5) == MM_ERR_DIM
    assert _replay(lib, p, W=0) == MM_ERR_DIM
    assert _replay(lib, p, k=4) == MM_ERR_DIM
    assert _replay(lib, p, k=-1) == MM_ERR_DIM
    assert _replay(lib, p, W=2, k=2) == MM_ERR_DIM
    for i in range(13):
        q = list(p)
        q[i] = ctypes.c_void_p(0)
        assert _replay(lib, q) == MM_ERR_NULL, i
    q = list(p)
    q[2] = ctypes.c_void_p(A + 2)  # B_ring rows are read 4 bf16 at a time
    assert _replay(lib, q) == MM_ERR_ALIGN
    q = list(p)
    q[11] = ctypes.c_void_p(p[11].value + 4)  # ssm_state needs 16 bytes
    assert _replay(lib, q) == MM_ERR_ALIGN
    q = list(p)
    q[12] = q[3]  # y aliases z
    assert _replay(lib, q) == MM_ERR_ALIAS
    q = list(p)
    q[11] = q[10]  # ssm_state overlaps conv_state
    assert _replay(lib, q) == MM_ERR_ALIAS
    assert _replay(lib, [ctypes.c_void_p(0)] * 13, Bs=0) == 0


def _multi(lib, ptrs, Bs=2, d=64, N=16, K=4, io=1, W=4, k0=0, k1=3, cstep=-1):
    return lib.mamba_mixer_decode_replay_multi(*ptrs, Bs, d, N, K, io, W, k0, k1, cstep, None)


def test_decode_replay_multi_validation(lib):
    p = _ptrs(13)
    assert _multi(lib, p, N=12) == MM_ERR_UNSUPPORTED
    assert _multi(lib, p, k0=2, k1=1) == MM_ERR_DIM
    assert _multi(lib, p, k1=4) == MM_ERR_DIM
    assert _multi(lib, p, W=2, k1=2) == MM_ERR_DIM
    assert _multi(lib, p, cstep=4) == MM_ERR_DIM
    assert _multi(lib, p, k1=2, cstep=3) == MM_ERR_DIM
    assert _multi(lib, p, cstep=-2) == MM_ERR_DIM
    for i in range(13):
        q = list(p)
        q[i] = ctypes.c_void_p(0)
        assert _multi(lib, q) == MM_ERR_NULL, i
    q = list(p)
    q[4] = ctypes.c_void_p(A + 2)  # C_ring rows are read 4 bf16 at a time
    assert _multi(lib, q) == MM_ERR_ALIGN
    q = list(p)
    q[12] = ctypes.c_void_p(p[3].value + 64)  # y_ring overlaps z_ring
    assert _multi(lib, q) == MM_ERR_ALIAS
    assert _multi(lib, [ctypes.c_void_p(0)] * 13, d=0) == 0


def _backward(lib, ptrs, S=2, T=100, d=64, N=16, K=4, io=1, ws=None, wsb=0):
    # ptrs: the 14 inputs, dy, then the 12 outputs; the checkpoint pointer (NULL) goes in after dy
    return lib.mamba_mixer_prefill_backward(*ptrs[:14], None, *ptrs[14:], S, T, d, N, K, io, ws, wsb, None, None, 0)


def test_backward_plan_and_validation(lib):
    # workspace: per-block checkpoints + per-channel-block dB/dC partials + parameter partials
    need = mm.backward_plan(2, 100, 64, 16)
    rows = (100 + 15) // 16 + 2
    assert need["kernels"] == 4
    assert need["workspace"] >= rows * 64 * 16 * 4 + 4 * 2 * 100 * 16 * 4
    assert lib.mamba_mixer_prefill_backward_workspace_bytes(2, 100, 64, 16, 4, 0) == need["workspace"]
    with_ck = mm.backward_plan(2, 100, 64, 16, has_ckpt=True)
    assert with_ck["kernels"] == 3
    assert with_ck["workspace"] == need["workspace"] - mm.checkpoint_bytes(2, 100, 64)
    assert mm.checkpoint_bytes(2, 100, 64) == rows * 64 * 16 * 4
    assert mm.backward_plan(0, 0, 64, 16) == {"workspace": 0, "kernels": 1}
    assert mm.backward_plan(3, 0, 64, 16)["kernels"] == 4
    p = _ptrs(26)
    ws = ctypes.c_void_p(0x7F000000)
    wsb = need["workspace"]
    assert _backward(lib, p, K=3, ws=ws, wsb=wsb) == MM_ERR_UNSUPPORTED
    assert _backward(lib, p, N=17, ws=ws, wsb=wsb) == MM_ERR_UNSUPPORTED
    assert _backward(lib, p, io=5, ws=ws, wsb=wsb) == MM_ERR_UNSUPPORTED
    assert _backward(lib, p, T=-1, ws=ws, wsb=wsb) == MM_ERR_DIM
    assert _backward(lib, p, S=0, T=10, ws=ws, wsb=wsb) == MM_ERR_DIM
    for i in range(26):
        q = list(p)
        q[i] = ctypes.c_void_p(0)
        assert _backward(lib, q, ws=ws, wsb=wsb) == MM_ERR_NULL, i
    q = list(p)
    q[14] = ctypes.c_void_p(p[14].value + 1)  # dx misaligned for bf16
    assert _backward(lib, q, ws=ws, wsb=wsb) == MM_ERR_ALIGN
    q = list(p)
    q[19] = ctypes.c_void_p(p[19].value + 2)  # dA_log misaligned for fp32
    assert _backward(lib, q, ws=ws, wsb=wsb) == MM_ERR_ALIGN
    assert _backward(lib, p, ws=ws, wsb=wsb - 1) == MM_ERR_WORKSPACE
    assert _backward(lib, p, ws=None, wsb=wsb) == MM_ERR_WORKSPACE
    assert _backward(lib, p, ws=ctypes.c_void_p(0x7F000010), wsb=wsb) == MM_ERR_ALIGN
    for out, other in ((14, 0), (18, 4), (24, 12), (25, 24), (19, 20)):  # an output on an input or another output
        q = list(p)
        q[out] = q[other]
        assert _backward(lib, q, ws=ws, wsb=wsb) == MM_ERR_ALIAS, (out, other)
    # d == 0 is a no-op; T == 0 needs only the parameter and state arrays
    assert _backward(lib, [ctypes.c_void_p(0)] * 26, d=0) == 0
    q = list(p)
    for i in (0, 1, 2, 3, 4, 13, 14, 15, 16, 17, 18):
        q[i] = ctypes.c_void_p(0)
    assert _backward(lib, q, T=0, ws=None, wsb=0) == MM_ERR_WORKSPACE  # passes the pointer checks


def test_prefill_train_validation(lib):
    p = _ptrs(15)  # the 14 prefill pointers (y last) and ckpt
    need = mm.workspace_bytes(2, 100, 64, 16, chunk_len=32, engine=mm.ENGINE_ROW)
    ws = ctypes.c_void_p(0x7F000000)

    def call(q, **kw):
        a = dict(S=2, T=100, d=64, N=16, K=4, io=1, chunk=32)
        a.update(kw)
        return lib.mamba_mixer_prefill_train(*q, a["S"], a["T"], a["d"], a["N"], a["K"], a["io"], a["chunk"], ws,
                                             need, None, None, 0)
    q = list(p)
    q[14] = ctypes.c_void_p(0)
    assert call(q) == MM_ERR_NULL
    q = list(p)
    q[14] = q[13]  # checkpoints on top of y
    assert call(q) == MM_ERR_ALIAS
    q = list(p)
    q[14] = ctypes.c_void_p(p[14].value + 2)
    assert call(q) == MM_ERR_ALIGN
    assert call([ctypes.c_void_p(0)] * 15, T=0) == 0


def test_project_validation(lib):
    # x, conv_w, conv_b, cu, conv_state, w_x, w_dt, dt, B, C
    p = _ptrs(10)
    need = lib.mamba_mixer_project_workspace_bytes(100, 64, 16, 4)
    # w_x re-laid, padded to 48 x 64, w_dt to 32 x 64, and dt_in's high and low parts [100][32], bf16
    assert need == 48 * 64 * 2 + 32 * 64 * 2 + 2 * ((100 * 32 * 2 + 255) // 256 * 256)
    assert lib.mamba_mixer_project_workspace_bytes(-1, 64, 16, 4) == 0
    ws = ctypes.c_void_p(0x7F000000)

    def call(q, S=2, T=100, d=64, N=16, R=4, K=4, io=1, wsb=need, w=ws):
        return lib.mamba_mixer_project(*q, S, T, d, N, R, K, io, w, wsb, None, None, 0)
    assert call(p, io=0) == MM_ERR_UNSUPPORTED       # fp32 io: not supported
    assert call(p, d=40) == MM_ERR_UNSUPPORTED       # d not a multiple of 16
    assert call(p, R=0) == MM_ERR_UNSUPPORTED
    assert call(p, R=257) == MM_ERR_UNSUPPORTED
    assert call(p, T=1, d=(1 << 22) + 16) == MM_ERR_UNSUPPORTED  # past the projection's channel limit
    assert call(p, S=0) == MM_ERR_DIM
    for i in range(10):
        q = list(p)
        q[i] = ctypes.c_void_p(0)
        assert call(q) == MM_ERR_NULL, i
    q = list(p)
    q[0] = ctypes.c_void_p(p[0].value + 2)  # x needs 16-byte rows
    assert call(q) == MM_ERR_ALIGN
    q = list(p)
    q[7] = q[0]  # dt on top of x
    assert call(q) == MM_ERR_ALIAS
    assert call(p, wsb=need - 1) == MM_ERR_WORKSPACE
    assert call([ctypes.c_void_p(0)] * 10, T=0) == 0


def test_row_engine_channel_limit(lib):
    """The row layout keeps per-lane tile offsets in 32 bits up to MM_ROW_MAX_D channels: past it
    the automatic plan takes the lane engine, and the row engine, the training forward and the
    backward report MM_ERR_UNSUPPORTED."""
    big = 4194304 + 16
    assert mm.plan(1, 64, 4194304, 16, 4, 0, mm.ENGINE_ROW)["engine_name"] == "row"
    assert mm.plan(1, 64, big, 16)["engine_name"] == "lane"
    with pytest.raises(mm.MambaMixError) as e:
        mm.plan(1, 64, big, 16, 4, 0, mm.ENGINE_ROW)
    assert e.value.code == MM_ERR_UNSUPPORTED
    with pytest.raises(mm.MambaMixError) as e:
        mm.backward_plan(1, 64, big, 16)
    assert e.value.code == MM_ERR_UNSUPPORTED
    assert lib.mamba_mixer_prefill_backward_workspace_bytes(1, 64, big, 16, 4, 0) == 0


def test_noalloc_prefill_rejects_plans_beyond_its_scratch(lib):
    """A plan whose workspace exceeds the fixed scratch (here 65.6 MB of lane-engine carries and
    packed B/C) is MM_ERR_WORKSPACE, found on the host before any device call; argument errors
    come first."""
    S, T, d, N = 8192, 327680, 256, 16
    need = mm.workspace_bytes(S, T, d, N)
    assert need > mm.NOALLOC_SCRATCH_BYTES
    big = 0x100000000  # fake device addresses 4 GiB apart: no two arrays overlap
    ptrs = [ctypes.c_void_p(0x1000000000 + i * big) for i in range(14)]
    assert lib.mamba_mixer_prefill_noalloc(*ptrs, S, T, d, N, 4, 1, None) == MM_ERR_WORKSPACE
    ptrs[3] = None
    assert lib.mamba_mixer_prefill_noalloc(*ptrs, S, T, d, N, 4, 1, None) == MM_ERR_NULL
    assert lib.mamba_mixer_prefill_noalloc(*ptrs, S, T, d, 17, 4, 1, None) == MM_ERR_UNSUPPORTED
    # nothing to do: success without touching a device
    assert lib.mamba_mixer_prefill_noalloc(*ptrs, S, 0, d, N, 4, 1, None) == 0


def test_replay_dual_host_checks(lib):
    """The dual-precision replay and its copy helper reject bad arguments on the host."""
    big = 0x100000000
    p = [ctypes.c_void_p(0x1000000000 + i * big) for i in range(15)]
    call = lambda ptrs, io=1, N=16, W=4, k=0: lib.mamba_mixer_decode_replay_dual(*ptrs, 2, 64, N, 4, io, W, k, 0, None)
    assert call(p, io=0) == MM_ERR_UNSUPPORTED  # bf16 io only
    assert call(p, N=8) == MM_ERR_UNSUPPORTED
    assert call(p, k=4) == MM_ERR_DIM
    q = list(p)
    q[13] = None  # ssm_lo
    assert call(q) == MM_ERR_NULL
    q = list(p)
    q[13] = ctypes.c_void_p(0x1000000000 + 13 * big + 8)  # ssm_lo not 16-byte aligned
    assert call(q) == MM_ERR_ALIGN
    q = list(p)
    q[13] = q[11]  # ssm_lo on top of ssm_state
    assert call(q) == MM_ERR_ALIAS
    c = [ctypes.c_void_p(0x1000000000 + i * big) for i in range(4)]
    assert lib.mamba_mixer_replay_checkpoint_lo(*c, 2, 64, 8, 4, None) == MM_ERR_UNSUPPORTED
    assert lib.mamba_mixer_replay_checkpoint_lo(c[0], c[1], c[0], c[3], 2, 64, 16, 4, None) == MM_ERR_ALIAS
    assert lib.mamba_mixer_replay_checkpoint_lo(c[0], c[1], c[2], None, 2, 64, 16, 4, None) == MM_ERR_NULL
    assert lib.mamba_mixer_replay_checkpoint_lo(*c, 0, 64, 16, 4, None) == 0


def test_check_cu_seqlens(lib):
    """The host check of the cu_seqlens preconditions (the calls never read the array on the
    host): starts at 0, never decreases, ends at T."""
    def rc(cu, T, S=None):
        a = np.ascontiguousarray(cu, dtype=np.int32)
        return lib.mamba_mixer_check_cu_seqlens(a.ctypes.data_as(ctypes.c_void_p),
                                                a.size - 1 if S is None else S, T)
    assert rc([0, 3, 3, 10], 10) == 0
    assert rc([0], 0) == 0                       # no sequences
    assert rc([0, 0, 0], 0) == 0                 # empty sequences only
    assert rc([1, 3, 10], 10) == MM_ERR_DIM      # does not start at 0
    assert rc([0, 5, 4, 10], 10) == MM_ERR_DIM   # decreases
    assert rc([0, 3, 9], 10) == MM_ERR_DIM       # does not end at T
    assert rc([0, 3, 10], -1) == MM_ERR_DIM
    assert rc([0, 3, 10], 10, S=-1) == MM_ERR_DIM
    assert lib.mamba_mixer_check_cu_seqlens(None, 2, 10) == MM_ERR_NULL
    mm.check_cu_seqlens(np.array([0, 4, 9], dtype=np.int32), 9)
    with pytest.raises(mm.MambaMixError):
        mm.check_cu_seqlens(np.array([0, 9, 4], dtype=np.int32), 4)
