"""libmambamix: the selective-SSM mixer core as a C-ABI HIP library for gfx950 (MI355X).

This module is a thin ctypes binding of ``include/mambamix.h``.  It only checks
shapes/dtypes, allocates outputs and workspace with torch (device memory and
streams are all torch is used for) and passes raw device pointers to the C ABI;
every step of the computation runs in the HIP kernels of ``libmambamix.so``.
There is no CPU or PyTorch fallback: if the library is missing the calls raise.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmambamix.so")

MM_OK = 0
MM_IO_F32 = 0
MM_IO_BF16 = 1
ENGINE_AUTO, ENGINE_LANE, ENGINE_ROW = 0, 1, 2
ENGINE_NAMES = {1: "lane", 2: "row"}
MAX_N = 16
CONV_K = 4

_lib = None


class MambaMixError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} (status {code})")


def load() -> ctypes.CDLL:
    """Load libmambamix.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    # torch first: the library then binds to the HIP runtime torch has loaded, the one that owns
    # the streams and device memory it is handed (loaded first, it would bring in a second one)
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.mamba_mixer_prefill.argtypes = [P] * 14 + [i32, i64, i32, i32, i32, i32, P, sz, P]
    lib.mamba_mixer_prefill.restype = ctypes.c_int
    lib.mamba_mixer_prefill_chunked.argtypes = [P] * 14 + [i32, i64, i32, i32, i32, i32, i64, P, sz, P]
    lib.mamba_mixer_prefill_chunked.restype = ctypes.c_int
    lib.mamba_mixer_prefill_noalloc.argtypes = [P] * 14 + [i32, i64, i32, i32, i32, i32, P]
    lib.mamba_mixer_prefill_noalloc.restype = ctypes.c_int
    lib.mamba_mixer_prefill_workspace_bytes.argtypes = [i32, i64, i32, i32, i32]
    lib.mamba_mixer_prefill_workspace_bytes.restype = sz
    lib.mamba_mixer_prefill_workspace_bytes_chunked.argtypes = [i32, i64, i32, i32, i32, i64]
    lib.mamba_mixer_prefill_workspace_bytes_chunked.restype = sz
    lib.mamba_mixer_prefill_ex.argtypes = [P] * 14 + [i32, i64, i32, i32, i32, i32, i64, i32, P, sz, P, P, i32]
    lib.mamba_mixer_prefill_ex.restype = ctypes.c_int
    lib.mamba_mixer_prefill_plan.argtypes = [i32, i64, i32, i32, i32, i64, i32, ctypes.POINTER(i64),
                                             ctypes.POINTER(i32), ctypes.POINTER(sz), ctypes.POINTER(i32)]
    lib.mamba_mixer_prefill_plan.restype = ctypes.c_int
    lib.mamba_mixer_prefill_kernel_name.argtypes = [i32, i64, i32, i32, i32, i64, i32, i32]
    lib.mamba_mixer_prefill_kernel_name.restype = ctypes.c_char_p
    lib.mamba_mixer_decode.argtypes = [P] * 13 + [i32, i32, i32, i32, i32, P]
    lib.mamba_mixer_decode.restype = ctypes.c_int
    lib.mamba_mixer_decode_replay.argtypes = [P] * 13 + [i32, i32, i32, i32, i32, i32, i32, i32, P]
    lib.mamba_mixer_decode_replay.restype = ctypes.c_int
    lib.mamba_mixer_decode_replay_dual.argtypes = [P] * 15 + [i32] * 8 + [P]
    lib.mamba_mixer_decode_replay_dual.restype = ctypes.c_int
    lib.mamba_mixer_replay_checkpoint_lo.argtypes = [P] * 4 + [i32] * 4 + [P]
    lib.mamba_mixer_replay_checkpoint_lo.restype = ctypes.c_int
    lib.mamba_mixer_decode_replay_multi.argtypes = [P] * 13 + [i32] * 9 + [P]
    lib.mamba_mixer_decode_replay_multi.restype = ctypes.c_int
    lib.mamba_mixer_prefill_backward.argtypes = [P] * 27 + [i32, i64, i32, i32, i32, i32, P, sz, P, P, i32]
    lib.mamba_mixer_prefill_backward.restype = ctypes.c_int
    lib.mamba_mixer_prefill_backward_plan.argtypes = [i32, i64, i32, i32, i32, i32, ctypes.POINTER(sz),
                                                      ctypes.POINTER(i32)]
    lib.mamba_mixer_prefill_backward_plan.restype = ctypes.c_int
    lib.mamba_mixer_prefill_backward_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i32]
    lib.mamba_mixer_prefill_backward_workspace_bytes.restype = sz
    lib.mamba_mixer_prefill_train.argtypes = [P] * 15 + [i32, i64, i32, i32, i32, i32, i64, P, sz, P, P, i32]
    lib.mamba_mixer_prefill_train.restype = ctypes.c_int
    lib.mamba_mixer_checkpoint_bytes.argtypes = [i32, i64, i32]
    lib.mamba_mixer_checkpoint_bytes.restype = sz
    lib.mamba_mixer_project.argtypes = [P] * 10 + [i32, i64, i32, i32, i32, i32, i32, P, sz, P, P, i32]
    lib.mamba_mixer_project.restype = ctypes.c_int
    lib.mamba_mixer_project_workspace_bytes.argtypes = [i64, i32, i32, i32]
    lib.mamba_mixer_project_workspace_bytes.restype = sz
    lib.mamba_mixer_status_string.argtypes = [ctypes.c_int]
    lib.mamba_mixer_status_string.restype = ctypes.c_char_p
    lib.mamba_mixer_version.argtypes = []
    lib.mamba_mixer_version.restype = ctypes.c_char_p
    lib.mamba_mixer_check_cu_seqlens.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64]
    lib.mamba_mixer_check_cu_seqlens.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().mamba_mixer_status_string(int(code)).decode()


def version() -> str:
    return load().mamba_mixer_version().decode()


# MAMBAMIX_CHECK_CU=1 makes every call check its cu_seqlens first (a device-to-host copy and a
# sync per call: for debugging).
CHECK_CU = os.environ.get("MAMBAMIX_CHECK_CU", "") == "1"


def check_cu_seqlens(cu_seqlens, T: int) -> None:
    """Raise MambaMixError unless cu_seqlens [S+1] (device or host int32) starts at 0, never
    decreases and ends at T: the precondition of every call that takes it."""
    import numpy as np

    cu = np.ascontiguousarray(cu_seqlens.detach().cpu().numpy() if hasattr(cu_seqlens, "detach") else cu_seqlens,
                              dtype=np.int32)
    if cu.ndim != 1 or cu.size < 1:
        raise ValueError("cu_seqlens: expected a 1-D array of S+1 >= 1 entries")
    rc = load().mamba_mixer_check_cu_seqlens(cu.ctypes.data_as(ctypes.c_void_p), cu.size - 1, int(T))
    if rc != 0:
        raise MambaMixError(rc, "mamba_mixer_check_cu_seqlens")


def plan(S: int, T: int, d: int, N: int, K: int = CONV_K, chunk_len: int = 0, engine: int = ENGINE_AUTO) -> dict:
    """What a prefill call with these sizes does: chunk length, engine, workspace bytes, kernel names."""
    lib = load()
    L, e, w, k = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_size_t(), ctypes.c_int32()
    rc = lib.mamba_mixer_prefill_plan(S, T, d, N, K, chunk_len, engine, ctypes.byref(L), ctypes.byref(e),
                                      ctypes.byref(w), ctypes.byref(k))
    if rc != MM_OK:
        raise MambaMixError(rc, "mamba_mixer_prefill_plan")
    names = [lib.mamba_mixer_prefill_kernel_name(S, T, d, N, K, chunk_len, engine, i).decode()
             for i in range(k.value)]
    return dict(chunk_len=L.value, engine=e.value, engine_name=ENGINE_NAMES.get(e.value, "none"),
                workspace_bytes=w.value, kernels=names)


def workspace_bytes(S: int, T: int, d: int, N: int, K: int = CONV_K, chunk_len: int = 0,
                    engine: int = ENGINE_AUTO) -> int:
    return plan(S, T, d, N, K, chunk_len, engine)["workspace_bytes"]


def chunk_len(S: int, T: int, d: int, N: int, K: int = CONV_K, engine: int = ENGINE_AUTO) -> int:
    return plan(S, T, d, N, K, 0, engine)["chunk_len"]


def kernel_names(S: int, T: int, d: int, N: int, K: int = CONV_K, chunk_len: int = 0,
                 engine: int = ENGINE_AUTO) -> list[str]:
    """Names of the kernels one prefill call enqueues, in order."""
    return plan(S, T, d, N, K, chunk_len, engine)["kernels"]


def _io_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return MM_IO_F32
    if t.dtype == torch.bfloat16:
        return MM_IO_BF16
    raise TypeError(f"io tensors must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(t, shape, dtype, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def prefill(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state, ssm_state,
            y=None, workspace=None, chunk_len: int = 0, stream=None, events=None, engine: int = ENGINE_AUTO):
    """Run the mixer over packed sequences; conv_state / ssm_state are updated in place.

    x, z, dt [T, d] and B, C [T, N] share one io dtype (float32 or bfloat16); A_log [d, N],
    D/dt_bias/conv_b [d], conv_w [d, 4], conv_state [S, d, 3], ssm_state [S, d, N] are float32;
    cu_seqlens [S+1] int32.  Returns y [T, d] (io dtype).
    """
    import torch

    T, d = x.shape
    N = B.shape[1]
    S = cu_seqlens.shape[0] - 1
    io = x.dtype
    for t, n in ((x, "x"), (z, "z"), (dt, "dt")):
        _check(t, (T, d), io, n)
    for t, n in ((B, "B"), (C, "C")):
        _check(t, (T, N), io, n)
    _check(A_log, (d, N), torch.float32, "A_log")
    for t, n in ((D, "D"), (dt_bias, "dt_bias"), (conv_b, "conv_b")):
        _check(t, (d,), torch.float32, n)
    _check(conv_w, (d, CONV_K), torch.float32, "conv_w")
    _check(cu_seqlens, (S + 1,), torch.int32, "cu_seqlens")
    if CHECK_CU:
        check_cu_seqlens(cu_seqlens, T)
    _check(conv_state, (S, d, CONV_K - 1), torch.float32, "conv_state")
    _check(ssm_state, (S, d, N), torch.float32, "ssm_state")
    if y is None:
        y = torch.empty((T, d), dtype=io, device=x.device)
    _check(y, (T, d), io, "y")
    if workspace is None:  # (a caller-provided workspace is size-checked by the library)
        need = workspace_bytes(S, T, d, N, CONV_K, chunk_len, engine) if T > 0 and d > 0 and S > 0 else 0
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wptr = _ptr(workspace) if workspace is not None else ctypes.c_void_p(0)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if events is None:
        ev, nev = None, 0
    else:  # raw hipEvent_t handles, recorded around each kernel of the call
        ev = (ctypes.c_void_p * len(events))(*events)
        nev = len(events)
    rc = load().mamba_mixer_prefill_ex(
        _ptr(x), _ptr(z), _ptr(dt), _ptr(B), _ptr(C), _ptr(A_log), _ptr(D), _ptr(dt_bias), _ptr(conv_w),
        _ptr(conv_b), _ptr(cu_seqlens), _ptr(conv_state), _ptr(ssm_state), _ptr(y),
        S, T, d, N, CONV_K, _io_code(x), int(chunk_len), int(engine), wptr, wbytes, _stream(stream), ev, nev)
    if rc != MM_OK:
        raise MambaMixError(rc, "mamba_mixer_prefill")
    return y


NOALLOC_SCRATCH_BYTES = 32 << 20  # MM_NOALLOC_SCRATCH_BYTES


def prefill_noalloc(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state, ssm_state, y=None,
                    stream=None):
    """``prefill`` through mamba_mixer_prefill_noalloc: the automatic plan with its workspace in the
    library's fixed per-GPU scratch (at most NOALLOC_SCRATCH_BYTES), so the call allocates no
    workspace; y is allocated here only when not given.  Calls that overlap on one GPU race on the
    scratch."""
    import torch

    T, d = x.shape
    N = B.shape[1]
    S = cu_seqlens.shape[0] - 1
    io = x.dtype
    for t, n in ((x, "x"), (z, "z"), (dt, "dt")):
        _check(t, (T, d), io, n)
    for t, n in ((B, "B"), (C, "C")):
        _check(t, (T, N), io, n)
    _check(A_log, (d, N), torch.float32, "A_log")
    for t, n in ((D, "D"), (dt_bias, "dt_bias"), (conv_b, "conv_b")):
        _check(t, (d,), torch.float32, n)
    _check(conv_w, (d, CONV_K), torch.float32, "conv_w")
    _check(cu_seqlens, (S + 1,), torch.int32, "cu_seqlens")
    if CHECK_CU:
        check_cu_seqlens(cu_seqlens, T)
    _check(conv_state, (S, d, CONV_K - 1), torch.float32, "conv_state")
    _check(ssm_state, (S, d, N), torch.float32, "ssm_state")
    if y is None:
        y = torch.empty((T, d), dtype=io, device=x.device)
    _check(y, (T, d), io, "y")
    rc = load().mamba_mixer_prefill_noalloc(
        _ptr(x), _ptr(z), _ptr(dt), _ptr(B), _ptr(C), _ptr(A_log), _ptr(D), _ptr(dt_bias), _ptr(conv_w),
        _ptr(conv_b), _ptr(cu_seqlens), _ptr(conv_state), _ptr(ssm_state), _ptr(y),
        S, T, d, N, CONV_K, _io_code(x), _stream(stream))
    if rc != MM_OK:
        raise MambaMixError(rc, "mamba_mixer_prefill_noalloc")
    return y


def backward_plan(S: int, T: int, d: int, N: int, K: int = CONV_K, has_ckpt: bool = False) -> dict:
    """Workspace bytes and kernel count of one prefill_backward call (host only)."""
    w, k = ctypes.c_size_t(0), ctypes.c_int32(0)
    rc = load().mamba_mixer_prefill_backward_plan(S, T, d, N, K, int(bool(has_ckpt)), ctypes.byref(w),
                                                  ctypes.byref(k))
    if rc != MM_OK:
        raise MambaMixError(rc, "mamba_mixer_prefill_backward_plan")
    return {"workspace": w.value, "kernels": k.value}


BACKWARD_GRADS = ("dx", "dz", "ddt", "dB", "dC", "dA_log", "dD", "ddt_bias", "dconv_w", "dconv_b",
                  "dconv_state", "dssm_state")


def checkpoint_bytes(S: int, T: int, d: int) -> int:
    return int(load().mamba_mixer_checkpoint_bytes(S, T, d))


def prefill_train(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state, ssm_state,
                  y=None, ckpt=None, workspace=None, chunk_len: int = 0, stream=None, events=None):
    """The forward of a training step: ``prefill`` on the row engine that also stores the state
    before every 16-token block.  Returns (y, ckpt); ckpt [ceil(T/16) + S, d, 16] float32 goes to
    ``prefill_backward(..., ckpt=ckpt)`` together with the INITIAL conv state."""
    import torch

    T, d = x.shape
    N = B.shape[1]
    S = cu_seqlens.shape[0] - 1
    io = x.dtype
    for t, n in ((x, "x"), (z, "z"), (dt, "dt")):
        _check(t, (T, d), io, n)
    for t, n in ((B, "B"), (C, "C")):
        _check(t, (T, N), io, n)
    _check(A_log, (d, N), torch.float32, "A_log")
    for t, n in ((D, "D"), (dt_bias, "dt_bias"), (conv_b, "conv_b")):
        _check(t, (d,), torch.float32, n)
    _check(conv_w, (d, CONV_K), torch.float32, "conv_w")
    _check(cu_seqlens, (S + 1,), torch.int32, "cu_seqlens")
    if CHECK_CU:
        check_cu_seqlens(cu_seqlens, T)
    _check(conv_state, (S, d, CONV_K - 1), torch.float32, "conv_state")
    _check(ssm_state, (S, d, N), torch.float32, "ssm_state")
    if y is None:
        y = torch.empty((T, d), dtype=io, device=x.device)
    _check(y, (T, d), io, "y")
    rows = (T + 15) // 16 + S
    if ckpt is None:
        ckpt = torch.empty((rows, d, 16), dtype=torch.float32, device=x.device)
    _check(ckpt, (rows, d, 16), torch.float32, "ckpt")
    if workspace is None:  # (a caller-provided workspace is size-checked by the library)
        need = workspace_bytes(S, T, d, N, CONV_K, chunk_len, ENGINE_ROW) if T > 0 and d > 0 and S > 0 else 0
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wptr = _ptr(workspace) if workspace is not None else ctypes.c_void_p(0)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ev, nev = (None, 0) if events is None else ((ctypes.c_void_p * len(events))(*events), len(events))
    rc = load().mamba_mixer_prefill_train(
        _ptr(x), _ptr(z), _ptr(dt), _ptr(B), _ptr(C), _ptr(A_log), _ptr(D), _ptr(dt_bias), _ptr(conv_w),
        _ptr(conv_b), _ptr(cu_seqlens), _ptr(conv_state), _ptr(ssm_state), _ptr(y), _ptr(ckpt),
        S, T, d, N, CONV_K, _io_code(x), int(chunk_len), wptr, wbytes, _stream(stream), ev, nev)
    if rc != MM_OK:
        raise MambaMixError(rc, "mamba_mixer_prefill_train")
    return y, ckpt


def prefill_backward(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, cu_seqlens, conv_state, ssm_state, dy,
                     ckpt=None, out=None, workspace=None, stream=None, events=None):
    """Gradients of a prefill call given dy = dL/dy; conv_state / ssm_state are the INITIAL
    states (read only; with ``ckpt`` from ``prefill_train`` the forward is not run again and
    ssm_state is not read, so it may be None).  Returns a dict of the tensors named in
    BACKWARD_GRADS: dx, dz, ddt [T, d] and dB, dC [T, N] in the io dtype, the rest float32
    (dconv_state, dssm_state are the gradients of the initial states).  `out` may pass
    preallocated tensors of that dict.
    """
    import torch

    T, d = x.shape
    N = B.shape[1]
    S = cu_seqlens.shape[0] - 1
    io = x.dtype
    for t, n in ((x, "x"), (z, "z"), (dt, "dt"), (dy, "dy")):
        _check(t, (T, d), io, n)
    for t, n in ((B, "B"), (C, "C")):
        _check(t, (T, N), io, n)
    _check(A_log, (d, N), torch.float32, "A_log")
    for t, n in ((D, "D"), (dt_bias, "dt_bias"), (conv_b, "conv_b")):
        _check(t, (d,), torch.float32, n)
    _check(conv_w, (d, CONV_K), torch.float32, "conv_w")
    _check(cu_seqlens, (S + 1,), torch.int32, "cu_seqlens")
    if CHECK_CU:
        check_cu_seqlens(cu_seqlens, T)
    _check(conv_state, (S, d, CONV_K - 1), torch.float32, "conv_state")
    if ssm_state is not None:
        _check(ssm_state, (S, d, N), torch.float32, "ssm_state")
    elif ckpt is None:
        raise ValueError("ssm_state is needed unless ckpt is given")
    if ckpt is not None:
        _check(ckpt, ((T + 15) // 16 + S, d, 16), torch.float32, "ckpt")
    shapes = {"dx": ((T, d), io), "dz": ((T, d), io), "ddt": ((T, d), io), "dB": ((T, N), io),
              "dC": ((T, N), io), "dA_log": ((d, N), torch.float32), "dD": ((d,), torch.float32),
              "ddt_bias": ((d,), torch.float32), "dconv_w": ((d, CONV_K), torch.float32),
              "dconv_b": ((d,), torch.float32), "dconv_state": ((S, d, CONV_K - 1), torch.float32),
              "dssm_state": ((S, d, N), torch.float32)}
    g = dict(out) if out is not None else {}
    for k, (shape, dt_) in shapes.items():
        if k not in g:
            g[k] = torch.empty(shape, dtype=dt_, device=x.device)
        _check(g[k], shape, dt_, k)
    if workspace is None:  # (a caller-provided workspace is size-checked by the library)
        need = backward_plan(S, T, d, N, has_ckpt=ckpt is not None)["workspace"] if d > 0 else 0
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wptr = _ptr(workspace) if workspace is not None else ctypes.c_void_p(0)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if events is None:
        ev, nev = None, 0
    else:
        ev = (ctypes.c_void_p * len(events))(*events)
        nev = len(events)
    rc = load().mamba_mixer_prefill_backward(
        _ptr(x), _ptr(z), _ptr(dt), _ptr(B), _ptr(C), _ptr(A_log), _ptr(D), _ptr(dt_bias), _ptr(conv_w),
        _ptr(conv_b), _ptr(cu_seqlens), _ptr(conv_state),
        _ptr(ssm_state) if ssm_state is not None else ctypes.c_void_p(0), _ptr(dy),
        _ptr(ckpt) if ckpt is not None else ctypes.c_void_p(0),
        *[_ptr(g[k]) for k in BACKWARD_GRADS],
        S, T, d, N, CONV_K, _io_code(x), wptr, wbytes, _stream(stream), ev, nev)
    if rc != MM_OK:
        raise MambaMixError(rc, "mamba_mixer_prefill_backward")
    return g


def project(x, conv_w, conv_b, cu_seqlens, conv_state, w_x, w_dt, dt=None, B=None, C=None, workspace=None,
            stream=None, events=None):
    """dt [T, d], B, C [T, N] (bf16) from x [T, d] (bf16): the conv activation times w_x [d, R + 2N]
    (columns: w_dt_in, w_B, w_C) and dt_in times w_dt [R, d], on the matrix cores.  conv_state is the
    initial conv state [S, d, 3] (read only).  Returns (dt, B, C)."""
    import torch

    T, d = x.shape
    S = cu_seqlens.shape[0] - 1
    R = w_dt.shape[0]
    P = w_x.shape[1]
    if (P - R) % 2 != 0 or P <= R:
        raise ValueError(f"w_x has {P} columns; expected R + 2N with R = {R}")
    N = (P - R) // 2
    _check(x, (T, d), torch.bfloat16, "x")
    _check(conv_w, (d, CONV_K), torch.float32, "conv_w")
    _check(conv_b, (d,), torch.float32, "conv_b")
    _check(cu_seqlens, (S + 1,), torch.int32, "cu_seqlens")
    if CHECK_CU:
        check_cu_seqlens(cu_seqlens, T)
    _check(conv_state, (S, d, CONV_K - 1), torch.float32, "conv_state")
    _check(w_x, (d, P), torch.bfloat16, "w_x")
    _check(w_dt, (R, d), torch.bfloat16, "w_dt")
    if dt is None:
        dt = torch.empty((T, d), dtype=torch.bfloat16, device=x.device)
    if B is None:
        B = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    if C is None:
        C = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _check(dt, (T, d), torch.bfloat16, "dt")
    _check(B, (T, N), torch.bfloat16, "B")
    _check(C, (T, N), torch.bfloat16, "C")
    if workspace is None:  # (a caller-provided workspace is size-checked by the library)
        need = int(load().mamba_mixer_project_workspace_bytes(T, d, N, R))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    rc = load().mamba_mixer_project(
        _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(cu_seqlens), _ptr(conv_state), _ptr(w_x), _ptr(w_dt), _ptr(dt),
        _ptr(B), _ptr(C), S, T, d, N, R, CONV_K, MM_IO_BF16, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream),
        (ctypes.c_void_p * len(events))(*events) if events is not None else None,
        len(events) if events is not None else 0)
    if rc != MM_OK:
        raise MambaMixError(rc, "mamba_mixer_project")
    return dt, B, C


def decode(x, z, dt, B, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state, y=None, stream=None):
    """One decode step for Bs rows (row r uses slot r); states are updated in place.  Returns y [Bs, d]."""
    import torch

    Bs, d = x.shape
    N = B.shape[1]
    io = x.dtype
    for t, n in ((x, "x"), (z, "z"), (dt, "dt")):
        _check(t, (Bs, d), io, n)
    for t, n in ((B, "B"), (C, "C")):
        _check(t, (Bs, N), io, n)
    _check(A_log, (d, N), torch.float32, "A_log")
    for t, n in ((D, "D"), (dt_bias, "dt_bias"), (conv_b, "conv_b")):
        _check(t, (d,), torch.float32, n)
    _check(conv_w, (d, CONV_K), torch.float32, "conv_w")
    _check(conv_state, (Bs, d, CONV_K - 1), torch.float32, "conv_state")
    _check(ssm_state, (Bs, d, N), torch.float32, "ssm_state")
    if y is None:
        y = torch.empty((Bs, d), dtype=io, device=x.device)
    _check(y, (Bs, d), io, "y")
    rc = load().mamba_mixer_decode(
        _ptr(x), _ptr(z), _ptr(dt), _ptr(B), _ptr(C), _ptr(A_log), _ptr(D), _ptr(dt_bias), _ptr(conv_w),
        _ptr(conv_b), _ptr(conv_state), _ptr(ssm_state), _ptr(y), Bs, d, N, CONV_K, _io_code(x),
        _stream(stream))
    if rc != MM_OK:
        raise MambaMixError(rc, "mamba_mixer_decode")
    return y


def decode_replay(x_ring, dt_ring, B_ring, z, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state, k: int,
                  commit: bool = False, y=None, stream=None):
    """Step k of a replay window (see ``mamba_mixer_decode_replay``).

    x_ring, dt_ring [W, Bs, d] and B_ring [W, Bs, N] hold the raw inputs of window steps 0..k
    (slot k is this step's); z [Bs, d] and C [Bs, N] are this step's.  conv_state / ssm_state
    are the checkpoint (the state before window step 0); they are overwritten with the state
    after step k when the call commits (commit=True or k == W - 1).  Returns y [Bs, d].
    """
    import torch

    W, Bs, d = x_ring.shape
    N = B_ring.shape[2]
    io = x_ring.dtype
    _check(x_ring, (W, Bs, d), io, "x_ring")
    _check(dt_ring, (W, Bs, d), io, "dt_ring")
    _check(B_ring, (W, Bs, N), io, "B_ring")
    _check(z, (Bs, d), io, "z")
    _check(C, (Bs, N), io, "C")
    _check(A_log, (d, N), torch.float32, "A_log")
    for t, n in ((D, "D"), (dt_bias, "dt_bias"), (conv_b, "conv_b")):
        _check(t, (d,), torch.float32, n)
    _check(conv_w, (d, CONV_K), torch.float32, "conv_w")
    _check(conv_state, (Bs, d, CONV_K - 1), torch.float32, "conv_state")
    _check(ssm_state, (Bs, d, N), torch.float32, "ssm_state")
    if y is None:
        y = torch.empty((Bs, d), dtype=io, device=x_ring.device)
    _check(y, (Bs, d), io, "y")
    rc = load().mamba_mixer_decode_replay(
        _ptr(x_ring), _ptr(dt_ring), _ptr(B_ring), _ptr(z), _ptr(C), _ptr(A_log), _ptr(D), _ptr(dt_bias),
        _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(ssm_state), _ptr(y), Bs, d, N, CONV_K, _io_code(x_ring),
        W, int(k), 1 if commit else 0, _stream(stream))
    if rc != MM_OK:
        raise MambaMixError(rc, "mamba_mixer_decode_replay")
    return y


def replay_checkpoint_lo(conv_state, ssm_state, conv_lo=None, ssm_lo=None, stream=None):
    """The bf16 copy of a replay checkpoint for ``decode_replay_dual``: returns (conv_lo [Bs, d, 4],
    ssm_lo [Bs, d, N]) as bfloat16 (conv entry 3 zero)."""
    import torch

    Bs, d, N = ssm_state.shape
    _check(conv_state, (Bs, d, CONV_K - 1), torch.float32, "conv_state")
    _check(ssm_state, (Bs, d, N), torch.float32, "ssm_state")
    if conv_lo is None:
        conv_lo = torch.empty((Bs, d, 4), dtype=torch.bfloat16, device=ssm_state.device)
    if ssm_lo is None:
        ssm_lo = torch.empty((Bs, d, N), dtype=torch.bfloat16, device=ssm_state.device)
    _check(conv_lo, (Bs, d, 4), torch.bfloat16, "conv_lo")
    _check(ssm_lo, (Bs, d, N), torch.bfloat16, "ssm_lo")
    rc = load().mamba_mixer_replay_checkpoint_lo(_ptr(conv_state), _ptr(ssm_state), _ptr(conv_lo), _ptr(ssm_lo),
                                                 Bs, d, N, CONV_K, _stream(stream))
    if rc != MM_OK:
        raise MambaMixError(rc, "mamba_mixer_replay_checkpoint_lo")
    return conv_lo, ssm_lo


def decode_replay_dual(x_ring, dt_ring, B_ring, z, C, A_log, D, dt_bias, conv_w, conv_b, conv_state, ssm_state,
                       conv_lo, ssm_lo, k: int, commit: bool = False, y=None, stream=None):
    """Step k of a replay window with the dual-precision checkpoint (see
    ``mamba_mixer_decode_replay_dual``): steps that do not commit read only the bf16 copy
    (conv_lo [Bs, d, 4], ssm_lo [Bs, d, N]); a committing step reads the fp32 checkpoint and
    rewrites both.  bf16 io.  Returns y [Bs, d]."""
    import torch

    W, Bs, d = x_ring.shape
    N = B_ring.shape[2]
    io = x_ring.dtype
    _check(x_ring, (W, Bs, d), io, "x_ring")
    _check(dt_ring, (W, Bs, d), io, "dt_ring")
    _check(B_ring, (W, Bs, N), io, "B_ring")
    _check(z, (Bs, d), io, "z")
    _check(C, (Bs, N), io, "C")
    _check(A_log, (d, N), torch.float32, "A_log")
    for t, n in ((D, "D"), (dt_bias, "dt_bias"), (conv_b, "conv_b")):
        _check(t, (d,), torch.float32, n)
    _check(conv_w, (d, CONV_K), torch.float32, "conv_w")
    _check(conv_state, (Bs, d, CONV_K - 1), torch.float32, "conv_state")
    _check(ssm_state, (Bs, d, N), torch.float32, "ssm_state")
    _check(conv_lo, (Bs, d, 4), torch.bfloat16, "conv_lo")
    _check(ssm_lo, (Bs, d, N), torch.bfloat16, "ssm_lo")
    if y is None:
        y = torch.empty((Bs, d), dtype=io, device=x_ring.device)
    _check(y, (Bs, d), io, "y")
    rc = load().mamba_mixer_decode_replay_dual(
        _ptr(x_ring), _ptr(dt_ring), _ptr(B_ring), _ptr(z), _ptr(C), _ptr(A_log), _ptr(D), _ptr(dt_bias),
        _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(ssm_state), _ptr(conv_lo), _ptr(ssm_lo), _ptr(y),
        Bs, d, N, CONV_K, _io_code(x_ring), W, int(k), 1 if commit else 0, _stream(stream))
    if rc != MM_OK:
        raise MambaMixError(rc, "mamba_mixer_decode_replay_dual")
    return y


def decode_replay_multi(x_ring, dt_ring, B_ring, z_ring, C_ring, A_log, D, dt_bias, conv_w, conv_b, conv_state,
                        ssm_state, k0: int, k1: int, commit_step: int = -1, y_ring=None, stream=None):
    """Window steps k0..k1 in one call (see ``mamba_mixer_decode_replay_multi``): outputs into
    y_ring slots k0..k1, no state written unless commit_step >= 0.  Returns y_ring [W, Bs, d]."""
    import torch

    W, Bs, d = x_ring.shape
    N = B_ring.shape[2]
    io = x_ring.dtype
    for t, n in ((x_ring, "x_ring"), (dt_ring, "dt_ring"), (z_ring, "z_ring")):
        _check(t, (W, Bs, d), io, n)
    _check(B_ring, (W, Bs, N), io, "B_ring")
    _check(C_ring, (W, Bs, N), io, "C_ring")
    _check(A_log, (d, N), torch.float32, "A_log")
    for t, n in ((D, "D"), (dt_bias, "dt_bias"), (conv_b, "conv_b")):
        _check(t, (d,), torch.float32, n)
    _check(conv_w, (d, CONV_K), torch.float32, "conv_w")
    _check(conv_state, (Bs, d, CONV_K - 1), torch.float32, "conv_state")
    _check(ssm_state, (Bs, d, N), torch.float32, "ssm_state")
    if y_ring is None:
        y_ring = torch.empty((W, Bs, d), dtype=io, device=x_ring.device)
    _check(y_ring, (W, Bs, d), io, "y_ring")
    rc = load().mamba_mixer_decode_replay_multi(
        _ptr(x_ring), _ptr(dt_ring), _ptr(B_ring), _ptr(z_ring), _ptr(C_ring), _ptr(A_log), _ptr(D), _ptr(dt_bias),
        _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(ssm_state), _ptr(y_ring), Bs, d, N, CONV_K,
        _io_code(x_ring), W, int(k0), int(k1), int(commit_step), _stream(stream))
    if rc != MM_OK:
        raise MambaMixError(rc, "mamba_mixer_decode_replay_multi")
    return y_ring
