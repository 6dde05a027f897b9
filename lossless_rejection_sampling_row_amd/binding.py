"""ctypes binding of ``libsv_verify.so`` (declared in ``include/sv_verify.h``).

This layer only marshals arguments. It checks torch tensors against the C
ABI's layout, passes their device pointers and the current HIP stream, and
returns torch tensors. Every step of the verify path runs in the library's
kernels. There is no fallback: if the library is missing, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_int, c_int32, c_size_t, c_uint64, c_void_p

ABI_VERSION = 2
# sv_batch_stats, in order: requests, rows_tested, accepted, rejected, null_rows, bonus, greedy,
# invalid, offered, noprop, bad_draft.
STATS_FIELDS = 11
SV_F32, SV_BF16 = 0, 1

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class SvError(RuntimeError):
    """A non-zero sv_status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class SvShape(ctypes.Structure):
    _fields_ = [("B", c_int32), ("R", c_int32), ("V", c_int32), ("dtype", c_int32)]


class SvTuning(ctypes.Structure):
    """sv_tuning: launch splits (0 = the library's choice; see include/sv_verify.h)."""
    _fields_ = [("w1", c_int32), ("w2", c_int32)]


class SvFilter(ctypes.Structure):
    """sv_filter: one side's top_k / top_p / min_p device arrays (NULL = off)."""
    _fields_ = [("top_k", c_void_p), ("top_p", c_void_p), ("min_p", c_void_p)]


def library_path() -> str:
    return os.environ.get("SV_LIBRARY", os.path.join(_PKG, "libsv_verify.so"))


def load_library():
    """Load the HIP library (once). Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m lossless_rejection_sampling_row_amd.build`")
    lib = ctypes.CDLL(path)
    common = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_uint64,
              c_void_p, c_void_p, SvShape, c_void_p, c_size_t, c_void_p]
    lib.sv_verify_batch.argtypes = common
    lib.sv_verify_batch.restype = c_int
    lib.sv_verify_batch_diag.argtypes = common + [c_void_p, c_void_p, POINTER(c_void_p)]
    lib.sv_verify_batch_diag.restype = c_int
    sched = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_uint64,
             c_void_p, c_void_p, SvShape, c_void_p, c_size_t, c_void_p, c_void_p, c_void_p]
    lib.sv_verify_batch_sched.argtypes = sched
    lib.sv_verify_batch_sched.restype = c_int
    lib.sv_row_acceptance.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, SvShape, c_void_p, c_size_t, c_void_p]
    lib.sv_row_acceptance.restype = c_int
    lib.sv_row_acceptance_filtered.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                               c_void_p, POINTER(SvFilter), POINTER(SvFilter), c_void_p, c_void_p,
                                               SvShape, c_void_p, c_size_t, c_void_p]
    lib.sv_row_acceptance_filtered.restype = c_int
    lib.sv_verify_batch_filtered.argtypes = sched[:8] + [POINTER(SvFilter), POINTER(SvFilter)] + sched[8:]
    lib.sv_verify_batch_filtered.restype = c_int
    lib.sv_filter_thresholds.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, POINTER(SvFilter),
                                         POINTER(SvFilter), c_void_p, SvShape, c_void_p, c_size_t, c_void_p]
    lib.sv_filter_thresholds.restype = c_int
    lib.sv_verify_batch_lazy.argtypes = common + [c_int]
    lib.sv_verify_batch_lazy.restype = c_int
    lib.sv_verify_batch_static.argtypes = common[:10] + [c_void_p]
    lib.sv_verify_batch_static.restype = c_int
    lib.sv_verify_batch_sampler_match.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_uint64, c_void_p,
                                                  c_void_p, SvShape, c_void_p, c_size_t, c_void_p]
    lib.sv_verify_batch_sampler_match.restype = c_int
    lib.sv_set_tuning.argtypes = [POINTER(SvTuning)]
    lib.sv_set_tuning.restype = None
    lib.sv_get_tuning.argtypes = [POINTER(SvTuning)]
    lib.sv_get_tuning.restype = None
    lib.sv_workspace_bytes.argtypes = [SvShape]
    lib.sv_workspace_bytes.restype = c_size_t
    lib.sv_status_string.argtypes = [c_int]
    lib.sv_status_string.restype = ctypes.c_char_p
    lib.sv_abi_version.argtypes = []
    lib.sv_abi_version.restype = c_int
    if lib.sv_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path}: ABI version {lib.sv_abi_version()} != {ABI_VERSION}")
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load_library().sv_status_string(status).decode()


def _check(status: int):
    if status != 0:
        raise SvError(status, status_string(status))


def dtype_code(dtype) -> int:
    import torch
    if dtype == torch.bfloat16:
        return SV_BF16
    if dtype == torch.float32:
        return SV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {dtype}")


def workspace_bytes(B: int, R: int, V: int, dtype_or_code) -> int:
    code = dtype_or_code if isinstance(dtype_or_code, int) else dtype_code(dtype_or_code)
    return int(load_library().sv_workspace_bytes(SvShape(B, R, V, code)))


def set_tuning(**fields) -> None:
    """Set the process-wide launch tuning (sv_set_tuning); unnamed fields are 0 (the library's
    choice). ``set_tuning()`` restores the defaults."""
    t = SvTuning(**{k: int(v) for k, v in fields.items()})
    load_library().sv_set_tuning(ctypes.byref(t))


def get_tuning() -> dict:
    t = SvTuning()
    load_library().sv_get_tuning(ctypes.byref(t))
    return {name: getattr(t, name) for name, _ in SvTuning._fields_}


_WORKSPACES: dict = {}


def _workspace(device, nbytes: int, stream):
    """A workspace per (device, stream), grown on demand and zeroed on that stream when made.
    Calls on different streams never share one, as the library requires of concurrent calls.
    record_stream keeps a replaced workspace's memory from being reused before the stream's
    work on it is done."""
    import torch
    key = (device.type, device.index, int(stream.cuda_stream))
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            ws.record_stream(stream)
        with torch.cuda.stream(stream):
            ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        ws.record_stream(stream)
        _WORKSPACES[key] = ws
    return ws


def _ptr(t):
    return c_void_p(t.data_ptr())


def _filter_struct(filt, B: int, dev):
    """An SvFilter from (top_k [B] int32 | None, top_p [B] float32 | None, min_p [B] float32 | None)."""
    import torch
    if filt is None:
        return None
    k, tp, mp = filt
    for name, t, dt in (("top_k", k, torch.int32), ("top_p", tp, torch.float32), ("min_p", mp, torch.float32)):
        if t is not None and (t.dtype != dt or t.numel() != B or t.device != dev or not t.is_contiguous()):
            raise ValueError(f"{name}: expected contiguous {dt} [{B}] on {dev}")
    f = SvFilter(*[None if t is None else t.data_ptr() for t in (k, tp, mp)])
    return ctypes.byref(f), f


def verify_batch(target, draft, draft_tokens, row_offsets, temperature, tau, seed: int, *,
                 out_tokens=None, out_accept_len=None, workspace=None, row_diag=None, stats=None,
                 events=None, stream=None, tau_step=None, min_cum=None, lazy_max_rows=None,
                 target_filter=None, draft_filter=None):
    """Verify a batch of speculative windows on the GPU.

    target, draft : [R, V] bfloat16 or float32 (same dtype), row-major, on one GPU.
    draft_tokens  : [R] int32 (-1 = no proposal).
    row_offsets   : [B+1] int32.
    temperature   : [B] float32 (0 = greedy).
    tau           : [B] float32 gate thresholds.
    seed          : 64-bit Philox key.
    row_diag      : optional [R, 8] int32 tensor that receives sv_row_diag records.
    stats         : optional [STATS_FIELDS] int64 tensor that receives sv_batch_stats.
    events        : optional sequence of three raw hipEvent_t handles (ints).
    tau_step      : optional [R] float32 per-row gate thresholds (see expand_schedule).
    min_cum       : optional [B] float32 cumulative floors (0 = off).
    With tau_step or min_cum the call goes to sv_verify_batch_sched (no events).
    target_filter, draft_filter : optional (top_k, top_p, min_p) triples of [B] tensors
                    (int32, float32, float32; any may be None). With either, the call goes to
                    sv_verify_batch_filtered (no events).
    lazy_max_rows : with a bound on every request's rows, the call goes to sv_verify_batch_lazy,
                    which reads rows only up to each request's first rejection (plain outputs only).
    stream        : optional torch stream (default: the current stream).

    Returns (out_tokens [R] int32, out_accept_len [B] int32). Work is enqueued
    and not synchronised.
    """
    import torch
    lib = load_library()
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("inputs must live on a GPU")
    if draft.dtype != target.dtype or draft.shape != target.shape:
        raise ValueError("target and draft must have the same dtype and shape")
    if target.dim() != 2:
        raise ValueError("logits must be [R, V]")
    R, V = int(target.shape[0]), int(target.shape[1])
    B = int(row_offsets.numel()) - 1
    checks = [("draft_tokens", draft_tokens, torch.int32, R), ("row_offsets", row_offsets, torch.int32, B + 1),
              ("temperature", temperature, torch.float32, B), ("tau", tau, torch.float32, B)]
    if tau_step is not None:
        checks.append(("tau_step", tau_step, torch.float32, R))
    if min_cum is not None:
        checks.append(("min_cum", min_cum, torch.float32, B))
    for name, t, dt, n in checks:
        if t.dtype != dt or t.numel() != n or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous {dt} [{n}] on {dev}")
    if not (target.is_contiguous() and draft.is_contiguous()):
        raise ValueError("logits must be contiguous")
    code = dtype_code(target.dtype)
    shape = SvShape(B, R, V, code)
    if out_tokens is None:
        out_tokens = torch.empty(R, dtype=torch.int32, device=dev)
    if out_accept_len is None:
        out_accept_len = torch.empty(max(B, 0), dtype=torch.int32, device=dev)
    need = int(lib.sv_workspace_bytes(shape))
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None:
        workspace = _workspace(dev, need, stream)
    args = [_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(row_offsets), _ptr(temperature),
            _ptr(tau), c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), _ptr(out_tokens),
            _ptr(out_accept_len), shape, _ptr(workspace), c_size_t(workspace.numel()),
            c_void_p(stream.cuda_stream)]
    if row_diag is not None and (row_diag.dtype != torch.int32 or row_diag.numel() != 8 * R):
        raise ValueError("row_diag must be an int32 tensor with 8*R elements")
    if stats is not None and (stats.dtype != torch.int64 or stats.numel() != STATS_FIELDS):
        raise ValueError(f"stats must be an int64 tensor with {STATS_FIELDS} elements")
    if target_filter is not None or draft_filter is not None:
        if events is not None or lazy_max_rows is not None:
            raise ValueError("the filtered verify takes no events and has no lazy form")
        tf = _filter_struct(target_filter, B, dev)
        df = _filter_struct(draft_filter, B, dev)
        fargs = args[:6] + [_ptr(tau_step) if tau_step is not None else None,
                            _ptr(min_cum) if min_cum is not None else None,
                            tf[0] if tf else None, df[0] if df else None] + args[6:]
        _check(lib.sv_verify_batch_filtered(*fargs, _ptr(row_diag) if row_diag is not None else None,
                                            _ptr(stats) if stats is not None else None))
    elif lazy_max_rows is not None:
        if any(x is not None for x in (row_diag, stats, events, tau_step, min_cum)):
            raise ValueError("the lazy verify has plain outputs only")
        _check(lib.sv_verify_batch_lazy(*args, c_int(int(lazy_max_rows))))
    elif tau_step is not None or min_cum is not None:
        if events is not None:
            raise ValueError("events are not supported together with tau_step / min_cum")
        sargs = args[:6] + [_ptr(tau_step) if tau_step is not None else None,
                            _ptr(min_cum) if min_cum is not None else None] + args[6:]
        _check(lib.sv_verify_batch_sched(*sargs, _ptr(row_diag) if row_diag is not None else None,
                                         _ptr(stats) if stats is not None else None))
    elif row_diag is None and stats is None and events is None:
        _check(lib.sv_verify_batch(*args))
    else:
        ev = None
        if events is not None:
            ev = (c_void_p * 3)(*[c_void_p(int(e)) for e in events])
        _check(lib.sv_verify_batch_diag(*args, _ptr(row_diag) if row_diag is not None else None,
                                        _ptr(stats) if stats is not None else None, ev))
    return out_tokens, out_accept_len


STATIC_WORKSPACE_BYTES = 32 << 20  # SV_STATIC_WORKSPACE_BYTES


def verify_batch_static(target, draft, draft_tokens, row_offsets, temperature, tau, seed: int, out_tokens,
                        out_accept_len, *, stream=None):
    """sv_verify_batch_static: verify_batch with the library's own per-GPU workspace. The caller
    passes the outputs ([R] and [B] int32 tensors); the call allocates nothing."""
    import torch
    lib = load_library()
    R, V = int(target.shape[0]), int(target.shape[1])
    B = int(row_offsets.numel()) - 1
    if out_tokens.dtype != torch.int32 or out_tokens.numel() != R or out_accept_len.dtype != torch.int32 \
            or out_accept_len.numel() != B:
        raise ValueError("out_tokens must be int32 [R] and out_accept_len int32 [B]")
    if stream is None:
        stream = torch.cuda.current_stream(target.device)
    shape = SvShape(B, R, V, dtype_code(target.dtype))
    _check(lib.sv_verify_batch_static(_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(row_offsets),
                                      _ptr(temperature), _ptr(tau), c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
                                      _ptr(out_tokens), _ptr(out_accept_len), shape, c_void_p(stream.cuda_stream)))
    return out_tokens, out_accept_len


def verify_sampler_match(target, draft_tokens, row_offsets, temperature, seed: int, *, out_tokens=None,
                         out_accept_len=None, workspace=None, stream=None):
    """The sampler-match comparison rule on the GPU (sv_verify_batch_sampler_match).

    Arguments as for verify_batch, without draft logits or tau. Returns (out_tokens [R] int32,
    out_accept_len [B] int32), enqueued and not synchronised.
    """
    import torch
    lib = load_library()
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("inputs must live on a GPU")
    if target.dim() != 2 or not target.is_contiguous():
        raise ValueError("logits must be a contiguous [R, V] tensor")
    R, V = int(target.shape[0]), int(target.shape[1])
    B = int(row_offsets.numel()) - 1
    for name, t, dt, n in [("draft_tokens", draft_tokens, torch.int32, R), ("row_offsets", row_offsets, torch.int32, B + 1),
                           ("temperature", temperature, torch.float32, B)]:
        if t.dtype != dt or t.numel() != n or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous {dt} [{n}] on {dev}")
    shape = SvShape(B, R, V, dtype_code(target.dtype))
    if out_tokens is None:
        out_tokens = torch.empty(R, dtype=torch.int32, device=dev)
    if out_accept_len is None:
        out_accept_len = torch.empty(max(B, 0), dtype=torch.int32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None:
        workspace = _workspace(dev, int(lib.sv_workspace_bytes(shape)), stream)
    _check(lib.sv_verify_batch_sampler_match(_ptr(target), _ptr(draft_tokens), _ptr(row_offsets), _ptr(temperature),
                                             c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), _ptr(out_tokens),
                                             _ptr(out_accept_len), shape, _ptr(workspace),
                                             c_size_t(workspace.numel()), c_void_p(stream.cuda_stream)))
    return out_tokens, out_accept_len


def filter_thresholds(target, draft, row_offsets, temperature, *, target_filter=None, draft_filter=None,
                      out_theta=None, workspace=None, stream=None):
    """Each row's keep-thresholds under the filter chain (sv_filter_thresholds).

    Filters as for verify_batch. Returns out_theta [R, 2] float32: column 0 the target's,
    column 1 the draft's; token x is kept iff its logit >= theta. Enqueued, not synchronised.
    """
    import torch
    lib = load_library()
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("inputs must live on a GPU")
    if draft.dtype != target.dtype or draft.shape != target.shape or target.dim() != 2:
        raise ValueError("target and draft must be [R, V] tensors of one dtype")
    if not (target.is_contiguous() and draft.is_contiguous()):
        raise ValueError("logits must be contiguous")
    R, V = int(target.shape[0]), int(target.shape[1])
    B = int(row_offsets.numel()) - 1
    for name, t, dt, n in (("row_offsets", row_offsets, torch.int32, B + 1),
                           ("temperature", temperature, torch.float32, B)):
        if t.dtype != dt or t.numel() != n or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous {dt} [{n}] on {dev}")
    shape = SvShape(B, R, V, dtype_code(target.dtype))
    if out_theta is None:
        out_theta = torch.empty((R, 2), dtype=torch.float32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None:
        workspace = _workspace(dev, int(lib.sv_workspace_bytes(shape)), stream)
    tf = _filter_struct(target_filter, B, dev)
    df = _filter_struct(draft_filter, B, dev)
    _check(lib.sv_filter_thresholds(_ptr(target), _ptr(draft), _ptr(row_offsets), _ptr(temperature),
                                    tf[0] if tf else None, df[0] if df else None, _ptr(out_theta), shape,
                                    _ptr(workspace), c_size_t(workspace.numel()), c_void_p(stream.cuda_stream)))
    return out_theta


def row_acceptance(target, draft, draft_tokens, row_offsets, temperature, tau, *, tau_step=None, min_cum=None,
                   out_sum_min=None, out_sum_pq=None, workspace=None, stream=None, target_filter=None,
                   draft_filter=None):
    """Per-row sum min(p, mu) and sum p q of a verify batch (sv_row_acceptance).

    Arguments as for verify_batch; with target_filter or draft_filter the call goes to
    sv_row_acceptance_filtered. Returns (sum_min [R] float32, sum_pq [R] float32), NaN on rows
    that are not proposal rows. Work is enqueued and not synchronised.
    """
    import torch
    lib = load_library()
    dev = target.device
    if dev.type != "cuda":
        raise ValueError("inputs must live on a GPU")
    if draft.dtype != target.dtype or draft.shape != target.shape or target.dim() != 2:
        raise ValueError("target and draft must be [R, V] tensors of one dtype")
    if not (target.is_contiguous() and draft.is_contiguous()):
        raise ValueError("logits must be contiguous")
    R, V = int(target.shape[0]), int(target.shape[1])
    B = int(row_offsets.numel()) - 1
    checks = [("draft_tokens", draft_tokens, torch.int32, R), ("row_offsets", row_offsets, torch.int32, B + 1),
              ("temperature", temperature, torch.float32, B), ("tau", tau, torch.float32, B)]
    if tau_step is not None:
        checks.append(("tau_step", tau_step, torch.float32, R))
    if min_cum is not None:
        checks.append(("min_cum", min_cum, torch.float32, B))
    for name, t, dt, n in checks:
        if t.dtype != dt or t.numel() != n or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous {dt} [{n}] on {dev}")
    shape = SvShape(B, R, V, dtype_code(target.dtype))
    if out_sum_min is None:
        out_sum_min = torch.empty(R, dtype=torch.float32, device=dev)
    if out_sum_pq is None:
        out_sum_pq = torch.empty(R, dtype=torch.float32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None:
        workspace = _workspace(dev, int(lib.sv_workspace_bytes(shape)), stream)
    head = [_ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(row_offsets), _ptr(temperature), _ptr(tau),
            _ptr(tau_step) if tau_step is not None else None, _ptr(min_cum) if min_cum is not None else None]
    tail = [_ptr(out_sum_min), _ptr(out_sum_pq), shape, _ptr(workspace), c_size_t(workspace.numel()),
            c_void_p(stream.cuda_stream)]
    if target_filter is not None or draft_filter is not None:
        tf = _filter_struct(target_filter, B, dev)
        df = _filter_struct(draft_filter, B, dev)
        _check(lib.sv_row_acceptance_filtered(*head, tf[0] if tf else None, df[0] if df else None, *tail))
    else:
        _check(lib.sv_row_acceptance(*head, *tail))
    return out_sum_min, out_sum_pq


def expand_schedule(schedule, row_offsets):
    """Per-row gate thresholds from a step schedule: row j of every request gets
    schedule[min(j, len(schedule) - 1)], the last threshold repeating for later steps
    (regolith audit "rank-1 moce and step-aware speculative retention", section schedule
    behavior). ``row_offsets`` is a host sequence; returns a host float32 numpy array [R]."""
    import numpy as np
    sched = [float(x) for x in schedule]
    if not 1 <= len(sched) <= 8:
        raise ValueError("a schedule has one to eight thresholds")
    ro = [int(x) for x in row_offsets]
    out = np.empty(ro[-1], dtype=np.float32)
    for b in range(len(ro) - 1):
        for j in range(ro[b + 1] - ro[b]):
            out[ro[b] + j] = sched[min(j, len(sched) - 1)]
    return out


def split_row_diag(row_diag):
    """View an [R, 8] int32 sv_row_diag tensor as (p_D, q_D, mu_D, u, resid_mass, verdict)."""
    import torch
    d = row_diag.view(-1, 8)
    f = d[:, :5].contiguous().view(torch.float32)
    return f[:, 0], f[:, 1], f[:, 2], f[:, 3], f[:, 4], d[:, 5]


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime (for sv_verify_batch_diag's timing hooks)."""

    def __init__(self, n: int = 3):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [POINTER(c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [POINTER(ctypes.c_float), c_void_p, c_void_p]
        self._hip.hipEventSynchronize.argtypes = [c_void_p]
        self._hip.hipEventDestroy.argtypes = [c_void_p]
        self.handles = []
        for _ in range(n):
            h = c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles.append(h.value)

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        self._hip.hipEventSynchronize(c_void_p(self.handles[j]))
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), c_void_p(self.handles[i]),
                                         c_void_p(self.handles[j])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for h in self.handles:
            self._hip.hipEventDestroy(c_void_p(h))
        self.handles = []
