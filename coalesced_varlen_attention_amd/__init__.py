"""Coalesced varlen attention for MI355X: thin Python binding of ``libzl.so``.

The library runs one GPU's share of a mixed image-video DiT batch (the "Coalesced
Attention Engine" of the Zellige page, §IV-D): whole sequences, Ulysses head subsets
and ring KV-split parts in one persistent launch each for forward and backward, plus
the exact LSE merge of ring parts. This module only marshals arguments: every step of
the computation runs in the HIP kernels behind the C ABI of ``include/zl.h``. PyTorch
provides device memory and the current stream.

If ``libzl.so`` is missing, the first call raises: there is no fallback.

Example: two sequences (1024 tokens at 24 heads, and a 4096-token one at 24 heads whose keys
are split into two ring parts), d_head 128::

    import torch, coalesced_varlen_attention_amd as zl
    segs = [(0, 0, 24, 0, 1024, 0, 1024, -1),                 # whole sequence, final rows
            (1, 0, 24, 0, 4096, 0, 2048, 0),                  # ring part 0
            (1, 0, 24, 0, 4096, 2048, 4096, 1)]               # ring part 1
    plan = zl.Plan([1024, 4096], [1024, 4096], [24, 24], segs, 128)
    rows = plan.info["q_rows"]                                 # (1024 + 4096) * 24
    q, k, v, do = (torch.randn(rows, 128, device="cuda").bfloat16() for _ in range(4))
    o, lse, o_part, lse_part = zl.attn_fwd(plan, q, k, v)
    zl.merge_groups(plan, o_part, lse_part, o, lse)            # exact merge of the ring parts
    dq, dk, dv = zl.attn_bwd(plan, q, k, v, o, lse, do)
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

__all__ = ["Plan", "ZlError", "attn_fwd", "attn_fwd_accumulate", "attn_bwd", "attn_bwd_noalloc", "lse_merge",
           "merge_groups", "lib", "lib_path", "SEGMENT_FIELDS", "NOALLOC_SCRATCH_BYTES"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libzl.so")

ZL_PLAN_HOST_ONLY = 1
ZL_PLAN_NO_SPLIT = 2
ZL_PLAN_QKV_PACKED = 4
ZL_PLAN_COUNT_VISITS = 8
ZL_PLAN_DEFERRED_UPLOAD = 16
ZL_PLAN_NARROW_ITEMS = 32
ZL_PLAN_WIDE_ITEMS = 64
BWD_PRE, BWD_DKDV, BWD_DQ, BWD_ALL = 1, 2, 4, 7
NOALLOC_SCRATCH_BYTES = 64 << 20  # ZL_NOALLOC_SCRATCH_BYTES
SEGMENT_FIELDS = ("seq", "head_begin", "head_end", "q_begin", "q_end", "kv_begin", "kv_end", "part")


class ZlError(RuntimeError):
    """A libzl call returned a non-zero status; the message is zl_last_error()."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libzl status {status}: {message}")
        self.status = status


class _Segment(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in SEGMENT_FIELDS]


class _PlanInfo(ctypes.Structure):
    _fields_ = [("ws_fwd", ctypes.c_size_t), ("ws_bwd", ctypes.c_size_t), ("q_rows", ctypes.c_int64),
                ("kv_rows", ctypes.c_int64), ("part_rows", ctypes.c_int64), ("n_groups", ctypes.c_int32),
                ("n_parts_max", ctypes.c_int32), ("fwd_tiles", ctypes.c_int64), ("bwd_tiles", ctypes.c_int64),
                ("fwd_flops", ctypes.c_double), ("bwd_flops", ctypes.c_double), ("d_head", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("dq_tiles", ctypes.c_int64), ("split_tiles", ctypes.c_int32),
                ("split_pieces", ctypes.c_int32), ("qkv_rows", ctypes.c_int64),
                ("dq_split_tiles", ctypes.c_int32), ("dq_split_pieces", ctypes.c_int32),
                ("kv_split_tiles", ctypes.c_int32), ("kv_split_pieces", ctypes.c_int32),
                ("visits_fwd", ctypes.c_int64), ("visits_dkdv", ctypes.c_int64), ("visits_dq", ctypes.c_int64),
                ("dev_bytes", ctypes.c_size_t), ("fwd_rows", ctypes.c_int32),
                ("dq_rows", ctypes.c_int32)]


class _GroupInfo(ctypes.Structure):
    _fields_ = [("n_parts", ctypes.c_int32), ("seq", ctypes.c_int32), ("n_rows", ctypes.c_int64),
                ("o_row", ctypes.c_int64), ("part_row", ctypes.c_int64), ("head_begin", ctypes.c_int32),
                ("head_end", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("q_begin", ctypes.c_int32),
                ("q_end", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m coalesced_varlen_attention_amd.build` "
                          "(there is no fallback path)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, U32, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float
    sig = {
        "zl_plan_build": (I32, [I32, P, P, P, I32, P, I32, F32, U32, ctypes.POINTER(P)]),
        "zl_plan_info": (I32, [P, ctypes.POINTER(_PlanInfo)]),
        "zl_plan_group": (I32, [P, I32, ctypes.POINTER(_GroupInfo)]),
        "zl_plan_tiles": (I32, [P, I32, P, I64, ctypes.POINTER(I64)]),
        "zl_plan_queues": (I32, [P, I32, P, I32, ctypes.POINTER(I32)]),
        "zl_plan_destroy": (None, [P]),
        "zl_plan_upload": (I32, [P, P, ctypes.c_size_t, P]),
        "zl_attn_fwd": (I32, [P, P, P, P, P, P, P, P, P, P]),
        "zl_attn_fwd_accumulate": (I32, [P, P, P, P, P, P, P, P]),
        "zl_lse_merge": (I32, [I32, I64, I32, P, P, P, P, P]),
        "zl_plan_merge": (I32, [P, P, P, P, P, P]),
        "zl_attn_bwd": (I32, [P, P, P, P, P, P, P, P, P, P, P, P]),
        "zl_attn_bwd_stages": (I32, [P, P, P, P, P, P, P, P, P, P, P, U32, P]),
        "zl_attn_bwd_noalloc": (I32, [P, P, P, P, P, P, P, P, P, P, P]),
        "zl_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded libzl.so (loaded on first use; raises if it is missing or stale)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def lib_path() -> str:
    return _LIB_PATH


def _check(status: int) -> None:
    if status != 0:
        raise ZlError(status, lib().zl_last_error().decode(errors="replace"))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class Plan:
    """A validated, lowered segment list (``zl_plan_build``).

    ``seq_q``/``seq_kv``: tokens per sequence; ``heads``: stored heads per sequence;
    ``segments``: tuples ``(seq, head_begin, head_end, q_begin, q_end, kv_begin, kv_end, part)``.
    ``count_visits``: the scheduler check of ``ZL_PLAN_COUNT_VISITS`` (read with ``visits``).
    ``deferred``: ``ZL_PLAN_DEFERRED_UPLOAD``; the plan runs after ``upload()``.
    ``item_rows``: 128 or 256 fixes the forward and dQ item sizes (``ZL_PLAN_NARROW_ITEMS`` /
    ``ZL_PLAN_WIDE_ITEMS``); None lets the plan choose (``info["fwd_rows"]``, ``info["dq_rows"]``).
    """

    def __init__(self, seq_q: Sequence[int], seq_kv: Sequence[int], heads: Sequence[int], segments, d: int,
                 scale: Optional[float] = None, host_only: bool = False, split: bool = True,
                 qkv_packed: bool = False, count_visits: bool = False, deferred: bool = False,
                 item_rows: Optional[int] = None):
        n = len(seq_q)
        if len(seq_kv) != n or len(heads) != n:
            raise ValueError("seq_q, seq_kv and heads must have the same length")
        cu_q = (ctypes.c_int64 * (n + 1))()
        cu_kv = (ctypes.c_int64 * (n + 1))()
        for i in range(n):
            cu_q[i + 1] = cu_q[i] + int(seq_q[i])
            cu_kv[i + 1] = cu_kv[i] + int(seq_kv[i])
        hs = (ctypes.c_int32 * n)(*[int(h) for h in heads])
        segs = (_Segment * len(segments))()
        for i, s in enumerate(segments):
            for name, val in zip(SEGMENT_FIELDS, s):
                setattr(segs[i], name, int(val))
        self._h = ctypes.c_void_p()
        flags = ((ZL_PLAN_HOST_ONLY if host_only else 0) | (0 if split else ZL_PLAN_NO_SPLIT) |
                 (ZL_PLAN_QKV_PACKED if qkv_packed else 0) | (ZL_PLAN_COUNT_VISITS if count_visits else 0) |
                 (ZL_PLAN_DEFERRED_UPLOAD if deferred else 0))
        if item_rows is not None:
            if item_rows not in (128, 256):
                raise ValueError("item_rows must be 128, 256 or None (the plan's choice)")
            flags |= ZL_PLAN_WIDE_ITEMS if item_rows == 256 else ZL_PLAN_NARROW_ITEMS
        self._tables = None
        _check(lib().zl_plan_build(n, ctypes.cast(cu_q, ctypes.c_void_p), ctypes.cast(cu_kv, ctypes.c_void_p),
                                  ctypes.cast(hs, ctypes.c_void_p), len(segments), ctypes.cast(segs, ctypes.c_void_p),
                                  int(d), float(scale) if scale else 0.0, flags, ctypes.byref(self._h)))
        info = _PlanInfo()
        _check(lib().zl_plan_info(self._h, ctypes.byref(info)))
        self.info = {name: getattr(info, name) for name, _ in _PlanInfo._fields_}
        self.d = int(d)
        self.groups: List[dict] = []
        for g in range(info.n_groups):
            gi = _GroupInfo()
            _check(lib().zl_plan_group(self._h, g, ctypes.byref(gi)))
            self.groups.append({name: getattr(gi, name) for name, _ in _GroupInfo._fields_})

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    def tiles(self, which: int) -> List[Tuple[int, ...]]:
        """Work queue items (segment, head, first row, rows): 0 forward, 1 backward dK/dV, 2 backward dQ;
        3 forward with (key begin, key end, split slot, piece | pieces << 16) appended; 4 dQ with
        (first block, end block of the key-block chain, split slot, piece | pieces << 16) appended;
        5 dK/dV in the same form over the segment's query blocks."""
        w = 8 if which >= 3 else 4
        cnt = ctypes.c_int64()
        _check(lib().zl_plan_tiles(self._h, which, None, 0, ctypes.byref(cnt)))
        buf = (ctypes.c_int32 * (w * cnt.value))()
        _check(lib().zl_plan_tiles(self._h, which, ctypes.cast(buf, ctypes.c_void_p), cnt.value, ctypes.byref(cnt)))
        return [tuple(buf[w * i:w * i + w]) for i in range(cnt.value)]

    def queues(self, which: int) -> List[int]:
        """Queue boundaries of a work list: items bounds[k]:bounds[k+1] of tiles(which) form queue k."""
        n = ctypes.c_int32()
        buf = (ctypes.c_int32 * 64)()
        _check(lib().zl_plan_queues(self._h, which, ctypes.cast(buf, ctypes.c_void_p), 64, ctypes.byref(n)))
        return list(buf[: n.value + 1])

    def upload(self, buffer=None, stream=None):
        """Copy a deferred plan's device tables into ``buffer`` (a device uint8 tensor of at least
        ``info["dev_bytes"]`` bytes, allocated here if None) on ``stream`` (default: the current
        stream), without waiting for the device (``zl_plan_upload``). The plan keeps a reference to
        the buffer. Returns the buffer."""
        import torch
        if buffer is None:
            buffer = torch.empty(self.info["dev_bytes"], dtype=torch.uint8, device="cuda")
        _check_workspace(buffer, self.info["dev_bytes"], _gpu_device(buffer, "buffer"))
        _check(lib().zl_plan_upload(self._h, buffer.data_ptr(), buffer.numel(), _stream_handle(stream)))
        self._tables = buffer
        return buffer

    def visits(self, ws_fwd=None, ws_bwd=None) -> dict:
        """Per-item visit counters of a ``count_visits`` plan, read from the workspaces of the last
        forward (``ws_fwd``) and backward (``ws_bwd``) launches: {"fwd" | "dkdv" | "dq": int32 tensor}."""
        import torch
        info = self.info
        if info["visits_fwd"] < 0:
            raise ValueError("the plan was not built with count_visits=True")
        out = {}
        for key, ws, off, n in (("fwd", ws_fwd, info["visits_fwd"], info["fwd_tiles"]),
                                ("dkdv", ws_bwd, info["visits_dkdv"], info["bwd_tiles"]),
                                ("dq", ws_bwd, info["visits_dq"], info["dq_tiles"])):
            if ws is not None:
                out[key] = ws[off:off + 4 * n].view(torch.int32).cpu()
        return out

    def close(self) -> None:
        if getattr(self, "_h", None) and self._h.value:
            lib().zl_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _input_rows(info):
    """Rows of q and of k / v: the packed buffer's for a QKV-packed plan."""
    if info["qkv_rows"]:
        return info["qkv_rows"], info["qkv_rows"]
    return info["q_rows"], info["kv_rows"]


def _gpu_device(t, name):
    """The device of ``t``, which must be a GPU tensor: the kernels dereference every pointer
    on the device, so a host pointer would fault there instead of failing here."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{name} is on {t.device}: the library needs device tensors")
    return t.device


def _check_tensor(t, name, dtype, rows, d, device):
    if _gpu_device(t, name) != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != rows * d:
        raise ValueError(f"{name} has {t.numel()} elements, expected {rows} x {d}")


def _check_workspace(ws, need, device):
    """A byte buffer on ``device`` of at least ``need`` bytes (its dtype fixes the byte count)."""
    import torch
    if _gpu_device(ws, "workspace") != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise TypeError("workspace must be a contiguous torch.uint8 tensor")
    if ws.numel() < need:
        raise ValueError(f"workspace has {ws.numel()} bytes, the plan needs {need}")


def attn_fwd(plan: Plan, q, k, v, o=None, lse=None, o_part=None, lse_part=None, workspace=None, stream=None):
    """Forward of every segment of ``plan`` in one launch (``zl_attn_fwd``).

    Returns ``(o, lse, o_part, lse_part)``; buffers not given are allocated with
    ``torch.empty`` on ``q``'s device (rows no segment covers are left as allocated).
    Ring groups still need ``merge_groups`` (or ``lse_merge``) to produce their final rows.
    """
    import torch
    info, d, dev = plan.info, plan.d, _gpu_device(q, "q")
    rq, rkv = _input_rows(info)
    _check_tensor(q, "q", torch.bfloat16, rq, d, dev)
    _check_tensor(k, "k", torch.bfloat16, rkv, d, dev)
    _check_tensor(v, "v", torch.bfloat16, rkv, d, dev)
    if o is None:
        o = torch.empty(info["q_rows"], d, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(info["q_rows"], dtype=torch.float32, device=dev)
    if info["n_groups"] > 0:
        if o_part is None:
            o_part = torch.empty(info["part_rows"], d, dtype=torch.float32, device=dev)
        if lse_part is None:
            lse_part = torch.empty(info["part_rows"], dtype=torch.float32, device=dev)
        _check_tensor(o_part, "o_part", torch.float32, info["part_rows"], d, dev)
        _check_tensor(lse_part, "lse_part", torch.float32, info["part_rows"], 1, dev)
    _check_tensor(o, "o", torch.float32, info["q_rows"], d, dev)
    _check_tensor(lse, "lse", torch.float32, info["q_rows"], 1, dev)
    if workspace is None:
        workspace = torch.empty(info["ws_fwd"], dtype=torch.uint8, device=dev)
    _check_workspace(workspace, info["ws_fwd"], dev)
    _check(lib().zl_attn_fwd(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            _ptr(o_part), _ptr(lse_part), workspace.data_ptr(), _stream_handle(stream)))
    return o, lse, o_part, lse_part


def attn_fwd_accumulate(plan: Plan, q, k, v, o, lse, workspace=None, stream=None):
    """Forward with a running merge (``zl_attn_fwd_accumulate``): every ring part of ``plan``
    folds its result into ``o``/``lse`` at its group's rows (set ``lse`` to -inf there before
    a group's first block); ``part == -1`` segments are written as in ``attn_fwd``. The plan
    may hold at most one part per group. Returns ``(o, lse)``."""
    import torch
    info, d, dev = plan.info, plan.d, _gpu_device(q, "q")
    rq, rkv = _input_rows(info)
    _check_tensor(q, "q", torch.bfloat16, rq, d, dev)
    _check_tensor(k, "k", torch.bfloat16, rkv, d, dev)
    _check_tensor(v, "v", torch.bfloat16, rkv, d, dev)
    _check_tensor(o, "o", torch.float32, info["q_rows"], d, dev)
    _check_tensor(lse, "lse", torch.float32, info["q_rows"], 1, dev)
    if workspace is None:
        workspace = torch.empty(info["ws_fwd"], dtype=torch.uint8, device=dev)
    _check_workspace(workspace, info["ws_fwd"], dev)
    _check(lib().zl_attn_fwd_accumulate(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        lse.data_ptr(), workspace.data_ptr(), _stream_handle(stream)))
    return o, lse


def lse_merge(n_parts: int, n_rows: int, d: int, o_part, lse_part, o, lse, stream=None) -> None:
    """Exact merge of ring partials (``zl_lse_merge``) on raw tensors or views.

    ``o_part``: ``n_parts*n_rows*d`` floats, ``lse_part``: ``n_parts*n_rows``; results to
    ``o`` (``n_rows*d``) and ``lse`` (``n_rows``). Views must be contiguous.
    """
    import torch
    dev = _gpu_device(o_part, "o_part")
    for t, name, n in ((o_part, "o_part", n_parts * n_rows * d), (lse_part, "lse_part", n_parts * n_rows),
                       (o, "o", n_rows * d), (lse, "lse", n_rows)):
        if _gpu_device(t, name) != dev:
            raise ValueError(f"lse_merge: {name} is on {t.device}, expected {dev}")
        if t.dtype != torch.float32:
            raise TypeError(f"lse_merge: {name} must be torch.float32, got {t.dtype}")
        if not t.is_contiguous() or t.numel() < n:
            raise ValueError(f"lse_merge: {name} has {t.numel()} elements (needs {n}) or is not contiguous")
    _check(lib().zl_lse_merge(int(n_parts), int(n_rows), int(d), o_part.data_ptr(), lse_part.data_ptr(),
                             o.data_ptr(), lse.data_ptr(), _stream_handle(stream)))


def merge_groups(plan: Plan, o_part, lse_part, o, lse, stream=None) -> None:
    """Merge every ring group of ``plan`` into its rows of ``o`` and ``lse`` (``zl_plan_merge``,
    one launch; head-subset groups land at their strided rows)."""
    import torch
    info, d = plan.info, plan.d
    if info["n_groups"] == 0:
        return
    dev = _gpu_device(o, "o")
    _check_tensor(o_part, "o_part", torch.float32, info["part_rows"], d, dev)
    _check_tensor(lse_part, "lse_part", torch.float32, info["part_rows"], 1, dev)
    _check_tensor(o, "o", torch.float32, info["q_rows"], d, dev)
    _check_tensor(lse, "lse", torch.float32, info["q_rows"], 1, dev)
    _check(lib().zl_plan_merge(plan.handle, o_part.data_ptr(), lse_part.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               _stream_handle(stream)))


def attn_bwd(plan: Plan, q, k, v, o, lse, do, dq=None, dk=None, dv=None, workspace=None, stream=None,
             stages: int = BWD_ALL):
    """Backward of every segment of ``plan`` (``zl_attn_bwd_stages``): returns ``(dq, dk, dv)``.

    ``stages`` selects launches (BWD_PRE, BWD_DKDV, BWD_DQ); DKDV and DQ need a PRE before
    each of them on the same workspace."""
    import torch
    info, d, dev = plan.info, plan.d, _gpu_device(q, "q")
    rq, rkv = _input_rows(info)
    _check_tensor(q, "q", torch.bfloat16, rq, d, dev)
    _check_tensor(k, "k", torch.bfloat16, rkv, d, dev)
    _check_tensor(v, "v", torch.bfloat16, rkv, d, dev)
    _check_tensor(do, "do", torch.bfloat16, info["q_rows"], d, dev)
    _check_tensor(o, "o", torch.float32, info["q_rows"], d, dev)
    _check_tensor(lse, "lse", torch.float32, info["q_rows"], 1, dev)
    if info["qkv_rows"]:  # one packed gradient buffer, passed as dq, dk and dv
        if dq is None:
            dq = torch.empty(info["qkv_rows"], d, dtype=torch.float32, device=dev)
        dk = dk if dk is not None else dq
        dv = dv if dv is not None else dq
    else:
        if dq is None:
            dq = torch.empty(info["q_rows"], d, dtype=torch.float32, device=dev)
        if dk is None:
            dk = torch.empty(info["kv_rows"], d, dtype=torch.float32, device=dev)
        if dv is None:
            dv = torch.empty(info["kv_rows"], d, dtype=torch.float32, device=dev)
    _check_tensor(dq, "dq", torch.float32, rq, d, dev)
    _check_tensor(dk, "dk", torch.float32, rkv, d, dev)
    _check_tensor(dv, "dv", torch.float32, rkv, d, dev)
    if workspace is None:
        workspace = torch.empty(info["ws_bwd"], dtype=torch.uint8, device=dev)
    _check_workspace(workspace, info["ws_bwd"], dev)
    _check(lib().zl_attn_bwd_stages(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                   workspace.data_ptr(), int(stages), _stream_handle(stream)))
    return dq, dk, dv


def attn_bwd_noalloc(plan: Plan, q, k, v, o, lse, do, dq, dk, dv, stream=None):
    """The backward with the library's fixed device scratch (``zl_attn_bwd_noalloc``): for
    callers that cannot allocate. The caller passes every output; calls on one device must
    not overlap. Returns ``(dq, dk, dv)``."""
    import torch
    info, d, dev = plan.info, plan.d, _gpu_device(q, "q")
    rq, rkv = _input_rows(info)
    _check_tensor(q, "q", torch.bfloat16, rq, d, dev)
    _check_tensor(k, "k", torch.bfloat16, rkv, d, dev)
    _check_tensor(v, "v", torch.bfloat16, rkv, d, dev)
    _check_tensor(do, "do", torch.bfloat16, info["q_rows"], d, dev)
    _check_tensor(o, "o", torch.float32, info["q_rows"], d, dev)
    _check_tensor(lse, "lse", torch.float32, info["q_rows"], 1, dev)
    _check_tensor(dq, "dq", torch.float32, rq, d, dev)
    _check_tensor(dk, "dk", torch.float32, rkv, d, dev)
    _check_tensor(dv, "dv", torch.float32, rkv, d, dev)
    _check(lib().zl_attn_bwd_noalloc(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                     _stream_handle(stream)))
    return dq, dk, dv
