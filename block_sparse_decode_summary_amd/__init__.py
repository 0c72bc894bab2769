"""Python binding of libfx: block-sparse decode attention for MI355X (gfx950).

The functions here carry the C names of include/fx.h and only marshal arguments:
torch tensors (device memory) become raw pointers, the current torch stream
becomes the hipStream_t.  Every step of the hot path runs in the HIP kernels of
libfx.so; there is no other code path.  If the library is not built, or a tensor
is not on the GPU, a call raises instead of computing anything.

Build the library in-tree with ``python -m block_sparse_decode_summary_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

__all__ = [
    "FX_F32", "FX_BF16", "FX_RETRIEVAL", "FX_STREAMING", "FX_NOSA",
    "FX_POOL_KEY", "FX_POOL_SCORE_SUM", "FX_POOL_SCORE_MAX", "fx_unit_summary_offset",
    "FX_ERR_SEQ_LEN", "FX_ERR_SEL_INDEX", "FX_ERR_SEL_COUNT", "FX_ERR_NONFINITE", "FX_ERR_SLOT_MAP",
    "fx_compact_update", "fx_unit_work_offset", "fx_unit_max_selected", "WorkingSet", "allocate_working_set",
    "FxError", "Plan", "library_path", "load_library",
    "fx_plan_create", "fx_plan_destroy", "fx_build_summaries", "fx_select",
    "fx_sparse_decode", "fx_sparse_decode_ed", "fx_sparse_decode_noalloc", "fx_noalloc_scratch_bytes",
    "fx_selection_delta", "fx_select_delta", "fx_read_error", "fx_status_string",
    "fx_stream_read",
    "StepBuffers", "allocate_step_buffers",
]

FX_OK, FX_E_INVALID, FX_E_UNSUPPORTED, FX_E_WORKSPACE, FX_E_HIP = 0, 1, 2, 3, 4
FX_F32, FX_BF16 = 0, 1
FX_RETRIEVAL, FX_STREAMING, FX_NOSA = 0, 1, 2
FX_POOL_KEY, FX_POOL_SCORE_SUM, FX_POOL_SCORE_MAX = 0, 1, 2
FX_ERR_SEQ_LEN, FX_ERR_SEL_INDEX, FX_ERR_SEL_COUNT, FX_ERR_NONFINITE = 1, 2, 4, 8
FX_ERR_SLOT_MAP = 16

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libfx.so")


class FxError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg}")
        self.status = status


class _PlanDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("t_cap", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("split_tokens", ctypes.c_int32), ("pooling", ctypes.c_int32)]


class _HeadPolicy(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("block", ctypes.c_int32), ("sub_block", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("budget", ctypes.c_float), ("k_evict", ctypes.c_int32),
                ("sink_tokens", ctypes.c_int32), ("local_tokens", ctypes.c_int32),
                ("force_sink", ctypes.c_int32), ("force_last", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32


def load_library(path: Optional[str] = None):
    """Load libfx.so (once; `path` overrides the in-tree build).  Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m block_sparse_decode_summary_amd.build`")
    lib = ctypes.CDLL(path)
    sig = {
        "fx_plan_create": (_I32, [ctypes.POINTER(_PlanDesc), ctypes.POINTER(_HeadPolicy), ctypes.POINTER(_P)]),
        "fx_plan_destroy": (_I32, [_P]),
        "fx_summary_bytes": (ctypes.c_size_t, [_P]),
        "fx_logits_bytes": (ctypes.c_size_t, [_P]),
        "fx_evict_mask_bytes": (ctypes.c_size_t, [_P]),
        "fx_workspace_bytes": (ctypes.c_size_t, [_P]),
        "fx_max_selected": (_I32, [_P]),
        "fx_unit_block_offset": (ctypes.c_int64, [_P, _I32]),
        "fx_unit_summary_offset": (ctypes.c_int64, [_P, _I32]),
        "fx_work_bytes": (ctypes.c_size_t, [_P]),
        "fx_unit_work_offset": (ctypes.c_int64, [_P, _I32]),
        "fx_unit_max_selected": (_I32, [_P, _I32]),
        "fx_compact_update": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                     _P]),
        "fx_split_tokens": (_I32, [_P]),
        "fx_status_string": (ctypes.c_char_p, [_I32]),
        "fx_read_error": (_I32, [_P, ctypes.POINTER(ctypes.c_uint32)]),
        "fx_build_summaries": (_I32, [_P, _P, _P, _I32, _I32, _P, _P]),
        "fx_select": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
        "fx_sparse_decode": (_I32, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P,
                                    ctypes.c_size_t, _P]),
        "fx_sparse_decode_ed": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P,
                                       _P, ctypes.c_size_t, _P]),
        "fx_sparse_decode_noalloc": (_I32, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P,
                                            _P]),
        "fx_noalloc_scratch_bytes": (ctypes.c_size_t, [_P]),
        "fx_selection_delta": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
        "fx_select_delta": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   ctypes.c_size_t, _P]),
        "fx_stream_read_sink_words": (ctypes.c_size_t, [ctypes.c_size_t]),
        "fx_stream_read": (_I32, [_P, ctypes.c_size_t, _P, _P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def fx_status_string(status: int) -> str:
    return load_library().fx_status_string(status).decode()


def _check(fn: str, status: int):
    if status != FX_OK:
        raise FxError(fn, status, fx_status_string(status))


def _stream(stream) -> Optional[int]:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, min_numel: int = 0,
         optional: bool = False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {min_numel}")
    return t.data_ptr()


@dataclass
class Plan:
    """An fx_plan_t and the sizes derived from it."""
    handle: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    t_cap: int
    dtype: int
    summary_bytes: int
    logits_bytes: int
    evict_mask_bytes: int
    workspace_bytes: int
    max_selected: int
    split_tokens: int
    pooling: int = 0
    work_bytes: int = 0

    @property
    def units(self) -> int:
        return self.batch * self.num_kv_heads

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == FX_F32 else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == FX_F32 else 2

    def unit_block_offset(self, unit: int) -> int:
        return int(load_library().fx_unit_block_offset(self.handle, unit))

    def __del__(self):
        if getattr(self, "handle", None):
            try:
                load_library().fx_plan_destroy(self.handle)
            except Exception:
                pass
            self.handle = None


def fx_plan_create(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, t_cap: int,
                   dtype: int, policies: Sequence, split_tokens: int = 0,
                   pooling: int = 0) -> Plan:
    """policies: one object per unit (u = b*Hkv + h) with the fields of fx_head_policy;
    pooling: FX_POOL_KEY, FX_POOL_SCORE_SUM or FX_POOL_SCORE_MAX."""
    lib = load_library()
    desc = _PlanDesc(batch, num_q_heads, num_kv_heads, head_dim, t_cap, dtype, split_tokens,
                     pooling)
    arr = (_HeadPolicy * len(policies))()
    for i, p in enumerate(policies):
        arr[i] = _HeadPolicy(int(p.mode), int(p.block), int(p.sub_block), int(p.top_k),
                             float(p.budget), int(p.k_evict), int(p.sink_tokens),
                             int(p.local_tokens), int(p.force_sink), int(p.force_last))
    if len(policies) != batch * num_kv_heads:
        raise ValueError("need one policy per (sequence, kv head)")
    h = _P()
    _check("fx_plan_create", lib.fx_plan_create(ctypes.byref(desc), arr, ctypes.byref(h)))
    return Plan(handle=h.value, batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                head_dim=head_dim, t_cap=t_cap, dtype=dtype,
                summary_bytes=lib.fx_summary_bytes(h), logits_bytes=lib.fx_logits_bytes(h),
                evict_mask_bytes=lib.fx_evict_mask_bytes(h),
                workspace_bytes=lib.fx_workspace_bytes(h), max_selected=lib.fx_max_selected(h),
                split_tokens=lib.fx_split_tokens(h), pooling=pooling,
                work_bytes=lib.fx_work_bytes(h))


def fx_plan_destroy(plan: Plan) -> None:
    if plan.handle:
        _check("fx_plan_destroy", load_library().fx_plan_destroy(plan.handle))
        plan.handle = None


def fx_unit_summary_offset(plan: Plan, unit: int) -> int:
    """First summary row of a unit (-1 if out of range)."""
    return int(load_library().fx_unit_summary_offset(plan.handle, int(unit)))


def fx_read_error(plan: Plan) -> int:
    w = ctypes.c_uint32(0)
    _check("fx_read_error", load_library().fx_read_error(plan.handle, ctypes.byref(w)))
    return int(w.value)


def _kv_numel(plan: Plan) -> int:
    return plan.batch * plan.num_kv_heads * plan.t_cap * plan.head_dim


def fx_build_summaries(plan: Plan, K: torch.Tensor, seq_lens: torch.Tensor, block_begin: int,
                       block_end: int, summaries: torch.Tensor, stream=None) -> None:
    dt = plan.torch_dtype
    _check("fx_build_summaries", load_library().fx_build_summaries(
        plan.handle, _ptr(K, "K", dt, _kv_numel(plan)),
        _ptr(seq_lens, "seq_lens", torch.int32, plan.batch), int(block_begin), int(block_end),
        _ptr(summaries, "summaries", dt, plan.summary_bytes // plan.elem_bytes), _stream(stream)))


def fx_select(plan: Plan, q: torch.Tensor, summaries: Optional[torch.Tensor],
              evict_logits: Optional[torch.Tensor], evicted_mask: Optional[torch.Tensor],
              seq_lens: torch.Tensor, sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
              workspace: torch.Tensor, stream=None) -> None:
    dt = plan.torch_dtype
    units = plan.units
    _check("fx_select", load_library().fx_select(
        plan.handle, _ptr(q, "q", dt, plan.batch * plan.num_q_heads * plan.head_dim),
        _ptr(summaries, "summaries", dt, plan.summary_bytes // plan.elem_bytes, optional=True),
        _ptr(evict_logits, "evict_logits", torch.float32, plan.logits_bytes // 4, optional=True),
        _ptr(evicted_mask, "evicted_mask", torch.int32, plan.evict_mask_bytes // 4, optional=True),
        _ptr(seq_lens, "seq_lens", torch.int32, plan.batch),
        _ptr(sel_idx, "sel_idx", torch.int32, units * plan.max_selected),
        _ptr(sel_cnt, "sel_cnt", torch.int32, units),
        _ptr(workspace, "workspace", torch.uint8, plan.workspace_bytes), workspace.numel(),
        _stream(stream)))


def fx_select_delta(plan: Plan, q: torch.Tensor, summaries: Optional[torch.Tensor],
                    evict_logits: Optional[torch.Tensor], evicted_mask: Optional[torch.Tensor],
                    seq_lens: torch.Tensor, prev_idx: torch.Tensor, prev_cnt: torch.Tensor,
                    sel_idx: torch.Tensor, sel_cnt: torch.Tensor, added: torch.Tensor,
                    added_cnt: torch.Tensor, removed: torch.Tensor, removed_cnt: torch.Tensor,
                    workspace: torch.Tensor, stream=None) -> None:
    dt = plan.torch_dtype
    n, u, i32 = plan.units * plan.max_selected, plan.units, torch.int32
    _check("fx_select_delta", load_library().fx_select_delta(
        plan.handle, _ptr(q, "q", dt, plan.batch * plan.num_q_heads * plan.head_dim),
        _ptr(summaries, "summaries", dt, plan.summary_bytes // plan.elem_bytes, optional=True),
        _ptr(evict_logits, "evict_logits", torch.float32, plan.logits_bytes // 4, optional=True),
        _ptr(evicted_mask, "evicted_mask", torch.int32, plan.evict_mask_bytes // 4, optional=True),
        _ptr(seq_lens, "seq_lens", i32, plan.batch),
        _ptr(prev_idx, "prev_idx", i32, n), _ptr(prev_cnt, "prev_cnt", i32, u),
        _ptr(sel_idx, "sel_idx", i32, n), _ptr(sel_cnt, "sel_cnt", i32, u),
        _ptr(added, "added", i32, n), _ptr(added_cnt, "added_cnt", i32, u),
        _ptr(removed, "removed", i32, n), _ptr(removed_cnt, "removed_cnt", i32, u),
        _ptr(workspace, "workspace", torch.uint8, plan.workspace_bytes), workspace.numel(),
        _stream(stream)))


def fx_sparse_decode(plan: Plan, q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                     seq_lens: torch.Tensor, sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
                     softmax_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor],
                     workspace: torch.Tensor, stream=None) -> None:
    dt = plan.torch_dtype
    nq = plan.batch * plan.num_q_heads
    _check("fx_sparse_decode", load_library().fx_sparse_decode(
        plan.handle, _ptr(q, "q", dt, nq * plan.head_dim), _ptr(K, "K", dt, _kv_numel(plan)),
        _ptr(V, "V", dt, _kv_numel(plan)), _ptr(seq_lens, "seq_lens", torch.int32, plan.batch),
        _ptr(sel_idx, "sel_idx", torch.int32, plan.units * plan.max_selected),
        _ptr(sel_cnt, "sel_cnt", torch.int32, plan.units), float(softmax_scale),
        _ptr(out, "out", dt, nq * plan.head_dim), _ptr(lse, "lse", torch.float32, nq, optional=True),
        _ptr(workspace, "workspace", torch.uint8, plan.workspace_bytes), workspace.numel(),
        _stream(stream)))


def fx_sparse_decode_ed(plan: Plan, q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                        seq_lens: torch.Tensor, sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
                        evict_logits: Optional[torch.Tensor], softmax_scale: float,
                        out: torch.Tensor, lse: Optional[torch.Tensor], workspace: torch.Tensor,
                        stream=None) -> None:
    dt = plan.torch_dtype
    nq = plan.batch * plan.num_q_heads
    _check("fx_sparse_decode_ed", load_library().fx_sparse_decode_ed(
        plan.handle, _ptr(q, "q", dt, nq * plan.head_dim), _ptr(K, "K", dt, _kv_numel(plan)),
        _ptr(V, "V", dt, _kv_numel(plan)), _ptr(seq_lens, "seq_lens", torch.int32, plan.batch),
        _ptr(sel_idx, "sel_idx", torch.int32, plan.units * plan.max_selected),
        _ptr(sel_cnt, "sel_cnt", torch.int32, plan.units),
        _ptr(evict_logits, "evict_logits", torch.float32, plan.logits_bytes // 4, optional=True),
        float(softmax_scale), _ptr(out, "out", dt, nq * plan.head_dim),
        _ptr(lse, "lse", torch.float32, nq, optional=True),
        _ptr(workspace, "workspace", torch.uint8, plan.workspace_bytes), workspace.numel(),
        _stream(stream)))


def fx_sparse_decode_noalloc(plan: Plan, q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                             seq_lens: torch.Tensor, sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
                             softmax_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor],
                             stream=None) -> None:
    """fx_sparse_decode without a workspace: the partials live in the library's static
    per-GPU array, so the call allocates nothing (calls on one GPU must not overlap)."""
    dt = plan.torch_dtype
    nq = plan.batch * plan.num_q_heads
    _check("fx_sparse_decode_noalloc", load_library().fx_sparse_decode_noalloc(
        plan.handle, _ptr(q, "q", dt, nq * plan.head_dim), _ptr(K, "K", dt, _kv_numel(plan)),
        _ptr(V, "V", dt, _kv_numel(plan)), _ptr(seq_lens, "seq_lens", torch.int32, plan.batch),
        _ptr(sel_idx, "sel_idx", torch.int32, plan.units * plan.max_selected),
        _ptr(sel_cnt, "sel_cnt", torch.int32, plan.units), float(softmax_scale),
        _ptr(out, "out", dt, nq * plan.head_dim), _ptr(lse, "lse", torch.float32, nq, optional=True),
        _stream(stream)))


def fx_noalloc_scratch_bytes(plan: Plan) -> int:
    """Bytes of the static array fx_sparse_decode_noalloc uses for this plan."""
    return int(load_library().fx_noalloc_scratch_bytes(plan.handle))


def fx_unit_max_selected(plan: Plan, unit: int) -> int:
    """A unit's selection bound, which is also its number of compaction slots."""
    return int(load_library().fx_unit_max_selected(plan.handle, int(unit)))


def fx_unit_work_offset(plan: Plan, unit: int) -> int:
    """First working-set row of a unit (-1 if out of range)."""
    return int(load_library().fx_unit_work_offset(plan.handle, int(unit)))


@dataclass
class WorkingSet:
    """Caller-owned state of fx_compact_update."""
    slot_map: torch.Tensor     # int32 [units][max_sel], -1 = free
    work_K: torch.Tensor       # elem [work_rows][d]
    work_V: torch.Tensor
    moved_cnt: torch.Tensor    # int32 [units]


def allocate_working_set(plan: Plan, device="cuda") -> WorkingSet:
    """Allocate (with torch) the block-slot working set of a plan, every slot free."""
    rows = plan.work_bytes // (plan.elem_bytes * plan.head_dim)
    return WorkingSet(
        slot_map=torch.full((plan.units, plan.max_selected), -1, dtype=torch.int32, device=device),
        work_K=torch.zeros((max(rows, 1), plan.head_dim), dtype=plan.torch_dtype, device=device),
        work_V=torch.zeros((max(rows, 1), plan.head_dim), dtype=plan.torch_dtype, device=device),
        moved_cnt=torch.zeros(plan.units, dtype=torch.int32, device=device))


def fx_compact_update(plan: Plan, K: torch.Tensor, V: torch.Tensor, seq_lens: torch.Tensor,
                      sel_idx: torch.Tensor, sel_cnt: torch.Tensor, ws: WorkingSet,
                      workspace: torch.Tensor, stream=None) -> None:
    dt = plan.torch_dtype
    n, u = plan.units * plan.max_selected, plan.units
    _check("fx_compact_update", load_library().fx_compact_update(
        plan.handle, _ptr(K, "K", dt, _kv_numel(plan)), _ptr(V, "V", dt, _kv_numel(plan)),
        _ptr(seq_lens, "seq_lens", torch.int32, plan.batch),
        _ptr(sel_idx, "sel_idx", torch.int32, n), _ptr(sel_cnt, "sel_cnt", torch.int32, u),
        _ptr(ws.slot_map, "slot_map", torch.int32, n),
        _ptr(ws.work_K, "work_K", dt, plan.work_bytes // plan.elem_bytes),
        _ptr(ws.work_V, "work_V", dt, plan.work_bytes // plan.elem_bytes),
        _ptr(ws.moved_cnt, "moved_cnt", torch.int32, u, optional=True),
        _ptr(workspace, "workspace", torch.uint8, plan.workspace_bytes), workspace.numel(),
        _stream(stream)))


def fx_selection_delta(plan: Plan, prev_idx: torch.Tensor, prev_cnt: torch.Tensor,
                       cur_idx: torch.Tensor, cur_cnt: torch.Tensor, added: torch.Tensor,
                       added_cnt: torch.Tensor, removed: torch.Tensor, removed_cnt: torch.Tensor,
                       stream=None) -> None:
    n, u = plan.units * plan.max_selected, plan.units
    i32 = torch.int32
    _check("fx_selection_delta", load_library().fx_selection_delta(
        plan.handle, _ptr(prev_idx, "prev_idx", i32, n), _ptr(prev_cnt, "prev_cnt", i32, u),
        _ptr(cur_idx, "cur_idx", i32, n), _ptr(cur_cnt, "cur_cnt", i32, u),
        _ptr(added, "added", i32, n), _ptr(added_cnt, "added_cnt", i32, u),
        _ptr(removed, "removed", i32, n), _ptr(removed_cnt, "removed_cnt", i32, u),
        _stream(stream)))


def fx_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read all of `src` once (the streaming-read bandwidth reference); sink: int32 GPU
    tensor of at least fx_stream_read_sink_words(src bytes) elements."""
    lib = load_library()
    nbytes = src.numel() * src.element_size()
    words = lib.fx_stream_read_sink_words(nbytes)
    _check("fx_stream_read", lib.fx_stream_read(_ptr(src, "src"), nbytes,
                                                _ptr(sink, "sink", torch.int32, words),
                                                _stream(stream)))


@dataclass
class StepBuffers:
    """Device buffers one decode step needs besides q, K, V and seq_lens."""
    summaries: torch.Tensor
    workspace: torch.Tensor
    evicted_mask: torch.Tensor
    sel_idx: torch.Tensor
    sel_cnt: torch.Tensor
    prev_idx: torch.Tensor
    prev_cnt: torch.Tensor
    added: torch.Tensor
    added_cnt: torch.Tensor
    removed: torch.Tensor
    removed_cnt: torch.Tensor
    out: torch.Tensor
    lse: torch.Tensor


def allocate_step_buffers(plan: Plan, device="cuda") -> StepBuffers:
    """Allocate (with torch) every buffer sized from the plan; masks and counts start at zero."""
    u, ms = plan.units, plan.max_selected
    i32 = torch.int32
    nq = plan.batch * plan.num_q_heads
    return StepBuffers(
        summaries=torch.zeros(plan.summary_bytes // plan.elem_bytes, dtype=plan.torch_dtype, device=device),
        workspace=torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=device),
        evicted_mask=torch.zeros(max(1, plan.evict_mask_bytes // 4), dtype=i32, device=device),
        sel_idx=torch.full((u, ms), -1, dtype=i32, device=device),
        sel_cnt=torch.zeros(u, dtype=i32, device=device),
        prev_idx=torch.full((u, ms), -1, dtype=i32, device=device),
        prev_cnt=torch.zeros(u, dtype=i32, device=device),
        added=torch.full((u, ms), -1, dtype=i32, device=device),
        added_cnt=torch.zeros(u, dtype=i32, device=device),
        removed=torch.full((u, ms), -1, dtype=i32, device=device),
        removed_cnt=torch.zeros(u, dtype=i32, device=device),
        out=torch.zeros((plan.batch, plan.num_q_heads, plan.head_dim), dtype=plan.torch_dtype, device=device),
        lse=torch.zeros((plan.batch, plan.num_q_heads), dtype=torch.float32, device=device),
    )
