"""ctypes binding of liboasis (see include/oasis.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of liboasis.so.  PyTorch provides device memory and the current HIP
stream.  Shapes, dtypes, devices and contiguity are checked here before any
pointer reaches the library, so that a kernel never sees a buffer smaller
than its grid assumes.  There is no fallback: without the built library every
call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Dict, Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liboasis.so")

OASIS_OK = 0
STATUS_NAMES = {0: "OASIS_OK", 1: "OASIS_ERR_INVALID_ARG", 2: "OASIS_ERR_UNSUPPORTED",
                3: "OASIS_ERR_WORKSPACE", 4: "OASIS_ERR_HIP"}


class OasisDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("num_queries", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("window_tokens", ctypes.c_int32),
        ("fetch_ratio", ctypes.c_double),
    ]

    def __repr__(self):
        return "OasisDims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class OasisError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_P = ctypes.c_void_p
_DIMS = ctypes.POINTER(OasisDims)
_SIGNATURES = {
    "oasis_abi_version": (ctypes.c_int, []),
    "oasis_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "oasis_last_error": (ctypes.c_char_p, []),
    "oasis_fetch_cap": (ctypes.c_int32, [_DIMS]),
    "oasis_table_stride": (ctypes.c_int32, [_DIMS]),
    "oasis_workspace_bytes": (ctypes.c_size_t, [_DIMS]),
    "oasis_workspace_clear": (ctypes.c_int, [_DIMS, _P, ctypes.c_size_t, _P]),
    "oasis_workspace_status_offset": (ctypes.c_size_t, [_DIMS]),
    "oasis_overlapped_selects_in_launch1": (ctypes.c_int32, [_DIMS]),
    "oasis_decode_step_redoes_touched_splits": (ctypes.c_int32, [_DIMS]),
    "oasis_attn_workspace_bytes": (ctypes.c_size_t, [_DIMS, ctypes.c_int32]),
    "oasis_build_summaries": (ctypes.c_int, [_DIMS, _P, _P, _P, _P]),
    "oasis_score_summaries": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P]),
    "oasis_topk_blocks": (ctypes.c_int, [_DIMS, _P, _P, _P, _P]),
    "oasis_build_plan": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "oasis_sparse_decode_attn": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, ctypes.c_int32, _P,
                                                ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]),
    "oasis_decode_step": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                         ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]),
    "oasis_decode_step_timed": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                               _P, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P,
                                               ctypes.POINTER(ctypes.c_void_p)]),
    "oasis_sparse_decode_attn_resident": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, ctypes.c_float,
                                                         _P, _P, _P, ctypes.c_size_t, _P]),
    "oasis_decode_step_overlapped": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                    _P, _P, ctypes.c_float, _P, _P, _P, ctypes.c_size_t,
                                                    _P]),
    "oasis_decode_step_overlapped_noalloc": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                            _P, _P, _P, ctypes.c_float, _P, _P, _P]),
    "oasis_decode_step_overlapped_timed": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                          _P, _P, _P, ctypes.c_float, _P, _P, _P,
                                                          ctypes.c_size_t, _P,
                                                          ctypes.POINTER(ctypes.c_void_p)]),
    "oasis_window_ring_slots": (ctypes.c_int32, [_DIMS]),
    "oasis_fill_working_set": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "oasis_execute_plan": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P]),
    "oasis_append_token": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "oasis_sparse_decode_attn_pool": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                                     _P, _P, _P, ctypes.c_size_t, _P]),
    "oasis_decode_step_pool": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                              _P, _P, _P, _P, ctypes.c_float, _P, _P, _P,
                                              ctypes.c_size_t, _P]),
    "oasis_decode_step_pool_async": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                    _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P,
                                                    ctypes.c_size_t, _P, _P, _P]),
    "oasis_decode_layer_pipelined": (ctypes.c_int, [_DIMS, _P, _P, ctypes.c_float, _P]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liboasis.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it first (python -m oasis_score_summaries_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols() -> Tuple[str, ...]:
    return tuple(_SIGNATURES)


def _check(status: int, where: str) -> None:
    if status != OASIS_OK:
        msg = load().oasis_last_error().decode(errors="replace")
        raise OasisError(status, where, msg)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _norm_device(dev) -> torch.device:
    dev = torch.device(dev)
    if dev.type == "cuda" and dev.index is None:
        return torch.device("cuda", torch.cuda.current_device())
    return dev


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: Tuple[int, ...], device=None,
          align: int = 4):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if device is not None and _norm_device(t.device) != _norm_device(device):
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.data_ptr() % align != 0:
        raise ValueError(f"{name} must be {align}-byte aligned")


def make_dims(batch: int, num_kv_heads: int, group: int, max_blocks: int, num_queries: int,
              top_k: int, window_tokens: int, fetch_ratio: float, head_dim: int = 128,
              block_size: int = 16) -> OasisDims:
    return OasisDims(batch, num_kv_heads, group, head_dim, block_size, max_blocks, num_queries,
                     top_k, window_tokens, float(fetch_ratio))


def dims_for(workload) -> OasisDims:
    """Dims of a synthetic workload (any object with the Workload fields)."""
    return make_dims(workload.batch, workload.num_kv_heads, workload.group, workload.max_blocks,
                     workload.queries, workload.top_k, workload.window, workload.fetch_ratio,
                     block_size=getattr(workload, "block", 16))


def fetch_cap(dims: OasisDims) -> int:
    c = load().oasis_fetch_cap(ctypes.byref(dims))
    if c < 0:
        _check(1, "oasis_fetch_cap")
    return c


def table_stride(dims: OasisDims) -> int:
    t = load().oasis_table_stride(ctypes.byref(dims))
    if t < 0:
        _check(1, "oasis_table_stride")
    return t


def workspace_bytes(dims: OasisDims, stride: Optional[int] = None) -> int:
    lib = load()
    n = (lib.oasis_workspace_bytes(ctypes.byref(dims)) if stride is None
         else lib.oasis_attn_workspace_bytes(ctypes.byref(dims), int(stride)))
    if n == 0:
        _check(1, "oasis_workspace_bytes")
    return n


def _shapes(d: OasisDims):
    B, H, G, Q, NB, K = d.batch, d.num_kv_heads, d.group, d.num_queries, d.max_blocks, d.top_k
    return {
        "q": (B, H, G, Q, 128), "kv": (B, H, NB, d.block_size, 128), "summ": (B, H, NB, 2, 128),
        "lens": (B,), "scores": (B, H, NB), "topk": (B, H, K), "resident": (B, H, K),
        "bh": (B, H), "out": (B, H, G, 128), "lse": (B, H, G),
    }


def build_summaries(dims: OasisDims, k: torch.Tensor, seq_lens: torch.Tensor,
                    summ: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    s = _shapes(dims)
    _need(k, "k", torch.bfloat16, s["kv"], align=16)
    _need(seq_lens, "seq_lens", torch.int32, s["lens"], k.device)
    if summ is None:
        summ = torch.empty(s["summ"], dtype=torch.bfloat16, device=k.device)
    _need(summ, "summ", torch.bfloat16, s["summ"], k.device, align=16)
    _check(load().oasis_build_summaries(ctypes.byref(dims), _ptr(k), _ptr(seq_lens), _ptr(summ),
                                        _stream(stream)), "oasis_build_summaries")
    return summ


def score_summaries(dims: OasisDims, q: torch.Tensor, summ: torch.Tensor, seq_lens: torch.Tensor,
                    scores: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    s = _shapes(dims)
    _need(q, "q", torch.bfloat16, s["q"], align=16)
    _need(summ, "summ", torch.bfloat16, s["summ"], q.device, align=16)
    _need(seq_lens, "seq_lens", torch.int32, s["lens"], q.device)
    if scores is None:
        scores = torch.empty(s["scores"], dtype=torch.float32, device=q.device)
    _need(scores, "scores", torch.float32, s["scores"], q.device)
    _check(load().oasis_score_summaries(ctypes.byref(dims), _ptr(q), _ptr(summ), _ptr(seq_lens),
                                        _ptr(scores), _stream(stream)), "oasis_score_summaries")
    return scores


def topk_blocks(dims: OasisDims, scores: torch.Tensor, seq_lens: torch.Tensor,
                topk: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    s = _shapes(dims)
    _need(scores, "scores", torch.float32, s["scores"])
    _need(seq_lens, "seq_lens", torch.int32, s["lens"], scores.device)
    if topk is None:
        topk = torch.empty(s["topk"], dtype=torch.int32, device=scores.device)
    _need(topk, "topk", torch.int32, s["topk"], scores.device)
    _check(load().oasis_topk_blocks(ctypes.byref(dims), _ptr(scores), _ptr(seq_lens), _ptr(topk),
                                    _stream(stream)), "oasis_topk_blocks")
    return topk


def _plan_outputs(dims: OasisDims, device, plan, plan_count, table, table_count):
    s = _shapes(dims)
    C, T = fetch_cap(dims), table_stride(dims)
    if plan is None:
        plan = torch.empty((dims.batch, dims.num_kv_heads, C, 3), dtype=torch.int32, device=device)
    if plan_count is None:
        plan_count = torch.empty(s["bh"], dtype=torch.int32, device=device)
    if table is None:
        table = torch.empty((dims.batch, dims.num_kv_heads, T), dtype=torch.int32, device=device)
    if table_count is None:
        table_count = torch.empty(s["bh"], dtype=torch.int32, device=device)
    _need(plan, "plan", torch.int32, (dims.batch, dims.num_kv_heads, C, 3), device)
    _need(plan_count, "plan_count", torch.int32, s["bh"], device)
    _need(table, "table", torch.int32, (dims.batch, dims.num_kv_heads, T), device)
    _need(table_count, "table_count", torch.int32, s["bh"], device)
    return plan, plan_count, table, table_count


def build_plan(dims: OasisDims, scores: torch.Tensor, topk: torch.Tensor, seq_lens: torch.Tensor,
               resident: torch.Tensor, plan=None, plan_count=None, table=None, table_count=None,
               stream=None) -> Dict[str, torch.Tensor]:
    """Applies the capped plan; ``resident`` is updated in place."""
    s = _shapes(dims)
    _need(scores, "scores", torch.float32, s["scores"])
    dev = scores.device
    _need(topk, "topk", torch.int32, s["topk"], dev)
    _need(seq_lens, "seq_lens", torch.int32, s["lens"], dev)
    _need(resident, "resident", torch.int32, s["resident"], dev)
    plan, plan_count, table, table_count = _plan_outputs(dims, dev, plan, plan_count, table, table_count)
    _check(load().oasis_build_plan(ctypes.byref(dims), _ptr(scores), _ptr(topk), _ptr(seq_lens),
                                   _ptr(resident), _ptr(plan if plan.numel() else None),
                                   _ptr(plan_count), _ptr(table), _ptr(table_count), _stream(stream)),
           "oasis_build_plan")
    return {"plan": plan, "plan_count": plan_count, "resident": resident, "table": table,
            "table_count": table_count}


def sparse_decode_attn(dims: OasisDims, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       table: torch.Tensor, table_count: torch.Tensor, seq_lens: torch.Tensor,
                       scale: Optional[float] = None, out=None, lse=None, ws=None,
                       stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    s = _shapes(dims)
    _need(q, "q", torch.bfloat16, s["q"], align=16)
    dev = q.device
    _need(k, "k", torch.bfloat16, s["kv"], dev, align=16)
    _need(v, "v", torch.bfloat16, s["kv"], dev, align=16)
    if table.dim() != 3:
        raise ValueError("table must be [B, H, table_stride]")
    stride = int(table.shape[2])
    _need(table, "table", torch.int32, (dims.batch, dims.num_kv_heads, stride), dev)
    _need(table_count, "table_count", torch.int32, s["bh"], dev)
    _need(seq_lens, "seq_lens", torch.int32, s["lens"], dev)
    if scale is None:
        scale = 1.0 / math.sqrt(128)
    if out is None:
        out = torch.empty(s["out"], dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(s["lse"], dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, s["out"], dev, align=16)
    _need(lse, "lse", torch.float32, s["lse"], dev)
    need = workspace_bytes(dims, stride)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if ws.device != dev or ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous uint8 GPU tensor on the inputs' device")
    _check(load().oasis_sparse_decode_attn(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(table),
                                           _ptr(table_count), stride, _ptr(seq_lens), float(scale),
                                           _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)),
           "oasis_sparse_decode_attn")
    return out, lse


def sparse_decode_attn_resident(dims: OasisDims, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                resident: torch.Tensor, seq_lens: torch.Tensor,
                                scale: Optional[float] = None, out=None, lse=None, ws=None,
                                stream=None):
    """Attention of the target queries over the resident slots plus the window
    (oasis_sparse_decode_attn_resident).  Returns (out, lse)."""
    s = _shapes(dims)
    _need(q, "q", torch.bfloat16, s["q"], align=16)
    dev = q.device
    _need(k, "k", torch.bfloat16, s["kv"], dev, align=16)
    _need(v, "v", torch.bfloat16, s["kv"], dev, align=16)
    _need(resident, "resident", torch.int32, s["resident"], dev)
    _need(seq_lens, "seq_lens", torch.int32, s["lens"], dev)
    if scale is None:
        scale = 1.0 / math.sqrt(128)
    if out is None:
        out = torch.empty(s["out"], dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(s["lse"], dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, s["out"], dev, align=16)
    _need(lse, "lse", torch.float32, s["lse"], dev)
    need = workspace_bytes(dims)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if ws.device != dev or ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous uint8 GPU tensor on the inputs' device")
    _check(load().oasis_sparse_decode_attn_resident(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(resident), _ptr(seq_lens), float(scale),
        _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)), "oasis_sparse_decode_attn_resident")
    return out, lse


def step_workspace(dims: OasisDims, device) -> torch.Tensor:
    """A workspace for the decode steps, zero-filled as the overlapped step's hand-off
    region requires before its first use (each step leaves it zero)."""
    return torch.zeros(workspace_bytes(dims), dtype=torch.uint8, device=_norm_device(device))


def overlapped_selects_in_launch1(dims: OasisDims) -> bool:
    """Whether the overlapped step's first launch holds the selection and plan
    (oasis_overlapped_selects_in_launch1)."""
    r = int(load().oasis_overlapped_selects_in_launch1(ctypes.byref(dims)))
    if r < 0:
        _check(1, "oasis_overlapped_selects_in_launch1")
    return r == 1


def decode_step_redoes_touched_splits(dims: OasisDims) -> bool:
    """Whether decode_step with its own ``resident_next`` runs as the overlapped
    step's first launch plus a launch that redoes only the splits the plan touched
    (oasis_decode_step_redoes_touched_splits)."""
    r = int(load().oasis_decode_step_redoes_touched_splits(ctypes.byref(dims)))
    if r < 0:
        _check(1, "oasis_decode_step_redoes_touched_splits")
    return r == 1


def workspace_clear(dims: OasisDims, ws: torch.Tensor, stream=None) -> None:
    """Zero-fills the hand-off region of a step workspace (oasis_workspace_clear)."""
    _check(load().oasis_workspace_clear(ctypes.byref(dims), _ptr(ws), ws.numel(), _stream(stream)),
           "oasis_workspace_clear")


def workspace_status(dims: OasisDims, ws: torch.Tensor) -> int:
    """The hand-off status word of a step workspace (0 unless a selection workgroup
    of the overlapped step timed out waiting for its scores); reads it after the work
    queued so far."""
    off = int(load().oasis_workspace_status_offset(ctypes.byref(dims)))
    if off == 0 or off + 4 > ws.numel():
        raise ValueError("the workspace is not a step workspace for these dims")
    return int(ws[off:off + 4].view(torch.int32).item())


class StepBuffers:
    """Outputs and workspace of oasis_decode_step, allocated once and reused."""

    def __init__(self, dims: OasisDims, device):
        s = _shapes(dims)
        dev = _norm_device(device)
        self.scores = torch.empty(s["scores"], dtype=torch.float32, device=dev)
        self.topk = torch.empty(s["topk"], dtype=torch.int32, device=dev)
        self.plan, self.plan_count, self.table, self.table_count = _plan_outputs(
            dims, dev, None, None, None, None)
        self.out = torch.empty(s["out"], dtype=torch.float32, device=dev)
        self.lse = torch.empty(s["lse"], dtype=torch.float32, device=dev)
        self.ws = step_workspace(dims, dev)
        self.dims = dims

    def status(self) -> int:
        """The workspace's hand-off status word (0 unless a wait timed out)."""
        return workspace_status(self.dims, self.ws)

    def as_dict(self) -> Dict[str, torch.Tensor]:
        return {n: getattr(self, n) for n in ("scores", "topk", "plan", "plan_count", "table",
                                              "table_count", "out", "lse")}


def decode_step(dims: OasisDims, q: torch.Tensor, summ: torch.Tensor, k: torch.Tensor,
                v: torch.Tensor, seq_lens: torch.Tensor, resident: torch.Tensor,
                scale: Optional[float] = None, buffers: Optional[StepBuffers] = None,
                resident_next: Optional[torch.Tensor] = None, stream=None) -> Dict[str, torch.Tensor]:
    """score -> top-K -> capped plan -> attention.  The updated resident set goes to
    ``resident_next`` if given (``resident`` is then only read), else in place."""
    s = _shapes(dims)
    _need(q, "q", torch.bfloat16, s["q"], align=16)
    dev = q.device
    _need(summ, "summ", torch.bfloat16, s["summ"], dev, align=16)
    _need(k, "k", torch.bfloat16, s["kv"], dev, align=16)
    _need(v, "v", torch.bfloat16, s["kv"], dev, align=16)
    _need(seq_lens, "seq_lens", torch.int32, s["lens"], dev)
    _need(resident, "resident", torch.int32, s["resident"], dev)
    if resident_next is not None:
        _need(resident_next, "resident_next", torch.int32, s["resident"], dev)
    if buffers is None:
        buffers = StepBuffers(dims, dev)
    b = buffers
    if scale is None:
        scale = 1.0 / math.sqrt(128)
    _check(load().oasis_decode_step(
        ctypes.byref(dims), _ptr(q), _ptr(summ), _ptr(k), _ptr(v), _ptr(seq_lens), _ptr(b.scores),
        _ptr(b.topk), _ptr(resident), _ptr(resident_next),
        _ptr(b.plan if b.plan.numel() else None), _ptr(b.plan_count),
        _ptr(b.table), _ptr(b.table_count), float(scale), _ptr(b.out), _ptr(b.lse), _ptr(b.ws),
        b.ws.numel(), _stream(stream)), "oasis_decode_step")
    res = b.as_dict()
    res["resident"] = resident if resident_next is None else resident_next
    return res


def decode_step_overlapped(dims: OasisDims, q: torch.Tensor, summ: torch.Tensor, k: torch.Tensor,
                           v: torch.Tensor, seq_lens: torch.Tensor, resident: torch.Tensor,
                           resident_next: torch.Tensor, scale: Optional[float] = None,
                           buffers: Optional[StepBuffers] = None, stream=None) -> Dict[str, torch.Tensor]:
    """Attention over ``resident`` (plus the window) and, alongside it, score ->
    top-K -> capped plan writing the next slot table to ``resident_next``
    (oasis_decode_step_overlapped)."""
    s = _shapes(dims)
    _need(q, "q", torch.bfloat16, s["q"], align=16)
    dev = q.device
    _need(summ, "summ", torch.bfloat16, s["summ"], dev, align=16)
    _need(k, "k", torch.bfloat16, s["kv"], dev, align=16)
    _need(v, "v", torch.bfloat16, s["kv"], dev, align=16)
    _need(seq_lens, "seq_lens", torch.int32, s["lens"], dev)
    _need(resident, "resident", torch.int32, s["resident"], dev)
    _need(resident_next, "resident_next", torch.int32, s["resident"], dev)
    if buffers is None:
        buffers = StepBuffers(dims, dev)
    b = buffers
    if scale is None:
        scale = 1.0 / math.sqrt(128)
    _check(load().oasis_decode_step_overlapped(
        ctypes.byref(dims), _ptr(q), _ptr(summ), _ptr(k), _ptr(v), _ptr(seq_lens), _ptr(b.scores),
        _ptr(b.topk), _ptr(resident), _ptr(resident_next),
        _ptr(b.plan if b.plan.numel() else None), _ptr(b.plan_count),
        _ptr(b.table), _ptr(b.table_count), float(scale), _ptr(b.out), _ptr(b.lse), _ptr(b.ws),
        b.ws.numel(), _stream(stream)), "oasis_decode_step_overlapped")
    res = b.as_dict()
    res["resident"] = resident_next
    return res


def decode_step_overlapped_noalloc(dims: OasisDims, q: torch.Tensor, summ: torch.Tensor, k: torch.Tensor,
                                   v: torch.Tensor, seq_lens: torch.Tensor, resident: torch.Tensor,
                                   resident_next: torch.Tensor, scale: Optional[float] = None,
                                   outputs: Optional[StepBuffers] = None, stream=None) -> Dict[str, torch.Tensor]:
    """decode_step_overlapped with the library's own scratch array as the workspace
    (oasis_decode_step_overlapped_noalloc); ``outputs``' workspace is not used."""
    s = _shapes(dims)
    _need(q, "q", torch.bfloat16, s["q"], align=16)
    dev = q.device
    _need(summ, "summ", torch.bfloat16, s["summ"], dev, align=16)
    _need(k, "k", torch.bfloat16, s["kv"], dev, align=16)
    _need(v, "v", torch.bfloat16, s["kv"], dev, align=16)
    _need(seq_lens, "seq_lens", torch.int32, s["lens"], dev)
    _need(resident, "resident", torch.int32, s["resident"], dev)
    _need(resident_next, "resident_next", torch.int32, s["resident"], dev)
    if outputs is None:
        outputs = StepBuffers(dims, dev)
    b = outputs
    if scale is None:
        scale = 1.0 / math.sqrt(128)
    _check(load().oasis_decode_step_overlapped_noalloc(
        ctypes.byref(dims), _ptr(q), _ptr(summ), _ptr(k), _ptr(v), _ptr(seq_lens), _ptr(b.scores),
        _ptr(b.topk), _ptr(resident), _ptr(resident_next),
        _ptr(b.plan if b.plan.numel() else None), _ptr(b.plan_count),
        _ptr(b.table), _ptr(b.table_count), float(scale), _ptr(b.out), _ptr(b.lse),
        _stream(stream)), "oasis_decode_step_overlapped_noalloc")
    res = b.as_dict()
    res["resident"] = resident_next
    return res


# ---------------------------------------------------------------------------
# Repeated steps: arguments marshalled once, HIP events for stage timing
# ---------------------------------------------------------------------------

_hip = None


# ---- executing the plan: the working set in HBM -----------------------------------

def window_ring_slots(dims: OasisDims) -> int:
    n = load().oasis_window_ring_slots(ctypes.byref(dims))
    if n < 0:
        _check(1, "oasis_window_ring_slots")
    return n


class WorkingSet:
    """The working set of every KV head in HBM: a pool of K block slots (slot s holds
    the block of resident slot s) and a ring of window blocks (window block j in
    ring slot j % window_ring_slots(dims)), K and V, bf16."""

    def __init__(self, dims: OasisDims, device):
        dev = _norm_device(device)
        B, H, K, WB = dims.batch, dims.num_kv_heads, dims.top_k, window_ring_slots(dims)
        self.dims = dims
        bs = dims.block_size
        self.pool_k = torch.zeros((B, H, K, bs, 128), dtype=torch.bfloat16, device=dev)
        self.pool_v = torch.zeros_like(self.pool_k)
        self.ring_k = torch.zeros((B, H, WB, bs, 128), dtype=torch.bfloat16, device=dev)
        self.ring_v = torch.zeros_like(self.ring_k)

    def check(self, device):
        B, H, K = self.dims.batch, self.dims.num_kv_heads, self.dims.top_k
        WB, bs = window_ring_slots(self.dims), self.dims.block_size
        for n in ("pool_k", "pool_v"):
            _need(getattr(self, n), n, torch.bfloat16, (B, H, K, bs, 128), device, align=16)
        for n in ("ring_k", "ring_v"):
            _need(getattr(self, n), n, torch.bfloat16, (B, H, WB, bs, 128), device, align=16)


def _cache_ptr(t: torch.Tensor, name: str, shape, device) -> ctypes.c_void_p:
    """Device address of a full-cache tensor: a GPU tensor on ``device``, or a pinned
    host tensor (its mapped address, read by the kernels over the host link)."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or tuple(t.shape) != tuple(shape) \
            or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bf16 tensor of shape {tuple(shape)}")
    if t.device.type == "cuda":
        _need(t, name, torch.bfloat16, shape, device, align=16)
        return _ptr(t)
    if not t.is_pinned():
        raise ValueError(f"{name} must be a GPU tensor or a pinned host tensor")
    h = _hip_runtime()
    dptr = ctypes.c_void_p()
    if h.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(t.data_ptr()), 0) != 0:
        raise RuntimeError(f"hipHostGetDevicePointer failed for {name}")
    return dptr


def fill_working_set(dims: OasisDims, resident: torch.Tensor, seq_lens: torch.Tensor, k: torch.Tensor,
                     v: torch.Tensor, wset: Optional[WorkingSet] = None, stream=None) -> WorkingSet:
    """Gathers the working set of slot table ``resident`` from the full cache k, v
    (GPU or pinned host tensors) into ``wset`` (new if None)."""
    s = _shapes(dims)
    _need(resident, "resident", torch.int32, s["resident"])
    dev = resident.device
    _need(seq_lens, "seq_lens", torch.int32, s["lens"], dev)
    kp, vp = _cache_ptr(k, "k", s["kv"], dev), _cache_ptr(v, "v", s["kv"], dev)
    if wset is None:
        wset = WorkingSet(dims, dev)
    wset.check(dev)
    _check(load().oasis_fill_working_set(ctypes.byref(dims), _ptr(resident), _ptr(seq_lens), kp, vp,
                                         _ptr(wset.pool_k), _ptr(wset.pool_v), _ptr(wset.ring_k),
                                         _ptr(wset.ring_v), _stream(stream)), "oasis_fill_working_set")
    return wset


def execute_plan(dims: OasisDims, plan: torch.Tensor, plan_count: torch.Tensor, k: torch.Tensor,
                 v: torch.Tensor, wset: WorkingSet, stream=None) -> None:
    """Copies every plan row's admitted block from the full cache into its pool slot."""
    s = _shapes(dims)
    _need(plan_count, "plan_count", torch.int32, s["bh"])
    dev = plan_count.device
    _need(plan, "plan", torch.int32, (dims.batch, dims.num_kv_heads, fetch_cap(dims), 3), dev)
    kp, vp = _cache_ptr(k, "k", s["kv"], dev), _cache_ptr(v, "v", s["kv"], dev)
    wset.check(dev)
    _check(load().oasis_execute_plan(ctypes.byref(dims), _ptr(plan if plan.numel() else None),
                                     _ptr(plan_count), kp, vp, _ptr(wset.pool_k), _ptr(wset.pool_v),
                                     _stream(stream)), "oasis_execute_plan")


def append_token(dims: OasisDims, k_new: torch.Tensor, v_new: torch.Tensor, seq_lens: torch.Tensor,
                 summ: torch.Tensor, wset: WorkingSet, k: Optional[torch.Tensor] = None,
                 v: Optional[torch.Tensor] = None, stream=None) -> None:
    """Writes one token per sequence at position seq_lens[b] into the ring, the full
    cache (if given) and its block's summary; seq_lens is left to the caller."""
    s = _shapes(dims)
    _need(k_new, "k_new", torch.bfloat16, (dims.batch, dims.num_kv_heads, 128), align=16)
    dev = k_new.device
    _need(v_new, "v_new", torch.bfloat16, (dims.batch, dims.num_kv_heads, 128), dev, align=16)
    _need(seq_lens, "seq_lens", torch.int32, s["lens"], dev)
    _need(summ, "summ", torch.bfloat16, s["summ"], dev, align=16)
    wset.check(dev)
    if (k is None) != (v is None):
        raise ValueError("k and v must both be given or both be None")
    kp = _cache_ptr(k, "k", s["kv"], dev) if k is not None else _ptr(None)
    vp = _cache_ptr(v, "v", s["kv"], dev) if v is not None else _ptr(None)
    _check(load().oasis_append_token(ctypes.byref(dims), _ptr(k_new), _ptr(v_new), _ptr(seq_lens),
                                     _ptr(summ), kp, vp, _ptr(wset.ring_k), _ptr(wset.ring_v),
                                     _stream(stream)), "oasis_append_token")


def sparse_decode_attn_pool(dims: OasisDims, q: torch.Tensor, wset: WorkingSet, resident: torch.Tensor,
                            seq_lens: torch.Tensor, scale: Optional[float] = None, out=None, lse=None,
                            ws=None, stream=None):
    """Attention of the target queries over the working set (oasis_sparse_decode_attn_pool).
    Returns (out, lse)."""
    s = _shapes(dims)
    _need(q, "q", torch.bfloat16, s["q"], align=16)
    dev = q.device
    wset.check(dev)
    _need(resident, "resident", torch.int32, s["resident"], dev)
    _need(seq_lens, "seq_lens", torch.int32, s["lens"], dev)
    scale = 1.0 / math.sqrt(128) if scale is None else scale
    out = torch.empty(s["out"], dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty(s["lse"], dtype=torch.float32, device=dev) if lse is None else lse
    _need(out, "out", torch.float32, s["out"], dev, align=16)
    _need(lse, "lse", torch.float32, s["lse"], dev)
    ws = torch.empty(workspace_bytes(dims), dtype=torch.uint8, device=dev) if ws is None else ws
    _check(load().oasis_sparse_decode_attn_pool(
        ctypes.byref(dims), _ptr(q), _ptr(wset.pool_k), _ptr(wset.pool_v), _ptr(wset.ring_k),
        _ptr(wset.ring_v), _ptr(resident), _ptr(seq_lens), float(scale), _ptr(out), _ptr(lse), _ptr(ws),
        ws.numel(), _stream(stream)), "oasis_sparse_decode_attn_pool")
    return out, lse


def decode_step_pool(dims: OasisDims, q: torch.Tensor, summ: torch.Tensor, k: torch.Tensor,
                     v: torch.Tensor, wset: WorkingSet, seq_lens: torch.Tensor, resident: torch.Tensor,
                     resident_next: torch.Tensor, scale: Optional[float] = None,
                     buffers: Optional["StepBuffers"] = None, stream=None) -> Dict[str, torch.Tensor]:
    """The overlapped step with the attention over the working set, then the plan's
    block copies from the full cache k, v (GPU or pinned host tensors) into the pool
    (oasis_decode_step_pool)."""
    s = _shapes(dims)
    _need(q, "q", torch.bfloat16, s["q"], align=16)
    dev = q.device
    _need(summ, "summ", torch.bfloat16, s["summ"], dev, align=16)
    kp, vp = _cache_ptr(k, "k", s["kv"], dev), _cache_ptr(v, "v", s["kv"], dev)
    wset.check(dev)
    _need(seq_lens, "seq_lens", torch.int32, s["lens"], dev)
    _need(resident, "resident", torch.int32, s["resident"], dev)
    _need(resident_next, "resident_next", torch.int32, s["resident"], dev)
    b = StepBuffers(dims, dev) if buffers is None else buffers
    scale = 1.0 / math.sqrt(128) if scale is None else scale
    _check(load().oasis_decode_step_pool(
        ctypes.byref(dims), _ptr(q), _ptr(summ), kp, vp, _ptr(wset.pool_k), _ptr(wset.pool_v),
        _ptr(wset.ring_k), _ptr(wset.ring_v), _ptr(seq_lens), _ptr(b.scores), _ptr(b.topk),
        _ptr(resident), _ptr(resident_next), _ptr(b.plan if b.plan.numel() else None),
        _ptr(b.plan_count), _ptr(b.table), _ptr(b.table_count), float(scale), _ptr(b.out), _ptr(b.lse),
        _ptr(b.ws), b.ws.numel(), _stream(stream)), "oasis_decode_step_pool")
    return {**b.as_dict(), "resident": resident_next}


def _hip_runtime() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        h.hipEventCreate.restype = ctypes.c_int
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventDestroy.restype = ctypes.c_int
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventSynchronize.restype = ctypes.c_int
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventElapsedTime.restype = ctypes.c_int
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventCreateWithFlags.restype = ctypes.c_int
        h.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
        h.hipHostGetDevicePointer.restype = ctypes.c_int
        _hip = h
    return _hip


class StageEvents:
    """HIP events bracketing the kernels of one step: five for the serial step
    (oasis_decode_step_timed), three for the overlapped one
    (oasis_decode_step_overlapped_timed)."""

    SERIAL_STAGES = ("score", "select_plan", "attn_split", "attn_merge")
    OVERLAPPED_STAGES = ("launch1", "launch2")

    def __init__(self, overlapped: bool = False):
        self.STAGES = self.OVERLAPPED_STAGES if overlapped else self.SERIAL_STAGES
        self.N = len(self.STAGES) + 1
        h = _hip_runtime()
        self.handles = (ctypes.c_void_p * self.N)()
        for i in range(self.N):
            ev = ctypes.c_void_p()
            if h.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles[i] = ev.value

    def elapsed_ms(self) -> Dict[str, float]:
        h = _hip_runtime()
        if h.hipEventSynchronize(self.handles[self.N - 1]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        out = {}
        for i, name in enumerate(self.STAGES):
            ms = ctypes.c_float()
            if h.hipEventElapsedTime(ctypes.byref(ms), self.handles[i], self.handles[i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out[name] = float(ms.value)
        return out

    def __del__(self):
        try:
            h = _hip_runtime()
            for i in range(self.N):
                if self.handles[i]:
                    h.hipEventDestroy(self.handles[i])
        except Exception:
            pass


class PreparedStep:
    """One fused decode step whose arguments are checked and marshalled once.

    Calling it queues oasis_decode_step on the current stream (with ``events``,
    oasis_decode_step_timed).  With ``overlapped``, it queues
    oasis_decode_step_overlapped instead: attention over ``resident`` alongside
    the scoring, selection and plan into ``resident_next`` (required).  The
    tensors must stay alive and keep their storage while the object is used.
    """

    def __init__(self, dims: OasisDims, q, summ, k, v, seq_lens, resident, buffers: StepBuffers,
                 resident_next=None, scale: Optional[float] = None, overlapped: bool = False):
        s = _shapes(dims)
        _need(q, "q", torch.bfloat16, s["q"], align=16)
        dev = q.device
        _need(summ, "summ", torch.bfloat16, s["summ"], dev, align=16)
        _need(k, "k", torch.bfloat16, s["kv"], dev, align=16)
        _need(v, "v", torch.bfloat16, s["kv"], dev, align=16)
        _need(seq_lens, "seq_lens", torch.int32, s["lens"], dev)
        _need(resident, "resident", torch.int32, s["resident"], dev)
        if resident_next is not None:
            _need(resident_next, "resident_next", torch.int32, s["resident"], dev)
        b = buffers
        for name, t in b.as_dict().items():
            if _norm_device(t.device) != _norm_device(dev):
                raise ValueError(f"buffer {name} is on {t.device}, expected {dev}")
        if b.ws.numel() < workspace_bytes(dims):
            raise ValueError("workspace too small")
        self.dims = dims
        self.buffers = b
        self.keep = (q, summ, k, v, seq_lens, resident, resident_next)
        scale = 1.0 / math.sqrt(128) if scale is None else float(scale)
        self.args = [ctypes.byref(dims), _ptr(q), _ptr(summ), _ptr(k), _ptr(v), _ptr(seq_lens),
                     _ptr(b.scores), _ptr(b.topk), _ptr(resident), _ptr(resident_next),
                     _ptr(b.plan if b.plan.numel() else None), _ptr(b.plan_count), _ptr(b.table),
                     _ptr(b.table_count), ctypes.c_float(scale), _ptr(b.out), _ptr(b.lse), _ptr(b.ws),
                     ctypes.c_size_t(b.ws.numel())]
        self.lib = load()
        self.overlapped = bool(overlapped)
        if self.overlapped and resident_next is None:
            raise ValueError("the overlapped step needs resident_next (the attention reads resident)")

    def __call__(self, stream=None, events: Optional[StageEvents] = None) -> None:
        st = _stream(stream)
        if self.overlapped:
            if events is not None:
                _check(self.lib.oasis_decode_step_overlapped_timed(*self.args, st, events.handles),
                       "oasis_decode_step_overlapped_timed")
            else:
                _check(self.lib.oasis_decode_step_overlapped(*self.args, st), "oasis_decode_step_overlapped")
        elif events is not None:
            _check(self.lib.oasis_decode_step_timed(*self.args, st, events.handles),
                   "oasis_decode_step_timed")
        else:
            _check(self.lib.oasis_decode_step(*self.args, st), "oasis_decode_step")


class HipEvent:
    """A HIP event without timing, for ordering work between streams."""

    def __init__(self):
        h = _hip_runtime()
        ev = ctypes.c_void_p()
        if h.hipEventCreateWithFlags(ctypes.byref(ev), 2) != 0:   # hipEventDisableTiming
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.handle = ev

    def __del__(self):
        try:
            if self.handle:
                _hip_runtime().hipEventDestroy(self.handle)
        except Exception:
            pass


class PreparedPoolStep:
    """oasis_decode_step_pool with its arguments checked and marshalled once (the
    full cache k, v may be pinned host tensors).  The tensors must stay alive and
    keep their storage while the object is used.  Called with ``transfer_stream``,
    it queues oasis_decode_step_pool_async instead: the plan's copies go to that
    stream after the plan is built (the caller orders this layer's next step after
    them)."""

    def __init__(self, dims: OasisDims, q, summ, k, v, wset: WorkingSet, seq_lens, resident,
                 buffers: StepBuffers, resident_next, scale: Optional[float] = None):
        s = _shapes(dims)
        _need(q, "q", torch.bfloat16, s["q"], align=16)
        dev = q.device
        _need(summ, "summ", torch.bfloat16, s["summ"], dev, align=16)
        kp, vp = _cache_ptr(k, "k", s["kv"], dev), _cache_ptr(v, "v", s["kv"], dev)
        wset.check(dev)
        _need(seq_lens, "seq_lens", torch.int32, s["lens"], dev)
        _need(resident, "resident", torch.int32, s["resident"], dev)
        _need(resident_next, "resident_next", torch.int32, s["resident"], dev)
        b = buffers
        if b.ws.numel() < workspace_bytes(dims):
            raise ValueError("workspace too small")
        self.keep = (q, summ, k, v, wset, seq_lens, resident, resident_next, b)
        scale = 1.0 / math.sqrt(128) if scale is None else float(scale)
        self.args = [ctypes.byref(dims), _ptr(q), _ptr(summ), kp, vp, _ptr(wset.pool_k),
                     _ptr(wset.pool_v), _ptr(wset.ring_k), _ptr(wset.ring_v), _ptr(seq_lens),
                     _ptr(b.scores), _ptr(b.topk), _ptr(resident), _ptr(resident_next),
                     _ptr(b.plan if b.plan.numel() else None), _ptr(b.plan_count), _ptr(b.table),
                     _ptr(b.table_count), ctypes.c_float(scale), _ptr(b.out), _ptr(b.lse), _ptr(b.ws),
                     ctypes.c_size_t(b.ws.numel())]
        self.lib = load()
        self.plan_ready = None

    def __call__(self, stream=None, transfer_stream=None) -> None:
        if transfer_stream is None:
            _check(self.lib.oasis_decode_step_pool(*self.args, _stream(stream)), "oasis_decode_step_pool")
            return
        if self.plan_ready is None:
            self.plan_ready = HipEvent()
        _check(self.lib.oasis_decode_step_pool_async(*self.args, _stream(stream), _stream(transfer_stream),
                                                     self.plan_ready.handle),
               "oasis_decode_step_pool_async")


class PreparedPlanCopy:
    """oasis_execute_plan with its arguments marshalled once."""

    def __init__(self, dims: OasisDims, plan, plan_count, k, v, wset: WorkingSet):
        s = _shapes(dims)
        _need(plan_count, "plan_count", torch.int32, s["bh"])
        dev = plan_count.device
        kp, vp = _cache_ptr(k, "k", s["kv"], dev), _cache_ptr(v, "v", s["kv"], dev)
        wset.check(dev)
        self.keep = (plan, plan_count, k, v, wset)
        self.args = [ctypes.byref(dims), _ptr(plan if plan.numel() else None), _ptr(plan_count), kp, vp,
                     _ptr(wset.pool_k), _ptr(wset.pool_v)]
        self.lib = load()

    def __call__(self, stream=None) -> None:
        _check(self.lib.oasis_execute_plan(*self.args, _stream(stream)), "oasis_execute_plan")


class LayerIO(ctypes.Structure):
    """oasis_layer_io: one layer's buffers for the layer-pipelined decode."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "q", "summ", "k", "v", "seq_lens", "resident", "resident_next", "scores", "topk", "plan",
        "plan_count", "table", "table_count", "out", "lse", "ws")] + [("ws_bytes", ctypes.c_size_t)]


class PipelinedLayers:
    """A sweep over two or more layers with each layer's selection and plan riding in
    the next layer's first launch (oasis_decode_layer_pipelined).  ``layers`` holds,
    per layer, (q, summ, k, v, seq_lens, resident); every layer gets its own outputs
    and next slot table, and all layers share one workspace (their launches run in
    stream order; one workspace also stays warm in the caches from layer to layer:
    0.8 us per layer at the Qwen3-8B shape).  Calling the object queues one decode step over all
    layers (the previous step's last layer is selected in the first layer's launch);
    ``drain()`` queues the last layer's pending selection.  The tensors must stay
    alive while the object is used."""

    def __init__(self, dims: OasisDims, layers, scale: Optional[float] = None):
        if len(layers) < 2:
            raise ValueError("the pipelined sweep needs at least two layers")
        s = _shapes(dims)
        self.dims = dims
        self.scale = 1.0 / math.sqrt(128) if scale is None else float(scale)
        self.lib = load()
        self.buffers, self.resident_next, self.ios, self.keep = [], [], [], []
        self.ws = None
        for (q, summ, k, v, seq_lens, resident) in layers:
            _need(q, "q", torch.bfloat16, s["q"], align=16)
            dev = q.device
            _need(summ, "summ", torch.bfloat16, s["summ"], dev, align=16)
            _need(k, "k", torch.bfloat16, s["kv"], dev, align=16)
            _need(v, "v", torch.bfloat16, s["kv"], dev, align=16)
            _need(seq_lens, "seq_lens", torch.int32, s["lens"], dev)
            _need(resident, "resident", torch.int32, s["resident"], dev)
            b = StepBuffers(dims, dev)
            if self.ws is None:
                self.ws = b.ws
            else:
                b.ws = self.ws
            rn = torch.empty_like(resident)
            io = LayerIO(q.data_ptr(), summ.data_ptr(), k.data_ptr(), v.data_ptr(), seq_lens.data_ptr(),
                         resident.data_ptr(), rn.data_ptr(), b.scores.data_ptr(), b.topk.data_ptr(),
                         b.plan.data_ptr() if b.plan.numel() else 0, b.plan_count.data_ptr(),
                         b.table.data_ptr(), b.table_count.data_ptr(), b.out.data_ptr(), b.lse.data_ptr(),
                         b.ws.data_ptr(), b.ws.numel())
            self.buffers.append(b)
            self.resident_next.append(rn)
            self.ios.append(io)
            self.keep.append((q, summ, k, v, seq_lens, resident))
        self.started = False

    def _call(self, layer, previous, stream):
        _check(self.lib.oasis_decode_layer_pipelined(
            ctypes.byref(self.dims), ctypes.byref(layer) if layer is not None else None,
            ctypes.byref(previous) if previous is not None else None, ctypes.c_float(self.scale),
            _stream(stream)), "oasis_decode_layer_pipelined")

    def __call__(self, stream=None) -> None:
        L = len(self.ios)
        for i in range(L):
            prev = self.ios[i - 1] if (i > 0 or self.started) else None
            self._call(self.ios[i], prev, stream)
        self.started = True

    def drain(self, stream=None) -> None:
        if self.started:
            self._call(None, self.ios[-1], stream)
            self.started = False
