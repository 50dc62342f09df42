"""Thin Python binding of libidx_logits.so, the MI355X lightning-indexer
scoring library ("MQA logits").  The C ABI is declared in include/idx_logits.h;
the functions here carry the same names and only marshal arguments: every step
of the computation runs in the library's HIP kernels.  PyTorch provides device
memory and the current stream.

If the library is missing the import still succeeds but every call raises, so
nothing can silently fall back to another implementation.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libidx_logits.so")

IDX_OK, IDX_E_INVALID, IDX_E_UNSUPPORTED, IDX_E_WORKSPACE, IDX_E_HIP = range(5)
IN_DTYPES = {"bf16": 0, "fp8": 1, "mxfp8": 2, "mxfp4": 3}
# idx_accum_t: "native" (the input format's matrix core) or "fp32" (exact
# products, fp32 sums, for every input)
ACCUM = {"native": 0, "fp32": 1}
ABI_VERSION = 3
FP_DTYPES = {torch.float32: 0, torch.bfloat16: 1}
EXPORTED = ("idx_abi_version", "idx_logits_plan_bytes", "idx_logits_plan", "idx_logits_plan_thd",
            "idx_logits_plan_paged", "idx_logits_prepare_paged", "idx_logits_run_paged", "idx_logits_score_paged",
            "idx_logits_topk", "idx_logits_topk_workspace_bytes", "idx_logits_run_topk",
            "idx_logits_workspace_bytes", "idx_logits_workspace_bytes_planned",
            "idx_logits_run", "idx_logits_run_noalloc", "idx_logits_noalloc_scratch_bytes", "idx_logits_prepare", "idx_logits_score", "idx_logits_plan_windows", "idx_last_error")


class IdxLogitsArgs(ctypes.Structure):
    """Mirror of idx_logits_args_t."""
    _fields_ = [("B", ctypes.c_int32), ("S_q", ctypes.c_int32), ("S_k", ctypes.c_int32), ("H", ctypes.c_int32),
                ("D", ctypes.c_int32), ("in_dtype", ctypes.c_int), ("q", ctypes.c_void_p),
                ("q_scale", ctypes.c_void_p), ("k", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("w", ctypes.c_void_p), ("w_dtype", ctypes.c_int), ("sm_scale", ctypes.c_float),
                ("out", ctypes.c_void_p), ("out_dtype", ctypes.c_int), ("out_row_stride", ctypes.c_int64),
                ("clean_logits", ctypes.c_int32), ("accumulate", ctypes.c_int32)]


class IdxPagedK(ctypes.Structure):
    """Mirror of idx_paged_k_t."""
    _fields_ = [("k_cache", ctypes.c_void_p), ("k_scale_cache", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("context_lens", ctypes.c_void_p), ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32)]


class IdxError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mqa_logits_scoring_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.idx_abi_version.restype = I32
        L.idx_abi_version.argtypes = []
        if L.idx_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.idx_abi_version()}, this binding {ABI_VERSION}: rebuild")
        L.idx_last_error.restype = ctypes.c_char_p
        L.idx_last_error.argtypes = []
        L.idx_logits_plan_bytes.restype = SZ
        L.idx_logits_plan_bytes.argtypes = [I32] * 5
        L.idx_logits_plan.restype = ctypes.c_int
        L.idx_logits_plan.argtypes = [I32] * 5 + [P, P, P, P, SZ, P]
        L.idx_logits_plan_thd.restype = ctypes.c_int
        L.idx_logits_plan_thd.argtypes = [I32, P, P] + [I32] * 5 + [P, SZ, P]
        L.idx_logits_plan_paged.restype = ctypes.c_int
        L.idx_logits_plan_paged.argtypes = [I32] * 5 + [P, P, SZ, P]
        L.idx_logits_prepare_paged.restype = ctypes.c_int
        L.idx_logits_prepare_paged.argtypes = [ctypes.POINTER(IdxLogitsArgs), ctypes.POINTER(IdxPagedK), P, SZ, P]
        L.idx_logits_run_paged.restype = ctypes.c_int
        L.idx_logits_run_paged.argtypes = [ctypes.POINTER(IdxLogitsArgs), ctypes.POINTER(IdxPagedK), P, P, SZ, P]
        L.idx_logits_score_paged.restype = ctypes.c_int
        L.idx_logits_score_paged.argtypes = [ctypes.POINTER(IdxLogitsArgs), ctypes.POINTER(IdxPagedK), P, P, SZ, P]
        L.idx_logits_topk.restype = ctypes.c_int
        L.idx_logits_topk.argtypes = [P] + [I32] * 5 + [P, ctypes.c_int, ctypes.c_int64, I32, ctypes.c_int, P, P, P]
        L.idx_logits_topk_workspace_bytes.restype = SZ
        L.idx_logits_topk_workspace_bytes.argtypes = [ctypes.POINTER(IdxLogitsArgs)]
        L.idx_logits_run_topk.restype = ctypes.c_int
        L.idx_logits_run_topk.argtypes = [ctypes.POINTER(IdxLogitsArgs), P, P, P, P, I32, ctypes.c_int, P, P, P, P,
                                          SZ, P]
        L.idx_logits_workspace_bytes.restype = SZ
        L.idx_logits_workspace_bytes.argtypes = [ctypes.POINTER(IdxLogitsArgs)]
        L.idx_logits_workspace_bytes_planned.restype = SZ
        L.idx_logits_workspace_bytes_planned.argtypes = [ctypes.POINTER(IdxLogitsArgs)]
        L.idx_logits_run.restype = ctypes.c_int
        L.idx_logits_run.argtypes = [ctypes.POINTER(IdxLogitsArgs), P, P, P, P, P, SZ, P]
        L.idx_logits_run_noalloc.restype = ctypes.c_int
        L.idx_logits_run_noalloc.argtypes = [ctypes.POINTER(IdxLogitsArgs), P, P, P, P, P]
        L.idx_logits_noalloc_scratch_bytes.restype = SZ
        L.idx_logits_noalloc_scratch_bytes.argtypes = []
        L.idx_logits_prepare.restype = ctypes.c_int
        L.idx_logits_prepare.argtypes = [ctypes.POINTER(IdxLogitsArgs), P, SZ, P]
        L.idx_logits_score.restype = ctypes.c_int
        L.idx_logits_score.argtypes = [ctypes.POINTER(IdxLogitsArgs), P, P, SZ, P]
        L.idx_logits_plan_windows.restype = ctypes.c_int
        L.idx_logits_plan_windows.argtypes = [P] + [I32] * 5 + [P, P, P]
        _lib = L
    return _lib


def idx_last_error() -> str:
    return lib().idx_last_error().decode()


def idx_abi_version() -> int:
    return int(lib().idx_abi_version())


def _check(fn: str, status: int):
    if status != IDX_OK:
        raise IdxError(fn, status, idx_last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev_i32(x, device) -> Optional[torch.Tensor]:
    if x is None:
        return None
    t = torch.as_tensor(x, dtype=torch.int32, device=device)
    return t.contiguous()


def idx_logits_plan_bytes(B: int, S_q: int, S_k: int, H: int = 64, D: int = 128) -> int:
    return int(lib().idx_logits_plan_bytes(B, S_q, S_k, H, D))


def idx_logits_plan(B: int, S_q: int, S_k: int, H: int = 64, D: int = 128, *, q_causal_offsets=None,
                    row_starts=None, row_ends=None, plan: Optional[torch.Tensor] = None, device=None,
                    stream=None) -> torch.Tensor:
    """Build a plan (windows + schedule) on the stream; returns the uint8 plan tensor."""
    device = torch.device(device if device is not None else (plan.device if plan is not None else "cuda"))
    nbytes = idx_logits_plan_bytes(B, S_q, S_k, H, D)
    if plan is None:
        plan = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    offs = _dev_i32(q_causal_offsets, device)
    st = _dev_i32(row_starts, device)
    en = _dev_i32(row_ends, device)
    _check("idx_logits_plan", lib().idx_logits_plan(B, S_q, S_k, H, D, _ptr(offs), _ptr(st), _ptr(en), _ptr(plan),
                                                      plan.numel() * plan.element_size(), _stream(stream, device)))
    plan._idx_keep = (offs, st, en)  # keep the window inputs alive until the stream has used them
    return plan


def idx_logits_plan_thd(cu_seqlens_q, cu_seqlens_k, ratio: int, T_q: int, m_total: int, H: int = 64,
                        D: int = 128, *, plan: Optional[torch.Tensor] = None, device=None,
                        stream=None) -> torch.Tensor:
    """Plan for packed variable-length rows over ratio-compressed keys (B = 1,
    S_q = T_q, S_k = m_total); returns the uint8 plan tensor."""
    device = torch.device(device if device is not None else (plan.device if plan is not None else "cuda"))
    nbytes = idx_logits_plan_bytes(1, T_q, m_total, H, D)
    if plan is None:
        plan = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    cq = _dev_i32(cu_seqlens_q, device)
    ck = _dev_i32(cu_seqlens_k, device)
    if cq is None or ck is None or cq.numel() != ck.numel() or cq.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need n_seg + 1 >= 2 entries each")
    _check("idx_logits_plan_thd", lib().idx_logits_plan_thd(cq.numel() - 1, _ptr(cq), _ptr(ck), int(ratio), T_q,
                                                              m_total, H, D, _ptr(plan),
                                                              plan.numel() * plan.element_size(),
                                                              _stream(stream, device)))
    plan._idx_keep = (cq, ck)
    return plan


def idx_logits_plan_windows(plan: torch.Tensor, B: int, S_q: int, S_k: int, H: int = 64, D: int = 128,
                            stream=None):
    """The per-row windows stored in a plan, as int32 [B, S_q] device tensors (start, end)."""
    ws = torch.empty((B, S_q), dtype=torch.int32, device=plan.device)
    we = torch.empty((B, S_q), dtype=torch.int32, device=plan.device)
    _check("idx_logits_plan_windows", lib().idx_logits_plan_windows(_ptr(plan), B, S_q, S_k, H, D, _ptr(ws),
                                                                      _ptr(we), _stream(stream, plan.device)))
    return ws, we


def _shape_info(q: torch.Tensor, k: torch.Tensor, in_dtype: str):
    if q.dim() == 3:
        q = q.unsqueeze(0)
    if k.dim() == 2:
        k = k.unsqueeze(0)
    if q.dim() != 4 or k.dim() != 3:
        raise ValueError("q must be [B,S_q,H,D'] or [S_q,H,D']; k [B,S_k,D'] or [S_k,D']")
    B, S_q, H, Dq = q.shape
    D = Dq * 2 if in_dtype == "mxfp4" else Dq
    return q, k, B, S_q, k.shape[1], H, D


def make_args(q: torch.Tensor, k: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor], *, in_dtype: str,
              q_scale=None, k_scale=None, sm_scale: float = 1.0, clean_logits: bool = True,
              accumulate: str = "native", out_dtype: Optional[torch.dtype] = None) -> IdxLogitsArgs:
    """Fill an idx_logits_args_t from tensors (no copies, no checks beyond
    shapes).  out may be None (fused top-k calls): out_dtype then gives the
    precision the scores are ranked in."""
    q4, k3, B, S_q, S_k, H, D = _shape_info(q, k, in_dtype)
    if out is not None:
        out_dtype = out.dtype
    if out_dtype not in FP_DTYPES or w.dtype not in FP_DTYPES:
        raise ValueError("w and out must be float32 or bfloat16")
    a = IdxLogitsArgs()
    a.B, a.S_q, a.S_k, a.H, a.D = B, S_q, S_k, H, D
    a.in_dtype = IN_DTYPES[in_dtype]
    a.q, a.k, a.w, a.out = _ptr(q), _ptr(k), _ptr(w), _ptr(out)
    a.q_scale, a.k_scale = _ptr(q_scale), _ptr(k_scale)
    a.w_dtype = FP_DTYPES[w.dtype]
    a.out_dtype = FP_DTYPES[out_dtype]
    a.sm_scale = float(sm_scale)
    a.out_row_stride = S_k if out is None else (out.stride(-2) if out.dim() >= 2 else S_k)
    a.clean_logits = 1 if clean_logits else 0
    a.accumulate = ACCUM[accumulate]
    return a


def idx_logits_workspace_bytes(args: IdxLogitsArgs) -> int:
    return int(lib().idx_logits_workspace_bytes(ctypes.byref(args)))


def idx_logits_workspace_bytes_planned(args: IdxLogitsArgs) -> int:
    return int(lib().idx_logits_workspace_bytes_planned(ctypes.byref(args)))


def idx_logits_run(q: torch.Tensor, k: torch.Tensor, w: torch.Tensor, *, in_dtype: str, q_scale=None,
                   k_scale=None, sm_scale: float = 1.0, clean_logits: bool = True,
                   out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.float32,
                   plan: Optional[torch.Tensor] = None, q_causal_offsets=None, row_starts=None, row_ends=None,
                   workspace: Optional[torch.Tensor] = None, accumulate: str = "native",
                   stream=None) -> torch.Tensor:
    """Score q against k on the stream; returns `out` ([B,S_q,S_k] or the caller's buffer).

    Tensors are passed as raw device buffers: q/k of any 1- or 2-byte dtype
    holding the codes (bf16 bits, e4m3 bytes, packed e2m1 bytes), scales as
    int32 (MX) or float32 (FP8 rows), w as float32 or bfloat16.  All must be
    contiguous; `out` may have a row stride larger than S_k."""
    for name, t in (("q", q), ("k", k), ("w", w), ("q_scale", q_scale), ("k_scale", k_scale)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    q4, k3, B, S_q, S_k, H, D = _shape_info(q, k, in_dtype)
    device = q.device
    if out is None:
        shape = (B, S_q, S_k) if q.dim() == 4 else (S_q, S_k)
        out = torch.empty(shape, dtype=out_dtype, device=device)
    args = make_args(q, k, w, out, in_dtype=in_dtype, q_scale=q_scale, k_scale=k_scale, sm_scale=sm_scale,
                     clean_logits=clean_logits, accumulate=accumulate)
    offs = st = en = None
    if plan is None:
        offs = _dev_i32(q_causal_offsets, device)
        st = _dev_i32(row_starts, device)
        en = _dev_i32(row_ends, device)
    # the workspace holds the reordered K, the weighted-query pieces or the
    # converted Q, and the plan of a call that builds it
    if workspace is None:
        nbytes = idx_logits_workspace_bytes(args) if plan is None else idx_logits_workspace_bytes_planned(args)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("idx_logits_run", lib().idx_logits_run(ctypes.byref(args), _ptr(plan), _ptr(offs), _ptr(st), _ptr(en),
                                                    _ptr(workspace), ws_bytes, _stream(stream, device)))
    return out


def idx_logits_noalloc_scratch_bytes() -> int:
    return int(lib().idx_logits_noalloc_scratch_bytes())


def idx_logits_run_noalloc(q: torch.Tensor, k: torch.Tensor, w: torch.Tensor, out: torch.Tensor, *, in_dtype: str,
                           q_scale=None, k_scale=None, sm_scale: float = 1.0, clean_logits: bool = True,
                           plan: Optional[torch.Tensor] = None, q_causal_offsets: Optional[torch.Tensor] = None,
                           row_starts: Optional[torch.Tensor] = None, row_ends: Optional[torch.Tensor] = None,
                           accumulate: str = "native", stream=None) -> torch.Tensor:
    """idx_logits_run on the library's per-device scratch: allocates nothing,
    so `out` and the window arrays (int32 device tensors) must be given."""
    for name, t in (("q", q), ("k", k), ("w", w), ("q_scale", q_scale), ("k_scale", k_scale)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, t in (("q_causal_offsets", q_causal_offsets), ("row_starts", row_starts), ("row_ends", row_ends)):
        if t is not None and (t.dtype != torch.int32 or t.device != q.device or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 tensor on q's device")
    args = make_args(q, k, w, out, in_dtype=in_dtype, q_scale=q_scale, k_scale=k_scale, sm_scale=sm_scale,
                     clean_logits=clean_logits, accumulate=accumulate)
    _check("idx_logits_run_noalloc",
           lib().idx_logits_run_noalloc(ctypes.byref(args), _ptr(plan), _ptr(q_causal_offsets), _ptr(row_starts),
                                        _ptr(row_ends), _stream(stream, q.device)))
    return out


def _workspace_for(args: IdxLogitsArgs, workspace: Optional[torch.Tensor], device, planned: bool = True):
    if workspace is None:
        nbytes = idx_logits_workspace_bytes_planned(args) if planned else idx_logits_workspace_bytes(args)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    return workspace


def idx_logits_prepare(args: IdxLogitsArgs, workspace: Optional[torch.Tensor] = None, *, device=None,
                       stream=None) -> torch.Tensor:
    """First phase of idx_logits_run: fill a workspace for `args` (made by
    make_args, whose tensors must stay alive); returns the workspace."""
    device = torch.device(device if device is not None else (workspace.device if workspace is not None else "cuda"))
    workspace = _workspace_for(args, workspace, device)
    _check("idx_logits_prepare", lib().idx_logits_prepare(ctypes.byref(args), _ptr(workspace),
                                                            workspace.numel() * workspace.element_size(),
                                                            _stream(stream, device)))
    return workspace


def idx_logits_score(args: IdxLogitsArgs, plan: torch.Tensor, workspace: torch.Tensor, *, stream=None) -> None:
    """Second phase of idx_logits_run: score into args.out from a workspace
    that idx_logits_prepare filled for the same inputs."""
    _check("idx_logits_score", lib().idx_logits_score(ctypes.byref(args), _ptr(plan), _ptr(workspace),
                                                        workspace.numel() * workspace.element_size(),
                                                        _stream(stream, workspace.device)))


def make_paged_k(k_cache: torch.Tensor, block_table: torch.Tensor, context_lens: torch.Tensor,
                 k_scale_cache: Optional[torch.Tensor] = None) -> IdxPagedK:
    """Fill an idx_paged_k_t from device tensors: k_cache [num_pages, page_size,
    row], block_table int32 [B, max_pages], context_lens int32 [B], k_scale_cache
    [num_pages, page_size] (FP8 / MX).  The tensors must outlive the calls."""
    for name, t in (("k_cache", k_cache), ("block_table", block_table), ("context_lens", context_lens),
                    ("k_scale_cache", k_scale_cache)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if block_table.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_table and context_lens must be int32")
    kv = IdxPagedK()
    kv.k_cache, kv.k_scale_cache = _ptr(k_cache), _ptr(k_scale_cache)
    kv.block_table, kv.context_lens = _ptr(block_table), _ptr(context_lens)
    kv.num_pages, kv.page_size = k_cache.shape[0], k_cache.shape[1]
    kv.max_pages = block_table.shape[1]
    return kv


def idx_logits_plan_paged(B: int, S_q: int, S_k: int, context_lens: torch.Tensor, H: int = 64, D: int = 128, *,
                          plan: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Plan for paged calls (windows from the context lengths)."""
    device = context_lens.device
    nbytes = idx_logits_plan_bytes(B, S_q, S_k, H, D)
    if plan is None:
        plan = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    ctx = _dev_i32(context_lens, device)
    _check("idx_logits_plan_paged", lib().idx_logits_plan_paged(B, S_q, S_k, H, D, _ptr(ctx), _ptr(plan),
                                                                  plan.numel() * plan.element_size(),
                                                                  _stream(stream, device)))
    plan._idx_keep = (ctx,)
    return plan


def make_paged_args(q: torch.Tensor, w: torch.Tensor, out: torch.Tensor, S_k: int, *, in_dtype: str, q_scale=None,
                    sm_scale: float = 1.0, clean_logits: bool = True, accumulate: str = "native") -> IdxLogitsArgs:
    """idx_logits_args_t of a paged call: q [B, S_q, H, D'], out [B, S_q, >= S_k];
    k and k_scale stay NULL (the keys come from an IdxPagedK)."""
    if q.dim() != 4:
        raise ValueError("q must be [B, S_q, H, D']")
    if out.dtype not in FP_DTYPES or w.dtype not in FP_DTYPES:
        raise ValueError("w and out must be float32 or bfloat16")
    for name, t in (("q", q), ("w", w), ("q_scale", q_scale)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, S_q, H, Dq = q.shape
    a = IdxLogitsArgs()
    a.B, a.S_q, a.S_k, a.H = B, S_q, S_k, H
    a.D = Dq * 2 if in_dtype == "mxfp4" else Dq
    a.in_dtype = IN_DTYPES[in_dtype]
    a.q, a.w, a.out, a.q_scale = _ptr(q), _ptr(w), _ptr(out), _ptr(q_scale)
    a.k = a.k_scale = None
    a.w_dtype, a.out_dtype = FP_DTYPES[w.dtype], FP_DTYPES[out.dtype]
    a.sm_scale = float(sm_scale)
    a.out_row_stride = out.stride(-2)
    a.clean_logits = 1 if clean_logits else 0
    a.accumulate = ACCUM[accumulate]
    return a


def idx_logits_prepare_paged(args: IdxLogitsArgs, kv: IdxPagedK, workspace: Optional[torch.Tensor] = None, *,
                             device=None, stream=None) -> torch.Tensor:
    """idx_logits_prepare for a paged call (args from make_paged_args, kv from
    make_paged_k); returns the workspace, which idx_logits_score then reads."""
    device = torch.device(device if device is not None else (workspace.device if workspace is not None else "cuda"))
    workspace = _workspace_for(args, workspace, device)
    _check("idx_logits_prepare_paged",
           lib().idx_logits_prepare_paged(ctypes.byref(args), ctypes.byref(kv), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream(stream, device)))
    return workspace


def idx_logits_run_paged(q: torch.Tensor, w: torch.Tensor, kv: IdxPagedK, S_k: int, *, in_dtype: str,
                         q_scale=None, sm_scale: float = 1.0, clean_logits: bool = True,
                         out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.float32,
                         plan: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         accumulate: str = "native", stream=None) -> torch.Tensor:
    """One paged call: q [B, S_q, H, D'] (the S_q newest tokens of each request),
    keys from `kv` (make_paged_k), output [B, S_q, S_k]."""
    if q.dim() != 4:
        raise ValueError("q must be [B, S_q, H, D']")
    device = q.device
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], S_k), dtype=out_dtype, device=device)
    a = make_paged_args(q, w, out, S_k, in_dtype=in_dtype, q_scale=q_scale, sm_scale=sm_scale,
                        clean_logits=clean_logits, accumulate=accumulate)
    workspace = _workspace_for(a, workspace, device, planned=plan is not None)
    _check("idx_logits_run_paged", lib().idx_logits_run_paged(ctypes.byref(a), ctypes.byref(kv), _ptr(plan),
                                                                _ptr(workspace),
                                                                workspace.numel() * workspace.element_size(),
                                                                _stream(stream, device)))
    return out


def idx_logits_score_paged(args: IdxLogitsArgs, kv: IdxPagedK, plan: torch.Tensor, workspace: torch.Tensor, *,
                           stream=None) -> None:
    """Second phase of a paged call: score into args.out from a workspace that
    idx_logits_prepare_paged filled for the same args and kv."""
    _check("idx_logits_score_paged",
           lib().idx_logits_score_paged(ctypes.byref(args), ctypes.byref(kv), _ptr(plan), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream, workspace.device)))


MAX_TOPK = 2048


TOPK_ORDERS = {"column": 0, "score": 1}


def idx_logits_topk(plan: torch.Tensor, logits: torch.Tensor, k: int, *, order: str = "column",
                    B: Optional[int] = None, H: int = 64, D: int = 128, S_k: Optional[int] = None,
                    with_values: bool = True, out_idx: Optional[torch.Tensor] = None,
                    out_val: Optional[torch.Tensor] = None, stream=None):
    """Top-k columns of every row's window in `logits` ([B, S_q, ld] or
    [S_q, ld], float32 or bfloat16, rows contiguous), from the plan the scores
    were made with, listed by ascending column (order="column") or in rank
    order (order="score").  Returns (idx int32 [..., S_q, k], val float32 or
    None)."""
    if logits.dtype not in FP_DTYPES:
        raise ValueError("logits must be float32 or bfloat16")
    if logits.stride(-1) != 1:
        raise ValueError("logits rows must be contiguous")
    lead = tuple(logits.shape[:-1])
    S_q = logits.shape[-2]
    if B is None:
        B = logits.shape[0] if logits.dim() == 3 else 1
    if logits.dim() == 3 and logits.stride(0) != S_q * logits.stride(-2):
        raise ValueError("logits batches must be packed at S_q * row stride")
    if S_k is None:
        S_k = logits.shape[-1]
    device = logits.device
    if out_idx is None:
        out_idx = torch.empty(lead + (k,), dtype=torch.int32, device=device)
    if with_values and out_val is None:
        out_val = torch.empty(lead + (k,), dtype=torch.float32, device=device)
    _check("idx_logits_topk", lib().idx_logits_topk(_ptr(plan), B, S_q, S_k, H, D, _ptr(logits),
                                                      FP_DTYPES[logits.dtype], logits.stride(-2), k,
                                                      TOPK_ORDERS[order], _ptr(out_idx),
                                                      _ptr(out_val) if with_values else None,
                                                      _stream(stream, device)))
    return out_idx, (out_val if with_values else None)


def idx_logits_topk_workspace_bytes(args: IdxLogitsArgs) -> int:
    return int(lib().idx_logits_topk_workspace_bytes(ctypes.byref(args)))


def idx_logits_run_topk(q: torch.Tensor, k: torch.Tensor, w: torch.Tensor, topk: int, *, in_dtype: str,
                        q_scale=None, k_scale=None, sm_scale: float = 1.0, out_dtype: torch.dtype = torch.float32,
                        order: str = "column", plan: Optional[torch.Tensor] = None, q_causal_offsets=None,
                        row_starts=None, row_ends=None, workspace: Optional[torch.Tensor] = None,
                        accumulate: str = "native", with_values: bool = True, out_idx: Optional[torch.Tensor] = None,
                        out_val: Optional[torch.Tensor] = None, n_redo: Optional[torch.Tensor] = None, stream=None):
    """Scoring and top-`topk` selection in one call, without the score
    matrix: the result of idx_logits_run (scores in out_dtype) followed by
    idx_logits_topk.  Returns (idx int32 [..., S_q, topk], val float32 or
    None); n_redo, an int32 device tensor of one element, receives the number
    of rows scored twice."""
    for name, t in (("q", q), ("k", k), ("w", w), ("q_scale", q_scale), ("k_scale", k_scale)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    q4, k3, B, S_q, S_k, H, D = _shape_info(q, k, in_dtype)
    device = q.device
    args = make_args(q, k, w, None, in_dtype=in_dtype, q_scale=q_scale, k_scale=k_scale, sm_scale=sm_scale,
                     clean_logits=False, accumulate=accumulate, out_dtype=out_dtype)
    lead = (B, S_q) if q.dim() == 4 else (S_q,)
    if out_idx is None:
        out_idx = torch.empty(lead + (topk,), dtype=torch.int32, device=device)
    if with_values and out_val is None:
        out_val = torch.empty(lead + (topk,), dtype=torch.float32, device=device)
    offs = st = en = None
    if plan is None:
        offs = _dev_i32(q_causal_offsets, device)
        st = _dev_i32(row_starts, device)
        en = _dev_i32(row_ends, device)
    if workspace is None:
        workspace = torch.empty(max(idx_logits_topk_workspace_bytes(args), 1), dtype=torch.uint8, device=device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("idx_logits_run_topk",
           lib().idx_logits_run_topk(ctypes.byref(args), _ptr(plan), _ptr(offs), _ptr(st), _ptr(en), int(topk),
                                     TOPK_ORDERS[order], _ptr(out_idx), _ptr(out_val) if with_values else None,
                                     _ptr(n_redo), _ptr(workspace), ws_bytes, _stream(stream, device)))
    return out_idx, (out_val if with_values else None)
