"""Helpers for the GPU tests: move a workload to the device, run the library
through its binding (which calls the C ABI), and compare with the oracle."""

from __future__ import annotations

import numpy as np
import torch

import mqa_logits_scoring_amd as lib
import oracle

DEV = "cuda"


def _codes(a, device):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16 if a.dtype == np.uint16 else np.uint8)).to(device)


def _scales(a, device):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a if a.dtype == np.float32 else a.view(np.int32)).to(device)


def dev_inputs(wl, device=DEV) -> dict:
    """Raw code buffers of a workload as device tensors."""
    d = {}
    d["q"] = torch.from_numpy(np.ascontiguousarray(wl.q).view(np.int16 if wl.q.dtype == np.uint16 else np.uint8)).to(device)
    d["k"] = _codes(wl.k, device)
    d["q_scale"] = None if wl.q_scale is None else torch.from_numpy(wl.q_scale.view(np.int32)).to(device)
    d["k_scale"] = _scales(wl.k_scale, device)
    if wl.w_dtype == "bf16":
        d["w"] = torch.from_numpy(wl.w.view(np.int16)).view(torch.bfloat16).to(device)
    else:
        d["w"] = torch.from_numpy(wl.w).to(device)
    d["offsets"] = None if wl.offsets is None else torch.from_numpy(np.asarray(wl.offsets, np.int32)).to(device)
    d["starts"] = None if wl.starts is None else torch.from_numpy(np.asarray(wl.starts, np.int32)).to(device)
    d["ends"] = None if wl.ends is None else torch.from_numpy(np.asarray(wl.ends, np.int32)).to(device)
    if getattr(wl, "paged", None) is not None:
        pg = wl.paged
        d["k_cache"] = _codes(pg["k_cache"], device)
        d["k_scale_cache"] = _scales(pg["k_scale_cache"], device)
        d["block_table"] = torch.from_numpy(np.ascontiguousarray(pg["block_table"], np.int32)).to(device)
        d["ctx"] = torch.from_numpy(np.ascontiguousarray(pg["ctx"], np.int32)).to(device)
        d["kv"] = lib.make_paged_k(d["k_cache"], d["block_table"], d["ctx"], d["k_scale_cache"])
    if getattr(wl, "thd", None) is not None:
        d["cu_q"] = torch.from_numpy(np.asarray(wl.thd["cu_q"], np.int32)).to(device)
        d["cu_k"] = torch.from_numpy(np.asarray(wl.thd["cu_k"], np.int32)).to(device)
    return d


def out_dtype(wl):
    return torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32


def make_plan(wl, d):
    if getattr(wl, "paged", None) is not None:
        return lib.idx_logits_plan_paged(wl.B, wl.S_q, wl.S_k, d["ctx"], wl.H, wl.D)
    if getattr(wl, "thd", None) is not None:
        return lib.idx_logits_plan_thd(d["cu_q"], d["cu_k"], wl.thd["ratio"], wl.S_q, wl.S_k, wl.H, wl.D,
                                       device=d["q"].device)
    return lib.idx_logits_plan(wl.B, wl.S_q, wl.S_k, wl.H, wl.D, q_causal_offsets=d["offsets"],
                               row_starts=d["starts"], row_ends=d["ends"], device=d["q"].device)


def run(wl, d, plan=None, out=None, clean=None, accumulate="native"):
    """One library call; plan None builds the plan inside the call (packed
    variable-length workloads build theirs with idx_logits_plan_thd first;
    paged workloads go through idx_logits_run_paged)."""
    if plan is None and getattr(wl, "thd", None) is not None:
        plan = make_plan(wl, d)
    if getattr(wl, "paged", None) is not None:
        return lib.idx_logits_run_paged(d["q"], d["w"], d["kv"], wl.S_k, in_dtype=wl.fmt, q_scale=d["q_scale"],
                                        sm_scale=wl.sm_scale, clean_logits=wl.clean if clean is None else clean,
                                        out=out, out_dtype=out_dtype(wl), plan=plan, accumulate=accumulate)
    return lib.idx_logits_run(d["q"], d["k"], d["w"], in_dtype=wl.fmt, q_scale=d["q_scale"], k_scale=d["k_scale"],
                              sm_scale=wl.sm_scale, clean_logits=wl.clean if clean is None else clean, out=out,
                              out_dtype=out_dtype(wl), plan=plan, q_causal_offsets=d["offsets"],
                              row_starts=d["starts"], row_ends=d["ends"], accumulate=accumulate)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 7), 0.0)


def compare_rows(wl, got: np.ndarray, ref: np.ndarray, bound: np.ndarray, clean: bool = True, what: str = "",
                 rel_tol: float = 1e-4):
    """got/ref/bound: [n_rows, S_k].  -inf placement bit-exact, values within
    rel_tol * bound (the stated 1e-4 unless a test says why not; + one bf16
    ulp of the reference for bf16 output).  Returns (max err / bound,
    rel-L2)."""
    inside = ~np.isneginf(ref)
    assert not np.any(np.isnan(got[inside])), f"{what}: NaN inside windows"
    if clean:
        bad = np.isneginf(got) != ~inside
        assert not np.any(bad), f"{what}: -inf placement differs at {np.argwhere(bad)[:5].tolist()}"
    tol = rel_tol * bound[inside]
    if wl.out_dtype == "bf16":
        tol = tol + bf16_ulp(ref[inside])
    err = np.abs(got[inside] - ref[inside])
    worst = np.argmax(err - tol) if err.size else 0
    assert np.all(err <= tol), (f"{what}: |err| {err[worst]:.3e} > tol {tol[worst]:.3e} "
                                f"(ref {ref[inside][worst]:.6e} got {got[inside][worst]:.6e})")
    ratio = float(np.max(err / np.maximum(bound[inside], 1e-300))) if err.size else 0.0
    den = float(np.sqrt(np.sum(ref[inside] ** 2)))
    rel_l2 = float(np.sqrt(np.sum(err ** 2)) / den) if den > 0 else 0.0
    return ratio, rel_l2


def mask_check_all_rows(wl, out: torch.Tensor, plan_ws=None):
    """-inf placement over every row, on the device: cell is -inf <=> outside the oracle's window."""
    ws, we = oracle.windows(wl)
    ws_t = torch.from_numpy(ws.reshape(-1)).to(out.device)
    we_t = torch.from_numpy(we.reshape(-1)).to(out.device)
    o = out.reshape(wl.B * wl.S_q, -1)[:, : wl.S_k]
    cols = torch.arange(wl.S_k, device=out.device)
    step = max(1, (1 << 26) // wl.S_k)
    for r0 in range(0, wl.B * wl.S_q, step):
        r1 = min(r0 + step, wl.B * wl.S_q)
        inside = (cols[None, :] >= ws_t[r0:r1, None]) & (cols[None, :] < we_t[r0:r1, None])
        ninf = torch.isneginf(o[r0:r1])
        bad = ninf == inside
        if bool(bad.any()):
            idx = torch.nonzero(bad)[:5].cpu().tolist()
            raise AssertionError(f"-inf placement wrong at rows/cols {[(r0 + a, b) for a, b in idx]}")
        assert not bool(torch.isnan(o[r0:r1]).any()), "NaN in output"


def sample_rows(wl, n_random: int = 12, seed: int = 0) -> np.ndarray:
    """Rows for value checks: ends and tile edges of every batch, empty rows, a few random ones."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(wl.B):
        base = b * wl.S_q
        for i in (0, 1, 7, 8, 9, wl.S_q // 2, wl.S_q - 9, wl.S_q - 8, wl.S_q - 2, wl.S_q - 1):
            if 0 <= i < wl.S_q:
                rows.add(base + i)
    ws, we = oracle.windows(wl)
    empt = np.argwhere((we <= ws).reshape(-1)).ravel()
    rows.update(int(x) for x in empt[:8])
    rows.update(int(x) for x in rng.integers(0, wl.B * wl.S_q, size=n_random))
    return np.array(sorted(rows), np.int64)


def inside_check_all_rows(wl, out: torch.Tensor):
    """Every in-window cell of every row holds a number (no NaN, no -inf): with
    the output pre-filled with NaN, a cell no unit wrote fails here."""
    ws, we = oracle.windows(wl)
    ws_t = torch.from_numpy(ws.reshape(-1)).to(out.device)
    we_t = torch.from_numpy(we.reshape(-1)).to(out.device)
    o = out.reshape(wl.B * wl.S_q, -1)[:, : wl.S_k]
    cols = torch.arange(wl.S_k, device=out.device)
    step = max(1, (1 << 26) // wl.S_k)
    for r0 in range(0, wl.B * wl.S_q, step):
        r1 = min(r0 + step, wl.B * wl.S_q)
        inside = (cols[None, :] >= ws_t[r0:r1, None]) & (cols[None, :] < we_t[r0:r1, None])
        bad = inside & ~torch.isfinite(o[r0:r1].float())
        if bool(bad.any()):
            idx = torch.nonzero(bad)[:5].cpu().tolist()
            raise AssertionError(f"in-window cell not written at rows/cols {[(r0 + a, b) for a, b in idx]}")


def compare_all_rows(wl, out: torch.Tensor, clean: bool = True, what: str = "", chunk: int = 256,
                     rel_tol: float = 1e-4):
    """Every cell of every row against the oracle, a chunk of rows at a time
    (bounded host memory at full size).  Returns (max err / bound, rel-L2)."""
    n = wl.B * wl.S_q
    o = out.reshape(n, -1)
    worst, num, den = 0.0, 0.0, 0.0
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(r0 + chunk, n), dtype=np.int64)
        ref, bound = oracle.logits(wl, rows=rows)
        got = to_f64(o[r0:r0 + rows.size, : wl.S_k])
        ratio, rel = compare_rows(wl, got, ref, bound, clean=clean, what=f"{what} rows {r0}..", rel_tol=rel_tol)
        worst = max(worst, ratio)
        inside = ~np.isneginf(ref)
        num += float(np.sum((got[inside] - ref[inside]) ** 2))
        den += float(np.sum(ref[inside] ** 2))
    return worst, (float(np.sqrt(num / den)) if den > 0 else 0.0)
