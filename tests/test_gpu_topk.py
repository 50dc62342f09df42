"""GPU top-k selection against the oracle's ranking.

The selection is integer work on given scores, so both sides rank the very
same fp32 (or bf16) scores: the ones the GPU wrote.  Indices and listed
scores must agree bit for bit.  The scores themselves are checked against the
fp64 oracle by the parity tests."""

import numpy as np
import pytest
import torch

import mqa_logits_scoring_amd as lib
import oracle
import workloads as W
from gpu_util import dev_inputs, make_plan, run

pytestmark = pytest.mark.gpu


def _check(plan, logits, k, ws, we, what, B=None, H=64, S_k=None, orders=("column", "score")):
    for order in orders:
        got = _check_one(plan, logits, k, ws, we, f"{what} by {order}", B, H, S_k, order)
    return got


def _check_one(plan, logits, k, ws, we, what, B, H, S_k, order):
    idx, val = lib.idx_logits_topk(plan, logits, k, order=order, B=B, H=H, S_k=S_k)
    torch.cuda.synchronize()
    S_k = logits.shape[-1] if S_k is None else S_k
    flat = logits.reshape(-1, logits.shape[-1])[:, :S_k]
    host = flat.view(torch.int16).cpu().numpy().view(np.uint16) if flat.dtype == torch.bfloat16 else flat.cpu().numpy()
    want_idx, want_val = oracle.topk(host, np.asarray(ws).reshape(-1), np.asarray(we).reshape(-1), k,
                                     by_column=order == "column")
    got_idx = idx.reshape(-1, k).cpu().numpy()
    got_val = val.reshape(-1, k).cpu().numpy()
    bad = np.argwhere(got_idx != want_idx)
    assert bad.size == 0, f"{what}: indices differ first at (row, rank) {bad[:3].tolist()}: " \
                          f"got {got_idx[tuple(bad[0])]} want {want_idx[tuple(bad[0])]}"
    nan = np.isnan(want_val)
    assert np.array_equal(np.isnan(got_val), nan), what
    assert np.array_equal(got_val[~nan].view(np.uint32), want_val[~nan].view(np.uint32)), f"{what}: scores differ"
    return got_idx


def _windows_plan(B, S_q, S_k, starts, ends, H=64):
    return lib.idx_logits_plan(B, S_q, S_k, H, 128, row_starts=torch.from_numpy(starts.astype(np.int32)).cuda(),
                               row_ends=torch.from_numpy(ends.astype(np.int32)).cuda(), device="cuda")


# ---------------------------------------------------------------------------
# scores made by the scoring kernels
# ---------------------------------------------------------------------------

SCORED = [
    ("bf16", dict(B=2, S_q=70, S_k=3000, offsets=[0, -900]), 64),
    ("mxfp8", dict(B=1, S_q=130, S_k=5000, windows="irregular"), 2048),
    ("mxfp4", dict(B=1, S_q=33, S_k=9000, windows="irregular", out_dtype="bf16", w_dtype="bf16"), 512),
    ("fp8", dict(B=3, S_q=17, S_k=40000, offsets=[0, -1, -39000]), 2048),   # rows past one 32768-column chunk
]


@pytest.mark.parametrize("fmt,kw,k", SCORED, ids=[f"{f}-k{k}" for f, _, k in SCORED])
def test_topk_of_scores(fmt, kw, k):
    kw = dict(kw)
    wl = W.make_random(fmt, kw.pop("B"), kw.pop("S_q"), kw.pop("S_k"), seed=71, **kw)
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    out = run(wl, d, plan=plan)
    ws, we = oracle.windows(wl)
    _check(plan, out, k, ws, we, f"{fmt} k={k}")
    # an unclean call leaves the cells outside the windows alone: same selection
    out2 = run(wl, d, plan=plan, clean=False, out=out.clone().fill_(float("nan")))
    _check(plan, out2, k, ws, we, f"{fmt} k={k} unclean")


def test_topk_full_size_c4():
    """Top-2048 of the MXFP8 Q2048/KV32768 call's scores (2048 rows of about 31k
    window columns), all rows."""
    wl = W.make("c4_mxfp8")
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    out = run(wl, d, plan=plan)
    ws, we = oracle.windows(wl)
    _check(plan, out, 2048, ws, we, "c4 top-2048")


# ---------------------------------------------------------------------------
# crafted scores: ties, signed zeros, NaN, -inf, windows of every size
# ---------------------------------------------------------------------------

def _crafted(rng, n_rows, S_k, kind):
    if kind == "ties":
        pool = np.array([-2.0, -0.0, 0.0, 0.5, 1.0, 3.0, -np.inf], np.float32)
        return pool[rng.integers(0, pool.size, size=(n_rows, S_k))]
    if kind == "nan":
        v = rng.standard_normal((n_rows, S_k)).astype(np.float32)
        v[rng.random(v.shape) < 0.2] = np.nan
        v[rng.random(v.shape) < 0.05] = -np.inf
        return v
    if kind == "mostly_nan":  # the sample's threshold lands on NaN's key: those rows go to the path from memory
        v = rng.standard_normal((n_rows, S_k)).astype(np.float32)
        v[rng.random(v.shape) < 0.97] = np.nan
        v[rng.random(v.shape) < 0.01] = -0.0
        return v
    if kind == "equal":
        return np.full((n_rows, S_k), 1.5, np.float32)
    return rng.standard_normal((n_rows, S_k)).astype(np.float32) * np.float32(1e-3)


CRAFTED = ["ties", "nan", "equal", "normal", "mostly_nan"]


@pytest.mark.parametrize("kind", CRAFTED)
@pytest.mark.parametrize("k", [1, 7, 300, 2048])
def test_topk_crafted(kind, k):
    rng = np.random.default_rng(CRAFTED.index(kind) * 10007 + k)
    B, S_q, S_k = 2, 9, 37000
    v = _crafted(rng, B * S_q, S_k, kind)
    starts = rng.integers(0, S_k, size=B * S_q)
    ends = np.minimum(S_k, starts + rng.integers(0, S_k, size=B * S_q))
    # edge rows: empty, one column, exactly k, k + 1, the whole row, the last column only
    starts[:6] = [5, 5, 100, 100, 0, S_k - 1]
    ends[:6] = [5, 6, 100 + k, 101 + k, S_k, S_k]
    plan = _windows_plan(B, S_q, S_k, starts, ends)
    ld = S_k + 3  # a row stride wider than S_k
    buf = np.full((B * S_q, ld), np.float32(7.0))  # the cells past S_k must never be picked
    buf[:, :S_k] = v
    logits = torch.from_numpy(buf).reshape(B, S_q, ld).cuda()
    _check(plan, logits, k, starts, ends, f"{kind} k={k}", S_k=S_k)
    # the same selection from bf16 scores (more ties)
    lb = logits.to(torch.bfloat16)
    _check(plan, lb, k, starts, ends, f"{kind} k={k} bf16", S_k=S_k)


@pytest.mark.parametrize("H", [8, 32])
def test_topk_other_head_counts(H):
    wl = W.make_random("mxfp8", 1, 150, 6000, H=H, seed=5, windows="irregular")
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    out = run(wl, d, plan=plan)
    ws, we = oracle.windows(wl)
    _check(plan, out, 1000, ws, we, f"H={H}", H=H)


def test_topk_without_values_and_plan_mismatch():
    rng = np.random.default_rng(3)
    v = torch.from_numpy(rng.standard_normal((1, 8, 500)).astype(np.float32)).cuda()
    starts, ends = np.zeros(8, np.int64), np.full(8, 500)
    plan = _windows_plan(1, 8, 500, starts, ends)
    idx, val = lib.idx_logits_topk(plan, v, 16, with_values=False)
    assert val is None
    want, _ = oracle.topk(v.reshape(8, 500).cpu().numpy(), starts, ends, 16, by_column=True)
    assert np.array_equal(idx.reshape(8, 16).cpu().numpy(), want)
    # a plan for other dimensions gives -1 / NaN everywhere, not a plausible list
    other = _windows_plan(1, 8, 400, starts, np.full(8, 400))
    idx, val = lib.idx_logits_topk(other, v, 16, S_k=500)
    torch.cuda.synchronize()
    assert bool((idx == -1).all()) and bool(torch.isnan(val).all())


@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_topk_window_sizes_around_the_stage(kind):
    """Windows on both sides of the sizes where the per-row selection changes
    method: staged whole (up to 4096 columns), thresholded from a sample (up
    to 65536), and selected from memory (wider, or many equal scores)."""
    rng = np.random.default_rng(17 + len(kind))
    S_k, k = 70000, 2048
    widths = [2049, 4095, 4096, 4097, 8192, 65535, 65536, 65537, 70000]
    n_rows = len(widths) + 3
    v = _crafted(rng, n_rows, S_k, kind)
    starts = np.zeros(n_rows, np.int64)
    ends = np.zeros(n_rows, np.int64)
    for i, wdt in enumerate(widths):
        starts[i] = rng.integers(0, S_k - wdt + 1)
        ends[i] = starts[i] + wdt
    starts[-3:], ends[-3:] = [1, 3, 0], [S_k - 2, S_k - 1, S_k]  # unaligned starts and ends
    plan = _windows_plan(1, n_rows, S_k, starts, ends)
    ld = S_k + 5
    buf = np.full((n_rows, ld), np.float32(9.0))
    buf[:, :S_k] = v
    logits = torch.from_numpy(buf).reshape(1, n_rows, ld).cuda()
    _check(plan, logits, k, starts, ends, f"{kind} widths", S_k=S_k, orders=("column",))
    _check(plan, logits.to(torch.bfloat16), k, starts, ends, f"{kind} widths bf16", S_k=S_k, orders=("column",))
