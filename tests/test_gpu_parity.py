"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, and
the exact relations the method fixes between GPU runs."""

import math

import json
import os

import numpy as np
import pytest
import torch

import mqa_logits_scoring_amd as lib
import oracle
import workloads as W
from gpu_util import (out_dtype, compare_all_rows, compare_rows, dev_inputs, inside_check_all_rows, make_plan,
                      mask_check_all_rows, run, sample_rows, to_f64)
import oracle_pins as P

pytestmark = pytest.mark.gpu


def _full_compare(wl, out, clean=True, what=""):
    ref, bound = oracle.logits(wl)
    got = to_f64(out).reshape(wl.B * wl.S_q, -1)[:, : wl.S_k]
    return compare_rows(wl, got, ref, bound, clean=clean, what=what or wl.name)


# ---------------------------------------------------------------------------
# plan: windows bit-exact against the oracle's window rules
# ---------------------------------------------------------------------------

WINDOW_CASES = [
    dict(B=1, S_q=128, S_k=512, offsets=[0]),
    dict(B=4, S_q=37, S_k=100, offsets=[0, -1, 5, -200]),
    dict(B=3, S_q=9, S_k=50, offsets=[2 ** 31 - 1, -2 ** 31, -49]),
    dict(B=2, S_q=21, S_k=300, windows="irregular"),
    dict(B=1, S_q=6, S_k=50, windows="explicit", starts=[[-5, 10, 60, 30, 7, 0]], ends=[[20, 70, 80, 10, 7, 50]]),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=[str(i) for i in range(len(WINDOW_CASES))])
def test_plan_windows_match_oracle(case):
    case = dict(case)
    wl = W.make_random("bf16", case.pop("B"), case.pop("S_q"), case.pop("S_k"), H=64, D=128, seed=3, **case)
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    ws, we = lib.idx_logits_plan_windows(plan, wl.B, wl.S_q, wl.S_k)
    ows, owe = oracle.windows(wl)
    assert np.array_equal(ws.cpu().numpy(), ows) and np.array_equal(we.cpu().numpy(), owe)


# ---------------------------------------------------------------------------
# small shapes, every format x weight type x output type x clean flag
# (3 tiles with a ragged tail, ragged key tails, irregular windows)
# ---------------------------------------------------------------------------

MATRIX = [(f, wd, od, cl) for f in W.FORMATS for wd in ("f32", "bf16") for od in ("f32", "bf16") for cl in (True, False)]


@pytest.mark.parametrize("fmt,w_dtype,o_dtype,clean", MATRIX, ids=["-".join(map(str, m)) for m in MATRIX])
def test_small_matrix(fmt, w_dtype, o_dtype, clean):
    wl = W.make_random(fmt, 2, 21, 300, w_dtype=w_dtype, out_dtype=o_dtype, sm_scale=0.3, clean=clean, seed=17,
                       windows="irregular")
    d = dev_inputs(wl)
    out = run(wl, d)
    torch.cuda.synchronize()
    _full_compare(wl, out, clean=clean)


@pytest.mark.parametrize("S_k", [1, 31, 32, 33, 63, 64, 65, 127, 129, 999, 4100])
@pytest.mark.parametrize("fmt", W.FORMATS)
def test_ragged_key_tails(fmt, S_k):
    """Windows reaching the last key column for S_k around the 32/64-column block edges."""
    wl = W.make_random(fmt, 1, 13, S_k, sm_scale=0.5, seed=S_k, offsets=[0])
    d = dev_inputs(wl)
    out = run(wl, d)
    torch.cuda.synchronize()
    _full_compare(wl, out)


@pytest.mark.parametrize("S_q", [3, 4, 5, 9, 12, 16])
@pytest.mark.parametrize("exact", [False, True], ids=["bf16", "fp8-exact"])
def test_half_tile_units_every_cell(S_q, exact):
    """BF16 operands (and FP8 converted to bf16 for exact accumulation) run
    one query row per wave, half a tile per workgroup: tiles whose second
    half is padding, partly padded, or full, over two batches, irregular
    windows, every cell against the oracle, and bitwise the same with the
    plan passed in and built inside."""
    wl = W.make_random("fp8" if exact else "bf16", 2, S_q, 1000, seed=60 + S_q, windows="irregular",
                       out_dtype="bf16" if S_q % 2 else "f32")
    d = dev_inputs(wl)
    acc = "fp32" if exact else "native"
    out = run(wl, d, accumulate=acc, out=torch.full((wl.B, wl.S_q, wl.S_k), float("nan"), device="cuda",
                                                     dtype=torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32))
    out2 = run(wl, d, plan=make_plan(wl, d), accumulate=acc)
    torch.cuda.synchronize()
    iv = torch.int16 if out.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(out.view(iv), out2.view(iv))
    _full_compare(wl, out)


def test_c1_full():
    wl = W.make("c1")
    d = dev_inputs(wl)
    out = run(wl, d)
    torch.cuda.synchronize()
    ratio, rel = _full_compare(wl, out)
    print(f"c1: max err/bound {ratio:.3e}, rel-L2 {rel:.3e}")


def test_c5_nonaligned_full():
    wl = W.make("c5_nonaligned")
    d = dev_inputs(wl)
    out = run(wl, d)
    torch.cuda.synchronize()
    ratio, rel = _full_compare(wl, out)
    print(f"c5 non-aligned: max err/bound {ratio:.3e}, rel-L2 {rel:.3e}")


# ---------------------------------------------------------------------------
# exact cases: small-integer codes and power-of-two weights make every
# intermediate exact in fp32, so the GPU must equal the oracle bitwise
# ---------------------------------------------------------------------------

class _Capture:
    """Stand-in oracle that records the workloads a pin builds and returns its real answers."""

    def __init__(self):
        self.real = oracle.default()
        self.seen = []

    def logits(self, wl, **kw):
        self.seen.append(wl)
        return self.real.logits(wl, **kw)

    def windows(self, wl):
        return self.real.windows(wl)

    def decode(self, f, c):
        return self.real.decode(f, c)


@pytest.mark.parametrize("pin", [P.pin_one_hot, P.pin_rank_one, P.pin_zero_workload], ids=lambda p: p.__name__)
def test_exact_cases_bitwise(pin):
    cap = _Capture()
    pin(cap)
    assert cap.seen
    for wl in cap.seen:
        ref, _ = oracle.logits(wl)
        d = dev_inputs(wl)
        out = run(wl, d)
        got = to_f64(out).reshape(wl.B * wl.S_q, -1)
        exact = ref.astype(np.float32).astype(np.float64) if wl.out_dtype == "f32" else None
        assert exact is not None
        same = (got == exact) | (np.isneginf(got) & np.isneginf(exact))
        assert np.all(same), f"{pin.__name__} {wl.fmt}: {np.argwhere(~same)[:5].tolist()} " \
                             f"got {got[~same][:5]} want {exact[~same][:5]}"


# ---------------------------------------------------------------------------
# exact relations between GPU runs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", W.FORMATS)
def test_determinism_and_plan_equivalence(fmt):
    wl = W.make_random(fmt, 2, 40, 700, seed=5, windows="irregular", w_dtype="bf16")
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    first = run(wl, d, plan=plan)
    for i in range(20):
        o = run(wl, d, plan=plan if i % 2 else None)
        assert torch.equal(o.view(torch.int32), first.view(torch.int32)), f"run {i} differs"


@pytest.mark.parametrize("fmt", W.FORMATS)
def test_prepare_then_score_equals_run(fmt):
    """The two-phase entry points give bitwise the output of idx_logits_run,
    and one prepared workspace serves several scoring calls (other output
    type, clean flag and sm_scale)."""
    wl = W.make_random(fmt, 2, 37, 650, seed=6, windows="irregular")
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    ref_f32 = run(wl.replace(out_dtype="f32"), d, plan=plan)
    ref_bf16 = run(wl.replace(out_dtype="bf16"), d, plan=plan)
    out_f32 = torch.full_like(ref_f32, 7.0)
    out_bf16 = torch.full_like(ref_bf16, 7.0)
    a32 = lib.make_args(d["q"], d["k"], d["w"], out_f32, in_dtype=fmt, q_scale=d["q_scale"], k_scale=d["k_scale"],
                        sm_scale=wl.sm_scale, clean_logits=True)
    ws = lib.idx_logits_prepare(a32, device=d["q"].device)
    lib.idx_logits_score(a32, plan, ws)
    a16 = lib.make_args(d["q"], d["k"], d["w"], out_bf16, in_dtype=fmt, q_scale=d["q_scale"], k_scale=d["k_scale"],
                        sm_scale=wl.sm_scale, clean_logits=True)
    lib.idx_logits_score(a16, plan, ws)
    assert torch.equal(out_f32.view(torch.int32), ref_f32.view(torch.int32))
    assert torch.equal(out_bf16.view(torch.int16), ref_bf16.view(torch.int16))
    # sm_scale is applied once at the end, so a power of two scales exactly
    a2 = lib.make_args(d["q"], d["k"], d["w"], out_f32, in_dtype=fmt, q_scale=d["q_scale"], k_scale=d["k_scale"],
                       sm_scale=wl.sm_scale * 2, clean_logits=False)
    lib.idx_logits_score(a2, plan, ws)
    fin = ~torch.isneginf(ref_f32)
    assert torch.equal(out_f32[fin], ref_f32[fin] * 2)
    assert bool(torch.isneginf(out_f32[~fin]).all()), "clean_logits=0 touched cells outside the windows"


@pytest.mark.parametrize("fmt", W.FORMATS)
def test_batch_invariance(fmt):
    wl = W.make_random(fmt, 3, 19, 260, seed=8, offsets=[0, -5, 3])
    d = dev_inputs(wl)
    out = run(wl, d)
    for b in range(3):
        sl = lambda a: None if a is None else a[b:b + 1]
        one = wl.replace(B=1, q=sl(wl.q), q_scale=sl(wl.q_scale), k=sl(wl.k), k_scale=sl(wl.k_scale), w=sl(wl.w),
                         offsets=wl.offsets[b:b + 1])
        o1 = run(one, dev_inputs(one))
        assert torch.equal(o1[0].view(torch.int32), out[b].view(torch.int32)), b


@pytest.mark.parametrize("fmt", W.FORMATS)
def test_w_bf16_equals_f32_holding_bf16(fmt):
    wl = W.make_random(fmt, 1, 16, 200, seed=9, w_dtype="bf16", offsets=[0])
    d = dev_inputs(wl)
    a = run(wl, d)
    d2 = dict(d, w=d["w"].float())
    b = run(wl.replace(w_dtype="f32"), d2)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("fmt", W.FORMATS)
def test_clean_and_unclean_agree_inside(fmt):
    wl = W.make_random(fmt, 1, 24, 500, seed=10, windows="irregular")
    d = dev_inputs(wl)
    a = run(wl, d, clean=True)
    sentinel = torch.full_like(a, 12345.0)
    b = run(wl, d, clean=False, out=sentinel)
    inside = ~torch.isneginf(a)
    assert torch.equal(a[inside], b[inside])
    assert bool((b[~inside] == 12345.0).all()), "clean_logits=0 touched cells outside the windows"


@pytest.mark.parametrize("fmt", W.FORMATS)
def test_weight_and_scale_doubling(fmt):
    wl = W.make_random(fmt, 1, 16, 300, seed=12, offsets=[0])
    d = dev_inputs(wl)
    base = run(wl, d)
    x4 = run(wl, dict(d, w=d["w"] * 4))
    fin = ~torch.isneginf(base)
    assert torch.equal(x4[fin], base[fin] * 4)
    if fmt in ("mxfp8", "mxfp4"):
        k2 = run(wl, dict(d, k_scale=d["k_scale"] + 0x01010101))
        assert torch.equal(k2[fin], base[fin] * 2)


def test_row_stride_guard_band():
    wl = W.make_random("mxfp8", 2, 11, 77, seed=13, offsets=[0, 4])
    d = dev_inputs(wl)
    buf = torch.full((wl.B, wl.S_q, 96), 777.0, device="cuda")
    run(wl, d, out=buf)
    assert bool((buf[..., 77:] == 777.0).all())
    ref = run(wl, d)
    assert torch.equal(buf[..., :77], ref)


@pytest.mark.parametrize("fmt", W.FORMATS)
def test_plan_dimension_mismatch_is_loud(fmt):
    """A plan of other dimensions fills every cell with NaN, whichever kernel
    (and whichever unit cleans a row) the call takes."""
    wl = W.make_random(fmt, 1, 16, 128, seed=14, offsets=[0])
    d = dev_inputs(wl)
    other = W.make_random(fmt, 1, 16, 256, seed=14, offsets=[0])
    plan = make_plan(other, dev_inputs(other))
    out = run(wl, d, plan=plan)
    assert bool(torch.isnan(out).all())


# Tiles whose rows all see nothing between tiles with windows (the plan sorts
# empty rows to the end of their segment: at 64 heads 16 empty rows of 40 fill
# two tiles of 8, at 8 heads 80 of 200 fill one tile of 64), keys long enough
# for several chunks per tile: every cell against the oracle, over a buffer
# that starts as NaN, so a cell no unit writes shows.
@pytest.mark.parametrize("fmt", W.FORMATS)
@pytest.mark.parametrize("S_k", [300, 9000])
@pytest.mark.parametrize("H", [64, 8])
def test_empty_tiles_every_cell(fmt, S_k, H):
    S_q, n_empty = (40, 16) if H == 64 else (200, 80)
    rng = np.random.default_rng(71)
    starts = rng.integers(0, S_k // 2, S_q)
    ends = starts + rng.integers(1, S_k // 2, S_q)
    starts[8:8 + n_empty] = S_k // 3
    ends[8:8 + n_empty] = S_k // 3  # empty
    wl = W.make_random(fmt, 1, S_q, S_k, H=H, seed=71, windows="explicit", starts=starts.tolist(),
                       ends=ends.tolist(), out_dtype="bf16" if fmt == "mxfp4" else "f32")
    d = dev_inputs(wl)
    out = run(wl, d, out=torch.full((1, S_q, S_k), float("nan"), device="cuda",
                                    dtype=torch.bfloat16 if fmt == "mxfp4" else torch.float32))
    torch.cuda.synchronize()
    assert bool(torch.isneginf(out[0, 8:8 + n_empty].float()).all())
    ratio, rel = compare_all_rows(wl, out, what=f"empty tiles {fmt} H={H} S_k={S_k}")
    print(f"empty tiles {fmt} H={H} S_k={S_k}: max err/bound {ratio:.3e}, rel-L2 {rel:.3e}")


# ---------------------------------------------------------------------------
# the named workloads at full size: sampled rows against the oracle, the
# -inf placement of every row, and plan / no-plan equality
# ---------------------------------------------------------------------------

NAMED = ["c2", "c3", "c3_noclean", "c4_mxfp8", "c4_mxfp4", "c4_mxfp8_zero", "c4_mxfp4_zero", "c5", "thd_bf16_r4",
         "paged_mxfp8_decode", "screen_h8", "screen_h32"]


@pytest.mark.parametrize("name", NAMED)
def test_named_full_size(name):
    wl = W.make(name)
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    # the output starts as NaN: a cell that no unit writes stays NaN, which the
    # checks of every row below catch (an unclean call leaves the cells
    # outside the windows as they were)
    odt = torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32
    out = run(wl, d, plan=plan, out=torch.full((wl.B, wl.S_q, wl.S_k), float("nan"), dtype=odt, device="cuda"))
    out2 = run(wl, d, out=torch.full_like(out, float("nan")))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32),
                       out2.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32))
    if wl.clean:
        mask_check_all_rows(wl, out)
    inside_check_all_rows(wl, out)
    rows = sample_rows(wl)
    ref, bound = oracle.logits(wl, rows=rows)
    got = to_f64(out.reshape(wl.B * wl.S_q, -1)[torch.from_numpy(rows).cuda()])
    ratio, rel = compare_rows(wl, got, ref, bound, clean=wl.clean, what=name)
    print(f"{name}: {len(rows)} rows, max err/bound {ratio:.3e}, rel-L2 {rel:.3e}")


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_q8192_kv65536_full_size(fmt):
    """The page's long case, Q8192 / KV65536 with windows [0, KV - Q + row):
    on all-zero inputs (the page's timing setup) every in-window cell is
    exactly 0 and every other one -inf, checked over all 537 M cells; on
    random inputs a spread of rows is within tolerance of the oracle."""
    wl = W.make(f"q8k_{fmt}_zero")
    d = dev_inputs(wl)
    out = run(wl, d, out=torch.full((wl.B, wl.S_q, wl.S_k), float("nan"), device="cuda"))
    torch.cuda.synchronize()
    mask_check_all_rows(wl, out)
    inside_check_all_rows(wl, out)
    assert bool((out[torch.isfinite(out)] == 0).all()), "a zero workload scored a nonzero cell"
    del out, d
    wl = W.make(f"q8k_{fmt}")
    d = dev_inputs(wl)
    out = run(wl, d, out=torch.full((wl.B, wl.S_q, wl.S_k), float("nan"), device="cuda"))
    torch.cuda.synchronize()
    mask_check_all_rows(wl, out)
    rows = np.array([0, 1, 2047, 4096, 8190, 8191])
    ref, bound = oracle.logits(wl, rows=rows)
    got = to_f64(out.reshape(wl.B * wl.S_q, -1)[torch.from_numpy(rows).cuda()])
    compare_rows(wl, got, ref, bound, what=f"q8192/kv65536 {fmt}")


@pytest.mark.parametrize("name", ["c3", "c4_mxfp8", "c4_mxfp4"])
def test_named_every_cell(name):
    """Every cell of the Q2048 / KV32768 workloads against the oracle (values
    within tolerance, -inf placement exact), not only sampled rows."""
    wl = W.make(name)
    d = dev_inputs(wl)
    out = run(wl, d, out=torch.full((wl.B, wl.S_q, wl.S_k), float("nan"), device="cuda"))
    torch.cuda.synchronize()
    ratio, rel = compare_all_rows(wl, out, what=name)
    print(f"{name}: every cell, max err/bound {ratio:.3e}, rel-L2 {rel:.3e}")


# Long key ranges with several tiles take the XCD-owned chunk mapping (chunk c
# of every tile on XCD c % 8, 128 chunks per tile here): every cell of it.
XCD_CASES = [(f, win) for f in W.FORMATS for win in ("offsets", "irregular")]


@pytest.mark.parametrize("fmt,windows", XCD_CASES, ids=[f"{f}-{w}" for f, w in XCD_CASES])
def test_xcd_chunk_mapping_every_cell(fmt, windows):
    wl = W.make_random(fmt, 1, 64, 65536, seed=70, windows=windows, offsets=[0] if windows == "offsets" else None,
                       w_dtype="bf16" if fmt == "mxfp4" else "f32", out_dtype="bf16" if fmt == "mxfp4" else "f32")
    d = dev_inputs(wl)
    out = run(wl, d, out=torch.full((1, wl.S_q, wl.S_k), float("nan"), device="cuda",
                                    dtype=torch.bfloat16 if fmt == "mxfp4" else torch.float32))
    torch.cuda.synchronize()
    ratio, rel = compare_all_rows(wl, out, what=f"xcd {fmt} {windows}")
    print(f"xcd {fmt} {windows}: max err/bound {ratio:.3e}, rel-L2 {rel:.3e}")


@pytest.mark.parametrize("fmt", ["mxfp4", "bf16"])
def test_reordered_plan_several_segments(fmt):
    """Explicit irregular windows make the plan reorder the rows of every
    1024-row segment; with several segments per batch, a partial last segment
    and a ragged last tile, every row still gets its own scores (all rows
    compared: values within tolerance, -inf placement exact), and the result
    is bitwise that of the call that builds its plan in place."""
    wl = W.make_random(fmt, 2, 2100, 2400, seed=21, windows="irregular", w_dtype="bf16", out_dtype="bf16")
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    out = run(wl, d, plan=plan)
    out2 = run(wl, d)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    ref, bound = oracle.logits(wl)
    got = to_f64(out).reshape(wl.B * wl.S_q, wl.S_k)
    compare_rows(wl, got, ref.reshape(wl.B * wl.S_q, wl.S_k), bound.reshape(wl.B * wl.S_q, wl.S_k),
                 what=f"reordered {fmt}")


# ---------------------------------------------------------------------------
# packed variable-length rows over ratio-compressed keys
# ---------------------------------------------------------------------------

THD_CASES = [((5, 7), 2), ((9,), 1), ((1027, 3003, 4162), 4), ((0, 13, 0, 40, 1, 22), 3), ((300, 2, 700), 7),
             ((2048,), 4), ((33, 64, 95, 128, 1), 1)]


@pytest.mark.parametrize("lens,ratio", THD_CASES, ids=[f"{len(l)}seg-r{r}" for l, r in THD_CASES])
def test_thd_plan_windows_match_oracle(lens, ratio):
    wl = W.make_thd("bf16", lens, ratio, H=64, D=128, seed=1)
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    ws, we = lib.idx_logits_plan_windows(plan, 1, wl.S_q, wl.S_k)
    ows, owe = oracle.windows(wl)
    assert np.array_equal(ws.cpu().numpy(), ows) and np.array_equal(we.cpu().numpy(), owe)


def test_thd_plan_golden_windows():
    """The hand-worked cases, including key counts that disagree with the rows and rows
    past the last segment."""
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "thd_windows.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        plan = lib.idx_logits_plan_thd(c["cu_q"], c["cu_k"], c["ratio"], c["T_q"], c["m_total"])
        ws, we = lib.idx_logits_plan_windows(plan, 1, c["T_q"], c["m_total"])
        assert ws.cpu().reshape(-1).tolist() == c["starts"] and we.cpu().reshape(-1).tolist() == c["ends"], c["what"]


@pytest.mark.parametrize("fmt", W.FORMATS)
def test_thd_scores_match_oracle(fmt):
    wl = W.make_thd(fmt, (37, 0, 300, 90, 1), 2, seed=9, w_dtype="bf16", out_dtype="bf16" if fmt == "mxfp4" else "f32")
    d = dev_inputs(wl)
    out = run(wl, d)
    ref, bound = oracle.logits(wl)
    compare_rows(wl, to_f64(out).reshape(wl.S_q, wl.S_k), ref, bound, what=f"thd {fmt}")


def test_thd_plan_rejects():
    with pytest.raises(lib.IdxError):
        lib.idx_logits_plan_thd([0, 4], [0, 2], 0, 4, 2)
    with pytest.raises(lib.IdxError):
        lib.idx_logits_plan_thd([0, 4], [0, 2], 2, 4, 2, H=24)


@pytest.mark.parametrize("sm_scale", [-0.7, 0.0, 1e-30, 3e4])
@pytest.mark.parametrize("fmt", W.FORMATS)
def test_sm_scale_sign_and_size(fmt, sm_scale):
    """sm_scale multiplies after the head-sum, whatever its sign or size: a negative one
    flips every score, zero gives exact zeros inside the windows."""
    wl = W.make_random(fmt, 1, 19, 130, seed=31, sm_scale=sm_scale, windows="irregular")
    d = dev_inputs(wl)
    out = run(wl, d)
    ref, bound = oracle.logits(wl)
    got = to_f64(out).reshape(wl.S_q, wl.S_k)
    compare_rows(wl, got, ref, bound, what=f"sm_scale {sm_scale}")
    if sm_scale == 0.0:
        inside = ~np.isneginf(ref)
        assert np.all(got[inside] == 0.0)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_extreme_block_scales(fmt):
    """E8M0 exponents spread over +-30 around 1 (products of Q and K scales span 2^-60..2^60):
    the MFMA block scales, the weighted-query pieces and the epilogue stay within tolerance."""
    wl = W.make_random(fmt, 1, 24, 200, seed=32, scale_lo=-30, scale_hi=30, windows="irregular")
    d = dev_inputs(wl)
    out = run(wl, d)
    ref, bound = oracle.logits(wl)
    compare_rows(wl, to_f64(out).reshape(wl.S_q, wl.S_k), ref, bound, what=f"extreme scales {fmt}")


def test_fp8_row_scale_extremes():
    """FP8 per-row K scales of 0, tiny and huge values (finite and >= 0 as required)."""
    wl = W.make_random("fp8", 1, 16, 96, seed=33, windows="irregular")
    ks = wl.k_scale.copy()
    ks[0, ::7] = 0.0
    ks[0, 1::7] = 1e-20
    ks[0, 2::7] = 1e20
    wl = wl.replace(k_scale=ks)
    d = dev_inputs(wl)
    out = run(wl, d)
    ref, bound = oracle.logits(wl)
    got = to_f64(out).reshape(wl.S_q, wl.S_k)
    compare_rows(wl, got, ref, bound, what="fp8 row scale extremes")
    inside = ~np.isneginf(ref)
    zero_cols = np.zeros(wl.S_k, bool)
    zero_cols[::7] = True
    assert np.all(got[inside & zero_cols[None, :]] == 0.0)


def test_mx_block_layout_probes():
    """The oracle's MX layout probes (one d-block populated, one scale byte raised,
    nibble order) run on the GPU: within tolerance of the oracle for every variant."""
    cap = _Capture()
    P.pin_mx_block_layout(cap)
    for wl in cap.seen:
        out = run(wl, dev_inputs(wl))
        torch.cuda.synchronize()
        _full_compare(wl, out, what=f"layout probe {wl.fmt}")


# ---------------------------------------------------------------------------
# decode-sized batches: at most two query rows per batch, where every wave of
# a unit scores the tile's two rows over its own share of the columns
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S_q", [1, 2])
@pytest.mark.parametrize("fmt", W.FORMATS)
def test_decode_rows_every_cell(fmt, S_q):
    """Every cell of B = 5 batches of one or two query rows, causal offsets of
    every size (an empty window, a window of one key, the whole of K) and
    S_k long enough to span several chunks per tile, output pre-filled with
    NaN so a cell no wave wrote is caught."""
    wl = W.make_random(fmt, 5, S_q, 20000, seed=80 + S_q, offsets=[0, -19999, -19998 - S_q, -7000, -12345],
                       w_dtype="bf16" if fmt == "mxfp4" else "f32")
    d = dev_inputs(wl)
    out = torch.full((wl.B, wl.S_q, wl.S_k), float("nan"), dtype=out_dtype(wl), device="cuda")
    run(wl, d, out=out)
    torch.cuda.synchronize()
    inside_check_all_rows(wl, out)
    _full_compare(wl, out, what=f"decode {fmt} S_q={S_q}")


# ---------------------------------------------------------------------------
# paged keys (decode)
# ---------------------------------------------------------------------------

# (B, next_n, context lengths, page size, S_k or None for the longest context)
PAGED_CASES = [
    (4, 1, [1, 700, 33, 2000], 64, None),
    (5, 3, [0, 2, 3, 129, 1000], 16, None),   # an empty context, contexts shorter than next_n
    (3, 2, [47, 4100, 6000], 48, 4100),       # pages not a multiple of 32 rows; a context past S_k
    (2, 4, [-5, 333], 100, 400),              # a negative context length sees nothing
]
PAGED_IDS = [f"b{c[0]}-n{c[1]}-p{c[3]}" for c in PAGED_CASES]


def _paged(fmt, case, seed=31, **kw):
    B, n, ctx, ps, S_k = case
    return W.make_paged(fmt, B, n, ctx, ps, S_k=S_k, seed=seed, **kw)


@pytest.mark.parametrize("case", PAGED_CASES, ids=PAGED_IDS)
def test_paged_plan_windows_match_oracle(case):
    wl = _paged("bf16", case)
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    ws, we = lib.idx_logits_plan_windows(plan, wl.B, wl.S_q, wl.S_k)
    ows, owe = oracle.windows(wl)
    assert np.array_equal(ws.cpu().numpy(), ows) and np.array_equal(we.cpu().numpy(), owe)


@pytest.mark.parametrize("case", PAGED_CASES, ids=PAGED_IDS)
@pytest.mark.parametrize("fmt", W.FORMATS)
def test_paged_scores_match_oracle(fmt, case):
    """Every cell of a paged call against the oracle over the gathered keys."""
    wl = _paged(fmt, case, w_dtype="bf16" if fmt == "mxfp4" else "f32")
    d = dev_inputs(wl)
    out = run(wl, d)
    _full_compare(wl, out, what=f"paged {fmt} {case}")


def _gather_dense(wl):
    """The request-major K a paged workload describes, gathered with numpy
    (zero rows past each clamped context)."""
    pg = wl.paged
    ps, bt = pg["page_size"], np.asarray(pg["block_table"])
    cache, scache = np.asarray(pg["k_cache"]), pg["k_scale_cache"]
    k = np.zeros((wl.B, wl.S_k) + cache.shape[2:], cache.dtype)
    ks = None if scache is None else np.zeros((wl.B, wl.S_k), np.asarray(scache).dtype)
    for b in range(wl.B):
        n = min(max(int(pg["ctx"][b]), 0), wl.S_k)
        j = np.arange(n)
        k[b, :n] = cache[bt[b, j // ps], j % ps]
        if ks is not None:
            ks[b, :n] = np.asarray(scache)[bt[b, j // ps], j % ps]
    return k, ks


@pytest.mark.parametrize("fmt", W.FORMATS)
def test_paged_equals_contiguous(fmt):
    """A paged call is bitwise the contiguous call on the gathered keys with the
    same windows given explicitly, clean or not."""
    wl = _paged(fmt, PAGED_CASES[2], out_dtype="bf16" if fmt == "fp8" else "f32")
    d = dev_inputs(wl)
    k, ks = _gather_dense(wl)
    ows, owe = oracle.windows(wl)
    dense = wl.replace(k=k, k_scale=ks, paged=None, starts=ows, ends=owe)
    dd = dev_inputs(dense)
    for clean in (True, False):
        got = run(wl, d, clean=clean)
        want = run(dense, dd, clean=clean)
        view = torch.int16 if got.dtype == torch.bfloat16 else torch.int32
        if clean:
            assert torch.equal(got.view(view), want.view(view))
        else:  # cells outside the windows are not written
            for b in range(wl.B):
                for i in range(wl.S_q):
                    s0, e = int(ows[b, i]), max(int(owe[b, i]), int(ows[b, i]))
                    assert torch.equal(got[b, i, s0:e].view(view), want[b, i, s0:e].view(view)), (b, i)


@pytest.mark.parametrize("fmt", W.FORMATS)
def test_paged_prepare_score_and_plan(fmt):
    """idx_logits_prepare_paged + idx_logits_score (keys NULL in the args), or +
    idx_logits_score_paged, with a plan from idx_logits_plan_paged is bitwise
    the one-call form, which gives
    the same result whether it builds its plan or takes it."""
    wl = _paged(fmt, PAGED_CASES[1])
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    one = run(wl, d)
    planned = run(wl, d, plan=plan)
    out = torch.empty_like(one)
    args = lib.make_paged_args(d["q"], d["w"], out, wl.S_k, in_dtype=fmt, q_scale=d["q_scale"], sm_scale=wl.sm_scale)
    ws = lib.idx_logits_prepare_paged(args, d["kv"])
    lib.idx_logits_score(args, plan, ws)
    out2 = torch.full_like(one, float("nan"))
    args2 = lib.make_paged_args(d["q"], d["w"], out2, wl.S_k, in_dtype=fmt, q_scale=d["q_scale"],
                                sm_scale=wl.sm_scale)
    lib.idx_logits_score_paged(args2, d["kv"], plan, ws)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int32), planned.view(torch.int32))
    assert torch.equal(one.view(torch.int32), out.view(torch.int32))
    assert torch.equal(one.view(torch.int32), out2.view(torch.int32))


# ---------------------------------------------------------------------------
# 8, 16 and 32 query heads sharing the key head (tiles of 512 / H rows)
# ---------------------------------------------------------------------------

HEAD_CASES = [(f, H) for f in W.FORMATS for H in (8, 16, 32)]
HEAD_IDS = [f"{f}-h{H}" for f, H in HEAD_CASES]


@pytest.mark.parametrize("fmt,H", HEAD_CASES, ids=HEAD_IDS)
def test_other_head_counts(fmt, H):
    """Every cell against the oracle: two batches of two full tiles and a
    ragged one, a ragged key tail, causal offsets of both signs, bf16 weights
    and output for half the cases; a precomputed plan gives the same bits."""
    tr = 512 // H
    bf = H != 16
    wl = W.make_random(fmt, 2, 2 * tr + 5, 3 * 32 * 7 + 13, H=H, seed=40 + H, offsets=[0, -17],
                       w_dtype="bf16" if bf else "f32", out_dtype="bf16" if bf else "f32",
                       sm_scale=1 / math.sqrt(128))
    d = dev_inputs(wl)
    out = run(wl, d)
    _full_compare(wl, out, what=f"{fmt} H={H}")
    out2 = run(wl, d, plan=make_plan(wl, d))
    view = torch.int16 if out.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(out.view(view), out2.view(view))


@pytest.mark.parametrize("fmt,H", HEAD_CASES, ids=HEAD_IDS)
def test_other_head_counts_irregular(fmt, H):
    """Irregular windows (reordered rows, empty rows, nonzero starts), clean
    and not: values inside the windows, -inf placement when cleaning."""
    wl = W.make_random(fmt, 1, 300, 1500, H=H, seed=60 + H, windows="irregular")
    d = dev_inputs(wl)
    _full_compare(wl, run(wl, d), what=f"{fmt} H={H} irregular")
    _full_compare(wl, run(wl, d, clean=False), clean=False, what=f"{fmt} H={H} irregular unclean")


@pytest.mark.parametrize("H", (8, 32))
def test_other_head_counts_thd_and_paged(H):
    """The packed variable-length and paged entry points at other head counts."""
    wl = W.make_thd("mxfp8", (37, 0, 300, 90, 1), 2, H=H, seed=9)
    d = dev_inputs(wl)
    ref, bound = oracle.logits(wl)
    compare_rows(wl, to_f64(run(wl, d)).reshape(wl.S_q, wl.S_k), ref, bound, what=f"thd H={H}")
    wl = _paged("mxfp4", PAGED_CASES[1], H=H)
    d = dev_inputs(wl)
    _full_compare(wl, run(wl, d), what=f"paged H={H}")


@pytest.mark.parametrize("n_req", [12, 40])
@pytest.mark.parametrize("fmt", ["fp8", "mxfp8"])
def test_paged_decode_wave_lengths(fmt, n_req):
    """Two-token decode over requests of random context up to 40000 keys: the
    units' waves stream from one to seven 64-column pairs of keys, odd and
    even counts, straight from the cache through a ring of four blocks.  The
    result is bitwise that of the gathered two-phase call (fragment-order
    keys, a ring of two), and sampled rows are within tolerance of the
    oracle."""
    rng = np.random.default_rng(43 + n_req)
    ctx = rng.integers(1, 40000, n_req).tolist()
    wl = W.make_paged(fmt, n_req, 2, ctx, 64, seed=44)
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    one = run(wl, d, plan=plan)
    out = torch.full_like(one, float("nan"))
    args = lib.make_paged_args(d["q"], d["w"], out, wl.S_k, in_dtype=fmt, q_scale=d["q_scale"], sm_scale=wl.sm_scale)
    ws = lib.idx_logits_prepare_paged(args, d["kv"])
    lib.idx_logits_score(args, plan, ws)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int32), out.view(torch.int32)), "paged and gathered keys differ"
    rows = np.array([0, 1, 2 * (n_req // 2), 2 * n_req - 1])
    ref, bound = oracle.logits(wl, rows=rows)
    got = to_f64(one.reshape(wl.B * wl.S_q, -1)[torch.from_numpy(rows).cuda()])[:, : wl.S_k]
    compare_rows(wl, got, ref, bound, clean=wl.clean, what=f"paged decode {fmt} r{n_req}")


@pytest.mark.parametrize("page_size", [32, 64, 128])
@pytest.mark.parametrize("fmt", W.FORMATS)
def test_paged_direct_equals_gather(fmt, page_size):
    """Pages of 32 * 2^j keys are scored straight from the cache by the one-call
    entry point; the result is bitwise that of the gathered two-phase call, and
    within tolerance of the oracle."""
    wl = W.make_paged(fmt, 3, 2, [5000, 1, 2300], page_size, seed=41, w_dtype="bf16" if fmt == "fp8" else "f32")
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    one = run(wl, d, plan=plan)
    out = torch.empty_like(one)
    args = lib.make_paged_args(d["q"], d["w"], out, wl.S_k, in_dtype=fmt, q_scale=d["q_scale"], sm_scale=wl.sm_scale)
    ws = lib.idx_logits_prepare_paged(args, d["kv"])
    lib.idx_logits_score(args, plan, ws)
    # the paged scoring phase takes the direct path where the one-call form does
    out2 = torch.full_like(one, float("nan"))
    args2 = lib.make_paged_args(d["q"], d["w"], out2, wl.S_k, in_dtype=fmt, q_scale=d["q_scale"],
                                sm_scale=wl.sm_scale)
    lib.idx_logits_score_paged(args2, d["kv"], plan, ws)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int32), out.view(torch.int32))
    assert torch.equal(one.view(torch.int32), out2.view(torch.int32))
    _full_compare(wl, one, what=f"paged direct {fmt} p{page_size}")
