"""Fused scoring + top-k (idx_logits_run_topk) against the oracle's ranking.

The fused call never stores the score matrix, so its result is checked
against the ranking of the scores a plain call stores: idx_logits_run with
the same inputs, plan and output type, then oracle.topk over those scores on
the host (integer work on the very same fp32 or bf16 values).  Indices and
listed scores must agree bit for bit, in both orders.  That the plain call's
scores match the fp64 oracle is the parity tests' job."""

import numpy as np
import pytest
import torch

import mqa_logits_scoring_amd as lib
import oracle
import workloads as W
from gpu_util import dev_inputs, make_plan, out_dtype, run

pytestmark = pytest.mark.gpu


def _host_scores(out, wl):
    flat = out.reshape(wl.B * wl.S_q, -1)[:, : wl.S_k]
    if flat.dtype == torch.bfloat16:
        return flat.view(torch.int16).cpu().numpy().view(np.uint16)
    return flat.cpu().numpy()


def _fused(wl, d, k, order, plan=None, accumulate="native", n_redo=None):
    return lib.idx_logits_run_topk(d["q"], d["k"], d["w"], k, in_dtype=wl.fmt, q_scale=d["q_scale"],
                                   k_scale=d["k_scale"], sm_scale=wl.sm_scale, out_dtype=out_dtype(wl), order=order,
                                   plan=plan, q_causal_offsets=d["offsets"], row_starts=d["starts"],
                                   row_ends=d["ends"], accumulate=accumulate, n_redo=n_redo)


def _assert_same(got_idx, got_val, want_idx, want_val, what):
    bad = np.argwhere(got_idx != want_idx)
    assert bad.size == 0, (f"{what}: indices differ first at (row, rank) {bad[:3].tolist()}: "
                           f"got {got_idx[tuple(bad[0])]} want {want_idx[tuple(bad[0])]}")
    nan = np.isnan(want_val)
    assert np.array_equal(np.isnan(got_val), nan), what
    assert np.array_equal(got_val[~nan].view(np.uint32), want_val[~nan].view(np.uint32)), f"{what}: scores differ"


def check_fused(wl, k, orders=("column", "score"), accumulate="native", built_plan=False, rows=None,
                expect_redo=None):
    """Fused result == oracle.topk over the plain call's scores (all rows, or
    `rows`); returns the number of rows scored twice."""
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    out = run(wl, d, plan=plan, accumulate=accumulate)
    ws, we = oracle.windows(wl)
    ws, we = ws.reshape(-1), we.reshape(-1)
    host = _host_scores(out, wl)
    del out
    sel = np.arange(wl.B * wl.S_q) if rows is None else np.asarray(rows)
    redo = None
    for order in orders:
        nr = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        idx, val = _fused(wl, d, k, order, plan=None if built_plan else plan, accumulate=accumulate, n_redo=nr)
        torch.cuda.synchronize()
        want_idx, want_val = oracle.topk(host[sel], ws[sel], we[sel], k, by_column=order == "column")
        got_idx = idx.reshape(-1, k).cpu().numpy()[sel]
        got_val = val.reshape(-1, k).cpu().numpy()[sel]
        _assert_same(got_idx, got_val, want_idx, want_val, f"{wl.name} k={k} by {order}")
        redo = int(nr.item())
        assert 0 <= redo <= wl.B * wl.S_q
        if expect_redo is not None:
            assert redo == expect_redo, (redo, expect_redo)
    return redo


FUSED = [
    ("bf16", dict(B=2, S_q=70, S_k=3000, offsets=[0, -900]), 64),
    ("mxfp8", dict(B=1, S_q=130, S_k=5000, windows="irregular"), 2048),
    ("mxfp8", dict(B=2, S_q=41, S_k=20000, offsets=[0, -7000]), 300),
    ("mxfp4", dict(B=1, S_q=33, S_k=9000, windows="irregular", out_dtype="bf16", w_dtype="bf16"), 512),
    ("fp8", dict(B=3, S_q=17, S_k=40000, offsets=[0, -1, -39000]), 2048),
    ("fp8", dict(B=1, S_q=9, S_k=1000, windows="irregular"), 1),
    ("mxfp8", dict(B=2, S_q=40, S_k=1500, windows="irregular"), 2048),   # no window holds more than k: no sample
]


@pytest.mark.parametrize("fmt,kw,k", FUSED, ids=[f"{f}-{kw['S_k']}-k{k}" for f, kw, k in FUSED])
def test_fused_topk_matches_oracle_ranking(fmt, kw, k):
    kw = dict(kw)
    wl = W.make_random(fmt, kw.pop("B"), kw.pop("S_q"), kw.pop("S_k"), seed=91, **kw)
    check_fused(wl, k)


def test_fused_topk_builds_its_plan():
    wl = W.make_random("mxfp8", 2, 50, 7000, seed=92, windows="irregular")
    check_fused(wl, 700, built_plan=True)
    wl = W.make_random("bf16", 1, 60, 4000, seed=93, offsets=[-100])
    check_fused(wl, 128, built_plan=True, orders=("score",))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8"])
def test_fused_topk_exact_accumulation(fmt):
    wl = W.make_random(fmt, 1, 40, 9000, seed=94, windows="irregular")
    check_fused(wl, 1024, accumulate="fp32")


@pytest.mark.parametrize("H", [8, 16, 32])
def test_fused_topk_other_head_counts(H):
    wl = W.make_random("mxfp8", 1, 150, 6000, H=H, seed=95, windows="irregular")
    check_fused(wl, 1000)
    wl = W.make_random("bf16", 1, 70, 3000, H=H, seed=96, offsets=[0], w_dtype="bf16", out_dtype="bf16")
    check_fused(wl, 256, orders=("score",))


def test_fused_topk_zero_inputs():
    """All-zero inputs: every score is 0, so the whole window ties and the
    selection is the window's first k columns (rows of up to 32768 candidates
    run the selection from memory, not LDS)."""
    wl = W.make_random("mxfp8", 1, 20, 32768, seed=97, offsets=[-1], zero=True)
    check_fused(wl, 2048, expect_redo=0)


def _doubled_keys_case(S_q=40, S_k=16384, H=64, seed=98):
    """BF16 inputs whose sampled keys (every 16th block of 32) are twice the
    others: every score of a sampled key is exactly twice that of any other
    key (positive weights, so ReLU and the head sum scale exactly), and the
    sample, ranking only its own keys, puts every row's threshold at the
    doubled score.  Windows of S_k - S_q + i + 1 > 2048 keys hold only about
    1024 sampled keys, so every row has fewer candidates than k = 2048 and
    must be scored a second time."""
    rng = np.random.default_rng(seed)
    q = torch.from_numpy(rng.standard_normal((S_q, H, 128)).astype(np.float32)).to(torch.bfloat16)
    base = torch.from_numpy(rng.standard_normal((1, 128)).astype(np.float32)).to(torch.bfloat16)
    k = base.repeat(S_k, 1)
    sampled = (torch.arange(S_k) // 32) % 16 == 0
    k[sampled] = (base.float() * 2).to(torch.bfloat16)
    w = torch.from_numpy(rng.random((S_q, H)).astype(np.float32) + 0.01)
    return q.cuda(), k.cuda(), w.cuda()


def test_fused_topk_second_pass_is_exact():
    S_q, S_k, kk = 40, 16384, 2048
    q, k, w = _doubled_keys_case(S_q, S_k)
    offs = torch.tensor([0], dtype=torch.int32, device="cuda")
    out = lib.idx_logits_run(q, k, w, in_dtype="bf16", sm_scale=0.125, q_causal_offsets=offs)
    torch.cuda.synchronize()
    host = out.reshape(S_q, S_k).cpu().numpy()
    ws = np.zeros(S_q, np.int64)
    we = S_k - S_q + np.arange(S_q) + 1
    for order in ("column", "score"):
        nr = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        idx, val = lib.idx_logits_run_topk(q, k, w, kk, in_dtype="bf16", sm_scale=0.125, q_causal_offsets=offs,
                                           order=order, n_redo=nr)
        torch.cuda.synchronize()
        want_idx, want_val = oracle.topk(host, ws, we, kk, by_column=order == "column")
        _assert_same(idx.reshape(S_q, kk).cpu().numpy(), val.reshape(S_q, kk).cpu().numpy(), want_idx, want_val,
                     f"second pass by {order}")
        assert int(nr.item()) == S_q, "every row should have gone through the second pass"


def test_fused_topk_plan_mismatch_is_loud():
    wl = W.make_random("mxfp8", 1, 16, 600, seed=99, offsets=[0])
    d = dev_inputs(wl)
    other = lib.idx_logits_plan(1, 16, 500, 64, 128, q_causal_offsets=d["offsets"], device="cuda")
    idx, val = _fused(wl, d, 32, "column", plan=other)
    torch.cuda.synchronize()
    assert bool((idx == -1).all()) and bool(torch.isnan(val).all())


def test_fused_topk_full_size_c4():
    """Top-2048 of the MXFP8 Q2048/KV32768 call, every row, both orders; with
    random inputs the sample's thresholds never need a second pass."""
    check_fused(W.make("c4_mxfp8"), 2048, expect_redo=0)


def test_fused_topk_full_size_c5():
    """Top-2048 of the MXFP4 Q8192/KV65536 irregular call (bf16 scores):
    every row against the plain call's top-k kernel (itself pinned to the
    oracle's ranking), a spread of rows against the oracle's ranking."""
    wl = W.make("c5")
    d = dev_inputs(wl)
    plan = make_plan(wl, d)
    out = run(wl, d, plan=plan)
    for order in ("column", "score"):
        ref_idx, ref_val = lib.idx_logits_topk(plan, out, 2048, order=order)
        idx, val = _fused(wl, d, 2048, order, plan=plan)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), f"c5 by {order}: indices differ from the two-phase result"
        assert torch.equal(val.view(torch.int32), ref_val.view(torch.int32)), f"c5 by {order}: scores differ"
    rows = np.unique(np.concatenate([np.arange(0, wl.S_q, 97), np.arange(wl.S_q - 8, wl.S_q)]))
    ws, we = oracle.windows(wl)
    host = out.reshape(wl.S_q, -1)[torch.from_numpy(rows).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    want_idx, want_val = oracle.topk(host, ws.reshape(-1)[rows], we.reshape(-1)[rows], 2048, by_column=False)
    _assert_same(idx.reshape(-1, 2048).cpu().numpy()[rows], val.reshape(-1, 2048).cpu().numpy()[rows], want_idx,
                 want_val, "c5 sampled rows by score")
