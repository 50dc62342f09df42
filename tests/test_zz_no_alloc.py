"""idx_logits_run_noalloc: the one-call entry point that allocates nothing
(its workspace is the library's per-device scratch), through the C ABI,
against idx_logits_run on the same inputs."""

import ctypes

import numpy as np
import pytest
import torch

import mqa_logits_scoring_amd as lib
import workloads as W
from gpu_util import dev_inputs, make_plan, out_dtype, run


def _noalloc(wl, d, out, plan=None, accumulate="native"):
    return lib.idx_logits_run_noalloc(d["q"], d["k"], d["w"], out, in_dtype=wl.fmt, q_scale=d["q_scale"],
                                      k_scale=d["k_scale"], sm_scale=wl.sm_scale, clean_logits=wl.clean, plan=plan,
                                      q_causal_offsets=d["offsets"] if plan is None else None,
                                      row_starts=d["starts"] if plan is None else None,
                                      row_ends=d["ends"] if plan is None else None, accumulate=accumulate)


def _view(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", W.FORMATS)
def test_noalloc_equals_run_two_calls(fmt):
    """Two calls in a row, the second with a smaller input (the scratch keeps
    the first call's contents), each bitwise the allocating entry point's
    output; with and without a precomputed plan."""
    big = W.make_random(fmt, 2, 300, 5000, seed=51, windows="irregular", w_dtype="bf16")
    small = W.make_random(fmt, 1, 37, 700, seed=52, offsets=[-3], out_dtype="bf16")
    for wl in (big, small):
        d = dev_inputs(wl)
        want = run(wl, d)
        got = _noalloc(wl, d, torch.full_like(want, float("nan")))
        torch.cuda.synchronize()
        assert torch.equal(_view(got), _view(want)), (fmt, wl.S_q, wl.S_k)
        plan = make_plan(wl, d)
        got2 = _noalloc(wl, d, torch.full_like(want, float("nan")), plan=plan)
        torch.cuda.synchronize()
        assert torch.equal(_view(got2), _view(want)), (fmt, wl.S_q, wl.S_k, "planned")


@pytest.mark.gpu
def test_noalloc_exact_accumulation_and_full_size():
    """The exact-accumulation conversion (the largest workspace of these) and
    the Q2048 / KV32768 MXFP8 call."""
    wl = W.make_random("fp8", 1, 200, 3000, seed=53, windows="irregular")
    d = dev_inputs(wl)
    want = run(wl, d, accumulate="fp32")
    got = _noalloc(wl, d, torch.empty_like(want), accumulate="fp32")
    torch.cuda.synchronize()
    assert torch.equal(_view(got), _view(want))
    wl = W.make("c4_mxfp8")
    d = dev_inputs(wl)
    want = run(wl, d)
    got = _noalloc(wl, d, torch.empty_like(want))
    torch.cuda.synchronize()
    assert torch.equal(_view(got), _view(want))


def test_noalloc_rejects_oversized_calls():
    """Checked on the host before anything else happens (no GPU needed): a
    call whose workspace exceeds the scratch returns IDX_E_WORKSPACE."""
    cap = lib.idx_logits_noalloc_scratch_bytes()
    assert cap == 64 << 20
    a = lib.IdxLogitsArgs()
    a.B, a.S_q, a.S_k, a.H, a.D = 1, 2048, 1 << 20, 64, 128  # 1M keys in fragment order: 128 MiB
    a.in_dtype = 2
    a.q = a.k = a.w = a.out = a.q_scale = a.k_scale = 1 << 20
    a.sm_scale = 1.0
    a.out_row_stride = a.S_k
    a.clean_logits = 1
    assert lib.idx_logits_workspace_bytes_planned(a) > cap
    st = lib.lib().idx_logits_run_noalloc(ctypes.byref(a), None, None, None, None, None)
    assert st == lib.IDX_E_WORKSPACE
    assert "idx_logits_run_noalloc" in lib.idx_last_error()
    a.in_dtype = 9
    assert lib.lib().idx_logits_run_noalloc(ctypes.byref(a), None, None, None, None, None) == lib.IDX_E_INVALID
