"""How the dot products are accumulated, against the per-cell tolerance.

The tolerance of a cell is 1e-4 * sm_scale * |k_j| * sum_h |w_h| |q_h|.  The
inputs here are built against the matrix core's own accumulation (see
workloads.make_adversarial): |q_d| proportional to |k_d| so that
sum_d |q_d k_d| meets |q| |k|, one large and seven small elements in every
group of eight consecutive d, the same q for all heads and weights of one
sign, so that every head's error adds.

- IDX_ACCUM_FP32 ("fp32") must meet the tolerance for every format.
- IDX_ACCUM_NATIVE ("native") meets it with the bf16 and e2m1 matrix cores.
  The e4m3 matrix core (FP8, MXFP8) sums each group of eight products in
  fixed point aligned to the group's largest, with 13 fraction bits,
  truncating: per dot the error is below 7 * 2^-13 of sum_d |q_d k_d| <=
  |q| |k|.  The |x| epilogue halves the sum of that error over the heads
  (sum_h |w_h| |S_h| error) and over the linear term (qt . k, whose error is
  at most the same), and adds the weighted-query pieces' residual (below
  2^-16 sqrt(32) / 2 of the basis) and fp32 rounding; native FP8 / MXFP8 are
  held to that derived bound, and print how much of it they use.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import compare_all_rows, compare_rows, dev_inputs, make_plan, run, to_f64

pytestmark = pytest.mark.gpu

TOL = 1e-4
NATIVE_E4M3_TOL = 7 * 2.0 ** -13 + 2.0 ** -16 * math.sqrt(32) / 2 + 2.0 ** -18


def _tol(fmt, accum):
    return NATIVE_E4M3_TOL if (accum == "native" and fmt in ("fp8", "mxfp8")) else TOL


CASES = [(f, H, a) for f in W.FORMATS for H in (64, 32) for a in ("native", "fp32")]


@pytest.mark.parametrize("fmt,H,accum", CASES, ids=[f"{f}-h{H}-{a}" for f, H, a in CASES])
def test_adversarial_accumulation(fmt, H, accum):
    wl = W.make_adversarial(fmt, 52, 700, H=H, seed=3, w_dtype="bf16" if H == 32 else "f32")
    d = dev_inputs(wl)
    out = run(wl, d, out=torch.full((1, wl.S_q, wl.S_k), float("nan"), device="cuda"), accumulate=accum)
    torch.cuda.synchronize()
    ratio, rel = compare_all_rows(wl, out, what=f"adversarial {fmt} H={H} {accum}", rel_tol=_tol(fmt, accum))
    print(f"adversarial {fmt} H={H} {accum}: max err/bound {ratio:.3e} (allowed {_tol(fmt, accum):.3e}), "
          f"rel-L2 {rel:.3e}")


EXACT_MATRIX = [(f, wd, od, H) for f in ("fp8", "mxfp8") for wd in ("f32", "bf16") for od in ("f32", "bf16")
                for H in (64, 16)]


@pytest.mark.parametrize("fmt,w_dtype,o_dtype,H", EXACT_MATRIX, ids=["-".join(map(str, m)) for m in EXACT_MATRIX])
def test_fp32_accumulation_matrix(fmt, w_dtype, o_dtype, H):
    """FP8 / MXFP8 with exact accumulation: every cell of irregular windows over
    several tiles and a ragged key tail, clean and not, against the oracle;
    with a precomputed plan the bits are those of the call that builds it."""
    wl = W.make_random(fmt, 2, 45, 333, H=H, w_dtype=w_dtype, out_dtype=o_dtype, sm_scale=0.3, seed=80 + H,
                       windows="irregular")
    d = dev_inputs(wl)
    out = run(wl, d, accumulate="fp32")
    out2 = run(wl, d, plan=make_plan(wl, d), accumulate="fp32")
    view = torch.int16 if out.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(out.view(view), out2.view(view))
    ref, bound = oracle.logits(wl)
    n = wl.B * wl.S_q
    ratio, _ = compare_rows(wl, to_f64(out).reshape(n, wl.S_k), ref, bound, what=f"fp32 accumulation {fmt}")
    sentinel = torch.full_like(out, 77.0)
    run(wl, d, out=sentinel, clean=False, accumulate="fp32")
    inside = ~torch.isneginf(out)
    assert torch.equal(sentinel[inside].view(view), out[inside].view(view))
    assert bool((sentinel[~inside] == 77.0).all())


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8"])
def test_fp32_accumulation_scales_and_paged(fmt):
    """Block scales spread over +-30 (folded into the bf16 operands) and paged
    keys (gathered and converted, never read straight from the cache)."""
    wl = W.make_random(fmt, 1, 24, 200, seed=32, scale_lo=-30, scale_hi=30, windows="irregular")
    d = dev_inputs(wl)
    ref, bound = oracle.logits(wl)
    compare_rows(wl, to_f64(run(wl, d, accumulate="fp32")).reshape(wl.S_q, wl.S_k), ref, bound,
                 what=f"fp32 accumulation, wide scales {fmt}")
    wl = W.make_paged(fmt, 3, 2, [5000, 1, 2300], 64, seed=41)
    d = dev_inputs(wl)
    out = run(wl, d, accumulate="fp32")
    ref, bound = oracle.logits(wl)
    compare_rows(wl, to_f64(out).reshape(wl.B * wl.S_q, wl.S_k), ref.reshape(-1, wl.S_k),
                 bound.reshape(-1, wl.S_k), what=f"fp32 accumulation, paged {fmt}")


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
def test_fp32_accumulation_is_native_for_exact_cores(fmt):
    """BF16 and MXFP4 run the same kernels either way: bitwise equal."""
    wl = W.make_random(fmt, 1, 30, 400, seed=90, windows="irregular")
    d = dev_inputs(wl)
    a = run(wl, d)
    b = run(wl, d, accumulate="fp32")
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
