"""The C ABI on the CPU: the library loads, exports every entry point its
header declares, and rejects bad arguments on the host before launching
anything (only cases that fail validation are called here)."""

import ctypes
import os
import re

import pytest

import mqa_logits_scoring_amd as lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "idx_logits.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(idx_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(lib.EXPORTED), names
    L = lib.lib()
    for n in names:
        assert hasattr(L, n), n
    assert lib.idx_abi_version() == lib.ABI_VERSION == 3


def test_plan_bytes():
    assert lib.idx_logits_plan_bytes(1, 128, 512) > 0
    # tiles hold 512 / H rows: fewer, taller tiles at fewer heads
    assert lib.idx_logits_plan_bytes(1, 4096, 512, H=8) < lib.idx_logits_plan_bytes(1, 4096, 512, H=64)
    assert lib.idx_logits_plan_bytes(1, 128, 512, H=24) == 0
    assert lib.idx_logits_plan_bytes(0, 128, 512) == 0
    assert lib.idx_logits_plan_bytes(1, -1, 512) == 0
    a = lib.idx_logits_plan_bytes(1, 2048, 32768)
    b = lib.idx_logits_plan_bytes(1, 2048, 64)
    assert a == b  # the plan does not grow with S_k


FAKE = 1 << 20  # never dereferenced: every call below fails validation first


def _args(**kw):
    a = lib.IdxLogitsArgs()
    a.B, a.S_q, a.S_k, a.H, a.D = 1, 16, 64, 64, 128
    a.in_dtype = 2
    a.q = a.k = a.w = a.out = a.q_scale = a.k_scale = FAKE
    a.w_dtype = a.out_dtype = 0
    a.sm_scale = 1.0
    a.out_row_stride = 64
    a.clean_logits = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _run(a, plan=None, ws=None, ws_bytes=0):
    return lib.lib().idx_logits_run(ctypes.byref(a), plan, None, None, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=24), lib.IDX_E_UNSUPPORTED),
    (dict(H=128), lib.IDX_E_UNSUPPORTED),
    (dict(D=64), lib.IDX_E_UNSUPPORTED),
    (dict(B=0), lib.IDX_E_INVALID),
    (dict(S_k=-3), lib.IDX_E_INVALID),
    (dict(in_dtype=9), lib.IDX_E_INVALID),
    (dict(w_dtype=5), lib.IDX_E_INVALID),
    (dict(q=None), lib.IDX_E_INVALID),
    (dict(q_scale=None), lib.IDX_E_INVALID),
    (dict(k_scale=None), lib.IDX_E_INVALID),
    (dict(out=FAKE + 4), lib.IDX_E_INVALID),
    (dict(out_row_stride=63), lib.IDX_E_INVALID),
    (dict(sm_scale=float("inf")), lib.IDX_E_INVALID),
    (dict(sm_scale=float("nan")), lib.IDX_E_INVALID),
])
def test_run_rejects(kw, status):
    assert _run(_args(**kw)) == status
    assert lib.idx_last_error() != ""


def test_run_needs_plan_or_workspace():
    assert _run(_args()) == lib.IDX_E_WORKSPACE
    assert _run(_args(), ws=FAKE, ws_bytes=16) == lib.IDX_E_WORKSPACE
    assert "workspace" in lib.idx_last_error()
    assert _run(_args(), ws=FAKE + 16, ws_bytes=1 << 20) == lib.IDX_E_INVALID  # misaligned
    assert _run(_args(), plan=FAKE + 8) == lib.IDX_E_INVALID


def test_plan_rejects():
    L = lib.lib()
    assert L.idx_logits_plan(1, 16, 64, 48, 128, None, None, None, FAKE, 1 << 20, None) == lib.IDX_E_UNSUPPORTED
    assert L.idx_logits_plan(1, 16, 64, 64, 128, None, FAKE, None, FAKE, 1 << 20, None) == lib.IDX_E_INVALID
    assert L.idx_logits_plan(1, 16, 64, 64, 128, None, None, None, None, 1 << 20, None) == lib.IDX_E_WORKSPACE
    assert L.idx_logits_plan(1, 16, 64, 64, 128, None, None, None, FAKE, 8, None) == lib.IDX_E_WORKSPACE
    assert L.idx_logits_plan(1, 16, 64, 64, 128, None, None, None, FAKE + 64, 1 << 20, None) == lib.IDX_E_INVALID


@pytest.mark.parametrize("kw,status", [
    (dict(H=24), lib.IDX_E_UNSUPPORTED),
    (dict(in_dtype=9), lib.IDX_E_INVALID),
    (dict(q=None), lib.IDX_E_INVALID),
    (dict(out_row_stride=63), lib.IDX_E_INVALID),
])
def test_prepare_and_score_share_the_checks(kw, status):
    L = lib.lib()
    a = _args(**kw)
    assert L.idx_logits_prepare(ctypes.byref(a), FAKE, 1 << 30, None) == status
    assert L.idx_logits_score(ctypes.byref(a), FAKE, FAKE, 1 << 30, None) == status


def test_prepare_needs_keys():
    L = lib.lib()
    assert L.idx_logits_prepare(ctypes.byref(_args(k=None)), FAKE, 1 << 30, None) == lib.IDX_E_INVALID
    assert L.idx_logits_prepare(ctypes.byref(_args(k_scale=None)), FAKE, 1 << 30, None) == lib.IDX_E_INVALID


def test_prepare_and_score_need_buffers():
    L = lib.lib()
    a = _args()
    assert L.idx_logits_prepare(ctypes.byref(a), None, 0, None) == lib.IDX_E_WORKSPACE
    assert L.idx_logits_prepare(ctypes.byref(a), FAKE, 16, None) == lib.IDX_E_WORKSPACE
    assert L.idx_logits_prepare(ctypes.byref(a), FAKE + 16, 1 << 30, None) == lib.IDX_E_INVALID
    assert L.idx_logits_score(ctypes.byref(a), None, FAKE, 1 << 30, None) == lib.IDX_E_WORKSPACE
    assert "plan" in lib.idx_last_error()
    assert L.idx_logits_score(ctypes.byref(a), FAKE + 8, FAKE, 1 << 30, None) == lib.IDX_E_INVALID
    assert L.idx_logits_score(ctypes.byref(a), FAKE, None, 0, None) == lib.IDX_E_WORKSPACE


def test_plan_thd_rejects():
    L = lib.lib()
    assert L.idx_logits_plan_thd(0, FAKE, FAKE, 2, 16, 8, 64, 128, FAKE, 1 << 20, None) == lib.IDX_E_INVALID
    assert L.idx_logits_plan_thd(2, FAKE, FAKE, 0, 16, 8, 64, 128, FAKE, 1 << 20, None) == lib.IDX_E_INVALID
    assert L.idx_logits_plan_thd(2, None, FAKE, 2, 16, 8, 64, 128, FAKE, 1 << 20, None) == lib.IDX_E_INVALID
    assert L.idx_logits_plan_thd(2, FAKE, FAKE, 2, 16, 8, 4, 128, FAKE, 1 << 20, None) == lib.IDX_E_UNSUPPORTED
    assert L.idx_logits_plan_thd(2, FAKE, FAKE, 2, 0, 8, 64, 128, FAKE, 1 << 20, None) == lib.IDX_E_INVALID
    assert L.idx_logits_plan_thd(2, FAKE, FAKE, 2, 16, 8, 64, 128, None, 1 << 20, None) == lib.IDX_E_WORKSPACE
    assert L.idx_logits_plan_thd(2, FAKE, FAKE, 2, 16, 8, 64, 128, FAKE, 8, None) == lib.IDX_E_WORKSPACE
    assert L.idx_logits_plan_thd(2, FAKE, FAKE, 2, 16, 8, 64, 128, FAKE + 64, 1 << 20, None) == lib.IDX_E_INVALID


def _paged(**kw):
    kv = lib.IdxPagedK()
    kv.k_cache = kv.k_scale_cache = kv.block_table = kv.context_lens = FAKE
    kv.num_pages, kv.page_size, kv.max_pages = 4, 16, 4
    for k, v in kw.items():
        setattr(kv, k, v)
    return kv


@pytest.mark.parametrize("kw,status", [
    (dict(k_cache=None), lib.IDX_E_INVALID),
    (dict(block_table=None), lib.IDX_E_INVALID),
    (dict(context_lens=None), lib.IDX_E_INVALID),
    (dict(k_scale_cache=None), lib.IDX_E_INVALID),
    (dict(k_cache=FAKE + 8), lib.IDX_E_INVALID),
    (dict(k_scale_cache=FAKE + 4), lib.IDX_E_INVALID),
    (dict(num_pages=0), lib.IDX_E_INVALID),
    (dict(page_size=-1), lib.IDX_E_INVALID),
    (dict(max_pages=0), lib.IDX_E_INVALID),
    (dict(max_pages=3), lib.IDX_E_INVALID),  # 3 * 16 < S_k = 64
])
def test_paged_rejects(kw, status):
    L = lib.lib()
    a = _args(k=None, k_scale=None)  # paged calls take no contiguous keys
    kv = _paged(**kw)
    assert L.idx_logits_prepare_paged(ctypes.byref(a), ctypes.byref(kv), FAKE, 1 << 30, None) == status
    assert L.idx_logits_run_paged(ctypes.byref(a), ctypes.byref(kv), None, FAKE, 1 << 30, None) == status
    assert L.idx_logits_score_paged(ctypes.byref(a), ctypes.byref(kv), FAKE, FAKE, 1 << 30, None) == status
    assert lib.idx_last_error() != ""


def test_paged_call_checks():
    L = lib.lib()
    kv = _paged()
    assert L.idx_logits_run_paged(ctypes.byref(_args(H=24)), ctypes.byref(kv), None, FAKE, 1 << 30,
                                  None) == lib.IDX_E_UNSUPPORTED
    assert L.idx_logits_run_paged(ctypes.byref(_args()), None, None, FAKE, 1 << 30, None) == lib.IDX_E_INVALID
    assert L.idx_logits_run_paged(ctypes.byref(_args()), ctypes.byref(kv), None, None, 0, None) == lib.IDX_E_WORKSPACE
    assert L.idx_logits_run_paged(ctypes.byref(_args()), ctypes.byref(kv), FAKE + 8, FAKE, 1 << 30,
                                  None) == lib.IDX_E_INVALID
    assert L.idx_logits_prepare_paged(ctypes.byref(_args()), ctypes.byref(kv), FAKE, 16, None) == lib.IDX_E_WORKSPACE
    # the scoring phase needs a plan, aligned, and a workspace
    assert L.idx_logits_score_paged(ctypes.byref(_args()), ctypes.byref(kv), None, FAKE, 1 << 30,
                                    None) == lib.IDX_E_WORKSPACE
    assert L.idx_logits_score_paged(ctypes.byref(_args()), ctypes.byref(kv), FAKE + 8, FAKE, 1 << 30,
                                    None) == lib.IDX_E_INVALID
    assert L.idx_logits_score_paged(ctypes.byref(_args()), ctypes.byref(kv), FAKE, FAKE, 16,
                                    None) == lib.IDX_E_WORKSPACE
    # BF16 keys carry no scales, so a NULL scale cache is fine there; the
    # call then fails only on its workspace
    a = _args(in_dtype=0, q_scale=None)
    assert L.idx_logits_prepare_paged(ctypes.byref(a), ctypes.byref(_paged(k_scale_cache=None)), None, 0,
                                      None) == lib.IDX_E_WORKSPACE


def test_plan_paged_rejects():
    L = lib.lib()
    assert L.idx_logits_plan_paged(1, 16, 64, 12, 128, FAKE, FAKE, 1 << 20, None) == lib.IDX_E_UNSUPPORTED
    assert L.idx_logits_plan_paged(0, 16, 64, 64, 128, FAKE, FAKE, 1 << 20, None) == lib.IDX_E_INVALID
    assert L.idx_logits_plan_paged(1, 16, 64, 64, 128, None, FAKE, 1 << 20, None) == lib.IDX_E_INVALID
    assert L.idx_logits_plan_paged(1, 16, 64, 64, 128, FAKE, None, 1 << 20, None) == lib.IDX_E_WORKSPACE
    assert L.idx_logits_plan_paged(1, 16, 64, 64, 128, FAKE, FAKE, 8, None) == lib.IDX_E_WORKSPACE
    assert L.idx_logits_plan_paged(1, 16, 64, 64, 128, FAKE, FAKE + 64, 1 << 20, None) == lib.IDX_E_INVALID


def test_topk_rejects():
    L = lib.lib()

    def call(plan=FAKE, B=1, S_q=16, S_k=64, H=64, D=128, logits=FAKE, dt=0, ld=64, k=8, order=0, idx=FAKE,
             val=FAKE):
        return L.idx_logits_topk(plan, B, S_q, S_k, H, D, logits, dt, ld, k, order, idx, val, None)

    assert call(H=24) == lib.IDX_E_UNSUPPORTED
    assert call(B=0) == lib.IDX_E_INVALID
    assert call(plan=None) == lib.IDX_E_WORKSPACE
    assert call(plan=FAKE + 64) == lib.IDX_E_INVALID
    assert call(dt=7) == lib.IDX_E_INVALID
    assert call(logits=None) == lib.IDX_E_INVALID
    assert call(idx=None) == lib.IDX_E_INVALID
    assert call(logits=FAKE + 2) == lib.IDX_E_INVALID   # fp32 scores need 4-byte alignment
    assert call(val=FAKE + 2) == lib.IDX_E_INVALID
    assert call(k=0) == lib.IDX_E_UNSUPPORTED
    assert call(k=lib.MAX_TOPK + 1) == lib.IDX_E_UNSUPPORTED
    assert call(order=2) == lib.IDX_E_INVALID
    assert call(ld=63) == lib.IDX_E_INVALID
    assert "ld" in lib.idx_last_error()


# ---------------------------------------------------------------------------
# the matrix-core throughput probe beside the library (include/idx_peak.h)
# ---------------------------------------------------------------------------

PEAK_HEADER = os.path.join(os.path.dirname(HEADER), "idx_peak.h")
PEAK_LIB = os.path.join(os.path.dirname(lib.LIB_PATH), "libidx_peak.so")


def _peak_lib():
    L = ctypes.CDLL(PEAK_LIB)
    L.idx_peak_mfma.restype = ctypes.c_int32
    L.idx_peak_mfma.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    L.idx_peak_flop_per_mfma.restype = ctypes.c_double
    L.idx_peak_flop_per_mfma.argtypes = [ctypes.c_int32]
    return L


def test_peak_probe_exports_and_checks():
    text = re.sub(r"/\*.*?\*/", "", open(PEAK_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(idx_[a-z_]+)\s*\(", text)))
    assert names == ["idx_peak_flop_per_mfma", "idx_peak_mfma"], names
    L = _peak_lib()
    assert [L.idx_peak_flop_per_mfma(k) for k in range(5)] == [32768.0, 131072.0, 65536.0, 131072.0, 65536.0]
    assert L.idx_peak_flop_per_mfma(9) == 0.0
    # rejected on the host, nothing launched
    assert L.idx_peak_mfma(1, 0, 10, 0, 16, None) == 1
    assert L.idx_peak_mfma(1, 4, 0, 0, 16, None) == 1
    assert L.idx_peak_mfma(1, 4, 10, 0, None, None) == 1
    assert L.idx_peak_mfma(9, 4, 10, 0, 16, None) == 2


@pytest.mark.gpu
def test_peak_probe_runs_every_shape():
    import torch
    L = _peak_lib()
    out = torch.zeros(8 * 256, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for kind in range(5):
        for zero in (0, 1):
            out.zero_()
            assert L.idx_peak_mfma(kind, 8, 3, zero, out.data_ptr(), s) == 0
            torch.cuda.synchronize()
            # every accumulator starts at a nonzero value; zero operands leave it
            assert bool(torch.isfinite(out).all()), (kind, zero)
            if zero:
                # 8 accumulators starting at 1..8, every element summed
                per = 16 if kind in (0, 1, 3) else 4
                assert bool((out == float(per * 36)).all()), (kind, out[:4])


# ---------------------------------------------------------------------------
# workspace sizes: a call given a plan needs no plan bytes; the accumulate
# field is checked like the others
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
@pytest.mark.parametrize("accum", [0, 1])
def test_workspace_sizes_and_checks(fmt, accum):
    L = lib.lib()
    a = _args(in_dtype=fmt, accumulate=accum, **({"q_scale": None, "k_scale": None} if fmt == 0 else {}))
    total = lib.idx_logits_workspace_bytes(a)
    planned = lib.idx_logits_workspace_bytes_planned(a)
    plan_bytes = lib.idx_logits_plan_bytes(a.B, a.S_q, a.S_k, a.H, a.D)
    assert 0 < planned < total and total - planned == plan_bytes
    # K in fragment order is always there: 32-key blocks of 256 (bf16
    # operands), 128 (e4m3) or 64 (e2m1) bytes per key
    conv = accum == 1 and fmt in (1, 2)
    row = 256 if (fmt == 0 or conv) else (64 if fmt == 3 else 128)
    assert planned >= 64 * row
    if conv:  # Q converted to bf16: rows x H x 256 bytes
        assert planned >= a.B * a.S_q * a.H * 256
    # a planned call is checked against the planned size, an unplanned one
    # against the total (both fail before any launch here)
    assert _run(a, plan=FAKE, ws=FAKE, ws_bytes=planned - 1) == lib.IDX_E_WORKSPACE
    assert _run(a, plan=None, ws=FAKE, ws_bytes=total - 1) == lib.IDX_E_WORKSPACE
    assert str(total) in lib.idx_last_error()
    assert L.idx_logits_prepare(ctypes.byref(a), FAKE, planned - 1, None) == lib.IDX_E_WORKSPACE
    assert L.idx_logits_score(ctypes.byref(a), FAKE, FAKE, planned - 1, None) == lib.IDX_E_WORKSPACE
    assert str(planned) in lib.idx_last_error()


def test_accumulate_mode_is_checked():
    for bad in (2, -1, 7):
        a = _args(accumulate=bad)
        assert _run(a, plan=FAKE, ws=FAKE, ws_bytes=1 << 30) == lib.IDX_E_INVALID
        assert "accumulate" in lib.idx_last_error()
        assert lib.idx_logits_workspace_bytes(a) == 0 and lib.idx_logits_workspace_bytes_planned(a) == 0


def test_exact_accumulation_only_changes_the_e4m3_formats():
    for fmt, changes in ((0, False), (1, True), (2, True), (3, False)):
        kw = {"q_scale": None, "k_scale": None} if fmt == 0 else {}
        a0 = _args(in_dtype=fmt, accumulate=0, **kw)
        a1 = _args(in_dtype=fmt, accumulate=1, **kw)
        same = lib.idx_logits_workspace_bytes(a0) == lib.idx_logits_workspace_bytes(a1)
        assert same != changes, fmt


def test_plan_windows_rejects():
    L = lib.lib()
    assert L.idx_logits_plan_windows(FAKE + 64, 1, 16, 64, 64, 128, FAKE, FAKE, None) == lib.IDX_E_INVALID
    assert L.idx_logits_plan_windows(FAKE, 1, 16, 64, 64, 128, FAKE + 2, FAKE, None) == lib.IDX_E_INVALID
    assert L.idx_logits_plan_windows(FAKE, 1, 16, 64, 64, 128, FAKE, FAKE + 1, None) == lib.IDX_E_INVALID
    assert L.idx_logits_plan_windows(None, 1, 16, 64, 64, 128, FAKE, FAKE, None) == lib.IDX_E_INVALID
    assert L.idx_logits_plan_windows(FAKE, 1, 16, 64, 24, 128, FAKE, FAKE, None) == lib.IDX_E_UNSUPPORTED


# ---------------------------------------------------------------------------
# fused scoring + top-k (idx_logits_run_topk): host-side checks only
# ---------------------------------------------------------------------------

def _run_topk(a, k=8, order=0, idx=FAKE, val=FAKE, n_redo=None, plan=None, ws=FAKE, ws_bytes=1 << 40):
    return lib.lib().idx_logits_run_topk(ctypes.byref(a), plan, None, None, None, k, order, idx, val, n_redo, ws,
                                         ws_bytes, None)


def test_run_topk_rejects():
    # out is not used: NULL or misaligned out passes the checks that fail here
    a = _args(out=None, out_row_stride=0)
    assert _run_topk(a, k=0) == lib.IDX_E_UNSUPPORTED
    assert _run_topk(a, k=lib.MAX_TOPK + 1) == lib.IDX_E_UNSUPPORTED
    assert _run_topk(a, order=2) == lib.IDX_E_INVALID
    assert _run_topk(a, idx=None) == lib.IDX_E_INVALID
    assert _run_topk(a, idx=FAKE + 2) == lib.IDX_E_INVALID
    assert _run_topk(a, val=FAKE + 1) == lib.IDX_E_INVALID
    assert _run_topk(a, n_redo=FAKE + 1) == lib.IDX_E_INVALID
    assert _run_topk(a, plan=FAKE + 64) == lib.IDX_E_INVALID
    assert _run_topk(a, ws=None) == lib.IDX_E_WORKSPACE
    assert "idx_logits_topk_workspace_bytes" in lib.idx_last_error()
    assert _run_topk(a, ws=FAKE + 16) == lib.IDX_E_INVALID
    need = lib.idx_logits_topk_workspace_bytes(a)
    assert _run_topk(a, ws_bytes=need - 1) == lib.IDX_E_WORKSPACE
    assert str(need) in lib.idx_last_error()
    for kw, st in ((dict(H=24), lib.IDX_E_UNSUPPORTED), (dict(q=None), lib.IDX_E_INVALID),
                   (dict(k_scale=None), lib.IDX_E_INVALID), (dict(in_dtype=9), lib.IDX_E_INVALID),
                   (dict(accumulate=3), lib.IDX_E_INVALID), (dict(sm_scale=float("nan")), lib.IDX_E_INVALID)):
        assert _run_topk(_args(out=None, **kw)) == st, kw


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_topk_workspace_holds_the_candidates(fmt):
    kw = {"q_scale": None, "k_scale": None} if fmt == 0 else {}
    for B, S_q, S_k in ((1, 16, 64), (2, 300, 5000), (1, 2048, 32768)):
        a = _args(in_dtype=fmt, B=B, S_q=S_q, S_k=S_k, out=None, **kw)
        total = lib.idx_logits_topk_workspace_bytes(a)
        base = lib.idx_logits_workspace_bytes(_args(in_dtype=fmt, B=B, S_q=S_q, S_k=S_k, out_row_stride=S_k, **kw))
        # the scoring call's own sections, then at least one (score, column)
        # pair per cell and the sample's scores (S_k / 16 columns per row)
        assert total >= base + 8 * B * S_q * S_k + 4 * B * S_q * (S_k // 16)
    assert lib.idx_logits_topk_workspace_bytes(_args(H=24)) == 0
