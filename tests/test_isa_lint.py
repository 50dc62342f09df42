"""Static checks on the gfx950 device code of the scoring kernels (CPU only).

The kernels rely on two properties that the compiler is free to break and no
parity test is sure to notice:

* No matrix instruction runs under a partial exec mask.  An MFMA writes every
  lane of its result whatever the exec mask says, so if the compiler sinks one
  into a divergent branch (it does so for a select on a lane-varying
  condition whose operand is an MFMA result), the masked-off lanes lose what
  the compiler assumed they still hold.
* No scratch: a spill in the main loop brings a full memory wait with it.
* No waterfall loop (a loop that takes a buffer resource held in vector
  registers one distinct value at a time) where the work is: between the
  first and last matrix instruction of a scoring kernel, or anywhere in the
  top-k kernels.  The compiler builds one when it cannot prove a resource's
  base or size the same in every lane (a wave index taken from the thread
  index without readfirstlane did that to every load of the top-k stream).

The check compiles each score source to device assembly and walks it in text
order: an if-region opens at s_and_saveexec / s_or_saveexec and closes at the
s_or_b64 exec restore of the same saved mask; a loop's exit mask opens at
s_andn2_b64 exec and closes at its restore; an unconditional branch or the end
of the program resets the state (the next label is entered with a full mask in
these kernels).  This is a conservative approximation of the control flow, so
a finding is a reason to read the assembly, not proof of a bug.
"""

from __future__ import annotations

import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from mqa_logits_scoring_amd import build as hip_build

SCORE_SOURCES = ["score_bf16.hip", "score_bf16rs.hip", "score_fp8.hip", "score_mxfp8.hip", "score_mxfp4.hip"]


def device_asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, src + ".s")
    cmd = [hip_build.hipcc(), *hip_build.flags_for(src), "--cuda-device-only", "-S",
           os.path.join(hip_build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr}"
    with open(out) as f:
        return f.read()


def mfma_under_partial_exec(asm: str) -> list[str]:
    """Lines of MFMA instructions that may run with part of the wave masked off."""
    found = []
    kern = None
    stack: list[str] = []  # saved-mask registers of the open regions
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            kern, stack = m.group(1), []
            continue
        s = line.split(";")[0].strip()
        if not s:
            continue
        m_if = re.match(r"s_(?:and|or)_saveexec_b64 (s\[\d+:\d+\])", s)
        m_loop = re.match(r"s_andn2_b64 exec, exec, (s\[\d+:\d+\])", s)
        m_end = re.match(r"s_or_b64 exec, exec, (s\[\d+:\d+\])", s)
        if m_if:
            stack.append(m_if.group(1))
        elif m_loop:
            if m_loop.group(1) not in stack:
                stack.append(m_loop.group(1))
        elif m_end:
            if m_end.group(1) in stack:
                while stack and stack.pop() != m_end.group(1):
                    pass
        elif s.startswith("s_branch") or s.startswith("s_endpgm"):
            stack = []
        elif s.startswith("v_mfma") and stack:
            found.append(f"{kern}: {s}")
    return found


def private_segment_sizes(asm: str) -> dict[str, int]:
    sizes = {}
    kern = None
    for line in asm.splitlines():
        m = re.match(r"\s*\.amdhsa_kernel (\S+)", line)
        if m:
            kern = m.group(1)
        m = re.match(r"\s*\.amdhsa_private_segment_fixed_size (\d+)", line)
        if m and kern:
            sizes[kern] = int(m.group(1))
    return sizes


def waterfall_loops(asm: str, hot_only: bool) -> list[str]:
    """Kernels and lines of waterfall loops: a compare of a 64-bit value in
    scalar registers with vector registers, followed within a few
    instructions by an exec save, a buffer or global access and the exec
    mask's flip that loops back.  hot_only: only those between the kernel's
    first and last matrix instruction."""
    found = []
    for m in re.finditer(r"^(_Z\w+):", asm, re.M):
        start = m.end()
        end = asm.find(".Lfunc_end", start)
        lines = [l.split(";")[0].strip() for l in asm[start:end].splitlines()]
        mf = [i for i, l in enumerate(lines) if l.startswith("v_mfma")]
        lo, hi = (mf[0], mf[-1]) if (hot_only and mf) else (0, len(lines))
        if hot_only and not mf:
            continue
        for i in range(lo, hi):
            l = lines[i]
            if l.startswith("v_cmp_eq_u64") and ", s[" in l:
                win = lines[i:i + 8]
                if (any("saveexec" in x for x in win) and any(x.startswith(("buffer_", "global_")) for x in win)
                        and any(x.startswith("s_xor_b64 exec") for x in win)):
                    found.append(f"{m.group(1)}: line {i}")
    return found


@pytest.fixture(scope="module")
def score_asm(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("asm"))
    with ThreadPoolExecutor(max_workers=4) as ex:
        return dict(zip(SCORE_SOURCES, ex.map(lambda s: device_asm(s, d), SCORE_SOURCES)))


def test_checker_flags_sunk_mfma():
    """The walker itself: an MFMA inside an if-region is found, one after the
    restore or after an unconditional branch is not."""
    asm = "\n".join([
        "_Zkern:",
        "  v_cmp_ge_i32_e32 vcc, v1, v2",
        "  s_and_saveexec_b64 s[0:1], vcc",
        "  v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
        "  s_or_b64 exec, exec, s[0:1]",
        "  v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
        "  s_and_saveexec_b64 s[2:3], vcc",
        "  s_branch .LBB0_1",
        ".LBB0_1:",
        "  v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
    ])
    assert len(mfma_under_partial_exec(asm)) == 1


@pytest.mark.parametrize("src", SCORE_SOURCES)
def test_no_mfma_under_partial_exec(score_asm, src):
    bad = mfma_under_partial_exec(score_asm[src])
    assert not bad, f"{src}: {len(bad)} MFMA may run under a partial exec mask, e.g. {bad[:3]}"


@pytest.mark.parametrize("src", SCORE_SOURCES)
def test_no_scratch(score_asm, src):
    sizes = private_segment_sizes(score_asm[src])
    assert sizes, f"{src}: no kernel descriptors found"
    spilled = {k: v for k, v in sizes.items() if v}
    assert not spilled, f"{src}: kernels use scratch: {spilled}"


def test_checker_flags_waterfall():
    asm = "\n".join([
        "_Zkern:",
        "  v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
        ".LBB0_1:",
        "  v_readfirstlane_b32 s8, v46",
        "  v_cmp_eq_u64_e32 vcc, s[8:9], v[46:47]",
        "  s_and_saveexec_b64 s[4:5], vcc",
        "  buffer_store_dword v9, v4, s[8:11], 0 offen",
        "  s_xor_b64 exec, exec, s[4:5]",
        "  s_cbranch_execnz .LBB0_1",
        "  v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
        ".Lfunc_end0:",
    ])
    assert len(waterfall_loops(asm, hot_only=True)) == 1
    assert not waterfall_loops(asm.replace("buffer_store_dword", "v_mov_b32"), hot_only=False)


@pytest.mark.parametrize("src", SCORE_SOURCES)
def test_no_waterfall_in_scoring_loops(score_asm, src):
    bad = waterfall_loops(score_asm[src], hot_only=True)
    assert not bad, f"{src}: {len(bad)} waterfall loops among the matrix instructions, e.g. {bad[:3]}"


@pytest.mark.parametrize("src", ["topk.hip", "topk_fused.hip"])
def test_no_waterfall_in_topk(src, tmp_path):
    bad = waterfall_loops(device_asm(src, str(tmp_path)), hot_only=False)
    assert not bad, f"{src}: {len(bad)} waterfall loops, e.g. {bad[:3]}"
