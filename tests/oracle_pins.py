"""Pins for the fp64 oracle: facts fixed by the pages or by mathematics, each
checked through a route that does not reuse the oracle's own code.

Every pin is a function taking an `oracle.Oracle` and raising AssertionError
when the oracle disagrees.  `tests/test_oracle.py` runs them against the real
oracle; `tests/test_oracle_mutations.py` runs them against deliberately broken
copies of it (built on the CPU) to show that each plausible mistake is caught.

Independent decoders used here: torch's bfloat16, float8_e4m3fn and
float8_e8m0fnu casts, and the literal E2M1 table in tests/golden/.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# independent decoding of workload codes (torch casts + literal table)
# --------------------------------------------------------------------------

def e2m1_table() -> dict[int, float]:
    tab = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            tab[int(c)] = float(v)
    return tab


def t_bf16(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def t_e4m3(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def t_e8m0(bytes_: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bytes_)).view(torch.float8_e8m0fnu).to(torch.float64).numpy()


def t_e2m1_unpacked(packed: np.ndarray) -> np.ndarray:
    tab = np.array([e2m1_table()[c] for c in range(16)])
    lo = tab[packed & 0xF]
    hi = tab[packed >> 4]
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,))
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def block_scales(words: np.ndarray, D: int) -> np.ndarray:
    """uint32 words [...] -> per-element scale [..., D] through a little-endian byte view."""
    by = np.ascontiguousarray(words.astype("<u4")).view(np.uint8).reshape(words.shape + (4,))
    s = t_e8m0(by)  # [..., 4]
    return np.repeat(s[..., : D // 32], 32, axis=-1)


def indep_dequant(wl):
    """(Qd [B,S_q,H,D], Kd [B,S_k,D], Wd [B,S_q,H]) as float64."""
    if wl.fmt == "bf16":
        Qd, Kd = t_bf16(wl.q), t_bf16(wl.k)
    elif wl.fmt in ("fp8", "mxfp8"):
        Qd, Kd = t_e4m3(wl.q), t_e4m3(wl.k)
    else:
        Qd, Kd = t_e2m1_unpacked(wl.q), t_e2m1_unpacked(wl.k)
    if wl.fmt == "fp8":
        Kd = Kd * wl.k_scale.astype(np.float64)[..., None]
    if wl.fmt in ("mxfp8", "mxfp4"):
        Qd = Qd * block_scales(wl.q_scale, wl.D)
        Kd = Kd * block_scales(wl.k_scale, wl.D)
    Wd = t_bf16(wl.w) if wl.w_dtype == "bf16" else wl.w.astype(np.float64)
    return Qd, Kd, Wd


def brute_scores(wl, ws, we):
    """numpy fp64 einsum over independently decoded inputs; -inf outside [ws, we)."""
    Qd, Kd, Wd = indep_dequant(wl)
    S = np.einsum("bihd,bjd->bihj", Qd, Kd)
    sc = wl.sm_scale * np.einsum("bih,bihj->bij", Wd, np.maximum(S, 0.0))
    j = np.arange(wl.S_k)
    inside = (j[None, None, :] >= ws[..., None]) & (j[None, None, :] < we[..., None])
    return np.where(inside, sc, -np.inf)


def full(orc, wl):
    ref, bound = orc.logits(wl)
    return ref.reshape(wl.B, wl.S_q, wl.S_k), bound.reshape(wl.B, wl.S_q, wl.S_k)


# --------------------------------------------------------------------------
# code writers for exactly representable values (input construction)
# --------------------------------------------------------------------------

def codes_for(fmt: str, values: np.ndarray) -> np.ndarray:
    """Exactly representable values -> element codes (unpacked for mxfp4)."""
    v = np.asarray(values, np.float64)
    if fmt == "bf16":
        out = W.bf16_bits(torch.from_numpy(v.astype(np.float32)))
        assert np.array_equal(t_bf16(out), v)
    elif fmt in ("fp8", "mxfp8"):
        out = W.e4m3_codes(torch.from_numpy(v.astype(np.float32)))
        assert np.array_equal(t_e4m3(out), v)
    else:
        out = W.e2m1_codes(v)
        tab = e2m1_table()
        assert all(tab[int(c)] == x for c, x in zip(out.ravel(), v.ravel()))
    return out


def pack(fmt: str, codes: np.ndarray) -> np.ndarray:
    return W.pack_nibbles(codes) if fmt == "mxfp4" else codes


def blank(fmt: str, B: int, S_q: int, S_k: int, H: int = 64, D: int = 128, w_dtype="f32", sm_scale=1.0,
          offsets=None, starts=None, ends=None):
    """Workload with all-zero codes, unit scales and zero weights, to be filled in."""
    wl = W.make_random(fmt, B, S_q, S_k, H, D, zero=True, w_dtype=w_dtype, sm_scale=sm_scale,
                       windows="explicit" if starts is not None else "offsets",
                       offsets=offsets if offsets is not None else [S_q - 1] * B, starts=starts, ends=ends)
    wl.w[...] = 0
    return wl


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

def pin_decoders(orc):
    """Element decoders equal torch's casts (bf16, e4m3fn, e8m0) and the OCP E2M1 table."""
    bits = np.arange(0, 1 << 16, 97, dtype=np.uint16)
    ref = t_bf16(bits)
    for b, r in zip(bits, ref):
        v = orc.decode("bf16", int(b))
        assert (math.isnan(v) and math.isnan(r)) or v == r, ("bf16", b, v, r)
    codes = np.arange(256, dtype=np.uint8)
    for name, ref in (("e4m3", t_e4m3(codes)), ("e8m0", t_e8m0(codes))):
        for c, r in zip(codes, ref):
            v = orc.decode(name, int(c))
            assert (math.isnan(v) and math.isnan(r)) or (v == r and math.copysign(1, v) == math.copysign(1, r)), \
                (name, c, v, r)
    for c, r in e2m1_table().items():
        v = orc.decode("e2m1", c)
        assert v == r and math.copysign(1, v) == math.copysign(1, r), ("e2m1", c, v, r)


def pin_zero_workload(orc):
    """All-zero Q/K, any W, unit scales: 0 inside [0, KV-Q+row), -inf outside (golden fixture)."""
    g = json.load(open(os.path.join(GOLDEN, "zero_workload.json")))
    for case in g["cases"]:
        m, n = case["m"], case["n"]
        starts = np.zeros((1, m), np.int32)
        ends = (np.arange(m) + n - m).astype(np.int32)[None]
        for fmt in case["formats"]:
            wl = W.make_random(fmt, 1, m, n, zero=True, windows="explicit", starts=starts, ends=ends, seed=11)
            if fmt in ("mxfp8", "mxfp4"):
                assert int(wl.q_scale.ravel()[0]) == g["scale_word_all_one"]
            ref, _ = full(orc, wl)
            cols = np.arange(n)[None, :]
            valid = cols < ends[0][:, None]
            assert np.array_equal(np.isneginf(ref[0]), ~valid), fmt
            assert np.all(ref[0][valid] == 0.0), fmt


def pin_brute_force(orc):
    """Tiny shapes: oracle == numpy einsum over torch-decoded inputs (all formats, both W types)."""
    rng = np.random.default_rng(7)
    for fmt in W.FORMATS:
        for (H, D) in ((64, 128), (3, 32)):
            for w_dtype in ("f32", "bf16"):
                B, S_q, S_k = 2, 5, 37
                st = rng.integers(-3, S_k, size=(B, S_q)).astype(np.int32)
                en = (st + rng.integers(-2, S_k, size=(B, S_q))).astype(np.int32)
                st[0, 0], en[0, 0] = 4, 4  # empty row
                wl = W.make_random(fmt, B, S_q, S_k, H, D, w_dtype=w_dtype, sm_scale=0.37, seed=int(rng.integers(1000000)),
                                   windows="explicit", starts=st, ends=en)
                ws = np.clip(st, 0, S_k)
                we = np.clip(np.maximum(en, ws), 0, S_k)
                exp = brute_scores(wl, ws, we)
                ref, bound = full(orc, wl)
                assert np.array_equal(np.isneginf(ref), np.isneginf(exp)), (fmt, H, D, w_dtype)
                fin = ~np.isneginf(exp)
                err = np.abs(ref[fin] - exp[fin])
                assert np.all(err <= 1e-12 * bound[fin] + 1e-300), (fmt, H, D, w_dtype, err.max())


def pin_one_hot(orc):
    """q[i,h,:] = a_ih e_d0, k[j,:] = b_j e_d0 (+ junk where q is zero):
    score = sm_scale * sum_h w_ih * max(a_ih b_j, 0), exact."""
    d0 = 37
    for fmt in W.FORMATS:
        S_q, S_k, H, D = 3, 7, 64, 128
        wl = blank(fmt, 1, S_q, S_k, H, D, sm_scale=0.25)
        a = np.array([[(1.0 if (h + i) % 3 else -2.0) * (0.5 if h % 5 == 0 else 1.0) for h in range(H)]
                      for i in range(S_q)])
        b = np.array([1.0, -1.0, 2.0, 0.0, -0.5, 3.0, 1.5])
        qv = np.zeros((1, S_q, H, D))
        qv[0, :, :, d0] = a
        kv = np.zeros((1, S_k, D))
        kv[0, :, d0] = b
        kv[0, :, d0 + 1] = 4.0   # q is zero there
        kv[0, :, 0] = -6.0
        wv = np.array([[2.0 ** -(h % 4) * (1 if h % 7 else -1) for h in range(H)] for _ in range(S_q)])
        wl.q = pack(fmt, codes_for(fmt, qv))
        wl.k = pack(fmt, codes_for(fmt, kv))
        wl.w = wv[None].astype(np.float32)
        if fmt == "mxfp8" or fmt == "mxfp4":
            # block d0//32 of every Q row scaled by 2^1, of every K row by 2^-1: net 1
            byte = d0 // 32
            sq = np.full(4, 127, np.uint8)
            sq[byte] = 128
            sk = np.full(4, 127, np.uint8)
            sk[byte] = 126
            wl.q_scale = np.full((1, S_q, H), W.pack_e8m0(sq), np.uint32)
            wl.k_scale = np.full((1, S_k), W.pack_e8m0(sk), np.uint32)
        ref, _ = full(orc, wl)
        for i in range(S_q):
            for j in range(S_k):
                exp = 0.25 * sum(wv[i, h] * max(a[i, h] * b[j], 0.0) for h in range(H))
                assert ref[0, i, j] == exp, (fmt, i, j, ref[0, i, j], exp)


def pin_rank_one(orc):
    """q[i,h] = s_h u, k[j] = t_j u: score = sm_scale * sum_h w_h * max(s_h t_j |u|^2, 0), exact;
    error scale = |sm_scale| |t_j| |u|^2 sum_h |w_h| |s_h|."""
    for fmt in W.FORMATS:
        S_q, S_k, H, D = 2, 5, 64, 128
        wl = blank(fmt, 1, S_q, S_k, H, D, sm_scale=0.5, w_dtype="bf16")
        u = np.array([[0.0, 0.5, -1.0, 1.0, -0.5][d % 5] for d in range(D)])
        u2 = float(np.sum(u * u))
        sgn = np.array([1.0 if h % 3 else -1.0 for h in range(H)])
        e_h = np.array([h % 3 - 1 for h in range(H)])          # Q scale exponent per head
        t = np.array([1.0, -1.0, 0.5, 2.0, -0.25])
        if fmt in ("mxfp8", "mxfp4"):
            qv = np.broadcast_to(sgn[None, None, :, None] * u, (1, S_q, H, D))
            kv = np.broadcast_to(np.sign(t)[None, :, None] * u, (1, S_k, D))
            qs = np.zeros((1, S_q, H), np.uint32)
            for h in range(H):
                qs[0, :, h] = W.pack_e8m0(np.full(4, 127 + e_h[h], np.uint8))
            ks = np.zeros((1, S_k), np.uint32)
            for j in range(S_k):
                ks[0, j] = W.pack_e8m0(np.full(4, 127 + int(np.log2(abs(t[j]))), np.uint8))
            wl.q_scale, wl.k_scale = qs, ks
            s = sgn * 2.0 ** e_h
        else:
            s = sgn * 2.0 ** e_h
            qv = np.broadcast_to(s[None, None, :, None] * u, (1, S_q, H, D))
            kv = np.broadcast_to(t[None, :, None] * u, (1, S_k, D))
            if fmt == "fp8":   # fold t_j's magnitude into the per-row fp32 scale
                kv = np.broadcast_to(np.sign(t)[None, :, None] * u, (1, S_k, D))
                wl.k_scale = np.abs(t)[None].astype(np.float32)
        wl.q = pack(fmt, codes_for(fmt, np.ascontiguousarray(qv)))
        wl.k = pack(fmt, codes_for(fmt, np.ascontiguousarray(kv)))
        wv = np.array([(h % 4 - 1.5) / 4 for h in range(H)])
        wl.w = W.bf16_bits(torch.from_numpy(np.tile(wv, (1, S_q, 1)).astype(np.float32)))
        ref, bound = full(orc, wl)
        for i in range(S_q):
            for j in range(S_k):
                exp = 0.5 * sum(wv[h] * max(s[h] * t[j] * u2, 0.0) for h in range(H))
                assert ref[0, i, j] == exp, (fmt, i, j, ref[0, i, j], exp)
                # parallel rows: |q_h| |k_j| = |s_h| |t_j| |u|^2, so the error scale is known
                exp_b = 0.5 * abs(t[j]) * u2 * sum(abs(wv[h]) * abs(s[h]) for h in range(H))
                assert abs(bound[0, i, j] - exp_b) <= 1e-14 * exp_b, (fmt, i, j, bound[0, i, j], exp_b)


def pin_matmul_reduction(orc):
    """w[i,:] = e_h0 and non-negative Q, K: ReLU is the identity, score = sm_scale * (Q_h0 K^T)."""
    for fmt in W.FORMATS:
        wl = W.make_random(fmt, 1, 6, 45, seed=5, sm_scale=0.75, offsets=[100])
        if fmt == "bf16":
            wl.q &= 0x7FFF
            wl.k &= 0x7FFF
        elif fmt in ("fp8", "mxfp8"):
            wl.q &= 0x7F
            wl.k &= 0x7F
            wl.q[wl.q == 0x7F] = 0x7E
            wl.k[wl.k == 0x7F] = 0x7E
        else:
            wl.q &= 0x77
            wl.k &= 0x77
        h0 = 29
        wl.w = np.zeros_like(wl.w)
        wl.w[:, :, h0] = 1.0
        Qd, Kd, _ = indep_dequant(wl)
        exp = 0.75 * np.matmul(Qd[0, :, h0, :], Kd[0].T)
        ref, bound = full(orc, wl)
        assert np.all(np.abs(ref[0] - exp) <= 1e-12 * bound[0] + 1e-300), fmt


def pin_scaling_invariants(orc):
    """Exact relations: W * 2^k -> out * 2^k; every K (then Q) E8M0 byte + 1 -> out * 2;
    FP8 k_scale * 4 -> out * 4."""
    for fmt in W.FORMATS:
        wl = W.make_random(fmt, 1, 4, 33, seed=9, sm_scale=0.5, offsets=[-3])
        base, _ = full(orc, wl)
        fin = ~np.isneginf(base)
        w2 = wl.replace(w=(wl.w * np.float32(8.0)))
        r2, _ = full(orc, w2)
        assert np.array_equal(r2[fin], base[fin] * 8.0), fmt
        if fmt in ("mxfp8", "mxfp4"):
            r3, _ = full(orc, wl.replace(k_scale=(wl.k_scale + np.uint32(0x01010101)).astype(np.uint32)))
            assert np.array_equal(r3[fin], base[fin] * 2.0), fmt
            r4, _ = full(orc, wl.replace(q_scale=(wl.q_scale + np.uint32(0x01010101)).astype(np.uint32)))
            assert np.array_equal(r4[fin], base[fin] * 2.0), fmt
        if fmt == "fp8":
            r5, _ = full(orc, wl.replace(k_scale=(wl.k_scale * np.float32(4.0)).astype(np.float32)))
            assert np.array_equal(r5[fin], base[fin] * 4.0), fmt


def pin_mx_block_layout(orc):
    """Codes only in d-block b: raising scale byte b doubles the output, raising any
    other byte changes nothing; an MXFP4 code in the low nibble of byte 0 is element 0."""
    for fmt in ("mxfp8", "mxfp4"):
        for blk in range(4):
            wl = W.make_random(fmt, 1, 3, 20, seed=20 + blk, offsets=[17])
            qv = np.zeros((1, 3, 64, 128))
            kv = np.zeros((1, 20, 128))
            rng = np.random.default_rng(blk)
            vals = np.array([0.5, 1.0, -1.0, 2.0, -0.5, 1.5])
            qv[..., 32 * blk:32 * blk + 32] = rng.choice(vals, size=(1, 3, 64, 32))
            kv[..., 32 * blk:32 * blk + 32] = rng.choice(vals, size=(1, 20, 32))
            wl.q = pack(fmt, codes_for(fmt, qv))
            wl.k = pack(fmt, codes_for(fmt, kv))
            base, _ = full(orc, wl)
            fin = ~np.isneginf(base)
            assert np.any(base[fin] != 0)
            for which in ("q", "k"):
                for byte in range(4):
                    bump = np.uint32(1 << (8 * byte))
                    if which == "q":
                        r, _ = full(orc, wl.replace(q_scale=(wl.q_scale + bump).astype(np.uint32)))
                    else:
                        r, _ = full(orc, wl.replace(k_scale=(wl.k_scale + bump).astype(np.uint32)))
                    want = base * 2.0 if byte == blk else base
                    assert np.array_equal(r[fin], want[fin]), (fmt, blk, which, byte)
    # nibble order: Q code 1.0 only at element 0 (low nibble of byte 0); K has 2.0 at
    # element 0 and -3.0 at element 1 (high nibble of byte 0)
    wl = blank("mxfp4", 1, 1, 1, offsets=[0])
    q = np.zeros((1, 1, 64, 64), np.uint8)
    q[..., 0] = 0x02                       # low nibble: code 2 = 1.0
    k = np.zeros((1, 1, 64), np.uint8)
    k[..., 0] = 0x04 | (0x0D << 4)         # low nibble code 4 = 2.0, high nibble code 13 = -3.0
    w = np.zeros((1, 1, 64), np.float32)
    w[..., 5] = 1.0
    r, _ = full(orc, wl.replace(q=q, k=k, w=w))
    assert r[0, 0, 0] == 2.0, r[0, 0, 0]
    q[..., 0] = 0x02 << 4                  # now element 1 holds 1.0: dot = -3 -> ReLU 0
    r, _ = full(orc, wl.replace(q=q, k=k, w=w))
    assert r[0, 0, 0] == 0.0, r[0, 0, 0]
    w[..., 5] = -1.0
    q[..., 0] = (0x0A << 4)                # element 1 holds -1.0: dot = 3 -> -3 after the weight
    r, _ = full(orc, wl.replace(q=q, k=k, w=w))
    assert r[0, 0, 0] == -3.0, r[0, 0, 0]


def pin_format_consistency(orc):
    """MXFP8 with unit scales == FP8 with k_scale 1; MXFP4 codes re-encoded as e4m3 give the same scores."""
    mx = W.make_random("mxfp8", 1, 4, 40, seed=31, offsets=[0], zero=False)
    mx.q_scale[...] = W.ONE_SCALE_WORD
    mx.k_scale[...] = W.ONE_SCALE_WORD
    f8 = mx.replace(fmt="fp8", q_scale=None, k_scale=np.ones((1, 40), np.float32))
    a, _ = full(orc, mx)
    b, _ = full(orc, f8)
    assert np.array_equal(a, b)
    m4 = W.make_random("mxfp4", 1, 4, 40, seed=32, offsets=[0])
    m4.q_scale[...] = W.ONE_SCALE_WORD
    m4.k_scale[...] = W.ONE_SCALE_WORD
    qv = t_e2m1_unpacked(m4.q)
    kv = t_e2m1_unpacked(m4.k)
    as8 = m4.replace(fmt="fp8", q=codes_for("fp8", qv), k=codes_for("fp8", kv), q_scale=None,
                     k_scale=np.ones((1, 40), np.float32))
    a, _ = full(orc, m4)
    b, _ = full(orc, as8)
    assert np.array_equal(a, b)


def pin_windows_named(orc):
    """Windows of the pages' workloads: offset 0 gives row i [0, S_k-S_q+i+1) (tiny causal
    and BF16 batch workloads); the MX reproducer's ends = arange(m)+n-m equal offset -1."""
    for name, S_q, S_k, B in (("c1", 128, 512, 1), ("c2", 2048, 4096, 4)):
        wl = W.make(name) if name == "c1" else W.make_random("bf16", B, S_q, S_k, H=1, D=2, offsets=[0] * B)
        ws, we = orc.windows(wl)
        assert np.all(ws == 0)
        assert np.array_equal(we, np.tile(np.arange(S_q) + S_k - S_q + 1, (B, 1)))
    m, n = 2048, 32768
    wl = W.make_random("fp8", 1, m, n, H=1, D=2, offsets=[-1])
    ws, we = orc.windows(wl)
    assert np.all(ws == 0) and np.array_equal(we[0], np.arange(m) + n - m)
    wl2 = W.make_random("fp8", 1, m, n, H=1, D=2, windows="explicit", starts=np.zeros((1, m)),
                        ends=(np.arange(m) + n - m)[None])
    ws2, we2 = orc.windows(wl2)
    assert np.array_equal(ws, ws2) and np.array_equal(we, we2)


def pin_windows_clamp(orc):
    """Clamping: start<0 -> 0, end>S_k -> S_k, end<start -> empty; extreme offsets do not overflow."""
    S_k = 50
    st = np.array([[-5, 10, 60, 30, 7, 0]], np.int32)
    en = np.array([[20, 70, 80, 10, 7, 50]], np.int32)
    wl = W.make_random("bf16", 1, 6, S_k, H=1, D=2, windows="explicit", starts=st, ends=en)
    ws, we = orc.windows(wl)
    assert ws.tolist() == [[0, 10, 50, 30, 7, 0]] and we.tolist() == [[20, 50, 50, 30, 7, 50]]
    i32 = np.iinfo(np.int32)
    wl = W.make_random("bf16", 3, 4, S_k, H=1, D=2, offsets=[i32.max, i32.min, -49])
    ws, we = orc.windows(wl)
    assert np.all(ws == 0)
    assert we.tolist() == [[50] * 4, [0] * 4, [0, 0, 0, 1]]


def pin_windows_thd_golden(orc):
    """Packed variable-length windows over ratio-compressed keys against the hand-worked
    cases of tests/golden/thd_windows.json (cudnn-frontend pull request 416, THD commit)."""
    with open(os.path.join(GOLDEN, "thd_windows.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        ws, we = orc.windows_thd(c["cu_q"], c["cu_k"], c["ratio"], c["T_q"], c["m_total"])
        assert ws.tolist() == c["starts"] and we.tolist() == c["ends"], c["what"]


def pin_windows_thd_structure(orc):
    """THD windows: one segment at ratio 1 is the causal mask [0, t+1); every window stays
    inside its segment's keys; ends never fall within a segment and grow by at most one key
    per row; a segment whose length is a multiple of the ratio ends seeing all its keys; and
    each key count v >= 1 below the last is seen by exactly `ratio` consecutive rows."""
    T = 37
    ws, we = orc.windows_thd([0, T], [0, T], 1, T, T)
    assert np.all(ws == 0) and np.array_equal(we, np.arange(1, T + 1))
    rng = np.random.default_rng(3)
    for ratio in (1, 2, 3, 4, 7):
        lens = rng.integers(0, 40, size=6)
        lens[2] = 4 * ratio  # one segment with a length that is a multiple of the ratio
        wl = W.make_thd("bf16", lens, ratio, H=1, D=2, seed=1)
        cq, ck = wl.thd["cu_q"], wl.thd["cu_k"]
        ws, we = orc.windows_thd(cq, ck, ratio, wl.S_q, wl.S_k)
        for sgi in range(len(lens)):
            a, b = cq[sgi], cq[sgi + 1]
            if a == b:
                continue
            s_, e_ = ws[a:b], we[a:b]
            assert np.all(s_ == ck[sgi]) and np.all(e_ <= ck[sgi + 1]) and np.all(e_ >= s_)
            d = np.diff(e_)
            assert np.all((d == 0) | (d == 1))
            if (b - a) % ratio == 0:
                assert e_[-1] == ck[sgi + 1]
            counts = np.bincount(e_ - s_)
            for v in range(1, len(counts) - 1):
                assert counts[v] == ratio, (ratio, sgi, v, counts)


def pin_windows_thd_isolation(orc):
    """Scores of a packed workload equal, row by row, those of each segment scored alone
    against its own keys with the same windows shifted to the segment: no row sees
    another segment's keys."""
    wl = W.make_thd("mxfp8", (5, 0, 9, 6), 2, seed=12, out_dtype="f32")
    ref, _ = orc.logits(wl)
    ws, we = orc.windows(wl)
    cq, ck = wl.thd["cu_q"], wl.thd["cu_k"]
    for sgi in range(4):
        a, b, ka, kb = cq[sgi], cq[sgi + 1], ck[sgi], ck[sgi + 1]
        if a == b or ka == kb:
            continue
        one = wl.replace(S_q=int(b - a), S_k=int(kb - ka), q=wl.q[:, a:b], q_scale=wl.q_scale[:, a:b],
                         w=wl.w[:, a:b], k=wl.k[:, ka:kb], k_scale=wl.k_scale[:, ka:kb], thd=None,
                         starts=(ws[:, a:b] - ka).astype(np.int32), ends=(we[:, a:b] - ka).astype(np.int32))
        r1, _ = orc.logits(one)
        seg = ref[a:b]
        assert np.array_equal(seg[:, ka:kb], r1)
        outside = np.concatenate([seg[:, :ka], seg[:, kb:]], axis=1)
        assert np.all(np.isneginf(outside))


def pin_paged_identity(orc):
    """Pages laid out in order (request b owns pages b*max_pages..) with every context full:
    the gathered K is the cache read straight through, and the scores equal those of the
    dense workload with causal offset 0 (row i sees [0, S_k - S_q + i + 1))."""
    for fmt in W.FORMATS:
        B, n, ps, S_k = 3, 4, 16, 80
        wl = W.make_paged(fmt, B, n, [S_k] * B, ps, extra_pages=0, seed=5)
        mp = wl.paged["block_table"].shape[1]
        wl.paged["block_table"] = np.arange(B * mp, dtype=np.int32).reshape(B, mp)
        k, ks = orc.gather_paged(wl)
        assert np.array_equal(k.reshape(-1), wl.paged["k_cache"].reshape(-1))
        dense = wl.replace(paged=None, k=k, k_scale=ks, offsets=np.zeros(B, np.int32))
        a, _ = full(orc, wl)
        b, _ = full(orc, dense)
        assert np.array_equal(a, b)


def pin_paged_relabel_and_unused(orc):
    """Renumbering the physical pages (block table relabelled to match) changes nothing,
    and neither do cache rows no request can see (unused pages, rows past a context)."""
    wl = W.make_paged("mxfp8", 3, 2, [37, 0, 64], 16, S_k=64, extra_pages=4, seed=6)
    base, _ = full(orc, wl)
    pg = wl.paged
    k, ks = orc.gather_paged(wl)  # the gather itself never reads past a context: zeros there
    for b, n in enumerate(pg["ctx"]):
        assert np.all(k[b, n:] == 0) and np.all(ks[b, n:] == 0)
    n_pages = pg["k_cache"].shape[0]
    relabel = np.random.default_rng(1).permutation(n_pages)
    inv = np.argsort(relabel)
    moved = dict(pg, k_cache=pg["k_cache"][inv], k_scale_cache=pg["k_scale_cache"][inv],
                 block_table=relabel[pg["block_table"]].astype(np.int32))
    a, _ = full(orc, wl.replace(paged=moved))
    assert np.array_equal(a, base)
    noisy = dict(pg, k_cache=pg["k_cache"].copy(), k_scale_cache=pg["k_scale_cache"].copy())
    used = set()
    for b in range(3):
        for j in range(int(pg["ctx"][b])):
            used.add((int(pg["block_table"][b, j // 16]), j % 16))
    for page in range(n_pages):
        for r in range(16):
            if (page, r) not in used:
                noisy["k_cache"][page, r] ^= 0x11
                noisy["k_scale_cache"][page, r] ^= 0x01010101
    a, _ = full(orc, wl.replace(paged=noisy))
    assert np.array_equal(a, base)


def pin_paged_windows(orc):
    """Context windows: the newest S_q tokens of a request with ctx keys see
    [0, ctx - S_q + i + 1); ctx past S_k is clamped; a context shorter than S_q leaves the
    first rows empty; they equal the causal offsets ctx - S_k of the dense path."""
    wl = W.make_paged("bf16", 4, 3, [50, 80, 2, 0], 8, S_k=50, H=1, D=2)
    ws, we = orc.windows(wl)
    assert np.all(ws == 0)
    assert we.tolist() == [[48, 49, 50], [48, 49, 50], [0, 1, 2], [0, 0, 0]]
    dense = W.make_random("bf16", 4, 3, 50, H=1, D=2, offsets=[0, 0, 2 - 50, 0 - 50])
    assert np.array_equal(orc.windows(dense)[1], we)


def pin_empty_and_batch(orc):
    """Empty windows are all -inf; each batch's slice equals a B=1 run on that batch alone."""
    for fmt in W.FORMATS:
        wl = W.make_random(fmt, 3, 20, 29, seed=41, windows="irregular")
        ref, _ = full(orc, wl)
        ws, we = orc.windows(wl)
        empty = we <= ws
        assert np.any(empty)
        assert np.all(np.isneginf(ref[empty]))
        for b in range(3):
            sl = lambda a: None if a is None else a[b:b + 1]
            one = wl.replace(B=1, q=sl(wl.q), q_scale=sl(wl.q_scale), k=sl(wl.k), k_scale=sl(wl.k_scale),
                             w=sl(wl.w), starts=sl(wl.starts), ends=sl(wl.ends))
            r1, _ = full(orc, one)
            assert np.array_equal(r1[0], ref[b]), (fmt, b)


def pin_permutation_and_wtype(orc):
    """Permuting K rows permutes output columns (full windows); fp32 W holding bf16 values == bf16 W."""
    for fmt in W.FORMATS:
        wl = W.make_random(fmt, 1, 3, 24, seed=51, offsets=[1000], w_dtype="bf16")
        base, _ = full(orc, wl)
        perm = np.random.default_rng(3).permutation(24)
        kp = wl.k[:, perm]
        ksp = None if wl.k_scale is None else wl.k_scale[:, perm]
        rp, _ = full(orc, wl.replace(k=kp, k_scale=ksp))
        assert np.array_equal(rp, base[:, :, perm]), fmt
        wf = t_bf16(wl.w).astype(np.float32)
        rf, _ = full(orc, wl.replace(w=wf, w_dtype="f32"))
        assert np.array_equal(rf, base), fmt


def pin_bound_dominates(orc):
    """|score| <= bound (Cauchy-Schwarz on every head's dot)."""
    for fmt in W.FORMATS:
        wl = W.make_random(fmt, 2, 5, 31, seed=61, sm_scale=1.3, windows="irregular")
        ref, bound = full(orc, wl)
        fin = ~np.isneginf(ref)
        assert np.all(np.abs(ref[fin]) <= bound[fin] * (1 + 1e-12))




# --------------------------------------------------------------------------
# top-k selection
# --------------------------------------------------------------------------

def _f32(s: str) -> np.float32:
    return np.float32(float(s))


def pin_topk_golden(orc):
    """The hand-worked selections of tests/golden/topk_cases.json (ties, signed zeros,
    NaN, -inf, short and empty windows)."""
    with open(os.path.join(GOLDEN, "topk_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        v = np.array([[_f32(x) for x in c["row"]]], np.float32)
        idx, val = orc.topk(v, [c["start"]], [c["end"]], c["k"])
        assert idx[0].tolist() == c["idx"], c["what"]
        want = np.array([_f32(x) for x in c["val"]], np.float32)
        # compare bit patterns (NaN and -0 included)
        assert np.array_equal(val[0].view(np.uint32), want.view(np.uint32)) or (
            np.array_equal(np.isnan(val[0]), np.isnan(want))
            and np.array_equal(val[0][~np.isnan(want)].view(np.uint32), want[~np.isnan(want)].view(np.uint32))), \
            c["what"]


def pin_topk_matches_stable_argsort(orc):
    """Without NaN the ranking is numpy's stable descending argsort of the window (a
    library routine): scores drawn from a handful of values (many ties, both zeros) and
    from a continuum, windows of every kind, k below, at and above the window size."""
    rng = np.random.default_rng(5)
    S_k = 300
    pool = np.array([-2.5, -1.0, -0.0, 0.0, 0.5, 3.0, -np.inf], np.float32)
    for trial in range(40):
        n_rows = 7
        if trial % 2:
            v = pool[rng.integers(0, pool.size, size=(n_rows, S_k))]
        else:
            v = rng.standard_normal((n_rows, S_k)).astype(np.float32)
        s = rng.integers(0, S_k, size=n_rows)
        e = np.minimum(S_k, s + rng.integers(0, S_k, size=n_rows))
        s[0], e[0] = 0, S_k
        k = int(rng.choice([1, 5, 64, 200, 400]))
        idx, val = orc.topk(v, s.astype(np.int32), e.astype(np.int32), k)
        for r in range(n_rows):
            order = np.argsort(-v[r, s[r]:e[r]], kind="stable")[:k] + s[r]
            m = order.size
            assert idx[r, :m].tolist() == order.tolist()
            assert np.all(idx[r, m:] == -1) and np.all(np.isneginf(val[r, m:]))
            assert np.array_equal(val[r, :m].view(np.uint32), v[r, order].view(np.uint32))


def pin_topk_selection_property(orc):
    """With NaN present: the selection holds min(k, n) distinct window columns, every
    selected score ranks at or above every unselected one (a number above NaN), an equal
    unselected score only ever sits at a larger column than every equal selected one, and
    the listed scores are those of the listed columns."""
    rng = np.random.default_rng(6)
    S_k = 120
    for _ in range(30):
        v = rng.integers(-3, 4, size=(5, S_k)).astype(np.float32)
        v[rng.random(v.shape) < 0.1] = np.nan
        s = rng.integers(0, 40, size=5).astype(np.int32)
        e = (s + rng.integers(0, 80, size=5)).astype(np.int32)
        k = int(rng.integers(1, 60))
        idx, val = orc.topk(v, s, e, k)
        for r in range(5):
            n = int(e[r] - s[r])
            sel = [j for j in idx[r].tolist() if j >= 0]
            assert len(sel) == min(k, n) and len(set(sel)) == len(sel)
            assert all(s[r] <= j < e[r] for j in sel)
            rest = [j for j in range(s[r], e[r]) if j not in set(sel)]
            for j in sel:
                for u in rest:
                    a, b = v[r, j], v[r, u]
                    if np.isnan(a):
                        assert np.isnan(b) and j < u
                    elif not np.isnan(b):
                        assert a > b or (a == b and j < u)
            got = val[r, :len(sel)]
            want = v[r, sel]
            assert np.array_equal(np.isnan(got), np.isnan(want))
            assert np.array_equal(got[~np.isnan(want)], want[~np.isnan(want)])


def pin_topk_by_column(orc):
    """Listing by column keeps the selection and orders it by ascending column: it is
    numpy's sort of the rank-order list (NaN-free ties and signed zeros included), and
    the padding stays at the end."""
    rng = np.random.default_rng(8)
    pool = np.array([-1.0, -0.0, 0.0, 2.0, 5.0], np.float32)
    v = pool[rng.integers(0, pool.size, size=(6, 90))]
    s = np.array([0, 3, 10, 50, 89, 40], np.int32)
    e = np.array([90, 60, 11, 50, 90, 70], np.int32)
    for k in (1, 4, 30, 95):
        ri, rv = orc.topk(v, s, e, k)
        ci, cv = orc.topk(v, s, e, k, by_column=True)
        for r in range(6):
            m = int(np.sum(ri[r] >= 0))
            order = np.argsort(ri[r, :m], kind="stable")
            assert ci[r, :m].tolist() == ri[r, :m][order].tolist()
            assert np.array_equal(cv[r, :m].view(np.uint32), rv[r, :m][order].view(np.uint32))
            assert np.all(ci[r, m:] == -1) and np.all(np.isneginf(cv[r, m:]))
            assert m == min(k, max(int(e[r] - s[r]), 0))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
