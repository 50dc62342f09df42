"""Seeded synthetic inputs for the lightning-indexer scoring path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only *produces input bytes* (element codes, scale bytes, weights,
window specifications); it contains none of the scoring arithmetic and never
decodes a code back into a number.

Shapes and value distributions follow the workloads the pages describe:

* DeepGEMM pull request 435 ("Improve SM100 MX MQA logits clean-output
  performance"), Performance section and the standalone reproducer: H=64,
  D=128, MXFP8 / MXFP4 Q and K with int32-packed E8M0 scales, FP32 weights,
  per-row windows [0, KV-Q+row), all-zero and random inputs, Q=2048/KV=32768
  and the non-aligned Q=129/KV=4100 case named in its Validation section.
* cudnn-frontend pull request 416 ("DSA indexer forward: add a lean SM100 fast
  path"), What / Support surface sections: BF16 Q/K, BF16 or FP32 W, batched
  uniform-length BSHD, causal windows from q_causal_offsets.

Encodings used for the narrow formats (public OCP 8-bit float and OCP
Microscaling v1.0 definitions, not the pages):

* e4m3fn codes come from torch's float -> float8_e4m3fn cast (round to nearest
  even) after clamping to +-448.
* e2m1 codes are round-to-nearest-even onto {0, .5, 1, 1.5, 2, 3, 4, 6} with
  saturation at 6, sign in bit 3; two codes per byte, the low nibble holding
  the even element.
* E8M0 scale bytes are 127 + U{lo..hi}; four of them are packed little-endian
  into one int32 word per (row, head) for Q and per row for K, byte b scaling
  elements [32b, 32b+32).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

FORMATS = ("bf16", "fp8", "mxfp8", "mxfp4")
FP_TYPES = ("f32", "bf16")


@dataclasses.dataclass
class Workload:
    """One seeded problem instance.  Arrays are host numpy arrays of raw codes.

    q       bf16: uint16 bits [B,S_q,H,D]; fp8/mxfp8: uint8 [B,S_q,H,D];
            mxfp4: uint8 [B,S_q,H,D/2] (low nibble = even element)
    q_scale MX only: uint32 [B,S_q,H]
    k       as q with [B,S_k,D] (mxfp4: [B,S_k,D/2])
    k_scale fp8: float32 [B,S_k]; MX: uint32 [B,S_k]; bf16: None
    w       f32: float32 [B,S_q,H]; bf16: uint16 bits [B,S_q,H]
    offsets int32 [B] or None; starts/ends int32 [B,S_q] or None (explicit
            windows win over offsets when both are given)
    """

    name: str
    B: int
    S_q: int
    S_k: int
    H: int
    D: int
    fmt: str
    w_dtype: str
    out_dtype: str
    sm_scale: float
    clean: bool
    q: np.ndarray
    q_scale: Optional[np.ndarray]
    k: np.ndarray
    k_scale: Optional[np.ndarray]
    w: np.ndarray
    offsets: Optional[np.ndarray]
    starts: Optional[np.ndarray]
    ends: Optional[np.ndarray]
    seed: int = 0
    # packed variable-length rows with ratio-compressed keys (B = 1): dict with
    # int32 arrays cu_q, cu_k (segment boundaries in rows and in keys) and the
    # int ratio; the windows then come from these instead of offsets / starts
    thd: Optional[dict] = None
    # paged keys (decode), k and k_scale then None: dict with k_cache
    # [num_pages, page_size, row], k_scale_cache [num_pages, page_size] or
    # None, block_table int32 [B, max_pages], ctx int32 [B] (keys each request
    # holds) and page_size; S_k is the widest context the output covers
    paged: Optional[dict] = None

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# --------------------------------------------------------------------------
# element encoders (input production only)
# --------------------------------------------------------------------------

def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """float tensor -> bf16 bit patterns (round to nearest even, torch cast)."""
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def e4m3_codes(x: torch.Tensor) -> np.ndarray:
    """float tensor -> e4m3fn byte codes (clamp to +-448, then RNE cast)."""
    return x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


# magnitudes of the eight e2m1 codes 0..7 (OCP MX v1.0 FP4 E2M1)
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


# midpoints between consecutive magnitudes
_E2M1_MID = (_E2M1_MAG[1:] + _E2M1_MAG[:-1]) / 2


def e2m1_codes(x: np.ndarray) -> np.ndarray:
    """float array -> 4-bit e2m1 codes (uint8 0..15), RNE with saturation at 6."""
    x = np.asarray(x)
    mag = np.minimum(np.abs(x), 6.0)
    code = np.searchsorted(_E2M1_MID, mag, side="left")  # number of midpoints strictly below mag
    # a magnitude exactly on a midpoint goes to the even code of the two
    on_mid = (code < 7) & (mag == _E2M1_MID[np.minimum(code, 6)])
    code = np.where(on_mid & (code % 2 == 1), code + 1, code).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 3
    return code | sign


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., D] 4-bit codes -> [..., D/2] bytes, low nibble = even element."""
    assert codes.shape[-1] % 2 == 0
    lo = codes[..., 0::2] & 0xF
    hi = codes[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def pack_e8m0(bytes_: np.ndarray) -> np.ndarray:
    """[..., 4] E8M0 bytes -> [...] uint32 words, byte b in bits 8b..8b+7."""
    assert bytes_.shape[-1] == 4
    b = bytes_.astype(np.uint32)
    return (b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)).astype(np.uint32)


def e8m0_words(rng: np.random.Generator, shape, lo: int = -2, hi: int = 2, nblocks: int = 4) -> np.ndarray:
    """Random E8M0 exponents U{lo..hi} around 1.0, packed into uint32 words."""
    by = (127 + rng.integers(lo, hi + 1, size=tuple(shape) + (nblocks,))).astype(np.uint8)
    if nblocks < 4:
        by = np.concatenate([by, np.full(tuple(shape) + (4 - nblocks,), 127, np.uint8)], axis=-1)
    return pack_e8m0(by)


ONE_SCALE_WORD = 0x7F7F7F7F  # every E8M0 byte = 127, i.e. all scales 1.0


# --------------------------------------------------------------------------
# windows
# --------------------------------------------------------------------------

def irregular_windows(S_q: int, S_k: int, rng: np.random.Generator):
    """Per-row windows for the large irregular MXFP4 workload.

    80 % of rows (rounded) are causal with a nonzero start: end = S_k-S_q+i,
    start = U{1..end-1}; 15 % (rounded) are random sub-windows with length
    L = U{1..S_k} and start = U{0..S_k-L}; the rest are empty rows with
    start = end = U{0..S_k}.  Which row gets which kind is a seeded shuffle.
    """
    n_causal = int(round(0.80 * S_q))
    n_sub = int(round(0.15 * S_q))
    n_empty = S_q - n_causal - n_sub
    perm = rng.permutation(S_q)
    kinds = np.empty(S_q, np.int8)
    kinds[perm[:n_causal]] = 0
    kinds[perm[n_causal:n_causal + n_sub]] = 1
    kinds[perm[n_causal + n_sub:]] = 2
    starts = np.zeros(S_q, np.int64)
    ends = np.zeros(S_q, np.int64)
    for i in range(S_q):
        if kinds[i] == 0:
            e = S_k - S_q + i
            assert e >= 2, "causal rows need end >= 2 for a nonzero start"
            ends[i] = e
            starts[i] = rng.integers(1, e)  # U{1..e-1}
        elif kinds[i] == 1:
            L = int(rng.integers(1, S_k + 1))
            s = int(rng.integers(0, S_k - L + 1))
            starts[i], ends[i] = s, s + L
        else:
            s = int(rng.integers(0, S_k + 1))
            starts[i] = ends[i] = s
    return starts.astype(np.int32), ends.astype(np.int32), kinds


# --------------------------------------------------------------------------
# generic generator
# --------------------------------------------------------------------------

def make_random(fmt: str, B: int, S_q: int, S_k: int, H: int = 64, D: int = 128, *,
                w_dtype: str = "f32", out_dtype: str = "f32", sm_scale: float = 1.0,
                clean: bool = True, seed: int = 0, offsets=None, starts=None, ends=None,
                windows: str = "offsets", value_dist: str = "normal", zero: bool = False,
                scale_lo: int = -2, scale_hi: int = 2, name: str = "custom") -> Workload:
    """Random workload with the pages' value distributions at any size.

    value_dist: "normal" -> N(0,1); "uniform_normal" -> U(-2,2)*N(0,1) (the FP8
    workload).  windows: "offsets" (use `offsets`, default all zero),
    "explicit" (use `starts`/`ends`), "irregular" (the 80/15/5 draw per batch).
    """
    assert fmt in FORMATS and w_dtype in FP_TYPES and out_dtype in FP_TYPES
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)

    def values(shape):
        if value_dist == "normal":
            return torch.randn(shape, generator=g, dtype=torch.float32)
        if value_dist == "uniform_normal":
            u = torch.rand(shape, generator=g, dtype=torch.float32) * 4.0 - 2.0
            return u * torch.randn(shape, generator=g, dtype=torch.float32)
        raise ValueError(value_dist)

    qshape, kshape = (B, S_q, H, D), (B, S_k, D)
    q_scale = k_scale = None
    if fmt == "bf16":
        q = bf16_bits(values(qshape)) if not zero else np.zeros(qshape, np.uint16)
        k = bf16_bits(values(kshape)) if not zero else np.zeros(kshape, np.uint16)
    elif fmt in ("fp8", "mxfp8"):
        q = e4m3_codes(values(qshape)) if not zero else np.zeros(qshape, np.uint8)
        k = e4m3_codes(values(kshape)) if not zero else np.zeros(kshape, np.uint8)
    else:  # mxfp4
        assert D % 2 == 0
        qc = e2m1_codes(values(qshape).numpy()) if not zero else np.zeros(qshape, np.uint8)
        kc = e2m1_codes(values(kshape).numpy()) if not zero else np.zeros(kshape, np.uint8)
        q, k = pack_nibbles(qc), pack_nibbles(kc)
    if fmt == "fp8":
        k_scale = (torch.rand((B, S_k), generator=g, dtype=torch.float32) * 1.5 + 0.5).numpy()
        if zero:
            k_scale = np.ones((B, S_k), np.float32)
    elif fmt in ("mxfp8", "mxfp4"):
        assert D % 32 == 0 and D <= 128
        nb = D // 32
        if zero:
            q_scale = np.full((B, S_q, H), ONE_SCALE_WORD, np.uint32)
            k_scale = np.full((B, S_k), ONE_SCALE_WORD, np.uint32)
        else:
            q_scale = e8m0_words(rng, (B, S_q, H), scale_lo, scale_hi, nb)
            k_scale = e8m0_words(rng, (B, S_k), scale_lo, scale_hi, nb)
    wf = torch.randn((B, S_q, H), generator=g, dtype=torch.float32) / 8.0
    w = bf16_bits(wf) if w_dtype == "bf16" else wf.numpy().copy()

    if windows == "offsets":
        offs = np.zeros(B, np.int32) if offsets is None else np.asarray(offsets, np.int32).reshape(B)
        wl_off, wl_s, wl_e = offs, None, None
    elif windows == "explicit":
        wl_off = None
        wl_s = np.asarray(starts, np.int32).reshape(B, S_q)
        wl_e = np.asarray(ends, np.int32).reshape(B, S_q)
    elif windows == "irregular":
        ss, ee = [], []
        for _ in range(B):
            s_, e_, _k = irregular_windows(S_q, S_k, rng)
            ss.append(s_)
            ee.append(e_)
        wl_off, wl_s, wl_e = None, np.stack(ss), np.stack(ee)
    else:
        raise ValueError(windows)
    return Workload(name=name, B=B, S_q=S_q, S_k=S_k, H=H, D=D, fmt=fmt, w_dtype=w_dtype,
                    out_dtype=out_dtype, sm_scale=float(sm_scale), clean=clean, q=q, q_scale=q_scale,
                    k=k, k_scale=k_scale, w=w, offsets=wl_off, starts=wl_s, ends=wl_e, seed=seed)


def make_thd(fmt: str, seg_lens, ratio: int, *, w_dtype: str = "f32", out_dtype: str = "f32",
             sm_scale: float = 1.0, clean: bool = True, seed: int = 0, name: str = "thd", **kw) -> Workload:
    """Packed variable-length query segments over ratio-compressed keys, the
    THD layout of cudnn-frontend pull request 416 (THD/varlen commit): the
    segments' query tokens are packed into one row range and their compressed
    keys into one column range; segment s has seg_lens[s] query tokens and
    floor(seg_lens[s] / ratio) compressed keys.  Values as make_random."""
    lens = np.asarray(seg_lens, np.int64)
    klens = lens // int(ratio)
    cu_q = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(klens)]).astype(np.int32)
    T_q, m_total = int(cu_q[-1]), int(cu_k[-1])
    wl = make_random(fmt, 1, T_q, max(m_total, 1), w_dtype=w_dtype, out_dtype=out_dtype, sm_scale=sm_scale,
                     clean=clean, seed=seed, name=name, **kw)
    return wl.replace(offsets=None, starts=None, ends=None,
                      thd={"cu_q": cu_q, "cu_k": cu_k, "ratio": int(ratio)})


def make_paged(fmt: str, B: int, next_n: int, ctx_lens, page_size: int, *, S_k: Optional[int] = None,
               extra_pages: int = 3, w_dtype: str = "f32", out_dtype: str = "f32", sm_scale: float = 1.0,
               clean: bool = True, seed: int = 0, name: str = "paged", **kw) -> Workload:
    """Decode-style workload over a paged K cache: B requests, each scoring its
    next_n newest query tokens against the ctx_lens[b] keys it holds in pages of
    page_size rows.  Every request owns ceil(S_k / page_size) logical pages
    (S_k defaults to the longest context); the physical pages are a seeded
    shuffle of all num_pages = B * max_pages + extra_pages pages, so pages are
    scattered and some are unused.  Values as make_random."""
    ctx = np.asarray(ctx_lens, np.int32).reshape(B)
    if S_k is None:
        S_k = max(int(ctx.max()), 1)
    max_pages = (S_k + page_size - 1) // page_size
    num_pages = B * max_pages + extra_pages
    base = make_random(fmt, 1, B * next_n, num_pages * page_size, w_dtype=w_dtype, out_dtype=out_dtype,
                       sm_scale=sm_scale, clean=clean, seed=seed, name=name, **kw)
    rng = np.random.default_rng(seed + 1000)
    perm = rng.permutation(num_pages).astype(np.int32)
    block_table = perm[: B * max_pages].reshape(B, max_pages)
    q = base.q.reshape((B, next_n) + base.q.shape[2:])
    k_cache = base.k.reshape((num_pages, page_size) + base.k.shape[2:])
    k_scale_cache = None if base.k_scale is None else base.k_scale.reshape(num_pages, page_size)
    return Workload(name=name, B=B, S_q=next_n, S_k=S_k, H=base.H, D=base.D, fmt=fmt, w_dtype=w_dtype,
                    out_dtype=out_dtype, sm_scale=float(sm_scale), clean=clean, q=q,
                    q_scale=None if base.q_scale is None else base.q_scale.reshape(B, next_n, -1), k=None,
                    k_scale=None, w=base.w.reshape(B, next_n, -1), offsets=None, starts=None, ends=None, seed=seed,
                    paged={"k_cache": k_cache, "k_scale_cache": k_scale_cache, "block_table": block_table,
                           "ctx": ctx, "page_size": int(page_size)})


# --------------------------------------------------------------------------
# inputs that maximise the matrix core's own accumulation error
# --------------------------------------------------------------------------

# small magnitudes of the adversarial inputs, per format, for a large
# element of 1.0 (6.0 for e2m1): every e4m3 subnormal m * 2^-9, a few
# normals, and for bf16 powers of two far below one
_ADV_SMALL = {
    "fp8": [m * 2.0 ** -9 for m in range(1, 8)] + [2.0 ** -6 * (1 + m / 8) for m in (0, 2, 4, 7)] + [2.0 ** -5,
                                                                                                  2.0 ** -4],
    "mxfp8": None,  # as fp8
    "bf16": [2.0 ** -e for e in (4, 6, 7, 8, 9, 12, 16, 20)],
    "mxfp4": [0.5, 1.0],
}


def make_adversarial(fmt: str, S_q: int, S_k: int, H: int = 64, D: int = 128, *, w_dtype: str = "f32",
                     out_dtype: str = "f32", seed: int = 0, sm_scale: float = 1.0,
                     name: str = "adversarial") -> Workload:
    """Inputs shaped against the accumulation of a matrix core that sums each
    group of 8 consecutive products of a dot in fixed point aligned to the
    group's largest product: in Q and K alike, element d of every group
    (d % 8 == 0) is large and the seven others are small, so Q and K are
    proportional in magnitude up to the small values (sum |q_d k_d| is then
    within a hair of |q| |k|, the tolerance's basis) and the small products
    fall just below or across the alignment's last kept bit.  Row i's small
    value is the (i mod n)-th of a list, column j's the (j mod n)-th, so
    every pair meets; the same q serves all H heads and the weights share one
    sign, so the per-head errors add.  Every fourth row is negated (its
    scores are then exactly 0 after the ReLU).  Windows: causal, offset 0.
    MX scales are random per block (the groups lie inside the blocks)."""
    assert fmt in FORMATS and D == 128
    small = _ADV_SMALL["fp8" if fmt == "mxfp8" else fmt]
    big = 6.0 if fmt == "mxfp4" else 1.0
    n = len(small)
    rng = np.random.default_rng(seed)
    g = torch.Generator().manual_seed(seed)
    grp = (np.arange(D) % 8) == 0
    qrow = np.where(grp[None, :], big, np.asarray([small[i % n] for i in range(S_q)])[:, None])
    qrow = qrow * np.where(np.arange(S_q) % 4 == 3, -1.0, 1.0)[:, None]
    krow = np.where(grp[None, :], big, np.asarray([small[j % n] for j in range(S_k)])[:, None])
    qv = torch.from_numpy(np.broadcast_to(qrow[:, None, :], (S_q, H, D)).copy()).float().reshape(1, S_q, H, D)
    kv = torch.from_numpy(krow).float().reshape(1, S_k, D)
    q_scale = k_scale = None
    if fmt == "bf16":
        q, k = bf16_bits(qv), bf16_bits(kv)
    elif fmt in ("fp8", "mxfp8"):
        q, k = e4m3_codes(qv), e4m3_codes(kv)
    else:
        q, k = pack_nibbles(e2m1_codes(qv.numpy())), pack_nibbles(e2m1_codes(kv.numpy()))
    if fmt == "fp8":
        k_scale = (torch.rand((1, S_k), generator=g, dtype=torch.float32) * 1.5 + 0.5).numpy()
    elif fmt in ("mxfp8", "mxfp4"):
        q_scale = e8m0_words(rng, (1, S_q, H))
        k_scale = e8m0_words(rng, (1, S_k))
    wf = (torch.rand((1, S_q, H), generator=g, dtype=torch.float32) + 0.5) / 8.0
    w = bf16_bits(wf) if w_dtype == "bf16" else wf.numpy().copy()
    return Workload(name=name, B=1, S_q=S_q, S_k=S_k, H=H, D=D, fmt=fmt, w_dtype=w_dtype, out_dtype=out_dtype,
                    sm_scale=float(sm_scale), clean=True, q=q, q_scale=q_scale, k=k, k_scale=k_scale, w=w,
                    offsets=np.zeros(1, np.int32), starts=None, ends=None, seed=seed)


# --------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------

def _c1(**kw):
    return make_random("bf16", 1, 128, 512, w_dtype="f32", sm_scale=1 / math.sqrt(128), seed=1,
                       offsets=[0], name="c1_tiny_causal_bf16", **kw)


def _c2(**kw):
    return make_random("bf16", 4, 2048, 4096, w_dtype="bf16", sm_scale=1 / math.sqrt(128), seed=2,
                       offsets=[0, 0, 0, 0], name="c2_bf16_batch", **kw)


def _c3(**kw):
    # rows see [0, S_k - S_q + i): q_causal_offset = -1 in end = S_k - S_q + off + i + 1
    return make_random("fp8", 1, 2048, 32768, w_dtype="f32", sm_scale=1.0, seed=3, offsets=[-1],
                       value_dist="uniform_normal", name="c3_fp8", **kw)


def _c4(fmt, zero=False, **kw):
    return make_random(fmt, 1, 2048, 32768, w_dtype="f32", sm_scale=1.0, seed=4, offsets=[-1], zero=zero,
                       name=f"c4_{fmt}{'_zero' if zero else ''}", **kw)


def _c5(S_q=8192, S_k=65536, seed=5, name="c5_mxfp4_irregular", **kw):
    return make_random("mxfp4", 1, S_q, S_k, w_dtype="bf16", out_dtype="bf16", sm_scale=1.0, seed=seed,
                       windows="irregular", name=name, **kw)


def _thd(**kw):
    # the ragged B=3, T_q=8192, ratio-4 shape the cudnn-frontend page times
    # (m_total = 2046): BF16 Q/K, FP32 W and scores; the segment lengths are
    # not printed there, these are one ragged choice with that T_q and m_total
    return make_thd("bf16", (1027, 3003, 4162), 4, w_dtype="f32", sm_scale=1 / math.sqrt(128), seed=7,
                    name="thd_bf16_r4", **kw)


def _paged_decode(**kw):
    # decode over a paged cache: 64 requests scoring their 2 newest tokens
    # against contexts of 1..32768 keys in 64-row pages, MXFP8 at the
    # contiguous MX shape's H, D and widest context; the paged entry writes no
    # -inf outside the windows (clean_logits off).  The pages name the paged
    # path and its sampled test shapes without printing them, so this one
    # plain decode shape stands in.
    ctx = np.random.default_rng(8).integers(1, 32769, size=64)
    return make_paged("mxfp8", 64, 2, ctx, 64, S_k=32768, w_dtype="f32", sm_scale=1.0, clean=False, seed=8,
                      name="paged_mxfp8_decode", **kw)


def _q8k(fmt, zero=False, **kw):
    # the long case of the DeepGEMM pull request 435 page's timing table
    # (Performance section): Q8192 / KV65536, windows [0, KV - Q + row), fp32
    # weights and scores; the page times it on all-zero inputs with scales 1
    return make_random(fmt, 1, 8192, 65536, w_dtype="f32", sm_scale=1.0, seed=11, offsets=[-1], zero=zero,
                       name=f"q8192_kv65536_{fmt}{'_zero' if zero else ''}", **kw)


def _screen(H, **kw):
    # the head-count screen of the DeepGEMM pull request 435 page (H = 8, 32,
    # 64 at Q = KV = 8192, Performance section): MXFP8, causal, fp32 weights
    # and scores; the screen's other settings are not printed
    return make_random("mxfp8", 1, 8192, 8192, H=H, w_dtype="f32", sm_scale=1.0, seed=10 + H, offsets=[0],
                       name=f"screen_h{H}_mxfp8_q8192", **kw)


NAMED = {
    "c1": _c1,
    "c2": _c2,
    "c3": _c3,
    "c3_noclean": lambda **kw: _c3(clean=False, **kw),
    "c4_mxfp8": lambda **kw: _c4("mxfp8", **kw),
    "c4_mxfp4": lambda **kw: _c4("mxfp4", **kw),
    "c4_mxfp8_zero": lambda **kw: _c4("mxfp8", zero=True, **kw),
    "c4_mxfp4_zero": lambda **kw: _c4("mxfp4", zero=True, **kw),
    "c5": _c5,
    "c5_nonaligned": lambda **kw: _c5(S_q=129, S_k=4100, seed=6, name="c5_nonaligned", **kw),
    "thd_bf16_r4": _thd,
    "paged_mxfp8_decode": _paged_decode,
    "q8k_mxfp8": lambda **kw: _q8k("mxfp8", **kw),
    "q8k_mxfp4": lambda **kw: _q8k("mxfp4", **kw),
    "q8k_mxfp8_zero": lambda **kw: _q8k("mxfp8", zero=True, **kw),
    "q8k_mxfp4_zero": lambda **kw: _q8k("mxfp4", zero=True, **kw),
    "screen_h8": lambda **kw: _screen(8, **kw),
    "screen_h32": lambda **kw: _screen(32, **kw),
    "screen_h64": lambda **kw: _screen(64, **kw),
}


def make(name: str, **kw) -> Workload:
    return NAMED[name](**kw)
