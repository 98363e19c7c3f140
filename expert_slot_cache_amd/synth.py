"""Seeded synthetic inputs shared by the library's tests, its benchmark and the oracle.

This module holds no arithmetic of the expert cache or of the MoE layer: it only
draws random numbers and packs them into the byte formats the library accepts.
Everything it returns is plain numpy, so both sides of a parity check read the
same arrays.

What it draws:

* routing traces ``ids[step, layer, token, k]`` (int32): a Zipf popularity over
  the experts (rank r has weight r**-s), mapped to expert ids by a seeded
  per-layer permutation, K distinct ids per token drawn without replacement by
  Gumbel-top-k (the draw order is the k order), optional repetition of the
  previous step's whole id row, optional reshuffling of the permutation;
* top-k gate weights ``w[step, token, k]`` (float32): a uniform point of the
  K-simplex per token (exponential draws divided by their sum), i.e. the
  renormalised top-k weights a router hands to the expert layer;
* activations N(0, 1) and expert weights N(0, 0.02), fp32 or bf16 (round to
  nearest even from fp32), or INT4-g128 with bf16 scales.

Expert byte format (the layout the library's ``load_expert`` accepts; every
region starts on a 256-byte boundary, regions in this order):

* ``f32``:  w13 [2I, H] fp32 row-major, then w2 [H, I] fp32 row-major;
* ``bf16``: the same two matrices as bf16;
* ``int4``: w13 codes [2I, H/8] uint32, w2 codes [H, I/8] uint32, then
  s13 [2I, H/128] bf16 and s2 [H, I/128] bf16.  Element j of a row sits in
  bits 4*(j % 8) of word j // 8, and decodes as (q - 8) * s[row, j // 128].
  Rows [0, I) of w13 are the gate projection, rows [I, 2I) the up projection.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

ALIGN = 256


# --------------------------------------------------------------------------
# Workloads: the shapes and routing statistics of the pages' experiments.
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    experts: int
    top_k: int
    hidden: int
    inter: int
    slots: int
    tokens: int
    steps: int
    wtype: str          # "f32" | "bf16" | "int4"
    atype: str          # "f32" | "bf16"
    zipf_s: float
    repeat_p: float     # chance that a step repeats the previous step's id rows
    reshuffle: int      # popularity permutation redrawn every this many steps (0 = never)
    seed: int

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # One fp32 MoE layer, 8 experts, top-2, 4 slots, 256 batch-1 decode steps.
    "tiny_f32_e8": Workload("tiny_f32_e8", 1, 8, 2, 64, 32, 4, 1, 256, "f32", "f32",
                            1.2, 0.8, 0, 20261202 + 1),
    # OLMoE-1B-7B shapes: 16 layers x 64 experts, top-8, bf16, 16 slots per layer.
    "olmoe_bf16_e64": Workload("olmoe_bf16_e64", 16, 64, 8, 2048, 1024, 16, 1, 512, "bf16",
                               "bf16", 1.0, 0.9, 0, 20261202 + 2),
    # 48 layers x 512 experts, top-10, INT4-g128 weights with bf16 scales.
    # s = 1.6 puts ~0.29 % of selections on the least used 10 % of experts.
    "fanout_int4_e512": Workload("fanout_int4_e512", 48, 512, 10, 2560, 640, 32, 1, 512,
                                 "int4", "bf16", 1.6, 0.0, 0, 20261202 + 3),
    # Prefill ubatches on the OLMoE shapes (512 tokens; 2048 is the other size).
    "prefill_bf16_e64": Workload("prefill_bf16_e64", 16, 64, 8, 2048, 1024, 16, 512, 4,
                                 "bf16", "bf16", 1.0, 0.0, 0, 20261202 + 4),
    # Batched decode, 64 sequences, 128 experts, top-8, drift every 256 steps.
    "batched_bf16_e128": Workload("batched_bf16_e128", 24, 128, 8, 4096, 1536, 32, 64, 1024,
                                  "bf16", "bf16", 1.0, 0.0, 256, 20261202 + 5),
}


def streams(wl: Workload):
    """Four independent generators: trace, weights, activations, gate weights."""
    ss = np.random.SeedSequence(wl.seed).spawn(4)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss]


# --------------------------------------------------------------------------
# Byte layout of one expert.
# --------------------------------------------------------------------------
def _up(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


def expert_regions(wtype: str, hidden: int, inter: int) -> dict:
    """Offsets and sizes (bytes) of each region of one expert, and the total."""
    H, I = hidden, inter
    if wtype == "f32":
        sizes = [("w13", 2 * I * H * 4), ("w2", H * I * 4)]
    elif wtype == "bf16":
        sizes = [("w13", 2 * I * H * 2), ("w2", H * I * 2)]
    elif wtype == "int4":
        if H % 128 or I % 128:
            raise ValueError("int4 needs hidden and inter divisible by 128")
        sizes = [("w13", 2 * I * H // 2), ("w2", H * I // 2),
                 ("s13", 2 * I * (H // 128) * 2), ("s2", H * (I // 128) * 2)]
    else:
        raise ValueError(wtype)
    out, off = {}, 0
    for name, n in sizes:
        out[name] = (off, n)
        off = _up(off + n)
    out["total"] = off
    return out


def expert_bytes(wtype: str, hidden: int, inter: int) -> int:
    return expert_regions(wtype, hidden, inter)["total"]


# --------------------------------------------------------------------------
# Number formats (packing only).
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = (rounded >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_NORMAL_TABLE = None


def _normal_table() -> np.ndarray:
    """65536 equal-probability quantiles of N(0, 1), as float32."""
    global _NORMAL_TABLE
    if _NORMAL_TABLE is None:
        from scipy.special import ndtri
        p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        _NORMAL_TABLE = ndtri(p).astype(np.float32)
    return _NORMAL_TABLE


def normal_bf16_bits(rng: np.random.Generator, n: int, std: float) -> np.ndarray:
    """n draws of N(0, std) as bf16 bits, by inverse-CDF lookup of uniform 16-bit draws.

    Used for the large stores, where a Ziggurat draw per weight would take minutes.
    The quantile grid (2**-16 in probability) is finer than bf16's own grid."""
    table = f32_to_bf16_bits(_normal_table() * np.float32(std))
    idx = np.frombuffer(rng.bytes(2 * n), dtype=np.uint16)
    return table[idx]


def quantize_int4_g128(w: np.ndarray):
    """Symmetric INT4 with one bf16 scale per 128 consecutive inputs of a row.

    s = bf16(max|w| / 7) over the group; q = clamp(rne(w / s) + 8, 0, 15).
    Returns (codes uint32 [rows, in/8], scales bf16 bits [rows, in/128])."""
    rows, cols = w.shape
    g = w.reshape(rows, cols // 128, 128).astype(np.float32)
    amax = np.abs(g).max(axis=2)
    s_bits = f32_to_bf16_bits(amax / np.float32(7.0))
    s = bf16_bits_to_f32(s_bits)
    s_safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint(g / s_safe[:, :, None]) + 8
    q = np.clip(q, 0, 15).astype(np.uint32).reshape(rows, cols // 8, 8)
    shifts = (np.arange(8, dtype=np.uint32) * 4)[None, None, :]
    codes = np.bitwise_or.reduce(q << shifts, axis=2).astype(np.uint32)
    return codes, s_bits


def _int4_nibble_table() -> np.ndarray:
    """256-entry map from a uniform byte to a code 0..15 whose distribution is that
    of quantize_int4_g128 applied to groups of 128 normal draws (Monte Carlo, fixed
    seed; resolution 1/256 in probability)."""
    rng = np.random.Generator(np.random.PCG64(7))
    g = rng.standard_normal((4096, 128)).astype(np.float32)
    codes, _ = quantize_int4_g128(g)
    q = ((codes[:, :, None] >> (np.arange(8, dtype=np.uint32) * 4)) & 15).ravel()
    pmf = np.bincount(q, minlength=16).astype(np.float64)
    cdf = np.cumsum(pmf) / pmf.sum()
    u = (np.arange(256) + 0.5) / 256.0
    return np.searchsorted(cdf, u).clip(0, 15).astype(np.uint8)


_BYTE_TABLES = None


def random_int4_codes(rng: np.random.Generator, n_words: int) -> np.ndarray:
    """n_words uint32 words of 8 codes each, distributed like quantised normal weights
    (each byte holds two codes, each drawn from 8 uniform bits)."""
    global _BYTE_TABLES
    if _BYTE_TABLES is None:
        nib = _int4_nibble_table()
        _BYTE_TABLES = (nib, (nib << 4).astype(np.uint8))
    lo, hi = _BYTE_TABLES
    u = np.frombuffer(rng.bytes(8 * n_words), dtype=np.uint8)
    b = lo[u[0::2]] | hi[u[1::2]]
    return b.view(np.uint32)


# --------------------------------------------------------------------------
# Experts.
# --------------------------------------------------------------------------
def pack_expert(wtype: str, hidden: int, inter: int, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """Pack fp32 matrices w13 [2I, H] and w2 [H, I] into one expert's bytes."""
    reg = expert_regions(wtype, hidden, inter)
    buf = np.zeros(reg["total"], dtype=np.uint8)

    def put(name, arr):
        off, n = reg[name]
        b = np.ascontiguousarray(arr).view(np.uint8).ravel()
        assert b.size == n, (name, b.size, n)
        buf[off:off + n] = b

    if wtype == "f32":
        put("w13", w13.astype(np.float32))
        put("w2", w2.astype(np.float32))
    elif wtype == "bf16":
        put("w13", f32_to_bf16_bits(w13))
        put("w2", f32_to_bf16_bits(w2))
    else:
        c13, s13 = quantize_int4_g128(w13)
        c2, s2 = quantize_int4_g128(w2)
        put("w13", c13)
        put("w2", c2)
        put("s13", s13)
        put("s2", s2)
    return buf


def draw_expert(rng: np.random.Generator, wtype: str, hidden: int, inter: int,
                std: float = 0.02, fast: bool = False) -> np.ndarray:
    """One expert's bytes with N(0, std) weights.

    fast=False draws fp32 normals and packs them (quantising for int4).
    fast=True draws bf16 by quantile lookup and int4 codes from the quantised
    normal code distribution with bf16 scales near max|w|/7 of a 128-group."""
    H, I = hidden, inter
    if not fast or wtype == "f32":
        w13 = (rng.standard_normal((2 * I, H), dtype=np.float32) * np.float32(std))
        w2 = (rng.standard_normal((H, I), dtype=np.float32) * np.float32(std))
        return pack_expert(wtype, H, I, w13, w2)
    reg = expert_regions(wtype, H, I)
    buf = np.zeros(reg["total"], dtype=np.uint8)
    if wtype == "bf16":
        for name in ("w13", "w2"):
            off, n = reg[name]
            buf[off:off + n] = normal_bf16_bits(rng, n // 2, std).view(np.uint8)
        return buf
    for name in ("w13", "w2"):
        off, n = reg[name]
        buf[off:off + n] = random_int4_codes(rng, n // 4).view(np.uint8)
    # the max of |N(0, std)| over 128 draws is ~2.6 std with a small spread
    for name in ("s13", "s2"):
        off, n = reg[name]
        amax = np.float32(std) * (np.float32(2.6) + np.float32(0.25) *
                                  rng.standard_normal(n // 2, dtype=np.float32))
        buf[off:off + n] = f32_to_bf16_bits(np.abs(amax) / np.float32(7.0)).view(np.uint8)
    return buf


class WindowedExperts:
    """Experts for stores too large to draw weight by weight (tens of GiB): every
    region of expert (layer, e) is a window, at a seeded random offset, into one
    seeded buffer of that region's format (N(0, std) fp32/bf16, quantised-normal
    INT4 codes, bf16 scales near max|w|/7).  Each expert's bytes differ; the value
    distribution is the same as draw_expert(fast=True)."""

    def __init__(self, wl: Workload, base_mib: int = 96, std: float = 0.02):
        rng = streams(wl)[1]
        self.wl = wl
        self.reg = expert_regions(wl.wtype, wl.hidden, wl.inter)
        nbytes = base_mib << 20
        names = ["w13", "w2"] + (["s13", "s2"] if wl.wtype == "int4" else [])
        self.base = {}
        if wl.wtype == "f32":
            b = (rng.standard_normal(nbytes // 4, dtype=np.float32) * np.float32(std))
            self.base["w"] = b.view(np.uint8)
        elif wl.wtype == "bf16":
            self.base["w"] = normal_bf16_bits(rng, nbytes // 2, std).view(np.uint8)
        else:
            self.base["w"] = random_int4_codes(rng, nbytes // 4).view(np.uint8)
            n_s = max(1 << 20, (self.reg["s13"][1] + self.reg["s2"][1]) * 4)
            amax = np.float32(std) * (np.float32(2.6) + np.float32(0.25) *
                                      rng.standard_normal(n_s // 2, dtype=np.float32))
            self.base["s"] = f32_to_bf16_bits(np.abs(amax) / np.float32(7.0)).view(np.uint8)
        self.offsets = {}
        for name in names:
            src = self.base["s" if name.startswith("s") else "w"]
            n = self.reg[name][1]
            span = (src.size - n) // 16
            if span <= 0:
                raise ValueError("base buffer too small")
            self.offsets[name] = rng.integers(0, span, size=(wl.layers, wl.experts)) * 16
        self.names = names

    def expert(self, layer: int, e: int, out: np.ndarray | None = None) -> np.ndarray:
        buf = np.zeros(self.reg["total"], np.uint8) if out is None else out
        for name in self.names:
            src = self.base["s" if name.startswith("s") else "w"]
            off, n = self.reg[name]
            o = int(self.offsets[name][layer, e])
            buf[off:off + n] = src[o:o + n]
        return buf


# --------------------------------------------------------------------------
# Activations and gate weights.
# --------------------------------------------------------------------------
def draw_activations(rng: np.random.Generator, shape, atype: str) -> np.ndarray:
    """N(0, 1) activations: float32, or bf16 bits (uint16) for atype == 'bf16'."""
    x = rng.standard_normal(shape, dtype=np.float32)
    return x if atype == "f32" else f32_to_bf16_bits(x)


def draw_gate_weights(rng: np.random.Generator, shape) -> np.ndarray:
    """A uniform point of the K-simplex per row (last axis = k), float32."""
    g = rng.exponential(1.0, size=shape)
    return (g / g.sum(axis=-1, keepdims=True)).astype(np.float32)


# --------------------------------------------------------------------------
# Routing traces.
# --------------------------------------------------------------------------
def zipf_logp(n: int, s: float) -> np.ndarray:
    r = np.arange(1, n + 1, dtype=np.float64)
    lp = -s * np.log(r)
    return lp - np.log(np.exp(lp).sum())


def gumbel_topk(rng: np.random.Generator, logp_by_expert: np.ndarray, n_rows: int, k: int) -> np.ndarray:
    """n_rows draws of k distinct experts without replacement, P(e) ~ exp(logp[e]);
    each row lists the experts in draw order."""
    E = logp_by_expert.shape[0]
    keys = logp_by_expert[None, :] + rng.gumbel(size=(n_rows, E))
    part = np.argpartition(-keys, k - 1, axis=1)[:, :k]
    kv = np.take_along_axis(keys, part, axis=1)
    order = np.argsort(-kv, axis=1, kind="stable")
    return np.take_along_axis(part, order, axis=1).astype(np.int32)


def make_trace(wl: Workload, steps: int | None = None, tokens: int | None = None,
               rng: np.random.Generator | None = None) -> np.ndarray:
    """ids[step, layer, token, k] int32 for the workload's routing statistics."""
    S = wl.steps if steps is None else steps
    T = wl.tokens if tokens is None else tokens
    L, E, K = wl.layers, wl.experts, wl.top_k
    rng = streams(wl)[0] if rng is None else rng
    base = zipf_logp(E, wl.zipf_s)
    ids = np.empty((S, L, T, K), dtype=np.int32)
    perms = np.stack([rng.permutation(E) for _ in range(L)])
    for s in range(S):
        if wl.reshuffle and s > 0 and s % wl.reshuffle == 0:
            perms = np.stack([rng.permutation(E) for _ in range(L)])
        for l in range(L):
            logp = np.empty(E)
            logp[perms[l]] = base          # expert perms[l][r] has popularity rank r
            ids[s, l] = gumbel_topk(rng, logp, T, K)
        if wl.repeat_p > 0 and s > 0:
            rep = rng.random(L) < wl.repeat_p
            ids[s, rep] = ids[s - 1, rep]
    return ids


def predictions(wl: Workload, trace: np.ndarray, accuracy: float, seed: int = 0) -> np.ndarray:
    """Stand-in for a cross-layer router prediction: for each (step, layer) the trace's
    own ids with probability `accuracy`, else the ids of an independent trace with the
    same statistics (same shape; seeded)."""
    rng = np.random.Generator(np.random.PCG64(wl.seed * 7919 + 17 + seed))
    other = make_trace(wl, steps=trace.shape[0], tokens=trace.shape[2], rng=rng)
    keep = rng.random(trace.shape[:2]) < accuracy
    return np.where(keep[:, :, None, None], trace, other).astype(np.int32)


def bottom_decile_share(ids_layer: np.ndarray, n_experts: int) -> float:
    """Share of selections that fall on the least selected 10 % of experts."""
    c = np.sort(np.bincount(ids_layer.ravel(), minlength=n_experts))
    m = max(1, n_experts // 10)
    return float(c[:m].sum() / max(1, c.sum()))
