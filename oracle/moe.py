"""Slot-indexed MoE layer in float64 -- the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What one layer computes, per token t with routed experts e_k and gate weights
w_k (k = 0..K-1), following the fused MoE the cached weights feed (vLLM PR
"Run MoE models exceeding VRAM via expert CPU offloading with GPU cache",
section "How it works": fused_experts over the slot buffers w13 / w2 with the
remapped ids; expert shapes w13 [2I, H] and w2 [H, I] as listed for the INT4
g128 experts in "Running 125B MoE on Two 32 GB Cards", section 1):

    h   = W13[e_k] @ x[t]                 (2I values)
    a   = silu(h[:I]) * h[I:]             silu(z) = z / (1 + exp(-z))
    y_k = W2[e_k] @ a                     (H values)
    out[t] = resid[t] + sum_k w_k * y_k   (resid = 0 when absent)

Readings: rows [0, I) of w13 are the gate, rows [I, 2I) the up projection; no
bias (the vLLM PR's cache is off for MoE layers with bias, Limitations (PR 1)); INT4-g128 weights
decode as (q - 8) * s with one bf16 scale per 128 inputs of a row and no zero
point (the 2.417 MiB per expert of the 125B-MoE post fixes the byte count at
codes plus bf16 scales only).

Every weight is widened exactly to float64 from the bytes the library is given;
all arithmetic is float64.  The float64 result is what the HIP path is compared
against (rounded to fp32 for the comparison).
"""
from __future__ import annotations

import math

import numpy as np

_ALIGN = 256


def _round_up(n: int) -> int:
    return -(-n // _ALIGN) * _ALIGN


def layout(wtype: str, H: int, I: int) -> dict:
    """Byte offset and length of each region of one expert (regions 256-B aligned,
    in the order w13, w2[, s13, s2])."""
    if wtype == "f32":
        parts = [("w13", 2 * I * H * 4), ("w2", H * I * 4)]
    elif wtype == "bf16":
        parts = [("w13", 2 * I * H * 2), ("w2", H * I * 2)]
    elif wtype == "int4":
        parts = [("w13", I * H), ("w2", H * I // 2),
                 ("s13", 2 * I * (H // 128) * 2), ("s2", H * (I // 128) * 2)]
    else:
        raise ValueError(wtype)
    out = {}
    pos = 0
    for name, n in parts:
        out[name] = (pos, n)
        pos = _round_up(pos + n)
    out["total"] = pos
    return out


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening: a bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def int4_g128_to_f64(words: np.ndarray, scale_bits: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Decode codes (uint32 [rows, cols/8], element j at bits 4*(j%8) of word j//8)
    and bf16 scales [rows, cols/128] into (q - 8) * s."""
    w = np.asarray(words, dtype=np.uint32).reshape(rows, cols // 8)
    q = np.empty((rows, cols), dtype=np.int64)
    for j in range(8):
        q[:, j::8] = (w >> np.uint32(4 * j)) & np.uint32(0xF)
    s = bf16_to_f64(np.asarray(scale_bits).reshape(rows, cols // 128))
    return (q - 8).astype(np.float64) * np.repeat(s, 128, axis=1)


def expert_matrices(buf: np.ndarray, wtype: str, H: int, I: int):
    """(W13 [2I, H], W2 [H, I]) in float64 from one expert's bytes."""
    buf = np.asarray(buf, dtype=np.uint8)
    lay = layout(wtype, H, I)

    def region(name, dtype):
        off, n = lay[name]
        return buf[off:off + n].view(dtype)

    if wtype == "f32":
        W13 = region("w13", np.float32).astype(np.float64).reshape(2 * I, H)
        W2 = region("w2", np.float32).astype(np.float64).reshape(H, I)
    elif wtype == "bf16":
        W13 = bf16_to_f64(region("w13", np.uint16)).reshape(2 * I, H)
        W2 = bf16_to_f64(region("w2", np.uint16)).reshape(H, I)
    else:
        W13 = int4_g128_to_f64(region("w13", np.uint32), region("s13", np.uint16), 2 * I, H)
        W2 = int4_g128_to_f64(region("w2", np.uint32), region("s2", np.uint16), H, I)
    return W13, W2


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_mlp(W13: np.ndarray, W2: np.ndarray, x: np.ndarray) -> np.ndarray:
    """One expert on one token: W2 @ (silu(gate) * up)."""
    I = W2.shape[1]
    h = W13 @ x
    a = silu(h[:I]) * h[I:]
    return W2 @ a


def activations_to_f64(x, atype: str) -> np.ndarray:
    if atype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    return bf16_to_f64(x)


def moe_layer(x: np.ndarray, ids: np.ndarray, w: np.ndarray, expert_bytes, wtype: str,
              H: int, I: int, resid: np.ndarray | None = None, atype: str = "f32",
              tokens=None) -> np.ndarray:
    """out[T, H] float64 for activations x[T, H] (fp32 values or bf16 bits),
    expert ids[T, K], gate weights w[T, K] and ``expert_bytes(e)`` giving expert e's
    bytes.  ``tokens`` restricts the computation to a subset of rows (the rows of
    the result for other tokens are left at zero)."""
    xs = activations_to_f64(x, atype)
    T, K = ids.shape
    out = np.zeros((T, H), dtype=np.float64)
    cache = {}
    rows = range(T) if tokens is None else tokens
    for t in rows:
        acc = np.zeros(H, dtype=np.float64)
        for k in range(K):
            e = int(ids[t, k])
            if e not in cache:
                cache[e] = expert_matrices(expert_bytes(e), wtype, H, I)
            W13, W2 = cache[e]
            acc += float(w[t, k]) * expert_mlp(W13, W2, xs[t])
        if resid is not None:
            acc += activations_to_f64(resid[t], atype)
        out[t] = acc
    return out


def tolerance(atype: str, wtype: str) -> float:
    """Relative bound on max|gpu - ref| / max|ref|: 1e-5 for an all-fp32 layer,
    2e-2 when weights or activations are bf16 or INT4."""
    return 1e-5 if (atype == "f32" and wtype == "f32") else 2e-2


def max_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    if scale == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / scale)
