"""Pins for the float64 MoE-layer oracle (CPU only).

Each check ties the oracle to something other than its own formula: torch's
library silu / linear on the dense special case, closed-form SwiGLU values that
separate the gate from the up half and the sign of silu, hand-written INT4 words,
the independent quantiser in the input generator, and algebraic properties of
the layer (linearity in the gate weights, permutation of the (id, w) pairs).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from expert_slot_cache_amd import synth
from oracle import moe

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32_expert(W13, W2):
    H = W13.shape[1]
    I = W2.shape[1]
    return synth.pack_expert("f32", H, I, W13.astype(np.float32), W2.astype(np.float32))


def test_layout_agrees_with_generator():
    for wtype, H, I in [("f32", 64, 32), ("bf16", 2048, 1024), ("int4", 2560, 640),
                        ("bf16", 4096, 1536), ("int4", 128, 128)]:
        a = moe.layout(wtype, H, I)
        b = synth.expert_regions(wtype, H, I)
        assert a == b
    # the 125B-MoE post's INT4 g128 expert: 2.417 MiB
    assert moe.layout("int4", 2560, 640)["total"] == 2534400
    assert abs(2534400 / 2**20 - 2.417) < 1e-3
    assert moe.layout("bf16", 2048, 1024)["total"] == 12 * 2**20


def test_dense_special_case_matches_torch_library():
    """E = K = 1 with w = 1 is a dense SwiGLU MLP: torch.nn.functional in float64."""
    rng = np.random.default_rng(0)
    H, I, T = 48, 20, 5
    W13 = rng.standard_normal((2 * I, H)).astype(np.float32) * 0.3
    W2 = rng.standard_normal((H, I)).astype(np.float32) * 0.3
    x = rng.standard_normal((T, H)).astype(np.float32)
    buf = _f32_expert(W13, W2)
    got = moe.moe_layer(x, np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32),
                        lambda e: buf, "f32", H, I)
    tx = torch.from_numpy(x).double()
    g, u = torch.nn.functional.linear(tx, torch.from_numpy(W13).double()).split(I, dim=1)
    ref = torch.nn.functional.linear(torch.nn.functional.silu(g) * u,
                                     torch.from_numpy(W2).double())
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_closed_form_gate_up_and_sign():
    """H = 2, I = 1: gate row picks x0, up row picks x1.  With x = (g, u):
    out = w * W2 * silu(g) * u.  silu(40) = 40 to 1e-15, silu(-40) ~ -1.7e-16,
    silu(0) = 0 and silu(ln 3) = 0.75 ln 3."""
    W13 = np.array([[1.0, 0.0], [0.0, 1.0]])
    W2 = np.array([[2.0], [-1.0]])
    buf = _f32_expert(W13, W2)
    cases = [((40.0, 0.5), 40.0 * 0.5), ((-40.0, 0.5), 0.0), ((0.0, 7.0), 0.0),
             ((math.log(3.0), 4.0), 0.75 * math.log(3.0) * 4.0)]
    for (g, u), a in cases:
        x = np.array([[g, u]], np.float32)
        out = moe.moe_layer(x, np.array([[0]]), np.array([[0.5]], np.float32),
                            lambda e: buf, "f32", 2, 1)
        a32 = float(np.float32(g)) if g else 0.0
        # expected with the fp32-rounded inputs the oracle actually reads
        gg, uu = float(np.float32(g)), float(np.float32(u))
        a_exact = gg / (1 + math.exp(-gg)) * uu
        assert abs(a_exact - a) < 1e-6 * max(1.0, abs(a))
        np.testing.assert_allclose(out[0], [0.5 * 2.0 * a_exact, -0.5 * a_exact],
                                   rtol=1e-14, atol=1e-14)


def test_resid_is_added():
    rng = np.random.default_rng(1)
    H, I = 8, 4
    buf = _f32_expert(rng.standard_normal((2 * I, H)), rng.standard_normal((H, I)))
    x = rng.standard_normal((3, H)).astype(np.float32)
    r = rng.standard_normal((3, H)).astype(np.float32)
    ids = np.zeros((3, 1), np.int32)
    w = np.full((3, 1), 0.25, np.float32)
    a = moe.moe_layer(x, ids, w, lambda e: buf, "f32", H, I)
    b = moe.moe_layer(x, ids, w, lambda e: buf, "f32", H, I, resid=r)
    np.testing.assert_allclose(b - a, r.astype(np.float64), rtol=0, atol=1e-15)


def test_int4_decode_golden_words():
    g = json.load(open(os.path.join(GOLDEN, "int4_words.json")))
    words = np.zeros(32, np.uint32)
    words[:4] = [int(h, 16) for h in g["words_hex_first4"]]
    words[4:16] = 0x88888888
    words[16:32] = 0x00000009
    scales = np.array([int(h, 16) for h in g["scales_bf16_hex"]], np.uint16)
    W = moe.int4_g128_to_f64(words, scales, 1, 256)
    assert W[0, :32].tolist() == g["expect_first32"]
    assert (W[0, 32:128] == 0).all()
    assert W[0, 128:136].tolist() == g["expect_col128_to_135"]


def test_int4_dequant_inverts_generator_quantiser():
    """|(q - 8) s - w| <= s / 2 for the generator's independent quantiser; the group
    maximum is reproduced to within bf16 rounding of s."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((6, 384)) * 0.02).astype(np.float32)
    codes, s_bits = synth.quantize_int4_g128(w)
    deq = moe.int4_g128_to_f64(codes, s_bits, 6, 384)
    s = np.repeat(moe.bf16_to_f64(s_bits), 128, axis=1)
    assert (np.abs(deq - w) <= s / 2 + 1e-12).all()
    # a mis-ordered nibble would move values by multiples of s
    assert np.corrcoef(deq.ravel(), w.ravel())[0, 1] > 0.99


def test_all_codes_eight_give_zero():
    H, I = 256, 128
    lay = moe.layout("int4", H, I)
    buf = np.zeros(lay["total"], np.uint8)
    for name in ("w13", "w2"):
        off, n = lay[name]
        buf[off:off + n] = 0x88
    for name in ("s13", "s2"):
        off, n = lay[name]
        buf[off:off + n].view(np.uint16)[:] = 0x3F80   # 1.0
    x = synth.f32_to_bf16_bits(np.random.default_rng(0).standard_normal((2, H)))
    out = moe.moe_layer(x, np.zeros((2, 1), np.int32), np.ones((2, 1), np.float32),
                        lambda e: buf, "int4", H, I, atype="bf16")
    assert (out == 0).all()


def test_bf16_widening_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # finite values only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(moe.bf16_to_f64(bits), ref)
    # the generator's fp32 -> bf16 rounding agrees with torch's
    v = np.random.default_rng(2).standard_normal(10000).astype(np.float32) * 3
    tb = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(v), tb)


def _rand_layer(rng, E, K, T, H, I, wtype):
    experts = [synth.draw_expert(rng, wtype, H, I, std=0.1) for _ in range(E)]
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = synth.draw_gate_weights(rng, (T, K))
    x = rng.standard_normal((T, H)).astype(np.float32)
    return experts, ids, w, x


@pytest.mark.parametrize("wtype", ["f32", "bf16", "int4"])
def test_linear_in_gate_weights_and_pair_order_free(wtype):
    rng = np.random.default_rng(9)
    H, I = 128, 128
    experts, ids, w, x = _rand_layer(rng, 6, 3, 4, H, I, wtype)
    w = w.astype(np.float64)       # the oracle reads w exactly; keep the sums exact too
    f = lambda ww, ii: moe.moe_layer(x, ii, ww, lambda e: experts[e], wtype, H, I)
    base = f(w, ids)
    np.testing.assert_allclose(f(2.5 * w, ids), 2.5 * base, rtol=1e-12, atol=1e-14)
    w2 = np.roll(w, 1, axis=1)
    np.testing.assert_allclose(f(w + w2, ids), base + f(w2, ids), rtol=1e-12, atol=1e-14)
    perm = np.array([2, 0, 1])
    np.testing.assert_allclose(f(w[:, perm], ids[:, perm]), base, rtol=1e-12, atol=1e-14)


def test_tolerance_metric():
    ref = np.array([1.0, -4.0, 2.0])
    assert moe.max_rel_err(ref + np.array([0, 0.04, 0]), ref) == pytest.approx(0.01)
    assert moe.tolerance("f32", "f32") == 1e-5
    assert moe.tolerance("bf16", "int4") == 2e-2


# ---------------------------------------------------------------------------
# expert_matrices, bf16 and INT4 branches, wired region by region: H != I and
# H != 2I, so a transposed or reshaped W2 and a swapped region cannot pass.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("H,I", [(24, 16), (40, 8), (8, 24)])
def test_bf16_expert_matrices_equal_torch_rounding(H, I):
    """Each matrix equals torch's own bf16 rounding of the fp32 matrix it was
    packed from, element by element (torch's conversion is independent of the
    generator's bit twiddling)."""
    rng = np.random.default_rng(H * 100 + I)
    W13 = rng.standard_normal((2 * I, H)).astype(np.float32)
    W2 = (rng.standard_normal((H, I)) * 7.0).astype(np.float32)   # another scale: a swap shows
    buf = synth.pack_expert("bf16", H, I, W13, W2)
    A13, A2 = moe.expert_matrices(buf, "bf16", H, I)
    r13 = torch.from_numpy(W13).to(torch.bfloat16).double().numpy()
    r2 = torch.from_numpy(W2).to(torch.bfloat16).double().numpy()
    assert A13.shape == (2 * I, H) and A2.shape == (H, I)
    np.testing.assert_array_equal(A13, r13)
    np.testing.assert_array_equal(A2, r2)


@pytest.mark.parametrize("H,I", [(256, 128), (128, 384), (384, 256)])
def test_int4_expert_matrices_within_half_a_step_of_their_own_group(H, I):
    """|W_hat - W| <= s/2 element by element, where s is the scale torch computes
    for that element's own row and 128-group (bf16 of max|w|/7; values chosen
    inside [-7s, 7s] so that no code clips).  W13 and W2 are drawn at scales 1000
    apart, so s13 and s2 differ and a swapped scale region fails."""
    rng = np.random.default_rng(H + 7 * I)
    W13 = rng.standard_normal((2 * I, H)).astype(np.float32)
    W2 = (rng.standard_normal((H, I)) * 1e-3).astype(np.float32)
    buf = synth.pack_expert("int4", H, I, W13, W2)
    A13, A2 = moe.expert_matrices(buf, "int4", H, I)
    assert A13.shape == (2 * I, H) and A2.shape == (H, I)
    for A, W in ((A13, W13), (A2, W2)):
        rows, cols = W.shape
        g = torch.from_numpy(W).reshape(rows, cols // 128, 128).abs().amax(dim=2)
        s = (g / 7.0).to(torch.bfloat16).double().numpy()         # [rows, groups]
        s_el = np.repeat(s, 128, axis=1)
        err = np.abs(A - W.astype(np.float64))
        # exact halves can round either way in the quantiser: allow s/2 plus rounding
        assert (err <= s_el * (0.5 + 1e-6) + 2.0 ** -30).all()
        # and the decoded values sit on the grid (q - 8) * s of their own group
        q = A / s_el
        np.testing.assert_allclose(q, np.rint(q), atol=1e-9)
        assert (np.rint(q) >= -8).all() and (np.rint(q) <= 7).all()


def test_int4_swapped_scale_regions_would_fail():
    """Guard for the test above: decoding with the scale regions exchanged (done
    here by hand on the raw bytes) is far outside the half-step bound."""
    H, I = 256, 128
    rng = np.random.default_rng(5)
    W13 = rng.standard_normal((2 * I, H)).astype(np.float32)
    W2 = (rng.standard_normal((H, I)) * 1e-3).astype(np.float32)
    buf = synth.pack_expert("int4", H, I, W13, W2)
    lay = moe.layout("int4", H, I)
    o13, n13 = lay["s13"]
    o2, n2 = lay["s2"]
    n = min(n13, n2)      # exchange the leading scales of the two regions
    bad = buf.copy()
    bad[o13:o13 + n] = buf[o2:o2 + n]
    bad[o2:o2 + n] = buf[o13:o13 + n]
    B13, _ = moe.expert_matrices(bad, "int4", H, I)
    assert np.abs(B13 - W13).max() > 0.5
