"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: hand-derived fixtures
under tests/golden/, closed forms, brute force over all code levels, invariants, a library
routine (torch's fp32->bf16/fp16 conversion) or an independent bit-level definition.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- 16-bit rounding


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_rne_matches_torch_cpu(dtype):
    """RNE to bf16/fp16 equals torch's CPU conversion, including exact ties, subnormals and NaN."""
    g = np.random.default_rng(7)
    a = np.concatenate(
        [
            g.standard_normal(20000).astype(np.float32) * np.float32(0.02),
            g.standard_normal(2000).astype(np.float32) * np.float32(1e-38),
            # exact bf16 ties: low 16 bits == 0x8000
            (g.integers(0, 2**15, 2000, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32).view(np.float32),
            np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65520.0, 1e-8, -1e-8], dtype=np.float32),
        ]
    )
    a = a[np.isfinite(a) | np.isinf(a)]
    t = torch.from_numpy(a.copy())
    ref = t.to(torch.bfloat16 if dtype == "bf16" else torch.float16).view(torch.int16).numpy().view(np.uint16)
    got = O.to_bits(dtype, a)
    np.testing.assert_array_equal(got, ref)
    nan = O.to_bits(dtype, np.array([np.nan], dtype=np.float32))
    assert np.isnan(O.bits_to_f64(dtype, nan))[0]


# ---------------------------------------------------------------- packing order


def test_pack_low_bits_first_4bit():
    q = np.arange(8)[None, :]
    assert O.pack_codes(q, 4)[0, 0] == 0x76543210
    q = np.arange(16)[None, :]
    np.testing.assert_array_equal(O.pack_codes(q, 4)[0], [0x76543210, 0xFEDCBA98])


def test_pack_low_bits_first_8bit_and_2bit():
    assert O.pack_codes(np.arange(4)[None, :], 8)[0, 0] == 0x03020100
    assert O.pack_codes(np.array([[255, 0, 0, 1]]), 8)[0, 0] == 0x010000FF
    assert O.pack_codes(np.array([[1, 2, 3, 0] * 4]), 2)[0, 0] == int("".join(["00", "11", "10", "01"] * 4), 2)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_unpack_inverts_pack(bits):
    g = np.random.default_rng(bits)
    q = g.integers(0, 1 << bits, size=(5, 128))
    np.testing.assert_array_equal(O.unpack_codes(O.pack_codes(q, bits), bits, 128), q)


def _stream_words_from_digits(codes, bits):
    """The row's bitstream read as one integer is the number whose base-2^bits digits (most
    significant first) are the codes in reverse order; written out as a digit string and parsed
    with Python's int(), then cut into little-endian 32-bit words (no shifts or masks)."""
    digits = "0123456789abcdefghijklmnopqrstuv"
    if bits in (1, 2, 3, 4, 5):
        text, base = "".join(digits[c] for c in reversed(codes)), 1 << bits
    elif bits == 6:  # two octal digits per code
        text, base = "".join(f"{c >> 3}{c & 7}" for c in reversed(codes)), 8
    elif bits == 7:  # seven binary digits per code
        text, base = "".join(f"{c:07b}" for c in reversed(codes)), 2
    else:  # bits == 8: two hex digits per code
        text, base = "".join(f"{c:02x}" for c in reversed(codes)), 16
    raw = int(text, base).to_bytes(len(codes) * bits // 8, "little")
    return np.frombuffer(raw, dtype="<u4")


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_pack_is_one_little_endian_stream_per_row(bits):
    """Every row is one continuous little-endian bitstream (GPTQModel wiki, "Packed layouts and
    exact transcoding"): compared with the digit-string construction on random rows."""
    g = np.random.default_rng(100 + bits)
    q = g.integers(0, 1 << bits, size=(4, 256))
    packed = O.pack_codes(q, bits)
    for r in range(q.shape[0]):
        np.testing.assert_array_equal(packed[r], _stream_words_from_digits([int(c) for c in q[r]], bits))


def test_pack_bitstream_golden_3_5_6bit():
    fx = _golden("affine_bitstream_3_5_6.json")
    for case in fx["cases"]:
        q = np.array([case["codes"]])
        words = np.array([int(w, 16) for w in case["words"]], dtype=np.uint32)
        np.testing.assert_array_equal(O.pack_codes(q, case["bits"])[0], words)
        np.testing.assert_array_equal(O.unpack_codes(words[None, :], case["bits"], q.shape[1]), q)


# ---------------------------------------------------------------- quantizer


@pytest.mark.parametrize("pdt", ["f16", "bf16"])
def test_quantize_golden_exact_group(pdt):
    fx = _golden("affine_g64_exact_group.json")
    w = np.array(fx["w"], dtype=np.float32)[None, :]
    packed, sb, bb = O.affine_quantize(w, 4, 64, pdt)
    np.testing.assert_array_equal(packed[0], np.array(fx["packed"], dtype=np.uint32))
    assert sb[0, 0] == fx["scale_bits"][pdt]
    assert bb[0, 0] == fx["bias_bits"][pdt]
    deq = O.affine_dequant_f32(packed, sb, bb, 4, 64, pdt, 64)
    np.testing.assert_array_equal(deq[0], w[0])


def _brute_codes(w, s, b, bits):
    """Nearest level index by exhaustive search over all 2^bits levels b + c*s in fp64, ties
    to the even index; also returns the distance gap between the two best levels."""
    L = (1 << bits) - 1
    c = np.arange(L + 1, dtype=np.float64)
    lv = b[..., None] + c * s[..., None]
    d = np.abs(w[..., None] - lv)
    best = d.min(axis=-1, keepdims=True)
    tie = np.isclose(d, best, rtol=0, atol=0)
    # among exact ties choose even index
    even_pref = np.where(tie, np.where(c % 2 == 0, 0, 1), 2)
    idx = np.argmin(even_pref * 1e6 + c * 0 + np.where(tie, 0, 1e9), axis=-1)
    ds = np.sort(d, axis=-1)
    gap = ds[..., 1] - ds[..., 0]
    return idx, gap


@pytest.mark.parametrize("bits,g,pdt", [(4, 64, "f16"), (4, 32, "bf16"), (8, 64, "bf16"), (8, 128, "f16"), (4, 128, "bf16"),
                                        (2, 64, "bf16"), (3, 32, "f16"), (5, 128, "bf16"), (6, 64, "f16")])
def test_quantize_codes_equal_brute_force_nearest_level(bits, g, pdt):
    n, k = 6, 256
    w = synth.weights_f32(11 + bits + g, n, k)
    packed, sb, bb = O.affine_quantize(w, bits, g, pdt)
    q = O.unpack_codes(packed, bits, k).reshape(n, k // g, g)
    s = O.bits_to_f64(pdt, sb)[..., None].repeat(g, -1)
    b = O.bits_to_f64(pdt, bb)[..., None].repeat(g, -1)
    wv = w.astype(np.float64).reshape(n, k // g, g)
    idx, gap = _brute_codes(wv, s, b, bits)
    diff = idx != q
    # A mismatch is allowed only where the two nearest levels are within fp32 rounding of a tie.
    assert np.all(gap[diff] <= 4e-7 * np.maximum(1.0, np.abs(wv[diff]) / s[diff]) * s[diff] + 1e-12)
    assert diff.sum() <= 2


@pytest.mark.parametrize("bits,pdt", [(4, "f16"), (4, "bf16"), (8, "bf16"), (8, "f16"), (3, "bf16"), (6, "f16")])
def test_quantize_scale_is_range_over_levels_and_bias_is_min(bits, pdt):
    """scale = RNE((max-min)/(2^bits-1)) and bias = RNE(min), with max/min found by a loop."""
    w = synth.weights_f32(5, 3, 128)
    g = 64
    _, sb, bb = O.affine_quantize(w, bits, g, pdt)
    for r in range(3):
        for j in range(2):
            vals = [float(v) for v in w[r, j * g:(j + 1) * g]]
            lo, hi = vals[0], vals[0]
            for v in vals:
                lo = v if v < lo else lo
                hi = v if v > hi else hi
            s32 = np.float32(np.float32(hi) - np.float32(lo)) / np.float32((1 << bits) - 1)
            want_s = torch.tensor([float(s32)], dtype=torch.float32).to(torch.bfloat16 if pdt == "bf16" else torch.float16)
            want_b = torch.tensor([lo], dtype=torch.float32).to(torch.bfloat16 if pdt == "bf16" else torch.float16)
            assert sb[r, j] == want_s.view(torch.int16).numpy().view(np.uint16)[0]
            assert bb[r, j] == want_b.view(torch.int16).numpy().view(np.uint16)[0]


@pytest.mark.parametrize("bits,g,pdt", [(4, 64, "bf16"), (4, 64, "f16"), (8, 32, "bf16"), (8, 64, "f16"), (2, 32, "bf16"),
                                        (5, 64, "f16"), (6, 128, "bf16")])
def test_quantize_round_trip_bound(bits, g, pdt):
    """|w - dequant| <= s/2 inside [b, b + L*s]; outside, only by the clamp distance, which is
    bounded by the storage rounding of the min and of the scale."""
    n, k = 64, 512
    w = synth.weights_f32(21 + bits, n, k)
    packed, sb, bb = O.affine_quantize(w, bits, g, pdt)
    deq = O.affine_dequant_f32(packed, sb, bb, bits, g, pdt, k).astype(np.float64).reshape(n, k // g, g)
    L = (1 << bits) - 1
    s = O.bits_to_f64(pdt, sb)[..., None]
    b = O.bits_to_f64(pdt, bb)[..., None]
    wv = w.astype(np.float64).reshape(n, k // g, g)
    err = np.abs(wv - deq)
    outside = np.maximum(0.0, np.maximum(b - wv, wv - (b + L * s)))
    assert np.all(err <= s / 2 * (1 + 1e-6) + outside + 1e-12)
    mn = wv.min(-1, keepdims=True)
    mx = wv.max(-1, keepdims=True)
    slack = np.abs(b - mn) + L * np.abs(s - (mx - mn) / L) + 1e-7 * np.abs(mx - mn)
    assert np.all(outside <= slack)


@pytest.mark.parametrize("bits,pdt", [(4, "bf16"), (4, "f16"), (8, "bf16"), (8, "f16")])
def test_quantize_identity_on_exact_grid(bits, pdt):
    """W = q*s + b with dyadic s, b (exact in fp32 and in the param dtype) and both end codes in
    every group requantizes to the same codes, scale and bias, bit for bit."""
    g = np.random.default_rng(3 + bits)
    n, k, gs = 8, 256, 64
    L = (1 << bits) - 1
    q = g.integers(0, L + 1, size=(n, k // gs, gs))
    q[..., 0] = 0
    q[..., 1] = L
    s = np.exp2(g.integers(-10, -4, size=(n, k // gs))).astype(np.float64)
    b = -np.exp2(g.integers(-6, -2, size=(n, k // gs))).astype(np.float64) * g.integers(1, 4, size=(n, k // gs))
    w = (q * s[..., None] + b[..., None]).astype(np.float32).reshape(n, k)
    packed, sb, bb = O.affine_quantize(w, bits, gs, pdt)
    np.testing.assert_array_equal(O.unpack_codes(packed, bits, k), q.reshape(n, k))
    np.testing.assert_array_equal(O.bits_to_f64(pdt, sb), s)
    np.testing.assert_array_equal(O.bits_to_f64(pdt, bb), b)


def test_quantize_constant_group_and_signed_zero():
    w = np.zeros((2, 64), dtype=np.float32)
    w[0, :] = 0.125
    w[1, :] = 0.0
    w[1, 5] = -0.0
    packed, sb, bb = O.affine_quantize(w, 4, 64, "bf16")
    assert np.all(packed == 0)
    assert sb[0, 0] == 0 and sb[1, 0] == 0
    assert bb[0, 0] == O.f32_to_bf16_bits(np.float32(0.125))
    assert bb[1, 0] == 0x8000  # min under the total order is -0
    mn, mx = O.group_min_max(np.array([[0.0, -0.0], [-0.0, -0.0], [0.0, 0.0]], dtype=np.float32))
    assert list(np.signbit(mn)) == [True, True, False]
    assert list(np.signbit(mx)) == [False, True, False]


# ---------------------------------------------------------------- dequant and apply


def test_dequant_closed_form_and_output_rounding():
    packed = O.pack_codes(np.array([[0, 1, 2, 15] * 16]), 4)
    sb = O.to_bits("f16", np.array([[0.5]], dtype=np.float32))
    bb = O.to_bits("f16", np.array([[-3.0]], dtype=np.float32))
    v = O.affine_dequant_f32(packed, sb, bb, 4, 64, "f16", 64)
    np.testing.assert_array_equal(v[0, :4], [-3.0, -2.5, -2.0, 4.5])
    # a value not representable in bf16 is rounded once to nearest even
    sb = O.to_bits("f16", np.array([[2.0 ** -10 * 1.0009765625]], dtype=np.float32))
    bb = O.to_bits("f16", np.array([[1.0]], dtype=np.float32))
    v = O.affine_dequant_f32(packed, sb, bb, 4, 64, "f16", 64)
    exact = 1.0 + 15 * O.bits_to_f64("f16", sb)[0, 0]
    assert float(v[0, 3]) == float(np.float32(exact))
    want = torch.tensor([float(v[0, 3])], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert O.affine_dequant_to("bf16", packed, sb, bb, 4, 64, "f16", 64)[0, 3] == want[0]


def test_apply_one_hot_gives_columns_and_matches_loops():
    w = synth.weights_f32(9, 12, 64)
    packed, sb, bb = O.affine_quantize(w, 4, 32, "bf16")
    D = O.affine_dequant_f32(packed, sb, bb, 4, 32, "bf16", 64)
    for j in (0, 17, 63):
        x = np.zeros((1, 64))
        x[0, j] = 1.0
        np.testing.assert_array_equal(O.apply(x, D)[0], D[:, j].astype(np.float64))
    x = O.bits_to_f64("bf16", synth.acts_bits(10, 3, 64, "bf16"))
    y = O.apply(x, D, layer_bias=np.arange(12) * 0.5)
    for m in range(3):
        for n in range(12):
            acc = math.fsum(float(x[m, kk]) * float(D[n, kk]) for kk in range(64)) + n * 0.5
            assert abs(y[m, n] - acc) <= 1e-12 * (1 + abs(acc))


# ---------------------------------------------------------------- MXFP4


def _e2m1_bit_level(c):
    """OCP MX E2M1 bit-level definition: S E1 E0 M; E>0: 2^(E-1)*(1+M/2); E=0: M*0.5."""
    sgn = -1.0 if c & 8 else 1.0
    e = (c >> 1) & 3
    m = c & 1
    mag = 2.0 ** (e - 1) * (1 + m / 2) if e > 0 else 0.5 * m
    return sgn * mag


def test_mxfp4_magnitude_table_equals_bit_level_definition():
    for c in range(16):
        tab = (-1.0 if c & 8 else 1.0) * O.MXFP4_MAGNITUDES[c & 7]
        assert tab == _e2m1_bit_level(c)
        assert math.copysign(1.0, tab) == math.copysign(1.0, _e2m1_bit_level(c))


def test_mxfp4_golden_row():
    fx = _golden("mxfp4_row_codes_0_15.json")
    codes = np.array(fx["codes"], dtype=np.uint8)[None, :]
    scales = np.array([[fx["scale"]]], dtype=np.uint8)
    got = O.mxfp4_dequant_f32(codes, scales)[0]
    want = np.array([float(v) for v in fx["values"]], dtype=np.float32)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(want))


def test_mxfp4_exhaustive_codes_and_scales():
    """All 16 codes x 256 scale bytes: NaN at 255, inf for magnitude >= 4 at 253 and >= 2 at 254,
    every other value exact (equal to its fp64 value), and exactly representable in bf16."""
    codes = np.array([[(c | (c << 4)) for c in range(16)] * 1], dtype=np.uint8)  # 32 values
    codes = np.repeat(codes, 256, axis=0)
    scales = np.arange(256, dtype=np.uint8)[:, None]
    v = O.mxfp4_dequant_f32(codes, scales)
    for s in range(256):
        for c in range(16):
            got = float(v[s, 2 * c])
            assert float(v[s, 2 * c + 1]) == got or (math.isnan(got) and math.isnan(float(v[s, 2 * c + 1])))
            mag = O.MXFP4_MAGNITUDES[c & 7]
            if s == 255:
                assert math.isnan(got)
            elif (s == 253 and mag >= 4) or (s == 254 and mag >= 2):
                assert math.isinf(got)
            else:
                assert got == _e2m1_bit_level(c) * 2.0 ** (s - 127)
                b = O.f32_to_bf16_bits(np.float32(got))
                assert float(O.bf16_bits_to_f32(b)) == got
    zero = O.mxfp4_dequant_f32(np.zeros((1, 16), np.uint8), np.zeros((1, 1), np.uint8))
    assert np.all(zero == 0) and not np.any(np.signbit(zero))


# ---------------------------------------------------------------- Q8_0


def test_q8_0_equals_8bit_g32_affine_with_offset_128():
    """GGUF Q8_0 is 8-bit group-32 affine with code q+128, scale d, bias -128*d."""
    blocks = synth.q8_0_random_blocks(4, 1, 8, 256)[0]
    v = O.q8_0_dequant_f32(blocks)
    blk = blocks.reshape(8, 8, 34)
    d_bits = blk[..., 0].astype(np.uint16) | (blk[..., 1].astype(np.uint16) << 8)
    q = blk[..., 2:].view(np.int8).astype(np.int64)
    codes = (q + 128).reshape(8, 256)
    d = O.bits_to_f64("f16", d_bits)
    packed = O.pack_codes(codes, 8)
    sb = d_bits
    bb = O.to_bits("f16", (-128.0 * d).astype(np.float32))  # -128*d is exact in fp16 unless it overflows
    np.testing.assert_array_equal(O.bits_to_f64("f16", bb), -128.0 * d)
    va = O.affine_dequant_f32(packed, sb, bb, 8, 32, "f16", 256)
    np.testing.assert_array_equal(v, va)


def test_q8_0_hand_block_and_zero_block():
    blk = np.zeros(34, dtype=np.uint8)
    blk[0], blk[1] = 0x00, 0x38  # fp16 0.5, little-endian
    blk[2:] = np.arange(-128, -96, dtype=np.int64).astype(np.int8).view(np.uint8)
    v = O.q8_0_dequant_f32(blk[None, :])[0]
    np.testing.assert_array_equal(v, np.arange(-128, -96) * 0.5)
    z = O.q8_0_dequant_f32(np.zeros((1, 68), np.uint8))
    assert np.all(z == 0)


def test_q8_0_quantize_golden_halves_away():
    fx = _golden("q8_0_halves_away_block.json")
    w = np.array(fx["w"], dtype=np.float32)[None, :]
    blk = O.q8_0_quantize(w)[0]
    assert int(blk[0]) | (int(blk[1]) << 8) == fx["d_bits"]
    np.testing.assert_array_equal(blk[2:].view(np.int8), np.array(fx["quants"], dtype=np.int8))


def test_q8_0_quantize_round_trip_bound():
    w = synth.weights_f32(31, 16, 512)
    v = O.q8_0_dequant_f32(O.q8_0_quantize(w)).astype(np.float64)
    wb = w.reshape(16, 16, 32).astype(np.float64)
    d32 = np.abs(wb).max(-1, keepdims=True) / 127
    d16 = O.bits_to_f64("f16", O.f32_to_f16_bits(d32.astype(np.float32)))
    bound = d32 / 2 * (1 + 1e-6) + 127 * np.abs(d16 - d32)
    assert np.all(np.abs(wb - v.reshape(16, 16, 32)) <= bound)


# ---------------------------------------------------------------- routing and apply_experts


def test_route_is_stable_counting_sort():
    g = np.random.default_rng(12)
    ids = g.integers(-2, 9, size=300)
    offsets, perm = O.route(ids, 7)
    pairs = sorted([(int(i), p) for p, i in enumerate(ids) if 0 <= i < 7])
    assert list(perm) == [p for _, p in pairs]
    for e in range(7):
        assert offsets[e + 1] - offsets[e] == int(np.sum(ids == e))
    assert offsets[0] == 0 and offsets[-1] == len(pairs)


def test_apply_experts_rows_and_out_of_range_zero():
    e, n, k = 4, 6, 64
    W = np.stack([O.affine_dequant_f32(*O.affine_quantize(synth.weights_f32(40 + j, n, k), 4, 32, "bf16"), 4, 32, "bf16", k) for j in range(e)])
    x = O.bits_to_f64("bf16", synth.acts_bits(41, 5, k, "bf16"))
    ids = np.array([[0, 3], [1, -1], [4, 2], [2, 2], [3, 0]])
    y = O.apply_experts(W, ids.reshape(-1), x, pos_per_row=2)
    for p, i in enumerate(ids.reshape(-1)):
        if 0 <= i < e:
            ref = np.array([math.fsum(x[p // 2, kk] * float(W[i, r, kk]) for kk in range(k)) for r in range(n)])
            np.testing.assert_allclose(y[p], ref, rtol=1e-12, atol=1e-15)
        else:
            assert np.all(y[p] == 0)


def test_rel_l2_tolerance_helper():
    ref = np.array([[3.0, 4.0], [0.0, 0.0]])
    y = np.array([[3.0, 4.0 + 5e-3], [0.0, 0.0]])
    np.testing.assert_allclose(O.rel_l2_per_row(y, ref), [1e-3, 0.0])


# ---------------------------------------------------------------- quantize_q8_0 non-finite rules,
# MXFP4 in GGUF blocks, take (Nx_quant API docs: quantize_q8_0; Weights: Mxfp4_blocks; take)


def _blk(b):
    b = np.asarray(b, dtype=np.uint8)
    return int(b[0]) | (int(b[1]) << 8), b[2:].view(np.int8).astype(np.int64)


def test_q8_0_quantize_nonfinite_and_edge_blocks_by_the_page():
    w = np.zeros((1, 6 * 32), np.float32)
    w[0, 0:32] = np.linspace(-1, 1, 32)
    w[0, 5] = np.inf  # a block holding an infinity: scale +inf, quants 0
    w[0, 32:64] = 0.5
    w[0, 40] = np.nan  # a block holding a NaN: NaN scale, quants 0 (even with an infinity beside it)
    w[0, 41] = -np.inf
    w[0, 64:96] = 1e-39  # 1/d infinite (amax below ~127 * 2^-128): zero bytes
    w[0, 96:128] = 0.0  # d = 0: zero bytes
    w[0, 128:160] = 1e7  # d = 1e7/127 rounds past fp16's largest: scale +inf, quants from the fp32 1/d
    w[0, 160:192] = np.arange(32, dtype=np.float32) - 16.0  # amax 16: d = 16/127
    blocks = O.q8_0_quantize(w)[0].reshape(6, 34)
    d, q = _blk(blocks[0])
    assert d == 0x7C00 and np.all(q == 0)
    d, q = _blk(blocks[1])
    assert d == 0x7E00 and np.all(q == 0)
    assert np.all(blocks[2] == 0) and np.all(blocks[3] == 0)
    d, q = _blk(blocks[4])
    assert d == 0x7C00 and np.all(q == 127)
    d, q = _blk(blocks[5])
    d32 = np.float32(16.0) / np.float32(127.0)
    assert d == int(np.float16(d32).view(np.uint16))
    inv = np.float32(1.0) / d32
    want = [int(math.copysign(math.floor(abs(float(np.float32(v) * inv)) + 0.5), v)) for v in w[0, 160:192]]
    assert list(q) == want and q[0] == -127


def test_mxfp4_blocks_equal_split_layout_rearranged_by_hand():
    """The same codes and scales written in both layouts decode to the same values: split layout
    value 2i in the low nibble of byte i; GGUF block: scale byte, then byte j with value j low and
    value j + 16 high (built here value by value)."""
    g = np.random.default_rng(17)
    n, k = 5, 96
    codes = g.integers(0, 256, size=(n, k // 2)).astype(np.uint8)
    scales = g.integers(100, 140, size=(n, k // 32)).astype(np.uint8)
    scales[1, 2] = 255
    blocks = np.zeros((n, k // 32 * 17), np.uint8)
    for r in range(n):
        for bi in range(k // 32):
            blocks[r, bi * 17] = scales[r, bi]
            for i in range(32):
                kk = bi * 32 + i
                nib = (codes[r, kk // 2] >> (4 * (kk % 2))) & 0xF
                byte = bi * 17 + 1 + (i % 16)
                blocks[r, byte] |= nib << (4 * (i // 16))
    a = O.mxfp4_blocks_dequant_f32(blocks)
    b = O.mxfp4_dequant_f32(codes, scales)
    np.testing.assert_array_equal(np.isnan(a), np.isnan(b))
    np.testing.assert_array_equal(a[~np.isnan(a)].view(np.uint32), b[~np.isnan(b)].view(np.uint32))


def test_mxfp4_blocks_hand_block():
    blk = np.zeros(17, np.uint8)
    blk[0] = 128  # 2^1
    for j in range(16):
        blk[1 + j] = j | ((15 - j) << 4)
    mag = {0: 0.0, 1: 0.5, 2: 1.0, 3: 1.5, 4: 2.0, 5: 3.0, 6: 4.0, 7: 6.0}
    e2m1 = lambda c: (-1.0 if c & 8 else 1.0) * mag[c & 7]
    want = [2 * e2m1(j) for j in range(16)] + [2 * e2m1(15 - j) for j in range(16)]
    np.testing.assert_array_equal(O.mxfp4_blocks_dequant_f32(blk[None, :])[0], np.array(want, np.float32))


def test_take_is_the_gather_of_dequantized_rows():
    """dequant(take(p, w)) equals the rows p of dequant(w) for positions in range; positions out of
    range gather zero bytes, which decode to zeros (Nx_quant API docs, take)."""
    n, k, bits, g = 40, 256, 4, 64
    pk, sb, bb = O.affine_quantize(synth.weights_f32(91, n, k), bits, g, "bf16")
    D = O.affine_dequant_f32(pk, sb, bb, bits, g, "bf16", k)
    pos = np.array([3, 0, 39, -1, 40, 7, 7, 1000])
    T = O.affine_dequant_f32(O.take(pos, pk), O.take(pos, sb), O.take(pos, bb), bits, g, "bf16", k)
    for i, p in enumerate(pos):
        want = D[p] if 0 <= p < n else np.zeros(k, np.float32)
        np.testing.assert_array_equal(T[i], want)
    # Q8_0 and MXFP4 parts: zero bytes decode to zeros as well
    assert np.all(O.q8_0_dequant_f32(np.zeros((1, 34), np.uint8)) == 0)
    assert np.all(O.mxfp4_blocks_dequant_f32(np.zeros((1, 17), np.uint8)) == 0)


# ---------------------------------------------------------------- GPTQ -> affine transcoder
# (GPTQModel wiki "MLX Apple Silicon", Packed layouts and exact transcoding; GPTQModel "Packing
# Formats and Compatibility", GPTQ and GPTQ_V2)


def _gptq_case(seed, k, n, bits, g, pow2_scales=False):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 1 << bits, size=(k, n))  # [in, out]
    zeros = rng.integers(0, 1 << bits, size=(k // g, n))
    # qweight: each column's codes as one stream down the input axis, built with the digit-string
    # construction (independent of the oracle's packer); qzeros likewise along the outputs
    qweight = np.stack([_stream_words_from_digits([int(c) for c in codes[:, j]], bits) for j in range(n)], axis=1)
    qzeros = np.stack([_stream_words_from_digits([int(z) for z in zeros[r]], bits) for r in range(k // g)])
    if pow2_scales:
        s = np.ldexp(1.0, rng.integers(-12, -2, size=(k // g, n))).astype(np.float32)
    else:
        s = (rng.random((k // g, n)) * 0.02 + 1e-3).astype(np.float32)
    return codes, zeros, qweight.astype(np.uint32), qzeros.astype(np.uint32), s


@pytest.mark.parametrize("bits,pdt", [(4, "f16"), (3, "f16"), (2, "bf16"), (8, "f16")])
def test_gptq_transcode_reconstructs_scale_times_code_minus_zero(bits, pdt):
    k, n, g = 256, 64, 64
    codes, zeros, qw, qz, s = _gptq_case(60 + bits, k, n, bits, g)
    sb = O.to_bits(pdt, s)
    pk, so, bo = O.gptq_transcode(qw, qz, sb, bits, g, k, n, pdt)
    deq = O.affine_dequant_f32(pk, so, bo, bits, g, pdt, k).astype(np.float64)
    # GPTQ's reconstruction written out directly from the drawn codes, zeros and stored scales
    sv = O.bits_to_f64(pdt, sb)
    want = np.repeat(sv.T, g, axis=1) * (codes.T - np.repeat(zeros.T, g, axis=1))
    # the only rounding beyond fp32's is the bias -zero*scale stored in the parameter dtype
    bias_exact = -(zeros.T.astype(np.float64)) * sv.T
    slack = np.abs(O.bits_to_f64(pdt, bo) - bias_exact)
    bound = np.repeat(slack, g, axis=1) + np.abs(want) * 2.0 ** -23 + 1e-30
    assert np.all(np.abs(deq - want) <= bound)
    np.testing.assert_array_equal(O.unpack_codes(pk, bits, k), codes.T)
    np.testing.assert_array_equal(so, sb.T)


def test_gptq_transcode_exact_when_bias_representable_and_v1_zeros():
    k, n, g, bits = 128, 32, 32, 4
    codes, zeros, qw, qz, s = _gptq_case(70, k, n, bits, g, pow2_scales=True)
    sb = O.to_bits("f16", s)
    pk, so, bo = O.gptq_transcode(qw, qz, sb, bits, g, k, n, "f16")
    deq = O.affine_dequant_f32(pk, so, bo, bits, g, "f16", k).astype(np.float64)
    want = np.repeat(s.T.astype(np.float64), g, axis=1) * (codes.T - np.repeat(zeros.T, g, axis=1))
    np.testing.assert_array_equal(deq, want)
    # v1 stores zero - 1: the same weight written that way (zeros >= 1 only) transcodes to the same
    zeros1 = np.maximum(zeros, 1)
    qz1 = np.stack([_stream_words_from_digits([int(z) - 1 for z in zeros1[r]], bits) for r in range(k // g)])
    qz2 = np.stack([_stream_words_from_digits([int(z) for z in zeros1[r]], bits) for r in range(k // g)])
    a = O.gptq_transcode(qw, qz1.astype(np.uint32), sb, bits, g, k, n, "f16", v1_zeros=True)
    b = O.gptq_transcode(qw, qz2.astype(np.uint32), sb, bits, g, k, n, "f16")
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("bits,pdt,g", [(4, "f16", 64), (3, "bf16", 32), (2, "f16", 128), (8, "bf16", 64)])
@pytest.mark.parametrize("v1", [False, True])
def test_gptq_dequant_is_scale_times_code_minus_zero(bits, pdt, g, v1):
    """GPTQ's reconstruction (GPTQModel "Packing Formats and Compatibility", GPTQ and GPTQ_V2:
    value = scale * (code - zero), v1 storing zero - 1) against the drawn codes, zeros and stored
    scales written out element by element in pure Python (no unpacking shared with the oracle:
    qweight and qzeros are built by the digit-string construction)."""
    k, n = 256, 32
    rng = np.random.default_rng(80 + bits + (7 if v1 else 0))
    codes = rng.integers(0, 1 << bits, size=(k, n))
    zeros = rng.integers(1 if v1 else 0, 1 << bits, size=(k // g, n))
    stored = zeros - 1 if v1 else zeros
    qw = np.stack([_stream_words_from_digits([int(c) for c in codes[:, j]], bits) for j in range(n)], axis=1)
    qz = np.stack([_stream_words_from_digits([int(z) for z in stored[r]], bits) for r in range(k // g)])
    sb = O.to_bits(pdt, (rng.random((k // g, n)) * 0.02 + 1e-3).astype(np.float32))
    got = O.gptq_dequant_f64(qw.astype(np.uint32), qz.astype(np.uint32), sb, bits, g, k, n, pdt, v1_zeros=v1)
    assert got.shape == (n, k)
    sv = O.bits_to_f64(pdt, sb)
    for j in range(n):
        for i in range(0, k, 7):  # every 7th input of every output column
            want = float(sv[i // g, j]) * (int(codes[i, j]) - int(zeros[i // g, j]))
            assert got[j, i] == want, (j, i)
    # a plausible misreading of the v1 convention (zero stored as is) shifts every value by one scale
    if v1:
        wrong = O.gptq_dequant_f64(qw.astype(np.uint32), qz.astype(np.uint32), sb, bits, g, k, n, pdt)
        np.testing.assert_allclose(wrong - got, np.repeat(sv.T, g, axis=1))


# ---------------------------------------------------------------- GPTQ_P (planar) -> affine transcoder
# (GPTQModel "Packing Formats and Compatibility", GPTQ_P: 32 codes per b adjacent words, planes low
# first, fields least significant first; the plane table; true zeros; 2/4/8-bit planes identical to
# the continuous words, 3-bit packing different)

# the page's table of planes per width, as printed (the oracle derives it from the width's bits)
_PLANES_TABLE = {2: (2,), 3: (2, 1), 4: (4,), 5: (4, 1), 6: (4, 2), 7: (4, 2, 1), 8: (8,)}


def _planar_words(codes, bits):
    """One GPTQ_P stream from codes: per block of 32, each plane's fields (the code's bits from the
    plane's offset up) written as one little-endian stream with the digit-string construction."""
    out = []
    for b0 in range(0, len(codes), 32):
        blk = [int(c) for c in codes[b0:b0 + 32]]
        off = 0
        for wp in _PLANES_TABLE[bits]:
            out.append(_stream_words_from_digits([(c // (1 << off)) % (1 << wp) for c in blk], wp))
            off += wp
    return np.concatenate(out).astype(np.uint32)


def test_gptq_planar_hand_blocks():
    """Blocks worked out by hand from the layout: 3 bits, codes i % 8 (low plane fields i % 4 in
    two words, high plane bits (i // 4) % 2 in one); 5 bits, codes i; 6 bits, codes 63 - i; 7 bits,
    codes 96 + i (mid plane fields 2 then 3, high plane all ones)."""
    cases = {
        3: ([0xE4E4E4E4, 0xE4E4E4E4, 0xF0F0F0F0], [i % 8 for i in range(32)]),
        5: ([0x76543210, 0xFEDCBA98, 0x76543210, 0xFEDCBA98, 0xFFFF0000], list(range(32))),
        6: ([0x89ABCDEF, 0x01234567, 0x89ABCDEF, 0x01234567, 0xFFFFFFFF, 0xAAAAAAAA], [63 - i for i in range(32)]),
        7: ([0x76543210, 0xFEDCBA98, 0x76543210, 0xFEDCBA98, 0xAAAAAAAA, 0xFFFFFFFF, 0xFFFFFFFF],
            [96 + i for i in range(32)]),
    }
    for bits, (words, want) in cases.items():
        assert O.gptq_planes(bits) == _PLANES_TABLE[bits]
        got = O.gptq_planar_codes(np.array([words], dtype=np.uint32), bits, 32)
        np.testing.assert_array_equal(got[0], want, err_msg=f"bits={bits}")
        np.testing.assert_array_equal(_planar_words(want, bits), words)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_gptq_planar_single_plane_is_the_continuous_stream(bits):
    """At 2, 4 and 8 bits the planar words are the continuous words (one plane)."""
    w = np.random.default_rng(300 + bits).integers(0, 1 << 32, size=(5, 4 * bits), dtype=np.uint64).astype(np.uint32)
    np.testing.assert_array_equal(O.gptq_planar_codes(w, bits, 128), O.unpack_codes(w, bits, 128))


def test_gptq_planar_three_bits_differs_from_continuous():
    w = np.random.default_rng(310).integers(0, 1 << 32, size=(4, 12), dtype=np.uint64).astype(np.uint32)
    assert not np.array_equal(O.gptq_planar_codes(w, 3, 128), O.unpack_codes(w, 3, 128))


def _planar_case(seed, k, n, bits, g, pow2_scales=False):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 1 << bits, size=(k, n))  # [in, out]
    zeros = rng.integers(0, 1 << bits, size=(k // g, n))
    qweight = np.stack([_planar_words(codes[:, j], bits) for j in range(n)], axis=1)
    qzeros = np.stack([_planar_words(zeros[r], bits) for r in range(k // g)])
    if pow2_scales:
        s = np.ldexp(1.0, rng.integers(-12, -2, size=(k // g, n))).astype(np.float32)
    else:
        s = (rng.random((k // g, n)) * 0.02 + 1e-3).astype(np.float32)
    return codes, zeros, qweight.astype(np.uint32), qzeros.astype(np.uint32), s


@pytest.mark.parametrize("bits,pdt,g", [(2, "f16", 64), (3, "bf16", 32), (4, "f16", 128), (5, "f16", 64),
                                        (6, "bf16", 64), (7, "f16", 32), (8, "bf16", 64)])
def test_gptq_planar_transcode_reconstructs_scale_times_code_minus_zero(bits, pdt, g):
    k, n = 256, 64
    codes, zeros, qw, qz, s = _planar_case(320 + bits, k, n, bits, g)
    sb = O.to_bits(pdt, s)
    pk, so, bo = O.gptq_planar_transcode(qw, qz, sb, bits, g, k, n, pdt)
    tb = 8 if bits == 7 else bits
    assert pk.shape == (n, k * tb // 32)
    np.testing.assert_array_equal(O.unpack_codes(pk, tb, k), codes.T)
    np.testing.assert_array_equal(so, sb.T)
    deq = O.affine_dequant_f32(pk, so, bo, tb, g, pdt, k).astype(np.float64)
    sv = O.bits_to_f64(pdt, sb)
    own = O.gptq_planar_dequant_f64(qw, qz, sb, bits, g, k, n, pdt)
    for j in range(0, n, 5):
        for i in range(0, k, 3):
            # true zeros: no v1 correction
            want = float(sv[i // g, j]) * (int(codes[i, j]) - int(zeros[i // g, j]))
            assert own[j, i] == want, (j, i)
            bias_err = abs(float(O.bits_to_f64(pdt, bo[j, i // g])) + float(zeros[i // g, j]) * float(sv[i // g, j]))
            assert abs(deq[j, i] - want) <= bias_err + abs(want) * 2.0 ** -23 + 1e-30, (j, i)


def test_gptq_planar_transcode_exact_with_power_of_two_scales():
    k, n, g, bits = 128, 64, 32, 6
    codes, zeros, qw, qz, s = _planar_case(330, k, n, bits, g, pow2_scales=True)
    sb = O.to_bits("f16", s)
    pk, so, bo = O.gptq_planar_transcode(qw, qz, sb, bits, g, k, n, "f16")
    deq = O.affine_dequant_f32(pk, so, bo, bits, g, "f16", k).astype(np.float64)
    want = np.repeat(s.T.astype(np.float64), g, axis=1) * (codes.T - np.repeat(zeros.T, g, axis=1))
    np.testing.assert_array_equal(deq, want)


# ---------------------------------------------------------------- AWQ GEMM -> affine transcoder
# (GPTQModel wiki "MLX Apple Silicon", Packed layouts and exact transcoding, AWQ GEMM row, and
# ParoQuant: the lane order [0,2,4,6,1,3,5,7]; GPTQModel "Packing Formats and Compatibility",
# AWQ GEMM: qweight [K, N/8], qzeros [G, N/8], scales [G, N])


def test_awq_lane_order_hand_words():
    """A word whose nibble i (from the low nibble up) holds the value i decodes, in natural column
    order, to the inverse of the page's lane order: column c holds the slot at which c appears in
    [0,2,4,6,1,3,5,7]."""
    w = np.array([[0x76543210, 0xFEDCBA98]], dtype=np.uint32)
    np.testing.assert_array_equal(O.awq_codes(w, 4, 16)[0],
                                  [0, 4, 1, 5, 2, 6, 3, 7, 8, 12, 9, 13, 10, 14, 11, 15])
    # a word holding columns 0..7 = 1,2,...,8 in AWQ order, written out nibble by nibble:
    # slots hold columns 0,2,4,6,1,3,5,7 -> values 1,3,5,7,2,4,6,8 -> 0x86427531
    np.testing.assert_array_equal(O.awq_codes(np.array([[0x86427531]], dtype=np.uint32), 4, 8)[0],
                                  [1, 2, 3, 4, 5, 6, 7, 8])
    # 8-bit rows are plain little-endian byte streams (no permutation); 2-bit likewise
    np.testing.assert_array_equal(O.awq_codes(np.array([[0x44332211]], dtype=np.uint32), 8, 4)[0],
                                  [0x11, 0x22, 0x33, 0x44])
    np.testing.assert_array_equal(O.awq_codes(np.array([[0xE4E4E4E4]], dtype=np.uint32), 2, 16)[0],
                                  [0, 1, 2, 3] * 4)


def _awq_stream_words(natural, bits):
    """One AWQ row from codes in natural column order: at 4 bits each 8-column block is written in
    the page's lane order (slot i takes column order[i]), then the row is one little-endian stream
    built with the digit-string construction."""
    natural = [int(c) for c in natural]
    if bits == 4:
        order = (0, 2, 4, 6, 1, 3, 5, 7)
        natural = [natural[8 * (i // 8) + order[i % 8]] for i in range(len(natural))]
    return _stream_words_from_digits(natural, bits)


def _awq_case(seed, k, n, bits, g, pow2_scales=False):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 1 << bits, size=(k, n))  # [in, out]
    zeros = rng.integers(0, 1 << bits, size=(k // g, n))
    qweight = np.stack([_awq_stream_words(codes[r], bits) for r in range(k)])
    qzeros = np.stack([_awq_stream_words(zeros[r], bits) for r in range(k // g)])
    if pow2_scales:
        s = np.ldexp(1.0, rng.integers(-12, -2, size=(k // g, n))).astype(np.float32)
    else:
        s = (rng.random((k // g, n)) * 0.02 + 1e-3).astype(np.float32)
    return codes, zeros, qweight.astype(np.uint32), qzeros.astype(np.uint32), s


@pytest.mark.parametrize("bits,pdt,g", [(4, "f16", 64), (3, "bf16", 32), (2, "f16", 128), (5, "f16", 64),
                                        (6, "bf16", 64), (7, "f16", 32), (8, "bf16", 64)])
def test_awq_transcode_reconstructs_scale_times_code_minus_zero(bits, pdt, g):
    k, n = 256, 64
    codes, zeros, qw, qz, s = _awq_case(90 + bits, k, n, bits, g)
    sb = O.to_bits(pdt, s)
    pk, so, bo = O.awq_transcode(qw, qz, sb, bits, g, k, n, pdt)
    tb = 8 if bits == 7 else bits
    assert pk.shape == (n, k * tb // 32)
    # the affine rows hold the drawn codes (a 7-bit source keeps its values in 8-bit words)
    np.testing.assert_array_equal(O.unpack_codes(pk, tb, k), codes.T)
    np.testing.assert_array_equal(so, sb.T)
    # AWQ's value scale * (code - zero), element by element from the drawn numbers, against the
    # affine value code * scale + bias; the only rounding is the bias's, to the parameter dtype
    deq = O.affine_dequant_f32(pk, so, bo, tb, g, pdt, k).astype(np.float64)
    sv = O.bits_to_f64(pdt, sb)
    own = O.awq_dequant_f64(qw, qz, sb, bits, g, k, n, pdt)
    for j in range(0, n, 5):
        for i in range(0, k, 3):
            want = float(sv[i // g, j]) * (int(codes[i, j]) - int(zeros[i // g, j]))
            assert own[j, i] == want, (j, i)
            bias_err = abs(float(O.bits_to_f64(pdt, bo[j, i // g])) + float(zeros[i // g, j]) * float(sv[i // g, j]))
            assert abs(deq[j, i] - want) <= bias_err + abs(want) * 2.0 ** -23 + 1e-30, (j, i)


def test_awq_transcode_exact_with_power_of_two_scales_and_misorder_fails():
    k, n, g, bits = 128, 32, 32, 4
    codes, zeros, qw, qz, s = _awq_case(97, k, n, bits, g, pow2_scales=True)
    sb = O.to_bits("f16", s)
    pk, so, bo = O.awq_transcode(qw, qz, sb, bits, g, k, n, "f16")
    deq = O.affine_dequant_f32(pk, so, bo, bits, g, "f16", k).astype(np.float64)
    want = np.repeat(s.T.astype(np.float64), g, axis=1) * (codes.T - np.repeat(zeros.T, g, axis=1))
    np.testing.assert_array_equal(deq, want)
    # reading the 4-bit words as plain streams (the permutation ignored) gives other codes
    plain = O.pack_codes(O.unpack_codes(qw, 4, n).T, 4)
    assert not np.array_equal(plain, pk)


# ---------------------------------------------------------------- Q4_K and Q6_K
# (Nx_quant API docs, "Weights": Q4_K and Q6_K block layouts and value formulas; the float32 rule
# for GGUF values: a Q6_K value and a Q4_K product are exact, a Q4_K value rounds once at its
# subtraction; a zero block decodes to zeros, -0 in Q6_K.)  The blocks below are written by a
# bit-level builder that places each field where the reading puts it, independently of the
# oracle's index tables.
from fractions import Fraction


def _put(buf, byte, bit, nbits, value):
    """Write `value` into `nbits` bits of buf starting at bit `bit` of byte `byte` (within the byte)."""
    assert 0 <= value < (1 << nbits) and bit + nbits <= 8
    mask = ((1 << nbits) - 1) << bit
    buf[byte] = (buf[byte] & ~mask & 0xFF) | (value << bit)


def _q4_k_block(d_bits, dmin_bits, sc, mn, q):
    buf = bytearray(144)
    buf[0:2] = int(d_bits).to_bytes(2, "little")
    buf[2:4] = int(dmin_bits).to_bytes(2, "little")
    for j in range(8):
        if j < 4:  # low 6 bits of scale bytes j (scale) and j + 4 (min)
            _put(buf, 4 + j, 0, 6, int(sc[j]))
            _put(buf, 4 + j + 4, 0, 6, int(mn[j]))
        else:  # low / high nibble of byte j + 4, top two bits of bytes j - 4 (scale) and j (min)
            _put(buf, 4 + j + 4, 0, 4, int(sc[j]) & 15)
            _put(buf, 4 + j + 4, 4, 4, int(mn[j]) & 15)
            _put(buf, 4 + j - 4, 6, 2, int(sc[j]) >> 4)
            _put(buf, 4 + j, 6, 2, int(mn[j]) >> 4)
    for v in range(256):  # 64-value chunks of 32 bytes: values 0..31 low nibbles, 32..63 high
        _put(buf, 16 + 32 * (v // 64) + v % 32, 4 * ((v % 64) // 32), 4, int(q[v]))
    return np.frombuffer(bytes(buf), dtype=np.uint8)


def _q6_k_block(d_bits, sc, q):
    buf = bytearray(210)
    for v in range(256):
        h, w = divmod(v, 128)
        g, l = divmod(w, 32)
        _put(buf, 64 * h + 32 * (g % 2) + l, 4 * (g // 2), 4, int(q[v]) & 15)
        _put(buf, 128 + 32 * h + l, 2 * g, 2, int(q[v]) >> 4)
    for i in range(16):
        buf[192 + i] = int(sc[i]) & 0xFF
    buf[208:210] = int(d_bits).to_bytes(2, "little")
    return np.frombuffer(bytes(buf), dtype=np.uint8)


def _f16_fraction(bits):
    return Fraction(float(O.f16_bits_to_f32(np.uint16(bits))))


def _rne_f32(x: Fraction) -> float:
    """x rounded to nearest even at 24 significant bits (x normal in fp32 or 0), exactly."""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    scale = Fraction(2) ** (23 - e)
    n = a * scale
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(Fraction(fl) / scale)


def test_q4_k_values_follow_the_formula_with_one_rounding():
    rng = np.random.default_rng(301)
    for trial in range(6):
        d_bits = int(O.f32_to_f16_bits(np.float32(rng.uniform(1e-4, 0.05))))
        dmin_bits = int(O.f32_to_f16_bits(np.float32(rng.uniform(1e-4, 0.05))))
        sc, mn = rng.integers(0, 64, 8), rng.integers(0, 64, 8)
        q = rng.integers(0, 16, 256)
        blk = _q4_k_block(d_bits, dmin_bits, sc, mn, q)
        got = O.q4_k_dequant_f32(blk[None, :])[0]
        d, dmin = _f16_fraction(d_bits), _f16_fraction(dmin_bits)
        for v in range(256):
            j = v // 32
            want = _rne_f32(d * int(sc[j]) * int(q[v]) - dmin * int(mn[j]))
            assert float(got[v]) == want, (trial, v)


def test_q4_k_rounds_once_at_the_subtraction():
    # d = 1, sc = 63, q = 15: 945 (ulp 2^-14 in fp32); dmin * m = 63 * (1 + 2^-10) * 2^-14 is not a
    # multiple of that ulp, so the difference rounds, once
    d_bits, dmin_bits = 0x3C00, 0x0401  # 1.0 and (1 + 2^-10) * 2^-14
    sc, mn = np.full(8, 63), np.full(8, 63)
    q = np.full(256, 15)
    got = O.q4_k_dequant_f32(_q4_k_block(d_bits, dmin_bits, sc, mn, q)[None, :])[0]
    exact = Fraction(945) - 63 * _f16_fraction(dmin_bits)
    assert float(got[0]) == _rne_f32(exact)
    assert Fraction(float(got[0])) != exact  # the value did need rounding
    # products kept exact: with d = 1 + 2^-10 the product d*sc*q = 945 (1 + 2^-10) has 20 significant
    # bits; a decode that rounded it to the fp16 scale dtype first (946) would give another value
    got2 = O.q4_k_dequant_f32(_q4_k_block(0x3C01, dmin_bits, sc, mn, q)[None, :])[0]
    exact2 = 945 * _f16_fraction(0x3C01) - 63 * _f16_fraction(dmin_bits)
    assert float(got2[0]) == _rne_f32(exact2)
    assert float(got2[0]) != _rne_f32(Fraction(946) - 63 * _f16_fraction(dmin_bits))


def test_q6_k_values_exact_and_zero_blocks_signed():
    rng = np.random.default_rng(302)
    for trial in range(6):
        d_bits = int(O.f32_to_f16_bits(np.float32(rng.uniform(1e-4, 0.05) * rng.choice([-1, 1]))))
        sc = rng.integers(-128, 128, 16)
        q = rng.integers(0, 64, 256)
        blk = _q6_k_block(d_bits, sc, q)
        got = O.q6_k_dequant_f32(blk[None, :])[0]
        d = _f16_fraction(d_bits)
        for v in range(256):
            want = d * int(sc[v // 16]) * (int(q[v]) - 32)
            assert Fraction(float(got[v])) == want, (trial, v)  # exact
    # extremes of the quant: 0 -> -32, 63 -> 31
    q = np.array([0, 63] * 128)
    got = O.q6_k_dequant_f32(_q6_k_block(0x3C00, np.ones(16, dtype=np.int64), q)[None, :])[0]
    assert got[0] == -32.0 and got[1] == 31.0
    # zero blocks: Q4_K gives +0, Q6_K gives -0 (0 * (0 - 32))
    z4 = O.q4_k_dequant_f32(np.zeros((2, 144), dtype=np.uint8))
    z6 = O.q6_k_dequant_f32(np.zeros((2, 210), dtype=np.uint8))
    assert np.all(z4 == 0) and not np.any(np.signbit(z4))
    assert np.all(z6 == 0) and np.all(np.signbit(z6))


def test_q4_k_q6_k_nonfinite_scales():
    q = np.arange(256) % 16
    inf4 = O.q4_k_dequant_f32(_q4_k_block(0x7C00, 0, np.full(8, 1), np.zeros(8, dtype=np.int64), q)[None, :])[0]
    assert np.all(np.isinf(inf4[q > 0])) and np.all(np.isnan(inf4[q == 0]))  # inf * 0 is NaN
    nan6 = O.q6_k_dequant_f32(_q6_k_block(0x7E00, np.ones(16, dtype=np.int64), np.arange(256) % 64)[None, :])[0]
    assert np.all(np.isnan(nan6))


def test_q4_k_q6_k_rows_of_blocks():
    """A row of several blocks decodes block by block (k = 512: two blocks per row, three rows)."""
    rng = np.random.default_rng(303)
    rows4, rows6, want4, want6 = [], [], [], []
    for r in range(3):
        b4, b6 = [], []
        for bi in range(2):
            blk4 = _q4_k_block(0x2000 + r * 16 + bi, 0x1800 + bi, rng.integers(0, 64, 8), rng.integers(0, 64, 8),
                               rng.integers(0, 16, 256))
            blk6 = _q6_k_block(0x2400 + r + bi, rng.integers(-128, 128, 16), rng.integers(0, 64, 256))
            b4.append(blk4)
            b6.append(blk6)
            want4.append(O.q4_k_dequant_f32(blk4[None, :])[0])
            want6.append(O.q6_k_dequant_f32(blk6[None, :])[0])
        rows4.append(np.concatenate(b4))
        rows6.append(np.concatenate(b6))
    got4 = O.q4_k_dequant_f32(np.stack(rows4))
    got6 = O.q6_k_dequant_f32(np.stack(rows6))
    np.testing.assert_array_equal(got4.reshape(-1), np.concatenate(want4))
    np.testing.assert_array_equal(got6.reshape(-1), np.concatenate(want6))
