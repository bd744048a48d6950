"""GPU parity of every entry point against the CPU oracle (run on an MI355X, -m gpu).

Bars: bit-exact for packed words, codes, scales, biases, dequantized values, routing indices;
relative l2 per output row <= 2e-3 (fp32 output vs the fp64 oracle) for products, with the
observed error printed.  Every input is seeded and synthetic (synth); every expected value is
computed by the oracle from oracle-side inputs.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_quantized_affine_amd as q
from gpu_helpers import (DEV, TDT, bits_to_dev, dev_to_bits, dev_to_u32, out_bits_or_f32, out_f64, same_values,
                         u32_to_dev, u8_to_dev)

pytestmark = pytest.mark.gpu
TOL = 2e-3  # the products' bound (relative l2 per output row), and the bound for 16-bit outputs
# Derived bounds for fp32 outputs of paths that round each weight once to fp16 (11 significant bits,
# a relative error within 2^-11 that is near-uniform, so about 2^-11/sqrt(3) = 2.8e-4 in a row's l2
# norm at most): the GEMM measures 2.7e-4 at most (8-bit rows; 3.5e-5 at the 9B-layer shapes) and
# the Q8_0 experts 2.6e-4; the bounds sit ~4x above the worst measured row.
GEMM_TOL = 1e-3
Q8_TOL = 1e-3


def _sync():
    torch.cuda.synchronize()


# ============================================================ quantize


def _check_quantize(w, bits, g, pdt):
    wt = torch.from_numpy(w).to(DEV)
    packed, scales, biases = q.qlinear_quantize(wt, bits, g, TDT[pdt])
    _sync()
    opk, osb, obb = O.affine_quantize(w, bits, g, pdt)
    np.testing.assert_array_equal(dev_to_u32(packed), opk)
    np.testing.assert_array_equal(dev_to_bits(scales), osb)
    np.testing.assert_array_equal(dev_to_bits(biases), obb)


def test_quantize_smoke_layer_bitexact():
    """256x512 fp32 ~N(0,0.02), 4-bit g64, fp16 scales/biases: 4096 words, 512 scales, 512 biases."""
    _check_quantize(synth.weights_f32(synth.seed_for(1), 256, 512), 4, 64, "f16")


@pytest.mark.parametrize("bits,g,pdt", [(4, 32, "bf16"), (4, 64, "bf16"), (4, 128, "f16"), (8, 32, "f16"),
                                        (8, 64, "bf16"), (8, 128, "bf16")])
def test_quantize_combinations_ragged_and_edge_groups(bits, g, pdt):
    n, k = 37, 384
    w = synth.weights_f32(100 + bits + g, n, k)
    w[1] *= 1000.0  # large values
    w[2] *= 1e-4  # tiny values
    w[3, :g] = 0.25  # constant group
    w[4, :g] = 0.0  # zeros of both signs
    w[4, 5] = -0.0
    w[5, g:2 * g] = -0.0
    w[6, :g] = np.linspace(-1, 1, g, dtype=np.float32)  # exact ties possible
    _check_quantize(w, bits, g, pdt)


def test_quantize_lm_head_full_size_sampled_rows():
    """Full 151936x1024 lm_head at 4-bit g64 bf16 (the decode workload); 512 sampled rows bit-exact."""
    n, k = 151936, 1024
    w = synth.weights_f32(synth.seed_for(2, 28, 0), n, k)
    wt = torch.from_numpy(w).to(DEV)
    packed, scales, biases = q.qlinear_quantize(wt, 4, 64, torch.bfloat16)
    _sync()
    rows = np.sort(np.random.default_rng(5).choice(n, 512, replace=False))
    rows[-1] = n - 1
    opk, osb, obb = O.affine_quantize(w[rows], 4, 64, "bf16")
    np.testing.assert_array_equal(dev_to_u32(packed[rows]), opk)
    np.testing.assert_array_equal(dev_to_bits(scales[rows]), osb)
    np.testing.assert_array_equal(dev_to_bits(biases[rows]), obb)


def test_quantize_deterministic():
    w = torch.from_numpy(synth.weights_f32(91, 1000, 1024)).to(DEV)
    a = q.qlinear_quantize(w, 4, 64, torch.bfloat16)
    b = q.qlinear_quantize(w, 4, 64, torch.bfloat16)
    _sync()
    assert all(torch.equal(u, v) for u, v in zip(a, b))


# ============================================================ dequant


@pytest.mark.parametrize("bits,g,pdt", [(4, 64, "f16"), (4, 32, "bf16"), (8, 128, "bf16"), (8, 64, "f16")])
@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
def test_dequant_affine_bitexact(bits, g, pdt, odt):
    n, k = 45, 512
    w = synth.weights_f32(7 + bits, n, k, std=0.5)
    opk, osb, obb = O.affine_quantize(w, bits, g, pdt)
    out = q.qlinear_dequant(q.QL_AFFINE, u32_to_dev(opk), bits_to_dev(osb, pdt), bits_to_dev(obb, pdt), rows=n, k=k,
                            bits=bits, group_size=g, out_dtype=TDT[odt])
    _sync()
    want = O.affine_dequant_to(odt, opk, osb, obb, bits, g, pdt, k)
    assert same_values(out_bits_or_f32(out, odt), want)


@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
def test_dequant_mxfp4_exhaustive_codes_and_scales(odt):
    """All 16 codes x all 256 scale bytes (NaN block, infinities, fp32 subnormals, -0)."""
    row = np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE] * 2, dtype=np.uint8)
    codes = np.tile(row, (256, 1))
    scales = np.arange(256, dtype=np.uint8)[:, None]
    out = q.qlinear_dequant(q.QL_MXFP4, u8_to_dev(codes), u8_to_dev(scales), rows=256, k=32, out_dtype=TDT[odt])
    _sync()
    want = O.round_f32_to(odt, O.mxfp4_dequant_f32(codes, scales))
    got = out_bits_or_f32(out, odt)
    if odt == "f32":
        assert same_values(got, want)
    else:
        nan = np.isnan(O.bits_to_f64(odt, want))
        assert np.array_equal(nan, np.isnan(O.bits_to_f64(odt, got)))
        assert np.array_equal(got[~nan], want[~nan])


def test_dequant_mxfp4_expert_stack_random():
    codes, scales = synth.mxfp4_codes_scales(11, 3, 50, 256)
    out = q.qlinear_dequant(q.QL_MXFP4, u8_to_dev(codes), u8_to_dev(scales), rows=150, k=256)
    _sync()
    assert same_values(out.cpu().numpy(), O.mxfp4_dequant_f32(codes, scales).reshape(150, 256))


@pytest.mark.parametrize("odt", ["f32", "bf16"])
def test_dequant_q8_0_bitexact(odt):
    blocks = np.concatenate([O.q8_0_quantize(synth.weights_f32(12, 40, 256)),
                             synth.q8_0_random_blocks(13, 1, 24, 256)[0],
                             np.zeros((1, 8 * 34), np.uint8)])
    rows = blocks.shape[0]
    out = q.qlinear_dequant(q.QL_Q8_0, u8_to_dev(blocks), rows=rows, k=256, out_dtype=TDT[odt])
    _sync()
    want = O.round_f32_to(odt, O.q8_0_dequant_f32(blocks))
    assert same_values(out_bits_or_f32(out, odt), want)


# ============================================================ products: shared helpers


def _affine_case(seed, n, k, bits, g, pdt, std=0.02):
    w = synth.weights_f32(seed, n, k, std=std)
    opk, osb, obb = O.affine_quantize(w, bits, g, pdt)
    D = O.affine_dequant_f32(opk, osb, obb, bits, g, pdt, k)
    return (u32_to_dev(opk), bits_to_dev(osb, pdt), bits_to_dev(obb, pdt)), D


def _x_case(seed, m, k, xdt):
    xb = synth.acts_bits(seed, m, k, xdt)
    return bits_to_dev(xb, xdt), O.bits_to_f64(xdt, xb)


def _assert_rel(y_dev, ref, tol=TOL, label=""):
    err = O.rel_l2_per_row(out_f64(y_dev), ref)
    print(f"{label} max rel-l2 {err.max():.3e}")
    assert err.max() <= tol, f"{label}: max rel-l2 {err.max():.3e}"
    return err.max()


# ============================================================ GEMV


def test_gemv_smoke_layer():
    """256x512, 4-bit g64, fp16 scales, x fp16 [1,512]: quantize, dequant and GEMV against the oracle."""
    (pk, sc, bi), D = _affine_case(synth.seed_for(1), 256, 512, 4, 64, "f16")
    x, xf = _x_case(synth.seed_for(1, part=1), 1, 512, "f16")
    y = q.qlinear_gemv(x, pk, sc, bi, bits=4, group_size=64, y_dtype=torch.float32)
    y16 = q.qlinear_gemv(x, pk, sc, bi, bits=4, group_size=64)
    _sync()
    ref = O.apply(xf, D)
    assert _assert_rel(y, ref, 1e-4, "gemv smoke f32")
    # fp16 output: compared with the oracle rounded once to fp16
    want16 = O.bits_to_f64("f16", O.to_bits("f16", ref.astype(np.float32)))
    _assert_rel(y16, want16, TOL, "gemv smoke f16-out vs RNE16(oracle)")


@pytest.mark.parametrize("bits,xdt", [(4, "bf16"), (4, "f16"), (8, "bf16"), (8, "f16")])
def test_gemv_one_hot_gives_exact_columns(bits, xdt):
    n, k = 70, 3072
    (pk, sc, bi), D = _affine_case(21, n, k, bits, 64, "bf16")
    js = [0, 1, 31, 32, 777, k - 1]
    xb = np.zeros((len(js), k), np.float32)
    for i, j in enumerate(js):
        xb[i, j] = 1.0
    x = bits_to_dev(O.to_bits(xdt, xb), xdt)
    y = q.qlinear_gemv(x, pk, sc, bi, bits=bits, group_size=64, y_dtype=torch.float32)
    _sync()
    np.testing.assert_array_equal(y.cpu().numpy(), D[:, js].T)


GEMV_CASES = [
    # m, n, k, bits, g, xdt, pdt, ydt
    (1, 2048, 1024, 4, 64, "bf16", "bf16", "f32"),
    (1, 1024, 3072, 4, 64, "bf16", "bf16", "bf16"),
    (1, 333, 160, 4, 32, "f16", "bf16", "f32"),
    (2, 517, 2048, 4, 128, "bf16", "f16", "f32"),
    (3, 300, 1024, 8, 64, "bf16", "bf16", "f32"),
    (4, 129, 384, 8, 32, "f16", "f16", "f16"),
    (5, 64, 3072, 8, 128, "bf16", "bf16", "f32"),
    (8, 1024, 1024, 8, 64, "bf16", "bf16", "f32"),
    (8, 250, 2048, 4, 64, "f16", "f16", "f32"),
    (11, 90, 512, 4, 64, "bf16", "bf16", "f32"),
    (1, 77, 96, 8, 32, "bf16", "f16", "bf16"),
    # 4-bit, k a multiple of 128: the matrix-core kernel (ragged rows, u-blocks past the row end,
    # every group size and row-count template, x rows that fill the accumulator rows partly)
    (1, 1000, 640, 4, 64, "bf16", "bf16", "f32"),
    (2, 64, 128, 4, 64, "f16", "f16", "f16"),
    (3, 257, 384, 4, 32, "f16", "bf16", "f32"),
    (4, 200, 1024, 4, 32, "bf16", "bf16", "f32"),
    (4, 130, 1152, 4, 128, "bf16", "f16", "bf16"),
    (6, 300, 2560, 4, 64, "bf16", "bf16", "f32"),
    (8, 70, 768, 4, 128, "bf16", "bf16", "f32"),
    (7, 1100, 3072, 4, 64, "f16", "bf16", "bf16"),
    # 5-8 x rows at 4 bits read whole lines regrouped through LDS: an odd u-block count (the last
    # step's second u-block clamped) and a single u-block per row
    (5, 200, 1152, 4, 64, "bf16", "bf16", "f32"),
    (8, 33, 128, 4, 64, "bf16", "f16", "f32"),
    # m = 5..8 with group size 32 needs 32 accumulator rows: the vector-ALU kernel
    (5, 100, 512, 4, 32, "bf16", "bf16", "f32"),
    # 8-bit, k a multiple of 128: the matrix-core kernel with f16 products (bf16 x converted)
    (1, 1000, 1024, 8, 64, "bf16", "bf16", "f32"),
    (1, 300, 3072, 8, 128, "f16", "bf16", "bf16"),
    (2, 257, 640, 8, 32, "bf16", "f16", "f32"),
    (4, 190, 1280, 8, 64, "f16", "f16", "f32"),
    (8, 500, 3072, 8, 64, "bf16", "bf16", "bf16"),
]


@pytest.mark.parametrize("m,n,k,bits,g,xdt,pdt,ydt", GEMV_CASES)
def test_gemv_parity(m, n, k, bits, g, xdt, pdt, ydt):
    (pk, sc, bi), D = _affine_case(1000 + m * 7 + n, n, k, bits, g, pdt)
    x, xf = _x_case(2000 + m + k, m, k, xdt)
    y = q.qlinear_gemv(x, pk, sc, bi, bits=bits, group_size=g, y_dtype=TDT[ydt])
    _sync()
    ref = O.apply(xf, D)
    if ydt == "f32":
        _assert_rel(y, ref, 1e-4, "gemv")
    else:
        want = O.bits_to_f64(ydt, O.to_bits(ydt, ref.astype(np.float32)))
        _assert_rel(y, want, TOL, "gemv 16-bit out vs rounded oracle")


@pytest.mark.parametrize("bits,m", [(8, 3), (8, 8), (4, 3)])
def test_gemv_x_row_magnitudes(bits, m):
    """x rows from 1e-30 to 1e30 (bf16): the per-row power-of-two factor of the f16 conversion
    keeps every row exact, so each row meets the same bound."""
    n, k = 300, 1024
    (pk, sc, bi), D = _affine_case(61, n, k, bits, 64, "bf16")
    mags = np.array([1e-30, 1.0, 1e30, 3e-5, 7e4, 1e-12, 1e12, 0.0][:m], np.float32)
    xb32 = synth.weights_f32(62, m, k, std=1.0) * mags[:, None]
    xbits = O.to_bits("bf16", xb32)
    y = q.qlinear_gemv(bits_to_dev(xbits, "bf16"), pk, sc, bi, bits=bits, group_size=64, y_dtype=torch.float32)
    _sync()
    ref = O.apply(O.bits_to_f64("bf16", xbits), D)
    got = out_f64(y)
    for r in range(m):
        if mags[r] == 0.0:
            assert np.all(got[r] == 0.0)
            continue
        err = np.linalg.norm(got[r] - ref[r]) / np.linalg.norm(ref[r])
        assert err <= 1e-4, f"row {r} (|x| ~ {mags[r]:g}): rel-l2 {err:.3e}"


def test_gemv_layer_bias_and_empty_k():
    (pk, sc, bi), D = _affine_case(31, 200, 1024, 4, 64, "bf16")
    x, xf = _x_case(32, 3, 1024, "bf16")
    lb_bits = synth.acts_bits(33, 1, 200, "bf16")[0]
    lb = bits_to_dev(lb_bits, "bf16")
    y = q.qlinear_gemv(x, pk, sc, bi, bits=4, group_size=64, layer_bias=lb, y_dtype=torch.float32)
    _sync()
    _assert_rel(y, O.apply(xf, D, layer_bias=O.bits_to_f64("bf16", lb_bits)), 1e-4, "gemv+bias")
    # k == 0: the product is the layer bias
    x0 = torch.empty((3, 0), dtype=torch.bfloat16, device=DEV)
    pk0 = torch.empty((200, 0), dtype=torch.int32, device=DEV)
    s0 = torch.empty((200, 0), dtype=torch.bfloat16, device=DEV)
    y0 = q.qlinear_gemv(x0, pk0, s0, s0, bits=4, group_size=64, layer_bias=lb, y_dtype=torch.float32)
    _sync()
    np.testing.assert_array_equal(y0.cpu().numpy(), np.tile(O.bf16_bits_to_f32(lb_bits), (3, 1)))


def test_gemv_deterministic():
    (pk, sc, bi), _ = _affine_case(41, 4096, 1024, 4, 64, "bf16")
    x, _ = _x_case(42, 1, 1024, "bf16")
    a = q.qlinear_gemv(x, pk, sc, bi, bits=4, group_size=64, y_dtype=torch.float32)
    b = q.qlinear_gemv(x, pk, sc, bi, bits=4, group_size=64, y_dtype=torch.float32)
    _sync()
    assert torch.equal(a, b)


# ============================================================ GEMM


GEMM_CASES = [
    # m, n, k, bits, g, xdt, pdt
    (300, 333, 1024, 4, 64, "bf16", "bf16"),
    (257, 256, 2048, 4, 128, "bf16", "f16"),
    (130, 200, 224, 4, 32, "bf16", "bf16"),  # k % 64 == 32: a half k-tile at the end
    (128, 128, 512, 8, 64, "bf16", "bf16"),
    (200, 160, 384, 8, 32, "f16", "f16"),
    (64, 129, 1024, 4, 64, "f16", "bf16"),
    (1, 100, 256, 4, 64, "bf16", "bf16"),
    (33, 64, 768, 8, 128, "bf16", "f16"),
    # few output tiles: k split in 2 (17 k-tiles: 9 + 8) and in 4 (65 k-tiles: 17 + 17 + 17 + 14)
    (70, 300, 1088, 4, 64, "bf16", "bf16"),
    (100, 100, 4160, 4, 64, "f16", "f16"),
    (90, 120, 2048, 8, 32, "bf16", "bf16"),
    # at least two output tiles per compute unit: two workgroups per CU, two LDS stages
    (4100, 4000, 256, 4, 64, "bf16", "bf16"),
    (4097, 4096, 192, 4, 32, "bf16", "f16"),
    # two tiles per compute unit only with 128-row tiles (ragged m, odd k-tile count)
    (2100, 4000, 320, 4, 64, "bf16", "bf16"),
    (2000, 4100, 192, 4, 32, "f16", "bf16"),
    (2050, 4096, 256, 8, 64, "bf16", "bf16"),
]


@pytest.mark.parametrize("m,n,k,bits,g,xdt,pdt", GEMM_CASES)
def test_gemm_parity(m, n, k, bits, g, xdt, pdt):
    (pk, sc, bi), D = _affine_case(3000 + m + n, n, k, bits, g, pdt)
    x, xf = _x_case(4000 + m + k, m, k, xdt)
    y = q.qlinear_gemm(x, pk, sc, bi, bits=bits, group_size=g, y_dtype=torch.float32)
    _sync()
    # the GEMM rounds each dequantized weight once to fp16 (2^-12 relative) before the fp32
    # accumulation: ~1.5e-4 per row, inside GEMM_TOL
    _assert_rel(y, O.apply(xf, D), GEMM_TOL, "gemm")


@pytest.mark.parametrize("std", [1e-7, 2e4])
def test_gemm_weight_magnitudes(std):
    """Rows far below and far above the fp16 range: the per-row power-of-two factor keeps each
    dequantized weight an fp16 normal, so the error stays that of one fp16 rounding."""
    m, n, k = 200, 300, 1024
    (pk, sc, bi), D = _affine_case(71, n, k, 4, 64, "bf16", std=std)
    x, xf = _x_case(72, m, k, "bf16")
    y = q.qlinear_gemm(x, pk, sc, bi, bits=4, group_size=64, y_dtype=torch.float32)
    _sync()
    _assert_rel(y, O.apply(xf, D), GEMM_TOL, "gemm magnitudes")


def test_gemm_one_hot_and_bias_and_bf16_out():
    n, k = 256, 1024
    (pk, sc, bi), D = _affine_case(51, n, k, 4, 64, "bf16")
    js = list(range(0, k, 7))[:130]
    xb = np.zeros((len(js), k), np.float32)
    for i, j in enumerate(js):
        xb[i, j] = 1.0
    x = bits_to_dev(O.to_bits("bf16", xb), "bf16")
    y = q.qlinear_gemm(x, pk, sc, bi, bits=4, group_size=64, y_dtype=torch.float32)
    _sync()
    # one-hot rows give the dequantized weights, each rounded once to fp16: within half an ulp
    np.testing.assert_allclose(y.cpu().numpy(), D[:, js].T, rtol=2.0 ** -11, atol=3e-8)
    xr, xf = _x_case(52, 150, k, "bf16")
    lb_bits = synth.acts_bits(53, 1, n, "bf16")[0]
    yb = q.qlinear_gemm(xr, pk, sc, bi, bits=4, group_size=64, layer_bias=bits_to_dev(lb_bits, "bf16"))
    _sync()
    ref = O.apply(xf, D, layer_bias=O.bits_to_f64("bf16", lb_bits))
    want = O.bits_to_f64("bf16", O.to_bits("bf16", ref.astype(np.float32)))
    _assert_rel(yb, want, TOL, "gemm bf16-out vs RNE_bf16(oracle)")


@pytest.mark.parametrize("name,k,n", synth.PREFILL_9B_LAYER)
def test_gemm_prefill_9b_full_size_sampled(name, k, n):
    """M=2048 prefill at the 9B layer shapes (4-bit g64, bf16 scales); the GPU quantizes W as the
    bench does, 48 sampled W rows are re-quantized by the oracle (bit-exact) and 48 sampled x
    rows x those W rows are checked against the oracle product; then 16 sampled x rows in whole
    (every output of the row) against the oracle's product with all of W."""
    m = 2048
    proj = [p[0] for p in synth.PREFILL_9B_LAYER].index(name)
    w = synth.weights_f32(synth.seed_for(4, 0, proj), n, k)
    xb = synth.acts_bits(synth.seed_for(4, 0, proj, 1), m, k, "bf16")
    pk, sc, bi = q.qlinear_quantize(torch.from_numpy(w).to(DEV), 4, 64, torch.bfloat16)
    y = q.qlinear_gemm(bits_to_dev(xb, "bf16"), pk, sc, bi, bits=4, group_size=64, y_dtype=torch.float32)
    _sync()
    g = np.random.default_rng(proj)
    rows = np.sort(g.choice(m, 48, replace=False))
    cols = np.sort(g.choice(n, 48, replace=False))
    cols[-1] = n - 1
    rows[-1] = m - 1
    opk, osb, obb = O.affine_quantize(w[cols], 4, 64, "bf16")
    np.testing.assert_array_equal(dev_to_u32(pk[cols]), opk)
    D = O.affine_dequant_f32(opk, osb, obb, 4, 64, "bf16", k)
    ref = O.apply(O.bits_to_f64("bf16", xb[rows]), D)
    got = y.cpu().numpy()[np.ix_(rows, cols)].astype(np.float64)
    err = O.rel_l2_per_row(got, ref)
    print(f"{name}: max rel-l2 over sampled rows {err.max():.3e}")
    assert err.max() <= GEMM_TOL
    xr = np.sort(g.choice(m, 16, replace=False))
    Df = np.empty((n, k), np.float32)
    for r0 in range(0, n, 4096):
        opk, osb, obb = O.affine_quantize(w[r0:r0 + 4096], 4, 64, "bf16")
        Df[r0:r0 + 4096] = O.affine_dequant_f32(opk, osb, obb, 4, 64, "bf16", k)
    refw = O.apply(O.bits_to_f64("bf16", xb[xr]), Df)
    errw = O.rel_l2_per_row(y.cpu().numpy()[xr].astype(np.float64), refw)
    print(f"{name}: whole rows max rel-l2 {errw.max():.3e}")
    assert errw.max() <= GEMM_TOL
    # a second call (its split-over-k partial sums are added in a fixed order) gives the same bits
    y2 = q.qlinear_gemm(bits_to_dev(xb, "bf16"), pk, sc, bi, bits=4, group_size=64, y_dtype=torch.float32)
    _sync()
    assert torch.equal(y, y2)


# ============================================================ batched GEMV


def _decode_problems(bits, m, shapes, seed_base, param_dtype="bf16", check_rows=8):
    """GPU-quantized weights (as the bench builds them) + oracle checks on sampled rows."""
    probs, checks = [], []
    for i, (name, k, n) in enumerate(shapes):
        w = synth.weights_f32(seed_base + 10 * i, n, k)
        pk, sc, bi = q.qlinear_quantize(torch.from_numpy(w).to(DEV), bits, 64, TDT[param_dtype])
        xb = synth.acts_bits(seed_base + 10 * i + 1, m, k, "bf16")
        x = bits_to_dev(xb, "bf16")
        y = torch.empty((m, n), dtype=torch.float32, device=DEV)
        probs.append(dict(x=x, packed=pk, scales=sc, biases=bi, y=y, bits=bits, group_size=64))
        rows = np.unique(np.concatenate([np.random.default_rng(i).choice(n, check_rows - 1), [n - 1]]))
        checks.append((w[rows], rows, xb, k, pk, y))
    return probs, checks


def _verify_decode(checks, bits, label):
    worst = 0.0
    for (wrows, rows, xb, k, pk, y) in checks:
        opk, osb, obb = O.affine_quantize(wrows, bits, 64, "bf16")
        np.testing.assert_array_equal(dev_to_u32(pk[rows]), opk)
        D = O.affine_dequant_f32(opk, osb, obb, bits, 64, "bf16", k)
        ref = O.apply(O.bits_to_f64("bf16", xb), D)
        err = O.rel_l2_per_row(y.cpu().numpy()[:, rows].astype(np.float64), ref)
        worst = max(worst, float(err.max()))
    print(f"{label}: max rel-l2 {worst:.3e}")
    assert worst <= 1e-4


def test_gemv_batched_mixed_bits_small_list():
    shapes = synth.QWEN3_0_6B_LAYER[:4]
    probs4, checks4 = _decode_problems(4, 1, shapes, 70000)
    probs8, checks8 = _decode_problems(8, 1, shapes[:2], 71000)
    probs = probs4 + probs8
    ws = torch.empty(q.qlinear_gemv_batched_workspace_size(probs), dtype=torch.uint8, device=DEV)
    q.qlinear_gemv_batched(probs, x_dtype=torch.bfloat16, param_dtype=torch.bfloat16, y_dtype=torch.float32,
                           workspace=ws)
    _sync()
    _verify_decode(checks4, 4, "batched 4-bit")
    _verify_decode(checks8, 8, "batched 8-bit")


@pytest.mark.parametrize("bits,m", [(4, 1), (4, 8), (8, 1), (8, 8), (2, 1), (3, 1), (5, 1), (6, 1), (2, 8), (6, 8)])
def test_gemv_batched_qwen3_0_6b_full_list(bits, m):
    """All 197 projections of the Qwen3-0.6B-shaped decode step in one problem-list launch (the
    bench's configuration), sampled rows of every projection against the oracle; a second launch
    reusing the uploaded table gives identical bits."""
    probs, checks = _decode_problems(bits, m, synth.QWEN3_0_6B_DECODE, synth.seed_for(2 if bits == 4 else 3),
                                     check_rows=4)
    ws = torch.empty(q.qlinear_gemv_batched_workspace_size(probs), dtype=torch.uint8, device=DEV)
    kw = dict(x_dtype=torch.bfloat16, param_dtype=torch.bfloat16, y_dtype=torch.float32, workspace=ws)
    q.qlinear_gemv_batched(probs, upload=True, **kw)
    _sync()
    first = [p["y"].clone() for p in probs]
    q.qlinear_gemv_batched(probs, upload=False, **kw)
    _sync()
    assert all(torch.equal(a, p["y"]) for a, p in zip(first, probs))
    _verify_decode(checks, bits, f"qwen3-0.6b decode {bits}-bit m={m}")


@pytest.mark.parametrize("bits,m", [(4, 1), (8, 8)])
def test_gemv_batched_whole_rows_layer0_and_lm_head(bits, m):
    """Whole output rows (the benchmark spec's per-row l2 bound) of one full layer set and the
    lm_head: the layer-0 projections and the 151936-row lm_head of the decode step, seeded as in
    the full list, in one problem-list launch; the oracle quantizes every row itself."""
    shapes = synth.QWEN3_0_6B_DECODE[:7] + synth.QWEN3_0_6B_DECODE[-1:]
    seed_base = synth.seed_for(2 if bits == 4 else 3)
    idx = list(range(7)) + [len(synth.QWEN3_0_6B_DECODE) - 1]
    probs, ws_rows = [], []
    for i, (name, k, n) in zip(idx, shapes):
        w = synth.weights_f32(seed_base + 10 * i, n, k)
        pk, sc, bi = q.qlinear_quantize(torch.from_numpy(w).to(DEV), bits, 64, torch.bfloat16)
        xb = synth.acts_bits(seed_base + 10 * i + 1, m, k, "bf16")
        y = torch.empty((m, n), dtype=torch.float32, device=DEV)
        probs.append(dict(x=bits_to_dev(xb, "bf16"), packed=pk, scales=sc, biases=bi, y=y, bits=bits, group_size=64))
        ws_rows.append((name, w, xb, k))
        del w
    ws = torch.empty(q.qlinear_gemv_batched_workspace_size(probs), dtype=torch.uint8, device=DEV)
    q.qlinear_gemv_batched(probs, x_dtype=torch.bfloat16, param_dtype=torch.bfloat16, y_dtype=torch.float32,
                           workspace=ws)
    _sync()
    worst = 0.0
    for (name, w, xb, k), p in zip(ws_rows, probs):
        ref = np.zeros((m, w.shape[0]))
        for r0 in range(0, w.shape[0], 32768):  # the oracle in slices of rows (memory)
            opk, osb, obb = O.affine_quantize(w[r0:r0 + 32768], bits, 64, "bf16")
            D = O.affine_dequant_f32(opk, osb, obb, bits, 64, "bf16", k)
            ref[:, r0:r0 + 32768] = O.apply(O.bits_to_f64("bf16", xb), D)
        err = O.rel_l2_per_row(p["y"].cpu().numpy().astype(np.float64), ref)
        print(f"{name} {bits}-bit m={m}: whole rows max rel-l2 {err.max():.3e}")
        worst = max(worst, float(err.max()))
    assert worst <= 1e-4


def test_gemv_batched_upload_is_asynchronous_and_capturable():
    """upload=True enqueues the table copy on the stream without waiting: the whole call, upload
    included, captured into a graph and replayed into a fresh workspace, gives the eager bits."""
    shapes = synth.QWEN3_0_6B_LAYER[:3]
    probs, _ = _decode_problems(4, 1, shapes, 72500)
    arr = q.qlinear_problem_list(probs)
    nbytes = q.qlinear_gemv_batched_workspace_size(arr)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    kw = dict(x_dtype=torch.bfloat16, param_dtype=torch.bfloat16, y_dtype=torch.float32)
    q.qlinear_gemv_batched(arr, upload=True, workspace=ws, **kw)
    _sync()
    eager = [p["y"].clone() for p in probs]
    ws2 = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    _sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.qlinear_gemv_batched(arr, upload=True, workspace=ws2, **kw)
    for rep in range(3):
        ws2.zero_()
        for p in probs:
            p["y"].fill_(rep + 7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ws2, ws), f"replay {rep}: table"
        assert all(torch.equal(a, p["y"]) for a, p in zip(eager, probs)), f"replay {rep}"


def test_gemv_batched_graph_replay_matches_eager():
    """The decode step captured in a HIP graph and replayed 5 times (eager work in between)
    gives the eager result bit for bit every time."""
    shapes = synth.QWEN3_0_6B_LAYER + [("head", 1024, 8192)]
    probs, _ = _decode_problems(4, 1, shapes, 72000)
    for p in probs:
        p["y"] = torch.empty(p["y"].shape, dtype=torch.bfloat16, device=DEV)
    arr = q.qlinear_problem_list(probs)
    ws = torch.empty(q.qlinear_gemv_batched_workspace_size(arr), dtype=torch.uint8, device=DEV)
    kw = dict(x_dtype=torch.bfloat16, param_dtype=torch.bfloat16, y_dtype=torch.bfloat16, workspace=ws)
    q.qlinear_gemv_batched(arr, upload=True, **kw)
    _sync()
    eager = [p["y"].clone() for p in probs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.qlinear_gemv_batched(arr, upload=False, **kw)
    for rep in range(5):
        for p in probs:
            p["y"].fill_(rep + 1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, p["y"]) for a, p in zip(eager, probs)), f"replay {rep}"


# ============================================================ routing and routed experts


@pytest.mark.parametrize("n_pos,e,lo,hi", [(2048, 32, 0, 32), (1000, 7, -3, 9), (5, 3, 0, 3), (0, 4, 0, 4),
                                           (20000, 300, -1, 300)])
def test_route_bitexact(n_pos, e, lo, hi):
    ids = np.random.default_rng(n_pos + e).integers(lo, hi, size=max(n_pos, 0)).astype(np.int64)
    off, perm = q.qlinear_route(torch.from_numpy(ids).to(DEV), e)
    _sync()
    o_off, o_perm = O.route(ids, e)
    np.testing.assert_array_equal(off.cpu().numpy(), o_off)
    np.testing.assert_array_equal(perm.cpu().numpy()[: o_off[-1]], o_perm)


def test_route_topk_ids_of_the_expert_workload():
    cfg = synth.EXPERTS_32x5760x2880
    ids = synth.topk_ids(synth.seed_for(5, part=2), cfg["tokens"], cfg["top"], cfg["e"]).reshape(-1)
    off, perm = q.qlinear_route(torch.from_numpy(ids).to(DEV), cfg["e"])
    _sync()
    o_off, o_perm = O.route(ids, cfg["e"])
    np.testing.assert_array_equal(off.cpu().numpy(), o_off)
    np.testing.assert_array_equal(perm.cpu().numpy(), o_perm)


def _experts_tol(fmt):
    # MXFP4 values are exact in bf16, so that product is fp32 accumulation only; Q8_0 weights are
    # rounded once to fp16 (d*q, 2^-12 relative), ~2e-4 per row, inside the 2e-3 bound on products
    return 1e-4 if fmt == q.QL_MXFP4 else Q8_TOL


def _experts_small(fmt, seed):
    e, n, k, tokens, top = 5, 200, 256, 37, 3
    if fmt == q.QL_MXFP4:
        codes, scales = synth.mxfp4_codes_scales(seed, e, n, k)
        W = O.mxfp4_dequant_f32(codes, scales)
        parts = (u8_to_dev(codes), u8_to_dev(scales))
    else:
        blocks = O.q8_0_quantize(synth.weights_f32(seed, e * n, k).reshape(e, n, k))
        W = O.q8_0_dequant_f32(blocks)
        parts = (u8_to_dev(blocks), None)
    ids = np.random.default_rng(seed).integers(-1, e + 1, size=(tokens, top)).astype(np.int64)
    ids[0] = [2, 2, 2]  # duplicate ids in one token
    xb = synth.acts_bits(seed + 1, tokens, k, "bf16")
    return parts, W, ids, xb, n, k, top


@pytest.mark.parametrize("fmt", [q.QL_MXFP4, q.QL_Q8_0])
@pytest.mark.parametrize("ydt", ["f32", "bf16", "f16"])
def test_apply_experts_small(fmt, ydt):
    (w0, w1), W, ids, xb, n, k, top = _experts_small(fmt, 61 + fmt)
    y = q.qlinear_apply_experts(fmt, w0, w1, torch.from_numpy(ids.reshape(-1)).to(DEV), bits_to_dev(xb, "bf16"), n=n,
                                k=k, pos_per_row=top, y_dtype=TDT[ydt])
    _sync()
    ref = O.apply_experts(W, ids.reshape(-1), O.bits_to_f64("bf16", xb), pos_per_row=top)
    out = out_f64(y)
    dead = ~((ids.reshape(-1) >= 0) & (ids.reshape(-1) < W.shape[0]))
    assert np.all(out[dead] == 0.0)
    if ydt == "f32":
        _assert_rel(y[torch.from_numpy(~dead).to(DEV)], ref[~dead], _experts_tol(fmt), "experts")
    else:
        want = O.bits_to_f64(ydt, O.to_bits(ydt, ref.astype(np.float32)))
        err = O.rel_l2_per_row(out[~dead], want[~dead])
        print(f"experts 16-bit out vs rounded oracle {err.max():.3e}")
        assert err.max() <= TOL


@pytest.mark.parametrize("fmt", [q.QL_MXFP4, q.QL_Q8_0])
def test_apply_experts_graph_replay_matches_eager(fmt):
    """Routed apply (routing and products launches) captured in a HIP graph and replayed 4 times,
    with eager work in between: every replay gives the eager bits."""
    (w0, w1), _, ids, xb, n, k, top = _experts_small(fmt, 81 + fmt)
    idt = torch.from_numpy(ids.reshape(-1)).to(DEV)
    x = bits_to_dev(xb, "bf16")
    y = torch.empty((ids.size, n), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(q.qlinear_apply_experts_workspace_size(ids.size, w0.shape[0]), dtype=torch.uint8, device=DEV)
    kw = dict(n=n, k=k, pos_per_row=top, y=y, workspace=ws)
    q.qlinear_apply_experts(fmt, w0, w1, idt, x, **kw)
    _sync()
    eager = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.qlinear_apply_experts(fmt, w0, w1, idt, x, **kw)
    for rep in range(4):
        y.fill_(rep + 1)
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {rep}"


@pytest.mark.parametrize("fmt", [q.QL_MXFP4, q.QL_Q8_0])
def test_apply_experts_f16_x(fmt):
    """fp16 activations (Nx_quant Products, apply_experts: any float x): MXFP4 takes them as the
    exact sum of two bf16 parts, Q8_0 as they are; the same bounds as bf16 x."""
    (w0, w1), W, ids, _, n, k, top = _experts_small(fmt, 71 + fmt)
    xh = synth.acts_bits(72 + fmt, ids.shape[0], k, "f16")
    xh[0, :8] = O.to_bits("f16", np.float32([1e-7, -3e-6, 6.0e4, -5.5e4, 1.0009765625, 2.0**-14, 0.0, -0.0]))
    y = q.qlinear_apply_experts(fmt, w0, w1, torch.from_numpy(ids.reshape(-1)).to(DEV), bits_to_dev(xh, "f16"), n=n,
                                k=k, pos_per_row=top, y_dtype=torch.float32)
    _sync()
    ref = O.apply_experts(W, ids.reshape(-1), O.bits_to_f64("f16", xh), pos_per_row=top)
    flat = ids.reshape(-1)
    live = (flat >= 0) & (flat < W.shape[0])
    assert np.all(out_f64(y)[~live] == 0.0)
    _assert_rel(y[torch.from_numpy(live).to(DEV)], ref[live], _experts_tol(fmt), "experts f16 x")


@pytest.mark.parametrize("fmt", [q.QL_MXFP4, q.QL_Q8_0])
@pytest.mark.parametrize("e,n,k,tokens,top,skew", [
    (3, 300, 288, 100, 2, True),    # one expert with ~150 positions (two chunks), k % 64 == 32
    (300, 64, 64, 50, 4, False),    # most experts empty; the expert order spans two workgroups
    (4, 520, 1024, 70, 4, False),   # weight-row tiles of 384 and 136 rows
    (2, 100, 4160, 20, 2, False),   # k too long for staging the scale bytes in LDS
])
def test_apply_experts_chunks_and_shapes(fmt, e, n, k, tokens, top, skew):
    seed = 700 + e + n
    if fmt == q.QL_MXFP4:
        codes, scales = synth.mxfp4_codes_scales(seed, e, n, k)
        W = O.mxfp4_dequant_f32(codes, scales)
        w0, w1 = u8_to_dev(codes), u8_to_dev(scales)
    else:
        blocks = O.q8_0_quantize(synth.weights_f32(seed, e * n, k).reshape(e, n, k))
        W = O.q8_0_dequant_f32(blocks)
        w0, w1 = u8_to_dev(blocks), None
    g = np.random.default_rng(seed)
    ids = g.integers(0, e, size=(tokens, top)).astype(np.int64)
    if skew:
        ids[:, 0] = 0
        ids[: tokens // 2, 1] = 0
    xb = synth.acts_bits(seed + 1, tokens, k, "bf16")
    y = q.qlinear_apply_experts(fmt, w0, w1, torch.from_numpy(ids.reshape(-1)).to(DEV), bits_to_dev(xb, "bf16"), n=n,
                                k=k, pos_per_row=top, y_dtype=torch.float32)
    _sync()
    ref = O.apply_experts(W, ids.reshape(-1), O.bits_to_f64("bf16", xb), pos_per_row=top)
    _assert_rel(y, ref, _experts_tol(fmt), "experts shapes")


def test_apply_experts_q8_0_scales_beyond_f16_products():
    """Q8_0 blocks whose scale d exceeds 511.75 (d*q can leave the fp16 range) and subnormal
    scales: the workgroups that meet a large scale recompute their outputs in fp32."""
    e, n, k, tokens, top = 3, 300, 512, 40, 2
    blocks = O.q8_0_quantize(synth.weights_f32(801, e * n, k).reshape(e, n, k))
    b4 = blocks.reshape(e, n, k // 32, 34)
    d = np.ascontiguousarray(b4[..., :2]).view(np.uint16)[..., 0]  # [e, n, k/32] fp16 bits of d
    d[1, 7, 3] = O.to_bits("f16", np.float32([1000.0]))[0]
    d[1, 290, 0] = O.to_bits("f16", np.float32([-3.0e4]))[0]
    d[2, 5, :] = O.to_bits("f16", np.float32([2.0**-20]))[0]  # fp16 subnormal scales
    b4[..., :2] = d[..., None].view(np.uint8)
    blocks = b4.reshape(e, n, k // 32 * 34)
    W = O.q8_0_dequant_f32(blocks)
    ids = np.random.default_rng(802).integers(0, e, size=(tokens, top)).astype(np.int64)
    xb = synth.acts_bits(803, tokens, k, "bf16")
    y = q.qlinear_apply_experts(q.QL_Q8_0, u8_to_dev(blocks), None, torch.from_numpy(ids.reshape(-1)).to(DEV),
                                bits_to_dev(xb, "bf16"), n=n, k=k, pos_per_row=top, y_dtype=torch.float32)
    _sync()
    ref = O.apply_experts(W, ids.reshape(-1), O.bits_to_f64("bf16", xb), pos_per_row=top)
    _assert_rel(y, ref, Q8_TOL, "q8_0 large scales")


@pytest.mark.parametrize("fmt", [q.QL_MXFP4, q.QL_Q8_0])
def test_apply_experts_full_size_sampled_and_row_independent(fmt):
    """32 experts of 5760x2880, 512 tokens x top-4 (the routed-experts workload): 64 sampled
    positions x 96 sampled output rows, and 16 positions' whole rows, against the oracle; a
    position's row keeps its bits when the other tokens' ids change; two runs are bitwise equal."""
    cfg = synth.EXPERTS_32x5760x2880
    e, n, k, tokens, top = cfg["e"], cfg["n"], cfg["k"], cfg["tokens"], cfg["top"]
    if fmt == q.QL_MXFP4:
        codes, scales = synth.mxfp4_codes_scales(synth.seed_for(5), e, n, k)
        w0, w1 = u8_to_dev(codes), u8_to_dev(scales)
    else:
        blocks = synth.q8_0_random_blocks(synth.seed_for(5, part=3), e, n, k)
        w0, w1 = u8_to_dev(blocks), None
    ids = synth.topk_ids(synth.seed_for(5, part=2), tokens, top, e).reshape(-1)
    xb = synth.acts_bits(synth.seed_for(5, part=1), tokens, k, "bf16")
    x = bits_to_dev(xb, "bf16")
    ids_d = torch.from_numpy(ids).to(DEV)
    y = q.qlinear_apply_experts(fmt, w0, w1, ids_d, x, n=n, k=k, pos_per_row=top, y_dtype=torch.float32)
    y2 = q.qlinear_apply_experts(fmt, w0, w1, ids_d, x, n=n, k=k, pos_per_row=top, y_dtype=torch.float32)
    _sync()
    assert torch.equal(y, y2)
    g = np.random.default_rng(9)
    pos = np.sort(g.choice(ids.size, 64, replace=False))
    cols = np.sort(g.choice(n, 96, replace=False))
    cols[-1] = n - 1
    worst = 0.0
    for p in pos:
        ex = ids[p]
        if fmt == q.QL_MXFP4:
            Wc = O.mxfp4_dequant_f32(codes[ex, cols], scales[ex, cols])
        else:
            Wc = O.q8_0_dequant_f32(blocks[ex, cols])
        ref = O.apply(O.bits_to_f64("bf16", xb[p // top])[None, :], Wc)[0]
        got = y[p, torch.from_numpy(cols).to(DEV)].cpu().numpy().astype(np.float64)
        worst = max(worst, float(np.linalg.norm(got - ref) / np.linalg.norm(ref)))
    print(f"experts fmt={fmt}: max rel-l2 over sampled rows {worst:.3e}")
    assert worst <= _experts_tol(fmt)
    # whole 5760-wide rows of 16 sampled positions (each expert decoded once by the oracle)
    wpos = np.sort(g.choice(ids.size, 16, replace=False))
    worst = 0.0
    for ex in np.unique(ids[wpos]):
        We = O.mxfp4_dequant_f32(codes[ex], scales[ex]) if fmt == q.QL_MXFP4 else O.q8_0_dequant_f32(blocks[ex])
        ps = wpos[ids[wpos] == ex]
        ref = O.apply(O.bits_to_f64("bf16", xb[ps // top]), We)
        got = y[torch.from_numpy(ps).to(DEV)].cpu().numpy().astype(np.float64)
        worst = max(worst, float(O.rel_l2_per_row(got, ref).max()))
    print(f"experts fmt={fmt}: max rel-l2 over whole rows {worst:.3e}")
    assert worst <= _experts_tol(fmt)
    # row independence: reroute every other token; untouched tokens keep their rows' bits
    ids_b = ids.reshape(tokens, top).copy()
    ids_b[1::2] = (ids_b[1::2] + 5) % e
    yb = q.qlinear_apply_experts(fmt, w0, w1, torch.from_numpy(ids_b.reshape(-1)).to(DEV), x, n=n, k=k,
                                 pos_per_row=top, y_dtype=torch.float32)
    _sync()
    keep = torch.from_numpy(np.repeat(np.arange(tokens) % 2 == 0, top)).to(DEV)
    assert torch.equal(yb[keep], y[keep])
