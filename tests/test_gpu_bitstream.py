"""GPU parity at the bitstream widths: affine rows of 2, 3, 5 and 6 bits (GPTQModel wiki "MLX
Apple Silicon", Packed layouts and exact transcoding: 2-bit codes whole in each word, 3/5/6-bit
codes crossing words in one little-endian stream per row).  Same bars as the 4/8-bit tests:
packed words, scales, biases and dequantized values bit-exact; products <= 2e-3 relative l2 per
row (fp32 output vs the fp64 oracle), one-hot x bit-exact for the GEMV.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_quantized_affine_amd as q
from gpu_helpers import DEV, TDT, bits_to_dev, dev_to_bits, dev_to_u32, out_bits_or_f32, out_f64, same_values, u32_to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3
STREAM_BITS = [2, 3, 5, 6]


def _sync():
    torch.cuda.synchronize()


def _affine_case(seed, n, k, bits, g, pdt, std=0.02):
    w = synth.weights_f32(seed, n, k, std=std)
    opk, osb, obb = O.affine_quantize(w, bits, g, pdt)
    D = O.affine_dequant_f32(opk, osb, obb, bits, g, pdt, k)
    return (u32_to_dev(opk), bits_to_dev(osb, pdt), bits_to_dev(obb, pdt)), D


def _x_case(seed, m, k, xdt):
    xb = synth.acts_bits(seed, m, k, xdt)
    return bits_to_dev(xb, xdt), O.bits_to_f64(xdt, xb)


def _assert_rel(y_dev, ref, tol, label):
    err = O.rel_l2_per_row(out_f64(y_dev), ref)
    print(f"{label} max rel-l2 {err.max():.3e}")
    assert err.max() <= tol, f"{label}: max rel-l2 {err.max():.3e}"


# ------------------------------------------------------------------ quantize / dequant


@pytest.mark.parametrize("bits", STREAM_BITS)
@pytest.mark.parametrize("g,pdt", [(32, "bf16"), (64, "f16"), (128, "bf16")])
def test_quantize_bitstream_bitexact_ragged_and_edge_groups(bits, g, pdt):
    n, k = 37, 384
    w = synth.weights_f32(500 + bits * 10 + g, n, k)
    w[1] *= 1000.0
    w[2] *= 1e-4
    w[3, :g] = 0.25  # constant group
    w[4, :g] = 0.0
    w[4, 5] = -0.0
    w[6, :g] = np.linspace(-1, 1, g, dtype=np.float32)  # exact ties possible
    packed, scales, biases = q.qlinear_quantize(torch.from_numpy(w).to(DEV), bits, g, TDT[pdt])
    _sync()
    opk, osb, obb = O.affine_quantize(w, bits, g, pdt)
    assert packed.shape == (n, k * bits // 32)
    np.testing.assert_array_equal(dev_to_u32(packed), opk)
    np.testing.assert_array_equal(dev_to_bits(scales), osb)
    np.testing.assert_array_equal(dev_to_bits(biases), obb)


@pytest.mark.parametrize("bits", [3, 6])
def test_quantize_bitstream_many_rows(bits):
    """1000 x 2048 (several waves and workgroups, every lane position of a chunk)."""
    w = synth.weights_f32(600 + bits, 1000, 2048)
    packed, scales, biases = q.qlinear_quantize(torch.from_numpy(w).to(DEV), bits, 64, torch.bfloat16)
    _sync()
    opk, osb, obb = O.affine_quantize(w, bits, 64, "bf16")
    np.testing.assert_array_equal(dev_to_u32(packed), opk)
    np.testing.assert_array_equal(dev_to_bits(scales), osb)
    np.testing.assert_array_equal(dev_to_bits(biases), obb)


@pytest.mark.parametrize("bits", STREAM_BITS)
@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
def test_dequant_bitstream_bitexact(bits, odt):
    n, k, g, pdt = 45, 512, 64, "bf16" if bits % 2 else "f16"
    w = synth.weights_f32(700 + bits, n, k, std=0.5)
    opk, osb, obb = O.affine_quantize(w, bits, g, pdt)
    out = q.qlinear_dequant(q.QL_AFFINE, u32_to_dev(opk), bits_to_dev(osb, pdt), bits_to_dev(obb, pdt), rows=n, k=k,
                            bits=bits, group_size=g, out_dtype=TDT[odt])
    _sync()
    assert same_values(out_bits_or_f32(out, odt), O.affine_dequant_to(odt, opk, osb, obb, bits, g, pdt, k))


# ------------------------------------------------------------------ GEMV


@pytest.mark.parametrize("bits", STREAM_BITS)
def test_gemv_bitstream_one_hot_gives_exact_columns(bits):
    n, k = 70, 3072
    (pk, sc, bi), D = _affine_case(800 + bits, n, k, bits, 64, "bf16")
    js = [0, 1, 31, 32, 777, k - 1]
    xb = np.zeros((len(js), k), np.float32)
    for i, j in enumerate(js):
        xb[i, j] = 1.0
    x = bits_to_dev(O.to_bits("bf16", xb), "bf16")
    y = q.qlinear_gemv(x, pk, sc, bi, bits=bits, group_size=64, y_dtype=torch.float32)
    _sync()
    np.testing.assert_array_equal(y.cpu().numpy(), D[:, js].T)


GEMV_STREAM_CASES = [
    # m, n, k, bits, g, xdt, pdt, ydt
    (1, 2048, 1024, 2, 64, "bf16", "bf16", "f32"),
    (1, 1024, 3072, 3, 64, "bf16", "bf16", "f32"),
    (1, 333, 160, 5, 32, "f16", "bf16", "f32"),
    (1, 8192, 1024, 6, 64, "bf16", "bf16", "bf16"),  # enough rows for 2 rows per wave
    (1, 5000, 2048, 2, 128, "bf16", "f16", "f32"),
    (2, 517, 2048, 6, 128, "bf16", "f16", "f32"),
    (3, 300, 1024, 2, 32, "f16", "f16", "f16"),
    (4, 129, 384, 5, 64, "bf16", "bf16", "f32"),
    (5, 64, 3072, 3, 32, "bf16", "bf16", "f32"),
    (8, 250, 8192, 6, 64, "bf16", "bf16", "f32"),  # x through LDS in 3 slices
    (8, 1024, 1024, 3, 64, "f16", "bf16", "f32"),
    (11, 90, 512, 5, 64, "bf16", "bf16", "f32"),  # 8 + 3 rows of x
    (1, 40, 33792, 2, 64, "bf16", "bf16", "f32"),  # one x row through LDS in 2 slices
    (8, 777, 2048, 2, 128, "f16", "bf16", "bf16"),  # 2 bits on the matrix cores: 8 x rows, ragged n
    (2, 1000, 1152, 2, 64, "bf16", "f16", "f32"),  # an odd count of 128-code blocks per row
    (2, 333, 1152, 3, 128, "bf16", "f16", "bf16"),  # 3 bits on the matrix cores, ragged n, odd blocks
    (4, 500, 2048, 3, 32, "f16", "bf16", "f32"),  # 3 bits, 4 x rows x 4 groups per block
    (4, 300, 1152, 6, 32, "f16", "bf16", "f32"),  # 6 bits on the matrix cores, odd blocks
    (8, 129, 1024, 6, 64, "bf16", "f16", "bf16"),  # 6 bits, 8 x rows, 16-bit output
    (8, 600, 2048, 5, 128, "f16", "f16", "f16"),  # 5 bits on the matrix cores, 8 x rows
    (1, 4096, 1152, 5, 64, "bf16", "bf16", "f32"),  # 5 bits, odd blocks
]


@pytest.mark.parametrize("m,n,k,bits,g,xdt,pdt,ydt", GEMV_STREAM_CASES)
def test_gemv_bitstream_parity(m, n, k, bits, g, xdt, pdt, ydt):
    (pk, sc, bi), D = _affine_case(900 + m * 7 + n + bits, n, k, bits, g, pdt)
    x, xf = _x_case(1900 + m + k + bits, m, k, xdt)
    y = q.qlinear_gemv(x, pk, sc, bi, bits=bits, group_size=g, y_dtype=TDT[ydt])
    _sync()
    ref = O.apply(xf, D)
    if ydt == "f32":
        _assert_rel(y, ref, 1e-4, "gemv bitstream")
    else:
        want = O.bits_to_f64(ydt, O.to_bits(ydt, ref.astype(np.float32)))
        _assert_rel(y, want, TOL, "gemv bitstream 16-bit out vs rounded oracle")


def test_gemv_bitstream_layer_bias_empty_k_and_determinism():
    (pk, sc, bi), D = _affine_case(31, 200, 1024, 3, 64, "bf16")
    x, xf = _x_case(32, 3, 1024, "bf16")
    lb_bits = synth.acts_bits(33, 1, 200, "bf16")[0]
    lb = bits_to_dev(lb_bits, "bf16")
    y = q.qlinear_gemv(x, pk, sc, bi, bits=3, group_size=64, layer_bias=lb, y_dtype=torch.float32)
    y2 = q.qlinear_gemv(x, pk, sc, bi, bits=3, group_size=64, layer_bias=lb, y_dtype=torch.float32)
    _sync()
    _assert_rel(y, O.apply(xf, D, layer_bias=O.bits_to_f64("bf16", lb_bits)), 1e-4, "gemv bitstream+bias")
    assert torch.equal(y, y2)
    x0 = torch.empty((3, 0), dtype=torch.bfloat16, device=DEV)
    pk0 = torch.empty((200, 0), dtype=torch.int32, device=DEV)
    s0 = torch.empty((200, 0), dtype=torch.bfloat16, device=DEV)
    y0 = q.qlinear_gemv(x0, pk0, s0, s0, bits=5, group_size=64, layer_bias=lb, y_dtype=torch.float32)
    _sync()
    np.testing.assert_array_equal(y0.cpu().numpy(), np.tile(O.bf16_bits_to_f32(lb_bits), (3, 1)))


# ------------------------------------------------------------------ GEMM


GEMM_STREAM_CASES = [
    # m, n, k, bits, g, xdt, pdt
    (300, 333, 1024, 2, 64, "bf16", "bf16"),
    (257, 256, 2048, 3, 128, "bf16", "f16"),
    (130, 200, 224, 5, 32, "bf16", "bf16"),  # half a k-tile at the end
    (128, 128, 512, 6, 64, "f16", "bf16"),
    (70, 300, 1088, 3, 64, "bf16", "bf16"),  # k split over 2 ranges
    (2050, 4096, 256, 6, 64, "bf16", "bf16"),
]


@pytest.mark.parametrize("m,n,k,bits,g,xdt,pdt", GEMM_STREAM_CASES)
def test_gemm_bitstream_parity(m, n, k, bits, g, xdt, pdt):
    (pk, sc, bi), D = _affine_case(3100 + m + n + bits, n, k, bits, g, pdt)
    x, xf = _x_case(4100 + m + k + bits, m, k, xdt)
    y = q.qlinear_gemm(x, pk, sc, bi, bits=bits, group_size=g, y_dtype=torch.float32)
    _sync()
    # each dequantized weight is rounded once to fp16 before the fp32 accumulation, as at 4/8 bits
    _assert_rel(y, O.apply(xf, D), TOL, "gemm bitstream")


def test_gemm_bitstream_equals_its_8bit_transcode():
    """The bitstream GEMM reads the codes re-packed as bytes: the same codes given directly in the
    8-bit layout (oracle repack) give bit-identical output."""
    m, n, k, bits, g = 200, 300, 1024, 5, 64
    w = synth.weights_f32(77, n, k)
    opk, osb, obb = O.affine_quantize(w, bits, g, "bf16")
    codes = O.unpack_codes(opk, bits, k)
    pk8 = O.pack_codes(codes, 8)
    x, _ = _x_case(78, m, k, "bf16")
    sc, bi = bits_to_dev(osb, "bf16"), bits_to_dev(obb, "bf16")
    y5 = q.qlinear_gemm(x, u32_to_dev(opk), sc, bi, bits=5, group_size=g, y_dtype=torch.float32)
    y8 = q.qlinear_gemm(x, u32_to_dev(pk8), sc, bi, bits=8, group_size=g, y_dtype=torch.float32)
    _sync()
    assert torch.equal(y5, y8)


def test_gemv_bitstream_graph_replay_matches_eager():
    """Three bitstream GEMVs captured in one HIP graph: every replay (with eager work and the
    outputs cleared in between) equals the eager results bit for bit."""
    cases = []
    for bits, (n, k) in zip((2, 3, 6), ((300, 1024), (1000, 3072), (4096, 1024))):
        (pk, sc, bi), _ = _affine_case(1300 + bits, n, k, bits, 64, "bf16")
        x, _ = _x_case(1400 + bits, 1, k, "bf16")
        y = torch.empty((1, n), dtype=torch.float32, device=DEV)
        cases.append((bits, x, pk, sc, bi, y))
    eager = [q.qlinear_gemv(x, pk, sc, bi, bits=b, group_size=64, y_dtype=torch.float32).clone()
             for (b, x, pk, sc, bi, _) in cases]
    _sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (b, x, pk, sc, bi, y) in cases:
            q.qlinear_gemv(x, pk, sc, bi, bits=b, group_size=64, y=y)
    _sync()
    for rep in range(3):
        for c in cases:
            c[5].zero_()
        _ = q.qlinear_gemv(cases[0][1], cases[0][2], cases[0][3], cases[0][4], bits=2, group_size=64)  # eager work
        _sync()
        g.replay()
        _sync()
        for c, want in zip(cases, eager):
            assert torch.equal(c[5], want), f"replay {rep}, {c[0]} bits"


def test_gemv_batched_with_bitstream_widths():
    """One problem list mixing 2, 3, 4, 5, 6 and 8 bits, 1 to 8 rows of x and every group size:
    each y against the oracle (fp32 output).  Most problems take the matrix-core kernel; those it
    does not take (8 x rows of k = 8192, 6 x rows at g = 32) run as one bitstream class, and those
    whose k is not a multiple of 128 in launches of their own."""
    specs = [  # bits, m, n, k, g
        (2, 1, 300, 1024, 64), (3, 1, 1000, 3072, 64), (6, 1, 2048, 1024, 128), (5, 3, 129, 384, 32),
        (2, 8, 250, 2048, 64), (6, 2, 517, 2048, 64), (4, 1, 400, 1024, 64), (8, 1, 300, 1024, 64),
        (3, 8, 64, 8192, 64), (2, 1, 7, 128, 32), (2, 6, 100, 1024, 32),
        # k not a multiple of 128: launches of their own, as qlinear_gemv runs them
        (3, 1, 200, 1056, 32), (5, 4, 96, 320, 64), (6, 8, 77, 96, 32), (2, 2, 33, 160, 32)]
    probs, refs = [], []
    for i, (bits, m, n, k, g) in enumerate(specs):
        (pk, sc, bi), D = _affine_case(1500 + i, n, k, bits, g, "bf16")
        x, xf = _x_case(1600 + i, m, k, "bf16")
        y = torch.empty((m, n), dtype=torch.float32, device=DEV)
        probs.append(dict(x=x, packed=pk, scales=sc, biases=bi, y=y, bits=bits, group_size=g))
        refs.append(O.apply(xf, D))
    arr = q.qlinear_problem_list(probs)
    ws = torch.empty(q.qlinear_gemv_batched_workspace_size(arr), dtype=torch.uint8, device=DEV)
    q.qlinear_gemv_batched(arr, x_dtype=torch.bfloat16, param_dtype=torch.bfloat16, y_dtype=torch.float32,
                           workspace=ws, upload=True)
    _sync()
    for p, ref, spec in zip(probs, refs, specs):
        _assert_rel(p["y"], ref, 1e-4, f"batched {spec}")
