"""GPU parity of the GPTQ -> affine transcoder (GPTQModel wiki "MLX Apple Silicon", Packed
layouts and exact transcoding; GPTQModel "Packing Formats and Compatibility", GPTQ and GPTQ_V2):
packed words, scales and biases bit-exact against the oracle, and the transcoded weight through
qlinear_gemv against GPTQ's own reconstruction scale * (code - zero)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_quantized_affine_amd as q
from gpu_helpers import DEV, bits_to_dev, dev_to_bits, dev_to_u32, out_f64, u32_to_dev

pytestmark = pytest.mark.gpu


def _gptq(seed, k, n, bits, g, pdt):
    rng = np.random.default_rng(seed)
    qw = rng.integers(0, 1 << 32, size=(k * bits // 32, n), dtype=np.uint64).astype(np.uint32)
    qz = rng.integers(0, 1 << 32, size=(k // g, n * bits // 32), dtype=np.uint64).astype(np.uint32)
    sb = O.to_bits(pdt, (rng.random((k // g, n)) * 0.02 + 1e-3).astype(np.float32))
    return qw, qz, sb


@pytest.mark.parametrize("k,n,bits,g,pdt,v1", [
    (4096, 4096, 4, 128, "f16", False),
    (1024, 96, 3, 64, "f16", False),  # 3-bit streams crossing words; n not a multiple of 64
    (2048, 130 * 16, 2, 32, "bf16", True),
    (512, 300 * 4 // 4 * 4, 8, 64, "f16", True),
    (96, 32, 4, 32, "bf16", False),  # a single ragged transpose tile
])
def test_transcode_gptq_bitexact(k, n, bits, g, pdt, v1):
    qw, qz, sb = _gptq(k + n + bits, k, n, bits, g, pdt)
    pk, so, bo = q.qlinear_transcode_gptq(u32_to_dev(qw), u32_to_dev(qz), bits_to_dev(sb, pdt), bits=bits,
                                          group_size=g, v1_zeros=v1)
    torch.cuda.synchronize()
    opk, oso, obo = O.gptq_transcode(qw, qz, sb, bits, g, k, n, pdt, v1_zeros=v1)
    np.testing.assert_array_equal(dev_to_u32(pk), opk)
    np.testing.assert_array_equal(dev_to_bits(so), oso)
    np.testing.assert_array_equal(dev_to_bits(bo), obo)


def test_transcoded_gptq_weight_through_gemv():
    k, n, bits, g = 2048, 1024, 4, 128
    qw, qz, sb = _gptq(5, k, n, bits, g, "f16")
    pk, so, bo = q.qlinear_transcode_gptq(u32_to_dev(qw), u32_to_dev(qz), bits_to_dev(sb, "f16"), bits=bits,
                                          group_size=g)
    xb = synth.acts_bits(6, 2, k, "bf16")
    y = q.qlinear_gemv(bits_to_dev(xb, "bf16"), pk, so, bo, bits=bits, group_size=g, y_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.apply(O.bits_to_f64("bf16", xb), O.gptq_dequant_f64(qw, qz, sb, bits, g, k, n, "f16"))
    err = O.rel_l2_per_row(out_f64(y), ref)
    print(f"gptq transcode + gemv max rel-l2 {err.max():.3e}")
    # the transcoded bias is -zero*scale rounded once to fp16 (2^-11 relative): well inside 2e-3
    assert err.max() <= 2e-3


def test_transcode_gptq_graph_replay_matches_eager():
    """The transcoder captured in a HIP graph: each replay (outputs cleared, eager work between)
    gives the eager outputs bit for bit."""
    k, n, bits, g = 1024, 512, 4, 64
    qw, qz, sb = _gptq(9, k, n, bits, g, "f16")
    args = (u32_to_dev(qw), u32_to_dev(qz), bits_to_dev(sb, "f16"))
    want = [t.clone() for t in q.qlinear_transcode_gptq(*args, bits=bits, group_size=g)]
    outs = [torch.empty_like(t) for t in want]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        q.qlinear_transcode_gptq(*args, bits=bits, group_size=g, packed=outs[0], scales_out=outs[1],
                                 biases_out=outs[2])
    for rep in range(3):
        for o in outs:
            o.zero_()
        q.qlinear_transcode_gptq(*args, bits=bits, group_size=g)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o, w), f"replay {rep}"


# ---------------------------------------------------------------- AWQ GEMM -> affine rows
# (GPTQModel wiki "MLX Apple Silicon", Packed layouts and exact transcoding, AWQ GEMM and
# seven-bit rows, ParoQuant's lane order; GPTQModel "Packing Formats and Compatibility", AWQ GEMM)


def _awq(seed, k, n, bits, g, pdt):
    rng = np.random.default_rng(seed)
    qw = rng.integers(0, 1 << 32, size=(k, n * bits // 32), dtype=np.uint64).astype(np.uint32)
    qz = rng.integers(0, 1 << 32, size=(k // g, n * bits // 32), dtype=np.uint64).astype(np.uint32)
    sb = O.to_bits(pdt, (rng.random((k // g, n)) * 0.02 + 1e-3).astype(np.float32))
    return qw, qz, sb


@pytest.mark.parametrize("k,n,bits,g,pdt", [
    (4096, 4096, 4, 128, "f16"),  # 32 x 32 whole tiles
    (1024, 1056, 4, 64, "bf16"),  # a ragged column of tiles (1056 = 8 * 128 + 32)
    (1088, 96, 3, 32, "f16"),  # 3-bit streams crossing words; ragged rows and columns
    (512, 224, 2, 128, "bf16"),
    (640, 160, 5, 64, "f16"),
    (384, 352, 6, 128, "bf16"),
    (256, 288, 7, 32, "f16"),  # 7-bit source into 8-bit rows
    (2048, 512, 8, 64, "bf16"),
    (32, 32, 4, 32, "f16"),  # one 32 x 32 block
])
def test_transcode_awq_bitexact(k, n, bits, g, pdt):
    qw, qz, sb = _awq(3 * k + n + bits, k, n, bits, g, pdt)
    print(f"awq transcode k={k} n={n} bits={bits} g={g} {pdt}", flush=True)
    pk, so, bo = q.qlinear_transcode_awq(u32_to_dev(qw), u32_to_dev(qz), bits_to_dev(sb, pdt), bits=bits,
                                         group_size=g)
    torch.cuda.synchronize()
    opk, oso, obo = O.awq_transcode(qw, qz, sb, bits, g, k, n, pdt)
    np.testing.assert_array_equal(dev_to_u32(pk), opk)
    np.testing.assert_array_equal(dev_to_bits(so), oso)
    np.testing.assert_array_equal(dev_to_bits(bo), obo)


def test_transcoded_awq_weight_through_gemv():
    k, n, bits, g = 2048, 1024, 4, 128
    qw, qz, sb = _awq(15, k, n, bits, g, "f16")
    pk, so, bo = q.qlinear_transcode_awq(u32_to_dev(qw), u32_to_dev(qz), bits_to_dev(sb, "f16"), bits=bits,
                                         group_size=g)
    xb = synth.acts_bits(16, 2, k, "bf16")
    y = q.qlinear_gemv(bits_to_dev(xb, "bf16"), pk, so, bo, bits=bits, group_size=g, y_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.apply(O.bits_to_f64("bf16", xb), O.awq_dequant_f64(qw, qz, sb, bits, g, k, n, "f16"))
    err = O.rel_l2_per_row(out_f64(y), ref)
    print(f"awq transcode + gemv max rel-l2 {err.max():.3e}")
    assert err.max() <= 2e-3


def test_transcode_awq_leaves_bytes_past_outputs():
    """Outputs sit inside larger sentinel-filled buffers: nothing past the last packed word, scale
    or bias is written (ragged tiles at both ends)."""
    k, n, bits, g = 1088, 160, 4, 64
    qw, qz, sb = _awq(21, k, n, bits, g, "f16")
    words, groups = k * bits // 32, k // g
    pk_buf = torch.full((n * words + 64,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    so_buf = torch.full((n * groups + 64,), 0x7777, dtype=torch.int16, device=DEV)
    bo_buf = torch.full((n * groups + 64,), 0x7777, dtype=torch.int16, device=DEV)
    q.qlinear_transcode_awq(u32_to_dev(qw), u32_to_dev(qz), bits_to_dev(sb, "f16"), bits=bits, group_size=g,
                            packed=pk_buf[: n * words].view(n, words), scales_out=so_buf[: n * groups].view(n, groups),
                            biases_out=bo_buf[: n * groups].view(n, groups))
    torch.cuda.synchronize()
    assert bool((pk_buf[n * words:] == 0x5A5A5A5A).all())
    assert bool((so_buf[n * groups:] == 0x7777).all()) and bool((bo_buf[n * groups:] == 0x7777).all())
    opk, _, _ = O.awq_transcode(qw, qz, sb, bits, g, k, n, "f16")
    np.testing.assert_array_equal(dev_to_u32(pk_buf[: n * words].view(n, words)), opk)


# ---------------------------------------------------------------- GPTQ_P (planar) -> affine
# (GPTQModel "Packing Formats and Compatibility", GPTQ_P: planar blocks of 32 codes, true zeros)


def _planar(seed, k, n, bits, g, pdt):
    rng = np.random.default_rng(seed)
    qw = rng.integers(0, 1 << 32, size=(k * bits // 32, n), dtype=np.uint64).astype(np.uint32)
    qz = rng.integers(0, 1 << 32, size=(k // g, n * bits // 32), dtype=np.uint64).astype(np.uint32)
    sb = O.to_bits(pdt, (rng.random((k // g, n)) * 0.02 + 1e-3).astype(np.float32))
    return qw, qz, sb


@pytest.mark.parametrize("k,n,bits,g,pdt", [
    (4096, 4096, 3, 128, "f16"),  # whole 512 x 64 tiles
    (1088, 96, 3, 32, "bf16"),  # ragged rows (1088 = 2 * 512 + 64) and columns (96 = 64 + 32)
    (640, 160, 5, 64, "f16"),
    (384, 352, 6, 128, "bf16"),
    (256, 288, 7, 32, "f16"),  # 7-bit source into 8-bit rows
    (1024, 224, 2, 64, "bf16"),  # single plane: GPTQ's continuous words
    (512, 96, 4, 128, "f16"),
    (2048, 64, 8, 64, "bf16"),
    (32, 32, 7, 32, "bf16"),  # one block
])
def test_transcode_gptq_planar_bitexact(k, n, bits, g, pdt):
    qw, qz, sb = _planar(5 * k + n + bits, k, n, bits, g, pdt)
    print(f"gptq_p transcode k={k} n={n} bits={bits} g={g} {pdt}", flush=True)
    pk, so, bo = q.qlinear_transcode_gptq_planar(u32_to_dev(qw), u32_to_dev(qz), bits_to_dev(sb, pdt), bits=bits,
                                                 group_size=g)
    torch.cuda.synchronize()
    opk, oso, obo = O.gptq_planar_transcode(qw, qz, sb, bits, g, k, n, pdt)
    np.testing.assert_array_equal(dev_to_u32(pk), opk)
    np.testing.assert_array_equal(dev_to_bits(so), oso)
    np.testing.assert_array_equal(dev_to_bits(bo), obo)


def test_transcoded_gptq_planar_weight_through_gemv():
    k, n, bits, g = 2048, 1024, 6, 128
    qw, qz, sb = _planar(25, k, n, bits, g, "f16")
    pk, so, bo = q.qlinear_transcode_gptq_planar(u32_to_dev(qw), u32_to_dev(qz), bits_to_dev(sb, "f16"), bits=bits,
                                                 group_size=g, g_idx=np.arange(k, dtype=np.int32) // g)
    xb = synth.acts_bits(26, 2, k, "bf16")
    y = q.qlinear_gemv(bits_to_dev(xb, "bf16"), pk, so, bo, bits=bits, group_size=g, y_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.apply(O.bits_to_f64("bf16", xb), O.gptq_planar_dequant_f64(qw, qz, sb, bits, g, k, n, "f16"))
    err = O.rel_l2_per_row(out_f64(y), ref)
    print(f"gptq_p transcode + gemv max rel-l2 {err.max():.3e}")
    assert err.max() <= 2e-3


def test_transcode_gptq_planar_leaves_bytes_past_outputs():
    k, n, bits, g = 1088, 160, 7, 64
    qw, qz, sb = _planar(31, k, n, bits, g, "bf16")
    words, groups = k * 8 // 32, k // g
    pk_buf = torch.full((n * words + 64,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    so_buf = torch.full((n * groups + 64,), 0x7777, dtype=torch.int16, device=DEV)
    bo_buf = torch.full((n * groups + 64,), 0x7777, dtype=torch.int16, device=DEV)
    q.qlinear_transcode_gptq_planar(u32_to_dev(qw), u32_to_dev(qz), bits_to_dev(sb, "bf16"), bits=bits, group_size=g,
                                    packed=pk_buf[: n * words].view(n, words),
                                    scales_out=so_buf[: n * groups].view(n, groups),
                                    biases_out=bo_buf[: n * groups].view(n, groups))
    torch.cuda.synchronize()
    assert bool((pk_buf[n * words:] == 0x5A5A5A5A).all())
    assert bool((so_buf[n * groups:] == 0x7777).all()) and bool((bo_buf[n * groups:] == 0x7777).all())
    opk, _, _ = O.gptq_planar_transcode(qw, qz, sb, bits, g, k, n, "bf16")
    np.testing.assert_array_equal(dev_to_u32(pk_buf[: n * words].view(n, words)), opk)
