"""GPU parity of quantize_q8_0, MXFP4 in GGUF blocks and take (Nx_quant API docs: quantize_q8_0;
Weights, Mxfp4_blocks; take): every byte and every decoded value bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_quantized_affine_amd as q
from gpu_helpers import DEV, TDT, bits_to_dev, out_bits_or_f32, same_values, u32_to_dev, u8_to_dev

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


def _q8_input(seed, rows, k):
    w = synth.weights_f32(seed, rows, k, std=0.3)
    nb = k // 32
    # edge blocks on the first rows: an infinity, a NaN (with an infinity beside it), a tiny block
    # (1/d infinite), zeros, a block whose d rounds past fp16's largest, exact halves, -0
    w[0, 3] = np.inf
    w[0, 32 + 7] = -np.inf
    if nb > 2:
        w[0, 64 + 1] = np.nan
        w[0, 64 + 2] = np.inf
    w[1, :32] = 1e-39
    w[1, 32:64] = 0.0
    w[1, 40] = -0.0
    w[2, :32] = 1e7
    w[2, 32:64] = np.float32(127.0) * (np.arange(32, dtype=np.float32) / 31.0)
    w[2, 33] = 2.5
    w[2, 34] = -3.5
    w[3, :32] = -1e-30
    return w


@pytest.mark.parametrize("rows,k", [(7, 96), (64, 2880), (1, 32), (300, 4096)])
def test_quantize_q8_0_bitexact(rows, k):
    w = _q8_input(100 + rows, max(rows, 4), k)[:rows] if rows >= 4 else synth.weights_f32(7, rows, k)
    blocks = q.qlinear_quantize_q8_0(torch.from_numpy(np.ascontiguousarray(w)).to(DEV))
    _sync()
    np.testing.assert_array_equal(blocks.cpu().numpy(), O.q8_0_quantize(w))


def test_quantize_q8_0_then_dequant():
    w = _q8_input(5, 16, 512)
    blocks = q.qlinear_quantize_q8_0(torch.from_numpy(w).to(DEV))
    out = q.qlinear_dequant(q.QL_Q8_0, blocks, rows=16, k=512, out_dtype=torch.float32)
    _sync()
    assert same_values(out.cpu().numpy(), O.q8_0_dequant_f32(O.q8_0_quantize(w)))


@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
def test_dequant_mxfp4_blocks_bitexact(odt):
    g = np.random.default_rng(31)
    rows, k = 37, 2880
    blocks = g.integers(0, 256, size=(rows, k // 32, 17)).astype(np.uint8)
    blocks[..., 0] = g.integers(110, 140, size=(rows, k // 32))
    blocks[0, :4, 0] = [0, 1, 254, 255]  # subnormal scales, overflow to inf, NaN
    blocks = blocks.reshape(rows, k // 32 * 17)
    out = q.qlinear_dequant(q.QL_MXFP4_BLOCKS, u8_to_dev(blocks), rows=rows, k=k, out_dtype=TDT[odt])
    _sync()
    want = O.round_f32_to(odt, O.mxfp4_blocks_dequant_f32(blocks))
    got = out_bits_or_f32(out, odt)
    if odt == "f32":
        assert same_values(got, want)
    else:  # the scale byte 255 gives NaN; its 16-bit sign and payload are not fixed by the page
        nan = np.isnan(O.bits_to_f64(odt, want))
        assert np.array_equal(nan, np.isnan(O.bits_to_f64(odt, got)))
        assert np.array_equal(got[~nan], want[~nan])


def test_take_affine_parts_and_blocks_bitexact():
    n, k = 300, 1024
    pk, sb, bb = O.affine_quantize(synth.weights_f32(41, n, k), 4, 64, "bf16")
    pos_np = np.array([5, 0, 299, -1, 300, 17, 17, 123456, 250], dtype=np.int64)
    pos = torch.from_numpy(pos_np).to(DEV)
    tp = q.qlinear_take(pos, u32_to_dev(pk))
    ts = q.qlinear_take(pos, bits_to_dev(sb, "bf16"))
    tb = q.qlinear_take(pos, bits_to_dev(bb, "bf16"))
    blocks = O.q8_0_quantize(synth.weights_f32(42, n, 96))  # 102-byte rows: byte copies
    tq = q.qlinear_take(pos, u8_to_dev(blocks))
    _sync()
    np.testing.assert_array_equal(tp.cpu().numpy().view(np.uint32), O.take(pos_np, pk))
    np.testing.assert_array_equal(ts.cpu().view(torch.int16).numpy().view(np.uint16), O.take(pos_np, sb))
    np.testing.assert_array_equal(tb.cpu().view(torch.int16).numpy().view(np.uint16), O.take(pos_np, bb))
    np.testing.assert_array_equal(tq.cpu().numpy(), O.take(pos_np, blocks))
    # and the gathered affine weight decodes to the gathered values (zeros out of range)
    D = q.qlinear_dequant(q.QL_AFFINE, tp, ts, tb, rows=len(pos_np), k=k, bits=4, group_size=64,
                          out_dtype=torch.float32)
    _sync()
    want = O.take(pos_np, O.affine_dequant_f32(pk, sb, bb, 4, 64, "bf16", k))
    np.testing.assert_array_equal(D.cpu().numpy(), want)


def test_take_experts_matrices():
    """Whole expert matrices of an MXFP4 stack (rows of n * k/2 bytes, several 32 KiB parts each)."""
    g = np.random.default_rng(43)
    e, n, k = 6, 192, 768
    codes = g.integers(0, 256, size=(e, n, k // 2)).astype(np.uint8)
    pos_np = np.array([4, -2, 0, 4, 6], dtype=np.int64)
    got = q.qlinear_take(torch.from_numpy(pos_np).to(DEV), u8_to_dev(codes))
    _sync()
    np.testing.assert_array_equal(got.cpu().numpy(), O.take(pos_np, codes))


def test_take_four_byte_rows_and_empty_source():
    """Rows of 12 bytes (4-byte units) and a source with no rows (every position out of range)."""
    g = np.random.default_rng(44)
    src = g.integers(0, 2**31, size=(50, 3)).astype(np.int32)
    pos_np = np.array([49, 0, -5, 50, 25], dtype=np.int64)
    got = q.qlinear_take(torch.from_numpy(pos_np).to(DEV), torch.from_numpy(src).to(DEV))
    empty = torch.empty((0, 3), dtype=torch.int32, device=DEV)
    got0 = q.qlinear_take(torch.from_numpy(pos_np).to(DEV), empty)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), O.take(pos_np, src))
    assert np.all(got0.cpu().numpy() == 0)


@pytest.mark.parametrize("e,n,k,tokens,top,xdt", [
    (3, 201, 288, 40, 2, "bf16"),   # 3 * 201 * 9 * 17 bytes: the blocks end inside a word
    (4, 384, 1024, 70, 4, "bf16"),  # whole tiles of 384 rows
    (2, 100, 4160, 20, 2, "f16"),   # long rows, fp16 x
])
def test_apply_experts_mxfp4_blocks(e, n, k, tokens, top, xdt):
    """The routed apply on MXFP4 in GGUF blocks (Nx_quant Products: apply_experts takes any weight;
    Weights, Mxfp4_blocks): against the oracle's fp64 sums of the decoded values, 1e-4 per row (the
    values are exact in bf16, so this is fp32 accumulation only)."""
    g = np.random.default_rng(e * 1000 + n + k)
    blocks = g.integers(0, 256, size=(e, n, k // 32, 17)).astype(np.uint8)
    blocks[..., 0] = g.integers(118, 131, size=(e, n, k // 32))
    blocks = blocks.reshape(e, n, k // 32 * 17)
    W = O.mxfp4_blocks_dequant_f32(blocks)
    ids = g.integers(-1, e + 1, size=(tokens, top)).astype(np.int64)
    xb = synth.acts_bits(e + n + k, tokens, k, xdt)
    print(f"mxfp4 blocks apply_experts e={e} n={n} k={k} x={xdt}", flush=True)
    y = q.qlinear_apply_experts(q.QL_MXFP4_BLOCKS, u8_to_dev(blocks), None, torch.from_numpy(ids.reshape(-1)).to(DEV),
                                bits_to_dev(xb, xdt), n=n, k=k, pos_per_row=top, y_dtype=torch.float32)
    _sync()
    flat = ids.reshape(-1)
    ref = O.apply_experts(W, flat, O.bits_to_f64(xdt, xb), pos_per_row=top)
    live = (flat >= 0) & (flat < e)
    out = y.cpu().numpy().astype(np.float64)
    assert np.all(out[~live] == 0.0)
    err = O.rel_l2_per_row(out[live], ref[live])
    print(f"mxfp4 blocks experts max rel-l2 {err.max():.3e}")
    assert err.max() <= 1e-4
