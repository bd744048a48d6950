"""Guard bands around every kernel's outputs: each output lives inside a larger buffer whose bytes
before and after it hold a sentinel pattern; after the call the sentinels must be intact (no write
past either end) and the output must be fully written.  Ragged shapes put the partial tiles, the
split-k partial sums and the odd-sized copy units at the edges."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_quantized_affine_amd as q
from gpu_helpers import DEV, bits_to_dev, u32_to_dev, u8_to_dev

pytestmark = pytest.mark.gpu

PAD = 4096      # guard bytes on each side (a multiple of 256: the output keeps its alignment)
SENT = 0xA5     # sentinel byte


def guarded(shape, dtype):
    """(view, buf): `view` [shape] of `dtype` inside `buf`, a uint8 buffer with PAD sentinel bytes on
    each side; the view itself is also pre-filled with the sentinel."""
    nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf = torch.full((PAD + nbytes + PAD,), SENT, dtype=torch.uint8, device=DEV)
    view = buf[PAD:PAD + nbytes].view(dtype).view(*shape)
    return view, buf


def check(buf, label, written=True):
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[:PAD] == SENT), f"{label}: bytes written before the output"
    assert np.all(b[-PAD:] == SENT), f"{label}: bytes written past the output"
    if written:
        inner = b[PAD:-PAD]
        # a fully written output is unlikely to keep a whole aligned 16-byte run of the sentinel
        runs = inner[: inner.size // 16 * 16].reshape(-1, 16)
        assert not np.any(np.all(runs == SENT, axis=1)), f"{label}: part of the output was not written"


def _affine(seed, n, k, bits, g, pdt="bf16"):
    w = synth.weights_f32(seed, n, k)
    return q.qlinear_quantize(torch.from_numpy(w).to(DEV), bits, g, torch.bfloat16 if pdt == "bf16" else torch.float16)


@pytest.mark.parametrize("bits,n,k", [(4, 257, 1024), (3, 131, 1056), (8, 77, 384), (2, 300, 160)])
def test_canary_quantize(bits, n, k):
    w = torch.from_numpy(synth.weights_f32(10 + bits, n, k)).to(DEV)
    words = k * bits // 32
    pk, bp = guarded((n, words), torch.int32)
    sc, bs = guarded((n, k // 32), torch.bfloat16)
    bi, bb = guarded((n, k // 32), torch.bfloat16)
    q.qlinear_quantize(w, bits, 32, torch.bfloat16, packed=pk, scales=sc, biases=bi)
    check(bp, f"quantize {bits}-bit packed")
    check(bs, "quantize scales")
    check(bb, "quantize biases")


@pytest.mark.parametrize("m,n,k,bits,g", [(1, 257, 1024, 4, 64), (3, 131, 1088, 4, 64), (8, 77, 1024, 8, 64),
                                          (5, 99, 1056, 3, 32), (2, 45, 384, 6, 128)])
def test_canary_gemv(m, n, k, bits, g):
    pk, sc, bi = _affine(20 + n, n, k, bits, g)
    x = bits_to_dev(synth.acts_bits(21 + n, m, k, "bf16"), "bf16")
    for ydt in (torch.float32, torch.bfloat16):
        y, b = guarded((m, n), ydt)
        q.qlinear_gemv(x, pk, sc, bi, bits=bits, group_size=g, y=y)
        check(b, f"gemv m={m} n={n} k={k} bits={bits} y={ydt}")


def test_canary_gemv_batched():
    shapes = [(1, 257, 1024, 4), (1, 131, 2048, 4), (8, 77, 1024, 8), (2, 50, 1056, 3)]
    probs, bufs = [], []
    for i, (m, n, k, bits) in enumerate(shapes):
        pk, sc, bi = _affine(30 + i, n, k, bits, 32 if bits == 3 else 64)
        x = bits_to_dev(synth.acts_bits(31 + i, m, k, "bf16"), "bf16")
        y, b = guarded((m, n), torch.float32)
        probs.append(dict(x=x, packed=pk, scales=sc, biases=bi, y=y, bits=bits, group_size=32 if bits == 3 else 64))
        bufs.append(b)
    ws = torch.empty(q.qlinear_gemv_batched_workspace_size(probs), dtype=torch.uint8, device=DEV)
    q.qlinear_gemv_batched(probs, x_dtype=torch.bfloat16, param_dtype=torch.bfloat16, y_dtype=torch.float32,
                           workspace=ws)
    for i, b in enumerate(bufs):
        check(b, f"batched problem {i}")


@pytest.mark.parametrize("m,n,k,bits", [
    (200, 300, 1024, 4),    # few output tiles: split over k, partial sums summed by a second pass
    (2100, 4000, 320, 4),   # ragged m and n tiles
    (130, 520, 512, 8),     # 8-bit, split over k
    (150, 200, 320, 6),     # re-packed 6-bit rows
])
def test_canary_gemm(m, n, k, bits):
    pk, sc, bi = _affine(40 + m, n, k, bits, 64)
    x = bits_to_dev(synth.acts_bits(41 + m, m, k, "bf16"), "bf16")
    for ydt in (torch.float32, torch.bfloat16):
        y, b = guarded((m, n), ydt)
        q.qlinear_gemm(x, pk, sc, bi, bits=bits, group_size=64, y=y)
        check(b, f"gemm m={m} n={n} k={k} bits={bits} y={ydt}")


def test_canary_dequant_every_format():
    rows = 37
    # affine 4-bit and 5-bit
    for bits, k in ((4, 1088), (5, 320)):
        pk, sc, bi = _affine(50 + bits, rows, k, bits, 32)
        out, b = guarded((rows, k), torch.bfloat16)
        q.qlinear_dequant(q.QL_AFFINE, pk, sc, bi, rows=rows, k=k, bits=bits, group_size=32, out=out)
        check(b, f"dequant affine {bits}-bit")
    k = 512
    codes, scales = synth.mxfp4_codes_scales(52, 1, rows, k)
    out, b = guarded((rows, k), torch.float32)
    q.qlinear_dequant(q.QL_MXFP4, u8_to_dev(codes[0]), u8_to_dev(scales[0]), rows=rows, k=k, out=out)
    check(b, "dequant mxfp4")
    blocks = synth.q8_0_random_blocks(53, 1, rows, k)[0]
    out, b = guarded((rows, k), torch.float16)
    q.qlinear_dequant(q.QL_Q8_0, u8_to_dev(blocks), rows=rows, k=k, out=out)
    check(b, "dequant q8_0")
    g = np.random.default_rng(54)
    mb = g.integers(0, 256, size=(rows, k // 32 * 17)).astype(np.uint8)
    out, b = guarded((rows, k), torch.float32)
    q.qlinear_dequant(q.QL_MXFP4_BLOCKS, u8_to_dev(mb), rows=rows, k=k, out=out)
    check(b, "dequant mxfp4 blocks")
    for fmt, name in ((q.QL_Q4_K, "q4_k"), (q.QL_Q6_K, "q6_k")):
        kb = synth.kquant_random_blocks(55 + fmt, rows, k, name)
        out, b = guarded((rows, k), torch.bfloat16)
        q.qlinear_dequant(fmt, u8_to_dev(kb), rows=rows, k=k, out=out)
        check(b, f"dequant {name}")


@pytest.mark.parametrize("row_bytes", [64, 68, 17, 1])  # 16-byte, 4-byte and 1-byte copy units
def test_canary_take(row_bytes):
    src_rows, n_pos = 50, 33
    src = u8_to_dev(np.random.default_rng(row_bytes).integers(0, 256, size=(src_rows, row_bytes)).astype(np.uint8))
    pos = torch.from_numpy(np.random.default_rng(60).integers(-2, src_rows + 2, size=n_pos).astype(np.int64)).to(DEV)
    dst, b = guarded((n_pos, row_bytes), torch.uint8)
    q.qlinear_take(pos, src, dst=dst)
    # rows out of range are zeros and some sources may hold the sentinel byte: check the bands only
    check(b, f"take row_bytes={row_bytes}", written=False)
    want = np.zeros((n_pos, row_bytes), np.uint8)
    p = pos.cpu().numpy()
    ok = (p >= 0) & (p < src_rows)
    want[ok] = src.cpu().numpy()[p[ok]]
    np.testing.assert_array_equal(dst.cpu().numpy(), want)


def test_canary_quantize_q8_0_and_transcoders():
    rows, k = 21, 96
    w = torch.from_numpy(synth.weights_f32(70, rows, k)).to(DEV)
    blocks, b = guarded((rows, k // 32 * 34), torch.uint8)
    q.qlinear_quantize_q8_0(w, blocks=blocks)
    check(b, "quantize_q8_0")
    k, n, bits, g = 1088, 160, 4, 64
    rng = np.random.default_rng(71)
    qw = rng.integers(0, 1 << 32, size=(k * bits // 32, n), dtype=np.uint64).astype(np.uint32)
    qz = rng.integers(0, 1 << 32, size=(k // g, n * bits // 32), dtype=np.uint64).astype(np.uint32)
    sb = O.to_bits("f16", (rng.random((k // g, n)) * 0.02 + 1e-3).astype(np.float32))
    pk, bp = guarded((n, k * bits // 32), torch.int32)
    so, bs = guarded((n, k // g), torch.float16)
    bo, bb = guarded((n, k // g), torch.float16)
    q.qlinear_transcode_gptq(u32_to_dev(qw), u32_to_dev(qz), bits_to_dev(sb, "f16"), bits=bits, group_size=g,
                             packed=pk, scales_out=so, biases_out=bo)
    check(bp, "gptq packed")
    check(bs, "gptq scales")
    check(bb, "gptq biases")


@pytest.mark.parametrize("fmt", ["mxfp4", "q8_0", "q4_k", "q6_k", "mxfp4_blocks"])
def test_canary_apply_experts(fmt):
    e, n, tokens, top = 3, 201, 37, 3
    k = 512 if fmt in ("q4_k", "q6_k") else 288
    rng = np.random.default_rng(80)
    if fmt == "mxfp4":
        codes, scales = synth.mxfp4_codes_scales(81, e, n, k)
        w0, w1, f = u8_to_dev(codes), u8_to_dev(scales), q.QL_MXFP4
    elif fmt == "q8_0":
        w0, w1, f = u8_to_dev(synth.q8_0_random_blocks(82, e, n, k)), None, q.QL_Q8_0
    elif fmt == "mxfp4_blocks":
        mb = rng.integers(0, 256, size=(e, n, k // 32, 17)).astype(np.uint8)
        mb[..., 0] = rng.integers(118, 131, size=(e, n, k // 32))
        w0, w1, f = u8_to_dev(mb.reshape(e, n, -1)), None, q.QL_MXFP4_BLOCKS
    else:
        f = q.QL_Q4_K if fmt == "q4_k" else q.QL_Q6_K
        w0, w1 = u8_to_dev(synth.kquant_random_blocks(83, e * n, k, fmt).reshape(e, n, -1)), None
    ids = torch.from_numpy(rng.integers(-1, e + 1, size=tokens * top).astype(np.int64)).to(DEV)
    x = bits_to_dev(synth.acts_bits(84, tokens, k, "bf16"), "bf16")
    for ydt in (torch.float32, torch.bfloat16):
        y, b = guarded((tokens * top, n), ydt)
        ws, bw = guarded((q.qlinear_apply_experts_workspace_size(tokens * top, e),), torch.uint8)
        q.qlinear_apply_experts(f, w0, w1, ids, x, n=n, k=k, pos_per_row=top, y=y, workspace=ws)
        check(b, f"experts {fmt} y={ydt}")
        check(bw, f"experts {fmt} workspace", written=False)
