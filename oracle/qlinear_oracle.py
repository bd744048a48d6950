"""Plain, slow, obviously correct NumPy oracle of the weight-only quantized linear path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the product path.  It shares no code with the
HIP library.

Sources (cited by page title and section):

* GPTQModel wiki, "MLX Apple Silicon": the Concepts table (MLX affine storage: packed uint32
  codes, scales and additive biases, value = code*scale + bias) and "Packed layouts and exact
  transcoding" (scales/biases laid out [out, groups]; each row one continuous little-endian
  bitstream of codes: whole codes per uint32 for 2/4/8 bits, codes crossing words for 3/5/6
  bits; GGUF Q8_0 maps to 8-bit group-32 affine with the signed byte plus 128).
* tinygpt PRD "Quantized inference ... QuantizedLinear", section "Problem": 8 four-bit values
  per uint32 with per-weight ``.scales`` and ``.biases`` companions.
* gguf2mlx-stream, section "01 Tensor-bounded streaming": MLX affine quantization into packed
  uint32 plus f16 scales/biases.
* Nx_quant API docs: "Weights" (Mxfp4 codes/scales layout, Q8_0 block layout, the MXFP4
  decode rule), ``quantize_q8_0``, and "Products" (``dequant``, ``apply``,
  ``apply_experts``).

Readings of points the pages leave open:

* quantizer: per (row, group of g along k): mn = min, mx = max over the group in fp32 (total
  order, -0 < +0); s32 = fl32(fl32(mx - mn) / (2^bits - 1)); stored s = RNE(s32), stored
  b = RNE(mn) in the parameter dtype; t = fl32(fl32(v - b) / s) with the stored b, s; code
  q = clamp(round-half-even(t), 0, 2^bits - 1); q = 0 where the stored s is 0.
* dequant: value = fl32(q*s + b) (one rounding; q*s is exact in fp32), then rounded once to
  the output dtype.
* apply: y = x . dequant(W)^T computed here exactly in fp64 from the fp32 values.
* quantize_q8_0: the NaN scale of a block holding a NaN is the fp16 quiet NaN 0x7E00 (the page
  fixes "a NaN scale", not its bits); a block holding an infinity and no NaN takes +inf (0x7C00).
* take: positions outside [0, rows) are out of range (negative ones too) and give zero bytes.
* Q4_K / Q6_K: the pages fix the block sizes, the field order and the value formulas and name
  ggml's block_q4_K / block_q6_K for the layout; the placement of the 6-bit scales and mins inside
  Q4_K's 12 bytes and of the quants inside the quant bytes follows that layout as this oracle
  reads it (_q4_k_fields, _q6_k_fields).  No ggml bytes are at hand to check it against.
* GPTQ_P: "weight packing follows rows" is read as the planar blocks running down each
  column of qweight (the input axis, as GPTQ's continuous streams do) and "zero packing follows
  columns" as the blocks running along each row of qzeros (the outputs).
* AWQ lane order [0,2,4,6,1,3,5,7]: read as the columns that the nibbles of a word hold, from
  the low nibble up (nibble 1 holds column 2), applied to 4-bit qweight and qzeros alike; other
  widths are plain streams along the outputs.

Float storage types travel as uint16 bit patterns (``'f16'`` or ``'bf16'``); fp32 as numpy
float32.  All arithmetic below is NumPy on the CPU.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "f32_to_f16_bits",
    "f16_bits_to_f32",
    "to_bits",
    "bits_to_f64",
    "round_f32_to",
    "AFFINE_BITS",
    "pack_codes",
    "unpack_codes",
    "group_min_max",
    "affine_quantize",
    "affine_dequant_f32",
    "affine_dequant_to",
    "apply",
    "MXFP4_MAGNITUDES",
    "mxfp4_dequant_f32",
    "q8_0_dequant_f32",
    "q8_0_quantize",
    "Q4_K_BYTES",
    "Q6_K_BYTES",
    "q4_k_dequant_f32",
    "q6_k_dequant_f32",
    "mxfp4_blocks_dequant_f32",
    "take",
    "gptq_transcode",
    "gptq_dequant_f64",
    "gptq_planes",
    "gptq_planar_codes",
    "gptq_planar_transcode",
    "gptq_planar_dequant_f64",
    "AWQ_LANE_ORDER",
    "awq_codes",
    "awq_transcode",
    "awq_dequant_f64",
    "route",
    "apply_experts",
    "rel_l2_per_row",
]

# --------------------------------------------------------------------------------------
# 16-bit float storage types (IEEE binary16 and bfloat16), round to nearest even.
# --------------------------------------------------------------------------------------


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round fp32 to bfloat16 (nearest, ties to even); NaN maps to a quiet NaN of the same sign."""
    a = np.asarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(a)
    if np.any(nan):
        r = r.copy()
        r[nan] = ((u[nan] >> np.uint64(16)).astype(np.uint16) | np.uint16(0x0040))
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(a) -> np.ndarray:
    """Round fp32 to IEEE binary16 (NumPy's conversion rounds to nearest even)."""
    return np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def to_bits(dtype: str, a_f32) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(a_f32)
    if dtype == "f16":
        return f32_to_f16_bits(a_f32)
    raise ValueError(f"not a 16-bit dtype: {dtype}")


def bits_to_f64(dtype: str, bits) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(bits).astype(np.float64)
    if dtype == "f16":
        return f16_bits_to_f32(bits).astype(np.float64)
    raise ValueError(f"not a 16-bit dtype: {dtype}")


def round_f32_to(dtype: str, a_f32):
    """Round an fp32 array once to ``dtype``: returns float32 for 'f32', bit patterns otherwise."""
    if dtype == "f32":
        return np.asarray(a_f32, dtype=np.float32)
    return to_bits(dtype, a_f32)


# --------------------------------------------------------------------------------------
# Affine storage (GPTQModel wiki "MLX Apple Silicon": Concepts; Packed layouts).
# --------------------------------------------------------------------------------------


AFFINE_BITS = (2, 3, 4, 5, 6, 8)


def _stream_unit(bits: int):
    """(codes, words) of the repeating unit of a row's bitstream: the fewest codes that fill
    whole uint32 words (8 codes in 1 word at 4 bits; 32 codes in 3 words at 3 bits)."""
    d = int(np.gcd(bits, 32))
    return 32 // d, bits // d


def pack_codes(q, bits: int) -> np.ndarray:
    """Pack integer codes [rows, k] into uint32 words [rows, k*bits/32], low bits first.

    GPTQModel wiki "MLX Apple Silicon", "Packed layouts and exact transcoding": each row is one
    continuous little-endian bitstream; code i of the row occupies stream bits
    [bits*i, bits*(i+1)) and stream bit j is bit j % 32 of word j // 32.  At 2, 4 and 8 bits
    whole codes sit in each word; at 3, 5 and 6 bits codes cross word boundaries."""
    q = np.asarray(q, dtype=np.int64)
    rows, k = q.shape
    assert bits in AFFINE_BITS
    uc, uw = _stream_unit(bits)
    assert k % uc == 0, "a row must fill whole words"
    assert q.min(initial=0) >= 0 and q.max(initial=0) < (1 << bits)
    qq = q.reshape(rows, k // uc, uc).astype(np.uint64)
    words = np.zeros((rows, k // uc, uw), dtype=np.uint64)
    for i in range(uc):
        w, sh = divmod(bits * i, 32)
        words[:, :, w] |= (qq[:, :, i] << np.uint64(sh)) & np.uint64(0xFFFFFFFF)
        if sh + bits > 32:  # the code's high bits start the next word
            words[:, :, w + 1] |= qq[:, :, i] >> np.uint64(32 - sh)
    return words.reshape(rows, (k // uc) * uw).astype(np.uint32)


def unpack_codes(packed, bits: int, k: int) -> np.ndarray:
    """Inverse of :func:`pack_codes`: words [rows, k*bits/32] -> codes [rows, k] (int64)."""
    packed = np.asarray(packed, dtype=np.uint32)
    assert bits in AFFINE_BITS
    uc, uw = _stream_unit(bits)
    rows = packed.shape[0]
    assert k % uc == 0 and packed.shape[1] * uc == k * uw
    ww = packed.reshape(rows, k // uc, uw).astype(np.uint64)
    mask = np.uint64((1 << bits) - 1)
    out = np.empty((rows, k // uc, uc), dtype=np.int64)
    for i in range(uc):
        w, sh = divmod(bits * i, 32)
        v = ww[:, :, w] >> np.uint64(sh)
        if sh + bits > 32:
            v = v | (ww[:, :, w + 1] << np.uint64(32 - sh))
        out[:, :, i] = (v & mask).astype(np.int64)
    return out.reshape(rows, k)


def group_min_max(v_f32):
    """Per-row min and max of fp32 values [..., g] under the IEEE total order (-0 < +0).

    Only finite inputs are in the domain."""
    v = np.asarray(v_f32, dtype=np.float32)
    assert np.all(np.isfinite(v)), "the affine quantizer is defined for finite weights only"
    mn = v.min(axis=-1)
    mx = v.max(axis=-1)
    neg0 = np.signbit(v) & (v == 0)
    pos0 = (~np.signbit(v)) & (v == 0)
    mn = np.where((mn == 0) & neg0.any(axis=-1), np.float32(-0.0), np.where(mn == 0, np.float32(0.0), mn))
    mx = np.where((mx == 0) & pos0.any(axis=-1), np.float32(0.0), np.where(mx == 0, np.float32(-0.0), mx))
    return mn.astype(np.float32), mx.astype(np.float32)


def affine_quantize(w_f32, bits: int, group_size: int, param_dtype: str):
    """Affine group quantizer: fp32 W [n, k] -> (packed u32 [n, k*bits/32], scale bits [n, k/g],
    bias bits [n, k/g]).

    Per (row, group): scale = (max - min) / (2^bits - 1), bias = min, stored in
    ``param_dtype`` (round to nearest even); codes are the nearest level to each value,
    computed as round-half-even((v - b) / s) with the stored b and s, clamped to
    [0, 2^bits - 1]; a zero stored scale gives code 0 (readings listed in the module doc)."""
    w = np.asarray(w_f32, dtype=np.float32)
    n, k = w.shape
    g = group_size
    assert k % g == 0 and k % 32 == 0
    levels = np.float32((1 << bits) - 1)
    v = w.reshape(n, k // g, g)
    mn, mx = group_min_max(v)
    with np.errstate(over="ignore"):
        s32 = ((mx - mn).astype(np.float32) / levels).astype(np.float32)
    s_bits = to_bits(param_dtype, s32)
    b_bits = to_bits(param_dtype, mn)
    s = bits_to_f64(param_dtype, s_bits).astype(np.float32)
    b = bits_to_f64(param_dtype, b_bits).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        t = ((v - b[..., None]).astype(np.float32) / s[..., None]).astype(np.float32)
    q = np.clip(np.rint(t), 0, levels)
    q = np.where(s[..., None] == 0, 0, q)
    q = np.where(np.isnan(q), 0, q).astype(np.int64).reshape(n, k)
    return pack_codes(q, bits), s_bits, b_bits


def affine_dequant_f32(packed, scale_bits, bias_bits, bits: int, group_size: int, param_dtype: str, k: int):
    """value = fl32(q*s + b) for every weight (Nx_quant "Products", dequant: a value is a
    float32 value).  q*s + b is exact in fp64 (q < 2^8, s has <= 11 significant bits), so the
    single rounding to fp32 here is the only one."""
    q = unpack_codes(packed, bits, k).astype(np.float64)
    n = q.shape[0]
    s = bits_to_f64(param_dtype, scale_bits)
    b = bits_to_f64(param_dtype, bias_bits)
    sg = np.repeat(s, group_size, axis=1).reshape(n, k)
    bg = np.repeat(b, group_size, axis=1).reshape(n, k)
    return (q * sg + bg).astype(np.float32)


def affine_dequant_to(out_dtype: str, packed, scale_bits, bias_bits, bits, group_size, param_dtype, k):
    """dequant at ``out_dtype``: the fp32 value rounded once (bit patterns for 16-bit types)."""
    return round_f32_to(out_dtype, affine_dequant_f32(packed, scale_bits, bias_bits, bits, group_size, param_dtype, k))


def apply(x_f64, w_values, layer_bias=None) -> np.ndarray:
    """Nx_quant "Products", apply: y = x . W^T with W the dequantized (fp32) weight values, here
    summed exactly enough in fp64 (NumPy matmul over fp64 copies).  x is [m, k], W [n, k]."""
    x = np.asarray(x_f64, dtype=np.float64)
    w = np.asarray(w_values, dtype=np.float64)
    y = x @ w.T
    if layer_bias is not None:
        y = y + np.asarray(layer_bias, dtype=np.float64)[None, :]
    return y


def gptq_transcode(qweight, qzeros, scale_bits, bits: int, group_size: int, k: int, n: int,
                   param_dtype: str, v1_zeros: bool = False):
    """GPTQ (continuous layout) -> MLX affine rows (GPTQModel wiki "MLX Apple Silicon", Packed
    layouts and exact transcoding: unpack the input-axis codes and the output-axis zeros, scales
    to [out, groups], additive bias -zero*scale, uint32 row streams; GPTQModel "Packing Formats
    and Compatibility", GPTQ and GPTQ_V2: qweight [K*b/32, N] codes as a continuous b-bit stream
    down each column, qzeros [G, N*b/32] a stream along the outputs, scales [G, N], value
    scale * (code - zero), v1 storing zero - 1).

    Returns (packed [n, k*bits/32], scales [n, G], biases [n, G]) with biases = RNE(-zero * scale)
    in param_dtype (the product is exact in fp32).  Groups are contiguous (g_idx[k] = k // g)."""
    qweight = np.asarray(qweight, dtype=np.uint32)
    qzeros = np.asarray(qzeros, dtype=np.uint32)
    G = k // group_size
    assert qweight.shape == (k * bits // 32, n) and qzeros.shape == (G, n * bits // 32)
    codes = unpack_codes(qweight.T, bits, k)  # column streams down the input axis -> [n, k]
    zeros = unpack_codes(qzeros, bits, n)  # row streams along the outputs -> [G, n]
    if v1_zeros:
        zeros = zeros + 1
    s = bits_to_f64(param_dtype, np.asarray(scale_bits, dtype=np.uint16))  # [G, n]
    b32 = (-(zeros.astype(np.float64)) * s).astype(np.float32)  # exact: |zero| <= 2^8, s has <= 11 bits
    return (pack_codes(codes, bits), np.ascontiguousarray(np.asarray(scale_bits, dtype=np.uint16).T),
            np.ascontiguousarray(to_bits(param_dtype, b32).T))


def gptq_dequant_f64(qweight, qzeros, scale_bits, bits: int, group_size: int, k: int, n: int, param_dtype: str,
                     v1_zeros: bool = False):
    """GPTQ's own reconstruction, scale * (code - zero), exactly in fp64: [n, k] (per output row)."""
    codes = unpack_codes(np.asarray(qweight, dtype=np.uint32).T, bits, k).astype(np.float64)
    zeros = unpack_codes(np.asarray(qzeros, dtype=np.uint32), bits, n).astype(np.float64) + (1 if v1_zeros else 0)
    s = bits_to_f64(param_dtype, np.asarray(scale_bits, dtype=np.uint16))
    sg = np.repeat(s.T, group_size, axis=1)
    zg = np.repeat(zeros.T, group_size, axis=1)
    return sg * (codes - zg)


def gptq_planes(bits: int) -> tuple:
    """Plane widths of a GPTQ_P stream, low plane first (GPTQModel "Packing Formats and
    Compatibility", GPTQ_P table: 3 = 2 + 1, 5 = 4 + 1, 6 = 4 + 2, 7 = 4 + 2 + 1, and one plane at
    2, 4 and 8 bits): the powers of two that make up ``bits``, the largest first."""
    assert 2 <= bits <= 8
    return tuple(w for w in (8, 4, 2, 1) if bits & w)


def gptq_planar_codes(words, bits: int, count: int) -> np.ndarray:
    """The first ``count`` codes of each row of GPTQ_P words (GPTQModel "Packing Formats and
    Compatibility", GPTQ_P): every 32 consecutive codes take ``bits`` adjacent words; those words
    hold the planes one after another, low plane first, a plane of width w taking w words whose
    32 w-bit fields are the block's codes in order, least significant field first; the code is
    the low plane's field, plus the next plane's field shifted past it, and so on."""
    w = np.asarray(words, dtype=np.uint32)
    rows = w.shape[0]
    assert count % 32 == 0 and w.shape[1] >= count // 32 * bits
    nb = count // 32
    blocks = w[:, : nb * bits].reshape(rows * nb, bits)
    codes = np.zeros((rows * nb, 32), dtype=np.int64)
    first, shift = 0, 0
    for wp in gptq_planes(bits):
        codes |= _read_stream(blocks[:, first:first + wp], wp, 32) << shift
        first += wp
        shift += wp
    return codes.reshape(rows, count)


def gptq_planar_transcode(qweight, qzeros, scale_bits, bits: int, group_size: int, k: int, n: int,
                          param_dtype: str):
    """GPTQ_P (planar) -> MLX affine rows (GPTQModel "Packing Formats and Compatibility", GPTQ_P:
    the GPTQ tensor names and shapes, qweight [K*b/32, N] with each column's codes as planar blocks
    down the input axis, qzeros [G, N*b/32] with each group's zeros as planar blocks along the
    outputs, zeros always true zero points (never the v1 minus-one form); GPTQModel wiki "MLX Apple
    Silicon", Packed layouts and exact transcoding: scales to [out, groups], additive bias
    -zero*scale, and a 7-bit source kept in 8-bit rows).

    Returns (packed [n, k*tb/32], scales [n, G], biases [n, G]) with tb = 8 for 7-bit sources and
    tb = bits otherwise; biases = RNE(-zero * scale) in param_dtype (exact in fp32 before that)."""
    G = k // group_size
    qweight = np.asarray(qweight, dtype=np.uint32)
    qzeros = np.asarray(qzeros, dtype=np.uint32)
    assert qweight.shape == (k * bits // 32, n) and qzeros.shape == (G, n * bits // 32)
    tb = 8 if bits == 7 else bits
    codes = gptq_planar_codes(qweight.T, bits, k)  # [n, k]
    zeros = gptq_planar_codes(qzeros, bits, n)  # [G, n]
    s = bits_to_f64(param_dtype, np.asarray(scale_bits, dtype=np.uint16))  # [G, n]
    b32 = (-(zeros.astype(np.float64)) * s).astype(np.float32)
    return (pack_codes(codes, tb), np.ascontiguousarray(np.asarray(scale_bits, dtype=np.uint16).T),
            np.ascontiguousarray(to_bits(param_dtype, b32).T))


def gptq_planar_dequant_f64(qweight, qzeros, scale_bits, bits: int, group_size: int, k: int, n: int,
                            param_dtype: str):
    """GPTQ_P's own reconstruction, scale * (code - zero) with true zeros, exactly in fp64: [n, k]."""
    codes = gptq_planar_codes(np.asarray(qweight, dtype=np.uint32).T, bits, k).astype(np.float64)
    zeros = gptq_planar_codes(qzeros, bits, n).astype(np.float64)
    s = bits_to_f64(param_dtype, np.asarray(scale_bits, dtype=np.uint16))
    return np.repeat(s.T, group_size, axis=1) * (codes - np.repeat(zeros.T, group_size, axis=1))


AWQ_LANE_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)


def _read_stream(words, bits: int, count: int) -> np.ndarray:
    """The first ``count`` codes of each row's little-endian ``bits``-wide stream (stream bit j is
    bit j % 32 of word j // 32), for any width 1..8: the words' bits are listed one by one
    (NumPy's unpackbits, least significant bit first over little-endian bytes) and cut into
    codes, bit i of a code weighing 2^i."""
    w = np.ascontiguousarray(np.asarray(words, dtype="<u4"))
    rows = w.shape[0]
    flat = np.unpackbits(w.view(np.uint8).reshape(rows, -1), axis=1, bitorder="little")
    assert flat.shape[1] >= count * bits
    b = flat[:, : count * bits].reshape(rows, count, bits).astype(np.int64)
    return (b << np.arange(bits, dtype=np.int64)).sum(axis=2)


def awq_codes(words, bits: int, count: int) -> np.ndarray:
    """Codes of AWQ GEMM rows packed along the outputs, in natural column order: each row is one
    continuous ``bits``-wide stream; at 4 bits the 8 nibbles of a word hold, from the low nibble
    up, columns 0, 2, 4, 6, 1, 3, 5, 7 of that word's 8 (GPTQModel wiki "MLX Apple Silicon",
    ParoQuant: the AWQ lane order; "Packed layouts and exact transcoding", AWQ GEMM row: the 4-bit
    lane permutation is undone before row packing)."""
    s = _read_stream(words, bits, count)
    if bits != 4:
        return s
    assert count % 8 == 0
    out = np.empty_like(s)
    for slot, col in enumerate(AWQ_LANE_ORDER):
        out[:, col::8] = s[:, slot::8]
    return out


def awq_transcode(qweight, qzeros, scale_bits, bits: int, group_size: int, k: int, n: int, param_dtype: str):
    """AWQ GEMM -> MLX affine rows (GPTQModel wiki "MLX Apple Silicon", Packed layouts and exact
    transcoding, AWQ GEMM and seven-bit rows; GPTQModel "Packing Formats and Compatibility", AWQ
    GEMM: qweight [K, N*b/32] codes packed along the outputs, qzeros [G, N*b/32] true zero points
    packed the same way, scales [G, N] group-major; value scale * (code - zero)).

    Returns (packed [n, k*tb/32], scales [n, G], biases [n, G]) where tb = 8 for 7-bit sources (no
    7-bit affine rows: the code values are kept in 8-bit words) and tb = bits otherwise, and
    biases = RNE(-zero * scale) in param_dtype (exact in fp32 before that rounding)."""
    G = k // group_size
    qweight = np.asarray(qweight, dtype=np.uint32)
    qzeros = np.asarray(qzeros, dtype=np.uint32)
    assert qweight.shape == (k, n * bits // 32) and qzeros.shape == (G, n * bits // 32)
    tb = 8 if bits == 7 else bits
    codes = awq_codes(qweight, bits, n)  # [k, n]
    zeros = awq_codes(qzeros, bits, n)  # [G, n]
    s = bits_to_f64(param_dtype, np.asarray(scale_bits, dtype=np.uint16))  # [G, n]
    b32 = (-(zeros.astype(np.float64)) * s).astype(np.float32)
    return (pack_codes(codes.T, tb), np.ascontiguousarray(np.asarray(scale_bits, dtype=np.uint16).T),
            np.ascontiguousarray(to_bits(param_dtype, b32).T))


def awq_dequant_f64(qweight, qzeros, scale_bits, bits: int, group_size: int, k: int, n: int, param_dtype: str):
    """AWQ's own reconstruction, scale * (code - zero), exactly in fp64: [n, k] (per output row)."""
    codes = awq_codes(qweight, bits, n).astype(np.float64)  # [k, n]
    zeros = awq_codes(qzeros, bits, n).astype(np.float64)  # [G, n]
    s = bits_to_f64(param_dtype, np.asarray(scale_bits, dtype=np.uint16))
    return np.repeat(s.T, group_size, axis=1) * (codes.T - np.repeat(zeros.T, group_size, axis=1))


# --------------------------------------------------------------------------------------
# MXFP4 with its scales apart (Nx_quant "Weights": Mxfp4; OCP Microscaling 2023 E2M1/E8M0).
# --------------------------------------------------------------------------------------

MXFP4_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def mxfp4_dequant_f32(codes_u8, scales_u8) -> np.ndarray:
    """codes [..., n, k/2] (value 2i in byte i's low nibble, 2i+1 in its high nibble) and E8M0
    scales [..., n, k/32] -> fp32 values [..., n, k].

    Code bit 3 is the sign, bits 2..0 index the magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; the value
    is sign * magnitude * 2^(s - 127), rounded to fp32 (exact unless it overflows to inf); the
    scale byte 255 makes its whole block NaN."""
    codes = np.asarray(codes_u8, dtype=np.uint8)
    scales = np.asarray(scales_u8, dtype=np.uint8)
    lead = codes.shape[:-1]
    k = codes.shape[-1] * 2
    assert scales.shape == lead + (k // 32,)
    nib = np.empty(lead + (k,), dtype=np.int64)
    nib[..., 0::2] = codes & 0x0F
    nib[..., 1::2] = codes >> 4
    mag = np.asarray(MXFP4_MAGNITUDES, dtype=np.float64)[nib & 7]
    sign = np.where(nib & 8, -1.0, 1.0)
    sc = np.repeat(scales.astype(np.int64), 32, axis=-1)
    with np.errstate(over="ignore", invalid="ignore"):
        val = sign * np.ldexp(mag, sc - 127)
        val = np.where(sc == 255, np.nan, val)
        return val.astype(np.float32)


# --------------------------------------------------------------------------------------
# Q8_0 blocks (Nx_quant "Weights": Q8_0; quantize_q8_0).
# --------------------------------------------------------------------------------------


def q8_0_dequant_f32(blocks_u8) -> np.ndarray:
    """blocks [..., n, k/32*34]: per 32 values a little-endian fp16 scale d then 32 int8 quants;
    value = d * q, exact in fp32."""
    b = np.asarray(blocks_u8, dtype=np.uint8)
    lead = b.shape[:-1]
    assert b.shape[-1] % 34 == 0
    nb = b.shape[-1] // 34
    blk = b.reshape(lead + (nb, 34))
    d_bits = blk[..., 0].astype(np.uint16) | (blk[..., 1].astype(np.uint16) << np.uint16(8))
    d = f16_bits_to_f32(d_bits).astype(np.float64)
    q = blk[..., 2:].view(np.int8).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return (d[..., None] * q).astype(np.float32).reshape(lead + (nb * 32,))


# --------------------------------------------------------------------------------------
# Q4_K and Q6_K (Nx_quant "Weights": per 256 values one block of 144 / 210 bytes in the layout of
# ggml's block_q4_K / block_q6_K; the value formulas and the rounding rule are the page's, the
# placement of the sub-fields inside the scale and quant bytes is a reading (below).
# --------------------------------------------------------------------------------------

Q4_K_BYTES, Q6_K_BYTES = 144, 210


def _q4_k_fields():
    """Index tables of the Q4_K reading: for value v of a block (0..255) the qs byte that holds its
    quant (16 + 32 (v // 64) + v % 32) and the nibble (low for v % 64 < 32, high otherwise); its
    sub-block is v // 32.  Sub-block j's 6-bit scale and min: for j < 4 the low 6 bits of scale
    bytes j and j + 4; for j >= 4 the scale is the low nibble of byte j + 4 with the top two bits of
    byte j - 4 above it, the min the high nibble of byte j + 4 with the top two bits of byte j."""
    v = np.arange(256)
    qbyte = 16 + 32 * (v // 64) + v % 32
    shift = 4 * ((v % 64) // 32)
    return qbyte, shift


def _q4_k_scale_min(sb):
    """(sc, m) [..., 8] from the 12 scale bytes [..., 12] (see _q4_k_fields)."""
    sb = sb.astype(np.int64)
    sc = np.empty(sb.shape[:-1] + (8,), dtype=np.int64)
    mn = np.empty_like(sc)
    for j in range(4):
        sc[..., j] = sb[..., j] & 63
        mn[..., j] = sb[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (sb[..., j + 4] & 15) | ((sb[..., j - 4] >> 6) << 4)
        mn[..., j] = (sb[..., j + 4] >> 4) | ((sb[..., j] >> 6) << 4)
    return sc, mn


def q4_k_dequant_f32(blocks_u8) -> np.ndarray:
    """blocks [..., n, k/256*144] -> values [..., n, k] (fp32).  Per block: little-endian fp16 d and
    dmin, 12 bytes of 6-bit scales and mins of the 8 sub-blocks of 32 values, 128 bytes of 4-bit
    quants (placement: _q4_k_fields).  value = d*sc*q - dmin*m (Nx_quant "Weights", Q4_K), its
    products exact and one rounding at the subtraction (Nx_quant, the float32 rule for GGUF values).

    Evaluated in fp64 and rounded once to fp32: d*sc*q and dmin*m have at most 21 significant bits;
    when their difference needs more than 53 bits, the smaller is below 2^-32 of the larger, so the
    exact difference and its fp64 rounding lie within a quarter ulp of the larger term, an fp32 value,
    and both round to it."""
    b = np.asarray(blocks_u8, dtype=np.uint8)
    lead = b.shape[:-1]
    assert b.shape[-1] % Q4_K_BYTES == 0
    nb = b.shape[-1] // Q4_K_BYTES
    blk = b.reshape(lead + (nb, Q4_K_BYTES))
    d = f16_bits_to_f32(blk[..., 0].astype(np.uint16) | (blk[..., 1].astype(np.uint16) << np.uint16(8))).astype(np.float64)
    dmin = f16_bits_to_f32(blk[..., 2].astype(np.uint16) | (blk[..., 3].astype(np.uint16) << np.uint16(8))).astype(np.float64)
    sc, mn = _q4_k_scale_min(blk[..., 4:16])
    qbyte, shift = _q4_k_fields()
    q = (blk[..., qbyte].astype(np.int64) >> shift) & 15  # [..., nb, 256]
    sub = np.arange(256) // 32
    with np.errstate(invalid="ignore"):
        a = (d[..., None] * sc[..., sub]) * q  # exact
        m = dmin[..., None] * mn[..., sub]  # exact
        return (a - m).astype(np.float32).reshape(lead + (nb * 256,))


def _q6_k_fields():
    """Index tables of the Q6_K reading: value v of a block (0..255), with h = v // 128, w = v % 128,
    g = w // 32, l = w % 32, takes its low 4 bits from ql byte 64 h + 32 (g % 2) + l (low nibble for
    g < 2, high for g >= 2) and its high 2 bits from bits 2g, 2g + 1 of qh byte 128 + 32 h + l; its
    sub-block (scale byte 192 + v // 16) is v // 16."""
    v = np.arange(256)
    h, w = v // 128, v % 128
    g, l = w // 32, w % 32
    lo_byte = 64 * h + 32 * (g % 2) + l
    lo_shift = 4 * (g // 2)
    hi_byte = 128 + 32 * h + l
    hi_shift = 2 * g
    return lo_byte, lo_shift, hi_byte, hi_shift


def q6_k_dequant_f32(blocks_u8) -> np.ndarray:
    """blocks [..., n, k/256*210] -> values [..., n, k] (fp32).  Per block: 128 bytes of the quants'
    low 4 bits, 64 of their high 2 bits, an int8 scale per sub-block of 16 values, a little-endian
    fp16 d (placement: _q6_k_fields).  value = d*sc*(q - 32) (Nx_quant "Weights", Q6_K), exact in
    fp32: d has at most 11 significant bits, |sc| <= 128 and |q - 32| <= 32, and 2047 * 128 * 32 is
    below 2^24.  An all-zero block gives -0 (0 * -32)."""
    b = np.asarray(blocks_u8, dtype=np.uint8)
    lead = b.shape[:-1]
    assert b.shape[-1] % Q6_K_BYTES == 0
    nb = b.shape[-1] // Q6_K_BYTES
    blk = b.reshape(lead + (nb, Q6_K_BYTES))
    d = f16_bits_to_f32(blk[..., 208].astype(np.uint16) | (blk[..., 209].astype(np.uint16) << np.uint16(8))).astype(np.float64)
    sc = blk[..., 192:208].view(np.int8).astype(np.float64)  # [..., nb, 16]
    lo_byte, lo_shift, hi_byte, hi_shift = _q6_k_fields()
    q = ((blk[..., lo_byte].astype(np.int64) >> lo_shift) & 15) | (((blk[..., hi_byte].astype(np.int64) >> hi_shift) & 3) << 4)
    sub = np.arange(256) // 16
    with np.errstate(invalid="ignore"):
        return ((d[..., None] * sc[..., sub]) * (q - 32)).astype(np.float32).reshape(lead + (nb * 256,))


def q8_0_quantize(w_f32) -> np.ndarray:
    """quantize_q8_0 (Nx_quant API docs, quantize_q8_0): fp32 [..., n, k] -> blocks [..., n, k/32*34].

    Per block of 32 values: d = amax/127 in fp32, stored as fp16 (nearest, so past fp16's largest
    it is +inf); quants are v * (1/d) in fp32 rounded half away from zero, with 1/d taken from the
    fp32 d.  Non-finite rules of the page: a block whose d is 0 or whose 1/d is infinite is all
    zero bytes; a block holding an infinity (and no NaN) has d = +inf and quants 0; a block
    holding a NaN has d = NaN (fp16 0x7E00) and quants 0."""
    w = np.asarray(w_f32, dtype=np.float32)
    lead = w.shape[:-1]
    k = w.shape[-1]
    assert k % 32 == 0
    v = w.reshape(lead + (k // 32, 32))
    has_nan = np.isnan(v).any(axis=-1)
    has_inf = np.isinf(v).any(axis=-1) & ~has_nan
    finite = ~(has_nan | has_inf)
    vf = np.where(finite[..., None], v, np.float32(0.0))
    amax = np.abs(vf).max(axis=-1).astype(np.float32)
    d = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        inv = np.where(d == 0, np.float32(0.0), (np.float32(1.0) / d)).astype(np.float32)
    zero_blk = finite & ((d == 0) | np.isinf(inv))
    inv = np.where(zero_blk | ~finite, np.float32(0.0), inv)
    prod = (vf * inv[..., None]).astype(np.float32).astype(np.float64)
    q = (np.sign(prod) * np.floor(np.abs(prod) + 0.5)).astype(np.int64)
    q = np.where((zero_blk | ~finite)[..., None], 0, q)
    assert q.min(initial=0) >= -128 and q.max(initial=0) <= 127
    with np.errstate(over="ignore"):
        d_bits = f32_to_f16_bits(d).astype(np.uint16)
    d_bits = np.where(zero_blk, np.uint16(0), d_bits)
    d_bits = np.where(has_inf, np.uint16(0x7C00), d_bits)
    d_bits = np.where(has_nan, np.uint16(0x7E00), d_bits).astype(np.uint16)
    out = np.empty(lead + (k // 32, 34), dtype=np.uint8)
    out[..., 0] = (d_bits & 0xFF).astype(np.uint8)
    out[..., 1] = (d_bits >> 8).astype(np.uint8)
    out[..., 2:] = q.astype(np.int8).view(np.uint8)
    return out.reshape(lead + (k // 32 * 34,))


def mxfp4_blocks_dequant_f32(blocks_u8) -> np.ndarray:
    """MXFP4 in GGUF's blocks (Nx_quant API docs, Weights: Mxfp4_blocks): [..., n, k/32*17] ->
    fp32 [..., n, k].  Per 32 values: the E8M0 scale byte, then 16 bytes, byte j holding value j
    in its low nibble and value j + 16 in its high one; values decode as in the split layout."""
    b = np.asarray(blocks_u8, dtype=np.uint8)
    lead = b.shape[:-1]
    assert b.shape[-1] % 17 == 0
    nb = b.shape[-1] // 17
    blk = b.reshape(lead + (nb, 17))
    scales = blk[..., 0]
    body = blk[..., 1:]
    nib = np.concatenate([body & 0x0F, body >> 4], axis=-1).astype(np.int64)  # values 0..15, 16..31
    mag = np.asarray(MXFP4_MAGNITUDES, dtype=np.float64)[nib & 7]
    sign = np.where(nib & 8, -1.0, 1.0)
    sc = scales.astype(np.int64)[..., None]
    with np.errstate(over="ignore", invalid="ignore"):
        val = sign * np.ldexp(mag, sc - 127)
        val = np.where(sc == 255, np.nan, val)
        return val.astype(np.float32).reshape(lead + (nb * 32,))


def take(pos, src) -> np.ndarray:
    """take (Nx_quant API docs): the rows (first axis) of a packed part at positions `pos`, bytes
    copied with no value decoded; a position outside [0, rows) gives a zero row."""
    src = np.asarray(src)
    pos = np.asarray(pos, dtype=np.int64)
    out = np.zeros((pos.shape[0],) + src.shape[1:], dtype=src.dtype)
    ok = (pos >= 0) & (pos < src.shape[0])
    out[ok] = src[pos[ok]]
    return out


# --------------------------------------------------------------------------------------
# Routing and apply_experts (Nx_quant "Products": apply_experts).
# --------------------------------------------------------------------------------------


def route(ids, e: int):
    """Group positions by expert: returns (offsets int32 [e+1], perm int32 [offsets[e]]).

    Positions p with 0 <= ids[p] < e are listed expert by expert, each expert's positions in
    increasing p (a stable counting sort); positions out of range are dropped."""
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    offsets = np.zeros(e + 1, dtype=np.int64)
    buckets = [[] for _ in range(e)]
    for p, i in enumerate(ids.tolist()):
        if 0 <= i < e:
            buckets[i].append(p)
    for j in range(e):
        offsets[j + 1] = offsets[j] + len(buckets[j])
    perm = np.array([p for bkt in buckets for p in bkt], dtype=np.int64)
    return offsets.astype(np.int32), perm.astype(np.int32)


def apply_experts(w_values_e, ids, x_f64, pos_per_row: int = 1) -> np.ndarray:
    """y[p, :] = x[p // pos_per_row] . W_{ids[p]}^T in fp64, zeros where ids[p] is not in [0, e).

    ``w_values_e`` is [e, n, k] (the experts' dequantized fp32 values), ``ids`` [P] and ``x`` is
    [P / pos_per_row, k]; the x row of a position is shared by ``pos_per_row`` consecutive
    positions (a token's top-k slots)."""
    w = np.asarray(w_values_e)
    e, n, k = w.shape
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    x = np.asarray(x_f64, dtype=np.float64)
    y = np.zeros((ids.size, n), dtype=np.float64)
    for j in range(e):
        pos = np.nonzero(ids == j)[0]
        if pos.size:
            y[pos] = x[pos // pos_per_row] @ w[j].astype(np.float64).T
    return y


def rel_l2_per_row(y, ref) -> np.ndarray:
    """||y - ref||_2 / ||ref||_2 for each row (rows whose reference is all zero use 1 as norm)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(((y - ref) ** 2).sum(axis=-1))
    den = np.sqrt((ref ** 2).sum(axis=-1))
    return num / np.where(den == 0, 1.0, den)
