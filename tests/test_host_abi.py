"""C-ABI checks that need no GPU: the library loads, exports every entry point the header
declares, and rejects bad arguments on the host before any launch (no compute call here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import weight_only_quantized_affine_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlinear.h")

QL_OK, QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_DTYPE, QL_ERR_ALIGN, QL_ERR_UNSUPPORTED, QL_ERR_WORKSPACE = range(7)
F32, F16, BF16 = 0, 1, 2
FAKE = 0x100000  # a 16-byte aligned non-NULL address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q.lib_path()):
        import __graft_entry__

        __graft_entry__.build()
    return q.load_library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S[^;(]*?\b(qlinear_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for want in ["qlinear_quantize", "qlinear_dequant", "qlinear_gemv", "qlinear_gemm", "qlinear_gemv_batched",
                 "qlinear_route", "qlinear_apply_experts", "qlinear_last_error"]:
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_library_exports_no_torch_types():
    # the boundary is plain C: no C++ mangled names among the qlinear_ symbols
    out = os.popen(f"nm -D --defined-only {q.lib_path()}").read()
    syms = [ln.split()[-1] for ln in out.splitlines() if ln.strip()]
    assert all(not s.startswith("_Z") for s in syms if "qlinear" in s)
    assert set(_declared()) <= set(syms)


def _err(lib):
    return lib.qlinear_last_error().decode()


def test_quantize_rejects_bad_arguments(lib):
    assert lib.qlinear_quantize(None, 4, 64, 4, 64, BF16, None, None, None, None) == QL_ERR_NULL
    assert "must not be NULL" in _err(lib)
    assert lib.qlinear_quantize(FAKE, 4, 64, 7, 64, BF16, FAKE, FAKE, FAKE, None) == QL_ERR_UNSUPPORTED
    assert "bits=7" in _err(lib)
    assert lib.qlinear_quantize(FAKE, 4, 64, 1, 64, BF16, FAKE, FAKE, FAKE, None) == QL_ERR_UNSUPPORTED
    assert lib.qlinear_quantize(FAKE, 4, 64, 4, 48, BF16, FAKE, FAKE, FAKE, None) == QL_ERR_UNSUPPORTED
    assert lib.qlinear_quantize(FAKE, 4, 96, 4, 64, BF16, FAKE, FAKE, FAKE, None) == QL_ERR_SHAPE
    assert lib.qlinear_quantize(FAKE, 4, 48, 4, 32, BF16, FAKE, FAKE, FAKE, None) == QL_ERR_SHAPE  # k % 32
    assert lib.qlinear_quantize(FAKE, -1, 64, 4, 64, BF16, FAKE, FAKE, FAKE, None) == QL_ERR_SHAPE
    assert lib.qlinear_quantize(FAKE, 4, 64, 4, 64, F32, FAKE, FAKE, FAKE, None) == QL_ERR_DTYPE
    assert lib.qlinear_quantize(FAKE + 4, 4, 64, 4, 64, BF16, FAKE, FAKE, FAKE, None) == QL_ERR_ALIGN
    assert lib.qlinear_quantize(FAKE, 4, 64, 4, 64, BF16, FAKE, FAKE + 1, FAKE, None) == QL_ERR_ALIGN
    # zero-size: OK without a launch
    assert lib.qlinear_quantize(None, 0, 64, 4, 64, BF16, None, None, None, None) == QL_OK
    assert _err(lib) == ""


def test_dequant_rejects_bad_arguments(lib):
    assert lib.qlinear_dequant(7, FAKE, FAKE, FAKE, BF16, 4, 64, 4, 64, FAKE, F32, None) == QL_ERR_UNSUPPORTED
    assert lib.qlinear_dequant(0, FAKE, FAKE, None, BF16, 4, 64, 4, 64, FAKE, F32, None) == QL_ERR_NULL
    assert lib.qlinear_dequant(0, FAKE, FAKE, FAKE, BF16, 4, 64, 4, 64, FAKE, 9, None) == QL_ERR_DTYPE
    assert lib.qlinear_dequant(1, FAKE, FAKE, FAKE, BF16, 4, 64, 0, 0, FAKE, F32, None) == QL_ERR_SHAPE  # w2 set
    assert lib.qlinear_dequant(1, FAKE, FAKE, None, BF16, 4, 48, 0, 0, FAKE, F32, None) == QL_ERR_SHAPE
    assert lib.qlinear_dequant(1, FAKE + 8, FAKE, None, BF16, 4, 64, 0, 0, FAKE, F32, None) == QL_ERR_ALIGN
    assert lib.qlinear_dequant(2, FAKE, FAKE, None, BF16, 4, 64, 0, 0, FAKE, F32, None) == QL_ERR_SHAPE  # w1 set
    assert lib.qlinear_dequant(2, FAKE + 1, None, None, BF16, 4, 64, 0, 0, FAKE, F32, None) == QL_ERR_ALIGN
    assert lib.qlinear_dequant(2, None, None, None, BF16, 0, 64, 0, 0, None, F32, None) == QL_OK


def _gemv_args(**kw):
    a = dict(x=FAKE, xdt=BF16, m=1, k=1024, packed=FAKE, scales=FAKE, biases=FAKE, pdt=BF16, n=256, bits=4, g=64,
             lb=None, y=FAKE, ydt=F32, s=None)
    a.update(kw)
    return [a[k] for k in ["x", "xdt", "m", "k", "packed", "scales", "biases", "pdt", "n", "bits", "g", "lb", "y",
                           "ydt", "s"]]


def test_gemv_rejects_bad_arguments(lib):
    assert lib.qlinear_gemv(*_gemv_args(x=None)) == QL_ERR_NULL
    assert lib.qlinear_gemv(*_gemv_args(y=None)) == QL_ERR_NULL
    assert lib.qlinear_gemv(*_gemv_args(xdt=F32)) == QL_ERR_DTYPE
    assert lib.qlinear_gemv(*_gemv_args(ydt=5)) == QL_ERR_DTYPE
    assert lib.qlinear_gemv(*_gemv_args(bits=7)) == QL_ERR_UNSUPPORTED
    assert lib.qlinear_gemv(*_gemv_args(bits=3, x=None)) == QL_ERR_NULL  # 3 bits passes the width check
    assert lib.qlinear_gemv(*_gemv_args(k=1000)) == QL_ERR_SHAPE
    assert lib.qlinear_gemv(*_gemv_args(m=-2)) == QL_ERR_SHAPE
    assert lib.qlinear_gemv(*_gemv_args(x=FAKE + 2)) == QL_ERR_ALIGN
    assert lib.qlinear_gemv(*_gemv_args(packed=FAKE + 4)) == QL_ERR_ALIGN
    assert lib.qlinear_gemv(*_gemv_args(ydt=F32, y=FAKE + 2)) == QL_ERR_ALIGN
    assert lib.qlinear_gemv(*_gemv_args(m=0, x=None, y=None)) == QL_OK
    assert lib.qlinear_gemv(*_gemv_args(n=0, x=None, y=None, packed=None)) == QL_OK


def test_gemm_rejects_missing_or_small_workspace(lib):
    need = lib.qlinear_gemm_workspace_size(2048, 4096, 4096, 4, 64)
    # fp16 copy of x, its row factors, the weight records (s, c) and row factors (each padded to
    # 256 bytes)
    assert need == 2048 * 4096 * 2 + 2048 * 4 + 4096 * 64 * 8 + 4096 * 4
    args = _gemv_args(m=2048, k=4096, n=4096)
    assert lib.qlinear_gemm(*args[:-1], None, 0, None) == QL_ERR_WORKSPACE
    assert lib.qlinear_gemm(*args[:-1], FAKE, need - 1, None) == QL_ERR_WORKSPACE
    assert "smaller" in _err(lib)
    assert lib.qlinear_gemm(*args[:-1], FAKE + 4, need, None) == QL_ERR_ALIGN
    assert lib.qlinear_gemm(*_gemv_args(bits=7)[:-1], FAKE, need, None) == QL_ERR_UNSUPPORTED
    # bitstream widths also hold the codes as bytes: the 4-bit workspace is too small (checked
    # before any launch)
    need5 = lib.qlinear_gemm_workspace_size(2048, 4096, 4096, 5, 64)
    assert need5 == need + 4096 * 4096
    assert lib.qlinear_gemm(*_gemv_args(m=2048, k=4096, n=4096, bits=5)[:-1], FAKE, need, None) == QL_ERR_WORKSPACE


def test_gemv_batched_validates_every_problem(lib):
    P = q._Problem
    good = P(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 256, 1024, 4, 64)
    bad = P(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 256, 1000, 4, 64)
    arr = (P * 2)(good, bad)
    need = lib.qlinear_gemv_batched_workspace_size((P * 2)(good, good), 2)
    assert need > 2 * ctypes.sizeof(P)
    assert lib.qlinear_gemv_batched(arr, 2, BF16, BF16, F32, FAKE, need, 1, None) == QL_ERR_SHAPE
    assert "problem 1" in _err(lib)
    big_m = P(FAKE, FAKE, FAKE, FAKE, None, FAKE, 9, 256, 1024, 4, 64)
    arr = (P * 2)(good, big_m)
    assert lib.qlinear_gemv_batched(arr, 2, BF16, BF16, F32, FAKE, need, 1, None) == QL_ERR_UNSUPPORTED
    # a 3-bit problem with k % 128 != 0 needs no table entry: the workspace is the same as without it
    stream_bits = P(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 256, 1056, 3, 32)
    assert lib.qlinear_gemv_batched_workspace_size((P * 2)(good, stream_bits), 2) == \
        lib.qlinear_gemv_batched_workspace_size((P * 1)(good), 1)
    arr = (P * 2)(good, good)
    assert lib.qlinear_gemv_batched(arr, 2, BF16, BF16, F32, FAKE, need - 1, 1, None) == QL_ERR_WORKSPACE
    assert lib.qlinear_gemv_batched(arr, 0, BF16, BF16, F32, None, 0, 1, None) == QL_OK


def test_route_and_experts_reject_bad_arguments(lib):
    assert lib.qlinear_route(FAKE, 16, 0, FAKE, FAKE, None) == QL_ERR_SHAPE
    assert lib.qlinear_route(FAKE, 16, 5000, FAKE, FAKE, None) == QL_ERR_SHAPE
    assert lib.qlinear_route(FAKE + 4, 16, 4, FAKE, FAKE, None) == QL_ERR_ALIGN
    assert lib.qlinear_route(FAKE, 16, 4, None, FAKE, None) == QL_ERR_NULL
    ws = lib.qlinear_apply_experts_workspace_size(2048, 32)
    assert ws >= 33 * 4 + 2048 * 4 + 32 * 4
    base = [1, FAKE, FAKE, 32, 5760, 2880, FAKE, 2048, FAKE, BF16, 4, FAKE, BF16, FAKE, ws, None]

    def call(**kw):
        a = list(base)
        names = ["fmt", "w0", "w1", "e", "n", "k", "ids", "n_pos", "x", "xdt", "ppr", "y", "ydt", "ws", "wsb", "s"]
        for key, v in kw.items():
            a[names.index(key)] = v
        return lib.qlinear_apply_experts(*a)

    assert call(fmt=0) == QL_ERR_UNSUPPORTED
    assert call(fmt=3) == QL_ERR_SHAPE  # MXFP4 in GGUF blocks takes no w1
    assert call(xdt=F32) == QL_ERR_DTYPE  # x is bf16 or fp16
    assert call(k=2881) == QL_ERR_SHAPE
    assert call(ppr=3) == QL_ERR_SHAPE
    assert call(wsb=ws - 1) == QL_ERR_WORKSPACE
    assert call(w1=None) == QL_ERR_NULL
    assert call(fmt=2) == QL_ERR_SHAPE  # Q8_0 takes no w1
    assert call(fmt=2, w1=None, w0=FAKE + 1) == QL_ERR_ALIGN
    assert call(n_pos=0) == QL_OK
    # Q4_K / Q6_K: k a multiple of 256, no w1, Q4_K blocks 16-byte aligned
    assert call(fmt=4, w1=None) == QL_ERR_SHAPE  # k = 2880 is not a multiple of 256
    assert call(fmt=5, w1=None, k=2816, w0=FAKE + 1) == QL_ERR_ALIGN
    assert call(fmt=4, w1=None, k=2816, w0=FAKE + 2) == QL_ERR_ALIGN
    assert call(fmt=4, k=2816) == QL_ERR_SHAPE  # w1 given
    assert call(fmt=6) == QL_ERR_UNSUPPORTED


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(q, "_LIB", None)
    monkeypatch.setattr(q, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        q.load_library()


def test_quantize_q8_0_take_and_blocks_reject_bad_arguments(lib):
    assert lib.qlinear_quantize_q8_0(FAKE, 4, 48, FAKE, None) == QL_ERR_SHAPE  # k % 32
    assert lib.qlinear_quantize_q8_0(None, 4, 64, FAKE, None) == QL_ERR_NULL
    assert lib.qlinear_quantize_q8_0(FAKE + 4, 4, 64, FAKE, None) == QL_ERR_ALIGN
    assert lib.qlinear_quantize_q8_0(FAKE, 4, 64, FAKE + 1, None) == QL_ERR_ALIGN
    assert lib.qlinear_quantize_q8_0(None, 0, 64, None, None) == QL_OK
    assert lib.qlinear_take(FAKE, -1, FAKE, 4, 16, FAKE, None) == QL_ERR_SHAPE
    assert lib.qlinear_take(None, 4, FAKE, 4, 16, FAKE, None) == QL_ERR_NULL
    assert lib.qlinear_take(FAKE, 4, None, 4, 16, FAKE, None) == QL_ERR_NULL
    assert lib.qlinear_take(FAKE + 4, 4, FAKE, 4, 16, FAKE, None) == QL_ERR_ALIGN
    assert lib.qlinear_take(None, 0, None, 0, 16, None, None) == QL_OK
    assert lib.qlinear_take(FAKE, 4, FAKE, 4, 0, FAKE, None) == QL_OK  # empty rows: nothing to copy
    # MXFP4 in GGUF blocks: one part only
    assert lib.qlinear_dequant(3, FAKE, FAKE, None, BF16, 4, 64, 0, 0, FAKE, F32, None) == QL_ERR_SHAPE
    assert lib.qlinear_dequant(3, FAKE, None, None, BF16, 4, 48, 0, 0, FAKE, F32, None) == QL_ERR_SHAPE
    assert lib.qlinear_dequant(3, FAKE, None, None, BF16, 4, 64, 0, 0, FAKE + 2, F32, None) == QL_ERR_ALIGN
    assert lib.qlinear_dequant(3, None, None, None, BF16, 0, 64, 0, 0, None, F32, None) == QL_OK
    assert lib.qlinear_dequant(6, FAKE, None, None, BF16, 4, 64, 0, 0, FAKE, F32, None) == QL_ERR_UNSUPPORTED
    # Q4_K / Q6_K: k a multiple of 256, one part, Q4_K blocks 16-byte aligned, Q6_K 2-byte
    for fmt in (4, 5):
        assert lib.qlinear_dequant(fmt, FAKE, None, None, BF16, 4, 384, 0, 0, FAKE, F32, None) == QL_ERR_SHAPE
        assert lib.qlinear_dequant(fmt, FAKE, FAKE, None, BF16, 4, 256, 0, 0, FAKE, F32, None) == QL_ERR_SHAPE
        assert lib.qlinear_dequant(fmt, None, None, None, BF16, 4, 256, 0, 0, FAKE, F32, None) == QL_ERR_NULL
        assert lib.qlinear_dequant(fmt, FAKE, None, None, BF16, 4, 256, 0, 0, FAKE + 8, F32, None) == QL_ERR_ALIGN
        assert lib.qlinear_dequant(fmt, None, None, None, BF16, 0, 256, 0, 0, None, F32, None) == QL_OK
    assert lib.qlinear_dequant(4, FAKE + 2, None, None, BF16, 4, 256, 0, 0, FAKE, F32, None) == QL_ERR_ALIGN
    assert lib.qlinear_dequant(5, FAKE + 1, None, None, BF16, 4, 256, 0, 0, FAKE, F32, None) == QL_ERR_ALIGN


def test_transcode_gptq_rejects_bad_arguments(lib):
    args = [FAKE, FAKE, FAKE, F16, 256, 64, 4, 64, 0, FAKE, FAKE, FAKE, None]

    def call(**kw):
        a = list(args)
        names = ["qw", "qz", "sc", "sdt", "k", "n", "bits", "g", "v1", "pk", "so", "bo", "s"]
        for key, v in kw.items():
            a[names.index(key)] = v
        return lib.qlinear_transcode_gptq(*a)

    assert call(bits=5) == QL_ERR_UNSUPPORTED
    assert call(g=16) == QL_ERR_UNSUPPORTED
    assert call(k=250) == QL_ERR_SHAPE
    assert call(bits=3, n=60) == QL_ERR_SHAPE  # 180 bits: qzeros rows would not fill words
    assert call(sdt=F32) == QL_ERR_DTYPE
    assert call(qw=None) == QL_ERR_NULL
    assert call(qz=FAKE + 2) == QL_ERR_ALIGN
    assert call(so=FAKE + 1) == QL_ERR_ALIGN
    assert call(k=0) == QL_OK


def test_transcode_awq_rejects_bad_arguments(lib):
    args = [FAKE, FAKE, FAKE, F16, 256, 64, 4, 64, FAKE, FAKE, FAKE, None]

    def call(**kw):
        a = list(args)
        names = ["qw", "qz", "sc", "sdt", "k", "n", "bits", "g", "pk", "so", "bo", "s"]
        for key, v in kw.items():
            a[names.index(key)] = v
        return lib.qlinear_transcode_awq(*a)

    assert call(bits=1) == QL_ERR_UNSUPPORTED
    assert call(bits=9) == QL_ERR_UNSUPPORTED
    assert call(g=16) == QL_ERR_UNSUPPORTED
    assert call(k=250) == QL_ERR_SHAPE
    assert call(k=96, g=64) == QL_ERR_SHAPE  # k not a multiple of the group
    assert call(n=48) == QL_ERR_SHAPE  # n must be a multiple of 32
    assert call(sdt=F32) == QL_ERR_DTYPE
    assert call(qz=None) == QL_ERR_NULL
    assert call(qw=FAKE + 2) == QL_ERR_ALIGN
    assert call(bo=FAKE + 1) == QL_ERR_ALIGN
    assert call(n=0) == QL_OK


def test_transcode_gptq_planar_rejects_bad_arguments(lib):
    args = [FAKE, FAKE, FAKE, F16, 256, 64, 5, 64, FAKE, FAKE, FAKE, None]

    def call(**kw):
        a = list(args)
        names = ["qw", "qz", "sc", "sdt", "k", "n", "bits", "g", "pk", "so", "bo", "s"]
        for key, v in kw.items():
            a[names.index(key)] = v
        return lib.qlinear_transcode_gptq_planar(*a)

    assert call(bits=1) == QL_ERR_UNSUPPORTED
    assert call(bits=9) == QL_ERR_UNSUPPORTED
    assert call(g=16) == QL_ERR_UNSUPPORTED
    assert call(k=250) == QL_ERR_SHAPE
    assert call(k=96, g=64) == QL_ERR_SHAPE
    assert call(n=48) == QL_ERR_SHAPE  # zeros come in planar blocks of 32 columns
    assert call(sdt=F32) == QL_ERR_DTYPE
    assert call(qw=None) == QL_ERR_NULL
    assert call(pk=FAKE + 2) == QL_ERR_ALIGN
    assert call(sc=FAKE + 1) == QL_ERR_ALIGN
    assert call(k=0) == QL_OK


def test_gptq_g_idx_check_on_host(lib):
    """The exact affine form needs g_idx == arange(k) // group_size (GPTQModel "Packing Formats and
    Compatibility": GPTQ holders require it; activation order is not dropped silently)."""
    k, g = 512, 128
    ok = np.ascontiguousarray(np.arange(k, dtype=np.int32) // g)
    assert lib.qlinear_gptq_check_g_idx(ok.ctypes.data, k, g) == QL_OK
    perm = ok.copy()
    perm[[3, 300]] = perm[[300, 3]]  # two inputs of different groups swapped: an activation order
    assert lib.qlinear_gptq_check_g_idx(perm.ctypes.data, k, g) == QL_ERR_UNSUPPORTED
    assert "g_idx[3]" in _err(lib)
    assert lib.qlinear_gptq_check_g_idx(ok.ctypes.data, k, 64) == QL_ERR_UNSUPPORTED  # another group size
    assert lib.qlinear_gptq_check_g_idx(None, k, g) == QL_ERR_NULL
    assert lib.qlinear_gptq_check_g_idx(None, 0, g) == QL_OK
    assert lib.qlinear_gptq_check_g_idx(ok.ctypes.data, k, 0) == QL_ERR_UNSUPPORTED
    with pytest.raises(q.QLError):
        q.qlinear_gptq_check_g_idx(perm, g)
    q.qlinear_gptq_check_g_idx(ok, g)


def test_apply_experts_noalloc_rejects_sizes_past_its_scratch(lib):
    # 100,000 positions need 12 bytes each of routing scratch: past the 1 MiB built-in array
    st = lib.qlinear_apply_experts_noalloc(1, FAKE, FAKE, 32, 64, 64, FAKE, 100_000, FAKE, BF16, 1, FAKE, BF16, None)
    assert st == QL_ERR_UNSUPPORTED
    assert "scratch" in _err(lib)
    assert lib.qlinear_apply_experts_noalloc(1, FAKE, FAKE, -1, 64, 64, FAKE, 4, FAKE, BF16, 1, FAKE, BF16,
                                             None) == QL_ERR_SHAPE


def test_gemm_grouped_rejects_bad_arguments(lib):
    W = q._GemmWeight
    arr = (W * 5)()
    for i in range(5):
        arr[i] = W(FAKE, FAKE, FAKE, None, FAKE, 64)
    assert lib.qlinear_gemm_grouped(FAKE, BF16, 8, 64, arr, 5, BF16, 4, 64, F32, FAKE, 1 << 20, None) == QL_ERR_SHAPE
    assert "count=5" in _err(lib)
    arr[1] = W(FAKE, FAKE, FAKE, None, FAKE, -1)
    assert lib.qlinear_gemm_grouped(FAKE, BF16, 8, 64, arr, 2, BF16, 4, 64, F32, FAKE, 1 << 20, None) == QL_ERR_SHAPE
    assert "weight 1" in _err(lib)
    arr[1] = W(FAKE, FAKE, FAKE, None, FAKE, 64)
    assert lib.qlinear_gemm_grouped(FAKE, BF16, 8, 64, arr, 2, BF16, 7, 64, F32, FAKE, 1 << 20, None) == QL_ERR_UNSUPPORTED
    assert lib.qlinear_gemm_grouped(FAKE, BF16, 8, 64, arr, 2, BF16, 4, 64, F32, None, 0, None) == QL_ERR_WORKSPACE
    assert lib.qlinear_gemm_grouped(FAKE, BF16, 0, 64, arr, 2, BF16, 4, 64, F32, None, 0, None) == QL_OK
    assert lib.qlinear_gemm_grouped(None, BF16, 8, 64, None, 0, BF16, 4, 64, F32, None, 0, None) == QL_OK


def test_gemm_grouped_workspace_at_bitstream_widths(lib):
    """With enough tiles for one launch over all weights, the grouped call at 2, 3, 5 and 6 bits
    holds every weight's codes as bytes after the 8-bit launch's own workspace; with too few it
    runs qlinear_gemm per weight and needs the largest single call's workspace."""
    W = q._GemmWeight
    m, k, ns = 2048, 4096, (4096, 1024, 1024)
    arr = (W * 3)(*[W(FAKE, FAKE, FAKE, None, FAKE, n) for n in ns])
    need8 = lib.qlinear_gemm_grouped_workspace_size(m, k, arr, 3, 8, 64)
    for bits in (2, 3, 5, 6):
        need = lib.qlinear_gemm_grouped_workspace_size(m, k, arr, 3, bits, 64)
        assert need == need8 + sum(n * k for n in ns), bits
    small = (W * 2)(W(FAKE, FAKE, FAKE, None, FAKE, 256), W(FAKE, FAKE, FAKE, None, FAKE, 512))
    assert lib.qlinear_gemm_grouped_workspace_size(64, k, small, 2, 6, 64) == \
        lib.qlinear_gemm_workspace_size(64, 512, k, 6, 64)
