"""GPU parity of the Q4_K and Q6_K paths (Nx_quant API docs, Weights: Q4_K and Q6_K; Products:
dequant and apply_experts): dequant bit-exact against the oracle at every output dtype, with zero
blocks (+0 / -0) and non-finite scales; the routed apply against the oracle's fp64 sums of the
decoded values, with ids out of range, ragged chunks and several 256-value blocks per row."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_quantized_affine_amd as q
from gpu_helpers import DEV, TDT, bits_to_dev, out_bits_or_f32, out_f64, same_values, u8_to_dev

pytestmark = pytest.mark.gpu

FMTS = {"q4_k": (q.QL_Q4_K, O.q4_k_dequant_f32, 144), "q6_k": (q.QL_Q6_K, O.q6_k_dequant_f32, 210)}


@pytest.mark.parametrize("name", ["q4_k", "q6_k"])
@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("rows,k", [(37, 256), (130, 1024), (3, 2816)])
def test_kquant_dequant_bitexact(name, odt, rows, k):
    fmt, deq, nbytes = FMTS[name]
    blocks = synth.kquant_random_blocks(900 + rows + k, rows, k, name)
    blocks[0, :nbytes] = 0  # a zero block: +0 (Q4_K) or -0 (Q6_K)
    print(f"{name} dequant rows={rows} k={k} -> {odt}", flush=True)
    out = q.qlinear_dequant(fmt, u8_to_dev(blocks), rows=rows, k=k, out_dtype=TDT[odt])
    torch.cuda.synchronize()
    want = O.round_f32_to(odt, deq(blocks))
    assert same_values(out_bits_or_f32(out, odt), want)


@pytest.mark.parametrize("name", ["q4_k", "q6_k"])
def test_kquant_dequant_nonfinite_scales(name):
    fmt, deq, nbytes = FMTS[name]
    rows, k = 4, 512
    blocks = synth.kquant_random_blocks(950, rows, k, name).reshape(rows, 2, nbytes)
    at = 0 if name == "q4_k" else 208
    blocks[1, 0, at:at + 2] = [0x00, 0x7C]  # d = +inf
    blocks[2, 1, at:at + 2] = [0x00, 0x7E]  # d = NaN
    blocks = blocks.reshape(rows, 2 * nbytes)
    out = q.qlinear_dequant(fmt, u8_to_dev(blocks), rows=rows, k=k).cpu().numpy()
    assert same_values(out, deq(blocks))


def _kq_case(name, seed, e, n, k, tokens, top, lo=0):
    fmt, deq, nbytes = FMTS[name]
    blocks = synth.kquant_random_blocks(seed, e * n, k, name).reshape(e, n, -1)
    W = deq(blocks)
    ids = np.random.default_rng(seed).integers(lo, e + (1 if lo < 0 else 0), size=(tokens, top)).astype(np.int64)
    xb = synth.acts_bits(seed + 1, tokens, k, "bf16")
    return fmt, blocks, W, ids, xb


@pytest.mark.parametrize("name", ["q4_k", "q6_k"])
@pytest.mark.parametrize("e,n,k,tokens,top", [
    (5, 200, 256, 37, 3),     # ids out of range on both sides; one block per row
    (3, 300, 1024, 100, 2),   # ragged weight-row tiles (300 = 2 * 128 + 44), chunks of 64 and more
    (4, 128, 2816, 20, 4),    # eleven blocks per row
])
def test_kquant_apply_experts(name, e, n, k, tokens, top):
    fmt, blocks, W, ids, xb = _kq_case(name, 1000 + e + n + k, e, n, k, tokens, top, lo=-1)
    print(f"{name} apply_experts e={e} n={n} k={k} tokens={tokens} top={top}", flush=True)
    y = q.qlinear_apply_experts(fmt, u8_to_dev(blocks), None, torch.from_numpy(ids.reshape(-1)).to(DEV),
                                bits_to_dev(xb, "bf16"), n=n, k=k, pos_per_row=top, y_dtype=torch.float32)
    yb = q.qlinear_apply_experts(fmt, u8_to_dev(blocks), None, torch.from_numpy(ids.reshape(-1)).to(DEV),
                                 bits_to_dev(xb, "bf16"), n=n, k=k, pos_per_row=top, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    flat = ids.reshape(-1)
    ref = O.apply_experts(W, flat, O.bits_to_f64("bf16", xb), pos_per_row=top)
    live = (flat >= 0) & (flat < e)
    out = out_f64(y)
    assert np.all(out[~live] == 0.0)
    # codes enter exactly and each sub-block's fp32 sum is scaled once: fp32 accumulation error only
    err = O.rel_l2_per_row(out[live], ref[live])
    print(f"{name} experts max rel-l2 per row {err.max():.3e}")
    assert err.max() <= 1e-5  # measured <= 1.3e-6 (8 x 3 shapes)
    want = O.bits_to_f64("bf16", O.to_bits("bf16", ref.astype(np.float32)))
    assert O.rel_l2_per_row(out_f64(yb)[live], want[live]).max() <= 2e-3


@pytest.mark.parametrize("name", ["q4_k", "q6_k"])
def test_kquant_apply_experts_f16_x(name):
    """fp16 activations take the f16 products (codes 128 + q, exact in fp16): the same fp32 bound."""
    e, n, k, tokens, top = 4, 256, 512, 30, 2
    fmt, blocks, W, ids, _ = _kq_case(name, 1200, e, n, k, tokens, top)
    xh = synth.acts_bits(1201, tokens, k, "f16")
    y = q.qlinear_apply_experts(fmt, u8_to_dev(blocks), None, torch.from_numpy(ids.reshape(-1)).to(DEV),
                                bits_to_dev(xh, "f16"), n=n, k=k, pos_per_row=top, y_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.apply_experts(W, ids.reshape(-1), O.bits_to_f64("f16", xh), pos_per_row=top)
    err = O.rel_l2_per_row(out_f64(y), ref)
    print(f"{name} experts f16 x max rel-l2 per row {err.max():.3e}")
    assert err.max() <= 1e-5
