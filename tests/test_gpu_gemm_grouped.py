"""The grouped prefill GEMM (qlinear_gemm_grouped: up to four weights reading one x) against the
oracle, and against qlinear_gemm on each weight alone (Nx_quant API docs, Products: apply)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_only_quantized_affine_amd as q
from gpu_helpers import DEV, TDT, bits_to_dev, out_f64, u32_to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-3  # the products' bound (relative l2 per row): 16-bit outputs
GEMM_TOL = 1e-3  # fp32 outputs: one fp16 rounding per weight, ~2^-11/sqrt(3) per row (2.7e-4 worst measured)


def _weight(seed, n, k, bits, g, pdt):
    w = synth.weights_f32(seed, n, k)
    opk, osb, obb = O.affine_quantize(w, bits, g, pdt)
    D = O.affine_dequant_f32(opk, osb, obb, bits, g, pdt, k)
    return dict(packed=u32_to_dev(opk), scales=bits_to_dev(osb, pdt), biases=bits_to_dev(obb, pdt)), D


@pytest.mark.parametrize("m,ns,k,bits,g,xdt,pdt,ydt", [
    # ragged m, n and k (k % 128 == 64 or 32: a last k-tile of one 64-value x block), layer biases
    (1100, (2000, 700, 1500), 1088, 4, 64, "bf16", "bf16", "f32"),
    (1030, (1800, 1200), 2080, 4, 32, "bf16", "f16", "bf16"),
    (900, (3000, 257, 1100, 500), 1024, 4, 128, "f16", "bf16", "f16"),
    (1200, (2300, 1000), 768, 8, 64, "bf16", "bf16", "f32"),
    (1000, (1500, 1700), 1088, 8, 32, "f16", "f16", "f32"),
    # bitstream widths: the codes of every weight as bytes, then the 8-bit launch over all of them
    (1100, (2600, 300, 700), 1024, 6, 64, "bf16", "bf16", "f32"),
    (1050, (2600, 1300), 1088, 3, 32, "f16", "bf16", "bf16"),
])
def test_gemm_grouped_ragged(m, ns, k, bits, g, xdt, pdt, ydt):
    weights, Ds, lbs = [], [], []
    for j, n in enumerate(ns):
        w, D = _weight(6000 + 10 * j + bits + m, n, k, bits, g, pdt)
        lb = synth.acts_bits(6100 + j, 1, n, xdt)[0] if j % 2 == 0 else None
        if lb is not None:
            w["layer_bias"] = bits_to_dev(lb, xdt)
        w["y"] = torch.full((m, n), float("nan"), dtype=TDT[ydt], device=DEV)
        weights.append(w)
        Ds.append(D)
        lbs.append(lb)
    xb = synth.acts_bits(6200 + m, m, k, xdt)
    x = bits_to_dev(xb, xdt)
    q.qlinear_gemm_grouped(x, weights, bits=bits, group_size=g)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(m).choice(m, 40, replace=False), [0, m - 1]]))
    xf = O.bits_to_f64(xdt, xb[rows])
    for j, (w, D, lb) in enumerate(zip(weights, Ds, lbs)):
        ref = O.apply(xf, D, layer_bias=None if lb is None else O.bits_to_f64(xdt, lb))
        got = out_f64(w["y"])
        assert not np.isnan(got).any(), f"weight {j}: unwritten outputs"
        if ydt != "f32":  # 16-bit outputs: against the oracle rounded once to that dtype
            ref = O.bits_to_f64(ydt, O.to_bits(ydt, ref.astype(np.float32)))
        err = O.rel_l2_per_row(got[rows], ref)
        print(f"weight {j} (n={w['packed'].shape[0]}): max rel-l2 {err.max():.3e}")
        assert err.max() <= (GEMM_TOL if ydt == "f32" else TOL)


def test_gemm_grouped_9b_qkv_matches_single_calls_and_oracle():
    """q|k|v of the 9B-class layer (M=2048, k=4096, 4-bit g64, bf16) in one grouped call: q is bit
    for bit the single call's result (same kernel, same tiles); k and v, whose single calls split the
    sum over k on another kernel, match the oracle on whole output rows of 24 sampled x rows."""
    m, k = 2048, 4096
    ns = (4096, 1024, 1024)
    weights, Ds = [], []
    for j, n in enumerate(ns):
        w = synth.weights_f32(synth.seed_for(4, 1, j), n, k)
        pk, sc, bi = q.qlinear_quantize(torch.from_numpy(w).to(DEV), 4, 64, torch.bfloat16)
        weights.append(dict(packed=pk, scales=sc, biases=bi, y=torch.empty((m, n), dtype=torch.float32, device=DEV)))
        Ds.append(w)
    xb = synth.acts_bits(synth.seed_for(4, 1, 9, 1), m, k, "bf16")
    x = bits_to_dev(xb, "bf16")
    q.qlinear_gemm_grouped(x, weights, bits=4, group_size=64)
    single_q = q.qlinear_gemm(x, weights[0]["packed"], weights[0]["scales"], weights[0]["biases"], bits=4,
                              group_size=64, y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(single_q, weights[0]["y"])
    rows = np.sort(np.random.default_rng(5).choice(m, 24, replace=False))
    xf = O.bits_to_f64("bf16", xb[rows])
    for j, (w, wf) in enumerate(zip(weights, Ds)):
        opk, osb, obb = O.affine_quantize(wf, 4, 64, "bf16")
        D = O.affine_dequant_f32(opk, osb, obb, 4, 64, "bf16", k)
        err = O.rel_l2_per_row(out_f64(w["y"])[rows], O.apply(xf, D))
        print(f"{'qkv'[j]}: max rel-l2 over whole rows {err.max():.3e}")
        assert err.max() <= GEMM_TOL


def test_gemm_grouped_small_shapes_fall_back_to_single_calls():
    """Too few tiles for the grouped kernel: the call runs qlinear_gemm per weight, bit for bit."""
    m, k = 100, 512
    weights = []
    for j, n in enumerate((300, 64)):
        w, _ = _weight(6300 + j, n, k, 4, 64, "bf16")
        weights.append(w)
    x = bits_to_dev(synth.acts_bits(6310, m, k, "bf16"), "bf16")
    outs = q.qlinear_gemm_grouped(x, weights, bits=4, group_size=64, y_dtype=torch.float32)
    for w, y in zip(weights, outs):
        ref = q.qlinear_gemm(x, w["packed"], w["scales"], w["biases"], bits=4, group_size=64, y_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(ref, y)
