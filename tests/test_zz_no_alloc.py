"""The routed apply without allocation (qlinear_apply_experts_noalloc) against the routed apply with
a workspace (qlinear_apply_experts), bit for bit, through the C ABI: two calls in a row on the same
GPU, the second with a smaller input, so the second call reuses the scratch array the first left
behind (Nx_quant API docs, Products: apply_experts)."""
import numpy as np
import pytest
import torch

import synth
import weight_only_quantized_affine_amd as q

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _mx_weights(seed, e, n, k):
    g = np.random.default_rng(seed)
    codes = torch.from_numpy(g.integers(0, 256, (e, n, k // 2), dtype=np.uint8)).to(DEV)
    scales = torch.from_numpy(g.integers(118, 131, (e, n, k // 32), dtype=np.uint8)).to(DEV)
    return codes, scales


def _q8_weights(seed, e, n, k):
    g = np.random.default_rng(seed)
    nb = k // 32
    d = np.exp2(g.uniform(-14, -9, (e, n, nb))).astype(np.float16).view(np.uint8).reshape(e, n, nb, 2)
    qv = g.integers(-127, 128, (e, n, nb, 32), dtype=np.int64).astype(np.int8).view(np.uint8)
    return torch.from_numpy(np.concatenate([d, qv], axis=3).reshape(e, n, nb * 34).copy()).to(DEV), None


@pytest.mark.parametrize("fmt", [q.QL_MXFP4, q.QL_Q8_0])
def test_noalloc_matches_workspace_call_twice(fmt):
    e, n, k = 8, 384, 512
    w0, w1 = (_mx_weights if fmt == q.QL_MXFP4 else _q8_weights)(900 + fmt, e, n, k)
    # first call: 300 tokens x top-3 (with an out-of-range id); second: 37 tokens x top-2
    for call, (tokens, top) in enumerate([(300, 3), (37, 2)]):
        ids_np = synth.topk_ids(910 + 10 * fmt + call, tokens, top, e).reshape(-1).copy()
        ids_np[5] = -1
        ids_np[-1] = e
        ids = torch.from_numpy(ids_np).to(DEV)
        x = torch.from_numpy(np.random.default_rng(920 + call).standard_normal((tokens, k)).astype(np.float32)).to(
            DEV).to(torch.bfloat16)
        ref = q.qlinear_apply_experts(fmt, w0, w1, ids, x, n=n, k=k, pos_per_row=top, y_dtype=torch.float32)
        got = torch.full((tokens * top, n), float("nan"), dtype=torch.float32, device=DEV)
        q.qlinear_apply_experts_noalloc(fmt, w0, w1, ids, x, n=n, k=k, y=got, pos_per_row=top)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"call {call}: outputs differ"
        assert torch.all(got[5] == 0) and torch.all(got[-1] == 0), f"call {call}: out-of-range rows not zero"


def test_noalloc_rejects_sizes_past_the_scratch_array():
    e, n, k = 2, 32, 64
    w0, w1 = _mx_weights(930, e, n, k)
    n_pos = 100_000  # 12 bytes per position of scratch: past 1 MiB
    ids = torch.zeros(n_pos, dtype=torch.int64, device=DEV)
    x = torch.zeros((n_pos, k), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((n_pos, n), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(q.QLError, match="scratch"):
        q.qlinear_apply_experts_noalloc(q.QL_MXFP4, w0, w1, ids, x, n=n, k=k, y=y)
