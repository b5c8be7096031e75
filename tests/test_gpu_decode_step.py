"""blasst_decode_step on the GPU: one call for the split kernel and the merge.

It must give exactly what blasst_decode followed by blasst_decode_combine gives
(the same kernels on the same stream, the partials in the caller's workspace),
bit for bit, and therefore the oracle's merged output within the parity
tolerances; the decision masks are the split kernel's.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as W
from parity import Report, compare_lse, compare_masks, compare_rows, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_flash_amd as bsa
    bsa._load()


STEP = [
    # B, Hq, Hkv, N, d, Bc, S, lambda
    (1, 32, 8, 32768, 128, 128, 16, 1e-3),  # decode_32k
    (2, 8, 2, 1000, 64, 64, 3, 1e-1),       # ragged N
    (3, 64, 1, 2000, 128, 128, 4, 1e-3),    # MQA
    (1, 128, 1, 1500, 128, 128, 2, 1e-2),   # two 64-head parts per split
    (4, 16, 4, 5000, 64, 64, 20, 0.0),      # 320 units
]


@pytest.mark.parametrize("shape", STEP, ids=lambda s: "B%d_Hq%d_Hkv%d_N%d_d%d_Bc%d_S%d_lam%g" % s)
def test_decode_step(shape):
    import torch
    import block_sparse_attention_flash_amd as bsa
    B, Hq, Hkv, N, d, Bc, S, lam = shape
    w = W.Workload("t", "decode", B=B, Hq=Hq, Hkv=Hkv, d=d, T=N, Bc=Bc, lambdas=(lam,), hot_rate=0.02, seed=1400 + N,
                   window=64, num_splits=S)
    x = W.generate(w)
    xd = {k: to_device(v) for k, v in x.items()}
    o, lse, skip, vskip = bsa.decode_step(xd["q"], xd["k"], xd["v"], lam, S, Bc=Bc)
    op, lp, skip2, vskip2 = bsa.decode(xd["q"], xd["k"], xd["v"], lam, S, Bc=Bc)
    o2, lse2 = bsa.decode_combine(op, lp)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    assert torch.equal(skip, skip2) and torch.equal(vskip, vskip2)
    ref = oracle.decode(x["q"], x["k"], x["v"], Bc, lam, S)
    rep = Report()
    diff = compare_masks(skip.cpu().numpy(), ref["skip_full"], ref["margin_full"], rep, "skip")
    if diff.any():  # adopt the GPU's decision on near-threshold blocks (both are valid results)
        f = np.where(diff, skip.cpu().numpy(), -1).astype(np.int8).reshape(B * Hkv, Hq // Hkv, -1)
        ref = oracle.decode(x["q"], x["k"], x["v"], Bc, lam, S, force=f)
    o_ref, lse_ref = oracle.combine(ref["o_part_full"], ref["lse_part_full"])
    compare_rows(o.cpu().numpy(), o_ref, rep, "o")
    compare_lse(lse.cpu().numpy(), lse_ref, rep, "lse")
    print("decode step", shape, rep, flush=True)
    sys.stdout.flush()


def test_decode_step_rejects_a_small_workspace():
    import torch
    import block_sparse_attention_flash_amd as bsa
    q = torch.zeros((1, 4, 1, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 512, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((1, 4, 128), dtype=torch.float32, device="cuda")
    need = bsa.decode_step_workspace_size(1, 4, 128, 2)
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(bsa.BlasstError) as e:
        bsa.blasst_decode_step(q, k, k, o, None, None, None, ws, 128, 1e-3, 2)
    assert e.value.status == bsa.ERR_INVALID_ARG
