"""The dense references (blasst_prefill_dense, blasst_decode_dense) on the GPU.

blasst_prefill_dense must equal the lambda = 0 call bit for bit (the same
kernel without the skip test; nothing is skipped at lambda = 0 either).
blasst_decode_dense runs a kernel of its own for groups of up to 32 heads (one
pass over K and V, an online softmax per wave, the waves merged by their
maxima), so it is compared with the oracle's dense limit (lambda = 0) at the
parity tolerances; for wider groups it is the skip kernel at lambda = 0 and
must equal that call bit for bit.
"""
import numpy as np
import pytest

import workloads as W
from parity import check_decode, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_flash_amd as bsa
    bsa._load()


@pytest.mark.parametrize("shape", [(1, 8, 2, 1000, 128, 128), (2, 4, 4, 300, 64, 64), (1, 6, 1, 513, 128, 64)],
                         ids=lambda s: "B%d_Hq%d_Hkv%d_T%d_d%d_Bc%d" % s)
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_dense_equals_lambda_zero(shape, causal):
    import torch
    import block_sparse_attention_flash_amd as bsa
    B, Hq, Hkv, T, d, Bc = shape
    w = W.Workload("t", "prefill", B=B, Hq=Hq, Hkv=Hkv, d=d, T=T, Bc=Bc, lambdas=(0.0,), hot_rate=0.03, seed=1001 + T)
    x = {k: to_device(v) for k, v in W.generate(w).items()}
    o0, l0, _ = bsa.prefill(x["q"], x["k"], x["v"], 0.0, Bc=Bc, causal=causal)
    o = torch.empty_like(o0)
    lse = torch.empty_like(l0)
    bsa.blasst_prefill_dense(x["q"], x["k"], x["v"], o, lse, Bc, causal)
    assert torch.equal(o, o0) and torch.equal(lse, l0)


DENSE_DECODE = [
    # B, Hq, Hkv, N, d, Bc, S
    (1, 32, 8, 32768, 128, 128, 32),   # decode_32k's shape at 32 splits: one workgroup per split
    (1, 32, 8, 32768, 128, 128, 16),   # decode_32k: two workgroups per split, each half of V's columns
    (1, 32, 8, 4096, 128, 128, 16),    # two blocks per split: one unit per wave
    (2, 8, 2, 1000, 64, 64, 3),        # ragged N, S not dividing nk
    (1, 16, 1, 1536, 128, 64, 24),     # one 64-key block per split: two of the four waves have no unit
    (1, 4, 1, 900, 128, 128, 7),       # last block with 4 keys: units with no key are not visited
    (2, 40, 2, 2500, 128, 64, 3),      # G = 20: two head tiles, the second partly filled
    (1, 64, 2, 3000, 64, 128, 5),      # G = 32
    (3, 2, 2, 777, 128, 128, 2),       # MHA
    (4, 64, 2, 3000, 64, 64, 20),      # 160 units: one workgroup per split, G = 32 at d = 64
    (3, 16, 4, 2000, 64, 128, 12),     # 144 units: one workgroup per split at d = 64
]


@pytest.mark.parametrize("shape", DENSE_DECODE, ids=lambda s: "B%d_Hq%d_Hkv%d_N%d_d%d_Bc%d_S%d" % s)
def test_decode_dense_matches_oracle(shape):
    import torch
    import block_sparse_attention_flash_amd as bsa
    B, Hq, Hkv, N, d, Bc, S = shape
    w = W.Workload("t", "decode", B=B, Hq=Hq, Hkv=Hkv, d=d, T=N, Bc=Bc, lambdas=(0.0,), hot_rate=0.02, seed=1002 + N,
                   window=64, num_splits=S)
    x = W.generate(w)
    xd = {k: to_device(v) for k, v in x.items()}
    nk = -(-N // Bc)
    op = torch.empty((B, Hq, S, d), dtype=torch.float32, device="cuda")
    lp = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    bsa.blasst_decode_dense(xd["q"], xd["k"], xd["v"], op, lp, Bc, S)
    o, lse = bsa.decode_combine(op, lp)
    torch.cuda.synchronize()
    gpu = dict(o_part=op.cpu().numpy(), lse_part=lp.cpu().numpy(), o=o.cpu().numpy(), lse=lse.cpu().numpy(),
               skip=np.zeros((B, Hq, nk), np.uint8), vskip=np.zeros((B, Hkv, nk), np.uint8))
    rep = check_decode(x, Bc, 0.0, S, gpu=gpu)
    print("decode dense", shape, rep, flush=True)


@pytest.mark.parametrize("shape", [(2, 64, 1, 3000, 64, 128, 5), (1, 128, 1, 2000, 128, 128, 4)],
                         ids=lambda s: "B%d_Hq%d_Hkv%d_N%d_d%d_Bc%d_S%d" % s)
def test_decode_dense_wide_groups_equal_lambda_zero(shape):
    import torch
    import block_sparse_attention_flash_amd as bsa
    B, Hq, Hkv, N, d, Bc, S = shape
    w = W.Workload("t", "decode", B=B, Hq=Hq, Hkv=Hkv, d=d, T=N, Bc=Bc, lambdas=(0.0,), hot_rate=0.02, seed=1002 + N,
                   num_splits=S)
    x = {k: to_device(v) for k, v in W.generate(w).items()}
    op0, lp0, _, _ = bsa.decode(x["q"], x["k"], x["v"], 0.0, S, Bc=Bc)
    op, lp = torch.empty_like(op0), torch.empty_like(lp0)
    bsa.blasst_decode_dense(x["q"], x["k"], x["v"], op, lp, Bc, S)
    assert torch.equal(op, op0) and torch.equal(lp, lp0)


@pytest.mark.parametrize("shape", [(1, 8, 32768, 128, 128, 16), (2, 2, 1000, 64, 64, 3), (1, 4, 900, 128, 128, 7)],
                         ids=lambda s: "B%d_Hkv%d_N%d_d%d_Bc%d_S%d" % s)
def test_load_ceiling_runs(shape):
    """The measurement call (the split kernel's loads alone) completes on ragged shapes and writes nothing."""
    import torch
    import block_sparse_attention_flash_amd as bsa
    B, Hkv, N, d, Bc, S = shape
    k = torch.randn((B, Hkv, N, d), device="cuda").to(torch.bfloat16)
    v = torch.randn((B, Hkv, N, d), device="cuda").to(torch.bfloat16)
    k0, v0 = k.clone(), v.clone()
    bsa.blasst_decode_load_ceiling(k, v, Bc, S)
    torch.cuda.synchronize()
    assert torch.equal(k, k0) and torch.equal(v, v0)
