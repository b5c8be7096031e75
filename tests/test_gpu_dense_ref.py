"""The dense references (blasst_prefill_dense, blasst_decode_dense) on the GPU:
they must equal the lambda = 0 calls, which the parity tests pin to the oracle's
dense limit, bit for bit (no tile or block is skipped at lambda = 0 either)."""
import pytest

import workloads as W
from parity import to_device

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


@pytest.mark.parametrize("shape", [(1, 32, 8, 4096, 128, 128, 16), (2, 64, 1, 3000, 64, 128, 5)],
                         ids=lambda s: "B%d_Hq%d_Hkv%d_N%d_d%d_Bc%d_S%d" % s)
def test_decode_dense_equals_lambda_zero(shape):
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
