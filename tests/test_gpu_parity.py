"""Parity of the HIP path (through the C ABI) with the FP64 oracle.

Small shapes cover the edge cases (ragged tails, one block per split, MHA /
GQA / MQA head mapping, d and Bc in {64, 128}, lambda from 0 to 0.5, T < Bc);
the five workload configurations run at full size, compared on every output
where the oracle is cheap, on whole heads at the 32K prefill, and on sampled
kv groups of the large decode batches.
"""
import sys

import numpy as np
import pytest

import workloads as W
from parity import check_decode, check_prefill, run_gpu_decode, run_gpu_prefill, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_flash_amd as bsa
    bsa._load()  # raises if the library is missing


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


DECODE_SMALL = [
    # B, Hq, Hkv, N, d, Bc, S, hot, window
    (1, 4, 1, 1000, 64, 64, 3, 0.02, 64),      # ragged N, S not dividing nk
    (2, 8, 2, 2048, 128, 128, 4, 0.01, 128),
    (1, 16, 1, 1536, 128, 64, 24, 0.02, 0),    # one block per split
    (1, 32, 1, 4096, 128, 128, 1, 0.02, 0),    # G = 32, a single split
    (2, 64, 1, 3000, 64, 128, 5, 0.02, 0),     # MQA, G = 64, ragged (paired workgroups)
    (33, 64, 1, 600, 64, 64, 4, 0.02, 0),      # MQA, 132 units: one workgroup per unit
    (1, 2, 2, 777, 128, 128, 2, 0.05, 0),      # MHA, ragged
    (1, 8, 2, 40960, 128, 128, 8, 0.01, 256),  # paired workgroups, 40 blocks per split: phases of 16, 16, 8
    (1, 4, 1, 9000, 64, 64, 2, 0.02, 128),     # paired, d = Bc = 64, 71 blocks per split: phases of 32, 32, 7
    (2, 40, 2, 2500, 128, 64, 3, 0.02, 0),     # G = 20: a partly filled 32-head tile
    (1, 128, 1, 3000, 128, 128, 4, 0.02, 128), # G = 128: two 64-head workgroups per split, ragged
    (2, 96, 1, 2100, 64, 64, 3, 0.02, 0),      # G = 96: the second 64-head part half filled
    # up to 16 heads, 129-256 (b, kv head, split) units: one 8-wave workgroup per split, two V slots
    (2, 32, 8, 4096, 128, 128, 16, 0.01, 128), # 256 units
    (1, 8, 2, 9000, 64, 64, 80, 0.02, 0),      # 160 units, 1-2 blocks per split, ragged N
    (2, 12, 3, 3000, 128, 64, 24, 0.02, 64),   # 144 units, G = 4, d = 128 with Bc = 64
    # up to 16 heads, more than 256 units: one 4-wave workgroup per split, four slots per wave
    (4, 16, 4, 5000, 64, 64, 20, 0.02, 64),    # 320 units, d = Bc = 64, ragged N
    (3, 8, 8, 3000, 128, 64, 12, 0.02, 0),     # 288 units, MHA, d = 128 with Bc = 64
    (6, 16, 4, 3000, 64, 128, 12, 0.02, 0),    # 288 units, d = 64 with Bc = 128
    # 33..64 heads at d = 128: the wide-group kernel (one 8-wave workgroup per split)
    (33, 64, 1, 600, 128, 128, 4, 0.02, 0),    # 132 units, ragged N (4.7 blocks), splits of 1-2 blocks
    (2, 48, 1, 3000, 128, 64, 5, 0.02, 64),    # G = 48: the fourth head tile empty; Bc = 64
    (4, 64, 2, 2000, 128, 128, 16, 0.02, 0),   # S = nk = 16: one block per split (one phase, no K ahead)
    (3, 40, 1, 5000, 128, 64, 3, 0.02, 128),   # G = 40: a half-filled head tile; 26 blocks per split
    (1, 64, 1, 9000, 128, 128, 1, 0.02, 256),  # one split of 71 blocks: decision bytes in chunks of 32, 32, 7
    (2, 56, 1, 8200, 128, 64, 2, 0.02, 0),     # G = 56, Bc = 64: 64 and 65 blocks per split (a 1-block chunk)
]


@pytest.mark.parametrize("shape", DECODE_SMALL, ids=lambda s: "B%d_Hq%d_Hkv%d_N%d_d%d_Bc%d_S%d" % s[:7])
@pytest.mark.parametrize("lam", [0.0, 1e-3, 1e-1, 0.99])
def test_decode_small(shape, lam):
    B, Hq, Hkv, N, d, Bc, S, hot, window = shape
    w = W.Workload("t", "decode", B=B, Hq=Hq, Hkv=Hkv, d=d, T=N, Bc=Bc, lambdas=(lam,), hot_rate=hot,
                   seed=101 + N, window=window, num_splits=S)
    x = W.generate(w)
    rep = check_decode(x, Bc, lam, S)
    say("decode", shape, lam, rep)


PREFILL_SMALL = [
    # B, Hq, Hkv, T, d, Bc, hot
    (1, 4, 1, 1024, 64, 64, 0.02),
    (1, 4, 2, 1000, 128, 128, 0.02),   # ragged
    (2, 2, 2, 300, 64, 128, 0.03),
    (1, 8, 2, 513, 128, 64, 0.02),
    (1, 1, 1, 50, 64, 64, 0.05),       # T < Bc
    # 16 (sequence, head group) pairs over 21 query blocks: on a 256-CU device 16 blocks are resident
    # at once, so the kv-group -> XCD map turns once
    (2, 16, 4, 2600, 128, 128, 0.02),
    # odd G (one head per workgroup): 24 head groups over 12 query blocks, 10 resident at once on a
    # 256-CU device, so the map turns there too
    (1, 24, 8, 1500, 128, 128, 0.02),
]


@pytest.mark.parametrize("shape", PREFILL_SMALL, ids=lambda s: "B%d_Hq%d_Hkv%d_T%d_d%d_Bc%d" % s[:6])
@pytest.mark.parametrize("lam", [0.0, 1e-4, 1e-2, 0.5, 0.99])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_small(shape, lam, causal):
    B, Hq, Hkv, T, d, Bc, hot = shape
    w = W.Workload("t", "prefill", B=B, Hq=Hq, Hkv=Hkv, d=d, T=T, Bc=Bc, lambdas=(lam,), hot_rate=hot,
                   seed=202 + T)
    x = W.generate(w)
    rep = check_prefill(x, Bc, lam, causal=causal)
    say("prefill", shape, lam, causal, rep)


# --------------------------------------------------------------------------- #
# The five workload configurations at full size
# --------------------------------------------------------------------------- #
def test_config_prefill_1k_tiny():
    w = W.CONFIGS["prefill_1k_tiny"]
    x = W.generate(w)
    for lam in w.lambdas + (0.0, 1e-2):
        rep = check_prefill(x, w.Bc, lam)
        say(w.name, lam, rep)


def test_config_decode_32k():
    w = W.CONFIGS["decode_32k"]
    x = W.generate(w)
    rep = check_decode(x, w.Bc, w.lambdas[0], w.num_splits)
    say(w.name, rep)
    assert rep.decisions == w.B * w.Hq * (w.T // w.Bc)


@pytest.fixture(scope="module")
def prefill_32k():
    w = W.CONFIGS["prefill_32k"]
    x = W.generate(w)
    return w, x, {k: to_device(v) for k, v in x.items()}


# two whole query heads per lambda, from different kv groups (every query block,
# every mask entry, every output row), and single query blocks of other heads
WHOLE_HEADS = {1e-4: (0, 29), 1e-3: (10, 19), 1e-2: (5, 30)}


@pytest.mark.parametrize("lam", [1e-4, 1e-3, 1e-2])
def test_config_prefill_32k(prefill_32k, lam):
    w, x, x_dev = prefill_32k
    nq = w.T // w.Bc
    heads = WHOLE_HEADS[lam]
    assert len({h // w.G for h in heads}) == len(heads)
    picks = [(7, nq - 2), (13, nq // 2), (31, 0), (20, 64), (3, 200), (26, 1), (31, nq - 1)]
    picks = [(h, i) for h, i in picks if h not in heads]
    # heaviest query blocks first, so the oracle's threads finish together
    units = [h * nq + i for h in heads for i in reversed(range(nq))] + [h * nq + i for h, i in picks]
    say(w.name, "lambda", lam, "whole heads", heads, "single query blocks", picks)
    gpu = run_gpu_prefill(x_dev, w.Bc, lam)
    mask = gpu["mask"].cpu().numpy()
    # properties over every decision of the full problem
    tri = np.tril(np.ones((nq, nq), bool))
    assert ((mask == 2) == ~tri[None, None]).all()
    assert np.isin(mask[:, :, tri], (0, 1)).all()
    assert bool(__import__("torch").isfinite(gpu["o"]).all())
    say("  sparsity %.4f" % float((mask[:, :, tri] == 1).mean()))
    rep = check_prefill(x, w.Bc, lam, units=units, gpu=gpu)
    say(" ", rep)
    assert rep.decisions == len(heads) * nq * (nq + 1) // 2 + sum(i + 1 for _, i in picks)


def test_config_decode_128k_b16_sampled():
    w = W.CONFIGS["decode_128k_b16"]
    x = W.generate(w)
    x_dev = {k: to_device(v) for k, v in x.items()}
    gpu = run_gpu_decode(x_dev, w.Bc, w.lambdas[0], w.num_splits)
    del x_dev
    units = [0, 9, 27, 42, 63, 64 + 5, 101, 127]
    rep = check_decode(x, w.Bc, w.lambdas[0], w.num_splits, units=units, gpu=gpu)
    say(w.name, rep)
    assert np.isin(gpu["skip"], (0, 1)).all()
    assert np.isfinite(gpu["o"]).all()


def test_config_decode_mqa_16k():
    w = W.CONFIGS["decode_mqa_16k"]
    x = W.generate(w)
    units = list(range(0, w.B, 4))
    rep = check_decode(x, w.Bc, w.lambdas[0], w.num_splits, units=units)
    say(w.name, rep)


# --------------------------------------------------------------------------- #
# Determinism, empty inputs, argument errors through the ABI
# --------------------------------------------------------------------------- #
def test_deterministic():
    import torch
    w = W.CONFIGS["decode_32k"]
    x_dev = {k: to_device(v) for k, v in W.generate(w).items()}
    a = run_gpu_decode(x_dev, w.Bc, 1e-3, w.num_splits)
    b = run_gpu_decode(x_dev, w.Bc, 1e-3, w.num_splits)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    wp = W.CONFIGS["prefill_1k_tiny"]
    xp = {k: to_device(v) for k, v in W.generate(wp).items()}
    p1 = run_gpu_prefill(xp, wp.Bc, 1e-2)
    p2 = run_gpu_prefill(xp, wp.Bc, 1e-2)
    for key in p1:
        assert torch.equal(p1[key], p2[key]), key


def test_empty_batch_is_a_no_op():
    import torch
    import block_sparse_attention_flash_amd as bsa
    q = torch.empty((0, 4, 1, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((0, 1, 256, 128), dtype=torch.bfloat16, device="cuda")
    o_part, lse_part, skip, vskip = bsa.decode(q, k, k, 1e-3, 2)
    assert o_part.numel() == 0
    qp = torch.empty((0, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    o, lse, mask = bsa.prefill(qp, qp, qp, 1e-3, Bc=64)
    assert o.numel() == 0


def test_argument_errors():
    import torch
    import block_sparse_attention_flash_amd as bsa
    q = torch.zeros((1, 4, 1, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 256, 128), dtype=torch.bfloat16, device="cuda")
    for lam, status in [(1.0, bsa.ERR_INVALID_ARG), (-0.1, bsa.ERR_INVALID_ARG), (float("nan"), bsa.ERR_INVALID_ARG)]:
        with pytest.raises(bsa.BlasstError) as e:
            bsa.decode(q, k, k, lam, 2)
        assert e.value.status == status
    with pytest.raises(bsa.BlasstError) as e:
        bsa.decode(q, k, k, 1e-3, 3)  # 3 splits > 2 blocks
    assert e.value.status == bsa.ERR_INVALID_ARG
    q96 = torch.zeros((1, 1, 64, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bsa.BlasstError) as e:
        bsa.prefill(q96, q96, q96, 1e-3, Bc=64)
    assert e.value.status == bsa.ERR_UNSUPPORTED


@pytest.mark.parametrize("d,S", [(128, 16), (64, 40), (512, 5)])
def test_combine_paths_agree(d, S):
    """The merge runs four columns per thread when the partials and the output are 16-byte
    aligned, one column per thread otherwise; both give bit-identical results, including a row
    whose splits are all empty and one with a single non-empty split (S = 40: the looped form)."""
    import torch
    import block_sparse_attention_flash_amd as bsa
    g = torch.Generator().manual_seed(d + S)
    B, Hq = 3, 5
    o_part = torch.randn((B, Hq, S, d), generator=g).cuda()
    lse_part = (torch.randn((B, Hq, S), generator=g) * 3).cuda()
    lse_part[0, 0, :] = float("-inf")
    lse_part[1, 2, 1:] = float("-inf")
    o_a, l_a = bsa.decode_combine(o_part, lse_part)

    def shifted(t):  # same values, 4 bytes past a 16-byte boundary
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v

    op_u, o_u, l_u = shifted(o_part), shifted(torch.zeros_like(o_a)), torch.empty_like(l_a)
    bsa.blasst_decode_combine(op_u, lse_part, o_u, l_u)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_u) and torch.equal(l_a, l_u)
    assert torch.all(o_a[0, 0] == 0) and l_a[0, 0] == float("-inf")
    assert torch.allclose(o_a[1, 2], o_part[1, 2, 0]) and l_a[1, 2] == lse_part[1, 2, 0]
