"""MLA decode on the GPU (through the C ABI) against the FP64 oracle.

Shapes cover both head-group widths of the kernel (32 and 64 heads per
workgroup), ragged contexts, one block per split and more splits than blocks
per split would allow for a plain decode; lambda from 0 (dense) to 0.1.  The
128-head, 32K-context configuration runs at full size, compared on sampled
(sequence, head) units.
"""
import math
import sys

import numpy as np
import pytest

import workloads as W
from parity import check_mla, run_gpu_mla, to_device

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(192.0)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_flash_amd as bsa
    bsa._load()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def mla_inputs(B, Hq, N, S, seed, hot=0.02, Bc=64):
    w = W.Workload("t", "decode", B=B, Hq=Hq, Hkv=1, d=576, T=N, Bc=Bc, lambdas=(1e-3,), hot_rate=hot, seed=seed,
                   window=128, num_splits=S, dv=512, scale=SCALE)
    x = W.generate(w, parts=("q", "k"))
    return np.ascontiguousarray(x["q"][:, :, 0]), np.ascontiguousarray(x["k"][:, 0])


MLA = [
    # B, Hq, N, S
    (2, 32, 1000, 3),     # 32 heads per workgroup, ragged context
    (1, 64, 2048, 32),    # one block per split
    (1, 128, 777, 2),     # four head groups, ragged
    (4, 128, 8192, 32),   # 64 heads per workgroup (256 workgroups)
]


MLA32 = [
    # B, Hq, N, S: 32-token blocks (64 heads per workgroup)
    (2, 64, 1000, 3),     # ragged context, stage ring shorter than a split
    (1, 64, 4096, 128),   # one block per split
    (2, 128, 777, 2),     # ragged, two head groups
    (4, 128, 8192, 16),
]


@pytest.mark.parametrize("shape,Bc", [(s, 64) for s in MLA] + [(s, 32) for s in MLA32],
                         ids=lambda v: ("B%d_Hq%d_N%d_S%d" % v) if isinstance(v, tuple) else "Bc%d" % v)
@pytest.mark.parametrize("lam", [0.0, 1e-3, 1e-1, 0.99])
def test_mla_small(shape, Bc, lam):
    B, Hq, N, S = shape
    q, kv = mla_inputs(B, Hq, N, S, seed=900 + N, Bc=Bc)
    units = None
    if B * Hq > 128:  # sample heads of every sequence (the oracle is the slow side)
        rng = np.random.default_rng(N)
        units = sorted(int(u) for u in rng.choice(B * Hq, size=96, replace=False))
    rep = check_mla(q, kv, Bc, lam, S, SCALE, 512, units=units)
    say("mla", shape, "Bc", Bc, lam, rep)


@pytest.mark.parametrize("Bc", [64, 32])
def test_mla_decode_mla_32k_sampled(Bc):
    w = W.MLA_CONFIGS["decode_mla_32k"]
    x = W.generate(w, parts=("q", "k"))
    q, kv = np.ascontiguousarray(x["q"][:, :, 0]), np.ascontiguousarray(x["k"][:, 0])
    del x
    gpu = run_gpu_mla(to_device(q), to_device(kv), Bc, w.lambdas[0], w.num_splits, w.score_scale, w.dv)
    rng = np.random.default_rng(11)
    units = sorted(int(u) for u in rng.choice(w.B * w.Hq, size=64, replace=False))
    rep = check_mla(q, kv, Bc, w.lambdas[0], w.num_splits, w.score_scale, w.dv, units=units, gpu=gpu)
    say("decode_mla_32k sampled Bc", Bc, rep, "block sparsity %.4f" % float(gpu["skip"].mean()))


def test_mla_deterministic_and_dense_equal_lambda_zero():
    import torch
    import block_sparse_attention_flash_amd as bsa
    q, kv = mla_inputs(2, 64, 3000, 4, seed=901)
    qd, kvd = to_device(q), to_device(kv)
    a = bsa.decode_mla(qd, kvd, 1e-3, 4, SCALE)
    b = bsa.decode_mla(qd, kvd, 1e-3, 4, SCALE)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
