"""Ragged batches on the GPU (through the C ABI): one length per sequence.

Every sequence of a ragged call must be the plain call at its own length, so
each sequence's slice of the GPU outputs is checked against the FP64 oracle run
on that sequence alone, with the tolerances and threshold-flip rule of the
plain parity tests.  Padded rows (O = 0, LSE = -inf) and mask entries past a
sequence's end (2) are checked exactly; a ragged call whose lengths are all the
capacity must equal the plain call bit for bit, and the values stored in the
padding must not matter.
"""
import sys

import numpy as np
import pytest

import workloads as W
from parity import check_decode, check_prefill, to_device

pytestmark = pytest.mark.gpu


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


def lens_dev(lens):
    import torch
    return torch.tensor(lens, dtype=torch.int32, device="cuda")


def run_prefill_ragged(xd, lens, Bc, lam, causal):
    import torch
    import block_sparse_attention_flash_amd as bsa
    o, lse, mask = bsa.prefill_ragged(xd["q"], xd["k"], xd["v"], lens_dev(lens), lam, Bc=Bc, causal=causal)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy(), mask.cpu().numpy()


def check_prefill_ragged(x, lens, Bc, lam, causal, xd=None):
    xd = xd or {k: to_device(v) for k, v in x.items()}
    o, lse, mask = run_prefill_ragged(xd, lens, Bc, lam, causal)
    reps = []
    for b, L in enumerate(lens):
        n = -(-L // Bc)
        assert np.all(o[b, :, L:] == 0) and np.all(np.isneginf(lse[b, :, L:])), "padded rows of sequence %d" % b
        assert np.all(mask[b, :, n:, :] == 2) and np.all(mask[b, :, :, n:] == 2), "mask past sequence %d" % b
        if L == 0:
            continue
        xb = {k: np.ascontiguousarray(v[b:b + 1, :, :L]) for k, v in x.items()}
        gb = dict(o=o[b:b + 1, :, :L], lse=lse[b:b + 1, :, :L], mask=mask[b:b + 1, :, :n, :n])
        reps.append(str(check_prefill(xb, Bc, lam, causal=causal, gpu=gb)))
    return reps


PREFILL = [
    # B, Hq, Hkv, T (capacity), d, Bc, lens
    (4, 4, 2, 700, 64, 64, [700, 0, 65, 300]),
    (3, 4, 1, 513, 128, 128, [1, 513, 256]),
    (2, 2, 2, 300, 128, 64, [299, 64]),
    # 8 head groups per sequence: the head-group -> XCD map turns once along the 21 query blocks
    (2, 16, 4, 2600, 128, 128, [2600, 1700]),
    # more than 64 sequences: the kv-group-per-XCD order instead of the in-kernel work list
    (72, 2, 2, 200, 64, 64, [(37 * b) % 201 for b in range(72)]),
]


@pytest.mark.parametrize("shape", PREFILL, ids=lambda s: "B%d_Hq%d_Hkv%d_T%d_d%d_Bc%d" % s[:6])
@pytest.mark.parametrize("lam", [0.0, 1e-3, 3e-2])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_ragged(shape, lam, causal):
    B, Hq, Hkv, T, d, Bc, lens = shape
    w = W.Workload("t", "prefill", B=B, Hq=Hq, Hkv=Hkv, d=d, T=T, Bc=Bc, lambdas=(lam,), hot_rate=0.03,
                   seed=505 + T)
    x = W.generate(w)
    say("prefill ragged", shape, lam, causal, check_prefill_ragged(x, lens, Bc, lam, causal))


def run_decode_ragged(xd, lens, Bc, lam, S):
    import torch
    import block_sparse_attention_flash_amd as bsa
    o_part, lse_part, skip, vskip = bsa.decode_ragged(xd["q"], xd["k"], xd["v"], lens_dev(lens), lam, S, Bc=Bc)
    o, lse = bsa.decode_combine(o_part, lse_part)
    torch.cuda.synchronize()
    return {k: t.cpu().numpy() for k, t in
            dict(o_part=o_part, lse_part=lse_part, skip=skip, vskip=vskip, o=o, lse=lse).items()}


def check_decode_ragged(x, lens, Bc, lam, S, xd=None):
    xd = xd or {k: to_device(v) for k, v in x.items()}
    g = run_decode_ragged(xd, lens, Bc, lam, S)
    reps = []
    for b, L in enumerate(lens):
        n = -(-L // Bc)
        assert np.all(g["skip"][b, :, n:] == 2) and np.all(g["vskip"][b, :, n:] == 2), "mask past sequence %d" % b
        xb = {"q": x["q"][b:b + 1], "k": np.ascontiguousarray(x["k"][b:b + 1, :, :L]),
              "v": np.ascontiguousarray(x["v"][b:b + 1, :, :L])}
        gb = {k: v[b:b + 1] for k, v in g.items()}
        gb["skip"], gb["vskip"] = gb["skip"][:, :, :n], gb["vskip"][:, :, :n]
        reps.append(str(check_decode(xb, Bc, lam, S, gpu=gb)))
    return reps


DECODE = [
    # B, Hq, Hkv, N (capacity), d, Bc, S, window, lens
    (5, 8, 2, 1000, 64, 64, 4, 64, [1000, 0, 100, 64, 999]),   # empty context, S > blocks
    (3, 32, 8, 4096, 128, 128, 16, 128, [4096, 1500, 129]),    # 16 splits over 2 blocks
    (2, 64, 1, 2000, 128, 128, 3, 0, [1, 2000]),               # MQA, a single key
    (4, 16, 1, 1536, 128, 64, 8, 0, [1536, 700, 300, 1]),
    (2, 8, 2, 40960, 128, 128, 8, 256, [40960, 23000]),      # paired workgroups, several phases per split
    (3, 128, 1, 1500, 128, 128, 4, 0, [1500, 0, 333]),         # G = 128: two head parts per split
    (2, 32, 8, 4096, 128, 128, 16, 128, [4096, 2000]),         # 256 units: one 8-wave workgroup per split
    (2, 8, 2, 9000, 64, 64, 40, 0, [9000, 3000]),              # 160 units at d = Bc = 64
    (6, 16, 4, 3000, 64, 128, 12, 0, [3000, 0, 1, 2999, 1500, 128]),  # 288 units: 4-wave workgroups, d = 64
]


@pytest.mark.parametrize("shape", DECODE, ids=lambda s: "B%d_Hq%d_Hkv%d_N%d_d%d_Bc%d_S%d" % s[:7])
@pytest.mark.parametrize("lam", [0.0, 1e-3, 1e-1])
def test_decode_ragged(shape, lam):
    B, Hq, Hkv, N, d, Bc, S, window, lens = shape
    w = W.Workload("t", "decode", B=B, Hq=Hq, Hkv=Hkv, d=d, T=N, Bc=Bc, lambdas=(lam,), hot_rate=0.02,
                   seed=606 + N, window=window, num_splits=S)
    x = W.generate(w)
    say("decode ragged", shape, lam, check_decode_ragged(x, lens, Bc, lam, S))


def test_decode_ragged_serving_batch():
    """16 sequences of 1K-32K context in a 32K-capacity cache (Llama-3.1-8B-like heads, 16 splits)."""
    rng = np.random.default_rng(7)
    lens = [int(v) for v in rng.integers(1024, 32769, size=16)]
    lens[3] = 32768
    w = W.Workload("t", "decode", B=16, Hq=32, Hkv=8, d=128, T=32768, Bc=128, lambdas=(1e-3,), hot_rate=0.01,
                   seed=707, window=512, num_splits=16)
    x = W.generate(w)
    reps = check_decode_ragged(x, lens, 128, 1e-3, 16)
    say("decode ragged serving batch", lens, reps[:3])


def test_full_lengths_equal_plain_calls_bitwise():
    import torch
    import block_sparse_attention_flash_amd as bsa
    w = W.Workload("t", "prefill", B=2, Hq=4, Hkv=2, d=128, T=600, Bc=128, lambdas=(1e-2,), hot_rate=0.03, seed=808)
    xd = {k: to_device(v) for k, v in W.generate(w).items()}
    a = bsa.prefill(xd["q"], xd["k"], xd["v"], 1e-2, Bc=128)
    r = bsa.prefill_ragged(xd["q"], xd["k"], xd["v"], lens_dev([600, 600]), 1e-2, Bc=128)
    for x, y in zip(a, r):
        assert torch.equal(x, y)
    w = W.Workload("t", "decode", B=2, Hq=32, Hkv=8, d=128, T=5000, Bc=128, lambdas=(1e-3,), hot_rate=0.01, seed=809,
                   num_splits=8)
    xd = {k: to_device(v) for k, v in W.generate(w).items()}
    a = bsa.decode(xd["q"], xd["k"], xd["v"], 1e-3, 8)
    r = bsa.decode_ragged(xd["q"], xd["k"], xd["v"], lens_dev([5000, 5000]), 1e-3, 8)
    for x, y in zip(a, r):
        assert torch.equal(x, y)


def test_padding_contents_do_not_matter():
    import torch
    import block_sparse_attention_flash_amd as bsa
    w = W.Workload("t", "decode", B=3, Hq=8, Hkv=2, d=128, T=3000, Bc=128, lambdas=(1e-3,), hot_rate=0.02, seed=810,
                   num_splits=4)
    xd = {k: to_device(v) for k, v in W.generate(w).items()}
    lens = [3000, 1234, 77]
    a = bsa.decode_ragged(xd["q"], xd["k"], xd["v"], lens_dev(lens), 1e-3, 4)
    for b, L in enumerate(lens):
        xd["k"][b, :, L:] = float("nan")
        xd["v"][b, :, L:] = float("inf")
    r = bsa.decode_ragged(xd["q"], xd["k"], xd["v"], lens_dev(lens), 1e-3, 4)
    for x, y in zip(a, r):
        assert torch.equal(x, y)
    w = W.Workload("t", "prefill", B=2, Hq=4, Hkv=1, d=64, T=500, Bc=64, lambdas=(1e-3,), hot_rate=0.03, seed=811)
    xd = {k: to_device(v) for k, v in W.generate(w).items()}
    lens = [321, 64]
    a = bsa.prefill_ragged(xd["q"], xd["k"], xd["v"], lens_dev(lens), 1e-3, Bc=64)
    for b, L in enumerate(lens):
        for t in ("q", "k", "v"):
            xd[t][b, :, L:] = float("nan")
    r = bsa.prefill_ragged(xd["q"], xd["k"], xd["v"], lens_dev(lens), 1e-3, Bc=64)
    for x, y in zip(a, r):
        assert torch.equal(x, y)
