"""The allocation-free decode step (blasst_decode_step_noalloc) through the C ABI.

Two calls in a row, the second with a smaller input, each compared with the
entry point it is a variant of (blasst_decode_step, the partials in a
caller-owned workspace): the outputs and masks must be equal bit for bit (the
same kernels), and the merged output must match the FP64 oracle within the
parity tolerances.  The second call must not change the free device memory,
and a call whose partials exceed the library's per-GPU array is rejected
before anything runs.  Every decode launch shape (4-wave and paired 16-head
workgroups, 32 heads, paired 64-head workgroups, head parts, the wide-group
kernel, up to 40 splits) is also run twice in a row through the array.
"""
import ctypes
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


def run_both(shape):
    import torch
    import block_sparse_attention_flash_amd as bsa
    B, Hq, Hkv, N, d, Bc, S, lam, seed = shape
    w = W.Workload("t", "decode", B=B, Hq=Hq, Hkv=Hkv, d=d, T=N, Bc=Bc, lambdas=(lam,), hot_rate=0.02, seed=seed,
                   window=64, num_splits=S)
    x = W.generate(w)
    xd = {k: to_device(v) for k, v in x.items()}
    nk = -(-N // Bc)
    outs = []
    for noalloc in (False, True):
        o = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        skip = torch.full((B, Hq, nk), 7, dtype=torch.uint8, device="cuda")
        vskip = torch.full((B, Hkv, nk), 7, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        if noalloc:
            free0 = torch.cuda.mem_get_info()[0]
            bsa.blasst_decode_step_noalloc(xd["q"], xd["k"], xd["v"], o, lse, skip, vskip, Bc, lam, S)
            torch.cuda.synchronize()
            free1 = torch.cuda.mem_get_info()[0]
        else:
            ws = torch.empty(bsa.decode_step_workspace_size(B, Hq, d, S), dtype=torch.uint8, device="cuda")
            bsa.blasst_decode_step(xd["q"], xd["k"], xd["v"], o, lse, skip, vskip, ws, Bc, lam, S)
            torch.cuda.synchronize()
        outs.append((o, lse, skip, vskip))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    o, lse, skip, _ = (t.cpu().numpy() for t in outs[1])
    ref = oracle.decode(x["q"], x["k"], x["v"], Bc, lam, S)
    rep = Report()
    diff = compare_masks(skip, ref["skip_full"], ref["margin_full"], rep, "skip")
    if diff.any():  # adopt the GPU's decision on near-threshold blocks (both are valid results)
        f = np.where(diff, skip, -1).astype(np.int8).reshape(B * Hkv, Hq // Hkv, -1)
        ref = oracle.decode(x["q"], x["k"], x["v"], Bc, lam, S, force=f)
    o_ref, lse_ref = oracle.combine(ref["o_part_full"], ref["lse_part_full"])
    compare_rows(o, o_ref, rep, "o")
    compare_lse(lse, lse_ref, rep, "lse")
    print("noalloc decode step", shape, rep, flush=True)
    sys.stdout.flush()
    return free0, free1


def test_noalloc_two_calls_second_smaller():
    # decode_32k, then a smaller batch: the second call reuses (and must fully rewrite) the array
    run_both((1, 32, 8, 32768, 128, 128, 16, 1e-3, 1501))
    free0, free1 = run_both((2, 8, 2, 3000, 64, 64, 3, 1e-1, 1502))
    assert free1 == free0


MERGE_SHAPES = [
    # B, Hq, Hkv, N, d, Bc, S, lambda, seed
    (4, 16, 4, 5000, 64, 64, 20, 1e-3, 1601),    # 320 units, 16 heads: 4-wave workgroups
    (2, 64, 2, 3000, 128, 128, 5, 1e-3, 1602),   # 32 heads
    (2, 64, 1, 3000, 64, 128, 5, 1e-1, 1603),    # 64 heads at d = 64: paired 64-head workgroups
    (1, 128, 1, 3000, 128, 128, 4, 1e-3, 1604),  # 128 heads: two head parts per split
    (2, 8, 2, 9000, 64, 64, 32, 0.5, 1605),      # 32 splits
    (3, 8, 8, 3000, 128, 64, 40, 1e-3, 1606),    # 40 splits (the merge's loop form)
    (8, 64, 1, 2000, 128, 128, 4, 1e-3, 1607),   # 64 heads at d = 128: the wide-group kernel
]


@pytest.mark.parametrize("shape", MERGE_SHAPES, ids=lambda s: "B%d_Hq%d_Hkv%d_N%d_d%d_Bc%d_S%d" % s[:7])
def test_noalloc_merge_paths_twice(shape):
    run_both(shape)
    run_both(shape)


def test_noalloc_rejects_partials_beyond_the_array():
    import torch
    import block_sparse_attention_flash_amd as bsa
    lib = bsa._load()
    cap = bsa.decode_step_noalloc_max_bytes()
    B, Hq, d, S, N = 64, 64, 128, 16, 2048
    assert B * Hq * S * (d + 1) * 4 > cap >= 32 << 20
    q = torch.zeros((B, Hq, 1, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, 1, N, d), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((B, Hq, d), dtype=torch.float32, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = lib.blasst_decode_step_noalloc(P(q), P(k), P(k), P(o), None, None, None, B, Hq, N, d, Hq, 128,
                                        ctypes.c_double(1e-3), 1, S, None)
    assert st == bsa.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0  # nothing ran
