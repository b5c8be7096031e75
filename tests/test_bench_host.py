"""Host logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte count
of a decode launch, and the counter records the bench line quotes."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU only" in p.stderr
    assert p.stdout == ""


def test_decode_bytes_by_hand():
    # B = 2, Hq = 4, Hkv = 2, N = 300 (blocks of 128, 128, 44), d = 64, 3 splits
    w = W.Workload("t", "decode", B=2, Hq=4, Hkv=2, d=64, T=300, Bc=128, lambdas=(1e-3,), hot_rate=0.0, seed=1,
                   num_splits=3)
    vskip = np.zeros((2, 2, 3), np.uint8)
    vskip[0, 1, 0] = 1   # a full block unread
    vskip[1, 0, 2] = 1   # the 44-row last block unread
    by = bench.decode_bytes(w, vskip)
    k = 2 * 2 * 300 * 64 * 2
    v_kept = (2 * 2 * 300 - 128 - 44) * 64 * 2
    q = 2 * 4 * 64 * 2
    part = 2 * 4 * 3 * (64 + 1) * 4
    masks = 2 * 4 * 3 + 2 * 2 * 3
    assert by["k"] == k and by["v_kept"] == v_kept and by["v_dense"] == k
    assert by["split"] == k + v_kept + q + part + masks
    assert by["combine"] == part + 2 * 4 * (64 + 1) * 4


def test_counter_records_match_the_sources():
    # the bench line quotes these; a kernel change without re-taken counters turns them to null
    assert bench.measured_traffic("decode_split_kernel", "decode_32k") is not None
    assert bench.measured_traffic("prefill_kernel", "prefill_32k") is not None


def test_rotation_defeats_the_infinity_cache():
    # every timed loop rotates at least 2 GiB of KV (8x the 256 MB Infinity Cache), whatever the
    # loads' cache policy keeps there; --copies overrides the count
    class Args:
        copies = None
    for name in ("decode_32k", "decode_128k_b16", "decode_mqa_16k"):
        w = W.CONFIGS[name]
        footprint = 2 * w.B * w.Hkv * w.T * w.d * 2
        n = bench.kv_copies(Args, footprint)
        assert n * footprint >= bench.ROTATE_BYTES and (n - 1) * footprint < bench.ROTATE_BYTES
    assert bench.kv_copies(Args, 2 * 1024 ** 3) == 1
    assert bench.kv_copies(Args, 134217728) == 16
    Args.copies = 3
    assert bench.kv_copies(Args, 134217728) == 3
