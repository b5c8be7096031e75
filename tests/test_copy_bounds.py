"""The SGPR-base tile copies of the prefill and wide-group decode kernels stay inside their tensors (host only).

tests/copy_bounds.cpp is compiled with the host compiler against the same
offset functions the kernels call (block_sparse_attention_flash_amd/csrc/tile_copy.h)
and enumerates every lane's 16-byte read and LDS write for every supported
(d, Bc), one or two heads per prefill workgroup, the eight-wave decode
workgroup, and sequence (context) lengths with tails of
0, 1 and Bc - 1 rows (ragged batches give each sequence such a length).
"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_flash_amd", "csrc")


def test_tile_copies_stay_in_bounds(tmp_path):
    exe = str(tmp_path / "copy_bounds")
    subprocess.check_call(["g++", "-std=c++17", "-O2", "-Wall", "-I", CSRC, os.path.join(ROOT, "tests", "copy_bounds.cpp"),
                           "-o", exe])
    p = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    print(p.stdout)
    assert p.returncode == 0, p.stdout
    assert p.stdout.startswith("OK")
