"""Host-only checks of the C ABI library: it loads, exports exactly what
include/blasst.h declares, and rejects bad arguments before touching HIP
(no GPU is needed for any call made here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "blasst.h")
LIB = os.path.join(ROOT, "block_sparse_attention_flash_amd", "libblasst.so")


def declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(blasst_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import block_sparse_attention_flash_amd as bsa
        bsa.build()
    return ctypes.CDLL(LIB)


def test_header_declares_the_entry_points():
    assert declared() == ["blasst_decode", "blasst_decode_combine", "blasst_decode_dense",
                          "blasst_decode_load_ceiling", "blasst_decode_margins", "blasst_decode_mla",
                          "blasst_decode_ragged", "blasst_decode_step", "blasst_decode_step_noalloc",
                          "blasst_decode_step_noalloc_max_bytes", "blasst_decode_step_workspace_size",
                          "blasst_prefill", "blasst_prefill_dense", "blasst_prefill_margins", "blasst_prefill_ragged",
                          "blasst_status_string"]


def test_exports_match_header(lib):
    for name in declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], stdout=subprocess.PIPE, text=True).stdout
    exported = sorted(set(re.findall(r"\b(blasst_\w+)\b", out)))
    assert exported == declared()


def test_status_strings(lib):
    lib.blasst_status_string.restype = ctypes.c_char_p
    names = [lib.blasst_status_string(i).decode() for i in range(5)]
    assert names[0] == "ok" and len(set(names)) == 5
    assert lib.blasst_status_string(99).decode() == "unknown status"


P = ctypes.c_void_p
I = ctypes.c_int
D = ctypes.c_double
FAKE = P(0x1000)   # 16-byte aligned, never dereferenced: validation fails first


def prefill(lib, q=FAKE, o=FAKE, B=1, Hq=4, T=256, d=128, G=4, Bc=128, lam=1e-3, causal=1):
    f = lib.blasst_prefill
    f.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, D, I, P]
    return f(q, FAKE, FAKE, o, None, None, B, Hq, T, d, G, Bc, lam, causal, None)


def decode(lib, q=FAKE, B=1, Hq=4, N=256, d=128, G=4, Bc=128, lam=1e-3, S=2, causal=1):
    f = lib.blasst_decode
    f.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, D, I, I, P]
    return f(q, FAKE, FAKE, FAKE, FAKE, None, None, B, Hq, N, d, G, Bc, lam, causal, S, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(B=-1), 1), (dict(T=-5), 1), (dict(G=0), 1),
    (dict(G=3), 1), (dict(lam=1.0), 1), (dict(lam=-1e-3), 1), (dict(lam=float("nan")), 1),
    (dict(causal=2), 1), (dict(q=P(0x1008)), 1), (dict(d=96), 2), (dict(Bc=32), 2), (dict(d=256), 2),
    (dict(B=0), 0), (dict(T=0), 0),
])
def test_prefill_validation(lib, kw, status):
    assert prefill(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(N=0), 1), (dict(S=0), 1), (dict(S=3), 1), (dict(G=5), 1),
    (dict(lam=1.5), 1), (dict(causal=-1), 1), (dict(d=80), 2), (dict(Bc=256, S=1), 2),
    (dict(Hq=256, G=256), 2), (dict(B=0), 0), (dict(Hq=0), 0),
])
def test_decode_validation(lib, kw, status):
    assert decode(lib, **kw) == status


def test_combine_validation(lib):
    f = lib.blasst_decode_combine
    f.argtypes = [P, P, P, P, I, I, I, I, P]
    assert f(None, FAKE, FAKE, None, 1, 4, 128, 2, None) == 1
    assert f(FAKE, FAKE, FAKE, None, 1, 4, 128, 0, None) == 1
    assert f(FAKE, FAKE, FAKE, None, 1, 4, 96, 2, None) == 2
    assert f(FAKE, FAKE, FAKE, None, 0, 4, 128, 2, None) == 0


def prefill_margins(lib, q=FAKE, margin=FAKE, B=1, Hq=4, T=256, d=128, G=4, Bc=128, causal=1):
    f = lib.blasst_prefill_margins
    f.argtypes = [P, P, P, I, I, I, I, I, I, I, P]
    return f(q, FAKE, margin, B, Hq, T, d, G, Bc, causal, None)


def decode_margins(lib, q=FAKE, margin=FAKE, B=1, Hq=4, N=256, d=128, G=4, Bc=128, S=2):
    f = lib.blasst_decode_margins
    f.argtypes = [P, P, P, P, I, I, I, I, I, I, I, P]
    return f(q, FAKE, margin, None, B, Hq, N, d, G, Bc, S, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(margin=None), 1), (dict(B=-1), 1), (dict(G=3), 1), (dict(causal=2), 1),
    (dict(q=P(0x1008)), 1), (dict(d=96), 2), (dict(Bc=32), 2), (dict(B=0), 0), (dict(T=0), 0),
])
def test_prefill_margins_validation(lib, kw, status):
    assert prefill_margins(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(margin=None), 1), (dict(N=0), 1), (dict(S=0), 1), (dict(S=3), 1), (dict(G=5), 1),
    (dict(d=80), 2), (dict(Hq=256, G=256), 2), (dict(B=0), 0), (dict(Hq=0), 0),
])
def test_decode_margins_validation(lib, kw, status):
    assert decode_margins(lib, **kw) == status


def prefill_ragged(lib, lens=FAKE, q=FAKE, B=2, Hq=4, T=256, d=128, G=4, Bc=128, lam=1e-3, causal=1):
    f = lib.blasst_prefill_ragged
    f.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, D, I, P]
    return f(q, FAKE, FAKE, FAKE, None, None, lens, B, Hq, T, d, G, Bc, lam, causal, None)


def decode_ragged(lib, lens=FAKE, q=FAKE, B=2, Hq=4, N=256, d=128, G=4, Bc=128, lam=1e-3, S=2):
    f = lib.blasst_decode_ragged
    f.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, D, I, P]
    return f(q, FAKE, FAKE, FAKE, FAKE, None, None, lens, B, Hq, N, d, G, Bc, lam, S, None)


@pytest.mark.parametrize("kw,status", [
    (dict(lens=None), 1), (dict(lens=P(0x1002)), 1), (dict(q=None), 1), (dict(T=-1), 1), (dict(G=3), 1),
    (dict(lam=1.0), 1), (dict(causal=2), 1), (dict(d=96), 2), (dict(B=0, lens=None), 0), (dict(T=0, lens=None), 0),
])
def test_prefill_ragged_validation(lib, kw, status):
    assert prefill_ragged(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(lens=None), 1), (dict(lens=P(0x1001)), 1), (dict(q=None), 1), (dict(N=0), 1), (dict(S=3), 1),
    (dict(S=0), 1), (dict(lam=-1.0), 1), (dict(Bc=256, S=1), 2), (dict(Hq=256, G=256), 2),
    (dict(B=0, lens=None), 0),
])
def test_decode_ragged_validation(lib, kw, status):
    assert decode_ragged(lib, **kw) == status


def decode_mla(lib, q=FAKE, kv=FAKE, B=2, Hq=128, N=4096, dqk=576, dv=512, Bc=64, scale=0.0722, lam=1e-3, S=4):
    f = lib.blasst_decode_mla
    f.argtypes = [P, P, P, P, P, I, I, I, I, I, I, D, D, I, P]
    return f(q, kv, FAKE, FAKE, None, B, Hq, N, dqk, dv, Bc, scale, lam, S, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(kv=None), 1), (dict(kv=P(0x1004)), 1), (dict(N=0), 1), (dict(S=0), 1),
    (dict(S=65), 1), (dict(dv=600), 1), (dict(scale=0.0), 1), (dict(scale=float("inf")), 1),
    (dict(scale=float("nan")), 1), (dict(lam=1.0), 1), (dict(dqk=128, dv=128), 2), (dict(Bc=128), 2),
    (dict(Hq=16), 2), (dict(Hq=48), 2), (dict(Bc=32, Hq=96), 2), (dict(Bc=16), 2), (dict(B=0), 0),
    (dict(Hq=0), 0), (dict(B=0, Bc=32), 0),
])
def test_decode_mla_validation(lib, kw, status):
    assert decode_mla(lib, **kw) == status


def test_combine_accepts_the_latent_width(lib):
    f = lib.blasst_decode_combine
    f.argtypes = [P, P, P, P, I, I, I, I, P]
    assert f(FAKE, FAKE, FAKE, None, 0, 128, 512, 16, None) == 0   # B = 0: validated, nothing launched
    assert f(FAKE, FAKE, FAKE, None, 0, 128, 256, 16, None) == 2


def test_dense_references_validate_like_the_plain_calls(lib):
    f = lib.blasst_prefill_dense
    f.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, P]
    assert f(None, FAKE, FAKE, FAKE, None, 1, 4, 256, 128, 4, 128, 1, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, None, 1, 4, 256, 96, 4, 128, 1, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, None, 0, 4, 256, 128, 4, 128, 1, None) == 0
    g = lib.blasst_decode_dense
    g.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, P]
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 256, 128, 4, 128, 3, None) == 1   # 3 splits > 2 blocks
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 256, 128, 4, 256, 1, None) == 2
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4, 256, 128, 4, 128, 1, None) == 0


def test_load_ceiling_validates_like_decode(lib):
    f = lib.blasst_decode_load_ceiling
    f.argtypes = [P, P, I, I, I, I, I, I, P]
    assert f(FAKE, FAKE, 1, 8, 256, 128, 128, 3, None) == 1     # 3 splits > 2 blocks
    assert f(FAKE, FAKE, 1, 8, 256, 96, 128, 1, None) == 2      # d = 96
    assert f(None, FAKE, 1, 8, 256, 128, 128, 1, None) == 1     # null k
    assert f(P(0x1008), FAKE, 1, 8, 256, 128, 128, 1, None) == 1  # misaligned k
    assert f(FAKE, FAKE, 0, 8, 256, 128, 128, 1, None) == 0     # empty batch: nothing launched


def test_decode_step_validates_its_workspace(lib):
    sz = lib.blasst_decode_step_workspace_size
    sz.argtypes = [I, I, I, I]
    sz.restype = ctypes.c_size_t
    assert sz(1, 32, 128, 16) == 32 * 16 * 129 * 4
    assert sz(1, 32, 128, 0) == 0 and sz(-1, 32, 128, 4) == 0
    f = lib.blasst_decode_step
    f.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_size_t, I, I, I, I, I, I, D, I, I, P]
    need = 4 * 2 * 129 * 4
    ok = (FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, need, 1, 4, 256, 128, 4, 128, 1e-3, 1, 2, None)

    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[{"o": 3, "ws": 7, "ws_bytes": 8, "B": 9, "S": 17, "lam": 15}[k]] = v
        return f(*a)
    assert call(ws=None) == 1
    assert call(ws=P(0x1004)) == 1                # misaligned workspace
    assert call(ws_bytes=need - 1) == 1           # too small
    assert call(o=None) == 1
    assert call(S=3, ws_bytes=10**6) == 1         # 3 splits > 2 blocks
    assert call(lam=1.0) == 1
    assert call(B=0, ws=None, o=None) == 0        # empty batch: validated, nothing launched


def test_decode_step_noalloc_validates_before_touching_hip(lib):
    cap = lib.blasst_decode_step_noalloc_max_bytes
    cap.argtypes = []
    cap.restype = ctypes.c_size_t
    assert cap() == 32 << 20
    f = lib.blasst_decode_step_noalloc
    f.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, D, I, I, P]
    assert f(FAKE, FAKE, FAKE, None, None, None, None, 1, 4, 256, 128, 4, 128, 1e-3, 1, 2, None) == 1  # NULL o
    assert f(FAKE, FAKE, FAKE, FAKE, None, None, None, 1, 4, 256, 128, 4, 128, 2.0, 1, 2, None) == 1   # lambda
    # partials of 64 x 64 heads x 16 splits x 129 fp32 exceed the 32 MiB array: rejected before any HIP call
    assert f(FAKE, FAKE, FAKE, FAKE, None, None, None, 64, 64, 2048, 128, 64, 128, 1e-3, 1, 16, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, None, None, None, 0, 4, 256, 128, 4, 128, 1e-3, 1, 2, None) == 0  # empty batch
