"""Host pins of the ragged-batch oracle (no GPU).

A ragged batch gives every sequence its own length inside padded tensors; each
sequence must be exactly the plain call at its length.  The pins are
independent of the oracle's C code: dense softmax attention written out in
numpy at lambda = 0, and the decisions at lambda > 0 from the numpy closed form
of the decode margins (block max minus the prefix max of the split's block
maxima).  Also pinned: the merge identity of an empty split (o = 0,
lse = -inf), and an empty context (O = 0, LSE = -inf).
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W


def f64(b):
    return W.bf16_bits_to_f32(b).astype(np.float64)


def dense(qf, kf, vf, causal):
    """Softmax attention in float64: rows of qf over keys kf (causal: row t sees keys <= t)."""
    s = qf @ kf.T / math.sqrt(qf.shape[1])
    if causal:
        s = np.where(np.tril(np.ones(s.shape, bool)), s, -np.inf)
    top = s.max(axis=1, keepdims=True)
    p = np.exp(s - top)
    l = p.sum(axis=1, keepdims=True)
    return (p @ vf) / l, (top + np.log(l))[:, 0]


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_ragged_dense_and_padding(causal):
    w = W.Workload("t", "prefill", B=4, Hq=4, Hkv=2, d=32, T=300, Bc=64, lambdas=(0.0,), hot_rate=0.03, seed=31)
    x = W.generate(w, threads=4)
    lens = [300, 0, 129, 64]
    r = oracle.prefill_ragged(x["q"], x["k"], x["v"], lens, w.Bc, 0.0, causal=causal, threads=4)
    for b, L in enumerate(lens):
        for h in range(w.Hq):
            if L:
                o, lse = dense(f64(x["q"][b, h, :L]), f64(x["k"][b, h // w.G, :L]), f64(x["v"][b, h // w.G, :L]),
                               causal)
                np.testing.assert_allclose(r["o_full"][b, h, :L], o, rtol=0, atol=1e-12)
                np.testing.assert_allclose(r["lse_full"][b, h, :L], lse, rtol=0, atol=1e-12)
            assert np.all(r["o_full"][b, h, L:] == 0) and np.all(np.isneginf(r["lse_full"][b, h, L:]))
            n = -(-L // w.Bc)
            assert np.all(r["mask_full"][b, h, n:, :] == 2) and np.all(r["mask_full"][b, h, :, n:] == 2)
            assert np.all(np.isnan(r["margin_full"][b, h, :, n:]))


def test_decode_ragged_dense_empty_splits_and_empty_context():
    S = 6
    w = W.Workload("t", "decode", B=5, Hq=8, Hkv=2, d=32, T=700, Bc=64, lambdas=(0.0,), hot_rate=0.02, seed=32,
                   num_splits=S)
    x = W.generate(w, threads=4)
    lens = [700, 100, 0, 64, 383]   # 11, 2 (< S: empty splits), 0, 1 and 6 blocks
    r = oracle.decode_ragged(x["q"], x["k"], x["v"], lens, w.Bc, 0.0, S, threads=4)
    o, lse = oracle.combine(r["o_part_full"], r["lse_part_full"])
    for b, L in enumerate(lens):
        nkb = -(-L // w.Bc)
        for h in range(w.Hq):
            for s in range(S):
                empty = (s + 1) * nkb // S == s * nkb // S
                if empty:
                    assert np.all(r["o_part_full"][b, h, s] == 0) and np.isneginf(r["lse_part_full"][b, h, s])
            if L == 0:
                assert np.all(o[b, h] == 0) and np.isneginf(lse[b, h])
                continue
            od, ld = dense(f64(x["q"][b, h]), f64(x["k"][b, h // w.G, :L]), f64(x["v"][b, h // w.G, :L]), False)
            np.testing.assert_allclose(o[b, h], od[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], ld[0], rtol=0, atol=1e-12)
        assert np.all(r["skip_full"][b, :, nkb:] == 2) and np.all(r["vskip_full"][b, :, nkb:] == 2)


@pytest.mark.parametrize("lam", [1e-3, 5e-2])
def test_decode_ragged_decisions_match_closed_form(lam):
    S = 3
    w = W.Workload("t", "decode", B=3, Hq=4, Hkv=1, d=32, T=900, Bc=64, lambdas=(lam,), hot_rate=0.02, seed=33,
                   window=64, num_splits=S)
    x = W.generate(w, threads=4)
    lens = [900, 450, 130]
    r = oracle.decode_ragged(x["q"], x["k"], x["v"], lens, w.Bc, lam, S, threads=4)
    for b, L in enumerate(lens):
        nkb = -(-L // w.Bc)
        kf = f64(x["k"][b, 0, :L])
        for h in range(w.Hq):
            s = kf @ f64(x["q"][b, h, 0]) / math.sqrt(w.d)
            bm = np.array([s[j * w.Bc:(j + 1) * w.Bc].max() for j in range(nkb)])
            want = np.empty(nkb, bool)
            for sp in range(S):
                j0, j1 = sp * nkb // S, (sp + 1) * nkb // S
                want[j0:j1] = bm[j0:j1] - np.maximum.accumulate(bm[j0:j1]) < math.log(lam)
            np.testing.assert_array_equal(r["skip_full"][b, h, :nkb].astype(bool), want)


def test_combine_ignores_empty_splits():
    rng = np.random.default_rng(2)
    o_part = rng.normal(size=(3, 4, 16))
    lse_part = rng.normal(size=(3, 4))
    o_ref, l_ref = oracle.combine(o_part[:, :2], lse_part[:, :2])
    o_part[:, 2:] = 0.0
    lse_part[:, 2:] = -np.inf
    o, l = oracle.combine(o_part, lse_part)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-15)
    np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-15)
