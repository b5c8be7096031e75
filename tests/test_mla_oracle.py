"""Host pins of the MLA decode oracle (no GPU).

MLA in its absorbed decode form is split-KV decode in which every head reads
one shared cache row per token and the value is the row's latent prefix.  The
pins do not reuse the oracle's C code path: dense softmax attention written
out in numpy (lambda = 0, the splits merged), the numpy closed form of the
per-head decisions (block max minus the prefix max of the split's block
maxima), and the reduction to the already-pinned GQA decode oracle when the
value is the whole row (d_v = d_qk, one kv head, v = k).
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W


def f64(b):
    return W.bf16_bits_to_f32(b).astype(np.float64)


def mla_inputs(B=2, Hq=8, N=700, dqk=96, seed=41, hot=0.02):
    w = W.Workload("t", "decode", B=B, Hq=Hq, Hkv=1, d=dqk, T=N, Bc=64, lambdas=(1e-3,), hot_rate=hot, seed=seed,
                   window=64, num_splits=3, dv=64, scale=1.0 / math.sqrt(48.0))
    x = W.generate(w, parts=("q", "k"), threads=4)
    return w, np.ascontiguousarray(x["q"][:, :, 0]), np.ascontiguousarray(x["k"][:, 0])


def test_dense_at_lambda_zero():
    w, q, kv = mla_inputs()
    r = oracle.decode_mla(q, kv, w.Bc, 0.0, w.num_splits, w.score_scale, w.dv, threads=4)
    o, lse = oracle.combine(r["o_part_full"], r["lse_part_full"])
    assert not r["skip_full"].any()
    for b in range(w.B):
        K = f64(kv[b])
        for h in range(w.Hq):
            s = K @ f64(q[b, h]) * w.score_scale
            top = s.max()
            p = np.exp(s - top)
            np.testing.assert_allclose(o[b, h], (p @ K[:, :w.dv]) / p.sum(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], top + math.log(p.sum()), rtol=0, atol=1e-12)


@pytest.mark.parametrize("lam", [1e-3, 3e-2])
def test_decisions_match_closed_form(lam):
    w, q, kv = mla_inputs(seed=42)
    r = oracle.decode_mla(q, kv, w.Bc, lam, w.num_splits, w.score_scale, w.dv, threads=4)
    nk = -(-w.T // w.Bc)
    S = w.num_splits
    for b in range(w.B):
        K = f64(kv[b])
        for h in range(w.Hq):
            s = K @ f64(q[b, h]) * w.score_scale
            bm = np.array([s[j * w.Bc:(j + 1) * w.Bc].max() for j in range(nk)])
            want = np.empty(nk, bool)
            for sp in range(S):
                j0, j1 = sp * nk // S, (sp + 1) * nk // S
                want[j0:j1] = bm[j0:j1] - np.maximum.accumulate(bm[j0:j1]) < math.log(lam)
            np.testing.assert_array_equal(r["skip_full"][b, h].astype(bool), want)
        np.testing.assert_array_equal(r["vskip_full"][b], r["skip_full"][b].min(axis=0))
    assert r["skip_full"].any()


def test_reduces_to_gqa_decode_when_the_value_is_the_whole_row():
    w, q, kv = mla_inputs(dqk=64, seed=43)
    lam = 1e-2
    r = oracle.decode_mla(q, kv, w.Bc, lam, w.num_splits, 1.0 / math.sqrt(64.0), 64, threads=4)
    g = oracle.decode(q[:, :, None, :], kv[:, None], kv[:, None], w.Bc, lam, w.num_splits, threads=4)
    np.testing.assert_array_equal(r["skip_full"], g["skip_full"])
    np.testing.assert_allclose(r["o_part_full"], g["o_part_full"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse_part_full"], g["lse_part_full"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["margin_full"] if "margin_full" in r else r["margin"].reshape(g["margin_full"].shape),
                               g["margin_full"], rtol=0, atol=1e-12)
