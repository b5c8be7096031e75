"""Pins for the FP64 oracle: it is checked against things other than itself.

* hand-worked cases (tests/golden/hand_cases.json) whose decisions and outputs
  were derived on paper from the BLASST blog's rule;
* the dense limit: lambda = 0 must give textbook softmax attention (scipy's
  softmax / logsumexp), for prefill and for every split count in decode;
* a closed form built on two facts the blog's rule implies: a skipped block
  never moves the running max, so the running max before block j is the prefix
  max of the block maxima, and the result is a plain softmax over the kept
  keys.  Decisions must match exactly and outputs to 1e-10;
* invariants from the blog's decision-rule and error-bound sections: a skipped
  token's true weight is < lambda, Z >= 1, the global-max block and any block
  that sets a new max are kept, the App. B error identity and bound, and
  monotonicity of the skip set in lambda.
None of these recomputes the oracle's own recurrence.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")
EXPR_NS = {"exp": math.exp, "log": math.log}


def bits(x):
    x = np.asarray(x, np.float32)
    b = W.to_bf16_bits(x)
    assert np.array_equal(W.bf16_bits_to_f32(b), x), "fixture value not exact in bf16"
    return b


def f64(b):
    return W.bf16_bits_to_f32(b).astype(np.float64)


def ev(expr):
    return eval(expr, {"__builtins__": {}}, EXPR_NS)  # fixture formulas: exp/log only


# --------------------------------------------------------------------------- #
# Hand-worked cases
# --------------------------------------------------------------------------- #
with open(GOLDEN) as fh:
    CASES = json.load(fh)


@pytest.mark.parametrize("case", [c for c in CASES["decode"] if "special" not in c], ids=lambda c: c["name"])
def test_golden_decode(case):
    Hkv = case.get("Hkv", 1)
    q = bits(case["q"])[None, :, None, :]  # [1,Hq,1,1]
    k = bits(case["k"]).reshape(1, Hkv, -1, 1)
    v = bits(case["v"]).reshape(1, Hkv, -1, 1)
    S = case["num_splits"]
    r = oracle.decode(q, k, v, case["Bc"], case["lambda"], S)
    assert r["skip_full"][0].tolist() == case["skip"]
    if "vskip" in case:
        assert r["vskip_full"][0].tolist() == case["vskip"]
    if "o_part" in case:
        want = np.array([[ev(e) for e in row] for row in case["o_part"]])
        np.testing.assert_allclose(r["o_part_full"][0, :, :, 0], want, rtol=1e-13)
        want = np.array([[ev(e) for e in row] for row in case["lse_part"]])
        np.testing.assert_allclose(r["lse_part_full"][0], want, rtol=1e-13, atol=1e-14)
    o, lse = oracle.combine(r["o_part_full"], r["lse_part_full"])
    np.testing.assert_allclose(o[0, :, 0], [ev(e) for e in case["o"]], rtol=1e-13)
    np.testing.assert_allclose(lse[0], [ev(e) for e in case["lse"]], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("case", CASES["prefill"], ids=lambda c: c["name"])
def test_golden_prefill(case):
    q = bits(case["q"])[None, None]
    k = bits(case["k"])[None, None]
    v = bits(case["v"])[None, None]
    r = oracle.prefill(q, k, v, case["Bc"], case["lambda"], causal=True)
    assert r["mask_full"][0, 0].tolist() == case["mask"]
    np.testing.assert_allclose(r["o_full"][0, 0, :, 0], [ev(e) for e in case["o"]], rtol=1e-13)
    np.testing.assert_allclose(r["lse_full"][0, 0], [ev(e) for e in case["lse"]], rtol=1e-13, atol=1e-14)


def test_golden_worked_mass_bound():
    """Blog, decision-rule section: at lambda=1e-3 a skipped 128-token block carries < 0.128."""
    case = next(c for c in CASES["decode"] if c["name"] == "worked_mass_bound_128")
    Bc, lam = case["Bc"], case["lambda"]
    keys = np.full(2 * Bc, -100.0, np.float32)
    keys[0] = 0.0
    keys[Bc:] = -7.0
    vals = np.arange(2 * Bc, dtype=np.float32) % 7
    q = bits([[1.0]])[None, :, None, :]
    k = bits(keys[:, None])[None, None]
    v = bits(vals[:, None])[None, None]
    r = oracle.decode(q, k, v, Bc, lam, 1)
    assert r["skip_full"][0].tolist() == case["skip"]
    s = keys.astype(np.float64)
    p = softmax(s)
    mass = p[Bc:].sum()
    assert mass == pytest.approx(ev(case["skipped_mass"]), rel=1e-12)
    assert mass < ev(case["mass_bound"])
    assert p[Bc:].max() < lam


# --------------------------------------------------------------------------- #
# Independent closed form (prefix max of block maxima + masked softmax)
# --------------------------------------------------------------------------- #
def closed_form_prefill(qf, kf, vf, Bc, Br, lam, causal=True):
    """qf [T,d], kf/vf [T,d] float64 -> mask [nq,nk], out [T,d], lse [T], scores."""
    T, d = qf.shape
    thr = math.log(lam) if lam > 0 else -math.inf
    s = qf @ kf.T / math.sqrt(d)
    if causal:
        s[np.triu_indices(T, 1)] = -np.inf
    nq, nk = -(-T // Br), -(-T // Bc)
    mask = np.full((nq, nk), 2, np.uint8)
    out = np.empty((T, d))
    lse = np.empty(T)
    for i in range(nq):
        r0, r1 = i * Br, min(T, (i + 1) * Br)
        jend = (r1 - 1) // Bc + 1 if causal else nk
        bm = np.stack([s[r0:r1, j * Bc:min(T, (j + 1) * Bc)].max(axis=1) for j in range(jend)], axis=1)
        prefix = np.maximum.accumulate(bm, axis=1)
        with np.errstate(invalid="ignore"):
            vote = np.isneginf(bm) | (bm - prefix < thr)
        skip = vote.all(axis=0)
        mask[i, :jend] = skip
        keep_cols = np.concatenate([np.arange(j * Bc, min(T, (j + 1) * Bc)) for j in range(jend) if not skip[j]])
        sk = s[r0:r1][:, keep_cols]
        out[r0:r1] = softmax(sk, axis=1) @ vf[keep_cols]
        lse[r0:r1] = logsumexp(sk, axis=1)
    return mask, out, lse, s


def closed_form_decode_row(qrow, kf, vf, Bc, lam, S):
    """One query row against [N,d] keys: per-split skip list, combined out/lse."""
    N, d = kf.shape
    thr = math.log(lam) if lam > 0 else -math.inf
    s = kf @ qrow / math.sqrt(d)
    nk = -(-N // Bc)
    bm = np.array([s[j * Bc:min(N, (j + 1) * Bc)].max() for j in range(nk)])
    skip = np.zeros(nk, bool)
    for sp in range(S):
        j0, j1 = sp * nk // S, (sp + 1) * nk // S
        prefix = np.maximum.accumulate(bm[j0:j1])
        skip[j0:j1] = bm[j0:j1] - prefix < thr
    keep = np.concatenate([np.arange(j * Bc, min(N, (j + 1) * Bc)) for j in range(nk) if not skip[j]])
    return skip, softmax(s[keep]) @ vf[keep], logsumexp(s[keep]), s


SMALL_PREFILL = [
    # (B, Hq, Hkv, T, d, Bc, hot)
    (1, 4, 2, 256, 32, 32, 0.02),
    (2, 2, 1, 200, 16, 32, 0.03),  # ragged last blocks
    (1, 3, 3, 128, 8, 16, 0.05),
]


def small_prefill(B, Hq, Hkv, T, d, Bc, hot, seed=7):
    w = W.Workload("t", "prefill", B=B, Hq=Hq, Hkv=Hkv, d=d, T=T, Bc=Bc, lambdas=(1e-3,),
                   hot_rate=hot, seed=seed)
    return w, W.generate(w, threads=4)


@pytest.mark.parametrize("shape", SMALL_PREFILL)
@pytest.mark.parametrize("lam", [0.0, 1e-4, 1e-3, 1e-2, 1e-1, 0.5])
def test_prefill_matches_closed_form(shape, lam):
    w, x = small_prefill(*shape)
    r = oracle.prefill(x["q"], x["k"], x["v"], w.Bc, lam, threads=4)
    G = w.G
    for b in range(w.B):
        for h in range(w.Hq):
            qf, kf, vf = f64(x["q"][b, h]), f64(x["k"][b, h // G]), f64(x["v"][b, h // G])
            mask, out, lse, _ = closed_form_prefill(qf, kf, vf, w.Bc, w.Bc, lam)
            marg = r["margin_full"][b, h]
            exact = ~(np.abs(marg) < 1e-9)  # float64 ties at the threshold are not pinned
            assert np.array_equal(r["mask_full"][b, h][exact], mask[exact])
            if exact.all():
                np.testing.assert_allclose(r["o_full"][b, h], out, rtol=1e-10, atol=1e-12)
                np.testing.assert_allclose(r["lse_full"][b, h], lse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("lam", [0.0, 1e-3, 3e-2, 0.3])
@pytest.mark.parametrize("S", [1, 3, 8])
def test_decode_matches_closed_form(lam, S):
    w = W.Workload("t", "decode", B=2, Hq=8, Hkv=2, d=32, T=1000, Bc=64, lambdas=(lam,),
                   hot_rate=0.02, seed=11, window=64, num_splits=S)
    x = W.generate(w, threads=4)
    r = oracle.decode(x["q"], x["k"], x["v"], w.Bc, lam, S, threads=4)
    o, lse = oracle.combine(r["o_part_full"], r["lse_part_full"])
    for b in range(w.B):
        vskip_cf = np.ones((w.Hkv, -(-w.T // w.Bc)), bool)
        for h in range(w.Hq):
            kf, vf = f64(x["k"][b, h // w.G]), f64(x["v"][b, h // w.G])
            skip, out, l, _ = closed_form_decode_row(f64(x["q"][b, h, 0]), kf, vf, w.Bc, lam, S)
            assert np.array_equal(r["skip_full"][b, h].astype(bool), skip)
            vskip_cf[h // w.G] &= skip
            np.testing.assert_allclose(o[b, h], out, rtol=1e-10, atol=1e-12)
            assert lse[b, h] == pytest.approx(l, rel=1e-12, abs=1e-12)
        assert np.array_equal(r["vskip_full"][b].astype(bool), vskip_cf)


# --------------------------------------------------------------------------- #
# Dense limit (lambda = 0 and lambda -> 0): textbook softmax attention
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("shape", SMALL_PREFILL)
@pytest.mark.parametrize("lam", [0.0, 1e-300])
def test_prefill_dense_limit(shape, lam):
    w, x = small_prefill(*shape)
    r = oracle.prefill(x["q"], x["k"], x["v"], w.Bc, lam, threads=4)
    assert (r["mask_full"] != 1).all()
    T, d = w.T, w.d
    causal = np.tril(np.ones((T, T), bool))
    for b in range(w.B):
        for h in range(w.Hq):
            s = f64(x["q"][b, h]) @ f64(x["k"][b, h // w.G]).T / math.sqrt(d)
            s = np.where(causal, s, -np.inf)
            np.testing.assert_allclose(r["o_full"][b, h], softmax(s, axis=1) @ f64(x["v"][b, h // w.G]),
                                       rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(r["lse_full"][b, h], logsumexp(s, axis=1), rtol=1e-12)


@pytest.mark.parametrize("S", [1, 2, 5, 16])
def test_decode_dense_limit_any_split(S):
    w = W.Workload("t", "decode", B=1, Hq=4, Hkv=1, d=16, T=1024, Bc=64, lambdas=(0.0,),
                   hot_rate=0.01, seed=3, num_splits=S)
    x = W.generate(w, threads=4)
    r = oracle.decode(x["q"], x["k"], x["v"], w.Bc, 0.0, S)
    assert not r["skip_full"].any()
    o, lse = oracle.combine(r["o_part_full"], r["lse_part_full"])
    kf, vf = f64(x["k"][0, 0]), f64(x["v"][0, 0])
    for h in range(w.Hq):
        s = kf @ f64(x["q"][0, h, 0]) / 4.0
        np.testing.assert_allclose(o[0, h], softmax(s) @ vf, rtol=1e-10, atol=1e-12)
        assert lse[0, h] == pytest.approx(logsumexp(s), rel=1e-13)


# --------------------------------------------------------------------------- #
# Invariants and the App. B error bound
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("lam", [1e-3, 1e-2, 1e-1])
def test_prefill_invariants_and_error_bound(lam):
    w, x = small_prefill(1, 4, 2, 256, 32, 32, 0.02, seed=5)
    r = oracle.prefill(x["q"], x["k"], x["v"], w.Bc, lam, threads=4)
    T, Bc, nq = w.T, w.Bc, w.T // w.Bc
    skipped_any = 0
    for h in range(w.Hq):
        qf, kf, vf = f64(x["q"][0, h]), f64(x["k"][0, h // w.G]), f64(x["v"][0, h // w.G])
        s = qf @ kf.T / math.sqrt(w.d)
        s[np.triu_indices(T, 1)] = -np.inf
        p = softmax(s, axis=1)  # true weights
        y = p @ vf
        M = s.max(axis=1)
        mask = r["mask_full"][0, h]
        yhat, lse = r["o_full"][0, h], r["lse_full"][0, h]
        vmax = np.linalg.norm(vf, axis=1).max()
        for t in range(T):
            i = t // Bc
            row_blocks = np.arange(t // Bc + 1)
            skipped = [j for j in row_blocks if mask[i, j] == 1]
            skipped_any += len(skipped)
            cols_skip = np.concatenate([np.arange(j * Bc, min(t + 1, (j + 1) * Bc)) for j in skipped]) \
                if skipped else np.array([], int)
            # every skipped token's true softmax weight is below lambda
            assert (p[t, cols_skip] < lam).all()
            # the block holding the row's global max is kept
            assert mask[i, int(np.argmax(s[t])) // Bc] == 0
            # Z_kept >= 1 (the max is kept), i.e. lse >= M; and lse <= dense lse
            assert lse[t] >= M[t] - 1e-12
            assert lse[t] <= logsumexp(s[t]) + 1e-12
            # App. B: yhat - y = delta (mean_kept - mean_skip); |yhat - y| <= 2 delta Vmax
            delta = p[t, cols_skip].sum()
            err = yhat[t] - y[t]
            if skipped:
                A = p[t] @ vf - p[t, cols_skip] @ vf[cols_skip]
                Bsk = p[t, cols_skip] @ vf[cols_skip]
                ident = delta * (A / (1 - delta) - Bsk / delta)
                np.testing.assert_allclose(err, ident, rtol=1e-7, atol=1e-12)
            assert np.linalg.norm(err) <= 2 * delta * vmax + 1e-12
            assert delta <= len(skipped) * Bc * lam
        # a block that raises some row's prefix max is never skipped
        for i in range(nq):
            rows = slice(i * Bc, (i + 1) * Bc)
            bm = np.stack([s[rows, j * Bc:(j + 1) * Bc].max(axis=1) for j in range(i + 1)], axis=1)
            prev = np.maximum.accumulate(np.concatenate([np.full((Bc, 1), -np.inf), bm], axis=1), axis=1)[:, :-1]
            new_max = (bm >= prev).any(axis=0)
            assert (mask[i, :i + 1][new_max] == 0).all()
    if lam >= 1e-2:
        assert skipped_any > 0, "workload too dense to exercise skipping"


@pytest.mark.parametrize("S", [1, 4])
def test_decode_invariants(S):
    lam = 1e-3
    w = W.Workload("t", "decode", B=1, Hq=8, Hkv=2, d=64, T=4096, Bc=128, lambdas=(lam,),
                   hot_rate=0.01, seed=9, window=256, num_splits=S)
    x = W.generate(w, threads=4)
    r = oracle.decode(x["q"], x["k"], x["v"], w.Bc, lam, S)
    o, lse = oracle.combine(r["o_part_full"], r["lse_part_full"])
    nk = w.T // w.Bc
    assert r["skip_full"].any()
    for h in range(w.Hq):
        kf, vf = f64(x["k"][0, h // w.G]), f64(x["v"][0, h // w.G])
        s = kf @ f64(x["q"][0, h, 0]) / 8.0
        p = softmax(s)
        sk = r["skip_full"][0, h].astype(bool)
        cols = np.array([c for j in range(nk) if sk[j] for c in range(j * w.Bc, (j + 1) * w.Bc)], int)
        assert (p[cols] < lam).all()
        assert not sk[int(np.argmax(s)) // w.Bc]
        for sp in range(S):  # each split's first block is kept
            assert not sk[sp * nk // S]
        assert lse[0, h] >= s.max() - 1e-12
        delta = p[cols].sum()
        err = o[0, h] - p @ vf
        assert np.linalg.norm(err) <= 2 * delta * np.linalg.norm(vf, axis=1).max() + 1e-12
        assert delta <= sk.sum() * w.Bc * lam
    # V is needed iff some head of the group keeps the block
    sk = r["skip_full"][0].reshape(w.Hkv, w.G, nk).all(axis=1)
    assert np.array_equal(r["vskip_full"][0].astype(bool), sk)


def test_skip_set_monotone_in_lambda():
    """Thresholds only move the cut: a block skipped at lambda is skipped at any larger lambda."""
    w, x = small_prefill(1, 4, 2, 256, 32, 32, 0.02, seed=13)
    prev = None
    for lam in [0.0, 1e-4, 1e-3, 1e-2, 1e-1, 0.9]:
        m = oracle.prefill(x["q"], x["k"], x["v"], w.Bc, lam)["mask_full"] == 1
        if prev is not None:
            assert (m | ~prev).all()
        prev = m
    assert prev.any()


def test_rejects_bad_lambda():
    w, x = small_prefill(1, 2, 1, 64, 8, 16, 0.05)
    for lam in [-1e-3, 1.0, 2.0, float("nan")]:
        with pytest.raises(ValueError):
            oracle.prefill(x["q"], x["k"], x["v"], w.Bc, lam)
