"""Host checks of the decision margins and of the lambda = a/L policy (no GPU).

* The oracle's margin (it reports D - ln(lambda)) gives the same D at every
  lambda -- the fact that makes a one-pass calibration possible (a skipped
  block never moves the running max) -- and D equals an independent numpy
  closed form: max over a query block's rows of (block max - prefix max of the
  block maxima), from the scores directly.
* The policy helpers: sparsity from margins against brute force, exact
  recovery of (alpha, beta) from points of the exponential model, and the
  run-time threshold as the model's inverse.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from block_sparse_attention_flash_amd import policy


def f64(b):
    return W.bf16_bits_to_f32(b).astype(np.float64)


def closed_form_prefill_margins(qf, kf, Bc, causal=True):
    """[nq, nk] margins (NaN above the diagonal) from the scaled scores."""
    T, d = qf.shape
    s = qf @ kf.T / math.sqrt(d)
    if causal:
        s[np.triu_indices(T, 1)] = -np.inf
    nq = -(-T // Bc)
    out = np.full((nq, nq), np.nan)
    for i in range(nq):
        r0, r1 = i * Bc, min(T, (i + 1) * Bc)
        jend = (r1 - 1) // Bc + 1 if causal else nq
        bm = np.stack([s[r0:r1, j * Bc:min(T, (j + 1) * Bc)].max(axis=1) for j in range(jend)], axis=1)
        prefix = np.maximum.accumulate(bm, axis=1)
        with np.errstate(invalid="ignore"):
            dr = np.where(np.isneginf(bm), -np.inf, bm - prefix)
        out[i, :jend] = dr.max(axis=0)
    return out


def closed_form_decode_margins(qrow, kf, Bc, S):
    N, d = kf.shape
    s = kf @ qrow / math.sqrt(d)
    nk = -(-N // Bc)
    bm = np.array([s[j * Bc:min(N, (j + 1) * Bc)].max() for j in range(nk)])
    out = np.empty(nk)
    for sp in range(S):
        j0, j1 = sp * nk // S, (sp + 1) * nk // S
        out[j0:j1] = bm[j0:j1] - np.maximum.accumulate(bm[j0:j1])
    return out


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_margin_is_lambda_free_and_matches_closed_form(causal):
    w = W.Workload("t", "prefill", B=1, Hq=4, Hkv=2, d=32, T=200, Bc=32, lambdas=(1e-3,), hot_rate=0.03, seed=5)
    x = W.generate(w, threads=4)
    Ds = []
    for lam in (1e-4, 1e-2, 0.3):
        r = oracle.prefill(x["q"], x["k"], x["v"], w.Bc, lam, causal=causal, threads=4)
        Ds.append(r["margin_full"] + math.log(lam))
    np.testing.assert_allclose(Ds[1], Ds[0], rtol=0, atol=1e-12, equal_nan=True)
    np.testing.assert_allclose(Ds[2], Ds[0], rtol=0, atol=1e-12, equal_nan=True)
    for h in range(w.Hq):
        cf = closed_form_prefill_margins(f64(x["q"][0, h]), f64(x["k"][0, h // w.G]), w.Bc, causal)
        np.testing.assert_allclose(Ds[0][0, h], cf, rtol=0, atol=1e-10, equal_nan=True)
    # the decisions at any lambda follow from D alone
    r = oracle.prefill(x["q"], x["k"], x["v"], w.Bc, 3e-2, causal=causal, threads=4)
    vis = ~np.isnan(Ds[0])
    assert np.array_equal(r["mask_full"][vis].astype(bool), Ds[0][vis] < math.log(3e-2))


@pytest.mark.parametrize("S", [1, 4])
def test_decode_margin_is_lambda_free_and_matches_closed_form(S):
    w = W.Workload("t", "decode", B=2, Hq=8, Hkv=2, d=32, T=900, Bc=64, lambdas=(1e-3,), hot_rate=0.02,
                   seed=9, window=64, num_splits=S)
    x = W.generate(w, threads=4)
    got = []
    for lam in (1e-3, 0.2):
        r = oracle.decode(x["q"], x["k"], x["v"], w.Bc, lam, S, threads=4)
        got.append((r["margin_full"] + math.log(lam), r["vmargin_full"] + math.log(lam)))
    np.testing.assert_allclose(got[1][0], got[0][0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[1][1], got[0][1], rtol=0, atol=1e-12)
    D, VD = got[0]
    for b in range(w.B):
        for h in range(w.Hq):
            cf = closed_form_decode_margins(f64(x["q"][b, h, 0]), f64(x["k"][b, h // w.G]), w.Bc, S)
            np.testing.assert_allclose(D[b, h], cf, rtol=0, atol=1e-10)
        for g in range(w.Hkv):
            np.testing.assert_allclose(VD[b, g], D[b, g * w.G:(g + 1) * w.G].max(axis=0), rtol=0, atol=1e-12)


def test_sparsity_at_brute_force():
    rng = np.random.default_rng(3)
    m = rng.normal(-5.0, 2.0, size=(3, 7, 11))
    m[0, 0, :4] = np.nan  # unvisited entries are not decisions
    lams = [0.0, 1e-4, 1e-3, 1e-2, 0.5]
    got = policy.sparsity_at(m, lams)
    flat = m[~np.isnan(m)]
    want = [0.0] + [float(np.mean(flat < math.log(l))) for l in lams[1:]]
    np.testing.assert_array_equal(got, np.asarray(want))
    with pytest.raises(ValueError):
        policy.sparsity_at(m, [1.0])


def test_margin_histogram_gives_sparsity_on_its_edges():
    rng = np.random.default_rng(5)
    m = rng.normal(-6.0, 3.0, size=5000)
    m[:7] = -np.inf   # a block no row of which sees a key
    m[7:11] = np.nan  # not visited
    lams = [1e-5, 1e-4, 1e-3, 1e-2, 1e-1]
    edges = [math.log(l) for l in lams]
    h = policy.margin_histogram(m, edges)
    assert h.sum() == 5000 - 4 and h.size == len(edges) + 1
    np.testing.assert_allclose(np.cumsum(h)[:-1] / h.sum(), policy.sparsity_at(m, lams), rtol=0, atol=1e-15)
    # brute-force bin counts
    flat = m[~np.isnan(m)]
    want = [np.sum(flat < edges[0])] + [np.sum((flat >= lo) & (flat < hi)) for lo, hi in zip(edges, edges[1:])] + \
        [np.sum(flat >= edges[-1])]
    np.testing.assert_array_equal(h, want)
    with pytest.raises(ValueError):
        policy.margin_histogram(m, [0.0, -1.0])


def test_fit_recovers_exponential_model_and_lambda_inverts_it():
    alpha, beta = 37.5, 4.25
    s = np.linspace(0.05, 0.9, 12)
    a = alpha * np.exp(beta * s)
    # saturated points (0% and 100%) are ignored by the fit
    a_all = np.concatenate([a, [1e-3, 1e9]])
    s_all = np.concatenate([s, [0.0, 1.0]])
    fa, fb = policy.fit_exponential(a_all, s_all)
    assert fa == pytest.approx(alpha, rel=1e-10) and fb == pytest.approx(beta, rel=1e-10)
    for L in (4096, 32768, 131072):
        for target in (0.3, 0.5, 0.7):
            lam = policy.lambda_for(target, L, fa, fb)
            assert lam * L == pytest.approx(alpha * math.exp(beta * target), rel=1e-10)
    with pytest.raises(ValueError):
        policy.fit_exponential(np.array([1.0, 2.0]), np.array([0.0, 1.0]))


def test_calibration_points_pairs_lambda_times_length_with_sparsity():
    rng = np.random.default_rng(4)
    margins = [rng.normal(-4.0, 1.5, size=100), rng.normal(-6.0, 1.5, size=400)]
    lengths = [1000, 4000]
    lams = [1e-3, 1e-2]
    a, s = policy.calibration_points(margins, lengths, lams)
    assert list(a) == [1.0, 10.0, 4.0, 40.0]
    np.testing.assert_array_equal(s[:2], policy.sparsity_at(margins[0], lams))
    np.testing.assert_array_equal(s[2:], policy.sparsity_at(margins[1], lams))


def test_lambda_at_sparsity_inverts_sparsity_at():
    rng = np.random.default_rng(11)
    m = rng.normal(-6.0, 3.0, size=4001)
    m = np.minimum(m, 0.0)
    m[:5] = -np.inf   # blocks no row of which sees a key: skipped at any lambda > 0
    m[5:9] = np.nan   # not visited
    m[9:40] = 0.0     # blocks that set the running max: never skipped below lambda = 1
    n = np.count_nonzero(~np.isnan(m))
    for target in (0.0, 1e-4, 0.1, 0.5, 0.719, 0.9):
        lam = policy.lambda_at_sparsity(m, target)
        assert 0.0 <= lam < 1.0
        got = round(policy.sparsity_at(m, [lam])[0] * n)
        k = math.ceil(target * n)
        flat = np.sort(m[~np.isnan(m)])
        want = 0 if k == 0 else int(np.count_nonzero(flat <= flat[k - 1]))  # k, or the whole tie group
        assert got == want, (target, got, want)
    # ties: the whole tie group is skipped
    t = np.array([-3.0, -2.0, -2.0, -2.0, -1.0])
    assert policy.sparsity_at(t, [policy.lambda_at_sparsity(t, 0.4)])[0] == 0.8
    # only -inf below the target: any lambda > 0 skips exactly those
    t = np.array([-np.inf, -np.inf, -1.0, 0.0])
    assert policy.sparsity_at(t, [policy.lambda_at_sparsity(t, 0.5)])[0] == 0.5
    # a target past the margin-0 decisions stops at them
    assert policy.sparsity_at(m, [policy.lambda_at_sparsity(m, 1.0)])[0] == np.count_nonzero(m < 0.0) / n
