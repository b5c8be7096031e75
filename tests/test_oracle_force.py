"""Pins for the oracle's adopt-a-decision ("force") mode and the parity checker's
flip path (no GPU).

Where fp32 and fp64 scores fall on opposite sides of the threshold, both
decisions are valid results of the rule (BLASST blog, section on the decision
rule, Eq. 5: skip iff the block max minus the updated running max is below
ln lambda).  The parity checker then reruns the oracle taking the GPU's
decision on exactly those blocks.  These tests pin that mode against numpy
closed forms that do not reuse the oracle's recurrence:

* decisions: a forced entry is what was forced; every other entry is the
  prefix-max rule (the running max before block j is the prefix max of the
  block maxima, whatever was kept), so forcing never changes another decision;
* outputs: a plain softmax over the kept keys (the forced kept set), with
  o = 0 and lse = -inf for a row (or split) left with no kept key;
* forced entries are read for the right unit: the oracle is called on a
  shuffled subset of units, each with its own force row.

The checker tests fabricate a "GPU result" from the oracle with one flipped
decision and check that (a) a flip inside the 1e-3 margin band passes and is
counted, (b) the same result with the unflipped outputs fails, so the rerun is
what makes it pass, and (c) a flip away from the threshold fails.
"""
import math
import os
import sys

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
import workloads as W

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import parity  # noqa: E402


def f64(b):
    return W.bf16_bits_to_f32(b).astype(np.float64)


def masked_softmax(s, vf, keep):
    """Rows of s [R, C] over the columns keep [R, C] (bool): out [R, d], lse [R]."""
    s = np.where(keep, s, -np.inf)
    out = np.zeros((s.shape[0], vf.shape[1]))
    lse = np.full(s.shape[0], -np.inf)
    for r in range(s.shape[0]):
        if np.isfinite(s[r]).any():
            lse[r] = logsumexp(s[r])
            out[r] = np.exp(s[r] - lse[r]) @ vf
    return out, lse


def random_force(rng, shape, visited=None, p=0.35):
    f = np.full(shape, -1, np.int8)
    pick = rng.random(shape) < p
    if visited is not None:
        pick &= visited
    f[pick] = rng.integers(0, 2, size=int(pick.sum()))
    return f


# --------------------------------------------------------------------------- #
# Prefill
# --------------------------------------------------------------------------- #
def _max_block(s, Bc, j_end):
    """The block holding the highest score of s [R, C] among blocks < j_end."""
    return int(np.argmax(s[:, : min(s.shape[1], j_end * Bc)].max(axis=0))) // Bc


@pytest.mark.parametrize("Br,Bc", [(32, 32), (64, 32), (16, 8)])
@pytest.mark.parametrize("lam", [1e-3, 1e-1, 0.6])
def test_prefill_force_matches_closed_form(Br, Bc, lam):
    """Br = 2 Bc gives rows that see no key of the last visited block, so a
    forced keep there must add nothing to those rows.  Each unit's block holding
    its highest score is forced to skip: later decisions must still be taken
    against the true prefix max."""
    w = W.Workload("t", "prefill", B=2, Hq=4, Hkv=2, d=32, T=224, Bc=Bc, lambdas=(lam,), hot_rate=0.03,
                   seed=101)
    x = W.generate(w, threads=4)
    T, d, G = w.T, w.d, w.G
    nq, nk = -(-T // Br), -(-T // Bc)
    thr = math.log(lam)
    rng = np.random.default_rng(5)
    all_units = np.arange(w.B * w.Hq * nq)
    units = rng.permutation(all_units)[: len(all_units) * 2 // 3]
    # visited blocks of each unit: j <= last row's block
    visited = np.array([[j <= (min(T, (u % nq + 1) * Br) - 1) // Bc for j in range(nk)] for u in units])
    force = random_force(rng, (len(units), nk), visited)
    for ui, u in enumerate(units):
        i = u % nq
        b, hq = divmod(u // nq, w.Hq)
        r0, r1 = i * Br, min(T, (i + 1) * Br)
        s = f64(x["q"][b, hq, r0:r1]) @ f64(x["k"][b, hq // G]).T
        s[np.arange(T)[None, :] > np.arange(r0, r1)[:, None]] = -np.inf
        jm = _max_block(s, Bc, (r1 - 1) // Bc + 1)
        if jm < (r1 - 1) // Bc:
            force[ui, jm] = 1
    r = oracle.prefill(x["q"], x["k"], x["v"], Bc, lam, Br=Br, units=units, force=force, threads=4)
    forced_any = 0
    for ui, u in enumerate(units):
        i = u % nq
        b, hq = divmod(u // nq, w.Hq)
        qf, kf, vf = f64(x["q"][b, hq]), f64(x["k"][b, hq // G]), f64(x["v"][b, hq // G])
        r0, r1 = i * Br, min(T, (i + 1) * Br)
        s = qf[r0:r1] @ kf.T / math.sqrt(d)
        rows = np.arange(r0, r1)[:, None]
        s[np.arange(T)[None, :] > rows] = -np.inf
        jend = (r1 - 1) // Bc + 1
        bm = np.stack([s[:, j * Bc:min(T, (j + 1) * Bc)].max(axis=1) for j in range(jend)], axis=1)
        prefix = np.maximum.accumulate(bm, axis=1)
        with np.errstate(invalid="ignore"):
            vote = np.isneginf(bm) | (bm - prefix < thr)
        skip = vote.all(axis=0).astype(np.int8)
        fu = force[ui, :jend]
        want = np.where(fu >= 0, fu, skip)
        forced_any += int((fu >= 0).sum())
        assert r["mask"][ui, :jend].tolist() == want.tolist(), "unit %d" % u
        assert (r["mask"][ui, jend:] == 2).all()
        keep_col = np.zeros(T, bool)
        for j in range(jend):
            if want[j] == 0:
                keep_col[j * Bc:min(T, (j + 1) * Bc)] = True
        out, lse = masked_softmax(s, vf, np.broadcast_to(keep_col, s.shape))
        np.testing.assert_allclose(r["o"][ui, : r1 - r0], out, rtol=1e-10, atol=1e-12)
        both_inf = np.isneginf(lse) & np.isneginf(r["lse"][ui, : r1 - r0])
        np.testing.assert_allclose(np.where(both_inf, 0, r["lse"][ui, : r1 - r0]), np.where(both_inf, 0, lse),
                                   rtol=1e-12, atol=1e-12)
    assert forced_any > 20


def test_prefill_force_skip_of_every_block_empties_the_rows():
    w = W.Workload("t", "prefill", B=1, Hq=2, Hkv=1, d=16, T=96, Bc=32, lambdas=(1e-3,), hot_rate=0.03, seed=3)
    x = W.generate(w, threads=2)
    units = [1, 4]  # (h0, i1) and (h1, i1)
    force = np.full((2, 3), -1, np.int8)
    force[:, :2] = 1
    r = oracle.prefill(x["q"], x["k"], x["v"], w.Bc, 1e-3, units=units, force=force)
    assert r["mask"].tolist() == [[1, 1, 2], [1, 1, 2]]
    assert (r["o"] == 0).all() and np.isneginf(r["lse"]).all()


# --------------------------------------------------------------------------- #
# Decode
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("lam,S", [(1e-3, 1), (1e-2, 3), (0.3, 4)])
def test_decode_force_matches_closed_form(lam, S):
    w = W.Workload("t", "decode", B=2, Hq=8, Hkv=4, d=32, T=900, Bc=64, lambdas=(lam,), hot_rate=0.02,
                   seed=202, window=64, num_splits=S)
    x = W.generate(w, threads=4)
    Bc, G, N = w.Bc, w.G, w.T
    nk = -(-N // Bc)
    thr = math.log(lam)
    rng = np.random.default_rng(9)
    units = np.array([5, 0, 6, 3])
    force = random_force(rng, (len(units), G, nk))
    # one split of one head with every block forced to skip: that split is empty
    force[1, 1, :nk // S] = 1
    r = oracle.decode(x["q"], x["k"], x["v"], Bc, lam, S, units=units, force=force, threads=4)
    o, lse = oracle.combine(r["o_part"], r["lse_part"])
    for ui, u in enumerate(units):
        b, hkv = divmod(int(u), w.Hkv)
        kf, vf = f64(x["k"][b, hkv]), f64(x["v"][b, hkv])
        vneed = np.zeros(nk, bool)
        for g in range(G):
            s = kf @ f64(x["q"][b, hkv * G + g, 0]) / math.sqrt(w.d)
            bm = np.array([s[j * Bc:min(N, (j + 1) * Bc)].max() for j in range(nk)])
            want = np.empty(nk, np.int8)
            keep_col = np.zeros(N, bool)
            for sp in range(S):
                j0, j1 = sp * nk // S, (sp + 1) * nk // S
                own = (bm[j0:j1] - np.maximum.accumulate(bm[j0:j1]) < thr).astype(np.int8)
                fs = force[ui, g, j0:j1]
                want[j0:j1] = np.where(fs >= 0, fs, own)
                ks = np.zeros(N, bool)
                for j in range(j0, j1):
                    if want[j] == 0:
                        ks[j * Bc:min(N, (j + 1) * Bc)] = True
                keep_col |= ks
                op, lp = masked_softmax(s[None], vf, ks[None])
                np.testing.assert_allclose(r["o_part"][ui, g, sp], op[0], rtol=1e-10, atol=1e-12)
                if np.isneginf(lp[0]):
                    assert np.isneginf(r["lse_part"][ui, g, sp])
                else:
                    assert r["lse_part"][ui, g, sp] == pytest.approx(lp[0], rel=1e-12, abs=1e-12)
            assert r["skip"][ui, g].tolist() == want.tolist(), "unit %d head %d" % (u, g)
            vneed |= want == 0
            oc, lc = masked_softmax(s[None], vf, keep_col[None])
            np.testing.assert_allclose(o[ui, g], oc[0], rtol=1e-10, atol=1e-12)
            assert lse[ui, g] == pytest.approx(lc[0], rel=1e-12, abs=1e-12)
        assert r["vskip"][ui].tolist() == (~vneed).astype(int).tolist()


# --------------------------------------------------------------------------- #
# MLA decode
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("lam", [1e-2, 0.4])
def test_mla_force_matches_closed_form(lam):
    S, Bc, dv = 3, 64, 48
    w = W.Workload("t", "decode", B=2, Hq=4, Hkv=1, d=80, T=700, Bc=Bc, lambdas=(lam,), hot_rate=0.02,
                   seed=303, window=64, num_splits=S, dv=dv, scale=1.0 / math.sqrt(40.0))
    x = W.generate(w, parts=("q", "k"), threads=4)
    q, kv = np.ascontiguousarray(x["q"][:, :, 0]), np.ascontiguousarray(x["k"][:, 0])
    N = w.T
    nk = -(-N // Bc)
    rng = np.random.default_rng(17)
    units = np.array([6, 1, 3, 4])
    force = random_force(rng, (len(units), nk))
    for ui, u in enumerate(units):  # skip each split's max block when it is not the split's last
        b, h = divmod(int(u), w.Hq)
        s = f64(kv[b]) @ f64(q[b, h])
        for sp in range(S):
            j0, j1 = sp * nk // S, (sp + 1) * nk // S
            jm = j0 + _max_block(s[None, j0 * Bc:min(N, j1 * Bc)], Bc, j1 - j0)
            if jm < j1 - 1:
                force[ui, jm] = 1
    r = oracle.decode_mla(q, kv, Bc, lam, S, w.score_scale, dv, units=units, force=force, threads=4)
    for ui, u in enumerate(units):
        b, h = divmod(int(u), w.Hq)
        K = f64(kv[b])
        s = K @ f64(q[b, h]) * w.score_scale
        bm = np.array([s[j * Bc:min(N, (j + 1) * Bc)].max() for j in range(nk)])
        for sp in range(S):
            j0, j1 = sp * nk // S, (sp + 1) * nk // S
            own = (bm[j0:j1] - np.maximum.accumulate(bm[j0:j1]) < math.log(lam)).astype(np.int8)
            want = np.where(force[ui, j0:j1] >= 0, force[ui, j0:j1], own)
            assert r["skip"][ui, j0:j1].tolist() == want.tolist()
            ks = np.zeros(N, bool)
            for j in range(j0, j1):
                if want[j - j0] == 0:
                    ks[j * Bc:min(N, (j + 1) * Bc)] = True
            op, lp = masked_softmax(s[None], K[:, :dv], ks[None])
            np.testing.assert_allclose(r["o_part"][ui, sp], op[0], rtol=1e-10, atol=1e-12)
            assert r["lse_part"][ui, sp] == pytest.approx(lp[0], rel=1e-12, abs=1e-12) or \
                (np.isneginf(lp[0]) and np.isneginf(r["lse_part"][ui, sp]))


# --------------------------------------------------------------------------- #
# The parity checker's flip path, on fabricated GPU results
# --------------------------------------------------------------------------- #
def _decode_case():
    w = W.Workload("t", "decode", B=1, Hq=8, Hkv=2, d=64, T=2048, Bc=64, lambdas=(1e-3,), hot_rate=0.01,
                   seed=404, window=128, num_splits=2)
    return w, W.generate(w, threads=4)


def _pick_decode_flip(w, x):
    """(lambda, unit, head, block): a block whose skip or keep changes o by > 2e-2,
    with lambda set so that its margin is 3e-4 (kept by a hair)."""
    S, nk = w.num_splits, w.T // w.Bc
    base = oracle.decode(x["q"], x["k"], x["v"], w.Bc, 0.5, S)  # margins at ln 0.5
    D = base["margin_full"] + math.log(0.5)                      # lambda-free D
    o0, _ = oracle.combine(base["o_part_full"], base["lse_part_full"])
    best = None
    for h in range(w.Hq):
        for j in range(nk):
            if j % (nk // S) == 0 or not (-4.0 < D[0, h, j] < -0.05):
                continue
            lam = math.exp(D[0, h, j] - 3e-4)
            f = np.full((w.Hkv, w.G, nk), -1, np.int8)
            f[h // w.G, h % w.G, j] = 1
            r = oracle.decode(x["q"], x["k"], x["v"], w.Bc, lam, S, force=f)
            ref = oracle.decode(x["q"], x["k"], x["v"], w.Bc, lam, S)
            o1, _ = oracle.combine(r["o_part_full"], r["lse_part_full"])
            o2, _ = oracle.combine(ref["o_part_full"], ref["lse_part_full"])
            gap = np.abs(o1 - o2).max()
            if best is None or gap > best[0]:
                best = (gap, lam, h, j)
    del o0
    assert best is not None and best[0] > 2e-2, "no flip with a visible effect"
    return best[1:]


def _fake_decode_gpu(w, x, lam, force):
    r = oracle.decode(x["q"], x["k"], x["v"], w.Bc, lam, w.num_splits, force=force)
    o, lse = oracle.combine(r["o_part_full"], r["lse_part_full"])
    f32 = lambda a: a.astype(np.float32)  # noqa: E731
    return dict(o_part=f32(r["o_part_full"]), lse_part=f32(r["lse_part_full"]), skip=r["skip_full"].copy(),
                vskip=r["vskip_full"].copy(), o=f32(o), lse=f32(lse))


def test_check_decode_adopts_a_near_margin_flip():
    w, x = _decode_case()
    lam, h, j = _pick_decode_flip(w, x)
    nk = w.T // w.Bc
    ref = oracle.decode(x["q"], x["k"], x["v"], w.Bc, lam, w.num_splits)
    assert abs(ref["margin_full"][0, h, j]) < parity.MARGIN and ref["skip_full"][0, h, j] == 0
    f = np.full((w.Hkv, w.G, nk), -1, np.int8)
    f[h // w.G, h % w.G, j] = 1
    gpu = _fake_decode_gpu(w, x, lam, f)
    rep = parity.check_decode(x, w.Bc, lam, w.num_splits, gpu=gpu)
    assert rep.mismatches == 1 and rep.near_margin == 1
    # the same flipped mask with the unflipped outputs must fail: the rerun is what passes it
    plain = _fake_decode_gpu(w, x, lam, None)
    bad = dict(plain, skip=gpu["skip"], vskip=gpu["vskip"])
    with pytest.raises(AssertionError):
        parity.check_decode(x, w.Bc, lam, w.num_splits, gpu=bad)


def test_check_decode_rejects_a_flip_away_from_the_threshold():
    w, x = _decode_case()
    lam = 1e-3
    nk = w.T // w.Bc
    ref = oracle.decode(x["q"], x["k"], x["v"], w.Bc, lam, w.num_splits)
    far = np.argwhere(np.abs(ref["margin_full"][0]) > 0.5)
    h, j = (int(v) for v in far[len(far) // 2])
    f = np.full((w.Hkv, w.G, nk), -1, np.int8)
    f[h // w.G, h % w.G, j] = 1 - int(ref["skip_full"][0, h, j])
    gpu = _fake_decode_gpu(w, x, lam, f)
    with pytest.raises(AssertionError, match="away from the threshold"):
        parity.check_decode(x, w.Bc, lam, w.num_splits, gpu=gpu)


def _prefill_case():
    w = W.Workload("t", "prefill", B=1, Hq=2, Hkv=1, d=32, T=512, Bc=32, lambdas=(1e-3,), hot_rate=0.01,
                   seed=505)
    return w, W.generate(w, threads=4)


def _fake_prefill_gpu(w, x, lam, force):
    r = oracle.prefill(x["q"], x["k"], x["v"], w.Bc, lam, force=force)
    return dict(o=r["o_full"].astype(np.float32), lse=r["lse_full"].astype(np.float32), mask=r["mask_full"].copy())


def test_check_prefill_adopts_a_near_margin_flip():
    w, x = _prefill_case()
    nq = nk = w.T // w.Bc
    base = oracle.prefill(x["q"], x["k"], x["v"], w.Bc, 0.5)
    D = base["margin_full"] + math.log(0.5)
    best = None
    for h in range(w.Hq):
        for i in range(nq):
            for j in range(i):  # off-diagonal visited tiles
                if not (-4.0 < D[0, h, i, j] < -0.05):
                    continue
                lam = math.exp(D[0, h, i, j] - 3e-4)
                f = np.full((w.B * w.Hq * nq, nk), -1, np.int8)
                f[h * nq + i, j] = 1
                a = oracle.prefill(x["q"], x["k"], x["v"], w.Bc, lam, force=f)["o_full"]
                b = oracle.prefill(x["q"], x["k"], x["v"], w.Bc, lam)["o_full"]
                gap = np.abs(a - b).max()
                if best is None or gap > best[0]:
                    best = (gap, lam, h, i, j, f)
    gap, lam, h, i, j, f = best
    assert gap > 2e-2
    ref = oracle.prefill(x["q"], x["k"], x["v"], w.Bc, lam)
    assert abs(ref["margin_full"][0, h, i, j]) < parity.MARGIN and ref["mask_full"][0, h, i, j] == 0
    gpu = _fake_prefill_gpu(w, x, lam, f)
    rep = parity.check_prefill(x, w.Bc, lam, gpu=gpu)
    assert rep.mismatches == 1 and rep.near_margin == 1
    bad = dict(_fake_prefill_gpu(w, x, lam, None), mask=gpu["mask"])
    with pytest.raises(AssertionError):
        parity.check_prefill(x, w.Bc, lam, gpu=bad)


def test_check_prefill_rejects_a_flip_away_from_the_threshold():
    w, x = _prefill_case()
    lam = 1e-2
    nq, nk = w.T // w.Bc, w.T // w.Bc
    ref = oracle.prefill(x["q"], x["k"], x["v"], w.Bc, lam)
    vis = ~np.isnan(ref["margin_full"][0])
    far = np.argwhere(vis & (np.abs(np.nan_to_num(ref["margin_full"][0])) > 0.5))
    h, i, j = (int(v) for v in far[len(far) // 2])
    f = np.full((w.B * w.Hq * nq, nk), -1, np.int8)
    f[h * nq + i, j] = 1 - int(ref["mask_full"][0, h, i, j])
    gpu = _fake_prefill_gpu(w, x, lam, f)
    with pytest.raises(AssertionError, match="away from the threshold"):
        parity.check_prefill(x, w.Bc, lam, gpu=gpu)


def test_check_mla_adopts_a_near_margin_flip_and_rejects_a_far_one():
    S, Bc, dv = 2, 64, 64
    w = W.Workload("t", "decode", B=1, Hq=4, Hkv=1, d=96, T=1024, Bc=Bc, lambdas=(1e-3,), hot_rate=0.01,
                   seed=606, window=64, num_splits=S, dv=dv, scale=1.0 / math.sqrt(48.0))
    x = W.generate(w, parts=("q", "k"), threads=4)
    q, kv = np.ascontiguousarray(x["q"][:, :, 0]), np.ascontiguousarray(x["k"][:, 0])
    nk = w.T // Bc
    base = oracle.decode_mla(q, kv, Bc, 0.5, S, w.score_scale, dv)
    D = base["margin_full"] + math.log(0.5)

    def fake(lam, force):
        r = oracle.decode_mla(q, kv, Bc, lam, S, w.score_scale, dv, force=force)
        o, lse = oracle.combine(r["o_part_full"], r["lse_part_full"])
        return dict(o_part=r["o_part_full"].astype(np.float32), lse_part=r["lse_part_full"].astype(np.float32),
                    skip=r["skip_full"].copy(), o=o.astype(np.float32), lse=lse.astype(np.float32))

    best = None
    for h in range(w.Hq):
        for j in range(nk):
            if j % (nk // S) == 0 or not (-4.0 < D[0, h, j] < -0.05):
                continue
            lam = math.exp(D[0, h, j] - 3e-4)
            f = np.full((w.Hq, nk), -1, np.int8)
            f[h, j] = 1
            gap = np.abs(fake(lam, f)["o"] - fake(lam, None)["o"]).max()
            if best is None or gap > best[0]:
                best = (gap, lam, f)
    gap, lam, f = best
    assert gap > 2e-2
    rep = parity.check_mla(q, kv, Bc, lam, S, w.score_scale, dv, gpu=fake(lam, f))
    assert rep.mismatches == 1 and rep.near_margin == 1
    with pytest.raises(AssertionError):
        parity.check_mla(q, kv, Bc, lam, S, w.score_scale, dv, gpu=dict(fake(lam, None), skip=fake(lam, f)["skip"]))
    # a flip far from the threshold
    lam = 1e-3
    ref = oracle.decode_mla(q, kv, Bc, lam, S, w.score_scale, dv)
    far = np.argwhere(np.abs(ref["margin_full"][0]) > 0.5)
    h, j = (int(v) for v in far[len(far) // 2])
    f = np.full((w.Hq, nk), -1, np.int8)
    f[h, j] = 1 - int(ref["skip_full"][0, h, j])
    with pytest.raises(AssertionError, match="away from the threshold"):
        parity.check_mla(q, kv, Bc, lam, S, w.score_scale, dv, gpu=fake(lam, f))
