"""GPU-vs-oracle comparison helpers for the parity tests (imported by tests only).

Tolerances (bf16 inputs, fp32 accumulation and output):
  * outputs: max-abs error <= 1e-2 and per-row relative L2 <= 5e-3; rows whose
    oracle norm is below 1e-3*sqrt(d) are held to the max-abs bound only;
  * LSE: abs error <= 1e-4 (the row sum is accumulated from unrounded fp32 P);
  * skip decisions: identical, except where the oracle's margin
    |D - ln(lambda)| is below 1e-3 (natural-log units), where fp32 and fp64
    scores may fall on different sides of the threshold.  Such blocks are
    counted; for the output comparison the oracle is rerun taking, on exactly
    those oracle-flagged blocks, the decision the GPU took (both are valid
    results of the rule), and its own decision everywhere else.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

import oracle

MAX_ABS = 1e-2
ROW_REL_L2 = 5e-3
LSE_ABS = 1e-4
MARGIN = 1e-3


def to_device(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


@dataclass
class Report:
    decisions: int = 0
    mismatches: int = 0
    near_margin: int = 0
    max_abs: float = 0.0
    worst_row_rel: float = 0.0
    max_lse_abs: float = 0.0
    notes: list = field(default_factory=list)

    def __str__(self):
        return ("decisions=%d mismatches=%d (near-margin=%d) max_abs=%.3g worst_row_rel_l2=%.3g max_lse_abs=%.3g"
                % (self.decisions, self.mismatches, self.near_margin, self.max_abs, self.worst_row_rel,
                   self.max_lse_abs))


def compare_masks(gpu: np.ndarray, ref: np.ndarray, margin: np.ndarray, rep: Report, what: str):
    """Decisions must agree exactly away from the threshold."""
    gpu = gpu.astype(np.uint8)
    ref = ref.astype(np.uint8)
    diff = gpu != ref
    near = np.abs(margin) < MARGIN
    bad = diff & ~near
    rep.decisions += int(ref.size)
    rep.mismatches += int(diff.sum())
    rep.near_margin += int((diff & near).sum())
    assert not bad.any(), "%s: %d decisions differ away from the threshold (first at %s)" % (
        what, int(bad.sum()), tuple(int(x) for x in np.argwhere(bad)[0]))
    return diff


def compare_rows(gpu: np.ndarray, ref: np.ndarray, rep: Report, what: str):
    """gpu/ref [..., d]: max-abs and per-row relative L2."""
    gpu = gpu.astype(np.float64)
    assert np.isfinite(gpu).all(), "%s: non-finite GPU output" % what
    d = ref.shape[-1]
    err = np.abs(gpu - ref)
    rep.max_abs = max(rep.max_abs, float(err.max(initial=0.0)))
    assert err.max(initial=0.0) <= MAX_ABS, "%s: max-abs %.4g > %g" % (what, err.max(), MAX_ABS)
    rn = np.linalg.norm(ref, axis=-1)
    en = np.linalg.norm(gpu - ref, axis=-1)
    sel = rn >= 1e-3 * math.sqrt(d)
    if sel.any():
        rel = en[sel] / rn[sel]
        rep.worst_row_rel = max(rep.worst_row_rel, float(rel.max()))
        assert rel.max() <= ROW_REL_L2, "%s: row relative L2 %.4g > %g" % (what, rel.max(), ROW_REL_L2)


def compare_lse(gpu: np.ndarray, ref: np.ndarray, rep: Report, what: str):
    gpu = gpu.astype(np.float64)
    both = np.isneginf(gpu) & np.isneginf(ref)  # an empty split or context on both sides
    with np.errstate(invalid="ignore"):
        err = np.where(both, 0.0, np.abs(gpu - ref))
    rep.max_lse_abs = max(rep.max_lse_abs, float(err.max(initial=0.0)))
    assert err.max(initial=0.0) <= LSE_ABS, "%s: lse abs %.4g > %g" % (what, err.max(), LSE_ABS)


# --------------------------------------------------------------------------- #
# Decode
# --------------------------------------------------------------------------- #
def run_gpu_decode(x_dev, Bc, lam, S):
    import block_sparse_attention_flash_amd as bsa
    o_part, lse_part, skip, vskip = bsa.decode(x_dev["q"], x_dev["k"], x_dev["v"], lam, S, Bc=Bc)
    o, lse = bsa.decode_combine(o_part, lse_part)
    import torch
    torch.cuda.synchronize()
    return {k: t.cpu().numpy() for k, t in
            dict(o_part=o_part, lse_part=lse_part, skip=skip, vskip=vskip, o=o, lse=lse).items()}


def check_decode(x: dict, Bc: int, lam: float, S: int, units=None, x_dev=None, gpu=None) -> Report:
    """Compare the GPU decode (+ combine) with the oracle on the given (b, hkv) units."""
    B, Hq, _, d = x["q"].shape
    Hkv = x["k"].shape[1]
    G = Hq // Hkv
    if gpu is None:
        if x_dev is None:
            x_dev = {k: to_device(v) for k, v in x.items()}
        gpu = run_gpu_decode(x_dev, Bc, lam, S)
    units = list(range(B * Hkv)) if units is None else list(units)
    ref = oracle.decode(x["q"], x["k"], x["v"], Bc, lam, S, units=units)
    rep = Report()
    nk = ref["skip"].shape[-1]
    force = np.full((len(units), G, nk), -1, np.int8)
    any_flip = False
    for ui, u in enumerate(units):
        b, hkv = divmod(u, Hkv)
        heads = slice(hkv * G, (hkv + 1) * G)
        diff = compare_masks(gpu["skip"][b, heads], ref["skip"][ui], ref["margin"][ui], rep, "skip b=%d hkv=%d" % (b, hkv))
        compare_masks(gpu["vskip"][b, hkv], ref["vskip"][ui], ref["vmargin"][ui], Report(), "vskip b=%d hkv=%d" % (b, hkv))
        if diff.any():
            any_flip = True
            force[ui][diff] = gpu["skip"][b, heads][diff]
    if any_flip:
        ref = oracle.decode(x["q"], x["k"], x["v"], Bc, lam, S, units=units, force=force)
    o_ref, lse_ref = oracle.combine(ref["o_part"], ref["lse_part"])
    for ui, u in enumerate(units):
        b, hkv = divmod(u, Hkv)
        heads = slice(hkv * G, (hkv + 1) * G)
        compare_rows(gpu["o_part"][b, heads], ref["o_part"][ui], rep, "o_part b=%d hkv=%d" % (b, hkv))
        compare_lse(gpu["lse_part"][b, heads], ref["lse_part"][ui], rep, "lse_part b=%d hkv=%d" % (b, hkv))
        compare_rows(gpu["o"][b, heads], o_ref[ui], rep, "o b=%d hkv=%d" % (b, hkv))
        compare_lse(gpu["lse"][b, heads], lse_ref[ui], rep, "lse b=%d hkv=%d" % (b, hkv))
    return rep


# --------------------------------------------------------------------------- #
# Prefill
# --------------------------------------------------------------------------- #
def run_gpu_prefill(x_dev, Bc, lam, causal=True):
    import torch
    import block_sparse_attention_flash_amd as bsa
    o, lse, mask = bsa.prefill(x_dev["q"], x_dev["k"], x_dev["v"], lam, Bc=Bc, causal=causal)
    torch.cuda.synchronize()
    return dict(o=o, lse=lse, mask=mask)


def check_prefill(x: dict, Bc: int, lam: float, causal=True, units=None, x_dev=None, gpu=None) -> Report:
    """Compare the GPU prefill with the oracle on query-block units (b*Hq + hq)*nq + i."""
    B, Hq, T, d = x["q"].shape
    nq = -(-T // Bc)
    if gpu is None:
        if x_dev is None:
            x_dev = {k: to_device(v) for k, v in x.items()}
        gpu = run_gpu_prefill(x_dev, Bc, lam, causal)
    units = list(range(B * Hq * nq)) if units is None else list(units)
    ref = oracle.prefill(x["q"], x["k"], x["v"], Bc, lam, causal=causal, units=units)
    rep = Report()
    mask_g = gpu["mask"].cpu().numpy() if hasattr(gpu["mask"], "cpu") else gpu["mask"]
    force = np.full(ref["mask"].shape, -1, np.int8)
    any_flip = False
    for ui, u in enumerate(units):
        i = u % nq
        b, hq = divmod(u // nq, Hq)
        g = mask_g[b, hq, i]
        r = ref["mask"][ui]
        visited = r != 2
        assert np.array_equal(g[~visited], r[~visited]), "unvisited entries differ at b=%d hq=%d i=%d" % (b, hq, i)
        diff = compare_masks(g[visited], r[visited], ref["margin"][ui][visited], rep, "mask b=%d hq=%d i=%d" % (b, hq, i))
        if diff.any():
            any_flip = True
            idx = np.nonzero(visited)[0][diff]
            force[ui][idx] = g[idx]
    if any_flip:
        ref = oracle.prefill(x["q"], x["k"], x["v"], Bc, lam, causal=causal, units=units, force=force)
    o_g, lse_g = gpu["o"], gpu["lse"]
    for ui, u in enumerate(units):
        i = u % nq
        b, hq = divmod(u // nq, Hq)
        r0, r1 = i * Bc, min(T, (i + 1) * Bc)
        og = o_g[b, hq, r0:r1]
        lg = lse_g[b, hq, r0:r1]
        og = og.cpu().numpy() if hasattr(og, "cpu") else og
        lg = lg.cpu().numpy() if hasattr(lg, "cpu") else lg
        compare_rows(og, ref["o"][ui][: r1 - r0], rep, "o b=%d hq=%d i=%d" % (b, hq, i))
        compare_lse(lg, ref["lse"][ui][: r1 - r0], rep, "lse b=%d hq=%d i=%d" % (b, hq, i))
    return rep


# --------------------------------------------------------------------------- #
# MLA decode
# --------------------------------------------------------------------------- #
def run_gpu_mla(q_dev, kv_dev, Bc, lam, S, scale, dv):
    import torch
    import block_sparse_attention_flash_amd as bsa
    o_part, lse_part, skip = bsa.decode_mla(q_dev, kv_dev, lam, S, scale, Bc=Bc, d_v=dv)
    o, lse = bsa.decode_combine(o_part, lse_part)
    torch.cuda.synchronize()
    return {k: t.cpu().numpy() for k, t in dict(o_part=o_part, lse_part=lse_part, skip=skip, o=o, lse=lse).items()}


def check_mla(q: np.ndarray, kv: np.ndarray, Bc: int, lam: float, S: int, scale: float, dv: int, units=None,
              gpu=None) -> Report:
    """Compare the GPU MLA decode (+ combine) with the oracle on (b, h) units b*Hq + h."""
    B, Hq = q.shape[0], q.shape[1]
    if gpu is None:
        gpu = run_gpu_mla(to_device(q), to_device(kv), Bc, lam, S, scale, dv)
    units = list(range(B * Hq)) if units is None else list(units)
    ref = oracle.decode_mla(q, kv, Bc, lam, S, scale, dv, units=units)
    rep = Report()
    force = np.full(ref["skip"].shape, -1, np.int8)
    any_flip = False
    for ui, u in enumerate(units):
        b, h = divmod(u, Hq)
        diff = compare_masks(gpu["skip"][b, h], ref["skip"][ui], ref["margin"][ui], rep, "skip b=%d h=%d" % (b, h))
        if diff.any():
            any_flip = True
            force[ui][diff] = gpu["skip"][b, h][diff]
    if any_flip:
        ref = oracle.decode_mla(q, kv, Bc, lam, S, scale, dv, units=units, force=force)
    o_ref, lse_ref = oracle.combine(ref["o_part"], ref["lse_part"])
    for ui, u in enumerate(units):
        b, h = divmod(u, Hq)
        compare_rows(gpu["o_part"][b, h], ref["o_part"][ui], rep, "o_part b=%d h=%d" % (b, h))
        compare_lse(gpu["lse_part"][b, h], ref["lse_part"][ui], rep, "lse_part b=%d h=%d" % (b, h))
        compare_rows(gpu["o"][b, h][None], o_ref[ui][None], rep, "o b=%d h=%d" % (b, h))
        compare_lse(gpu["lse"][b, h][None], lse_ref[ui][None], rep, "lse b=%d h=%d" % (b, h))
    return rep
