"""FP64 CPU oracle for skip-softmax block-sparse attention — test infrastructure.

Only the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import this package.  The product path (``block_sparse_attention_flash_amd``)
never does, and this package never imports the product.

The arithmetic lives in ``blasst_oracle.c`` (plain C, double precision, one
OpenMP thread per unit); this file only builds/loads that library and
marshals numpy arrays.  Inputs are bf16 bit patterns (uint16 numpy arrays),
exactly the bytes the GPU reads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "blasst_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i, dbl = ctypes.c_int, ctypes.c_double
        lib.oracle_prefill.argtypes = [P, P, P, i, i, i, i, i, i, i, dbl, i, P, i, P, P, P, P, P, i]
        lib.oracle_prefill.restype = i
        lib.oracle_decode.argtypes = [P, P, P, i, i, i, i, i, i, dbl, i, P, i, P, P, P, P, P, P, P, i]
        lib.oracle_decode.restype = i
        lib.oracle_combine.argtypes = [P, P, i, i, i, P, P]
        lib.oracle_combine.restype = i
        lib.oracle_decode_mla.argtypes = [P, P, i, i, i, i, i, i, dbl, dbl, i, P, i, P, P, P, P, P, i]
        lib.oracle_decode_mla.restype = i
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns (uint16), got %s" % a.dtype)
    return a


def _threads(n):
    return n if n else min(16, len(os.sched_getaffinity(0)))


def prefill(q, k, v, Bc: int, lam: float, causal: bool = True, Br: Optional[int] = None,
            units: Optional[Sequence[int]] = None, force: Optional[np.ndarray] = None,
            threads: Optional[int] = None) -> dict:
    """Blockwise causal prefill.  q [B,Hq,T,d], k/v [B,Hkv,T,d] (bf16 bits).

    units: query-block units (b*Hq + hq)*nq + i to compute (default: all).
    Returns per-unit arrays o [U,Br,d], lse [U,Br], mask [U,nk] (0 kept /
    1 skipped / 2 not visited), margin [U,nk] (skipped iff < 0); with all
    units also o_full [B,Hq,T,d], lse_full [B,Hq,T], mask_full [B,Hq,nq,nk].
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    Br = Br or Bc
    nq, nk = -(-T // Br), -(-T // Bc)
    all_units = units is None
    units = np.arange(B * Hq * nq, dtype=np.int64) if all_units else np.asarray(units, np.int64)
    U = len(units)
    o = np.full((U, Br, d), np.nan)
    lse = np.full((U, Br), np.nan)
    mask = np.empty((U, nk), np.uint8)
    margin = np.empty((U, nk))
    f = None if force is None else np.ascontiguousarray(force, np.int8).reshape(U, nk)
    rc = _load().oracle_prefill(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, T, d, Bc, Br, float(lam),
                                int(causal), _ptr(units), U, _ptr(f), _ptr(o), _ptr(lse),
                                _ptr(mask), _ptr(margin), _threads(threads))
    if rc:
        raise ValueError("oracle_prefill rejected its arguments")
    out = dict(o=o, lse=lse, mask=mask, margin=margin, units=units)
    if all_units:
        out["o_full"] = o.reshape(B, Hq, nq * Br, d)[:, :, :T]
        out["lse_full"] = lse.reshape(B, Hq, nq * Br)[:, :, :T]
        out["mask_full"] = mask.reshape(B, Hq, nq, nk)
        out["margin_full"] = margin.reshape(B, Hq, nq, nk)
    return out


def decode(q, k, v, Bc: int, lam: float, num_splits: int,
           units: Optional[Sequence[int]] = None, force: Optional[np.ndarray] = None,
           threads: Optional[int] = None) -> dict:
    """Split-KV decode.  q [B,Hq,1,d], k/v [B,Hkv,N,d] (bf16 bits).

    units: kv-head units b*Hkv + hkv (default: all).  Returns per-unit
    o_part [U,G,S,d], lse_part [U,G,S], skip [U,G,nk], vskip [U,nk],
    margin [U,G,nk], vmargin [U,nk]; with all units also the same arrays in
    [B,Hq,...] / [B,Hkv,...] form under *_full keys.
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, one, d = q.shape
    assert one == 1
    Hkv, N = k.shape[1], k.shape[2]
    G, S, nk = Hq // Hkv, num_splits, -(-N // Bc)
    all_units = units is None
    units = np.arange(B * Hkv, dtype=np.int64) if all_units else np.asarray(units, np.int64)
    U = len(units)
    o_part = np.full((U, G, S, d), np.nan)
    lse_part = np.full((U, G, S), np.nan)
    skip = np.empty((U, G, nk), np.uint8)
    vskip = np.empty((U, nk), np.uint8)
    margin = np.empty((U, G, nk))
    vmargin = np.empty((U, nk))
    f = None if force is None else np.ascontiguousarray(force, np.int8).reshape(U, G, nk)
    rc = _load().oracle_decode(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, N, d, Bc, float(lam), S,
                               _ptr(units), U, _ptr(f), _ptr(o_part), _ptr(lse_part), _ptr(skip),
                               _ptr(vskip), _ptr(margin), _ptr(vmargin), _threads(threads))
    if rc:
        raise ValueError("oracle_decode rejected its arguments")
    out = dict(o_part=o_part, lse_part=lse_part, skip=skip, vskip=vskip, margin=margin,
               vmargin=vmargin, units=units)
    if all_units:
        out["o_part_full"] = o_part.reshape(B, Hq, S, d)
        out["lse_part_full"] = lse_part.reshape(B, Hq, S)
        out["skip_full"] = skip.reshape(B, Hq, nk)
        out["vskip_full"] = vskip.reshape(B, Hkv, nk)
        out["margin_full"] = margin.reshape(B, Hq, nk)
        out["vmargin_full"] = vmargin.reshape(B, Hkv, nk)
    return out


def prefill_ragged(q, k, v, lens, Bc: int, lam: float, causal: bool = True,
                   threads: Optional[int] = None) -> dict:
    """A ragged batch: sequence b is its first lens[b] rows of the padded [B,H,T,d]
    tensors, and is exactly one plain prefill of that length (nothing else of the
    batch is read).  Padded rows get o = 0 and lse = -inf; mask (and margin) entries
    of query or KV blocks past a sequence's end are 2 (NaN), not visited.
    Returns o_full, lse_full, mask_full, margin_full."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, T, d = q.shape
    nq = -(-T // Bc)
    o = np.zeros((B, Hq, T, d))
    lse = np.full((B, Hq, T), -np.inf)
    mask = np.full((B, Hq, nq, nq), 2, np.uint8)
    margin = np.full((B, Hq, nq, nq), np.nan)
    for b, L in enumerate(lens):
        L = int(L)
        if L <= 0:
            continue
        r = prefill(q[b:b + 1, :, :L], k[b:b + 1, :, :L], v[b:b + 1, :, :L], Bc, lam, causal=causal,
                    threads=threads)
        n = -(-L // Bc)
        o[b, :, :L] = r["o_full"][0]
        lse[b, :, :L] = r["lse_full"][0]
        mask[b, :, :n, :n] = r["mask_full"][0]
        margin[b, :, :n, :n] = r["margin_full"][0]
    return dict(o_full=o, lse_full=lse, mask_full=mask, margin_full=margin)


def decode_ragged(q, k, v, lens, Bc: int, lam: float, num_splits: int,
                  threads: Optional[int] = None) -> dict:
    """A ragged decode batch: sequence b attends to the first lens[b] keys of its
    padded [N, d] cache rows, exactly one plain decode of that context length with
    the same num_splits (a split left with no block holds o = 0, lse = -inf).  Mask
    entries of blocks past a sequence's end are 2.  Returns o_part_full,
    lse_part_full, skip_full, vskip_full."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, _, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    nk, S = -(-N // Bc), num_splits
    o_part = np.zeros((B, Hq, S, d))
    lse_part = np.full((B, Hq, S), -np.inf)
    skip = np.full((B, Hq, nk), 2, np.uint8)
    vskip = np.full((B, Hkv, nk), 2, np.uint8)
    for b, L in enumerate(lens):
        L = max(int(L), 0)
        r = decode(q[b:b + 1], k[b:b + 1, :, :L], v[b:b + 1, :, :L], Bc, lam, S, threads=threads)
        n = -(-L // Bc)
        o_part[b] = r["o_part_full"][0]
        lse_part[b] = r["lse_part_full"][0]
        skip[b, :, :n] = r["skip_full"][0]
        vskip[b, :, :n] = r["vskip_full"][0]
    return dict(o_part_full=o_part, lse_part_full=lse_part, skip_full=skip, vskip_full=vskip)


def decode_mla(q, kv, Bc: int, lam: float, num_splits: int, scale: float, dv: int,
               units: Optional[Sequence[int]] = None, force: Optional[np.ndarray] = None,
               threads: Optional[int] = None) -> dict:
    """MLA decode (absorbed latent form).  q [B,Hq,dqk] (or [B,Hq,1,dqk]), kv [B,N,dqk]
    (bf16 bits); token t's value is kv[..., t, :dv]; scores are (q . kv_t) * scale.

    units: (b, h) units b*Hq + h (default: all).  Returns per-unit o_part [U,S,dv],
    lse_part [U,S], skip [U,nk], margin [U,nk] (skipped iff < 0); with all units also
    o_part_full [B,Hq,S,dv], lse_part_full [B,Hq,S], skip_full [B,Hq,nk], margin_full [B,Hq,nk], and
    vskip_full [B,nk] / vmargin_full [B,nk]: no head kept the block (its P V is not
    formed for any head) iff vmargin < 0.
    """
    q, kv = _u16(q), _u16(kv)
    B, Hq, dqk = q.shape[0], q.shape[1], q.shape[-1]
    N = kv.shape[1]
    if q.size != B * Hq * dqk or kv.shape != (B, N, dqk):
        raise ValueError("q must be [B,Hq,dqk] and kv [B,N,dqk]")
    S, nk = num_splits, -(-N // Bc)
    all_units = units is None
    units = np.arange(B * Hq, dtype=np.int64) if all_units else np.asarray(units, np.int64)
    U = len(units)
    o_part = np.full((U, S, dv), np.nan)
    lse_part = np.full((U, S), np.nan)
    skip = np.empty((U, nk), np.uint8)
    margin = np.empty((U, nk))
    f = None if force is None else np.ascontiguousarray(force, np.int8).reshape(U, nk)
    rc = _load().oracle_decode_mla(_ptr(q), _ptr(kv), B, Hq, N, dqk, dv, Bc, float(scale), float(lam), S,
                                   _ptr(units), U, _ptr(f), _ptr(o_part), _ptr(lse_part), _ptr(skip), _ptr(margin),
                                   _threads(threads))
    if rc:
        raise ValueError("oracle_decode_mla rejected its arguments")
    out = dict(o_part=o_part, lse_part=lse_part, skip=skip, margin=margin, units=units)
    if all_units:
        out["o_part_full"] = o_part.reshape(B, Hq, S, dv)
        out["lse_part_full"] = lse_part.reshape(B, Hq, S)
        out["skip_full"] = skip.reshape(B, Hq, nk)
        out["margin_full"] = margin.reshape(B, Hq, nk)
        out["vskip_full"] = skip.reshape(B, Hq, nk).min(axis=1)
        out["vmargin_full"] = margin.reshape(B, Hq, nk).max(axis=1)
    return out


def combine(o_part: np.ndarray, lse_part: np.ndarray):
    """Log-sum-exp merge over the split axis: o_part [..., S, d], lse_part [..., S]."""
    lead = o_part.shape[:-2]
    S, d = o_part.shape[-2:]
    rows = int(np.prod(lead)) if lead else 1
    op = np.ascontiguousarray(o_part, np.float64).reshape(rows, S, d)
    lp = np.ascontiguousarray(lse_part, np.float64).reshape(rows, S)
    o = np.empty((rows, d))
    lse = np.empty(rows)
    rc = _load().oracle_combine(_ptr(op), _ptr(lp), rows, S, d, _ptr(o), _ptr(lse))
    if rc:
        raise ValueError("oracle_combine rejected its arguments")
    return o.reshape(*lead, d), lse.reshape(lead)
