"""Skip-softmax (BLASST) block-sparse attention on AMD Instinct MI355X.

A thin ctypes binding over ``libblasst.so`` (C ABI in ``include/blasst.h``).
The functions named like the C entry points take PyTorch tensors that already
live on the GPU and only marshal pointers, sizes and the current HIP stream;
every step of the computation runs in the library's HIP kernels.  If the
library is missing or fails to load, importing the binding's functions raises:
there is no CPU or PyTorch fallback.

The convenience wrappers ``prefill``, ``decode``, ``decode_combine``,
``prefill_margins`` and ``decode_margins`` allocate their outputs with PyTorch
and call the entry points.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["blasst_prefill", "blasst_decode", "blasst_decode_combine", "blasst_prefill_margins",
           "blasst_decode_margins", "blasst_prefill_ragged", "blasst_decode_ragged", "blasst_decode_mla", "blasst_prefill_dense",
           "blasst_decode_dense", "blasst_decode_load_ceiling", "blasst_decode_step", "decode_step_workspace_size",
           "blasst_decode_step_noalloc",
           "decode_step", "status_string",
           "prefill", "decode", "decode_combine", "prefill_margins", "decode_margins", "prefill_ragged",
           "decode_ragged", "decode_mla",
           "BlasstError", "library_path", "build"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libblasst.so")
_lib = None

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_INTERNAL = 0, 1, 2, 3, 4


class BlasstError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (status %d)" % (fn, status_string(status), status))
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def build(verbose: bool = False) -> str:
    """Compile libblasst.so in-tree with hipcc for gfx950."""
    from . import _build
    return _build.build(verbose=verbose)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libblasst.so is not built (%s); run "
                              "`python -m block_sparse_attention_flash_amd._build`" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        P, i, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.blasst_prefill.argtypes = [P, P, P, P, P, P, i, i, i, i, i, i, d, i, P]
        lib.blasst_prefill.restype = i
        lib.blasst_decode.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, i, d, i, i, P]
        lib.blasst_decode.restype = i
        lib.blasst_decode_combine.argtypes = [P, P, P, P, i, i, i, i, P]
        lib.blasst_decode_combine.restype = i
        lib.blasst_prefill_margins.argtypes = [P, P, P, i, i, i, i, i, i, i, P]
        lib.blasst_prefill_margins.restype = i
        lib.blasst_decode_margins.argtypes = [P, P, P, P, i, i, i, i, i, i, i, P]
        lib.blasst_decode_margins.restype = i
        lib.blasst_prefill_ragged.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, i, d, i, P]
        lib.blasst_prefill_ragged.restype = i
        lib.blasst_decode_ragged.argtypes = [P, P, P, P, P, P, P, P, i, i, i, i, i, i, d, i, P]
        lib.blasst_decode_ragged.restype = i
        lib.blasst_decode_mla.argtypes = [P, P, P, P, P, i, i, i, i, i, i, d, d, i, P]
        lib.blasst_decode_mla.restype = i
        lib.blasst_prefill_dense.argtypes = [P, P, P, P, P, i, i, i, i, i, i, i, P]
        lib.blasst_prefill_dense.restype = i
        lib.blasst_decode_dense.argtypes = [P, P, P, P, P, i, i, i, i, i, i, i, P]
        lib.blasst_decode_dense.restype = i
        lib.blasst_decode_step.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_size_t, i, i, i, i, i, i, d, i, i, P]
        lib.blasst_decode_step.restype = i
        lib.blasst_decode_step_noalloc.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, i, d, i, i, P]
        lib.blasst_decode_step_noalloc.restype = i
        lib.blasst_decode_step_noalloc_max_bytes.argtypes = []
        lib.blasst_decode_step_noalloc_max_bytes.restype = ctypes.c_size_t
        lib.blasst_decode_step_workspace_size.argtypes = [i, i, i, i]
        lib.blasst_decode_step_workspace_size.restype = ctypes.c_size_t
        lib.blasst_decode_load_ceiling.argtypes = [P, P, i, i, i, i, i, i, P]
        lib.blasst_decode_load_ceiling.restype = i
        lib.blasst_status_string.argtypes = [i]
        lib.blasst_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return _load().blasst_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream: Optional[torch.cuda.Stream]):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, status: int):
    if status != OK:
        raise BlasstError(fn, status)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype):
    if not (t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError("%s must be a contiguous %s tensor on the GPU" % (name, dtype))


def _prefill_shapes(q, k, v, o, lse, skip_mask, Bc):
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16)
    _need(o, "o", torch.float32)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if Hkv == 0 or Hq % Hkv or k.shape != (B, Hkv, T, d) or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("inconsistent prefill shapes")
    nq = -(-T // Bc)
    if lse is not None:
        _need(lse, "lse", torch.float32)
        if lse.shape != (B, Hq, T):
            raise ValueError("lse must be [B,Hq,T]")
    if skip_mask is not None:
        _need(skip_mask, "skip_mask", torch.uint8)
        if skip_mask.shape != (B, Hq, nq, nq):
            raise ValueError("skip_mask must be [B,Hq,nq,nq]")
    return B, Hq, T, d, Hkv


def _lens(seq_lens, B):
    _need(seq_lens, "seq_lens", torch.int32)
    if seq_lens.shape != (B,):
        raise ValueError("seq_lens must be [B]")
    return seq_lens


def blasst_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                   lse: Optional[torch.Tensor], skip_mask: Optional[torch.Tensor], Bc: int,
                   lam: float, causal: bool = True, stream=None) -> None:
    """q [B,Hq,T,d], k/v [B,Hkv,T,d] bf16; o [B,Hq,T,d] fp32; lse [B,Hq,T] fp32 or None;
    skip_mask [B,Hq,nq,nq] uint8 or None."""
    B, Hq, T, d, Hkv = _prefill_shapes(q, k, v, o, lse, skip_mask, Bc)
    st = _load().blasst_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(skip_mask), B, Hq, T, d,
                                Hq // Hkv, Bc, float(lam), int(bool(causal)), _stream(stream))
    _check("blasst_prefill", st)


def blasst_prefill_ragged(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                          lse: Optional[torch.Tensor], skip_mask: Optional[torch.Tensor], seq_lens: torch.Tensor,
                          Bc: int, lam: float, causal: bool = True, stream=None) -> None:
    """As blasst_prefill on padded [B,H,T,d] tensors; seq_lens int32 [B] on the device (rows per sequence)."""
    B, Hq, T, d, Hkv = _prefill_shapes(q, k, v, o, lse, skip_mask, Bc)
    _lens(seq_lens, B)
    st = _load().blasst_prefill_ragged(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(skip_mask),
                                       _ptr(seq_lens), B, Hq, T, d, Hq // Hkv, Bc, float(lam), int(bool(causal)),
                                       _stream(stream))
    _check("blasst_prefill_ragged", st)


def _decode_shapes(q, k, v, o_part, lse_part, skip_mask, vskip_mask, Bc, num_splits):
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16)
    _need(o_part, "o_part", torch.float32)
    _need(lse_part, "lse_part", torch.float32)
    B, Hq, one, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    S = num_splits
    if one != 1 or Hkv == 0 or Hq % Hkv or k.shape != (B, Hkv, N, d) or v.shape != k.shape:
        raise ValueError("inconsistent decode shapes")
    if o_part.shape != (B, Hq, S, d) or lse_part.shape != (B, Hq, S):
        raise ValueError("o_part must be [B,Hq,S,d] and lse_part [B,Hq,S]")
    nk = -(-N // Bc)
    if skip_mask is not None:
        _need(skip_mask, "skip_mask", torch.uint8)
        if skip_mask.shape != (B, Hq, nk):
            raise ValueError("skip_mask must be [B,Hq,nk]")
    if vskip_mask is not None:
        _need(vskip_mask, "vskip_mask", torch.uint8)
        if vskip_mask.shape != (B, Hkv, nk):
            raise ValueError("vskip_mask must be [B,Hkv,nk]")
    return B, Hq, N, d, Hkv


def blasst_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o_part: torch.Tensor,
                  lse_part: torch.Tensor, skip_mask: Optional[torch.Tensor], vskip_mask: Optional[torch.Tensor],
                  Bc: int, lam: float, num_splits: int, causal: bool = True, stream=None) -> None:
    """q [B,Hq,1,d], k/v [B,Hkv,N,d] bf16; o_part [B,Hq,S,d], lse_part [B,Hq,S] fp32;
    skip_mask [B,Hq,nk] / vskip_mask [B,Hkv,nk] uint8 or None."""
    B, Hq, N, d, Hkv = _decode_shapes(q, k, v, o_part, lse_part, skip_mask, vskip_mask, Bc, num_splits)
    st = _load().blasst_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part), _ptr(skip_mask),
                               _ptr(vskip_mask), B, Hq, N, d, Hq // Hkv, Bc, float(lam), int(bool(causal)),
                               num_splits, _stream(stream))
    _check("blasst_decode", st)


def blasst_prefill_dense(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                         lse: Optional[torch.Tensor], Bc: int, causal: bool = True, stream=None) -> None:
    """blasst_prefill without the skip test (every tile kept)."""
    B, Hq, T, d, Hkv = _prefill_shapes(q, k, v, o, lse, None, Bc)
    st = _load().blasst_prefill_dense(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, T, d, Hq // Hkv, Bc,
                                      int(bool(causal)), _stream(stream))
    _check("blasst_prefill_dense", st)


def blasst_decode_dense(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o_part: torch.Tensor,
                        lse_part: torch.Tensor, Bc: int, num_splits: int, stream=None) -> None:
    """blasst_decode without the skip test (every block kept, V always loaded)."""
    B, Hq, N, d, Hkv = _decode_shapes(q, k, v, o_part, lse_part, None, None, Bc, num_splits)
    st = _load().blasst_decode_dense(_ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part), B, Hq, N, d,
                                     Hq // Hkv, Bc, num_splits, _stream(stream))
    _check("blasst_decode_dense", st)


def decode_step_workspace_size(B: int, Hq: int, d: int, num_splits: int) -> int:
    """Bytes of the split partials blasst_decode_step needs."""
    return int(_load().blasst_decode_step_workspace_size(B, Hq, d, num_splits))


def blasst_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: Optional[torch.Tensor],
                       skip_mask: Optional[torch.Tensor], vskip_mask: Optional[torch.Tensor], workspace: torch.Tensor,
                       Bc: int, lam: float, num_splits: int, stream: Optional[torch.cuda.Stream] = None) -> None:
    """One decode step (split kernel + merge) with the partials in `workspace` (uint8 on the GPU)."""
    B, Hq, one, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16)
    _need(v, "v", torch.bfloat16)
    _need(o, "o", torch.float32)
    _need(workspace, "workspace", torch.uint8)
    if one != 1 or v.shape != k.shape or o.shape != (B, Hq, d) or (lse is not None and lse.shape != (B, Hq)):
        raise ValueError("q [B,Hq,1,d], k and v [B,Hkv,N,d], o [B,Hq,d], lse [B,Hq]")
    if lse is not None:
        _need(lse, "lse", torch.float32)
    nk = -(-N // Bc)
    for t, shp, nm in ((skip_mask, (B, Hq, nk), "skip_mask"), (vskip_mask, (B, Hkv, nk), "vskip_mask")):
        if t is not None:
            _need(t, nm, torch.uint8)
            if t.shape != shp:
                raise ValueError("%s must be %s" % (nm, shp))
    st = _load().blasst_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(skip_mask), _ptr(vskip_mask),
                                    _ptr(workspace), workspace.numel(), B, Hq, N, d, Hq // Hkv, Bc, float(lam), 1,
                                    num_splits, _stream(stream))
    _check("blasst_decode_step", st)


def blasst_decode_step_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                               lse: Optional[torch.Tensor], skip_mask: Optional[torch.Tensor],
                               vskip_mask: Optional[torch.Tensor], Bc: int, lam: float, num_splits: int,
                               stream: Optional[torch.cuda.Stream] = None) -> None:
    """blasst_decode_step with the partials in the library's own per-GPU array: allocates nothing."""
    B, Hq, one, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16)
    _need(v, "v", torch.bfloat16)
    _need(o, "o", torch.float32)
    if one != 1 or v.shape != k.shape or o.shape != (B, Hq, d) or (lse is not None and lse.shape != (B, Hq)):
        raise ValueError("q [B,Hq,1,d], k and v [B,Hkv,N,d], o [B,Hq,d], lse [B,Hq]")
    if lse is not None:
        _need(lse, "lse", torch.float32)
    nk = -(-N // Bc)
    for t, shp, nm in ((skip_mask, (B, Hq, nk), "skip_mask"), (vskip_mask, (B, Hkv, nk), "vskip_mask")):
        if t is not None:
            _need(t, nm, torch.uint8)
            if t.shape != shp:
                raise ValueError("%s must be %s" % (nm, shp))
    st = _load().blasst_decode_step_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(skip_mask),
                                            _ptr(vskip_mask), B, Hq, N, d, Hq // Hkv, Bc, float(lam), 1, num_splits,
                                            _stream(stream))
    _check("blasst_decode_step_noalloc", st)


def decode_step_noalloc_max_bytes() -> int:
    return int(_load().blasst_decode_step_noalloc_max_bytes())


def decode_step(q, k, v, lam: float, num_splits: int, Bc: int = 128, with_masks: bool = True):
    """Allocating wrapper: returns (o [B,Hq,d], lse [B,Hq], skip or None, vskip or None)."""
    B, Hq, _, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    nk = -(-N // Bc)
    o = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    skip = torch.empty((B, Hq, nk), dtype=torch.uint8, device=q.device) if with_masks else None
    vskip = torch.empty((B, Hkv, nk), dtype=torch.uint8, device=q.device) if with_masks else None
    ws = torch.empty(max(16, decode_step_workspace_size(B, Hq, d, num_splits)), dtype=torch.uint8, device=q.device)
    blasst_decode_step(q, k, v, o, lse, skip, vskip, ws, Bc, lam, num_splits)
    return o, lse, skip, vskip


def blasst_decode_load_ceiling(k: torch.Tensor, v: torch.Tensor, Bc: int, num_splits: int,
                               stream: Optional[torch.cuda.Stream] = None) -> None:
    """Measurement only: the decode split kernel's HBM reads at lambda = 0, with nothing computed."""
    _need(k, "k", torch.bfloat16)
    _need(v, "v", torch.bfloat16)
    if k.shape != v.shape or k.dim() != 4:
        raise ValueError("k and v must be [B, Hkv, N, d] and of one shape")
    B, Hkv, N, d = k.shape
    st = _load().blasst_decode_load_ceiling(_ptr(k), _ptr(v), B, Hkv, N, d, Bc, num_splits, _stream(stream))
    _check("blasst_decode_load_ceiling", st)


def blasst_decode_ragged(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o_part: torch.Tensor,
                         lse_part: torch.Tensor, skip_mask: Optional[torch.Tensor],
                         vskip_mask: Optional[torch.Tensor], seq_lens: torch.Tensor, Bc: int, lam: float,
                         num_splits: int, stream=None) -> None:
    """As blasst_decode on a padded [B,Hkv,N,d] cache; seq_lens int32 [B] on the device (keys per sequence)."""
    B, Hq, N, d, Hkv = _decode_shapes(q, k, v, o_part, lse_part, skip_mask, vskip_mask, Bc, num_splits)
    _lens(seq_lens, B)
    st = _load().blasst_decode_ragged(_ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part), _ptr(skip_mask),
                                      _ptr(vskip_mask), _ptr(seq_lens), B, Hq, N, d, Hq // Hkv, Bc, float(lam),
                                      num_splits, _stream(stream))
    _check("blasst_decode_ragged", st)


def blasst_decode_combine(o_part: torch.Tensor, lse_part: torch.Tensor, o: torch.Tensor,
                          lse: Optional[torch.Tensor], stream=None) -> None:
    """o_part [B,Hq,S,d], lse_part [B,Hq,S] -> o [B,Hq,d], lse [B,Hq] or None (fp32)."""
    _need(o_part, "o_part", torch.float32)
    _need(lse_part, "lse_part", torch.float32)
    _need(o, "o", torch.float32)
    B, Hq, S, d = o_part.shape
    if lse_part.shape != (B, Hq, S) or o.shape != (B, Hq, d):
        raise ValueError("inconsistent combine shapes")
    if lse is not None:
        _need(lse, "lse", torch.float32)
        if lse.shape != (B, Hq):
            raise ValueError("lse must be [B,Hq]")
    st = _load().blasst_decode_combine(_ptr(o_part), _ptr(lse_part), _ptr(o), _ptr(lse), B, Hq, d, S,
                                       _stream(stream))
    _check("blasst_decode_combine", st)


def blasst_prefill_margins(q: torch.Tensor, k: torch.Tensor, margin: torch.Tensor, Bc: int,
                           causal: bool = True, stream=None) -> None:
    """q [B,Hq,T,d], k [B,Hkv,T,d] bf16 -> margin [B,Hq,nq,nq] fp32 (natural log; NaN = not visited)."""
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16)
    _need(margin, "margin", torch.float32)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if Hkv == 0 or Hq % Hkv or k.shape != (B, Hkv, T, d):
        raise ValueError("inconsistent prefill shapes")
    nq = -(-T // Bc)
    if margin.shape != (B, Hq, nq, nq):
        raise ValueError("margin must be [B,Hq,nq,nq]")
    st = _load().blasst_prefill_margins(_ptr(q), _ptr(k), _ptr(margin), B, Hq, T, d, Hq // Hkv, Bc,
                                        int(bool(causal)), _stream(stream))
    _check("blasst_prefill_margins", st)


def blasst_decode_margins(q: torch.Tensor, k: torch.Tensor, margin: torch.Tensor, vmargin: Optional[torch.Tensor],
                          Bc: int, num_splits: int, stream=None) -> None:
    """q [B,Hq,1,d], k [B,Hkv,N,d] bf16 -> margin [B,Hq,nk], vmargin [B,Hkv,nk] or None (fp32, natural log)."""
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16)
    _need(margin, "margin", torch.float32)
    B, Hq, one, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    if one != 1 or Hkv == 0 or Hq % Hkv or k.shape != (B, Hkv, N, d):
        raise ValueError("inconsistent decode shapes")
    nk = -(-N // Bc)
    if margin.shape != (B, Hq, nk):
        raise ValueError("margin must be [B,Hq,nk]")
    if vmargin is not None:
        _need(vmargin, "vmargin", torch.float32)
        if vmargin.shape != (B, Hkv, nk):
            raise ValueError("vmargin must be [B,Hkv,nk]")
    st = _load().blasst_decode_margins(_ptr(q), _ptr(k), _ptr(margin), _ptr(vmargin), B, Hq, N, d, Hq // Hkv, Bc,
                                       num_splits, _stream(stream))
    _check("blasst_decode_margins", st)


def prefill_margins(q, k, Bc: int = 128, causal: bool = True) -> torch.Tensor:
    """Allocating wrapper: margin fp32 [B,Hq,nq,nq]."""
    B, Hq, T, d = q.shape
    nq = -(-T // Bc)
    margin = torch.empty((B, Hq, nq, nq), dtype=torch.float32, device=q.device)
    blasst_prefill_margins(q, k, margin, Bc, causal)
    return margin


def decode_margins(q, k, num_splits: int, Bc: int = 128) -> Tuple[torch.Tensor, torch.Tensor]:
    """Allocating wrapper: (margin [B,Hq,nk], vmargin [B,Hkv,nk]), fp32."""
    B, Hq, _, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    nk = -(-N // Bc)
    margin = torch.empty((B, Hq, nk), dtype=torch.float32, device=q.device)
    vmargin = torch.empty((B, Hkv, nk), dtype=torch.float32, device=q.device)
    blasst_decode_margins(q, k, margin, vmargin, Bc, num_splits)
    return margin, vmargin


def prefill(q, k, v, lam: float, Bc: int = 128, causal: bool = True,
            with_mask: bool = True) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """Allocating wrapper: returns (o fp32 [B,Hq,T,d], lse [B,Hq,T], mask [B,Hq,nq,nq] or None)."""
    B, Hq, T, d = q.shape
    nq = -(-T // Bc)
    o = torch.empty((B, Hq, T, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    mask = torch.empty((B, Hq, nq, nq), dtype=torch.uint8, device=q.device) if with_mask else None
    blasst_prefill(q, k, v, o, lse, mask, Bc, lam, causal)
    return o, lse, mask


def decode(q, k, v, lam: float, num_splits: int, Bc: int = 128, with_masks: bool = True):
    """Allocating wrapper: returns (o_part, lse_part, skip [B,Hq,nk], vskip [B,Hkv,nk])."""
    B, Hq, _, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    nk = -(-N // Bc)
    o_part = torch.empty((B, Hq, num_splits, d), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((B, Hq, num_splits), dtype=torch.float32, device=q.device)
    skip = torch.empty((B, Hq, nk), dtype=torch.uint8, device=q.device) if with_masks else None
    vskip = torch.empty((B, Hkv, nk), dtype=torch.uint8, device=q.device) if with_masks else None
    blasst_decode(q, k, v, o_part, lse_part, skip, vskip, Bc, lam, num_splits)
    return o_part, lse_part, skip, vskip


def prefill_ragged(q, k, v, seq_lens, lam: float, Bc: int = 128, causal: bool = True, with_mask: bool = True):
    """Allocating wrapper for a ragged batch: returns (o, lse, mask or None) as prefill()."""
    B, Hq, T, d = q.shape
    nq = -(-T // Bc)
    o = torch.empty((B, Hq, T, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    mask = torch.empty((B, Hq, nq, nq), dtype=torch.uint8, device=q.device) if with_mask else None
    blasst_prefill_ragged(q, k, v, o, lse, mask, seq_lens, Bc, lam, causal)
    return o, lse, mask


def decode_ragged(q, k, v, seq_lens, lam: float, num_splits: int, Bc: int = 128, with_masks: bool = True):
    """Allocating wrapper for a ragged batch: returns (o_part, lse_part, skip, vskip) as decode()."""
    B, Hq, _, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    nk = -(-N // Bc)
    o_part = torch.empty((B, Hq, num_splits, d), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((B, Hq, num_splits), dtype=torch.float32, device=q.device)
    skip = torch.empty((B, Hq, nk), dtype=torch.uint8, device=q.device) if with_masks else None
    vskip = torch.empty((B, Hkv, nk), dtype=torch.uint8, device=q.device) if with_masks else None
    blasst_decode_ragged(q, k, v, o_part, lse_part, skip, vskip, seq_lens, Bc, lam, num_splits)
    return o_part, lse_part, skip, vskip


def blasst_decode_mla(q: torch.Tensor, kv: torch.Tensor, o_part: torch.Tensor, lse_part: torch.Tensor,
                      skip_mask: Optional[torch.Tensor], Bc: int, softmax_scale: float, lam: float,
                      num_splits: int, d_v: int = 512, stream=None) -> None:
    """q [B,Hq,d_qk] (or [B,Hq,1,d_qk]), kv [B,N,d_qk] bf16; o_part [B,Hq,S,d_v], lse_part [B,Hq,S] fp32;
    skip_mask [B,Hq,nk] uint8 or None."""
    _need(q, "q", torch.bfloat16)
    _need(kv, "kv", torch.bfloat16)
    _need(o_part, "o_part", torch.float32)
    _need(lse_part, "lse_part", torch.float32)
    B, Hq, d_qk = q.shape[0], q.shape[1], q.shape[-1]
    N = kv.shape[1]
    S = num_splits
    if q.numel() != B * Hq * d_qk or kv.shape != (B, N, d_qk):
        raise ValueError("q must be [B,Hq,d_qk] and kv [B,N,d_qk]")
    if o_part.shape != (B, Hq, S, d_v) or lse_part.shape != (B, Hq, S):
        raise ValueError("o_part must be [B,Hq,S,d_v] and lse_part [B,Hq,S]")
    if skip_mask is not None:
        _need(skip_mask, "skip_mask", torch.uint8)
        if skip_mask.shape != (B, Hq, -(-N // Bc)):
            raise ValueError("skip_mask must be [B,Hq,nk]")
    st = _load().blasst_decode_mla(_ptr(q), _ptr(kv), _ptr(o_part), _ptr(lse_part), _ptr(skip_mask), B, Hq, N,
                                   d_qk, d_v, Bc, float(softmax_scale), float(lam), S, _stream(stream))
    _check("blasst_decode_mla", st)


def decode_mla(q, kv, lam: float, num_splits: int, softmax_scale: float, Bc: int = 64, d_v: int = 512,
               with_mask: bool = True):
    """Allocating wrapper: returns (o_part [B,Hq,S,d_v], lse_part [B,Hq,S], skip [B,Hq,nk] or None)."""
    B, Hq = q.shape[0], q.shape[1]
    N = kv.shape[1]
    o_part = torch.empty((B, Hq, num_splits, d_v), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((B, Hq, num_splits), dtype=torch.float32, device=q.device)
    skip = torch.empty((B, Hq, -(-N // Bc)), dtype=torch.uint8, device=q.device) if with_mask else None
    blasst_decode_mla(q, kv, o_part, lse_part, skip, Bc, softmax_scale, lam, num_splits, d_v)
    return o_part, lse_part, skip


def decode_combine(o_part, lse_part):
    """Allocating wrapper: returns (o [B,Hq,d], lse [B,Hq])."""
    B, Hq, S, d = o_part.shape
    o = torch.empty((B, Hq, d), dtype=torch.float32, device=o_part.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=o_part.device)
    blasst_decode_combine(o_part, lse_part, o, lse)
    return o, lse
