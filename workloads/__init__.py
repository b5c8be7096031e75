"""Seeded synthetic inputs for skip-softmax block-sparse attention.

This module only draws numbers.  It holds none of the attention arithmetic, so
that the HIP path and the FP64 oracle can both take their inputs from here
without sharing any of the method's code.

The recipe stands in for the long-context workloads the BLASST blog measures on
(Llama-3.1-8B / Qwen3-8B attention over RULER, LongBench and reasoning tasks at
4K-128K context; blog sections on fixed thresholds, Table 6 and Fig 2).  Those
datasets and trained weights are not used: attention on them is heavy-tailed
(a few tokens take most of the softmax mass, blog section on the problem), and
the generator reproduces that shape with a planted direction:

* u: one unit vector per workload, drawn from N(0, I_d) and normalised.
* Q = N(0,1) + a*u for every query, K = N(0,1), V = N(0,1).
* "hot" keys (attention sinks at positions 0..sinks-1, plus round(r*T)
  positions drawn uniformly without replacement from [sinks, T)) get + a*u.
  With a = sqrt(8*sqrt(d)) a hot key's scaled logit is about a^2/sqrt(d) = +8
  over an N(0, 1 + a^2/d) background.
* optionally the last `window` keys get + c_w*u with c_w = window_logit*sqrt(d)/a,
  i.e. a recent-window bias of +window_logit in the scaled logit.
* the score scale is 1/sqrt(d) unless a workload sets another (MLA: the
  model's scale over d = 576 cache columns); amplitudes are set so that the
  scaled logits above hold at that scale.
* optionally (logit_tail = tau > 0) every key j gets + e_j*sqrt(d)/a * u with
  e_j ~ Exponential(mean tau): an extra scaled logit of about e_j, so that the
  scores have an exponential upper tail and the running max of a row grows like
  tau * ln(position).  This is the length-sweep family: with sinks and hot keys
  off, a fixed threshold skips more blocks the longer the context (the drift of
  the blog's Table 6 / Fig 2 right), which the planted hot keys alone do not
  show because their +8 logit fixes the max early.
* every tensor is rounded to bfloat16 with round-to-nearest-even; the same
  bytes go to the GPU and to the oracle.

Every (tensor, batch, head) slice has its own PCG64 stream keyed by
SeedSequence(seed, spawn_key=(tag, b, h)), so a slice can be regenerated on its
own (the oracle only needs the slices it samples) and the full tensors can be
drawn in parallel threads.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence, Tuple, Union

import numpy as np

_TAG_DIR, _TAG_Q, _TAG_K, _TAG_V, _TAG_HOT, _TAG_RATE, _TAG_TAIL = 0, 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention call's shape plus the generator recipe for its inputs."""

    name: str
    kind: str  # "prefill" or "decode"
    B: int
    Hq: int
    Hkv: int
    d: int
    T: int  # prefill: sequence length; decode: context length N
    Bc: int
    lambdas: Tuple[float, ...]
    hot_rate: Union[float, Tuple[float, float]]  # fixed r, or (lo, hi) drawn per sequence
    seed: int
    sinks: int = 4
    window: int = 0
    window_logit: float = 3.0
    hot_logit: float = 8.0
    num_splits: int = 1  # decode only
    logit_tail: float = 0.0  # mean of the exponential extra logit per key (0: off)
    dv: int = 0              # MLA: value width (the first dv columns of a cache row); 0: not MLA
    scale: float = 0.0       # softmax scale of the scores; 0: 1/sqrt(d)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def Tq(self) -> int:
        return self.T if self.kind == "prefill" else 1

    @property
    def score_scale(self) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(self.d)

    @property
    def amplitude(self) -> float:
        # hot logit = a^2 * scale (a^2 / sqrt(d) at the default scale)
        return math.sqrt(self.hot_logit / self.score_scale)

    @property
    def window_coef(self) -> float:
        return self.window_logit / (self.score_scale * self.amplitude)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _seed(cfg_id: int) -> int:
    return 20261202 + 1000 * cfg_id


# The five workloads the measurements are quoted on (Llama-3.1-8B-like heads).
CONFIGS = {
    "prefill_1k_tiny": Workload("prefill_1k_tiny", "prefill", B=1, Hq=4, Hkv=1, d=64, T=1024,
                                Bc=64, lambdas=(1e-3,), hot_rate=0.02, seed=_seed(1)),
    "decode_32k": Workload("decode_32k", "decode", B=1, Hq=32, Hkv=8, d=128, T=32768, Bc=128,
                           lambdas=(1e-3,), hot_rate=0.01, seed=_seed(2), window=512,
                           num_splits=16),
    "prefill_32k": Workload("prefill_32k", "prefill", B=1, Hq=32, Hkv=8, d=128, T=32768,
                            Bc=128, lambdas=(1e-4, 1e-3, 1e-2), hot_rate=0.01, seed=_seed(3)),
    "decode_128k_b16": Workload("decode_128k_b16", "decode", B=16, Hq=32, Hkv=8, d=128,
                                T=131072, Bc=128, lambdas=(1e-3,), hot_rate=(0.005, 0.03),
                                seed=_seed(4), num_splits=32),
    "decode_mqa_16k": Workload("decode_mqa_16k", "decode", B=64, Hq=64, Hkv=1, d=128, T=16384,
                               Bc=128, lambdas=(1e-3,), hot_rate=0.02, seed=_seed(5),
                               num_splits=4),  # 64 x 4 splits: one workgroup per CU
}

# MLA decode (DeepSeek-V3-like absorbed attention: 128 heads over 512 latent +
# 64 rotary columns, softmax scale 1/sqrt(128 + 64)); the cache is the "k"
# tensor with one kv head, the value is its first dv columns.
MLA_CONFIGS = {
    "decode_mla_32k": Workload("decode_mla_32k", "decode", B=8, Hq=128, Hkv=1, d=576, T=32768, Bc=64,
                               lambdas=(1e-3,), hot_rate=0.01, seed=_seed(8), window=512, num_splits=16,
                               dv=512, scale=1.0 / math.sqrt(192.0)),
}


# The length-sweep family: heavy-tailed scores with no planted structure, at a
# context length L per call.  "calibration" and "evaluation" draw different
# sequences (seed sets), so a threshold fitted on one is checked on the other.
SWEEP_LENGTHS = (4096, 8192, 16384, 32768, 65536, 131072)


def sweep_workload(kind: str, L: int, split: str = "calibration", B: Optional[int] = None) -> Workload:
    base = {"calibration": _seed(6), "evaluation": _seed(7)}[split]
    if kind == "decode":
        return Workload("sweep_decode_%d" % L, "decode", B=B or 4, Hq=32, Hkv=8, d=128, T=L, Bc=128,
                        lambdas=(1e-3, 3e-3), hot_rate=0.0, seed=base + L // 1024, sinks=0,
                        logit_tail=1.0, num_splits=1)
    if kind == "prefill":
        return Workload("sweep_prefill_%d" % L, "prefill", B=B or 1, Hq=32, Hkv=8, d=128, T=L, Bc=128,
                        lambdas=(1e-3, 3e-3), hot_rate=0.0, seed=base + L // 1024 + 500, sinks=0,
                        logit_tail=1.0)
    raise ValueError("kind is prefill or decode")


def _rng(w: Workload, tag: int, b: int = 0, h: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed, spawn_key=(tag, b, h))))


def direction(w: Workload) -> np.ndarray:
    """The planted unit direction u (float32, [d])."""
    g = _rng(w, _TAG_DIR).standard_normal(w.d)
    return (g / np.linalg.norm(g)).astype(np.float32)


def sequence_hot_rate(w: Workload, b: int) -> float:
    if isinstance(w.hot_rate, tuple):
        lo, hi = w.hot_rate
        rates = _rng(w, _TAG_RATE).uniform(lo, hi, size=w.B)
        return float(rates[b])
    return float(w.hot_rate)


def hot_positions(w: Workload, b: int, hkv: int) -> np.ndarray:
    """Sorted key positions of kv-head (b, hkv) that carry the planted direction."""
    T = w.T
    sinks = min(w.sinks, T)
    n_hot = int(round(sequence_hot_rate(w, b) * T))
    n_hot = min(n_hot, T - sinks)
    drawn = _rng(w, _TAG_HOT, b, hkv).choice(np.arange(sinks, T), size=n_hot, replace=False)
    return np.sort(np.concatenate([np.arange(sinks), drawn]).astype(np.int64))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def q_slice(w: Workload, b: int, hq: int) -> np.ndarray:
    """bf16 bits [Tq, d] of query head (b, hq)."""
    x = _rng(w, _TAG_Q, b, hq).standard_normal((w.Tq, w.d), dtype=np.float32)
    x += np.float32(w.amplitude) * direction(w)
    return to_bf16_bits(x)


def k_slice(w: Workload, b: int, hkv: int) -> np.ndarray:
    """bf16 bits [T, d] of key head (b, hkv)."""
    x = _rng(w, _TAG_K, b, hkv).standard_normal((w.T, w.d), dtype=np.float32)
    u = direction(w)
    x[hot_positions(w, b, hkv)] += np.float32(w.amplitude) * u
    if w.window > 0:
        x[max(0, w.T - w.window):] += np.float32(w.window_coef) * u
    if w.logit_tail > 0:
        e = _rng(w, _TAG_TAIL, b, hkv).exponential(w.logit_tail, size=w.T).astype(np.float32)
        x += (e * np.float32(1.0 / (w.score_scale * w.amplitude)))[:, None] * u[None, :]
    return to_bf16_bits(x)


def v_slice(w: Workload, b: int, hkv: int) -> np.ndarray:
    """bf16 bits [T, d] of value head (b, hkv)."""
    return to_bf16_bits(_rng(w, _TAG_V, b, hkv).standard_normal((w.T, w.d), dtype=np.float32))


def generate(w: Workload, threads: Optional[int] = None,
             parts: Sequence[str] = ("q", "k", "v")) -> dict:
    """Full bf16-bit tensors: q [B,Hq,Tq,d], k and v [B,Hkv,T,d] (uint16)."""
    threads = threads or min(16, (len(__import__("os").sched_getaffinity(0)) or 1))
    out = {}
    jobs = []
    if "q" in parts:
        out["q"] = np.empty((w.B, w.Hq, w.Tq, w.d), np.uint16)
        jobs += [("q", b, h) for b in range(w.B) for h in range(w.Hq)]
    if "k" in parts:
        out["k"] = np.empty((w.B, w.Hkv, w.T, w.d), np.uint16)
        jobs += [("k", b, h) for b in range(w.B) for h in range(w.Hkv)]
    if "v" in parts:
        out["v"] = np.empty((w.B, w.Hkv, w.T, w.d), np.uint16)
        jobs += [("v", b, h) for b in range(w.B) for h in range(w.Hkv)]
    fn = {"q": q_slice, "k": k_slice, "v": v_slice}

    def run(job):
        t, b, h = job
        out[t][b, h] = fn[t](w, b, h)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, jobs))
    return out


def generate_group(w: Workload, b: int, hkv: int) -> dict:
    """The slices one kv-head group needs: q [1,G,Tq,d], k and v [1,1,T,d]."""
    G = w.G
    q = np.stack([q_slice(w, b, hkv * G + g) for g in range(G)])[None]
    return {"q": q, "k": k_slice(w, b, hkv)[None, None], "v": v_slice(w, b, hkv)[None, None]}
