"""Seeded synthetic inputs for DropKV eviction scoring.

This module only draws and rounds input tensors; it holds none of the
scoring arithmetic, so both the HIP path and the fp64 oracle can take their
inputs from it without sharing any of the method.

The workloads stand in for the long-context evaluations the DropKV pages
describe (Llama-3.1-8B / Qwen2.5-7B layer shapes up to 128K tokens; atlas
summary, "Experimental setup" and "Key results"; the write-up's tiny synthetic
protocol in section 数据协议与运行): Gaussian Q/K/V with a planted attention
sink and planted "needle" keys along the mean query direction of each GQA
group. Real K/V statistics (outlier channels, trained sinks) are not
reproduced.

Layout of one sequence (one batch element):
  q: [Hq][window][d]   the queries of the last `window` positions
  k, v: [Hkv][n][d]    the full causal K/V
Query head h belongs to KV head h // (Hq // Hkv).
bf16 tensors are returned as uint16 bit patterns (round-to-nearest-even from
the fp32 draw); fp32 tensors as float32.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Config",
    "CONFIGS",
    "Case",
    "bf16_round_bits",
    "bf16_bits_to_float32",
    "n_evict_for_keep_pct",
    "make_case",
    "make_gaussian_case",
    "prefill_queries",
]


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even.

    NaN stays a quiet NaN; +-inf and values that round past the largest
    finite bf16 become +-inf, as IEEE rounding prescribes.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    nan = np.isnan(x)
    if nan.any():
        rounded = np.where(nan, ((bits >> np.uint64(16)).astype(np.uint32) | np.uint32(0x40)), rounded)
    return rounded.astype(np.uint16)


def bf16_bits_to_float32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for host-side use)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def n_evict_for_keep_pct(n: int, keep_pct: int) -> int:
    """Budget as a percentage of n kept -> number evicted, in integers.

    n_keep = floor(n * pct / 100); the protected window counts toward the
    kept tokens.
    """
    n_keep = (n * int(keep_pct)) // 100
    return n - n_keep


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    Hq: int
    Hkv: int
    d: int
    n: int
    window: int
    dtype: str  # "f32" or "bf16"
    pool_kernel: int
    keep_pct: Tuple[int, ...] = ()
    n_evict_fixed: Optional[int] = None
    needles: int = 0
    sink: bool = False
    batch: int = 1
    layers: int = 1
    seeds: Tuple[int, int, int] = (42, 43, 44)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def n_evicts(self) -> Tuple[int, ...]:
        if self.n_evict_fixed is not None:
            return (self.n_evict_fixed,)
        return tuple(n_evict_for_keep_pct(self.n, p) for p in self.keep_pct)

    def layer_seeds(self, layer: int, b: int) -> Tuple[int, int, int]:
        off = 1000 * layer + 100 * b
        return tuple(s + off for s in self.seeds)  # type: ignore[return-value]


# The five workloads: a tiny exactness case, and Llama-3.1-8B / Qwen2.5-7B
# shaped layers from 4K to 128K tokens.
CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", Hq=4, Hkv=2, d=8, n=22, window=3, dtype="f32",
                   pool_kernel=3, n_evict_fixed=7),
    "llama_4k": Config("llama_4k", Hq=32, Hkv=8, d=128, n=4096, window=32,
                       dtype="bf16", pool_kernel=7, keep_pct=(5,), needles=16, sink=True),
    "llama_32k": Config("llama_32k", Hq=32, Hkv=8, d=128, n=32768, window=64,
                        dtype="bf16", pool_kernel=7, keep_pct=(5, 20), needles=16, sink=True),
    "llama_128k": Config("llama_128k", Hq=32, Hkv=8, d=128, n=131072, window=64,
                         dtype="bf16", pool_kernel=7, keep_pct=(5,), needles=64, sink=True),
    "qwen_128k_sweep": Config("qwen_128k_sweep", Hq=28, Hkv=4, d=128, n=131072, window=64,
                              dtype="bf16", pool_kernel=7, keep_pct=(5,), needles=64, sink=True,
                              batch=2, layers=28),
}


@dataclasses.dataclass
class Case:
    """One sequence's inputs. q/k/v are uint16 (bf16 bits) or float32."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    n: int
    window: int
    Hq: int
    Hkv: int
    d: int
    dtype: str
    needle_pos: Optional[np.ndarray] = None

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_gaussian_case(Hq: int, Hkv: int, d: int, n: int, window: int, *,
                       dtype: str = "f32", seeds=(42, 43, 44),
                       one_stream_seed: Optional[int] = None,
                       sink: bool = False, needles: int = 0,
                       sink_scale: float = 3.0, needle_scale: float = 2.5) -> Case:
    """N(0,1) Q/K/V, optionally with a planted sink and needles.

    seeds: (Q seed, K seed, V seed), one PCG64 stream each.
    one_stream_seed: if given, Q then K then V are drawn from one stream.
    Sink and needles (per KV head g): u = mean of the group's fp32 queries
    over its G heads and window rows, normalised; key 0 := sink_scale*sqrt(d)*u,
    `needles` keys at positions drawn without replacement from [1, n-window)
    on the K stream := needle_scale*sqrt(d)*u. V is untouched. Rounding to bf16
    (if asked) happens last, once.
    """
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if one_stream_seed is not None:
        rq = rk = rv = np.random.default_rng(one_stream_seed)
    else:
        rq, rk, rv = (np.random.default_rng(s) for s in seeds)
    q = _normal(rq, (Hq, window, d))
    k = _normal(rk, (Hkv, n, d))
    v = _normal(rv, (Hkv, n, d))
    G = Hq // Hkv
    needle_pos = None
    if sink or needles:
        span = n - window - 1
        if needles > max(span, 0):
            raise ValueError("too many needles for this n/window")
        all_pos = []
        for g in range(Hkv):
            mu = q[g * G:(g + 1) * G].reshape(-1, d).astype(np.float64).mean(axis=0)
            u = (mu / np.linalg.norm(mu)).astype(np.float32)
            if sink:
                k[g, 0] = np.float32(sink_scale * math.sqrt(d)) * u
            if needles:
                pos = rk.choice(span, size=needles, replace=False) + 1
                k[g, pos] = np.float32(needle_scale * math.sqrt(d)) * u
                all_pos.append(np.sort(pos))
        if needles:
            needle_pos = np.stack(all_pos)
    if dtype == "bf16":
        q, k, v = bf16_round_bits(q), bf16_round_bits(k), bf16_round_bits(v)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return Case(q=q, k=k, v=v, n=n, window=window, Hq=Hq, Hkv=Hkv, d=d,
                dtype=dtype, needle_pos=needle_pos)


def make_decode_case(Hq: int, Hkv: int, d: int, n_total: int, *, seeds=(42, 43, 44),
                     sink: bool = True, needles: int = 0, sink_scale: float = 3.0,
                     needle_scale: float = 2.5):
    """A cache grown token by token: query rows of every position and the keys
    and values, bf16 bit patterns, q_all [Hq][n_total][d], k, v [Hkv][n_total][d].

    N(0,1) draws (Q, K, V from one PCG64 stream each); per KV head the sink
    (key 0) and `needles` keys at positions drawn from [1, n_total // 2) on the
    K stream point along the normalised mean of the group's queries, as in
    make_gaussian_case. Rounded to bf16 once, last.
    """
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    rq, rk, rv = (np.random.default_rng(s) for s in seeds)
    q = _normal(rq, (Hq, n_total, d))
    k = _normal(rk, (Hkv, n_total, d))
    v = _normal(rv, (Hkv, n_total, d))
    G = Hq // Hkv
    for g in range(Hkv):
        mu = q[g * G:(g + 1) * G].reshape(-1, d).astype(np.float64).mean(axis=0)
        u = (mu / np.linalg.norm(mu)).astype(np.float32)
        if sink:
            k[g, 0] = np.float32(sink_scale * math.sqrt(d)) * u
        if needles:
            pos = rk.choice(n_total // 2 - 1, size=needles, replace=False) + 1
            k[g, pos] = np.float32(needle_scale * math.sqrt(d)) * u
    return bf16_round_bits(q), bf16_round_bits(k), bf16_round_bits(v)


def make_case(cfg: Config, *, layer: int = 0, b: int = 0, dtype: Optional[str] = None,
              one_stream_seed: Optional[int] = None, n: Optional[int] = None) -> Case:
    """Inputs of one sequence of a named workload (optionally another n/dtype)."""
    seeds = cfg.layer_seeds(layer, b)
    return make_gaussian_case(cfg.Hq, cfg.Hkv, cfg.d, n if n is not None else cfg.n, cfg.window,
                              dtype=dtype or cfg.dtype, seeds=seeds,
                              one_stream_seed=one_stream_seed,
                              sink=cfg.sink, needles=cfg.needles)


def prefill_queries(case: Case, seed: int) -> np.ndarray:
    """Queries of every position for a prefill of `case`: [Hq][n][d].

    The last `window` positions hold the case's own window queries; the
    earlier positions are N(0,1) draws from their own PCG64 stream (`seed`),
    rounded like the case's tensors (bf16 bit patterns or float32).
    """
    rng = np.random.default_rng(seed)
    prefix = _normal(rng, (case.Hq, case.n - case.window, case.d))
    if case.dtype == "bf16":
        prefix = bf16_round_bits(prefix)
    out = np.empty((case.Hq, case.n, case.d), dtype=case.q.dtype)
    out[:, : case.n - case.window] = prefix
    out[:, case.n - case.window:] = case.q
    return out
