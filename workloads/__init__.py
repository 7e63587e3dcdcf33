"""Seeded synthetic inputs for the MoE expert-layer path.

This module is shared by the tests, the benchmark and the oracle's callers. It
holds only random draws, shape presets and dtype storage conversion; none of
the method's arithmetic (routing, permutation, expert FFN, combine) lives here.

Presets follow the workloads named for the path: a tiny fp32 layer, a dense
8-expert bf16 layer, a fine-grained 64-expert layer with two shared experts, a
skewed-routing stress case, and one expert-tensor-parallel rank's local shard
(32 experts, D=7168, F cut 4-way to 512, routing given as input); and two decode
steps (64 and 128 tokens through the dense and the fine-grained layer) on the masked
layout. Sizes of the
expert weights follow the SwiGLU layout w1/w3 [E,F,D], w2 [E,D,F] (HyperParallel
issue 104, "Expert Tensor Parallel" design note, section 4.3 weight placement).

Generator recipe (numpy PCG64, ``default_rng(seed)``):

* every array draws from its own stream ``default_rng([seed, tag, block])``
  (block = expert index for expert stacks, 1024-row block for x), so arrays
  are independent of one another and slabs can be drawn in parallel;
* x ~ N(0, 1); every weight ~ N(0, 1/sqrt(fan_in)) with fan_in = D for Wg,
  w1, w3 and fan_in = F for w2 (std = 1/sqrt(fan_in));
* draws are float32, and bf16 presets round them to bf16 with
  round-to-nearest-even, stored as uint16 bit patterns;
* large weights are drawn expert by expert so host memory stays bounded;
* the output gradient of the backward, dout [T, D] ~ N(0, 1), has a stream of its
  own (a unit-variance upstream gradient, stored in the preset's dtype).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

__all__ = [
    "MoEConfig", "PRESETS", "preset", "shrink", "generate", "router_inputs", "output_grad",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "as_f32",
]


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens (for given-routing presets: derived from the drawn counts)
    D: int            # model dimension
    F: int            # expert intermediate dimension
    E: int            # experts
    k: int            # experts per token
    m_tile: int       # GEMM M-tile every expert segment is padded to
    dtype: str        # "f32" or "bf16"
    n_shared: int = 0         # always-active shared experts
    F_shared: int = 0         # intermediate dimension of each shared expert
    routing: str = "softmax_topk"   # "softmax_topk" or "given"
    zipf_s: float = 0.0       # >0: router bias b_e = -zipf_s * zipf_beta * ln(rank_e)
    zipf_beta: float = 1.0
    poisson_mean: float = 0.0  # given routing: rows per expert ~ Poisson(mean)
    cap: int = 0               # >0: the masked (fixed-capacity slab) layout with cap rows per expert

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


# Skew strength of the Zipf router bias: the smallest beta in {1.5, 2, 2.5, 3} whose
# seeded routing puts >= 24% of the assignments on one expert (top-4 caps a share at
# 25%) and leaves at least one expert empty (tests/test_workloads.py checks this rule).
SKEW_BETA = 2.0

PRESETS: Dict[str, MoEConfig] = {
    "tiny_f32": MoEConfig("tiny_f32", T=256, D=128, F=256, E=8, k=2, m_tile=16, dtype="f32"),
    "dense8_bf16": MoEConfig("dense8_bf16", T=4096, D=4096, F=14336, E=8, k=2, m_tile=128,
                             dtype="bf16"),
    "fine64_shared2_bf16": MoEConfig("fine64_shared2_bf16", T=8192, D=2048, F=1408, E=64, k=6,
                                     m_tile=128, dtype="bf16", n_shared=2, F_shared=1408),
    "skew32_zipf_bf16": MoEConfig("skew32_zipf_bf16", T=16384, D=4096, F=2048, E=32, k=4,
                                  m_tile=128, dtype="bf16", zipf_s=1.2, zipf_beta=SKEW_BETA),
    "etp_shard32_bf16": MoEConfig("etp_shard32_bf16", T=0, D=7168, F=512, E=32, k=8,
                                  m_tile=128, dtype="bf16", routing="given",
                                  poisson_mean=512.0),
    # decode steps on the masked layout: a small batch of tokens, slabs of cap = T rows
    # per expert (no slot can be dropped)
    "decode8_bf16": MoEConfig("decode8_bf16", T=64, D=4096, F=14336, E=8, k=2, m_tile=128,
                              dtype="bf16", cap=64),
    "decode64_shared2_bf16": MoEConfig("decode64_shared2_bf16", T=128, D=2048, F=1408, E=64,
                                       k=6, m_tile=128, dtype="bf16", n_shared=2,
                                       F_shared=1408, cap=128),
}


def preset(name: str) -> MoEConfig:
    return PRESETS[name]


def shrink(cfg: MoEConfig, **kw) -> MoEConfig:
    """Same structure at other sizes (for parity runs the oracle finishes quickly)."""
    name = kw.pop("name", cfg.name + "_small")
    return dataclasses.replace(cfg, name=name, **kw)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even.

    Storage conversion of drawn inputs (inputs are finite)."""
    u = np.array(a, dtype=np.float32, copy=True).view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    u += r
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# Every array (and every expert slab or row block of it) draws from its own PCG64
# stream keyed by (seed, tag, block), so slabs can be drawn in parallel threads and a
# slab's values do not depend on which other arrays were drawn.
_TAGS = {"routing": 10, "x": 1, "wg": 2, "w1": 3, "w3": 4, "w2": 5,
         "ws1": 6, "ws3": 7, "ws2": 8, "bias": 9, "dout": 11}
_X_ROWS_PER_BLOCK = 1024
_POOL_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _rng(seed: int, name: str, block: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, _TAGS[name], block])


def _slab(seed, name, block, shape, std, dtype):
    a = _rng(seed, name, block).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a if dtype == "f32" else f32_to_bf16_bits(a)


def _expert_stack(seed, name, E, rows, cols, std, dtype, pool) -> np.ndarray:
    out = np.empty((E, rows, cols), dtype=np.float32 if dtype == "f32" else np.uint16)

    def fill(e):
        out[e] = _slab(seed, name, e, (rows, cols), std, dtype)
    list(pool.map(fill, range(E)))
    return out


def _activations(seed, T, D, dtype, pool) -> np.ndarray:
    out = np.empty((T, D), dtype=np.float32 if dtype == "f32" else np.uint16)
    nb = -(-T // _X_ROWS_PER_BLOCK)

    def fill(b):
        r0 = b * _X_ROWS_PER_BLOCK
        r1 = min(T, r0 + _X_ROWS_PER_BLOCK)
        out[r0:r1] = _slab(seed, "x", b, (r1 - r0, D), 1.0, dtype)
    list(pool.map(fill, range(nb)))
    return out


def _given_routing(rng: np.random.Generator, E: int, k: int, mean: float):
    """Routing of one expert-tensor-parallel rank: rows per local expert ~ Poisson(mean),
    a token never holds one expert twice, slots that live on other ranks are -1, and the
    top-k weights come from a Dirichlet(1) draw renormalised to sum 1 in float32."""
    counts = rng.poisson(mean, E).astype(np.int64)
    N = int(counts.sum())
    T = -(-N // k)
    if int(counts.max()) > T:
        raise ValueError("an expert holds more rows than there are tokens")
    flat = np.concatenate([np.repeat(np.arange(E, dtype=np.int32), counts),
                           np.full(k * T - N, -1, dtype=np.int32)])
    slots = flat.reshape(k, T).T.copy()          # slots[t, j] = flat[j*T + t]
    slots = slots[rng.permutation(T)]
    slots = rng.permuted(slots, axis=1)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    w = w / w.sum(axis=1, keepdims=True, dtype=np.float32)
    w = w.astype(np.float32)
    w[slots < 0] = 0.0
    return np.ascontiguousarray(slots, dtype=np.int32), np.ascontiguousarray(w), T


def generate(cfg: MoEConfig, seed: int = 0) -> dict:
    """Draw every input of ``cfg``. bf16 arrays are uint16 bit patterns.

    Returns keys: x [T,D]; wg [E,D] (routed presets); bias [E] float32 (skewed preset);
    w1, w3 [E,F,D]; w2 [E,D,F]; ws1, ws3 [n_shared,F_shared,D], ws2 [n_shared,D,F_shared]
    (shared-expert preset); topk_idx [T,k] int32 and topk_w [T,k] float32 (given-routing
    preset); and "cfg", the preset with T filled in.
    """
    out: dict = {}
    T, D, F, E, k, dt = cfg.T, cfg.D, cfg.F, cfg.E, cfg.k, cfg.dtype
    if cfg.routing == "given":
        idx, w, T = _given_routing(_rng(seed, "routing"), E, k, cfg.poisson_mean)
        cfg = dataclasses.replace(cfg, T=T)
        out["topk_idx"], out["topk_w"] = idx, w
    with ThreadPoolExecutor(_POOL_THREADS) as pool:
        out.update(router_inputs(cfg, seed, pool))
        out["w1"] = _expert_stack(seed, "w1", E, F, D, 1.0 / math.sqrt(D), dt, pool)
        out["w3"] = _expert_stack(seed, "w3", E, F, D, 1.0 / math.sqrt(D), dt, pool)
        out["w2"] = _expert_stack(seed, "w2", E, D, F, 1.0 / math.sqrt(F), dt, pool)
        if cfg.n_shared:
            S, Fs = cfg.n_shared, cfg.F_shared
            out["ws1"] = _expert_stack(seed, "ws1", S, Fs, D, 1.0 / math.sqrt(D), dt, pool)
            out["ws3"] = _expert_stack(seed, "ws3", S, Fs, D, 1.0 / math.sqrt(D), dt, pool)
            out["ws2"] = _expert_stack(seed, "ws2", S, D, Fs, 1.0 / math.sqrt(Fs), dt, pool)
    out["cfg"] = cfg
    return out


def router_inputs(cfg: MoEConfig, seed: int = 0, pool=None) -> dict:
    """The router's inputs of ``cfg`` (T filled in), drawn as ``generate`` draws them:
    x [T,D], and for routed presets wg [E,D] and (skewed preset) the bias [E]."""
    T, D, E, dt = cfg.T, cfg.D, cfg.E, cfg.dtype
    out = {}
    if pool is None:
        with ThreadPoolExecutor(_POOL_THREADS) as own:
            out["x"] = _activations(seed, T, D, dt, own)
    else:
        out["x"] = _activations(seed, T, D, dt, pool)
    if cfg.routing != "given":
        out["wg"] = _slab(seed, "wg", 0, (E, D), 1.0 / math.sqrt(D), dt)
    if cfg.zipf_s:
        rank = _rng(seed, "bias").permutation(E).astype(np.float64) + 1.0
        out["bias"] = (-cfg.zipf_s * cfg.zipf_beta * np.log(rank)).astype(np.float32)
    return out


def output_grad(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """dout [T, D] ~ N(0, 1) in cfg's dtype (``cfg`` with T filled in, as ``generate``
    returns it), drawn in 1024-row blocks like x."""
    T, D, dt = cfg.T, cfg.D, cfg.dtype
    out = np.empty((T, D), dtype=np.float32 if dt == "f32" else np.uint16)
    for b in range(-(-T // _X_ROWS_PER_BLOCK)):
        r0 = b * _X_ROWS_PER_BLOCK
        r1 = min(T, r0 + _X_ROWS_PER_BLOCK)
        out[r0:r1] = _slab(seed, "dout", b, (r1 - r0, D), 1.0, dt)
    return out


def as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Values of a stored array as float32 (bf16 bit patterns are widened exactly)."""
    return a if dtype == "f32" else bf16_bits_to_f32(a)
